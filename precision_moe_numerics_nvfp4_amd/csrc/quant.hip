// NVFP4 quantization (per token / per expert) and row-wise MXFP8 quantization.
//
// NVFP4, after "Inkling 2 Small uses four-bit training ..." (ai-primer),
// section "Block scales and per-token activations": per outer-scale group
// A = max|x|, s = A / 2688, block scale S = E4M3_RNE(max|x_block| / (6 s)),
// codes E2M1_RNE(x * (1 / (S s))). One wavefront owns one row: each lane owns
// whole 16-element blocks (16 consecutive bfloat16 = 32 contiguous bytes, so
// consecutive lanes read consecutive bytes), the row maximum is a wavefront
// shuffle reduction, and every block is packed to 8 bytes of codes plus one
// scale byte without leaving registers. For per-expert scales a first pass
// reduces max|x| over each expert with one atomic max per workgroup (the
// outer-scale buffer holds the float bits meanwhile), then the quantizer runs
// with that maximum, then a tiny pass stores s = A / 2688.
//
// MXFP8 row-wise (dY, "NVFP4 forward, MXFP8 backward"): four lanes share one
// 32-element block (8 elements each), reduce the block maximum with two
// shuffles, pick the smallest exponent that keeps the block inside 448 and
// round each element to nearest-even E4M3.
#include "codecs.hpp"
#include "internal.hpp"

namespace nvfp4moe {

namespace {

template <bool BF16>
struct Row16 {  // 16 consecutive input elements held as raw words
  static constexpr int W = BF16 ? 8 : 16;
  uint32_t w[W];
  __device__ __forceinline__ float get(int j) const {
    if constexpr (BF16) return (j & 1) ? u2f(w[j >> 1] & 0xFFFF0000u) : u2f(w[j >> 1] << 16);
    else return u2f(w[j]);
  }
};

template <bool BF16>
__device__ __forceinline__ void load16(const void* base, int64_t elem, Row16<BF16>& r) {
  if constexpr (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    const uint4 a = ld_stream16(p), b = ld_stream16(p + 1);
    r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
    r.w[4] = b.x; r.w[5] = b.y; r.w[6] = b.z; r.w[7] = b.w;
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 a = ld_stream16(p + i);
      r.w[4 * i] = a.x; r.w[4 * i + 1] = a.y; r.w[4 * i + 2] = a.z; r.w[4 * i + 3] = a.w;
    }
  }
}

// One wavefront per row; lane l owns blocks l, l+64, ...
// gamax != nullptr: per-group mode, A is read from the group-max pass.
// SR: block scales rounded up to the next E4M3 value and codes rounded
// stochastically, the draw of element (row, c) at index row * cols + c.
// NT: non-temporal stores (outputs larger than the Infinity Cache, which
// the next kernel reads from HBM anyway).
template <bool BF16, int BPL, bool SR = false, bool NT = false>
__device__ __forceinline__ void quantize_row(
    const void* __restrict__ x, int64_t row, int nb, const uint32_t* __restrict__ gamax,
    int64_t rpg, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ outer, uint64_t seed = 0, uint32_t tag = 0) {
  const int lane = threadIdx.x & 63;
  Row16<BF16> v[BPL];
  float bmax[BPL];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int b = lane + 64 * i;
    bmax[i] = 0.0f;
    if (b < nb) {
      load16<BF16>(x, (row * nb + b) * 16, v[i]);
#pragma unroll
      for (int j = 0; j < 16; ++j) bmax[i] = fmaxf(bmax[i], fabsf(v[i].get(j)));
    }
    amax = fmaxf(amax, bmax[i]);
  }
  const float A = gamax ? u2f(gamax[row / rpg]) : wave_max(amax);
  const float s = __fdiv_rn(A, 2688.0f);
  const float d = __fmul_rn(6.0f, s);
  if (!gamax && lane == 0) outer[row] = s;

#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int b = lane + 64 * i;
    if (b >= nb) continue;
    uint32_t sc = 0;
    if (A > 0.0f) {
      if constexpr (SR) sc = e4m3_ceil_pos(__fdiv_rn(bmax[i], d));
      else sc = e4m3_rne_sat_pos(__fdiv_rn(bmax[i], d));
    }
    uint32_t lo = 0, hi = 0;
    const uint64_t q = (uint64_t)(row * nb + b) * 2;   // Philox counter: (row * cols + 16 b) / 8
    if (sc) {
      const float r = __fdiv_rn(1.0f, __fmul_rn(e4m3_pos_to_f32(sc), s));
      float a[8], b[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        a[j] = __fmul_rn(v[i].get(j), r);
        b[j] = __fmul_rn(v[i].get(j + 8), r);
      }
      if constexpr (SR) {
        const Draws8 d0 = draws8(q, seed, tag), d1 = draws8(q + 1, seed, tag);
        uint32_t u0[8], u1[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          u0[j] = d0.get(j);
          u1[j] = d1.get(j);
        }
        lo = e2m1x8_sr(a, u0);
        hi = e2m1x8_sr(b, u1);
      } else {
        lo = e2m1x8_rne(a);
        hi = e2m1x8_rne(b);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        lo |= ((f2u(v[i].get(j)) >> 28) & 8u) << (4 * j);
        hi |= ((f2u(v[i].get(j + 8)) >> 28) & 8u) << (4 * j);
      }
    }
    const int64_t blk = row * nb + b;
    if constexpr (NT) {
      typedef uint32_t u32x2n __attribute__((ext_vector_type(2)));
      __builtin_nontemporal_store(u32x2n{lo, hi}, reinterpret_cast<u32x2n*>(codes + blk * 8));
      __builtin_nontemporal_store((uint8_t)sc, scales + blk);
    } else {
      *reinterpret_cast<uint2*>(codes + blk * 8) = make_uint2(lo, hi);
      scales[blk] = (uint8_t)sc;
    }
  }
}

// 4 rows per workgroup, one per wavefront.
template <bool BF16, int BPL, bool NT>
__global__ __launch_bounds__(256) void k_nvfp4_quantize(
    const void* __restrict__ x, int64_t rows, int nb, const uint32_t* __restrict__ gamax,
    int64_t rpg, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ outer) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform per wavefront
  quantize_row<BF16, BPL, false, NT>(x, row, nb, gamax, rpg, codes, scales, outer);
}

// Row-wise NVFP4 with stochastic rounding (per-row outer scales), 4 rows per
// workgroup.
template <bool BF16, int BPL>
__global__ __launch_bounds__(256) void k_nvfp4_quantize_sr(
    const void* __restrict__ x, int64_t rows, int nb, uint64_t seed, uint32_t tag,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ outer) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform per wavefront
  quantize_row<BF16, BPL, true>(x, row, nb, nullptr, 1, codes, scales, outer, seed, tag);
}

// Per-row outer scales for the first *n_live rows of a capacity-sized
// buffer (the count is device data, so the grid walks the rows).
template <bool BF16, int BPL>
__global__ __launch_bounds__(256) void k_nvfp4_quantize_live(
    const void* __restrict__ x, int64_t rows, const int64_t* __restrict__ n_live, int nb,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ outer) {
  const int64_t live = *n_live;
  const int64_t n = live < rows ? live : rows;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < n;
       row += (int64_t)gridDim.x * 4)
    quantize_row<BF16, BPL>(x, row, nb, nullptr, 1, codes, scales, outer);
}

// 16x16-tile NVFP4 (one E4M3 scale per tile, outer scale per group of rows):
// a workgroup covers 16 rows x 256 columns; thread (r = tid % 16, c = tid /
// 16) owns row r of tile column c (16 elements), the 16 lanes of a tile reduce
// its maximum with four shuffles, and each lane packs its 16 codes. The group
// maximum comes from the same pass as the per-expert quantizer.
template <bool BF16>
__global__ __launch_bounds__(256) void k_nvfp4_quantize_tile16(
    const void* __restrict__ x, int64_t cols, const uint32_t* __restrict__ gamax, int64_t rpg,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int r = threadIdx.x & 15, c = threadIdx.x >> 4;
  const int64_t ty = blockIdx.y;                          // tile row
  const int64_t tc = (int64_t)blockIdx.x * 16 + c;        // tile column
  const int64_t ntc = cols / 16;
  const bool live = tc < ntc;                             // the same for a tile's 16 lanes
  const int64_t row = ty * 16 + r;
  Row16<BF16> v;
  float m = 0.0f;
  if (live) {
    load16<BF16>(x, row * cols + tc * 16, v);
#pragma unroll
    for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(v.get(j)));
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (!live) return;
  const float A = u2f(gamax[row / rpg]);
  const float s = __fdiv_rn(A, 2688.0f);
  const float d = __fmul_rn(6.0f, s);
  uint32_t sc = 0;
  if (A > 0.0f) sc = e4m3_rne_sat_pos(__fdiv_rn(m, d));
  uint32_t lo = 0, hi = 0;
  if (sc) {
    const float rc = __fdiv_rn(1.0f, __fmul_rn(e4m3_pos_to_f32(sc), s));
    float a[8], b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[j] = __fmul_rn(v.get(j), rc);
      b[j] = __fmul_rn(v.get(j + 8), rc);
    }
    lo = e2m1x8_rne(a);
    hi = e2m1x8_rne(b);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lo |= ((f2u(v.get(j)) >> 28) & 8u) << (4 * j);
      hi |= ((f2u(v.get(j + 8)) >> 28) & 8u) << (4 * j);
    }
  }
  *reinterpret_cast<uint2*>(codes + row * (cols / 2) + tc * 8) = make_uint2(lo, hi);
  if (r == 0) scales[ty * ntc + tc] = (uint8_t)sc;
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// max|x| over each group of `per` contiguous elements; blockIdx.y = group.
// 1024-thread workgroups, about one per compute unit, each thread keeping
// eight 16-byte loads in flight; one atomic max per workgroup (atomics on
// one address serialize, so there are few of them).
template <bool BF16>
__global__ __launch_bounds__(1024) void k_group_amax(const void* __restrict__ x, int64_t per,
                                                     uint32_t* __restrict__ amax_bits) {
  __shared__ float red[16];
  constexpr int U = 8;                                // loads in flight per thread
  const int64_t g = blockIdx.y;
  const uint8_t* base = static_cast<const uint8_t*>(x) + g * per * (BF16 ? 2 : 4);
  const int64_t nl = per / (BF16 ? 8 : 4);            // 16-byte pieces in the group
  const int64_t stride = (int64_t)gridDim.x * 1024;
  float m = 0.0f;
  for (int64_t i0 = (int64_t)blockIdx.x * 1024 + threadIdx.x; i0 < nl; i0 += stride * U) {
    uint4 a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + u * stride;
      a[u] = i < nl ? ld_stream16(reinterpret_cast<const uint4*>(base) + i) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t w[4] = {a[u].x, a[u].y, a[u].z, a[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (BF16) {
          m = fmaxf(m, fabsf(u2f(w[j] << 16)));
          m = fmaxf(m, fabsf(u2f(w[j] & 0xFFFF0000u)));
        } else {
          m = fmaxf(m, fabsf(u2f(w[j])));
        }
      }
    }
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x < 64) {
    m = threadIdx.x < 16 ? red[threadIdx.x] : 0.0f;
    m = wave_max(m);
    if (threadIdx.x == 0) atomicMax(amax_bits + g, f2u(m));  // non-negative floats order like their bits
  }
}

__global__ void k_outer_from_amax(float* __restrict__ outer, int64_t G) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g < G) outer[g] = __fdiv_rn(outer[g], 2688.0f);
}

// Row-wise MXFP8: 4 lanes per 32-element block, 8 elements per lane; each
// thread handles U chunks per round, U * 64 chunks apart, loads issued first.
template <bool BF16>
__global__ __launch_bounds__(256) void k_mx_rowwise(const void* __restrict__ x, int64_t nchunks,
                                                    uint8_t* __restrict__ q,
                                                    uint8_t* __restrict__ e8) {
  constexpr int U = 4;
  const int64_t padded = (nchunks + 63) & ~63LL;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t c0 = (int64_t)blockIdx.x * 256 + threadIdx.x; c0 < padded; c0 += stride * U) {
    float v[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * stride;
      const bool ok = c < nchunks;  // 8 elements per chunk
      if constexpr (BF16) {
        const uint4 a = ok ? ld_stream16(reinterpret_cast<const uint4*>(
                                 static_cast<const uint16_t*>(x) + c * 8))
                           : make_uint4(0, 0, 0, 0);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[u][2 * j] = u2f(w[j] << 16);
          v[u][2 * j + 1] = u2f(w[j] & 0xFFFF0000u);
        }
      } else {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + c * 8);
        const uint4 a = ok ? ld_stream16(p) : make_uint4(0, 0, 0, 0);
        const uint4 b = ok ? ld_stream16(p + 1) : make_uint4(0, 0, 0, 0);
        v[u][0] = u2f(a.x); v[u][1] = u2f(a.y); v[u][2] = u2f(a.z); v[u][3] = u2f(a.w);
        v[u][4] = u2f(b.x); v[u][5] = u2f(b.y); v[u][6] = u2f(b.z); v[u][7] = u2f(b.w);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * stride;
      if (c >= padded) break;                       // uniform per wavefront
      float mf = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) mf = fmaxf(mf, fabsf(v[u][j]));
      const uint32_t code = e8m0_code_bits(quad_max_bits(f2u(mf)));   // E8M0 byte = e + 127
      const float scale = u2f(code << 23);
      const uint32_t lo = e4m3x4_rne_scaled(v[u][0], v[u][1], v[u][2], v[u][3], scale);
      const uint32_t hi = e4m3x4_rne_scaled(v[u][4], v[u][5], v[u][6], v[u][7], scale);
      if (c < nchunks) {
        *reinterpret_cast<uint2*>(q + c * 8) = make_uint2(lo, hi);
        if ((c & 3) == 0) e8[c >> 2] = (uint8_t)code;
      }
    }
  }
}

int g_cu_count = 0;

}  // namespace

int device_cu_count() {
  // one cache per process; every MI355X has the same count
  if (g_cu_count == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      g_cu_count = n;
    else
      g_cu_count = 256;
  }
  return g_cu_count;
}

constexpr double kNtStoreBytes = 256.0 * 1024 * 1024;   // MI355X Infinity Cache

template <bool BF16, bool NT>
static void launch_quantize_rows(int nb, unsigned grid, hipStream_t stream, const void* x,
                                 int64_t rows, const uint32_t* gamax, int64_t rpg,
                                 uint8_t* codes, uint8_t* scales, float* outer) {
  if (nb <= 64)
    k_nvfp4_quantize<BF16, 1, NT><<<grid, 256, 0, stream>>>(x, rows, nb, gamax, rpg, codes, scales, outer);
  else if (nb <= 128)
    k_nvfp4_quantize<BF16, 2, NT><<<grid, 256, 0, stream>>>(x, rows, nb, gamax, rpg, codes, scales, outer);
  else if (nb <= 256)
    k_nvfp4_quantize<BF16, 4, NT><<<grid, 256, 0, stream>>>(x, rows, nb, gamax, rpg, codes, scales, outer);
  else
    k_nvfp4_quantize<BF16, 8, NT><<<grid, 256, 0, stream>>>(x, rows, nb, gamax, rpg, codes, scales, outer);
}

template <bool BF16>
static hipError_t quantize_impl(const void* x, int64_t rows, int64_t cols, bool per_group,
                                int64_t rpg, uint8_t* codes, uint8_t* scales, float* outer,
                                hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int nb = (int)(cols / 16);
  const uint32_t* gamax = nullptr;
  if (per_group) {
    const int64_t G = rows / rpg;
    uint32_t* bits = reinterpret_cast<uint32_t*>(outer);
    k_fill_u32<<<(unsigned)((G + 255) / 256), 256, 0, stream>>>(bits, G, 0u);
    const int64_t per = rpg * cols;
    // about one 1024-thread workgroup per compute unit over all groups
    const int64_t pieces = per / (BF16 ? 8 : 4);
    int64_t gx = ((int64_t)device_cu_count() + G - 1) / G;
    const int64_t most = (pieces + 1023) / 1024;
    if (gx > most) gx = most;
    gx = gx < 1 ? 1 : (gx > 65535 ? 65535 : gx);
    k_group_amax<BF16><<<dim3((unsigned)gx, (unsigned)G), 1024, 0, stream>>>(x, per, bits);
    gamax = bits;
  }
  const unsigned grid = (unsigned)((rows + 3) / 4);
  // codes and scales past the Infinity Cache's size: non-temporal stores
  // (measured on 1 GiB of bf16: 4% faster)
  if ((double)rows * (double)cols * (0.5 + 1.0 / 16) >= kNtStoreBytes)
    launch_quantize_rows<BF16, true>(nb, grid, stream, x, rows, gamax, rpg, codes, scales, outer);
  else
    launch_quantize_rows<BF16, false>(nb, grid, stream, x, rows, gamax, rpg, codes, scales, outer);
  if (per_group) {
    const int64_t G = rows / rpg;
    k_outer_from_amax<<<(unsigned)((G + 255) / 256), 256, 0, stream>>>(outer, G);
  }
  return hipGetLastError();
}

hipError_t launch_nvfp4_quantize(const void* x, bool bf16, int64_t rows, int64_t cols,
                                 bool per_group, int64_t rpg, uint8_t* codes, uint8_t* scales,
                                 float* outer, hipStream_t stream) {
  return bf16 ? quantize_impl<true>(x, rows, cols, per_group, rpg, codes, scales, outer, stream)
              : quantize_impl<false>(x, rows, cols, per_group, rpg, codes, scales, outer, stream);
}

template <bool BF16>
static hipError_t quantize_live_impl(const void* x, int64_t rows, int64_t cols,
                                     const int64_t* n_live, uint8_t* codes, uint8_t* scales,
                                     float* outer, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int nb = (int)(cols / 16);
  int64_t grid = (rows + 3) / 4;
  const int64_t most = (int64_t)device_cu_count() * 16;   // 16 workgroups per CU at most
  if (grid > most) grid = most;
  if (nb <= 64)
    k_nvfp4_quantize_live<BF16, 1><<<(unsigned)grid, 256, 0, stream>>>(x, rows, n_live, nb, codes, scales, outer);
  else if (nb <= 128)
    k_nvfp4_quantize_live<BF16, 2><<<(unsigned)grid, 256, 0, stream>>>(x, rows, n_live, nb, codes, scales, outer);
  else if (nb <= 256)
    k_nvfp4_quantize_live<BF16, 4><<<(unsigned)grid, 256, 0, stream>>>(x, rows, n_live, nb, codes, scales, outer);
  else
    k_nvfp4_quantize_live<BF16, 8><<<(unsigned)grid, 256, 0, stream>>>(x, rows, n_live, nb, codes, scales, outer);
  return hipGetLastError();
}

hipError_t launch_nvfp4_quantize_live(const void* x, bool bf16, int64_t rows, int64_t cols,
                                      const int64_t* n_live, uint8_t* codes, uint8_t* scales,
                                      float* outer, hipStream_t stream) {
  return bf16 ? quantize_live_impl<true>(x, rows, cols, n_live, codes, scales, outer, stream)
              : quantize_live_impl<false>(x, rows, cols, n_live, codes, scales, outer, stream);
}

template <bool BF16>
static hipError_t quantize_sr_impl(const void* x, int64_t rows, int64_t cols, uint64_t seed,
                                   uint32_t tag, uint8_t* codes, uint8_t* scales, float* outer,
                                   hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int nb = (int)(cols / 16);
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (nb <= 64)
    k_nvfp4_quantize_sr<BF16, 1><<<grid, 256, 0, stream>>>(x, rows, nb, seed, tag, codes, scales, outer);
  else if (nb <= 128)
    k_nvfp4_quantize_sr<BF16, 2><<<grid, 256, 0, stream>>>(x, rows, nb, seed, tag, codes, scales, outer);
  else if (nb <= 256)
    k_nvfp4_quantize_sr<BF16, 4><<<grid, 256, 0, stream>>>(x, rows, nb, seed, tag, codes, scales, outer);
  else
    k_nvfp4_quantize_sr<BF16, 8><<<grid, 256, 0, stream>>>(x, rows, nb, seed, tag, codes, scales, outer);
  return hipGetLastError();
}

hipError_t launch_nvfp4_quantize_sr(const void* x, bool bf16, int64_t rows, int64_t cols,
                                    uint64_t seed, uint32_t tag, uint8_t* codes, uint8_t* scales,
                                    float* outer, hipStream_t stream) {
  return bf16 ? quantize_sr_impl<true>(x, rows, cols, seed, tag, codes, scales, outer, stream)
              : quantize_sr_impl<false>(x, rows, cols, seed, tag, codes, scales, outer, stream);
}

template <bool BF16>
static hipError_t quantize_tile16_impl(const void* x, int64_t rows, int64_t cols, int64_t rpg,
                                       uint8_t* codes, uint8_t* scales, float* outer,
                                       hipStream_t stream) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const int64_t G = rows / rpg;
  uint32_t* bits = reinterpret_cast<uint32_t*>(outer);
  k_fill_u32<<<(unsigned)((G + 255) / 256), 256, 0, stream>>>(bits, G, 0u);
  const int64_t per = rpg * cols;
  const int64_t pieces = per / (BF16 ? 8 : 4);
  int64_t gx = ((int64_t)device_cu_count() + G - 1) / G;
  const int64_t most = (pieces + 1023) / 1024;
  if (gx > most) gx = most;
  gx = gx < 1 ? 1 : (gx > 65535 ? 65535 : gx);
  k_group_amax<BF16><<<dim3((unsigned)gx, (unsigned)G), 1024, 0, stream>>>(x, per, bits);
  const dim3 grid((unsigned)((cols / 16 + 15) / 16), (unsigned)(rows / 16));
  k_nvfp4_quantize_tile16<BF16><<<grid, 256, 0, stream>>>(x, cols, bits, rpg, codes, scales);
  k_outer_from_amax<<<(unsigned)((G + 255) / 256), 256, 0, stream>>>(outer, G);
  return hipGetLastError();
}

hipError_t launch_nvfp4_quantize_tile16(const void* x, bool bf16, int64_t rows, int64_t cols,
                                        int64_t rpg, uint8_t* codes, uint8_t* scales,
                                        float* outer, hipStream_t stream) {
  return bf16 ? quantize_tile16_impl<true>(x, rows, cols, rpg, codes, scales, outer, stream)
              : quantize_tile16_impl<false>(x, rows, cols, rpg, codes, scales, outer, stream);
}

hipError_t launch_mxfp8_quantize_rowwise(const void* x, bool bf16, int64_t rows, int64_t cols,
                                         uint8_t* q, uint8_t* e8, hipStream_t stream) {
  const int64_t nchunks = rows * cols / 8;
  if (nchunks == 0) return hipSuccess;
  int64_t grid = (nchunks + 1023) / 1024;               // about one round of 4 chunks per thread
  const int64_t cap = (int64_t)device_cu_count() * 16;
  if (grid > cap) grid = cap;
  if (bf16)
    k_mx_rowwise<true><<<(unsigned)grid, 256, 0, stream>>>(x, nchunks, q, e8);
  else
    k_mx_rowwise<false><<<(unsigned)grid, 256, 0, stream>>>(x, nchunks, q, e8);
  return hipGetLastError();
}

}  // namespace nvfp4moe
