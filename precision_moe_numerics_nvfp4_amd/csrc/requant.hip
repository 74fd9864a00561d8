// Grouped transpose + MXFP8 (or NVFP4) quantization along the token dimension.
//
// Users:
//  * mxfp8_requant_sr: the saved NVFP4 activations / weights are dequantized
//    to float32, transposed, and re-quantized to MXFP8 with stochastic
//    rounding ("Inkling 2 Small uses four-bit training ...", section
//    "Stochastic rounding across transposes");
//  * mxfp8_quantize (COLWISE_GROUPED): dY is transposed and quantized with
//    round-to-nearest-even, giving the wgrad operand;
//  * the NVFP4 backward (nvfp4_requant_sr, nvfp4_quantize_sr colwise): the
//    same transposes with NVFP4 output: blocks of 16 tokens (two neighbouring
//    lanes), E4M3 block scales rounded up, E2M1 codes rounded stochastically,
//    one outer scale per group from maximum passes over the group's rows
//    (k_row_amax, k_group_max) run before; optionally written per group
//    ([G, cols, group length], the transposed weights of each expert).
//
// Output [cols, P]: input rows [offsets[g], offsets[g+1]) of group g land in
// columns padded_offsets[g] + (r - offsets[g]); the rest of each group's
// 32-aligned segment is zero, so every 32-element MXFP8 block of an output row
// lies in one group.
//
// Tiling: a workgroup owns a 128-token x 128-column tile. The input rows are
// staged in LDS in their stored form (4-bit codes + scales, or bf16/f32), so
// HBM is read once, row-contiguously. Each thread then owns an 8-column x
// 8-token micro-tile: it reads the 8 tokens' values of its 8 columns from LDS
// (the transpose), four neighbouring lanes cover one 32-token block and
// reduce its maximum with two quad DPP exchanges, and each thread writes 8
// contiguous output bytes per column (16 threads write one 128-byte output
// row segment). The stochastic draws for those 8 bytes are exactly one Philox
// call, because the draw index is the output's linear index and 8 consecutive
// indices share one counter. The block scale's division is folded into the
// scaled conversion instructions (exact; see codecs.hpp).
//
// LDS layout: tile row r (token) lives in slot 16 * (r & 7) + (r >> 3). A
// thread's 8 tokens are rows 8 * pc + i, so for a fixed i the 16 lanes pc =
// 0..15 of a wavefront read 16 consecutive slots; with a code pitch of 18
// words those land on distinct LDS banks (18 * pc mod 32 is 16 distinct even
// values), as do the per-slot scale and outer arrays.
//
// Workgroup order: the grid is one-dimensional over the live tiles (those
// below the padded total read on the device). Consecutive workgroup indices go
// to different XCDs, so each XCD is given a contiguous band of tiles, column
// tile fastest: the workgroups that read the same input rows (and the same
// 128-byte lines of codes and scales) run together on one XCD and share its
// L2, and the E8M0 bytes of neighbouring token tiles are written close in
// time.
#include "codecs.hpp"
#include "internal.hpp"

namespace nvfp4moe {

namespace {

constexpr int TP = 128;  // tokens per tile
constexpr int TK = 128;  // columns per tile

enum class Src { NVFP4, BF16, F32 };

__device__ __forceinline__ int slot_of(int r) { return 16 * (r & 7) + (r >> 3); }

template <Src S>
struct Tile;

template <>
struct Tile<Src::NVFP4> {
  static constexpr int CW = 18;              // code words per slot (16 used)
  uint32_t codes[TP * CW];
  uint32_t scales[TP][TK / 64];              // 8 E4M3 bytes per slot
  float outer[TP];
};
template <>
struct Tile<Src::BF16> {
  static constexpr int PITCH = TK + 8;       // bf16 elements per slot (+pad)
  uint16_t v[TP][PITCH];
};
template <>
struct Tile<Src::F32> {
  static constexpr int PITCH = TK + 4;
  float v[TP][PITCH];
};

// Group maxima for the NVFP4 outputs, in two passes without atomics:
// k_row_amax writes each live row's maximum magnitude (float bits) to a
// scratch array, k_group_max reduces each group's rows with one workgroup.
// NVFP4 rows give max |e2m1 * S| times their outer scale, the value the
// transpose dequantizes them to (rounding is monotone, so the maximum of the
// rounded products is the rounded product of the maximum).
template <Src S>
__global__ __launch_bounds__(256) void k_row_amax(
    const void* __restrict__ src, const uint8_t* __restrict__ src_scales,
    const float* __restrict__ src_outer, int64_t rpg, int64_t cols,
    const int64_t* __restrict__ offsets, int G, uint32_t* __restrict__ row_bits) {
  const int lane = threadIdx.x & 63;
  const int64_t rows = offsets[G];
  // lane-partial maximum of one 16-byte chunk at byte c of row r
  auto chunk_max = [&](int64_t r, int64_t c) -> float {
    float m = 0.0f;
    if constexpr (S == Src::NVFP4) {
      const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(src) +
                                                      r * (cols / 2) + c);
      const uint32_t sc2 = *reinterpret_cast<const uint16_t*>(src_scales + r * (cols / 16) + c / 8);
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        uint32_t mx = 0;                      // largest magnitude code (order = value order)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int n = 0; n < 8; ++n) mx = max(mx, (wd[2 * blk + h] >> (4 * n)) & 7u);
        float e0, e1;
        e2m1x2_to_f32(mx, 0, e0, e1);
        m = fmaxf(m, __fmul_rn(e0, e4m3_pos_to_f32((sc2 >> (8 * blk)) & 0x7Fu)));
      }
    } else {
      constexpr int EB = (S == Src::BF16) ? 2 : 4;
      const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(src) +
                                                      r * cols * EB + c);
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (S == Src::BF16) {
          m = fmaxf(m, fabsf(u2f(wd[j] << 16)));
          m = fmaxf(m, fabsf(u2f(wd[j] & 0xFFFF0000u)));
        } else {
          m = fmaxf(m, fabsf(u2f(wd[j])));
        }
      }
    }
    return m;
  };
  const int64_t row_bytes = S == Src::NVFP4 ? cols / 2 : cols * (S == Src::BF16 ? 2 : 4);
  constexpr int U = 4;                        // rows whose loads are in flight together
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t rb = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * U; rb < rows; rb += nw * U) {
    float m[U];
#pragma unroll
    for (int u = 0; u < U; ++u) m[u] = 0.0f;
    for (int64_t c = 16 * lane; c < row_bytes; c += 16 * 64) {
      float part[U];
#pragma unroll
      for (int u = 0; u < U; ++u) part[u] = chunk_max(rb + u < rows ? rb + u : rows - 1, c);
#pragma unroll
      for (int u = 0; u < U; ++u) m[u] = fmaxf(m[u], part[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = rb + u;
      float mu = wave_max(m[u]);
      if constexpr (S == Src::NVFP4) mu = __fmul_rn(mu, src_outer[rpg ? (r < rows ? r : 0) / rpg
                                                                        : (r < rows ? r : 0)]);
      if (lane == 0 && r < rows) row_bits[r] = f2u(mu);
    }
  }
}

// bits[g] = maximum of row_bits over group g's rows (0 for an empty group).
__global__ __launch_bounds__(256) void k_group_max(const uint32_t* __restrict__ row_bits,
                                                   const int64_t* __restrict__ offsets,
                                                   uint32_t* __restrict__ bits) {
  __shared__ uint32_t part[4];
  const int g = blockIdx.x;
  const int64_t a = offsets[g], b = offsets[g + 1];
  uint32_t m = 0;
  for (int64_t r = a + threadIdx.x; r < b; r += 256) m = max(m, row_bits[r]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) bits[g] = max(max(part[0], part[1]), max(part[2], part[3]));
}

__global__ void k_zero_u32(uint32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

__global__ void k_bits_to_outer(float* __restrict__ outer, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) outer[i] = __fdiv_rn(outer[i], 2688.0f);     // maximum bits -> A / (6 * 448)
}

__device__ __forceinline__ int64_t xcd_band(int64_t w, int64_t live) {
  const int64_t x = w & 7, s = w >> 3;
  const int64_t q = live >> 3, r = live & 7;
  return x * q + (x < r ? x : r) + s;
}

// ROWS (float sources only): the staged tile also yields the row-wise MXFP8
// quantization of its rows (blocks of 32 along the columns), written to
// row_out [rows, cols] and row_e8 [rows, cols/32] at the source row.
// NVO: NVFP4 output instead (codes to out, E4M3 scales to out_e8, group maxima
// as float bits in gbits); BLK: each group's part written as its own
// [cols, group length] block (MXFP8: starting at element cols * padded[g];
// NVFP4, groups of equal length: at element g * cols * length).
template <Src S, bool SR, bool ROWS = false, bool NVO = false, bool BLK = false>
__global__ __launch_bounds__(256) void k_transpose_mx(
    const void* __restrict__ src, const uint8_t* __restrict__ src_scales,
    const float* __restrict__ src_outer, int64_t rpg, int64_t cols,
    const int64_t* __restrict__ offsets, const int64_t* __restrict__ padded, int G, int64_t P,
    uint64_t seed, uint32_t tag, uint8_t* __restrict__ out, uint8_t* __restrict__ out_e8,
    uint8_t* __restrict__ row_out = nullptr, uint8_t* __restrict__ row_e8 = nullptr,
    const uint32_t* __restrict__ gbits = nullptr) {
  __shared__ Tile<S> tile;
  __shared__ int64_t row_of[TP];  // source row of each tile token, -1 = padding
  __shared__ int grp_of[TP];      // group of each tile token

  const int tid = threadIdx.x;
  const int64_t n_ct = cols / TK;
  const int64_t plim = min(padded[G], P);
  const int64_t live = (plim + TP - 1) / TP * n_ct;
  if ((int64_t)blockIdx.x >= live) return;  // uniform per workgroup
  const int64_t t_idx = xcd_band(blockIdx.x, live);
  const int64_t p0 = (t_idx / n_ct) * TP;
  const int64_t k0 = (t_idx % n_ct) * TK;

  if (tid < TP) {
    const int64_t p = p0 + tid;
    int64_t r = -1;
    if (p < plim) {
      int lo = 0, hi = G;  // last g with padded[g] <= p
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (padded[mid] <= p) lo = mid; else hi = mid;
      }
      const int64_t i = p - padded[lo];
      if (i < offsets[lo + 1] - offsets[lo]) r = offsets[lo] + i;
      grp_of[tid] = lo;
    } else {
      grp_of[tid] = 0;
    }
    row_of[tid] = r;
  }
  __syncthreads();

  // ---- stage the input rows of this tile
  if constexpr (S == Src::NVFP4) {
    const uint8_t* codes = static_cast<const uint8_t*>(src);
    {  // 64 code bytes per row: 2 threads x 32 bytes
      const int t = tid >> 1, h = tid & 1;
      const int64_t r = row_of[t];
      uint4 a = make_uint4(0, 0, 0, 0), b = a;
      if (r >= 0) {
        const uint4* g = reinterpret_cast<const uint4*>(codes + r * (cols / 2) + k0 / 2 + h * 32);
        a = ld_stream16(g);
        b = ld_stream16(g + 1);
      }
      uint2* d = reinterpret_cast<uint2*>(&tile.codes[slot_of(t) * Tile<S>::CW + 8 * h]);
      d[0] = make_uint2(a.x, a.y); d[1] = make_uint2(a.z, a.w);
      d[2] = make_uint2(b.x, b.y); d[3] = make_uint2(b.z, b.w);
    }
    if (tid < TP) {
      const int64_t r = row_of[tid];
      uint2 sc = make_uint2(0, 0);
      float o = 0.0f;
      if (r >= 0) {
        sc = *reinterpret_cast<const uint2*>(src_scales + r * (cols / 16) + k0 / 16);
        o = src_outer[rpg ? r / rpg : r];
      }
      const int sl = slot_of(tid);
      tile.scales[sl][0] = sc.x;
      tile.scales[sl][1] = sc.y;
      tile.outer[sl] = o;
    }
  } else {
    constexpr int EB = (S == Src::BF16) ? 2 : 4;        // bytes per element
    constexpr int V16 = TK * EB / 16;                   // 16-byte vectors per row
    constexpr int NV = TP * V16 / 256;                  // vectors per thread
    // all of the thread's loads are issued before any is stored
    uint4 a[NV];
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      const int i = tid + 256 * n;
      const int t = i / V16, c = i % V16;
      const int64_t r = row_of[t];
      a[n] = r >= 0 ? ld_stream16(reinterpret_cast<const uint4*>(
                          static_cast<const uint8_t*>(src) + (r * cols + k0) * EB) + c)
                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      const int i = tid + 256 * n;
      const int t = i / V16, c = i % V16;
      *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(&tile.v[slot_of(t)][0]) + c * 16) =
          a[n];
    }
  }
  __syncthreads();

  if constexpr (ROWS && S != Src::NVFP4) {
    // row-wise pass over the staged tile: lane l takes 8 columns (chunk l % 16)
    // of token (l / 16) + 16 it; the four lanes of a quad hold one 32-column
    // block. Same exponent rule and rounding as the row-wise kernel.
    const int c = tid & 15;
#pragma unroll 2
    for (int it = 0; it < 8; ++it) {
      const int t = (tid >> 4) + 16 * it;
      const int64_t r = row_of[t];
      float v[8];
      if constexpr (S == Src::BF16) {
        const uint4 a = *reinterpret_cast<const uint4*>(&tile.v[slot_of(t)][8 * c]);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[2 * j] = u2f(w[j] << 16);
          v[2 * j + 1] = u2f(w[j] & 0xFFFF0000u);
        }
      } else {
        const float4 a = *reinterpret_cast<const float4*>(&tile.v[slot_of(t)][8 * c]);
        const float4 b = *reinterpret_cast<const float4*>(&tile.v[slot_of(t)][8 * c + 4]);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      }
      float mf = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) mf = fmaxf(mf, fabsf(v[j]));
      const uint32_t code = e8m0_code_bits(quad_max_bits(f2u(mf)));
      const float scale = u2f(code << 23);
      const uint32_t lo = e4m3x4_rne_scaled(v[0], v[1], v[2], v[3], scale);
      const uint32_t hi = e4m3x4_rne_scaled(v[4], v[5], v[6], v[7], scale);
      if (r >= 0) {
        *reinterpret_cast<uint2*>(row_out + r * cols + k0 + 8 * c) = make_uint2(lo, hi);
        if ((c & 3) == 0) row_e8[r * (cols / 32) + (k0 + 8 * c) / 32] = (uint8_t)code;
      }
    }
  }

  // ---- micro-tile: 8 columns x 8 tokens per thread
  const int pc = tid & 15;   // token chunk: tokens 8*pc .. 8*pc+7 of the tile
  const int kc = tid >> 4;   // column chunk: columns 8*kc .. 8*kc+7
  float v[8][8];             // [column][token]
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int sl = 16 * i + pc;            // slot of token 8*pc + i
    if constexpr (S == Src::NVFP4) {
      const uint32_t w = tile.codes[sl * Tile<S>::CW + kc];
      // E4M3 scale of the 16-block holding these 8 columns (exact decode)
      const uint32_t sb = reinterpret_cast<const uint8_t*>(tile.scales[sl])[kc >> 1];
      const float Sb = __builtin_amdgcn_cvt_f32_fp8((int)sb, 0);
      const float o = tile.outer[sl];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float e0, e1;
        e2m1x2_to_f32(w, j, e0, e1);
        v[2 * j][i] = __fmul_rn(__fmul_rn(e0, Sb), o);       // e2m1 * S is exact
        v[2 * j + 1][i] = __fmul_rn(__fmul_rn(e1, Sb), o);
      }
    } else if constexpr (S == Src::BF16) {
      const uint4 a = *reinterpret_cast<const uint4*>(&tile.v[sl][8 * kc]);
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j][i] = u2f(w[j] << 16);
        v[2 * j + 1][i] = u2f(w[j] & 0xFFFF0000u);
      }
    } else {
      const float4 a = *reinterpret_cast<const float4*>(&tile.v[sl][8 * kc]);
      const float4 b = *reinterpret_cast<const float4*>(&tile.v[sl][8 * kc + 4]);
      v[0][i] = a.x; v[1][i] = a.y; v[2][i] = a.z; v[3][i] = a.w;
      v[4][i] = b.x; v[5][i] = b.y; v[6][i] = b.z; v[7][i] = b.w;
    }
  }

  const int64_t p = p0 + 8 * pc;                 // first output column of this thread
  const bool live_p = p < plim;                  // whole 8-chunk shares liveness
  if constexpr (NVO) {
    // 16-token blocks: this lane and its neighbour (pc ^ 1) hold one block
    const int g = grp_of[8 * pc];
    const float sg = __fdiv_rn(u2f(gbits[g]), 2688.0f);
    const float dg = __fmul_rn(6.0f, sg);
    const int64_t kt = k0 + 8 * kc;              // first output row of this thread
    int64_t lin, step;                           // linear index of (kt, p), per output row
    if constexpr (BLK) {
      const int64_t pg = padded[g], glen = padded[g + 1] - pg;
      lin = (int64_t)g * cols * glen + kt * glen + (p - pg);
      step = glen;
    } else {
      lin = kt * P + p;
      step = P;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float mf = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) mf = fmaxf(mf, fabsf(v[j][i]));
      uint32_t mb = f2u(mf);
      mb = max(mb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0xB1, 0xF, 0xF, true));
      const uint32_t sc = sg > 0.0f ? e4m3_ceil_pos(__fdiv_rn(u2f(mb), dg)) : 0u;
      uint32_t w = 0;
      if (sc) {
        const float r = __fdiv_rn(1.0f, __fmul_rn(e4m3_pos_to_f32(sc), sg));
        const Draws8 u = draws8((uint64_t)(lin >> 3), seed, tag);
        float y[8];
        uint32_t uu[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          y[i] = __fmul_rn(v[j][i], r);
          uu[i] = u.get(i);
        }
        w = e2m1x8_sr(y, uu);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) w |= ((f2u(v[j][i]) >> 28) & 8u) << (4 * i);
      }
      if (live_p) {
        *reinterpret_cast<uint32_t*>(out + (lin >> 1)) = w;
        if ((pc & 1) == 0) out_e8[lin >> 4] = (uint8_t)sc;
      }
      lin += step;
    }
    return;
  }
  const int64_t kt = k0 + 8 * kc;                // first output row of this thread
  // output position: [cols, P], or with BLK group g's block [cols, glen] at
  // cols * padded[g] (a 32-token chunk never straddles groups); the draw index
  // is the [cols, P] position either way
  int64_t ostep, estep;
  uint8_t* o8;
  uint8_t* oe;
  if constexpr (BLK) {
    const int g = grp_of[8 * pc];
    const int64_t pg = padded[g], glen = padded[g + 1] - pg;
    ostep = glen;
    estep = glen / 32;
    o8 = out + cols * pg + kt * glen + (p - pg);
    oe = out_e8 + cols * (pg / 32) + kt * estep + ((p - pg) >> 5);
  } else {
    ostep = P;
    estep = P / 32;
    o8 = out + kt * P + p;
    oe = out_e8 + kt * estep + (p >> 5);
  }
  uint64_t q = (uint64_t)kt * (uint64_t)(P >> 3) + (uint64_t)(p >> 3);   // Philox counter
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float mf = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) mf = fmaxf(mf, fabsf(v[j][i]));
    const uint32_t m = quad_max_bits(f2u(mf));
    const uint32_t code = e8m0_code_bits(m);
    const float scale = u2f(code << 23);         // 2^(code - 127)
    uint32_t lo, hi;
    if constexpr (SR) {
      const Draws8 u = draws8(q, seed, tag);
      lo = e4m3x4_sr_scaled(v[j][0], v[j][1], v[j][2], v[j][3], u.w[0] << 16,
                            u.w[0] & 0xFFFF0000u, u.w[1] << 16, u.w[1] & 0xFFFF0000u, scale);
      hi = e4m3x4_sr_scaled(v[j][4], v[j][5], v[j][6], v[j][7], u.w[2] << 16,
                            u.w[2] & 0xFFFF0000u, u.w[3] << 16, u.w[3] & 0xFFFF0000u, scale);
    } else {
      lo = e4m3x4_rne_scaled(v[j][0], v[j][1], v[j][2], v[j][3], scale);
      hi = e4m3x4_rne_scaled(v[j][4], v[j][5], v[j][6], v[j][7], scale);
    }
    if (live_p) {
      *reinterpret_cast<uint2*>(o8) = make_uint2(lo, hi);
      if ((pc & 3) == 0) *oe = (uint8_t)code;
    }
    o8 += ostep;
    oe += estep;
    q += (uint64_t)(P >> 3);
  }
}

template <Src S, bool SR, bool ROWS = false, bool NV = false, bool BLK = false>
hipError_t run(const void* src, const uint8_t* sc, const float* so, int64_t rpg, int64_t rows,
               int64_t cols, const int64_t* offsets, const int64_t* padded, int G, int64_t P,
               uint64_t seed, uint32_t tag, uint8_t* out, uint8_t* out_e8, hipStream_t stream,
               uint8_t* row_out = nullptr, uint8_t* row_e8 = nullptr,
               const uint32_t* gbits = nullptr) {
  (void)rows;
  if (P == 0 || cols == 0 || G == 0) return hipSuccess;
  const int64_t grid = (P + TP - 1) / TP * (cols / TK);
  k_transpose_mx<S, SR, ROWS, NV, BLK><<<(unsigned)grid, 256, 0, stream>>>(
      src, sc, so, rpg, cols, offsets, padded, G, P, seed, tag, out, out_e8, row_out, row_e8,
      gbits);
  return hipGetLastError();
}

// NVFP4 output: row maxima into out (free until the transpose writes it),
// group maxima into out_outer, the transpose, maxima into outer scales.
template <Src S, bool BLK>
hipError_t run_nv(const void* src, const uint8_t* sc, const float* so, int64_t rpg, int64_t cols,
                  const int64_t* offsets, const int64_t* padded, int G, int64_t P, uint64_t seed,
                  uint32_t tag, uint8_t* out, uint8_t* out_sc, float* out_outer,
                  int64_t m_cap, hipStream_t stream) {
  if (G == 0) return hipSuccess;
  uint32_t* bits = reinterpret_cast<uint32_t*>(out_outer);
  uint32_t* row_bits = reinterpret_cast<uint32_t*>(out);
  if (cols > 0 && m_cap > 0) {
    int64_t grid = (m_cap + 15) / 16;         // four rows per wavefront and round
    const int64_t most = (int64_t)device_cu_count() * 8;
    if (grid > most) grid = most;
    k_row_amax<S><<<(unsigned)grid, 256, 0, stream>>>(src, sc, so, rpg, cols, offsets, G,
                                                      row_bits);
    k_group_max<<<(unsigned)G, 256, 0, stream>>>(row_bits, offsets, bits);
  } else {
    k_zero_u32<<<(unsigned)((G + 255) / 256), 256, 0, stream>>>(bits, G);
  }
  hipError_t e = run<S, true, false, true, BLK>(src, sc, so, rpg, 0, cols, offsets, padded, G, P,
                                                seed, tag, out, out_sc, stream, nullptr, nullptr,
                                                bits);
  if (e != hipSuccess) return e;
  k_bits_to_outer<<<(unsigned)((G + 255) / 256), 256, 0, stream>>>(out_outer, G);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_requant_sr(const uint8_t* codes, const uint8_t* scales, const float* outer,
                             int64_t rpg, int64_t rows, int64_t cols, const int64_t* offsets,
                             const int64_t* padded, int G, int64_t P, bool blocked, uint64_t seed,
                             uint32_t tag, uint8_t* out, uint8_t* out_e8, hipStream_t stream) {
  if (blocked)
    return run<Src::NVFP4, true, false, false, true>(codes, scales, outer, rpg, rows, cols,
                                                     offsets, padded, G, P, seed, tag, out,
                                                     out_e8, stream);
  return run<Src::NVFP4, true>(codes, scales, outer, rpg, rows, cols, offsets, padded, G, P, seed,
                               tag, out, out_e8, stream);
}

hipError_t launch_nvfp4_requant_sr(const uint8_t* codes, const uint8_t* scales,
                                   const float* outer, int64_t rpg, int64_t rows, int64_t cols,
                                   const int64_t* offsets, const int64_t* padded, int G, int64_t P,
                                   bool blocked, uint64_t seed, uint32_t tag, uint8_t* out,
                                   uint8_t* out_sc, float* out_outer, hipStream_t stream) {
  if (blocked)
    return run_nv<Src::NVFP4, true>(codes, scales, outer, rpg, cols, offsets, padded, G, P, seed,
                                    tag, out, out_sc, out_outer, rows, stream);
  return run_nv<Src::NVFP4, false>(codes, scales, outer, rpg, cols, offsets, padded, G, P, seed,
                                   tag, out, out_sc, out_outer, rows, stream);
}

hipError_t launch_nvfp4_quantize_sr_colwise(const void* x, bool bf16, int64_t rows,
                                            int64_t cols, const int64_t* offsets,
                                            const int64_t* padded, int G, int64_t P,
                                            uint64_t seed, uint32_t tag, uint8_t* out,
                                            uint8_t* out_sc, float* out_outer,
                                            hipStream_t stream) {
  if (bf16)
    return run_nv<Src::BF16, false>(x, nullptr, nullptr, 0, cols, offsets, padded, G, P, seed,
                                    tag, out, out_sc, out_outer, rows, stream);
  return run_nv<Src::F32, false>(x, nullptr, nullptr, 0, cols, offsets, padded, G, P, seed, tag,
                                 out, out_sc, out_outer, rows, stream);
}

hipError_t launch_mxfp8_quantize_colwise(const void* x, bool bf16, int64_t rows, int64_t cols,
                                         const int64_t* offsets, const int64_t* padded, int G,
                                         int64_t P, uint8_t* out, uint8_t* out_e8,
                                         hipStream_t stream) {
  if (bf16)
    return run<Src::BF16, false>(x, nullptr, nullptr, 0, rows, cols, offsets, padded, G, P, 0, 0,
                                 out, out_e8, stream);
  return run<Src::F32, false>(x, nullptr, nullptr, 0, rows, cols, offsets, padded, G, P, 0, 0,
                              out, out_e8, stream);
}

hipError_t launch_mxfp8_quantize_dual(const void* x, bool bf16, int64_t rows, int64_t cols,
                                      const int64_t* offsets, const int64_t* padded, int G,
                                      int64_t P, uint8_t* row_out, uint8_t* row_e8, uint8_t* out,
                                      uint8_t* out_e8, hipStream_t stream) {
  if (bf16)
    return run<Src::BF16, false, true>(x, nullptr, nullptr, 0, rows, cols, offsets, padded, G, P,
                                       0, 0, out, out_e8, stream, row_out, row_e8);
  return run<Src::F32, false, true>(x, nullptr, nullptr, 0, rows, cols, offsets, padded, G, P, 0,
                                    0, out, out_e8, stream, row_out, row_e8);
}

}  // namespace nvfp4moe
