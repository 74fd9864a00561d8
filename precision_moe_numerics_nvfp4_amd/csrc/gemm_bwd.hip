// MXFP8 dgrad and wgrad grouped GEMMs on gfx950's block-scaled MFMA.
//
// Pages: the backward pass computes gradients with MXFP8 matmuls on the
// re-quantized saved tensors ("Inkling 2 Small uses four-bit training ...",
// sections "NVFP4 forward, MXFP8 backward" and "Stochastic rounding across
// transposes").
//
// MXFP8 (E4M3 elements, one E8M0 power of two per 32 along the contraction)
// is exactly the operand format of v_mfma_scale_f32_32x32x64_f8f6f4: each of
// its two 32-element k-blocks per row takes one E8M0 byte, so products are
// exact and accumulation is float32.
// Both GEMMs are "row x row" contractions: each operand is stored with the
// contraction dimension contiguous (that is what the re-quantization's
// transpose is for), so one main loop serves both:
//   dgrad: dX[r, k]    = sum_n dY8[r, n] * W8[k, g*N + n]    (rows r of expert g)
//   wgrad: dW[g, n, k] = sum_p dYT8[n, p] * XT8[k, p]        (p in g's padded segment)
// Workgroup tile 128 x 128, four wavefronts of 64 x 64 (2 x 2 MFMA tiles),
// 128 contraction elements (4 MX blocks) per double-buffered LDS stage.
// Contraction ranges are multiples of 32; a partial last stage is zero-filled.
#include "codecs.hpp"
#include "internal.hpp"

namespace nvfp4moe {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int RP = BK + 16;   // staged bytes per row (+pad)
constexpr int SPB = BK / 32;  // scale bytes per row per stage

struct Stage {
  uint8_t a[BM][RP];
  uint8_t b[BN][RP];
  uint8_t as[BM][SPB];
  uint8_t bs[BN][SPB];
};

struct Operand {
  const uint8_t* q;    // elements, row-major
  const uint8_t* e;    // E8M0 scales, row-major
  int64_t ld;          // elements per row (bytes)
  int64_t c0;          // first contraction element of this tile
  int64_t row0;        // first row of the tile
  int64_t row_end;     // rows >= row_end are zero
};

// acc[i][j] += A[64 rows of wave] x B[64 rows of wave]^T over L contraction elements.
__device__ __forceinline__ void mainloop(Stage* st, const Operand& A, const Operand& B, int64_t L,
                                         f32x16 (&acc)[2][2]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // thread t stages 64 bytes (4 x 16) of A row t/2 and of B row t/2, half t&1,
  // and the 4 scale bytes of A row t (t < 128) or B row t-128.
  const int lr = tid >> 1, lh = tid & 1;
  const int64_t arow = A.row0 + lr;
  const bool aok = arow < A.row_end;
  const uint8_t* ag = A.q + (aok ? arow : 0) * A.ld + A.c0 + lh * 64;
  const int64_t brow = B.row0 + lr;
  const bool bok = brow < B.row_end;
  const uint8_t* bg = B.q + (bok ? brow : 0) * B.ld + B.c0 + lh * 64;
  const int sr = tid & 127;
  const bool s_is_a = tid < 128;
  const Operand& SO = s_is_a ? A : B;
  const int64_t srow = SO.row0 + sr;
  const bool sok = srow < SO.row_end;
  const uint8_t* sg = SO.e + (sok ? srow : 0) * (SO.ld / 32) + SO.c0 / 32;

  uint4 ra[4], rb[4];
  uint32_t rs;
  auto gload = [&](int64_t kt) {
    const int64_t c = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = (c + lh * 64 + i * 16) < L;     // L is a multiple of 32
      ra[i] = (aok && in) ? *reinterpret_cast<const uint4*>(ag + c + i * 16) : make_uint4(0, 0, 0, 0);
      rb[i] = (bok && in) ? *reinterpret_cast<const uint4*>(bg + c + i * 16) : make_uint4(0, 0, 0, 0);
    }
    rs = 0;
    if (sok) {
#pragma unroll
      for (int i = 0; i < SPB; ++i)
        if (c + 32 * i < L) rs |= (uint32_t)sg[kt * SPB + i] << (8 * i);
    }
  };
  auto sstore = [&](Stage& s) {
    uint4* da = reinterpret_cast<uint4*>(&s.a[lr][lh * 64]);
    uint4* db = reinterpret_cast<uint4*>(&s.b[lr][lh * 64]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      da[i] = ra[i];
      db[i] = rb[i];
    }
    *reinterpret_cast<uint32_t*>(s_is_a ? &s.as[sr][0] : &s.bs[sr][0]) = rs;
  };

  const int64_t nk = (L + BK - 1) / BK;
  if (nk == 0) return;
  gload(0);
  sstore(st[0]);
  __syncthreads();
  const int half = lane >> 5;
  const int r32 = lane & 31;
  for (int64_t kt = 0; kt < nk; ++kt) {
    Stage& cur = st[kt & 1];
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 64; ++ks) {
      // Operand layout of the 64-deep block-scaled MFMA: lane l supplies
      // elements 16*(l/32) .. +15 of the step's MX block 0 in bytes 0-15 and
      // the same elements of MX block 1 in bytes 16-31; its scale byte is the
      // one of row l%32, MX block l/32.
      const int blk = 2 * ks + half;           // MX block of this lane's scale
      i32x8 af[2], bf[2];
      int32_t asc[2], bsc[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + r32;
        const uint4 x0 = *reinterpret_cast<const uint4*>(&cur.a[r][ks * 64 + half * 16]);
        const uint4 x1 = *reinterpret_cast<const uint4*>(&cur.a[r][ks * 64 + 32 + half * 16]);
        af[i] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                      (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        asc[i] = cur.as[r][blk];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = wn * 64 + j * 32 + r32;
        const uint4 x0 = *reinterpret_cast<const uint4*>(&cur.b[c][ks * 64 + half * 16]);
        const uint4 x1 = *reinterpret_cast<const uint4*>(&cur.b[c][ks * 64 + 32 + half * 16]);
        bf[j] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                      (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        bsc[j] = cur.bs[c][blk];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af[i], bf[j], acc[i][j], 0 /*A: E4M3*/, 0 /*B: E4M3*/, 0, asc[i], 0, bsc[j]);
    }
    if (kt + 1 < nk) sstore(st[(kt + 1) & 1]);
    __syncthreads();
  }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_dgrad(const uint8_t* __restrict__ dy,
                                               const uint8_t* __restrict__ dye,
                                               const uint8_t* __restrict__ w,
                                               const uint8_t* __restrict__ we,
                                               const int64_t* __restrict__ offsets, int G,
                                               int64_t N, int64_t K, void* __restrict__ dx) {
  __shared__ Stage st[2];
  // virtual m-tile -> (expert, first row)
  int64_t vt = blockIdx.y;
  int g = -1;
  int64_t row0 = 0, row_end = 0;
  for (int e = 0; e < G; ++e) {
    const int64_t a = offsets[e], b = offsets[e + 1];
    const int64_t nt = (b - a + BM - 1) / BM;
    if (vt < nt) {
      g = e;
      row0 = a + vt * BM;
      row_end = b;
      break;
    }
    vt -= nt;
  }
  if (g < 0) return;
  const int64_t k0 = (int64_t)blockIdx.x * BN;
  Operand A{dy, dye, N, 0, row0, row_end};
  Operand B{w, we, (int64_t)G * N, (int64_t)g * N, k0, k0 + BN};
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  mainloop(st, A, B, N, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, half = lane >> 5;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = k0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = row0 + wm * 64 + i * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
        if (row < row_end) {
          if constexpr (OUT_BF16)
            static_cast<uint16_t*>(dx)[row * K + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][e]);
          else
            static_cast<float*>(dx)[row * K + col] = acc[i][j][e];
        }
      }
    }
}

__global__ __launch_bounds__(256) void k_wgrad(const uint8_t* __restrict__ dyT,
                                               const uint8_t* __restrict__ dyTe,
                                               const uint8_t* __restrict__ xT,
                                               const uint8_t* __restrict__ xTe,
                                               const int64_t* __restrict__ padded, int64_t P,
                                               int64_t N, int64_t K, float* __restrict__ dw) {
  __shared__ Stage st[2];
  const int g = blockIdx.z;
  const int64_t n0 = (int64_t)blockIdx.x * BM;
  const int64_t k0 = (int64_t)blockIdx.y * BN;
  const int64_t c0 = padded[g];
  const int64_t L = padded[g + 1] - c0;
  Operand A{dyT, dyTe, P, c0, n0, n0 + BM};
  Operand B{xT, xTe, P, c0, k0, k0 + BN};
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  mainloop(st, A, B, L, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, half = lane >> 5;
  float* out = dw + (int64_t)g * N * K;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = k0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = n0 + wm * 64 + i * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
        out[row * K + col] = acc[i][j][e];
      }
    }
}

}  // namespace

hipError_t launch_dgrad(const uint8_t* dy, const uint8_t* dye, const uint8_t* w,
                        const uint8_t* we, const int64_t* offsets, int G, int64_t m_cap,
                        int64_t N, int64_t K, void* dx, bool dx_bf16, hipStream_t stream) {
  if (m_cap == 0 || G == 0) return hipSuccess;
  const dim3 grid((unsigned)(K / BN), (unsigned)((m_cap + BM - 1) / BM + G));
  if (dx_bf16)
    k_dgrad<true><<<grid, 256, 0, stream>>>(dy, dye, w, we, offsets, G, N, K, dx);
  else
    k_dgrad<false><<<grid, 256, 0, stream>>>(dy, dye, w, we, offsets, G, N, K, dx);
  return hipGetLastError();
}

hipError_t launch_wgrad(const uint8_t* dyT, const uint8_t* dyTe, const uint8_t* xT,
                        const uint8_t* xTe, const int64_t* padded, int G, int64_t P, int64_t N,
                        int64_t K, float* dw, hipStream_t stream) {
  if (G == 0) return hipSuccess;
  const dim3 grid((unsigned)(N / BM), (unsigned)(K / BN), (unsigned)G);
  k_wgrad<<<grid, 256, 0, stream>>>(dyT, dyTe, xT, xTe, padded, P, N, K, dw);
  return hipGetLastError();
}

}  // namespace nvfp4moe
