// NVFP4 forward grouped GEMM on gfx950.
//
// Pages: the expert-layer forward matmuls run in NVFP4 ("Inkling 2 Small uses
// four-bit training ...", section "NVFP4 forward, MXFP8 backward").
//
// Numerics. An NVFP4 element is e2m1 * S with S an E4M3 scale shared by 16
// elements; the product has up to 6 significant bits. gfx950's block-scaled
// MFMA takes 4-bit elements with one power-of-two (E8M0) scale per 32, so it
// cannot carry the E4M3 mantissa of a per-16 scale exactly. The kernel
// therefore dequantizes each element to f16 (11 significant bits, range
// 2^-14..65504: every e2m1 * S is exact) right before the MFMA and runs
// v_mfma_f32_32x32x16_f16: exact products, float32 accumulation. The per-row
// and per-expert outer scales are applied in the epilogue:
//   y = (acc * s_x[row]) * s_w[g].
//
// Structure. Workgroup tile BM x BN (tokens x outputs) of one expert; the
// tile list is implicit: blockIdx.y walks the experts' m-tiles in order
// (sum over g of ceil(M_g / BM) <= ceil(m_cap / BM) + G), blockIdx.x is the
// n-tile. NVFP4 bytes (not dequantized values) are staged in LDS, double
// buffered, so HBM and LDS traffic stay at 4.5 bits per element. Each lane
// reads one whole 16-element block (8 bytes + its scale) per A/B fragment and
// turns it into the operands of two consecutive K=16 MFMAs: lanes 0-31 take
// block 2j, lanes 32-63 block 2j+1, first their low 8 elements, then their
// high 8. A and B use the same permutation of k, so the sum is unchanged.
#include "codecs.hpp"
#include "internal.hpp"

namespace nvfp4moe {

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 128;   // BK in elements (8 NVFP4 blocks)
constexpr int CP = BK / 2 + 8;                // staged code bytes per row (+pad, 8B aligned)
constexpr int SP = BK / 16;                   // staged scale bytes per row
constexpr int WM = 2, WN = 2;                 // 32x32 MFMA tiles per wave (rows, cols)

struct Stage {
  uint8_t a[BM][CP];
  uint8_t b[BN][CP];
  uint8_t as[BM][SP];
  uint8_t bs[BN][SP];
};

// 16 E2M1 codes (8 bytes) times one E4M3 scale -> two f16x8 MFMA operands
// (elements 0..7 and 8..15). The products are exact in f16.
__device__ __forceinline__ void dequant16(uint2 w, uint32_t scode, f16x8& lo, f16x8& hi) {
  const _Float16 S = (_Float16)e4m3_pos_to_f32(scode);  // exact
  const f16x2 s2 = {S, S};
  f16x2 p[8];
  p[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.x, 1.0f, 0);
  p[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.x, 1.0f, 1);
  p[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.x, 1.0f, 2);
  p[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.x, 1.0f, 3);
  p[4] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.y, 1.0f, 0);
  p[5] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.y, 1.0f, 1);
  p[6] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.y, 1.0f, 2);
  p[7] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.y, 1.0f, 3);
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = p[i] * s2;
  lo = f16x8{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
  hi = f16x8{p[4][0], p[4][1], p[5][0], p[5][1], p[6][0], p[6][1], p[7][0], p[7][1]};
}

// Locate virtual m-tile vt among the experts' tiles. Returns false when vt is
// past the last real tile.
__device__ __forceinline__ bool find_tile(const int64_t* __restrict__ offsets, int G, int64_t vt,
                                          int bm, int& g, int64_t& row0, int64_t& row_end) {
  for (int e = 0; e < G; ++e) {
    const int64_t a = offsets[e], b = offsets[e + 1];
    const int64_t nt = (b - a + bm - 1) / bm;
    if (vt < nt) {
      g = e;
      row0 = a + vt * bm;
      row_end = b;
      return true;
    }
    vt -= nt;
  }
  return false;
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_fwd(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const float* __restrict__ ao,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, const float* __restrict__ bo,
    const int64_t* __restrict__ offsets, int G, int64_t N, int64_t K, void* __restrict__ y) {
  __shared__ Stage st[2];

  int g;
  int64_t row0, row_end;
  if (!find_tile(offsets, G, blockIdx.y, BM, g, row0, row_end)) return;
  const int64_t n0 = (int64_t)blockIdx.x * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;   // 2x2 waves, each 64x64

  const int64_t KB = K / 2;    // code bytes per row
  const int64_t KS = K / 16;   // scale bytes per row

  // global -> register staging: thread t loads 32 code bytes of A row t/2 and
  // of B row t/2 (half t&1), and 8 scale bytes of A (t < 128) or B row.
  const int lr = tid >> 1, lh = tid & 1;
  const int64_t arow = row0 + lr;
  const bool aok = arow < row_end;
  const uint8_t* ag = ac + (aok ? arow : 0) * KB + lh * 32;
  const uint8_t* bg = bc + ((int64_t)g * N + n0 + lr) * KB + lh * 32;
  const int sr = tid & 127;
  const bool s_is_a = tid < 128;
  const int64_t srow = s_is_a ? row0 + sr : (int64_t)g * N + n0 + sr;
  const bool sok = s_is_a ? (srow < row_end) : true;
  const uint8_t* sg = (s_is_a ? as : bs) + (sok ? srow : 0) * KS;

  uint4 ra0, ra1, rb0, rb1;
  uint2 rs;
  auto gload = [&](int64_t kt) {
    const int64_t cb = kt * (BK / 2);
    if (aok) {
      ra0 = *reinterpret_cast<const uint4*>(ag + cb);
      ra1 = *reinterpret_cast<const uint4*>(ag + cb + 16);
    } else {
      ra0 = ra1 = make_uint4(0, 0, 0, 0);
    }
    rb0 = *reinterpret_cast<const uint4*>(bg + cb);
    rb1 = *reinterpret_cast<const uint4*>(bg + cb + 16);
    rs = sok ? *reinterpret_cast<const uint2*>(sg + kt * SP) : make_uint2(0, 0);
  };
  auto sstore = [&](Stage& s) {
    uint2* da = reinterpret_cast<uint2*>(&s.a[lr][lh * 32]);
    da[0] = make_uint2(ra0.x, ra0.y); da[1] = make_uint2(ra0.z, ra0.w);
    da[2] = make_uint2(ra1.x, ra1.y); da[3] = make_uint2(ra1.z, ra1.w);
    uint2* db = reinterpret_cast<uint2*>(&s.b[lr][lh * 32]);
    db[0] = make_uint2(rb0.x, rb0.y); db[1] = make_uint2(rb0.z, rb0.w);
    db[2] = make_uint2(rb1.x, rb1.y); db[3] = make_uint2(rb1.z, rb1.w);
    *reinterpret_cast<uint2*>(s_is_a ? &s.as[sr][0] : &s.bs[sr][0]) = rs;
  };

  f32x16 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int64_t nk = K / BK;
  gload(0);
  sstore(st[0]);
  __syncthreads();

  const int half = lane >> 5;      // which block of a pair this lane dequantizes
  const int r32 = lane & 31;
  for (int64_t kt = 0; kt < nk; ++kt) {
    Stage& cur = st[kt & 1];
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kp = 0; kp < BK / 32; ++kp) {     // pairs of NVFP4 blocks
      const int blk = 2 * kp + half;
      f16x8 alo[WM], ahi[WM], blo[WN], bhi[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const int r = wm * 64 + i * 32 + r32;
        const uint2 w = *reinterpret_cast<const uint2*>(&cur.a[r][blk * 8]);
        dequant16(w, cur.as[r][blk], alo[i], ahi[i]);
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int c = wn * 64 + j * 32 + r32;
        const uint2 w = *reinterpret_cast<const uint2*>(&cur.b[c][blk * 8]);
        dequant16(w, cur.bs[c][blk], blo[j], bhi[j]);
      }
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[i], blo[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[i], bhi[j], acc[i][j], 0, 0, 0);
        }
    }
    if (kt + 1 < nk) {
      sstore(st[(kt + 1) & 1]);
    }
    __syncthreads();
  }

  // epilogue: lane holds column (lane & 31) and rows 8*q + 4*half + v
  const float sw = bo[g];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + r32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = row0 + wm * 64 + i * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
        if (row < row_end) {
          const float v = __fmul_rn(__fmul_rn(acc[i][j][e], ao[row]), sw);
          if constexpr (OUT_BF16)
            static_cast<uint16_t*>(y)[row * N + col] = (uint16_t)f32_to_bf16_rne(v);
          else
            static_cast<float*>(y)[row * N + col] = v;
        }
      }
    }
}

}  // namespace

hipError_t launch_fwd_grouped_gemm(const uint8_t* ac, const uint8_t* as, const float* ao,
                                   const uint8_t* bc, const uint8_t* bs, const float* bo,
                                   const int64_t* offsets, int G, int64_t m_cap, int64_t N,
                                   int64_t K, void* y, bool y_bf16, hipStream_t stream) {
  if (m_cap == 0 || G == 0) return hipSuccess;
  const dim3 grid((unsigned)(N / BN), (unsigned)((m_cap + BM - 1) / BM + G));
  if (y_bf16)
    k_fwd<true><<<grid, 256, 0, stream>>>(ac, as, ao, bc, bs, bo, offsets, G, N, K, y);
  else
    k_fwd<false><<<grid, 256, 0, stream>>>(ac, as, ao, bc, bs, bo, offsets, G, N, K, y);
  return hipGetLastError();
}

}  // namespace nvfp4moe
