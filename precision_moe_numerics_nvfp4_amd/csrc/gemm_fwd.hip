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
// 2^-14..65504: every e2m1 * S is exact) and runs v_mfma_f32_32x32x16_f16:
// exact products, float32 accumulation. The per-row and per-expert outer
// scales are applied in the epilogue: y = (acc * s_x[row]) * s_w[g].
//
// Structure (large tiles). A workgroup of 4 wavefronts owns a 256 x 256 tile
// (tokens x outputs) of one expert; each wavefront owns 128 x 128 (4 x 4 MFMA
// tiles, 256 accumulator registers). The K loop moves 64 elements per stage:
// every thread loads its share of the stage's NVFP4 bytes from HBM one stage
// ahead, dequantizes them once per workgroup (v_cvt_scalef32_pk_f16_fp4 with
// a unit scale, then an exact v_pk_mul_f16 by the block's E4M3 scale) and
// stores f16 into a double-buffered LDS tile whose 16-byte chunks are
// XOR-swizzled by row, so the fragment reads (ds_read_b128, 32 rows at one
// k offset) spread over the banks. HBM traffic stays at 4.5 bits per element.
//
// Tile order. Tiles are enumerated expert by expert, n-tile by n-tile, m-tile
// fastest, and only the live ones (sum over g of ceil(M_g/BM) * N/BN, read
// from the device offsets) are handed out; workgroup w goes to XCD w % 8, so
// the live tiles are split into 8 contiguous ranges, one per XCD, and the
// workgroups running together on one XCD share B (weight) tiles in its L2.
//
// Small groups (decode: a few rows per expert) use a 32-row variant in which
// the four wavefronts split N instead of M.
#include "codecs.hpp"
#include "internal.hpp"

namespace nvfp4moe {

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 64;                 // K elements per stage (4 NVFP4 blocks)

// 32 codes (16 bytes, two NVFP4 blocks) times their two E4M3 scales -> 32 f16
// (four 16-byte chunks). Products are exact in f16.
__device__ __forceinline__ void dequant32(const uint4 w, uint32_t s2, u32x4 out[4]) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const _Float16 S = (_Float16)e4m3_pos_to_f32((s2 >> (8 * blk)) & 0xFFu);  // exact
    const f16x2 s = {S, S};
#pragma unroll
    for (int h = 0; h < 2; ++h) {            // 8 elements = one 16-byte chunk
      const uint32_t x = wd[2 * blk + h];
      f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 0) * s;
      f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 1) * s;
      f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2) * s;
      f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 3) * s;
      out[2 * blk + h] = u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                               __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
    }
  }
}

// f16 element offset of 16-byte chunk c (0..7) of LDS row `row` (64 f16 per row)
__device__ __forceinline__ int swz(int row, int c) { return row * BK + ((c ^ (row & 7)) << 3); }

// Live tile t -> (expert, first row, row end, n-tile). Tiles: expert-major,
// then n-tile, then m-tile.
__device__ __forceinline__ bool tile_of(const int64_t* __restrict__ offsets, int G, int64_t t,
                                        int bm, int64_t ntn, int& g, int64_t& row0,
                                        int64_t& row_end, int64_t& nt) {
  for (int e = 0; e < G; ++e) {
    const int64_t a = offsets[e], b = offsets[e + 1];
    const int64_t mt = (b - a + bm - 1) / bm;
    const int64_t cnt = mt * ntn;
    if (t < cnt) {
      g = e;
      nt = t / mt;
      row0 = a + (t % mt) * bm;
      row_end = b;
      return true;
    }
    t -= cnt;
  }
  return false;
}

__device__ __forceinline__ int64_t live_tiles(const int64_t* __restrict__ offsets, int G, int bm,
                                              int64_t ntn) {
  int64_t n = 0;
  for (int e = 0; e < G; ++e) n += (offsets[e + 1] - offsets[e] + bm - 1) / bm;
  return n * ntn;
}

// Workgroup w of `live` -> live tile index, XCD-contiguous (w % 8 = XCD).
__device__ __forceinline__ int64_t xcd_tile(int64_t w, int64_t live) {
  const int64_t x = w & 7, s = w >> 3;
  const int64_t q = live >> 3, r = live & 7;
  return x * q + (x < r ? x : r) + s;
}

// Raw NVFP4 bytes of one staging item: 32 codes (two blocks) + their scales.
struct RawItem {
  uint4 c;
  uint32_t s;
};

// BM x BN workgroup tile; WGM x WGN wavefronts (WGM*WGN == 4), each owning
// (BM/WGM) x (BN/WGN) = (32*TM) x (32*TN).
//
// Pipeline per K stage kt (one basic block, no branches): raw NVFP4 bytes of
// stage kt+2 are loaded into registers while the MFMAs of stage kt run from
// LDS buffer kt&1 and the raw bytes of stage kt+1 (loaded an iteration ago)
// are dequantized into LDS buffer (kt+1)&1, one staging item per K16 step,
// so the scheduler can overlap VALU/LDS-write work with the MFMA pipe.
template <int BM, int BN, int WGM, int WGN, bool OUT_BF16>
__global__ __launch_bounds__(256, 1) void k_fwd(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const float* __restrict__ ao,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, const float* __restrict__ bo,
    const int64_t* __restrict__ offsets, int G, int64_t N, int64_t K, void* __restrict__ y) {
  constexpr int TM = BM / WGM / 32, TN = BN / WGN / 32;
  // staging items: (row, pair) with pair p = NVFP4 blocks 2p, 2p+1 of the stage
  // (16 code bytes + 2 scale bytes); item it = tid + 256 * i, row it >> 1
  constexpr int APT = (2 * BM + 255) / 256;
  constexpr int BPT = (2 * BN + 255) / 256;
  constexpr int NIT = APT + BPT;
  constexpr int KS = BK / 16;
  static_assert(NIT <= KS, "at most one staging item per K16 step");
  extern __shared__ _Float16 smem[];
  _Float16* sa = smem;                     // [2][BM * BK]
  _Float16* sb = smem + 2 * BM * BK;       // [2][BN * BK]

  const int64_t ntn = N / BN;
  const int64_t live = live_tiles(offsets, G, BM, ntn);
  if ((int64_t)blockIdx.x >= live) return;
  int g;
  int64_t row0, row_end, nt;
  tile_of(offsets, G, xcd_tile(blockIdx.x, live), BM, ntn, g, row0, row_end, nt);
  const int64_t n0 = nt * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int64_t KB = K / 2, KSB = K / 16;
  const int pp = tid & 1;

  // per item: source pointers (rows clamped to a valid one), validity, LDS row
  const uint8_t* gc[NIT];
  const uint8_t* gs[NIT];
  bool ok[NIT];
  int lrow[NIT];
  bool isa[NIT];
#pragma unroll
  for (int i = 0; i < NIT; ++i) {
    const bool A = i < APT;
    const int it = tid + 256 * (A ? i : i - APT);
    const int lr = it >> 1;
    isa[i] = A;
    lrow[i] = lr;
    int64_t r;
    if (A) {
      ok[i] = lr < BM && row0 + lr < row_end;
      r = ok[i] ? row0 + lr : row0;
      gc[i] = ac + r * KB + pp * 16;
      gs[i] = as + r * KSB + pp * 2;
    } else {
      ok[i] = lr < BN;
      r = (int64_t)g * N + n0 + (ok[i] ? lr : 0);
      gc[i] = bc + r * KB + pp * 16;
      gs[i] = bs + r * KSB + pp * 2;
    }
  }

  uint32_t okm[NIT];
#pragma unroll
  for (int i = 0; i < NIT; ++i) okm[i] = 0u - (uint32_t)ok[i];

  const int64_t nk = K / BK;
  auto gload = [&](RawItem* dst, int64_t kt) {
    const int64_t cb = kt * (BK / 2), sbo = kt * (BK / 16);
    // rows past the group end read a valid row; they are zeroed when the
    // item is dequantized (an iteration later), so no use of the loaded
    // registers here forces a wait on this load
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      dst[i].c = *reinterpret_cast<const uint4*>(gc[i] + cb);
      dst[i].s = *reinterpret_cast<const uint16_t*>(gs[i] + sbo);
    }
  };
  auto store_item = [&](const RawItem& it, int i, int buf) {
    // items of a tile dimension below 128 rows are only partly populated
    if constexpr ((2 * BM) % 256 != 0 || (2 * BN) % 256 != 0)
      if (!(isa[i] ? lrow[i] < BM : lrow[i] < BN)) return;
    u32x4 v[4];
    const uint32_t m = okm[i];              // all ones or zero: no branch
    const uint4 c = make_uint4(it.c.x & m, it.c.y & m, it.c.z & m, it.c.w & m);
    dequant32(c, it.s & m, v);
    _Float16* d = isa[i] ? sa + buf * BM * BK : sb + buf * BN * BK;
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(d + swz(lrow[i], 4 * pp + c)) = v[c];
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  RawItem raw1[NIT], raw2[NIT];
  gload(raw1, 0);
#pragma unroll
  for (int i = 0; i < NIT; ++i) store_item(raw1[i], i, 0);
  gload(raw1, nk > 1 ? 1 : 0);
  __syncthreads();

  const int half = lane >> 5, r32 = lane & 31;
  f16x8 af[2][TM], bf[2][TN];
  auto read_frags = [&](int fbuf, int buf, int ks) {
    const _Float16* ca = sa + buf * BM * BK;
    const _Float16* cbp = sb + buf * BN * BK;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      af[fbuf][i] = *reinterpret_cast<const f16x8*>(ca + swz(wm * TM * 32 + i * 32 + r32, 2 * ks + half));
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bf[fbuf][j] = *reinterpret_cast<const f16x8*>(cbp + swz(wn * TN * 32 + j * 32 + r32, 2 * ks + half));
  };
  auto mfmas = [&](int fbuf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[fbuf][i], bf[fbuf][j], acc[i][j], 0, 0, 0);
  };
  // interleave hint: each MFMA followed by a few VALU (dequant) instructions,
  // LDS reads/writes spread between them
  auto interleave = [&]() {
#pragma unroll
    for (int m = 0; m < TM * TN; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);                   // up to 4 VALU
      if (m % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
      if (m % 4 == 1) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // 1 LDS write
    }
  };

  // Stage kt: K16 steps 0..KS-2 run before the barrier (their MFMAs queue
  // up while the barrier waits), step KS-1 after it, with its operands
  // already in registers, hiding the first fragment reads of stage kt+1.
  read_frags(0, 0, 0);
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    gload(raw2, kt + 2 < nk ? kt + 2 : nk - 1);
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
      read_frags((ks + 1) & 1, cur, ks + 1);
      mfmas(ks & 1);
      if (ks < NIT) store_item(raw1[ks], ks, cur ^ 1);
      if (ks == KS - 2)
#pragma unroll
        for (int i = KS - 1; i < NIT; ++i) store_item(raw1[i], i, cur ^ 1);
      interleave();
    }
    __syncthreads();
    if (kt + 1 < nk) read_frags(0, cur ^ 1, 0);
    mfmas((KS - 1) & 1);
#pragma unroll
    for (int i = 0; i < NIT; ++i) raw1[i] = raw2[i];
  }

  // epilogue: lane holds column (lane & 31) and rows 8*q + 4*half + v of each tile
  const float sw = bo[g];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t row = row0 + wm * TM * 32 + i * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
      if (row >= row_end) continue;
      const float sx = ao[row];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = n0 + wn * TN * 32 + j * 32 + r32;
        const float v = __fmul_rn(__fmul_rn(acc[i][j][e], sx), sw);
        if constexpr (OUT_BF16)
          static_cast<uint16_t*>(y)[row * N + col] = (uint16_t)f32_to_bf16_rne(v);
        else
          static_cast<float*>(y)[row * N + col] = v;
      }
    }
  }
}

template <int BM, int BN, int WGM, int WGN>
hipError_t launch_cfg(const uint8_t* ac, const uint8_t* as, const float* ao, const uint8_t* bc,
                      const uint8_t* bs, const float* bo, const int64_t* offsets, int G,
                      int64_t m_cap, int64_t N, int64_t K, void* y, bool y_bf16,
                      hipStream_t stream) {
  const size_t lds = (size_t)2 * (BM + BN) * BK * sizeof(_Float16);
  const int64_t tiles = ((m_cap + BM - 1) / BM + G) * (N / BN);   // bound on live tiles
  auto k = y_bf16 ? k_fwd<BM, BN, WGM, WGN, true> : k_fwd<BM, BN, WGM, WGN, false>;
  static bool attr_set[2] = {false, false};
  if (!attr_set[y_bf16]) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set[y_bf16] = true;
  }
  k<<<(unsigned)tiles, 256, lds, stream>>>(ac, as, ao, bc, bs, bo, offsets, G, N, K, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_grouped_gemm(const uint8_t* ac, const uint8_t* as, const float* ao,
                                   const uint8_t* bc, const uint8_t* bs, const float* bo,
                                   const int64_t* offsets, int G, int64_t m_cap, int64_t N,
                                   int64_t K, void* y, bool y_bf16, hipStream_t stream) {
  if (m_cap == 0 || G == 0) return hipSuccess;
  // few rows per expert (decode): 32-row tiles, the wavefronts split N
  if (m_cap <= 64 * (int64_t)G || N % 256 != 0)
    return launch_cfg<32, 128, 1, 4>(ac, as, ao, bc, bs, bo, offsets, G, m_cap, N, K, y, y_bf16,
                                     stream);
  return launch_cfg<256, 256, 2, 2>(ac, as, ao, bc, bs, bo, offsets, G, m_cap, N, K, y, y_bf16,
                                    stream);
}

}  // namespace nvfp4moe
