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
// Structure (large tiles). A workgroup owns a 256 x 256 tile (tokens x
// outputs) of one expert. The K loop moves 128 elements per stage: the
// stage's raw NVFP4 code bytes (64 per row of A and of B) go from global
// memory straight into LDS by buffer loads with the LDS-destination bit,
// three stages in flight, and the E4M3 block scales through a two-block LDS
// ring, so LDS carries 4.5 bits per element and no registers stage the loads.
// The wavefronts convert the raw codes of their own fragment rows to f16
// (v_cvt_scalef32_pk_f16_fp4 at unit scale, then an exact v_pk_mul_f16 by
// the block's E4M3 scale) a step ahead of the MFMAs that use them, so the
// conversions co-issue with the matrix pipe. One barrier per stage.
// k_fwd_lds4 runs four wavefronts, one per SIMD, of 128 x 128 (it is also the
// NVFP4 weight-gradient kernel); an eight-wavefront form (two per SIMD, 128 x
// 64 each, so one's waits overlap the other's MFMAs, but 6 conversions per 4
// MFMAs where this one has 4 per 4) measured 3-6% slower at contractions of
// 1024 and 1536 and 2-4% at 4096, and was removed. A wavefront's 32-row
// blocks alternate with the other wavefront row's (block 2i + wm), so a
// partial tile's rows are spread over all SIMDs. It runs persistent (one
// workgroup per compute unit looping over the tiles) when the bound on live
// tiles is far above one round.
//
// Tile order. Five parts: every group's full 256-row tiles, then the partial
// last tiles by their count of 64-row blocks (4, 3, 2, 1), the costliest
// first (a partial tile runs MFMAs only for its valid row blocks). Each part
// is split into 8 contiguous ranges, one per XCD (workgroup w runs on XCD
// w % 8), and within a group the tiles go in blocks of 4 n-tiles, m-tile
// fastest, so the workgroups an XCD runs together share weight and
// activation tiles in its L2. An XCD's list is its range of part 0, then of
// part 1, and so on; its workgroups take the list a round at a time, in
// reverse order in odd rounds, so the workgroup that drew one of a round's
// costlier tiles draws one of the next round's cheaper ones (the static
// round-robin left the most loaded compute unit 14-19% above the mean at
// the expert share's shapes).
//
// Other kernels. k_fwd_stream streams the weights for groups of a few rows
// (decode: 16-row units), and takes the short tails of the 256-row tiles in a
// second launch when they alone would start a second round of workgroups;
// k_fwd (32 x 128 tiles, f16 dequantized into LDS) covers the shapes the
// other two do not.
#include <type_traits>

#include "codecs.hpp"
#include "internal.hpp"
#include "tiles.hpp"

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

// ---------------------------------------------------------------------------
// Large tiles: raw NVFP4 staged in LDS, dequantized per wavefront.
//
// A workgroup of 4 wavefronts owns a 256 x 256 tile of one expert; each
// wavefront owns 128 x 128 (4 x 4 MFMA tiles). The K loop moves 128 elements
// per stage. The stage's raw bytes (64 code bytes and 8 scale bytes per row of
// A and of B) go from global memory straight into LDS (buffer loads with the
// LDS-destination bit: no registers, no VALU), NS stages in flight. Each
// wavefront reads the raw codes of its fragment rows (32 bytes per lane and
// row per stage), converts them to f16 right before the MFMAs that use them
// (v_cvt_scalef32_pk_f16_fp4 at unit scale, then an exact v_pk_mul_f16 by the
// block's E4M3 scale), so LDS carries 4.5 bits per element instead of 16.
//
// K order inside a stage. The f16 MFMA's lane (row r, half h) supplies 8
// consecutive k of a 16-deep step; any permutation of k shared by A and B
// leaves the dot product unchanged, so step s takes k = s*8..s*8+7 from lanes
// with h = 0 and k = 64+s*8..+7 from lanes with h = 1. A lane then needs
// bytes 32h..32h+31 of its row's 64 stage bytes (two 16-byte reads) and the
// scales of blocks 4h..4h+3 (one 32-bit read).
//
// LDS rows are 64 bytes (four 16-byte chunks); chunk c of row r sits at
// position c ^ chunk_key(r), so the lanes of a read phase (consecutive rows,
// one chunk) hit distinct 16-byte bank groups. A DMA load writes 16 bytes per
// lane at consecutive positions, so each lane fetches the global chunk that
// belongs at its position.
constexpr int LBK = 128;                  // K elements per stage
constexpr int LCB = LBK / 2;              // code bytes per row per stage
constexpr int LSB = LBK / 16;             // scale bytes per row per stage
constexpr int LT = 256;                   // tile rows (A) and columns (B)
constexpr int kStageBytes = 2 * LT * LCB;           // one stage's codes, A then B
constexpr int SBK = 4;                                // stages per scale block
constexpr int kScaleRow = SBK * LSB;                  // scale bytes of a row per block
// LDS pitch of a row's scale bytes: 36 = 9 dwords, so the 32 consecutive rows
// a 32-bit read covers (one per lane) fall in 32 distinct banks
constexpr int kScalePitch = kScaleRow + 4;
constexpr int kScaleSlot = 2 * LT * kScalePitch;      // one block, A rows then B rows
constexpr int kScaleRing = 2 * kScaleSlot;            // two blocks
template <int NS>
constexpr int kMainLds = NS * kStageBytes + kScaleRing;
constexpr int kBufWord3 = 0x00020000;     // raw buffer, 32-bit data format

// Parts of the live-tile order (see "Tile order" above): part 0 the full
// m-tiles, part p = 1..4 the partial last m-tiles with 5 - p 64-row blocks.
constexpr int kParts = 5;
__device__ __forceinline__ int tiles_in_part(int64_t m, int part) {
  const int64_t rem = m % LT;
  return part == 0 ? (int)(m / LT) : (rem != 0 && (int)((rem + 63) / 64) == kParts - part);
}

// Element i of XCD x's list (x of nx ranges): its range of part 0, then of
// part 1, ... up to part nparts - 1, each part's tiles being pre[p*G] ..
// pre[(p+1)*G] - 1; -1 past the list's end.
__device__ __forceinline__ int xcd_list_tile(const int* pre, int G, int nparts, int x, int nx,
                                             int i) {
  for (int p = 0; p < nparts; ++p) {
    const int a = pre[p * G], n = pre[(p + 1) * G] - a;
    const int q = n / nx, r = n - q * nx;
    const int c = q + (x < r ? 1 : 0);
    if (i < c) return a + x * q + (x < r ? x : r) + i;
    i -= c;
  }
  return -1;
}

// N dwords to LDS at a 4-byte-aligned address (the scale rows' pitch is not
// a multiple of 8)
template <int N, typename V>
__device__ __forceinline__ void st_dwords(uint8_t* p, const V& v) {
#pragma unroll
  for (int i = 0; i < N; ++i) reinterpret_cast<uint32_t*>(p)[i] = v[i];
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void* first_lane_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}

// WG: the NVFP4 weight gradient with the same main loop. A = dY^T NVFP4
// [N, P] and B = X^T NVFP4 [K, P] (row stride P / 2 bytes), group g's
// contraction is columns [offsets[g], offsets[g+1]) (multiples of 128: no
// stage straddles two groups), outer scales ao[g], bo[g] per group, output
// y = dW [G, N, K] float32; all tiles are full (N, K multiples of 256).
template <int NS, bool OUT_BF16, bool WG = false>
__global__ __launch_bounds__(256, 1) void k_fwd_lds4(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const float* __restrict__ ao,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, const float* __restrict__ bo,
    const int64_t* __restrict__ offsets, int G, int64_t N, int64_t K, void* __restrict__ y,
    int64_t P, int tail_cus, int persist) {
  constexpr int TM = 4, TN = 4;
  extern __shared__ __attribute__((aligned(16))) uint8_t lsm[];

  // Tiles in the order described at the top of the file (not WG).
  const int ntn = (int)(N / LT);
  // persist: the grid is at most one workgroup per compute unit and each
  // workgroup loops over its XCD's list (the scan of tile counts kept in LDS
  // past the stage buffers); otherwise one tile per workgroup (the scan's
  // memory is then reused by the stages; the grid covers the longest list).
  int* pre = reinterpret_cast<int*>(persist ? lsm + kMainLds<NS> : lsm);      // [5G+1]
  // the tile's 256 per-row outer scales (not WG), loaded by DMA with the first stage
  float* rscale = reinterpret_cast<float*>(
      lsm + kMainLds<NS> + (persist ? ((kParts * G + 1) * 4 + 15) & ~15 : 0));
  int nparts = 0;
  if constexpr (!WG) {
    tile_prefix(kParts * G, [&](int e) {
      const int part = e / G, gg = e - part * G;
      return tiles_in_part(offsets[gg + 1] - offsets[gg], part) * ntn;
    }, pre);
    // tail_cus > 0 (the compute-unit count): when the full and larger
    // partial tiles (parts 0-2, more than 128 rows) fit in one round of
    // workgroups and the short tails would start a second one, the tails are
    // left to the streaming kernel launched right after this one (it takes
    // the same decision)
    const int nbig = pre[3 * G], all = pre[kParts * G];
    nparts = tail_cus > 0 && nbig <= tail_cus && all > tail_cus ? 3 : kParts;
  }
  // workgroup b is the j-th of its XCD's workgroups (nx XCDs when the grid
  // is a multiple of 8, else one list)
  const int nx = (gridDim.x & 7) == 0 ? 8 : 1, per = (int)gridDim.x / nx;
  const int xcd = (int)blockIdx.x % nx, j0 = (int)blockIdx.x / nx;
  for (int v = (int)blockIdx.x, round = 0;; v += (int)gridDim.x, ++round) {
  int g, nt;
  int64_t row0, row_end;
  if constexpr (WG) {
    // tiles expert by expert; inside an expert, blocks of 4 output-column
    // tiles with the output-row tile fastest
    const int nrt = (int)(N / LT), nct = (int)(K / LT);
    const int pg = nrt * nct, total_wg = G * pg;
    if (v >= total_wg) return;
    const int tt = (int)xcd_tile(v, total_wg);
    g = tt / pg;
    int mi, ni;
    block_order(tt - g * pg, nrt, nct, mi, ni);
    nt = ni;
    row0 = (int64_t)mi * LT;
    row_end = row0 + LT;
  } else {
    const int j = (round & 1) ? per - 1 - j0 : j0;
    const int tt = xcd_list_tile(pre, G, nparts, xcd, nx, round * per + j);
    if (tt < 0) return;
    const int e = tile_group(pre, kParts * G, tt);
    const int loc = tt - pre[e];
    g = e % G;
    const int64_t o0 = offsets[g];
    row_end = offsets[g + 1];
    const int64_t fm = (row_end - o0) / LT;
    if (e < G) {
      // blocks of 4 n-tiles, m then n inside a block: the ~32 tiles an XCD
      // runs together share 8 A tiles and 4 weight tiles in its L2
      int mi, ni;
      block_order(loc, (int)fm, ntn, mi, ni);
      nt = ni;
      row0 = o0 + (int64_t)mi * LT;
    } else {
      nt = loc;
      row0 = o0 + fm * LT;
    }
    // the scan's memory (one tile), or the previous tile's epilogue staging
    // (persistent), is overwritten by the stages below
    __syncthreads();
  }
  const int64_t n0 = (int64_t)nt * LT;

  // the thread index through an empty asm: per-lane values derived from it
  // are computed per tile rather than hoisted out of the persistent tile
  // loop and held (spilled) across it
  int tid_ = threadIdx.x;
  asm volatile("" : "+v"(tid_));
  const int tid = tid_, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);     // uniform per wavefront
  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5, r32 = lane & 31;
  // row strides (bytes) of codes and scales; WG: contraction starts at the
  // group's first column
  const int64_t KB = WG ? P / 2 : K / 2, KSB = WG ? P / 16 : K / 16;
  const int64_t cb0 = WG ? offsets[g] / 2 : 0, sb0 = WG ? offsets[g] / 16 : 0;
  const int arows = __builtin_amdgcn_readfirstlane(
      (int)(row_end - row0 < LT ? row_end - row0 : LT));          // valid A rows

  // buffer resources (tile-relative, uniform)
  const __amdgpu_buffer_rsrc_t rac = __builtin_amdgcn_make_buffer_rsrc(
      first_lane_ptr(ac + row0 * KB + cb0), (short)0, (int)(uint32_t)(arows * KB), kBufWord3);
  const __amdgpu_buffer_rsrc_t ras = __builtin_amdgcn_make_buffer_rsrc(
      first_lane_ptr(as + row0 * KSB + sb0), (short)0, (int)(uint32_t)(arows * KSB), kBufWord3);
  const int64_t brow0 = WG ? n0 : (int64_t)g * N + n0;
  const __amdgpu_buffer_rsrc_t rbc = __builtin_amdgcn_make_buffer_rsrc(
      first_lane_ptr(bc + brow0 * KB + cb0), (short)0, (int)(uint32_t)(LT * KB), kBufWord3);
  const __amdgpu_buffer_rsrc_t rbs = __builtin_amdgcn_make_buffer_rsrc(
      first_lane_ptr(bs + brow0 * KSB + sb0), (short)0, (int)(uint32_t)(LT * KSB), kBufWord3);
  if constexpr (!WG) {
    // rows row0 .. row0+255 (0 past the group), one wavefront per 64 rows,
    // issued before the first stage so the prologue's wait covers it
    const __amdgpu_buffer_rsrc_t rao = __builtin_amdgcn_make_buffer_rsrc(
        first_lane_ptr(ao + row0), (short)0, (int)(uint32_t)(arows * 4), kBufWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rao, (lds_void*)(rscale + wave * 64), 4,
                                             (uint32_t)((wave * 64 + lane) * 4), 0, 0, 0);
  }

  // DMA offsets of this lane: code instruction i of wavefront w fills rows
  // (4i + w) * 16 + lane / 4 at position lane % 4. Rows past the group end
  // read the tile's first row (results discarded).
  uint32_t oac[4], obc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (4 * i + wave) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ chunk_key(r);
    const int ra = r < arows ? r : 0;
    oac[i] = (uint32_t)(ra * KB + c * 16);
    obc[i] = (uint32_t)(r * KB + c * 16);
  }
  // Scales. A block of SBK stages holds 32 scale bytes per row ([slot][A rows,
  // then B rows][32]); in stage s of a block each thread loads the 16-byte
  // half tid & 1 of row s * 128 + tid / 2 of the 512 (A for s < 2, B after)
  // of the next block, and writes it to the ring in stage s + 1, before that
  // stage's barrier. Rows past the group end read the tile's first row.
  uint32_t osc[SBK];
#pragma unroll
  for (int q = 0; q < SBK; ++q) {
    const int r = (q & 1) * 128 + (tid >> 1);
    const int rr = q < 2 ? (r < arows ? r : 0) : r;
    osc[q] = (uint32_t)(rr * KSB + (tid & 1) * 16);
  }
  // Stage kt goes to LDS buffer kt % NS. A stage past the end (kt >= nk) is
  // issued too, through buffer resources of size 0: such loads return zeros
  // without a memory access and keep the count of loads per stage, and so the
  // wait counts, fixed. Choosing the resource (scalar registers) rather than
  // adding an offset keeps each load's address register untouched, so no
  // load waits for its predecessor to have read a shared one.
  const __amdgpu_buffer_rsrc_t rnull = __builtin_amdgcn_make_buffer_rsrc(
      first_lane_ptr(bc), (short)0, 0, kBufWord3);
  // part 0: the A tile's codes, 1: the weight tile's, 2: both
  auto issue = [&](int64_t kt, int64_t nk, int part) {
    uint8_t* st = lsm + (kt % NS) * kStageBytes;
    const bool real = kt < nk;
    const int64_t ks = real ? kt : 0;
    const int so = (int)(ks * LCB);
    const __amdgpu_buffer_rsrc_t xac = real ? rac : rnull, xbc = real ? rbc : rnull;
    if (part != 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xac, (lds_void*)(st + (4 * i + wave) * 1024), 16,
                                                 oac[i], so, 0, 0);
    }
    if (part != 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xbc, (lds_void*)(st + LT * LCB + (4 * i + wave) * 1024), 16, obc[i], so, 0, 0);
    }
  };
  constexpr int kPerStage = 8;             // code DMA instructions per stage and wavefront
  // the scale piece written in stage kt (group kt % SBK of block kt / SBK + 1),
  // loaded one stage earlier; blocks past the contraction's end read zeros or
  // other rows' bytes that only stages past the end would use
  u32x4 spiece;
  auto load_piece = [&](int64_t kt) {
    const int q = (int)(kt % SBK);
    const int64_t blk = kt / SBK + 1;
    const uint32_t off = osc[0] * (q == 0) + osc[1] * (q == 1) + osc[2] * (q == 2) +
                         osc[3] * (q == 3) + (uint32_t)(blk * kScaleRow);
    spiece = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(q < 2 ? ras : rbs,
                                                                             off, 0, 0));
  };
  // thread tid moves 16-byte piece tid % 2 of row q * 128 + tid / 2
  const int piece_dst = (tid >> 1) * kScalePitch + (tid & 1) * 16;
  auto store_piece = [&](int64_t kt) {
    const int q = (int)(kt % SBK);
    const int64_t blk = kt / SBK + 1;
    st_dwords<4>(lsm + NS * kStageBytes + (blk & 1) * kScaleSlot + q * 128 * kScalePitch +
                 piece_dst, spiece);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int64_t nk = WG ? (offsets[g + 1] - offsets[g]) / LBK : K / LBK;

  // per-lane LDS byte offsets of the fragment reads (stage-relative). The
  // tile's 32-row blocks alternate between the two rows of wavefronts (block
  // 2i + wm is the wavefront's i-th), so a partial tile's valid blocks are
  // shared by all four wavefronts instead of leaving two without rows.
  int fa[TM][2], fb[TN][2], sa_off[TM], sb_off[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = (2 * i + wm) * 32 + r32;
#pragma unroll
    for (int c = 0; c < 2; ++c) fa[i][c] = r * LCB + (((2 * half + c) ^ chunk_key(r)) << 4);
    sa_off[i] = NS * kStageBytes + r * kScalePitch + half * 4;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int r = wn * 128 + j * 32 + r32;
#pragma unroll
    for (int c = 0; c < 2; ++c) fb[j][c] = LT * LCB + r * LCB + (((2 * half + c) ^ chunk_key(r)) << 4);
    sb_off[j] = NS * kStageBytes + (LT + r) * kScalePitch + half * 4;
  }

  // The wavefront's rows of A: TA of its TM 32-row blocks hold valid rows
  // (a partial tile has fewer); only those are read, converted and
  // multiplied. TA = 0 keeps only the loads and barriers.
  auto mainloop = [&](auto ta_c) {
  constexpr int TA = decltype(ta_c)::value;
  constexpr int TAA = TA > 0 ? TA : 1;            // array extent
  // Registers: c0/c1 = raw code chunks 0/1 of the lane's rows (steps 0-3 and
  // 4-7), sc = raw scale words, sf[.][p] = f16 scales of blocks 2p, 2p+1.
  u32x4 c0a[TAA], c0b[TN], c1a[TAA], c1b[TN];
  uint32_t sca[TAA], scb[TN];
  f16x2 sfa[TAA][2], sfb[TN][2];
  auto read_chunk = [&](const uint8_t* st, int c, u32x4 (&xa)[TAA], u32x4 (&xb)[TN]) {
    if constexpr (TA == 0) return;
#pragma unroll
    for (int i = 0; i < TA; ++i) xa[i] = *reinterpret_cast<const u32x4*>(st + fa[i][c]);
#pragma unroll
    for (int j = 0; j < TN; ++j) xb[j] = *reinterpret_cast<const u32x4*>(st + fb[j][c]);
  };
  auto read_scales = [&](int64_t kt) {        // stage kt's: block kt / SBK, bytes 8 (kt % SBK)
    if constexpr (TA == 0) return;
    const uint8_t* sc = lsm + ((kt / SBK) & 1) * kScaleSlot + (kt % SBK) * LSB;
#pragma unroll
    for (int i = 0; i < TA; ++i) sca[i] = *reinterpret_cast<const uint32_t*>(sc + sa_off[i]);
#pragma unroll
    for (int j = 0; j < TN; ++j) scb[j] = *reinterpret_cast<const uint32_t*>(sc + sb_off[j]);
  };
  auto cvt_scales = [&](int p) {       // E4M3 -> f16, exact
    if constexpr (TA == 0) return;
#pragma unroll
    for (int i = 0; i < TA; ++i)
      sfa[i][p] = p ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sca[i], 1.0f, true)
                    : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sca[i], 1.0f, false);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      sfb[j][p] = p ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scb[j], 1.0f, true)
                    : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scb[j], 1.0f, false);
  };
  auto deq = [&](uint32_t x, f16x2 sp, int hi) -> f16x8 {
    const _Float16 S = hi ? sp[1] : sp[0];
    const f16x2 s2 = {S, S};
    const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 0) * s2;
    const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 1) * s2;
    const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2) * s2;
    const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 3) * s2;
    return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  };
  struct Frags {
    f16x8 a[TAA], b[TN];
  };
  // step s: raw word s % 4 of chunk s / 4; scale block s / 2 of the lane's four
  auto deq_step = [&](int s, Frags& f) {
    if constexpr (TA == 0) return;
#pragma unroll
    for (int i = 0; i < TA; ++i)
      f.a[i] = deq((s < 4 ? c0a[i] : c1a[i])[s & 3], sfa[i][s >> 2], (s >> 1) & 1);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      f.b[j] = deq((s < 4 ? c0b[j] : c1b[j])[s & 3], sfb[j][s >> 2], (s >> 1) & 1);
  };
  // One region: the MFMAs of step s interleaved with the conversions of the
  // next step; the scheduling barrier keeps other steps' conversions (and
  // their registers) out of it.
  // `extra` (DMA issues or LDS reads of later steps) runs at the start of the
  // region, its NV buffer loads and ND LDS reads spread one per MFMA so that
  // their issue overlaps the matrix cores' work.
  auto region = [&](const Frags& cur, Frags& nxt, int s_next, auto&& extra, auto nv_c, auto nd_c) {
    constexpr int NV = decltype(nv_c)::value, ND = decltype(nd_c)::value;
    if constexpr (TA == 0) {
      extra();
      return;
    }
    __builtin_amdgcn_sched_barrier(0);
    extra();
    deq_step(s_next, nxt);
#pragma unroll
    for (int i = 0; i < TA; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        // W fragment first: the lane then holds 4 consecutive output columns
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.b[j], cur.a[i], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < TA * TN; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);    // 4 VALU
      if constexpr (NV > 0)
        if (m < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // 1 buffer load
      if constexpr (ND > 0)
        if (m < ND) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto none = [] {};
  using Z = std::integral_constant<int, 0>;

  // Pipeline. NS stages are in flight in LDS. Iteration kt runs steps 0-3,
  // reading chunk 1 of stage kt under the MFMAs of step 0; then (mid-stage)
  // waits for stage kt+1's loads and synchronizes: every wavefront has read
  // stage kt, whose buffer is reused for stage kt+NS. Steps 4-7 use chunk 1
  // and the upper scale halves only; under their MFMAs go the DMA issues of
  // stage kt+NS (steps 4 and 5) and the reads of chunk 0 and the scales of
  // stage kt+1 (step 6); the lower scale halves are converted before the last
  // region, which converts step 0 of kt+1. One barrier per stage.
  //
  // Scales: the piece loaded in region 5 of stage kt (before that stage's
  // code DMAs, so waiting for it never waits for them) is written in region
  // 1 of stage kt+1, before its barrier; block b+1 is complete at the
  // barrier of stage 4b+3, whose region 7 reads stage 4b+4's scales. Its
  // ring slot held block b-1, last read in region 7 of stage 4b-2.
  static_assert(kPerStage == 8, "wait counts assume 8 code loads per stage and wavefront");
  static_assert(NS == 3 && SBK == 4, "wait counts assume 3 stages in flight");
  {
    // prologue: scale block 0 (four pieces) and the piece stage 0 writes,
    // then the code stages 0..NS-1
    u32x4 p0[SBK];
#pragma unroll
    for (int q = 0; q < SBK; ++q)
      p0[q] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(q < 2 ? ras : rbs, osc[q], 0, 0));
    load_piece(0);
#pragma unroll
    for (int p = 0; p < NS; ++p) issue(p, nk, 2);
#pragma unroll
    for (int q = 0; q < SBK; ++q)
      st_dwords<4>(lsm + NS * kStageBytes + q * 128 * kScalePitch + piece_dst, p0[q]);
  }
  asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");   // stage 0 landed
  read_chunk(lsm, 0, c0a, c0b);
  read_scales(0);
  cvt_scales(0);
  Frags f0, f1;
  deq_step(0, f0);

  for (int64_t kt = 0; kt < nk; ++kt) {
    const uint8_t* st = lsm + (kt % NS) * kStageBytes;
    const uint8_t* sn = lsm + ((kt + 1) % NS) * kStageBytes;
    cvt_scales(1);
    region(f0, f1, 1, [&] { store_piece(kt); read_chunk(st, 1, c1a, c1b); }, Z{},
           std::integral_constant<int, TA + TN>{});
    region(f1, f0, 2, none, Z{}, Z{});
    region(f0, f1, 3, none, Z{}, Z{});
    region(f1, f0, 4, none, Z{}, Z{});
    // Every wavefront has finished reading stage kt, and stage kt+1 has
    // landed once only stage kt+2's loads are pending. Branch-free: after the
    // last stage the reads below fetch data that is never used.
    asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    region(f0, f1, 5, [&] { load_piece(kt + 1); issue(kt + NS, nk, 0); },
           std::integral_constant<int, 5>{}, Z{});
    region(f1, f0, 6, [&] { issue(kt + NS, nk, 1); }, std::integral_constant<int, 4>{}, Z{});
    region(f0, f1, 7, [&] { read_chunk(sn, 0, c0a, c0b); read_scales(kt + 1); }, Z{},
           std::integral_constant<int, 2 * (TA + TN)>{});
    cvt_scales(0);
    region(f1, f0, 0, none, Z{}, Z{});   // step 0 of stage kt+1 (unused after the last stage)
  }
  };
  if constexpr (WG) {
    mainloop(std::integral_constant<int, 4>{});        // weight-gradient tiles are full
  } else {
    // valid 32-row blocks of this wavefront: blocks wm, wm + 2, ... below nblk
    const int nblk = (arows + 31) >> 5;
    const int act = nblk > wm ? (nblk - wm + 1) >> 1 : 0;
    if (act >= 4) mainloop(std::integral_constant<int, 4>{});
    else if (act == 3) mainloop(std::integral_constant<int, 3>{});
    else if (act == 2) mainloop(std::integral_constant<int, 2>{});
    else if (act == 1) mainloop(std::integral_constant<int, 1>{});
    else mainloop(std::integral_constant<int, 0>{});
  }

  // Epilogue. acc[i][j][4q+v] = Y[row, col] with row = (2i + wm)*32 + lane%32
  // and col = wn*128 + j*32 + 8q + 4*half + v (the MFMAs took W first). Each
  // wavefront stages one 32-row block at a time in LDS (row-major, scaled and
  // converted), then writes it out 16 bytes per lane along the rows, so the
  // global stores cover whole row segments.
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");   // stage buffers are free
  constexpr int ES = OUT_BF16 ? 2 : 4;                   // output element bytes
  constexpr int RS = 128 * ES + 16;                     // LDS row stride (padded)
  uint8_t* ep = lsm + wave * (32 * RS);
  const float sw = bo[g];
  const int64_t col0 = n0 + wn * 128;
  const int64_t ldo = WG ? K : N;                        // output row stride (elements)
  const int64_t obase = WG ? (int64_t)g * N * K : 0;    // WG: expert g's dW
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const float sx = WG ? ao[g] : rscale[(2 * i + wm) * 32 + r32];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = __fmul_rn(__fmul_rn(acc[i][j][4 * q + t], sx), sw);
        uint8_t* d = ep + r32 * RS + (j * 32 + 8 * q + 4 * half) * ES;
        if constexpr (OUT_BF16) {
          const uint32_t lo = pk_bf16(v[0], v[1]);
          const uint32_t hi = pk_bf16(v[2], v[3]);
          *reinterpret_cast<uint2*>(d) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    // 32 rows x 128 columns: each lane copies 16-byte pieces along the rows
    constexpr int PPR = 128 * ES / 16;                  // pieces per row
#pragma unroll
    for (int it = 0; it < 32 * PPR / 64; ++it) {
      const int pc = it * 64 + lane, r = pc / PPR, c = pc % PPR;
      const u32x4 val = *reinterpret_cast<const u32x4*>(ep + r * RS + c * 16);
      const int64_t orow = row0 + (2 * i + wm) * 32 + r;
      // non-temporal: every workgroup writes its tile at about the same time,
      // 32 MB on the small MoE layer, past what the L2s hold (2 us faster)
      if (orow < row_end)
        __builtin_nontemporal_store(
            val, reinterpret_cast<u32x4*>(static_cast<uint8_t*>(y) +
                                          (obase + orow * ldo + col0) * ES + c * 16));
    }
  }
  if (WG || !persist) return;
  }
}

#ifndef NVFP4MOE_FWD_PERSIST
#define NVFP4MOE_FWD_PERSIST 1
#endif
constexpr bool kFwdPersist = NVFP4MOE_FWD_PERSIST != 0;
constexpr int kPersistFactor = 2;            // bound on tiles above this many per CU
constexpr size_t kMaxPreBytes = 16384;       // tile-count scan kept in LDS (G <= 818)
static_assert(kMainLds<3> + kMaxPreBytes <= 160 * 1024, "LDS budget of k_fwd_lds4");
constexpr size_t kRowScaleBytes = LT * 4;     // a tile's per-row outer scales
static_assert(kMainLds<3> + kMaxPreBytes + kRowScaleBytes <= 160 * 1024, "LDS budget of the tiles");
constexpr int kMaxTileGroups = 4096;         // the scan of 5G + 1 counts fits the stage buffers
static_assert((kParts * kMaxTileGroups + 1) * 4 <= kMainLds<3>, "tile-count scan of one tile");

// Grid of the one-tile-per-workgroup mode for a bound of `tiles` live tiles:
// a multiple of 8 with room for the longest XCD list (each of the five parts
// adds at most one tile above an even split).
inline int64_t one_tile_grid(int64_t tiles) { return (tiles + 8 * kParts + 7) / 8 * 8; }

template <int NS>
hipError_t launch_lds4(const uint8_t* ac, const uint8_t* as, const float* ao, const uint8_t* bc,
                       const uint8_t* bs, const float* bo, const int64_t* offsets, int G,
                       int64_t m_cap, int64_t N, int64_t K, void* y, bool y_bf16,
                       int tail_cus, hipStream_t stream) {
  const int64_t tiles = ((m_cap + LT - 1) / LT + G) * (N / LT);   // bound on live tiles
  // Persistent (one workgroup per compute unit, each looping over tiles)
  // when the bound on the tile count is well above the live tiles it may
  // hold: workgroups past the live tiles only start and exit, but the
  // dispatcher issues them one after another at the end of the launch
  // (e.g. a capacity-sized down-projection: 17152 workgroups for 2336 tiles).
  // The tile-count scan then stays in LDS beside the stages.
  const int64_t cus = device_cu_count();
  const size_t pre_bytes = ((size_t)(kParts * G + 1) * 4 + 15) & ~(size_t)15;
  const bool persist = kFwdPersist && pre_bytes <= kMaxPreBytes &&
                       tiles > (int64_t)kPersistFactor * cus;
  const size_t lds = (size_t)kMainLds<NS> + (persist ? pre_bytes : 0) + kRowScaleBytes;
  auto k = y_bf16 ? k_fwd_lds4<NS, true> : k_fwd_lds4<NS, false>;
  static bool attr_set[2] = {false, false};
  if (!attr_set[y_bf16]) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)((size_t)kMainLds<NS> + kMaxPreBytes + kRowScaleBytes));
    if (e != hipSuccess) return e;
    attr_set[y_bf16] = true;
  }
  const int64_t grid = persist ? cus : one_tile_grid(tiles);
  k<<<(unsigned)grid, 256, lds, stream>>>(ac, as, ao, bc, bs, bo, offsets, G, N, K, y, 0,
                                          tail_cus, persist ? 1 : 0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Few routed rows per expert (decode): weight streaming through LDS.
//
// Units of 16 routed rows of one expert by 64 outputs (64 weight rows) are
// enumerated expert by expert. One persistent workgroup per compute unit
// takes units round-robin and runs through their K stages (512 elements
// each) as one stream: each stage's weight bytes (64 rows x 256 code bytes
// + 32 scale bytes) and activation bytes (16 rows, same) go from HBM straight
// into an LDS ring of SK_S stages (buffer loads with the LDS-destination
// bit), so about 90 KB per compute unit are in flight without holding
// registers. Eight wavefronts, two per SIMD so that one computes while the
// other waits: wavefront w owns outputs 16 (w % 4) .. +15 and half of each
// stage's K (sub-chunks 2 (w / 4) and 2 (w / 4) + 1 of 128 elements); it
// converts its weight and activation codes to f16 and runs
// v_mfma_f32_16x16x32_f16. The two halves' sums meet in LDS at the end of a
// unit.
//
// K order inside a 128-element sub-chunk: A and B share one permutation of
// k; the lanes with l / 16 = q supply k = 32q .. 32q+31, eight per step.
// LDS rows hold 16 pieces of 16 bytes; piece p of row r sits at position
// p ^ (r & 15), so the 16 rows read at one piece offset hit distinct banks.
constexpr int SK_T = 16;                      // routed rows per unit
constexpr int SK_N = 64;                      // outputs (weight rows) per unit
constexpr int SK_K = 512;                     // K elements per stage
constexpr int SK_S = 5;                       // stages in the LDS ring
constexpr int SK_RB = SK_K / 2;               // code bytes per row per stage
constexpr int SK_SB = SK_K / 16;              // scale bytes per row per stage
constexpr int SK_WC = 0;                      // [64][256] weight codes
constexpr int SK_XC = SK_WC + SK_N * SK_RB;   // [16][256] activation codes
constexpr int SK_WS = SK_XC + SK_T * SK_RB;   // [64][32] weight scales
constexpr int SK_XS = SK_WS + SK_N * SK_SB;   // [16][32] activation scales
constexpr int SK_STAGE = SK_XS + SK_T * SK_SB;
constexpr int SK_DMA = 5;                     // DMA instructions per stage and wavefront
constexpr int SK_RED = 4 * 64 * 16;           // partial sums of the upper K halves
constexpr int SK_USC = 8 * 128 * 4;           // output scales of 8 units: [8][64 rows + 64 x group]
constexpr int SK_MAXG = 1024;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x8 deq8(uint32_t x, f16x2 sp, int hi) {
  const _Float16 S = hi ? sp[1] : sp[0];
  const f16x2 s2 = {S, S};
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 0) * s2;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 1) * s2;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2) * s2;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 3) * s2;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

template <bool OUT_BF16>
__global__ __launch_bounds__(512, 1) void k_fwd_stream(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const float* __restrict__ ao,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, const float* __restrict__ bo,
    const int64_t* __restrict__ offsets, int G, int64_t N, int64_t K, void* __restrict__ y,
    int tail) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lsm[];
  float* red = reinterpret_cast<float*>(lsm + SK_S * SK_STAGE);      // [4][64 lanes][4]
  // a unit's 16 row scales and its expert's scale, by DMA with its first stage
  float* usc = reinterpret_cast<float*>(lsm + SK_S * SK_STAGE + SK_RED);        // [8][128]
  int64_t* off = reinterpret_cast<int64_t*>(lsm + SK_S * SK_STAGE + SK_RED + SK_USC);   // [G+1]
  int* pre = reinterpret_cast<int*>(off + G + 1);                     // [G+1]
  const int nnb = (int)(N / SK_N);
  for (int e = threadIdx.x; e <= G; e += 512) off[e] = offsets[e];
  // Rows of group e that this launch covers: all of them, or (tail > 0) only
  // the last partial 256-row tile when it has at most 128 rows, the rows the
  // 256 x 256 tile kernel leaves out; they end at the group's end either way.
  auto rows_of = [&](int64_t a, int64_t b) -> int64_t {
    const int64_t m = b - a, rem = m % LT;
    return !tail ? m : (rem != 0 && rem <= LT / 2 ? rem : 0);
  };
  if (tail) {
    // the 256 x 256 kernel's decision (tail = its compute-unit count): the
    // tails are here only if its other tiles fit in one round and the tails
    // would have started a second
    const int ntn = (int)(N / LT);
    tile_prefix(G, [&](int e) {
      const int64_t m = offsets[e + 1] - offsets[e];
      return (int)(m / LT + (m % LT > LT / 2 ? 1 : 0)) * ntn;
    }, pre);
    const int nbig = pre[G];
    tile_prefix(G, [&](int e) {
      const int64_t rem = (offsets[e + 1] - offsets[e]) % LT;
      return rem != 0 && rem <= LT / 2 ? ntn : 0;
    }, pre);
    const int nsmall = pre[G];
    if (!(nbig <= tail && nbig + nsmall > tail)) return;     // the same for the whole workgroup
  }
  tile_prefix(G, [&](int e) {
    return (int)((rows_of(offsets[e], offsets[e + 1]) + SK_T - 1) / SK_T) * nnb;
  }, pre);
  const int total = pre[G];
  if ((int)blockIdx.x >= total) return;
  const int nunits = (total - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int nst = (int)(K / SK_K);                  // stages per unit
  const int nall = nunits * nst;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wn = wave & 3, wk = wave >> 2;          // output block, K half
  const int r = lane & 15, q = lane >> 4;
  const int64_t KB = K / 2, KSB = K / 16;

  struct Unit {
    int g, nb;
    int64_t row0, row_end;
  };
  auto rfl64 = [](int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
  };
  auto unit = [&](int j) {            // the same for the whole workgroup
    const int t = (int)blockIdx.x + j * (int)gridDim.x;
    Unit u;
    u.g = __builtin_amdgcn_readfirstlane(tile_group(pre, G, t));
    const int loc = t - pre[u.g];
    u.nb = __builtin_amdgcn_readfirstlane(loc % nnb);
    u.row0 = rfl64(off[u.g + 1] - rows_of(off[u.g], off[u.g + 1]) + (int64_t)(loc / nnb) * SK_T);
    u.row_end = rfl64(off[u.g + 1]);
    return u;
  };

  // DMA lane offsets (stage- and unit-relative). Codes: instruction m fills
  // rows 4m .. 4m+3 (lane: row 4m + lane/16, position lane%16). Scales:
  // instruction m fills rows 8m .. 8m+7 (lane: row 8m + lane/8, dword lane%8).
  // Wavefronts 4-7 repeat the activation loads of 0-3 (same bytes, same place).
  int wrow_c[2], wpiece[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 4 * (2 * wave + i) + (lane >> 4);
    wrow_c[i] = row;
    wpiece[i] = (lane & 15) ^ (row & 15);
  }
  const int xrow_c = 4 * wn + (lane >> 4);
  const int xpiece = (lane & 15) ^ (xrow_c & 15);
  const int wrow_s = 8 * wave + (lane >> 3);
  const int xrow_s = 8 * (wave & 1) + (lane >> 3);
  const int sdw = (lane & 7) * 4;

  // Issue cursor: stage ist of unit ij goes to ring buffer ibuf. The unit's
  // buffer resources are rebuilt only when the cursor enters a new unit.
  // Past the end of the stream the last stage is re-issued with offsets
  // outside the ranges (zeros, no memory traffic), keeping the count per stage.
  int ij = 0, ist = 0, ibuf = 0;
  __amdgpu_buffer_rsrc_t rwc, rws, rxc, rxs, rxo, rgo;
  int ixrows = 0;
  auto set_unit = [&](int j) {
    const Unit u = unit(j);
    const int64_t wr0 = (int64_t)u.g * N + (int64_t)u.nb * SK_N;
    ixrows = (int)(u.row_end - u.row0 < SK_T ? u.row_end - u.row0 : SK_T);
    rwc = __builtin_amdgcn_make_buffer_rsrc(first_lane_ptr(bc + wr0 * KB), (short)0,
                                            (int)(uint32_t)(SK_N * KB), kBufWord3);
    rws = __builtin_amdgcn_make_buffer_rsrc(first_lane_ptr(bs + wr0 * KSB), (short)0,
                                            (int)(uint32_t)(SK_N * KSB), kBufWord3);
    rxc = __builtin_amdgcn_make_buffer_rsrc(first_lane_ptr(ac + u.row0 * KB), (short)0,
                                            (int)(uint32_t)(ixrows * KB), kBufWord3);
    rxs = __builtin_amdgcn_make_buffer_rsrc(first_lane_ptr(as + u.row0 * KSB), (short)0,
                                            (int)(uint32_t)(ixrows * KSB), kBufWord3);
    rxo = __builtin_amdgcn_make_buffer_rsrc(first_lane_ptr(ao + u.row0), (short)0,
                                            (int)(uint32_t)(ixrows * 4), kBufWord3);
    rgo = __builtin_amdgcn_make_buffer_rsrc(first_lane_ptr(bo + u.g), (short)0, 4, kBufWord3);
  };
  set_unit(0);
  auto issue = [&]() {
    const uint32_t away = ij < nunits ? 0u : 0x40000000u;
    // the first stage of a unit also brings the unit's output scales (wave 0:
    // row r's at slot + r, rows past the unit read 0; the expert's at slot + 64
    // + lane); issued after the stage's loads, so each wait that covers the
    // stage covers them, and read at the unit's last stage
    const bool first = ist == 0 && ij < nunits;
    float* uslot = usc + (ij & 7) * 128;
    const __amdgpu_buffer_rsrc_t uxo = rxo, ugo = rgo;
    uint8_t* sb = lsm + ibuf * SK_STAGE;
    const int cofs = ist * SK_RB, sofs = ist * SK_SB;
#pragma unroll
    for (int k = 0; k < 2; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rwc, (lds_void*)(sb + SK_WC + (2 * wave + k) * 1024), 16,
          (uint32_t)(wrow_c[k] * KB + wpiece[k] * 16) + away, cofs, 0, 0);
    {
      const int xr = xrow_c < ixrows ? xrow_c : 0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rxc, (lds_void*)(sb + SK_XC + wn * 1024), 16,
                                               (uint32_t)(xr * KB + xpiece * 16) + away, cofs, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rws, (lds_void*)(sb + SK_WS + wave * 256), 4,
                                             (uint32_t)(wrow_s * KSB + sdw) + away, sofs, 0, 0);
    {
      const int xr = xrow_s < ixrows ? xrow_s : 0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rxs, (lds_void*)(sb + SK_XS + (wave & 1) * 256), 4,
                                               (uint32_t)(xr * KSB + sdw) + away, sofs, 0, 0);
    }
    if (first && wave == 0) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(uxo, (lds_void*)uslot, 4, (uint32_t)(lane * 4), 0,
                                               0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ugo, (lds_void*)(uslot + 64), 4, 0u, 0, 0, 0);
    }
    ibuf = ibuf + 1 == SK_S ? 0 : ibuf + 1;
    if (ij < nunits && ++ist == nst) {
      ist = 0;
      if (++ij < nunits) set_unit(ij);
      else ist = nst - 1;                     // stay on the last stage
    }
  };

  // fragment read offsets (stage-relative): weight row 16 wn + r and
  // activation row r, sub-chunks 2 wk and 2 wk + 1
  const int wr = 16 * wn + r;
  int wfo[2], xfo[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int sc = 2 * wk + h;
    wfo[h] = SK_WC + wr * SK_RB + (((4 * sc + q) ^ (wr & 15)) << 4);
    xfo[h] = SK_XC + r * SK_RB + (((4 * sc + q) ^ (r & 15)) << 4);
  }
  const int wso = SK_WS + wr * SK_SB + q * 2 + wk * 16, xso = SK_XS + r * SK_SB + q * 2 + wk * 16;

  static_assert(SK_DMA == 5 && SK_S == 5, "the wait count assumes 5 loads per stage, 5 stages");
#pragma unroll
  for (int p = 0; p < SK_S - 1; ++p) issue();

  f32x4 part[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) part[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // compute cursor: stage cst of unit cj, in ring buffer cbuf
  int cj = 0, cst = 0, cbuf = 0;
  Unit cu = unit(0);
  for (int i = 0; i < nall; ++i) {
    // stage i has landed once only the 3 younger stages' loads are pending,
    // and every wavefront is done with the buffer that stage i+4 reuses
    asm volatile("s_waitcnt vmcnt(15)\n\ts_barrier" ::: "memory");
    issue();
    const int st = cst;
    const uint8_t* sb = lsm + cbuf * SK_STAGE;
    cbuf = cbuf + 1 == SK_S ? 0 : cbuf + 1;
    u32x4 wv[2], xv[2];
    uint32_t wsc[2], xsc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      wv[h] = *reinterpret_cast<const u32x4*>(sb + wfo[h]);
      xv[h] = *reinterpret_cast<const u32x4*>(sb + xfo[h]);
      wsc[h] = *reinterpret_cast<const uint16_t*>(sb + wso + h * 8);
      xsc[h] = *reinterpret_cast<const uint16_t*>(sb + xso + h * 8);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f16x2 sw2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wsc[h], 1.0f, false);
      const f16x2 sx2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(xsc[h], 1.0f, false);
#pragma unroll
      for (int k = 0; k < 4; ++k)    // k = 32q + 8k .. +7 of the sub-chunk: word k, block k/2
        part[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(deq8(wv[h][k], sw2, k >> 1),
                                                         deq8(xv[h][k], sx2, k >> 1), part[k],
                                                         0, 0, 0);
    }
    if (st == nst - 1) {
      // unit done: D[n][t] with n = 4q + v, t = r; the upper K half is added
      // to the lower one through LDS
      f32x4 acc = (part[0] + part[1]) + (part[2] + part[3]);
      if (wk == 1) *reinterpret_cast<f32x4*>(red + (wn * 64 + lane) * 4) = acc;
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (wk == 0) {
        acc += *reinterpret_cast<const f32x4*>(red + (wn * 64 + lane) * 4);
        const Unit u = cu;
        const float sx = usc[(cj & 7) * 128 + r], sg = usc[(cj & 7) * 128 + 64];
        const int64_t row = u.row0 + r;
        if (row < u.row_end) {
          float o[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] = __fmul_rn(__fmul_rn(acc[v], sx), sg);
          const int64_t col = (int64_t)u.nb * SK_N + 16 * wn + 4 * q;
          if constexpr (OUT_BF16) {
            const uint32_t lo = pk_bf16(o[0], o[1]);
            const uint32_t hi = pk_bf16(o[2], o[3]);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + row * N + col) =
                make_uint2(lo, hi);
          } else {
            *reinterpret_cast<float4*>(static_cast<float*>(y) + row * N + col) =
                make_float4(o[0], o[1], o[2], o[3]);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) part[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      cst = 0;
      if (++cj < nunits) cu = unit(cj);
    } else {
      ++cst;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // drain the trailing (unused) loads
}

hipError_t launch_stream(const uint8_t* ac, const uint8_t* as, const float* ao, const uint8_t* bc,
                         const uint8_t* bs, const float* bo, const int64_t* offsets, int G,
                         int64_t m_cap, int64_t N, int64_t K, void* y, bool y_bf16,
                         bool tail, hipStream_t stream) {
  auto k = y_bf16 ? k_fwd_stream<true> : k_fwd_stream<false>;
  const size_t base = (size_t)SK_S * SK_STAGE + SK_RED + SK_USC;
  const size_t lds = base + (size_t)(G + 1) * (sizeof(int64_t) + sizeof(int));
  static bool attr_set[2] = {false, false};
  if (!attr_set[y_bf16]) {
    const size_t maxl = base + (size_t)(SK_MAXG + 1) * 12;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)maxl);
    if (e != hipSuccess) return e;
    attr_set[y_bf16] = true;
  }
  int64_t rb = (m_cap + SK_T - 1) / SK_T + G;                  // row units, upper bound
  if (tail && rb > (int64_t)G * (LT / 2 / SK_T)) rb = (int64_t)G * (LT / 2 / SK_T);
  const int64_t bound = rb * (N / SK_N);
  const int64_t slots = device_cu_count();
  const int64_t grid = bound < slots ? bound : slots;
  k<<<(unsigned)grid, 512, lds, stream>>>(ac, as, ao, bc, bs, bo, offsets, G, N, K, y,
                                          tail ? (int)device_cu_count() : 0);
  return hipGetLastError();
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
  // a few rows per expert (decode): weight streaming, 16-row tiles
  if (m_cap <= 32 * (int64_t)G && K % SK_K == 0 && N % SK_N == 0 && G <= SK_MAXG &&
      ((m_cap + SK_T - 1) / SK_T + G) * (N / SK_N) < (int64_t)1 << 31)
    return launch_stream(ac, as, ao, bc, bs, bo, offsets, G, m_cap, N, K, y, y_bf16, false,
                         stream);
  // 32-row tiles, the wavefronts split N
  if (m_cap <= 64 * (int64_t)G || N % 256 != 0 || G > kMaxTileGroups)
    return launch_cfg<32, 128, 1, 4>(ac, as, ao, bc, bs, bo, offsets, G, m_cap, N, K, y, y_bf16,
                                     stream);
  // 256 x 256 tiles; when the partial last m-tiles of at most 128 rows would
  // be all that runs in a second round of 256 x 256 workgroups (nearly as
  // costly as the first, for a few rows each), they go to the streaming
  // kernel right after instead (decided on the device from the offsets)
  // (no second launch when even the bound on the tile count fits one round)
  const bool tails = ((m_cap + LT - 1) / LT + G) * (N / LT) > (int64_t)device_cu_count() &&
                     K % SK_K == 0 && N % SK_N == 0 && G <= SK_MAXG &&
                     (int64_t)G * (LT / 2 / SK_T) * (N / SK_N) < (int64_t)1 << 31;
  hipError_t e = launch_lds4<3>(ac, as, ao, bc, bs, bo, offsets, G, m_cap, N, K, y, y_bf16,
                                tails ? (int)device_cu_count() : 0, stream);
  if (e != hipSuccess || !tails) return e;
  return launch_stream(ac, as, ao, bc, bs, bo, offsets, G, m_cap, N, K, y, y_bf16, true, stream);
}

// NVFP4 weight gradient (see WG above).
hipError_t launch_wgrad_nvfp4(const uint8_t* ac, const uint8_t* as, const float* ao,
                              const uint8_t* bc, const uint8_t* bs, const float* bo,
                              const int64_t* padded, int G, int64_t P, int64_t N, int64_t K,
                              float* dw, hipStream_t stream) {
  constexpr int NS = 3;
  const size_t lds = (size_t)kMainLds<NS>;
  const int64_t tiles = (int64_t)G * (N / LT) * (K / LT);
  if (tiles == 0) return hipSuccess;
  auto k = k_fwd_lds4<NS, false, true>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  k<<<(unsigned)tiles, 256, lds, stream>>>(ac, as, ao, bc, bs, bo, padded, G, N, K, dw, P, 0, 0);
  return hipGetLastError();
}

}  // namespace nvfp4moe
