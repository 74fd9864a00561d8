// MXFP8 dgrad and wgrad grouped GEMMs on gfx950's block-scaled MFMA.
//
// Pages: the backward pass computes gradients with MXFP8 matmuls on the
// re-quantized saved tensors ("Inkling 2 Small uses four-bit training ...",
// sections "NVFP4 forward, MXFP8 backward" and "Stochastic rounding across
// transposes").
//
// MXFP8 (E4M3 elements, one E8M0 power of two per 32 along the contraction)
// is exactly the operand format of v_mfma_scale_f32_32x32x64_f8f6f4: each of
// its two 32-element k-blocks per row takes one E8M0 byte. Its arithmetic is
// not plain float32 accumulation: each product is exact, but a 32-element
// block's products are summed by aligning them to the block's largest and
// dropping bits about 14 binades below it (measured with in-bounds probes: a
// 448 x 448 product absorbs a 4.5 one), and only the block sums are added in
// float32. The error this adds is bounded per element by the sum over blocks
// of 31 * 2^-13 * max|a b| of the block; results meet the 1e-3 per-group
// contract of the expert layer but not an elementwise 1e-3 near cancellation.
// Both GEMMs are "row x row" contractions: each operand is stored with the
// contraction dimension contiguous (that is what the re-quantization's
// transpose is for), so one main loop serves both:
//   dgrad: dX[r, k]    = sum_n dY8[r, n] * W8[g, k, n]       (rows r of expert g)
//   wgrad: dW[g, n, k] = sum_p dYT8[n, p] * XT8[k, p]        (p in g's padded segment)
// The dgrad kernels take the second operand's layout as parameters (row
// stride, and per group a contraction offset and a row offset), which also
// covers the all-MXFP8 forward GEMM:
//   fwd:   Y[r, n]     = sum_k X8[r, k] * W8[g*N + n, k]     (weights stored [G, N, K])
//
// Two kernel families. The main one (further down) streams both operands
// into an LDS ring by DMA, with 256 x 256 workgroup tiles, or 320 x 128 for
// the row x row GEMM when about one round of those covers the output (8
// groups of ~1024 rows x 1024 columns: 256 tiles of 320 x 128 keep every
// compute unit busy where ~140 tiles of 256 x 256 leave 116 idle). The
// fallback for shapes it does not take (sizes not multiples of 256, few rows
// per group) stages through registers:
//
// Structure (fallback). A workgroup of 4 wavefronts owns a T x T output tile
// (T = 128 as launched); each wavefront owns (T/2) x (T/2).
// The contraction advances 128 bytes (4 MX blocks) per stage, so every
// operand row contributes one full 128-byte line per stage. Each thread loads
// its 16-byte chunks of stage kt+1 into registers at the top of iteration kt
// and stores them into the other LDS buffer after the MFMAs of stage kt have
// been issued; 16-byte chunks are XOR-swizzled by row so the fragment reads
// (32 rows at one offset) spread over the LDS banks. Rows past a group's end
// are read from a valid row and their results discarded; contraction
// elements past a ragged end (wgrad's last stage of a group) are masked to
// zero when stored to LDS.
//
// Tile order. dgrad: live tiles only, XCD-contiguous (workgroup w runs on XCD
// w % 8), m-tile fastest within (group, n-tile), so the workgroups an XCD runs
// together share the B tile in its L2. wgrad: groups longest first (a tile's
// cost is its group's token count).
#include "codecs.hpp"
#include "internal.hpp"
#include "tiles.hpp"

namespace nvfp4moe {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 128;                       // contraction bytes (= elements) per stage
constexpr int CPR = BK / 16;                  // 16-byte chunks per row per stage
constexpr int SCB = BK / 32;                  // scale bytes per row per stage
constexpr int kBufferWord3 = 0x00020000;      // raw buffer, 32-bit data format

// The tile coordinates are the same for the whole workgroup; saying so keeps
// buffer resources in scalar registers.
__device__ __forceinline__ void* uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int uniform_u32(int64_t n) {
  return (int)__builtin_amdgcn_readfirstlane((uint32_t)(n < 0xFFFFFFFFll ? n : 0xFFFFFFFFll));
}

// byte offset of 16-byte chunk c of row r in a [rows][BK] stage buffer
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ (r & 7)) << 4); }

struct Operand {
  const uint8_t* q;    // elements, row-major
  const uint8_t* e;    // E8M0 scales, row-major
  int64_t ld;          // elements per row
  int64_t c0;          // first contraction element of this tile
  int64_t row0;        // first row of the tile
  int64_t row_end;     // rows >= row_end are not part of the result
};

__device__ __forceinline__ int64_t xcd_tile(int64_t w, int64_t live) {
  const int64_t x = w & 7, s = w >> 3;
  const int64_t q = live >> 3, r = live & 7;
  return x * q + (x < r ? x : r) + s;
}

// acc += A[rows of this wave] x B[rows of this wave]^T over L contraction
// elements (L a multiple of 32). T x T workgroup tile (T = 256 or 128), 2 x 2
// wavefronts of (T/2) x (T/2).
template <int T>
__device__ __forceinline__ void mainloop(uint8_t* smem, const Operand& A, const Operand& B,
                                         int64_t L, f32x16 (&acc)[T / 64][T / 64]) {
  constexpr int TM = T / 64, TN = T / 64;
  constexpr int LD_CH = T * CPR / 256;                // 16-byte chunks per thread per operand
  constexpr int SROWS = 2 * T / 256;                  // scale rows per thread (both operands)
  uint8_t* sq = smem;                                 // [2 bufs][2 operands][T][BK]
  uint8_t* ss = smem + 2 * 2 * T * BK;                // [2 bufs][2 operands][T][SCB]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5, r32 = lane & 31;

  // Loads go through buffer resources whose range ends at the operand's last
  // valid row, so the over-read of a ragged contraction tail on that row, or
  // of the stage after the last, returns zeros instead of touching memory
  // past the tensor. Offsets are 32-bit (the host checks (T + 1) * ld < 2^32).
  // Chunk i of operand o for this thread: row (tid >> 3) + 32 * i, chunk tid & 7.
  // Scale row s of this thread: operand so[s], row sr[s].
  const int crow = tid >> 3, cch = tid & 7;
  __amdgpu_buffer_rsrc_t rq[2], re[2];
  uint32_t off[2][LD_CH], eoff[SROWS];
#pragma unroll
  for (int o = 0; o < 2; ++o) {
    const Operand& X = o ? B : A;
    // the tile's rows only: a group may be longer, and the range must stay 32-bit
    const int64_t nrow = X.row_end - X.row0 < T ? X.row_end - X.row0 : T;
    rq[o] = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(X.q + X.row0 * X.ld), (short)0,
                                              uniform_u32(nrow * X.ld), kBufferWord3);
    re[o] = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(X.e + X.row0 * (X.ld / 32)), (short)0,
                                              uniform_u32(nrow * (X.ld / 32)), kBufferWord3);
#pragma unroll
    for (int i = 0; i < LD_CH; ++i) {
      const int64_t r = crow + 32 * i;
      const int64_t rr = r < nrow ? r : 0;      // a valid row
      off[o][i] = (uint32_t)(rr * X.ld + X.c0 + cch * 16);
    }
  }
  int sop[SROWS], srw[SROWS];
#pragma unroll
  for (int s2 = 0; s2 < SROWS; ++s2) {
    const int id = tid + 256 * s2;            // 0 .. 2T-1
    sop[s2] = __builtin_amdgcn_readfirstlane(id / T);   // the same for the whole wavefront
    srw[s2] = id % T;
    const Operand& X = sop[s2] ? B : A;
    const int64_t nrow = X.row_end - X.row0;
    const int64_t rs = srw[s2] < nrow ? srw[s2] : 0;
    eoff[s2] = (uint32_t)(rs * (X.ld / 32) + X.c0 / 32);
  }

  const int64_t nk = (L + BK - 1) / BK;
  if (nk == 0) return;
  u32x4 stq[2][LD_CH];
  uint8_t sts[SROWS][SCB];   // combined only when stored, so the loads stay in flight
  auto gload = [&](int64_t kt) {
    // the whole offset goes in the vector operand: the range check covers
    // only that part, not the scalar offset
    const uint32_t so = (uint32_t)(kt * BK), se = (uint32_t)(kt * SCB);
#pragma unroll
    for (int o = 0; o < 2; ++o)
#pragma unroll
      for (int i = 0; i < LD_CH; ++i)
        stq[o][i] = __builtin_amdgcn_raw_buffer_load_b128(rq[o], (int)(off[o][i] + so), 0, 0);
#pragma unroll
    for (int s2 = 0; s2 < SROWS; ++s2)
#pragma unroll
      for (int b = 0; b < SCB; ++b)
        sts[s2][b] = __builtin_amdgcn_raw_buffer_load_b8(sop[s2] ? re[1] : re[0],
                                                         (int)(eoff[s2] + se + b), 0, 0);
  };
  auto sstore = [&](int buf, int64_t kt) {
    // contraction elements at or past L are stored as zero (L is a multiple of 32)
    const int64_t c = kt * BK + cch * 16;
    const uint32_t m = c < L ? ~0u : 0u;
    const int64_t rem = L - kt * BK;
    const uint32_t smask = rem >= BK ? ~0u : (rem <= 0 ? 0u : ((1u << (8 * (rem / 32))) - 1u));
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      uint8_t* d = sq + (buf * 2 + o) * T * BK;
#pragma unroll
      for (int i = 0; i < LD_CH; ++i)
        *reinterpret_cast<u32x4*>(d + swz(crow + 32 * i, cch)) = stq[o][i] & m;
    }
#pragma unroll
    for (int s2 = 0; s2 < SROWS; ++s2) {
      uint8_t* d = ss + ((buf * 2 + sop[s2]) * T + srw[s2]) * SCB;
#pragma unroll
      for (int b = 0; b < SCB; ++b) d[b] = sts[s2][b] & (uint8_t)(smask >> (8 * b));
    }
  };

  // Operand layout of the 64-deep block-scaled MFMA: lane l supplies elements
  // 16*(l/32) .. +15 of the step's MX block 0 in bytes 0-15 and the same
  // elements of MX block 1 in bytes 16-31; its scale is the one of row l%32,
  // MX block l/32. A row's four stage scales are read as one word, shifted so
  // that byte 2*ks of it is this lane's block of step ks (selected by op_sel).
  struct Frag {
    i32x8 a[TM], b[TN];
  };
  auto read_frags = [&](const uint8_t* qa, const uint8_t* qb, int ks, Frag& f) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * TM * 32 + i * 32 + r32;
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(qa + swz(r, 4 * ks + half));
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(qa + swz(r, 4 * ks + 2 + half));
      f.a[i] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                     (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn * TN * 32 + j * 32 + r32;
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(qb + swz(r, 4 * ks + half));
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(qb + swz(r, 4 * ks + 2 + half));
      f.b[j] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                     (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    }
  };

  gload(0);
  sstore(0, 0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    // Stage kt+1 is loaded (and stored) even after the last stage: the read
    // stays inside the buffer range and the LDS buffer is not read again.
    // Keeping the body free of branches lets its parts be interleaved.
    gload(kt + 1);
    const uint8_t* qa = sq + (cur * 2 + 0) * T * BK;
    const uint8_t* qb = sq + (cur * 2 + 1) * T * BK;
    const uint32_t* sa = reinterpret_cast<const uint32_t*>(ss + (cur * 2 + 0) * T * SCB);
    const uint32_t* sb = reinterpret_cast<const uint32_t*>(ss + (cur * 2 + 1) * T * SCB);
    int32_t asc[TM], bsc[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) asc[i] = (int32_t)(sa[wm * TM * 32 + i * 32 + r32] >> (8 * half));
#pragma unroll
    for (int j = 0; j < TN; ++j) bsc[j] = (int32_t)(sb[wn * TN * 32 + j * 32 + r32] >> (8 * half));
    Frag f0, f1;
    read_frags(qa, qb, 0, f0);
    read_frags(qa, qb, 1, f1);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            f0.a[i], f0.b[j], acc[i][j], 0 /*A: E4M3*/, 0 /*B: E4M3*/, 0, asc[i], 0, bsc[j]);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            f1.a[i], f1.b[j], acc[i][j], 0, 0, 2 /*byte 2*/, asc[i], 2, bsc[j]);
    sstore(cur ^ 1, kt + 1);
    // Issue order: next-stage loads, scale words and step-0 fragments, then
    // step-0 MFMAs interleaved with the step-1 fragment reads, then step-1
    // MFMAs interleaved with the LDS stores of the next stage.
    constexpr int NL = 2 * LD_CH + SROWS * SCB;
    constexpr int NR = 2 * (TM + TN);
    constexpr int NM = TM * TN;
    constexpr int NW = 2 * LD_CH + SROWS * SCB;
    __builtin_amdgcn_sched_group_barrier(0x020, NL, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NR + TM + TN, 0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, (NR + NM - 1) / NM, 0);
    }
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, (NW + NM - 1) / NM, 0);
    }
    __syncthreads();
  }
}

template <int TM>
__device__ __forceinline__ void zero(f32x16 (&acc)[TM][TM]) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
}

// Live dgrad tile t -> (group, first row, row end, n-tile over K).
__device__ __forceinline__ bool dgrad_tile(const int64_t* __restrict__ offsets, int G, int64_t t,
                                           int64_t ntn, int BM, int& g, int64_t& row0,
                                           int64_t& row_end, int64_t& nt) {
  for (int e = 0; e < G; ++e) {
    const int64_t a = offsets[e], b = offsets[e + 1];
    const int64_t mt = (b - a + BM - 1) / BM;
    if (t < mt * ntn) {
      g = e;
      nt = t / mt;
      row0 = a + (t % mt) * BM;
      row_end = b;
      return true;
    }
    t -= mt * ntn;
  }
  return false;
}

// Second operand of the grouped row x row GEMM: group g's rows are
// row_step * g + (output column), its contraction starts at c0_step * g.
struct BLayout {
  int64_t ld, c0_step, row_step;
};

template <int T, bool OUT_BF16>
__global__ __launch_bounds__(256, 1) void k_dgrad(const uint8_t* __restrict__ dy,
                                                  const uint8_t* __restrict__ dye,
                                                  const uint8_t* __restrict__ w,
                                                  const uint8_t* __restrict__ we,
                                                  const int64_t* __restrict__ offsets, int G,
                                                  int64_t L, int64_t ncols, BLayout bl,
                                                  void* __restrict__ dx) {
  constexpr int BM = T, BN = T, TM = T / 64, TN = T / 64;
  extern __shared__ uint8_t smem[];
  const int64_t N = L, K = ncols;                 // contraction, output columns
  const int64_t ntn = K / BN;
  int64_t live = 0;
  for (int e = 0; e < G; ++e) live += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
  live *= ntn;
  if ((int64_t)blockIdx.x >= live) return;
  int g;
  int64_t row0, row_end, nt;
  dgrad_tile(offsets, G, xcd_tile(blockIdx.x, live), ntn, BM, g, row0, row_end, nt);
  const int64_t k0 = nt * BN;
  Operand A{dy, dye, N, 0, row0, row_end};
  const int64_t br0 = (int64_t)g * bl.row_step + k0;
  Operand B{w, we, bl.ld, (int64_t)g * bl.c0_step, br0, br0 + BN};
  f32x16 acc[TM][TN];
  zero<TM>(acc);
  mainloop<T>(smem, A, B, N, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, half = lane >> 5;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t row = row0 + wm * TM * 32 + i * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
      if (row >= row_end) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = k0 + wn * TN * 32 + j * 32 + (lane & 31);
        if constexpr (OUT_BF16)
          static_cast<uint16_t*>(dx)[row * K + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][e]);
        else
          static_cast<float*>(dx)[row * K + col] = acc[i][j][e];
      }
    }
}

template <int T>
__global__ __launch_bounds__(256, 1) void k_wgrad(const uint8_t* __restrict__ dyT,
                                                  const uint8_t* __restrict__ dyTe,
                                                  const uint8_t* __restrict__ xT,
                                                  const uint8_t* __restrict__ xTe,
                                                  const int64_t* __restrict__ padded, int G,
                                                  int64_t P, int64_t N, int64_t K,
                                                  float* __restrict__ dw) {
  constexpr int BM = T, BN = T, TM = T / 64, TN = T / 64;
  extern __shared__ uint8_t smem[];
  // A tile's cost grows with its group's token count, so the groups are taken
  // longest first (ties by index): workgroups are dispatched in index order,
  // and the longest tiles start first. Within a group, tiles are n-major; with
  // tk a multiple of 8 every XCD keeps the same k-tiles of all n-tiles.
  const int64_t tn = N / BM, tk = K / BN, per = tn * tk;
  const int64_t rank = blockIdx.x / per, rem = blockIdx.x % per;
  int g = 0;
  if (G > 1) {
    int* seg = reinterpret_cast<int*>(smem);    // [G] segment lengths, then the answer
    for (int h = threadIdx.x; h < G; h += 256) seg[h] = (int)(padded[h + 1] - padded[h]);
    __syncthreads();
    for (int h = threadIdx.x; h < G; h += 256) {
      const int lh = seg[h];
      int rk = 0;
      for (int e = 0; e < G; ++e) {
        const int le = seg[e];
        rk += (le > lh) | ((le == lh) & (e < h));
      }
      if (rk == rank) seg[G] = h;
    }
    __syncthreads();
    g = seg[G];
    __syncthreads();    // the main loop reuses the memory
  }
  const int64_t n0 = (rem / tk) * BM, k0 = (rem % tk) * BN;
  const int64_t c0 = padded[g];
  const int64_t L = padded[g + 1] - c0;
  Operand A{dyT, dyTe, P, c0, n0, n0 + BM};
  Operand B{xT, xTe, P, c0, k0, k0 + BN};
  f32x16 acc[TM][TN];
  zero<TM>(acc);
  mainloop<T>(smem, A, B, L, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, half = lane >> 5;
  float* out = dw + (int64_t)g * N * K;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t row = n0 + wm * TM * 32 + i * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = k0 + wn * TN * 32 + j * 32 + (lane & 31);
        out[row * K + col] = acc[i][j][e];
      }
    }
}

// ---------------------------------------------------------------------------
// BM x BN tiles (256 x 256 or 320 x 128) through an LDS ring filled by DMA.
//
// The operands' code bytes go from global memory straight into LDS (buffer
// loads with the LDS-destination bit), four 64-element stages in flight, so
// the wavefronts hold no staging registers for them. A stage is BM (A) and
// BN (B) rows x 64 bytes (16-byte pieces, piece c of row r at position
// c ^ chunk_key(r), so the rows of a read phase hit distinct banks).
// Each stage is one 64-deep MFMA step; the fragments of stage kt+1 are read
// from LDS while the MFMAs of stage kt run.
//
// The E8M0 scales (two bytes per row and stage) come in blocks of SB = 4
// stages: each thread loads the 12 bytes from the dword below a row's 8
// bytes (the row's scales for 4 stages start at whatever byte alignment the
// group's contraction offset and the row pitch give; buffer loads address
// whole dwords), shifts the 8 out with v_alignbyte and writes them to a
// two-block LDS ring, [block % 2][row][12] (8 bytes used).
// Loaded per stage, one byte per lane, they cost one cache line per lane and
// byte: twice the line traffic of the codes themselves.
//
// A ragged contraction end (wgrad) is a multiple of 32: when the last stage
// holds only its first MX block, the second block's bytes are zeroed in the
// fragments and its scale set to 1.
constexpr int DK = 64;                                // contraction elements per stage
constexpr int DS = 4;                                 // stages in the ring
constexpr int SB = 4;                                 // stages per scale block (8 bytes a row)
#ifndef NVFP4MOE_DMA_WN256
#define NVFP4MOE_DMA_WN256 4
#endif
// wavefront columns of a 256 x 256 tile: 4 (eight wavefronts, two per SIMD) or 2
constexpr int kDmaWn256 = NVFP4MOE_DMA_WN256;
static_assert(kDmaWn256 == 2 || kDmaWn256 == 4, "2 or 4 wavefront columns");
#ifndef NVFP4MOE_DMA_PERSIST
#define NVFP4MOE_DMA_PERSIST 1
#endif
constexpr bool kDmaPersist = NVFP4MOE_DMA_PERSIST != 0;
constexpr size_t kDmaMaxPreBytes = 16384;              // persistent tile-count scan (G < 4096)

// Workgroup tile BM x BN (rows of A x rows of B), 2 x WN wavefronts of
// (BM/2) x (BN/WN), that is TM x TN MFMA tiles of 32 x 32 each: WN = 2 puts
// one wavefront on each SIMD, WN = 4 two (so one's loads and barrier waits
// overlap the other's MFMAs). A code DMA instruction fills 16 rows, so every
// wavefront issues NL = (BM + BN) / (16 NW) loads per stage; a scale block is
// NSL loads per thread (row t, t + 64 NW, ... of the BM + BN rows; threads
// past the last row load row 0 into a spare slot, so every wavefront issues
// the same count).
template <int BM, int BN, int WN = 2>
struct DmaTile {
  static constexpr int NW = 2 * WN;                   // wavefronts
  static constexpr int NT = 64 * NW;                  // threads
  static constexpr int TM = BM / 64, TN = BN / (32 * WN);
  static constexpr int CA = BM / (16 * NW), CB = BN / (16 * NW);   // code loads per stage, wavefront
  static constexpr int NL = CA + CB;
  static constexpr int R = BM + BN;                   // scale rows
  static constexpr int NSL = (R + NT - 1) / NT;       // scale loads per thread and block
  static constexpr int A0 = 0, B0 = BM * DK;          // code planes [rows][64]
  static constexpr int STAGE = (BM + BN) * DK;
  // a row's 8 scale bytes of a block at a 12-byte pitch (3 dwords: the 32
  // consecutive rows of a byte read fall in 32 distinct banks)
  static constexpr int SP = 12;
  static constexpr int SBLK = (NSL * NT) * SP;        // one scale block, spare rows included
  static constexpr int SC = DS * STAGE;               // scale ring after the code stages
  static constexpr int LDS = SC + 2 * SBLK;
  static_assert(BM % 64 == 0 && BN % (32 * WN) == 0 && BM % (16 * NW) == 0 &&
                BN % (16 * NW) == 0 && BN % 64 == 0, "tile shape");
};

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt vmcnt(N) [lgkmcnt(0)] then s_barrier (N an immediate: the tile
// shapes' load counts)
template <int N, bool LGKM = false>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N == 4 || N == 5 || N == 7 || N == 8 || N == 9 || N == 10 || N == 14 || N == 16,
                "add the count");
#define NVFP4MOE_WAIT(n)                                                              \
  if constexpr (N == n) {                                                             \
    if constexpr (LGKM) asm volatile("s_waitcnt vmcnt(" #n ") lgkmcnt(0)\n\ts_barrier" ::: "memory"); \
    else asm volatile("s_waitcnt vmcnt(" #n ")\n\ts_barrier" ::: "memory");           \
  }
  NVFP4MOE_WAIT(4) NVFP4MOE_WAIT(5) NVFP4MOE_WAIT(7) NVFP4MOE_WAIT(8) NVFP4MOE_WAIT(9)
  NVFP4MOE_WAIT(10) NVFP4MOE_WAIT(14) NVFP4MOE_WAIT(16)
#undef NVFP4MOE_WAIT
}

// Workgroup tile BM x BN, 2 x WN wavefronts. (A class template's member
// rather than a function template: the kernels that call it are templates
// whose host-side instantiation would otherwise reject the device-only
// callee.)
template <int BM, int BN, int WN>
struct DmaLoop {
  using C = DmaTile<BM, BN, WN>;
static __device__ __forceinline__ void run(uint8_t* lsm, const Operand& A, const Operand& B,
                                           int64_t L, f32x16 (&acc)[C::TM][C::TN]) {
  constexpr int TM = C::TM, TN = C::TN, NL = C::NL, NSL = C::NSL, NW = C::NW, NT = C::NT;
  // the thread index through an empty asm: everything derived from it is
  // computed here, per tile, rather than hoisted out of a persistent
  // kernel's tile loop and held (spilled) across it
  int tid_ = threadIdx.x;
  asm volatile("" : "+v"(tid_));
  const int tid = tid_, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5, r32 = lane & 31;
  const int64_t nk = (L + DK - 1) / DK;
  if (nk == 0) return;

  __amdgpu_buffer_rsrc_t rq[2], re[2];
  int nrow[2];
  int64_t ld[2], c0[2];
#pragma unroll
  for (int o = 0; o < 2; ++o) {
    const Operand& X = o ? B : A;
    const int64_t cap = o ? BN : BM;
    const int64_t n = X.row_end - X.row0 < cap ? X.row_end - X.row0 : cap;   // the tile's rows
    nrow[o] = __builtin_amdgcn_readfirstlane((int)n);
    ld[o] = X.ld;
    c0[o] = X.c0;
    rq[o] = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(X.q + X.row0 * X.ld), (short)0,
                                              uniform_u32(n * X.ld), kBufferWord3);
    re[o] = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(X.e + X.row0 * (X.ld / 32)), (short)0,
                                              uniform_u32(n * (X.ld / 32)), kBufferWord3);
  }
  // lane offsets: code instruction i of this wavefront fills rows 16m .. 16m+15
  // (m = NW i + wave; lane: row 16m + lane/4, position lane%4)
  constexpr int CM = C::CA > C::CB ? C::CA : C::CB;
  uint32_t oq[2][CM];
#pragma unroll
  for (int o = 0; o < 2; ++o)
#pragma unroll
    for (int i = 0; i < (o ? C::CB : C::CA); ++i) {
      const int row = 16 * (NW * i + wave) + (lane >> 2);
      const int piece = (lane & 3) ^ chunk_key(row);
      const int rr = row < nrow[o] ? row : 0;
      oq[o][i] = (uint32_t)(rr * ld[o] + c0[o] + piece * 16);
    }
  // stage kt -> buffer kt % DS; past the end: offsets outside the ranges
  // (zeros, no memory traffic) so every stage has the same load count.
  // Load d of a stage: A's code loads first, then B's.
  auto issue_one = [&](int64_t kt, int d) {
    uint8_t* st = lsm + (kt % DS) * C::STAGE;
    const bool real = kt < nk;
    const uint32_t away = real ? 0u : 0x40000000u;
    const uint32_t kq = real ? (uint32_t)(kt * DK) : 0u;
    const int o = d < C::CA ? 0 : 1, i = d < C::CA ? d : d - C::CA;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rq[o], (lds_void*)(st + (o ? C::B0 : C::A0) + (NW * i + wave) * 1024), 16,
        oq[o][i] + kq + away, 0, 0, 0);
  };
  // scale rows of this thread: row q = tid + NT u of the BM + BN (A first);
  // rows past the tile's valid rows read the tile's first row; q >= BM + BN
  // (spare slots) read row 0 of A
  uint32_t eo[NSL], esh[NSL];          // dword-aligned offset, byte shift
  bool eb_[NSL];
#pragma unroll
  for (int u = 0; u < NSL; ++u) {
    const int q = tid + NT * u;
    const int o = q < BM ? 0 : (q < C::R ? 1 : 0);
    const int rr0 = q < BM ? q : (q < C::R ? q - BM : 0);
    const int rr = rr0 < nrow[o] ? rr0 : 0;
    // the operand is the same across a wavefront (BM and BM + BN are
    // multiples of 64): a scalar select of the buffer descriptor
    eb_[u] = __builtin_amdgcn_readfirstlane(o) == 1;
    const uint32_t byte_off = (uint32_t)(rr * (ld[o] / 32) + c0[o] / 32);
    eo[u] = byte_off & ~3u;
    esh[u] = byte_off & 3u;
  }
  typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x3v __attribute__((ext_vector_type(3)));
  u32x3v sreg[NSL];
  // block blk's 8 bytes of each of this thread's rows into registers (past
  // the operand's end the loads return zeros; bytes past the contraction's
  // end belong to stages that are masked below)
  auto load_scales = [&](int64_t blk) {
    const uint32_t off = (uint32_t)(blk * 2 * SB);
#pragma unroll
    for (int u = 0; u < NSL; ++u)
      sreg[u] = __builtin_bit_cast(
          u32x3v, __builtin_amdgcn_raw_buffer_load_b96(eb_[u] ? re[1] : re[0], eo[u] + off, 0, 0));
  };
  auto store_scales = [&](int64_t blk) {
    uint8_t* d = lsm + C::SC + (blk & 1) * C::SBLK;
#pragma unroll
    for (int u = 0; u < NSL; ++u) {
      const u32x2v w = {__builtin_amdgcn_alignbyte(sreg[u][1], sreg[u][0], esh[u]),
                        __builtin_amdgcn_alignbyte(sreg[u][2], sreg[u][1], esh[u])};
      uint32_t* q = reinterpret_cast<uint32_t*>(d + (tid + NT * u) * C::SP);
      q[0] = w[0];
      q[1] = w[1];
    }
  };

  // fragment addresses (stage-relative) and scale rows (block-relative) of
  // fragment 0; fragment i sits i * 32 rows further (same swizzle: the piece
  // position depends on row bits 2-3 only), a constant offset
  int fa[2], fb[2];
  const int ra0 = wm * (BM / 2) + r32, rb0 = wn * (BN / WN) + r32;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    fa[c] = C::A0 + ra0 * DK + (((2 * c + half) ^ chunk_key(ra0)) << 4);
    fb[c] = C::B0 + rb0 * DK + (((2 * c + half) ^ chunk_key(rb0)) << 4);
  }
  const int sa = C::SC + ra0 * C::SP + half, sbo = C::SC + (BM + rb0) * C::SP + half;
  // Fragments: A single-buffered (fragment i of the next stage is read into
  // the registers of this stage's fragment i right after its last MFMA), B
  // double-buffered (every MFMA of a stage row uses all of B). The scale
  // bytes follow their fragments.
  i32x8 fa_[TM], fb_[2][TN];
  int32_t fas[TM], fbs[2][TN];
  auto stage_ptrs = [&](int64_t kt, const uint8_t*& p0, const uint8_t*& p1, const uint8_t*& ps,
                        int f0, int f1, int fs) {
    const uint8_t* st = lsm + (kt % DS) * C::STAGE;
    p0 = st + f0;
    p1 = st + f1;
    // stage kt's scale bytes: block kt / SB in the ring, bytes 2 (kt % SB) + half
    ps = lsm + fs + (int)(((kt / SB) & 1) * C::SBLK + 2 * (kt % SB));
  };
  auto frag = [&](const uint8_t* p0, const uint8_t* p1, int at) {
    const u32x4 x0 = *reinterpret_cast<const u32x4*>(p0 + at);
    const u32x4 x1 = *reinterpret_cast<const u32x4*>(p1 + at);
    return i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                 (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  };
  // Contraction elements past L are zero: MX block 1 of a last stage that
  // holds 32 elements, and whole stages past the end (the loop runs an even
  // number of stages; their DMAs already gave zero codes, the masks also
  // neutralise the scale bytes there). Applied, on a uniform branch, only to
  // a stage that ends past L.
  auto mask = [&](int64_t kt, auto pb) {
    constexpr int PB = decltype(pb)::value;
    const int64_t rem = L - kt * DK;
    const int keep0 = rem > 0 ? -1 : 0, keep1 = rem > 32 ? -1 : 0;
    const int keeps = half ? keep1 : keep0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        fa_[i][e] &= keep0;
        fa_[i][e + 4] &= keep1;
      }
      fas[i] = keeps ? fas[i] : 127;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        fb_[PB][j][e] &= keep0;
        fb_[PB][j][e + 4] &= keep1;
      }
      fbs[PB][j] = keeps ? fbs[PB][j] : 127;
    }
  };

  static_assert(DS == 4 && 2 * NL < 64, "the wait counts assume 4 stages, NL loads per stage");
  static_assert(SB == 4, "a loop iteration is half a scale block");
  // prologue: scale block 0 to LDS, stages 0-2 in flight; once stage 0 has
  // landed and the scale writes are done, everybody may read stage 0
  load_scales(0);
#pragma unroll
  for (int p = 0; p < DS - 1; ++p)
#pragma unroll
    for (int d = 0; d < NL; ++d) issue_one(p, d);
  store_scales(0);
  wait_vm_barrier<2 * NL, true>();
  {
    const uint8_t *pa0, *pa1, *psa, *pb0, *pb1, *psb;
    stage_ptrs(0, pa0, pa1, psa, fa[0], fa[1], sa);
    stage_ptrs(0, pb0, pb1, psb, fb[0], fb[1], sbo);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      fa_[i] = frag(pa0, pa1, i * 32 * DK);
      fas[i] = psa[i * 32 * C::SP];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      fb_[0][j] = frag(pb0, pb1, j * 32 * DK);
      fbs[0][j] = psb[j * 32 * C::SP];
    }
  }
  // One stage: the MFMAs of stage kt_read - 1 (B buffer PB) in TM rows of TN;
  // after row i, A fragment i of stage kt_read; B fragment j of stage kt_read
  // (into the other buffer) and the NL DMA issues of stage kt_issue spread
  // over the rows. MASK: the stage may end past L (then its fragments are
  // masked first).
  constexpr int PD = (NL + TM - 1) / TM;                 // DMA issues per row
  auto stage = [&](int64_t kt_issue, int64_t kt_read, auto pb, auto masked) {
    constexpr int PB = decltype(pb)::value, QB = 1 - PB;
    if constexpr (decltype(masked)::value) mask(kt_read - 1, pb);
    const uint8_t *pa0, *pa1, *psa, *pb0, *pb1, *psb;
    stage_ptrs(kt_read, pa0, pa1, psa, fa[0], fa[1], sa);
    stage_ptrs(kt_read, pb0, pb1, psb, fb[0], fb[1], sbo);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
        // B (output-column operand) first: the lane then holds 4 consecutive columns
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fb_[PB][j], fa_[i], acc[i][j], 0 /*E4M3*/, 0 /*E4M3*/, 0, fbs[PB][j], 0, fas[i]);
#pragma unroll
      for (int d = i * PD; d < (i + 1) * PD && d < NL; ++d) issue_one(kt_issue, d);
      fa_[i] = frag(pa0, pa1, i * 32 * DK);
      fas[i] = psa[i * 32 * C::SP];
      // B fragments of the next stage over the first rows (the first MFMAs of
      // the next stage need all of them)
      static_assert(TN <= TM, "one B fragment per row");
      if (i < TN) {
        const int j = i;
        fb_[QB][j] = frag(pb0, pb1, j * 32 * DK);
        fbs[QB][j] = psb[j * 32 * C::SP];
      }
      __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);                // the row's MFMAs
      __builtin_amdgcn_sched_group_barrier(0x020, PD, 0);                // its DMA issues
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);                 // its LDS reads
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // One scale block: runs stages kt .. kt+3 (kt = 4b) and reads stages kt+1
  // .. kt+4. After the first wait it loads block b+1's scales into registers;
  // in the third stage it writes them to the ring slot of block b-1, which
  // every wavefront finished reading with stage 4b, before the barrier that
  // precedes the read of stage 4b + 4. No branch inside (a branch lets the
  // compiler move one stage's MFMAs past the next barrier), except in the
  // masked last block, which stops after the stage that runs stage nk - 1.
  //
  // Waits: before a stage that reads stage k+1, every load but the most
  // recent NL (stage k+2's DMAs) is complete. The scale loads (NSL) go right
  // after the first wait, before that stage's DMAs, so the next wait allows
  // NL + NSL outstanding; they are complete at the wait after that, long
  // before the third stage writes them out.
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  auto block = [&](int64_t kt, auto masked) {
    constexpr bool M = decltype(masked)::value;
    wait_vm_barrier<NL>();
    load_scales(kt / SB + 1);
    stage(kt + DS - 1, kt + 1, P0{}, masked);
    if (M && kt + 1 >= nk) return;
    wait_vm_barrier<NL + NSL>();
    stage(kt + DS, kt + 2, P1{}, masked);
    if (M && kt + 2 >= nk) return;
    wait_vm_barrier<NL>();
    store_scales(kt / SB + 1);
    stage(kt + DS + 1, kt + 3, P0{}, masked);
    if (M && kt + 3 >= nk) return;
    wait_vm_barrier<NL, true>();                         // scale writes visible
    stage(kt + DS + 2, kt + 4, P1{}, masked);
  };
  const int64_t nfull = L / DK;                          // stages that end at or before L
  int64_t kt = 0;
  for (; kt + SB <= nfull; kt += SB) block(kt, std::false_type{});
  if (kt < nk) block(kt, std::true_type{});
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");      // ring drained, LDS free
}
};

// Epilogue through LDS: acc[i][j][4q+v] = C[row, col] with row = wm*128 + i*32
// + lane%32 and col = wn*128 + j*32 + 8q + 4*(lane/32) + v. Each wavefront
// stages 32-row blocks in LDS, then writes 16 bytes per lane along the rows.
// Workgroup tile (64 TM) x (64 TN), read from the accumulator array's shape.
template <typename OutT, int WN, int TM, int TN, typename Store>
__device__ __forceinline__ void store_tile_lds(uint8_t* lsm, const f32x16 (&acc)[TM][TN],
                                               int64_t rows_left, Store store) {
  constexpr int BM = 64 * TM;
  constexpr int ES = sizeof(OutT);
  constexpr int WC = 32 * TN;                          // columns of a wavefront
  constexpr int RS = WC * ES + 16;
  int tid_ = threadIdx.x;
  asm volatile("" : "+v"(tid_));                       // per tile (see DmaLoop)
  const int lane = tid_ & 63, wave = tid_ >> 6;
  const int wm = wave / WN, half = lane >> 5, r32 = lane & 31;
  uint8_t* ep = lsm + wave * (32 * RS);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint8_t* d = ep + r32 * RS + (j * 32 + 8 * q + 4 * half) * ES;
        if constexpr (ES == 2) {
          const uint32_t lo = pk_bf16(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
          const uint32_t hi = pk_bf16(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          *reinterpret_cast<uint2*>(d) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<float4*>(d) = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                                      acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
      }
    constexpr int PPR = WC * ES / 16;                // 16-byte pieces per row
#pragma unroll
    for (int it = 0; it < 32 * PPR / 64; ++it) {
      const int pc = it * 64 + lane, r = pc / PPR, c = pc % PPR;
      const u32x4 val = *reinterpret_cast<const u32x4*>(ep + r * RS + c * 16);
      const int lr = wm * (BM / 2) + i * 32 + r;     // tile row
      if (lr < rows_left) store(lr, c * 16 / ES, val);
    }
  }
}

// persist: the grid is at most one workgroup per compute unit, each looping
// over tiles v = blockIdx.x, blockIdx.x + gridDim.x, ...; the tile-count scan
// then sits in LDS after the ring. Otherwise one tile per workgroup (the
// scan's LDS is reused by the ring).
template <bool OUT_BF16, int BM, int BN, int WN>
__global__ __launch_bounds__(128 * WN, 1) void k_dgrad_dma(const uint8_t* __restrict__ dy,
                                                      const uint8_t* __restrict__ dye,
                                                      const uint8_t* __restrict__ w,
                                                      const uint8_t* __restrict__ we,
                                                      const int64_t* __restrict__ offsets, int G,
                                                      int64_t L, int64_t ncols, BLayout bl,
                                                      void* __restrict__ dx, int persist) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lsm[];
  const int64_t N = L, K = ncols;                 // contraction, output columns
  const int ntn = (int)(K / BN);
  int* pre = reinterpret_cast<int*>(persist ? lsm + DmaTile<BM, BN, WN>::LDS : lsm);
  tile_prefix(G, [&](int e) { return (int)((offsets[e + 1] - offsets[e] + BM - 1) / BM) * ntn; }, pre);
  const int total = pre[G];
  for (int v = (int)blockIdx.x;; v += (int)gridDim.x) {
    if (v >= total) return;
    int g, nt;
    int64_t row0, row_end;
    {
      const int t = (int)xcd_tile(v, total);
      g = tile_group(pre, G, t);
      const int loc = t - pre[g];
      const int64_t a = offsets[g];
      row_end = offsets[g + 1];
      const int mt = (int)((row_end - a + BM - 1) / BM);
      // Within a group, tiles go in blocks of 4 n-tiles, m-tiles then n-tiles
      // inside a block, so the ~32 consecutive tiles one XCD runs together
      // share 8 A tiles and 4 B tiles in its L2.
      int mi, ni;
      block_order(loc, mt, ntn, mi, ni);
      nt = ni;
      row0 = a + (int64_t)mi * BM;
      __syncthreads();   // the scan's memory (one tile) or the last epilogue's staging is reused
    }
    const int64_t k0 = (int64_t)nt * BN;
    Operand A{dy, dye, N, 0, row0, row_end};
    const int64_t br0 = (int64_t)g * bl.row_step + k0;
    Operand B{w, we, bl.ld, (int64_t)g * bl.c0_step, br0, br0 + BN};
    constexpr int TM = DmaTile<BM, BN, WN>::TM, TN = DmaTile<BM, BN, WN>::TN;
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    DmaLoop<BM, BN, WN>::run(lsm, A, B, N, acc);
    const int64_t col0 = k0 + ((threadIdx.x >> 6) % WN) * (BN / WN);
    if constexpr (OUT_BF16)
      store_tile_lds<uint16_t, WN>(lsm, acc, row_end - row0, [&](int lr, int col, const u32x4& v) {
        // non-temporal: the gradients are read back much later, not from this L2
        __builtin_nontemporal_store(
            v, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(dx) + (row0 + lr) * K + col0 + col));
      });
    else
      store_tile_lds<float, WN>(lsm, acc, row_end - row0, [&](int lr, int col, const u32x4& v) {
        __builtin_nontemporal_store(
            v, reinterpret_cast<u32x4*>(static_cast<float*>(dx) + (row0 + lr) * K + col0 + col));
      });
    if (!persist) return;
  }
}

template <int WN>
__global__ __launch_bounds__(128 * WN, 1) void k_wgrad_dma(const uint8_t* __restrict__ dyT,
                                                      const uint8_t* __restrict__ dyTe,
                                                      const uint8_t* __restrict__ xT,
                                                      const uint8_t* __restrict__ xTe,
                                                      const int64_t* __restrict__ padded, int G,
                                                      int64_t P, int64_t N, int64_t K,
                                                      float* __restrict__ dw) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lsm[];
  // groups longest first (a tile's cost is its group's token count)
  const int64_t tn = N / 256, tk = K / 256, per = tn * tk;
  const int64_t rank = blockIdx.x / per, rem = blockIdx.x % per;
  int g = 0;
  if (G > 1) {
    int* seg = reinterpret_cast<int*>(lsm);
    for (int h = threadIdx.x; h < G; h += blockDim.x) seg[h] = (int)(padded[h + 1] - padded[h]);
    __syncthreads();
    for (int h = threadIdx.x; h < G; h += blockDim.x) {
      const int lh = seg[h];
      int rk = 0;
      for (int e = 0; e < G; ++e) {
        const int le = seg[e];
        rk += (le > lh) | ((le == lh) & (e < h));
      }
      if (rk == rank) seg[G] = h;
    }
    __syncthreads();
    g = seg[G];
    __syncthreads();
  }
  const int64_t n0 = (rem / tk) * 256, k0 = (rem % tk) * 256;
  const int64_t c0 = padded[g];
  const int64_t L = padded[g + 1] - c0;
  Operand A{dyT, dyTe, P, c0, n0, n0 + 256};
  Operand B{xT, xTe, P, c0, k0, k0 + 256};
  constexpr int TM = DmaTile<256, 256, WN>::TM, TN = DmaTile<256, 256, WN>::TN;
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  DmaLoop<256, 256, WN>::run(lsm, A, B, L, acc);
  float* out = dw + (int64_t)g * N * K;
  const int64_t col0 = k0 + ((threadIdx.x >> 6) % WN) * (256 / WN);
  store_tile_lds<float, WN>(lsm, acc, 256, [&](int lr, int col, const u32x4& v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + (n0 + lr) * K + col0 + col));
  });
}

template <int T>
constexpr size_t lds_bytes() { return (size_t)2 * 2 * T * BK + (size_t)2 * 2 * T * SCB; }

template <typename Kern>
hipError_t set_lds(Kern k, size_t bytes, bool& done) {
  if (done) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done = true;
  return e;
}

template <int T>
hipError_t dgrad_t(const uint8_t* dy, const uint8_t* dye, const uint8_t* w, const uint8_t* we,
                   const int64_t* offsets, int G, int64_t m_cap, int64_t L, int64_t ncols,
                   BLayout bl, void* dx, bool bf16, hipStream_t stream) {
  static bool done[2] = {false, false};
  const int64_t tiles = ((m_cap + T - 1) / T + G) * (ncols / T);   // bound on live tiles
  auto k = bf16 ? k_dgrad<T, true> : k_dgrad<T, false>;
  hipError_t e = set_lds(k, lds_bytes<T>(), done[bf16]);
  if (e != hipSuccess) return e;
  k<<<(unsigned)tiles, 256, lds_bytes<T>(), stream>>>(dy, dye, w, we, offsets, G, L, ncols, bl,
                                                      dx);
  return hipGetLastError();
}

template <int BM, int BN>
hipError_t rowxrow_dma(const uint8_t* a, const uint8_t* ae, const uint8_t* b, const uint8_t* be,
                       const int64_t* offsets, int G, int64_t m_cap, int64_t L, int64_t ncols,
                       BLayout bl, void* out, bool out_bf16, hipStream_t stream) {
  static bool done[2] = {false, false};
  // 256 x 256 tiles run eight wavefronts (two per SIMD, 2 x 4 of 128 x 64 each),
  // so one wavefront's MFMA chain covers the other's LDS reads and waits
  constexpr int WN = (BM == 256 && BN == 256) ? kDmaWn256 : 2;
  constexpr size_t ring = (size_t)DmaTile<BM, BN, WN>::LDS;
  static_assert(ring + kDmaMaxPreBytes <= 160 * 1024, "LDS budget of k_dgrad_dma");
  auto k = out_bf16 ? k_dgrad_dma<true, BM, BN, WN> : k_dgrad_dma<false, BM, BN, WN>;
  hipError_t e = set_lds(k, ring + kDmaMaxPreBytes, done[out_bf16]);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((m_cap + BM - 1) / BM + G) * (ncols / BN);   // bound on live tiles
  // Persistent (one workgroup per compute unit, looping over the tiles) when
  // the bound is well above what the compute units take in one round:
  // workgroups past the live tiles only start and exit, but the dispatcher
  // issues them one after another (e.g. a capacity-sized call with 7x as
  // many tile slots as tiles).
  const int64_t cus = device_cu_count();
  const size_t pre_bytes = ((size_t)(G + 1) * 4 + 15) & ~(size_t)15;
  const bool persist = kDmaPersist && pre_bytes <= kDmaMaxPreBytes && tiles > 2 * cus;
  const size_t lds = ring + (persist ? pre_bytes : 0);
  const int64_t grid = persist ? cus : tiles;
  k<<<(unsigned)grid, 128 * WN, lds, stream>>>(a, ae, b, be, offsets, G, L, ncols, bl, out,
                                               persist ? 1 : 0);
  return hipGetLastError();
}

// Grouped row x row MXFP8 GEMM: out[r, c] = sum_l A[r, l] * B(g)[c, l] for the
// rows r of group g, out [m_cap, ncols] row-major.
hipError_t launch_rowxrow(const uint8_t* a, const uint8_t* ae, const uint8_t* b,
                          const uint8_t* be, const int64_t* offsets, int G, int64_t m_cap,
                          int64_t L, int64_t ncols, BLayout bl, void* out, bool out_bf16,
                          hipStream_t stream) {
  if (m_cap == 0 || G == 0) return hipSuccess;
  if (ncols % 256 == 0 && m_cap >= 256 * (int64_t)G && G <= 8192) {
    // 320 x 128 tiles when about one round of them covers the problem: then
    // they keep every compute unit busy where 256 x 256 tiles leave many idle
    // (e.g. 8 groups of ~1024 rows, 1024 columns: ~144 tiles of 256 x 256 on
    // 256 compute units; 256 tiles of 320 x 128)
    const int64_t cus = device_cu_count();
    const int64_t est = (m_cap / 320 + G / 2) * (ncols / 128);
    if (est <= cus) return rowxrow_dma<320, 128>(a, ae, b, be, offsets, G, m_cap, L, ncols, bl, out,
                                                 out_bf16, stream);
    return rowxrow_dma<256, 256>(a, ae, b, be, offsets, G, m_cap, L, ncols, bl, out, out_bf16,
                                 stream);
  }
  return dgrad_t<128>(a, ae, b, be, offsets, G, m_cap, L, ncols, bl, out, out_bf16, stream);
}

template <int T>
hipError_t wgrad_t(const uint8_t* dyT, const uint8_t* dyTe, const uint8_t* xT, const uint8_t* xTe,
                   const int64_t* padded, int G, int64_t P, int64_t N, int64_t K, float* dw,
                   hipStream_t stream) {
  static bool done = false;
  hipError_t e = set_lds(k_wgrad<T>, lds_bytes<T>(), done);
  if (e != hipSuccess) return e;
  const int64_t tiles = (int64_t)G * (N / T) * (K / T);
  k_wgrad<T><<<(unsigned)tiles, 256, lds_bytes<T>(), stream>>>(dyT, dyTe, xT, xTe, padded, G, P, N,
                                                             K, dw);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dgrad(const uint8_t* dy, const uint8_t* dye, const uint8_t* w,
                        const uint8_t* we, const int64_t* offsets, int G, int64_t m_cap,
                        int64_t N, int64_t K, void* dx, bool dx_bf16, hipStream_t stream) {
  // W8 [G, K, N]: group g's K rows start at row g*K, row stride N, the
  // contraction from 0 (each expert's block contiguous: a tile's 256 rows
  // span 256 N bytes, not 256 G N)
  return launch_rowxrow(dy, dye, w, we, offsets, G, m_cap, N, K, BLayout{N, 0, K}, dx, dx_bf16,
                        stream);
}

hipError_t launch_fwd_mxfp8(const uint8_t* x, const uint8_t* xe, const uint8_t* w,
                            const uint8_t* we, const int64_t* offsets, int G, int64_t m_cap,
                            int64_t N, int64_t K, void* y, bool y_bf16, hipStream_t stream) {
  // W8 [G*N, K]: group g's rows start at g*N, contraction from 0
  return launch_rowxrow(x, xe, w, we, offsets, G, m_cap, K, N, BLayout{K, 0, N}, y, y_bf16,
                        stream);
}

hipError_t launch_wgrad(const uint8_t* dyT, const uint8_t* dyTe, const uint8_t* xT,
                        const uint8_t* xTe, const int64_t* padded, int G, int64_t P, int64_t N,
                        int64_t K, float* dw, hipStream_t stream) {
  if (G == 0) return hipSuccess;
  if (N % 256 == 0 && K % 256 == 0) {
    static bool done = false;
    constexpr int WN = kDmaWn256;
    const size_t lds = (size_t)DmaTile<256, 256, WN>::LDS;
    hipError_t e = set_lds(k_wgrad_dma<WN>, lds, done);
    if (e != hipSuccess) return e;
    const int64_t tiles = (int64_t)G * (N / 256) * (K / 256);
    k_wgrad_dma<WN><<<(unsigned)tiles, 128 * WN, lds, stream>>>(dyT, dyTe, xT, xTe, padded, G, P, N,
                                                                K, dw);
    return hipGetLastError();
  }
  return wgrad_t<128>(dyT, dyTe, xT, xTe, padded, G, P, N, K, dw, stream);
}

}  // namespace nvfp4moe
