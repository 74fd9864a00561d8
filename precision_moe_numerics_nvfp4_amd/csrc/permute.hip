// Token-to-expert grouping, group-offset scans and the NVFP4 row gather.
//
// Pages: each token is routed to 8 of 384 experts ("Thinking Machines' Inkling
// 2 Small Trains a 594B Model in 68 Hours", section "594B weights, 17B at
// work") and travels to them already in NVFP4 ("Inkling 2 Small uses four-bit
// training ...", section "Quantized NVLink and BBBK"). On one GPU this is a
// stable counting sort of the (token, slot) pairs by local expert plus a copy
// of each routed token's NVFP4 row.
//
// Small inputs (at most 16384 pairs) take one launch: each workgroup owns 64
// consecutive flat pairs, reads all expert ids (a few tens of KB from L2),
// builds in LDS the per-expert totals and the per-expert counts of the pairs
// before its own, scans them into its output bases, ranks its 64 pairs with
// ballots and copies their rows. Workgroup 0 also writes the offsets.
//
// Larger inputs take three launches, no atomics on the output order:
//   1. histogram: one workgroup per chunk of 256 flat pairs counts pairs per
//      local expert (LDS atomics; only the counts depend on them) into
//      ws[e][chunk];
//   2. scan: one workgroup of 1024 threads turns the table into the first
//      output row of every (chunk, expert) run, in expert-major order. Thread
//      (e, part) owns a contiguous range of chunks of expert e; one block-wide
//      scan of the per-thread sums (threads ordered expert-major) gives every
//      range its start, and a second pass over the range writes the running
//      starts back. The same workgroup writes the offsets and the 32-padded
//      offsets;
//   3. scatter + copy: one workgroup per chunk, one pair per thread. Lanes of a
//      wavefront holding the same expert find each other with one ballot per
//      bit of the expert index, so a pair's rank among earlier pairs of its
//      expert is a popcount; per-wavefront counts in LDS give the rank across
//      the workgroup. Row order inside an expert is flat index order.
// In both forms the workgroup then copies the NVFP4 rows (codes, scales, outer
// scale) of its routed pairs to their output rows: all 256 threads walk the
// (row, 16-byte piece) pairs with eight loads in flight before the stores.
#include <mutex>

#include "codecs.hpp"
#include "internal.hpp"

namespace nvfp4moe {

namespace {

constexpr int kChunk = 256;   // flat pairs per workgroup in passes 1 and 3
constexpr int kScanRegs = 32; // table entries a scan thread keeps in registers

// Copy the NVFP4 rows lsrc[i] -> ldst[i], i < nv (lists in LDS), with the
// 256 threads of the workgroup. SC16: scale rows are whole 16-byte pieces
// (K % 256 == 0, both scale arrays 16-byte aligned); otherwise bytes.
template <bool SC16>
__device__ __forceinline__ void copy_rows(int nv, const int32_t* ldst, const int32_t* lsrc,
                                          const uint8_t* __restrict__ qc,
                                          const uint8_t* __restrict__ qs,
                                          const float* __restrict__ qo, int64_t K,
                                          uint8_t* __restrict__ pc, uint8_t* __restrict__ ps,
                                          float* __restrict__ po) {
  // No branches in a round: indices past the end are clamped to the last
  // item, whose bytes are then copied again to the same place (same value),
  // so the eight loads of a round are all in flight before the stores.
  const int tid = threadIdx.x;
  const int64_t rb = K / 2;                 // code bytes per row
  const int n16 = (int)(K / 32);
  const int items = nv * n16;
  for (int i0 = tid; i0 < items; i0 += 256 * 8) {
    uint4 v[8];
    int64_t d[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = min(i0 + 256 * u, items - 1);
      const int r = i / n16, c = i - r * n16;
      v[u] = *reinterpret_cast<const uint4*>(qc + (int64_t)lsrc[r] * rb + 16 * c);
      d[u] = (int64_t)ldst[r] * rb + 16 * c;
    }
    __builtin_amdgcn_sched_barrier(0);      // keep the loads ahead of the stores
#pragma unroll
    for (int u = 0; u < 8; ++u) *reinterpret_cast<uint4*>(pc + d[u]) = v[u];
  }
  const int64_t sb = K / 16;                // scale bytes per row
  if constexpr (SC16) {
    const int ns = (int)(K / 256);
    const int sitems = nv * ns;
    for (int i0 = tid; i0 < sitems; i0 += 256 * 4) {
      uint4 v[4];
      int64_t d[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = min(i0 + 256 * u, sitems - 1);
        const int r = i / ns, c = i - r * ns;
        v[u] = *reinterpret_cast<const uint4*>(qs + (int64_t)lsrc[r] * sb + 16 * c);
        d[u] = (int64_t)ldst[r] * sb + 16 * c;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) *reinterpret_cast<uint4*>(ps + d[u]) = v[u];
    }
  } else {
    const int ns = (int)sb;
    const int sitems = nv * ns;
    for (int i0 = tid; i0 < sitems; i0 += 256 * 8) {
      uint8_t v[8];
      int64_t d[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = min(i0 + 256 * u, sitems - 1);
        const int r = i / ns, c = i - r * ns;
        v[u] = qs[(int64_t)lsrc[r] * sb + c];
        d[u] = (int64_t)ldst[r] * sb + c;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) ps[d[u]] = v[u];
    }
  }
  for (int i = tid; i < nv; i += 256) po[ldst[i]] = qo[lsrc[i]];
}

// Exclusive scan of v over the 256 threads of the workgroup; returns the
// exclusive prefix and sets total. Ends with a barrier.
__device__ __forceinline__ int64_t block_scan_256(int64_t v, int64_t& total) {
  __shared__ int64_t sh4[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int64_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t u = __shfl_up(incl, d, 64);
    if (lane >= d) incl += u;
  }
  if (lane == 63) sh4[w] = incl;
  __syncthreads();
  int64_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t s = sh4[i];
    before += i < w ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + incl - v;
}

constexpr int kSmallChunk = 64;       // flat pairs per workgroup, one-launch form
constexpr int64_t kSmallMax = 16384;  // largest T*k taking the one-launch form

template <bool SC16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4))) void k_permute_small(
    const int32_t* __restrict__ ids, int64_t n, int k, int e0, int n_local, int nbits,
    const uint8_t* __restrict__ qc, const uint8_t* __restrict__ qs,
    const float* __restrict__ qo, int64_t K, int64_t* __restrict__ offsets,
    int64_t* __restrict__ padded, int32_t* __restrict__ row_token,
    int32_t* __restrict__ row_slot, int32_t* __restrict__ pair_row, uint8_t* __restrict__ pc,
    uint8_t* __restrict__ ps, float* __restrict__ po) {
  __shared__ int32_t tot[1024];   // pairs per local expert, all of them
  __shared__ int32_t pre[1024];   // pairs per local expert before this workgroup's
  __shared__ int32_t list_dst[kSmallChunk];
  __shared__ int32_t list_src[kSmallChunk];
  __shared__ int32_t nv_sh;
  const int tid = threadIdx.x;
  for (int e = tid; e < n_local; e += 256) {
    tot[e] = 0;
    pre[e] = 0;
  }
  __syncthreads();
  // Count: each wavefront takes 64 consecutive ids per step, eight steps'
  // loads in flight; lanes of one expert are grouped by ballots and only the
  // lowest lane of each group adds the group's size. A step lies wholly before
  // or wholly after this workgroup's pairs (both are 64-aligned).
  const int64_t f_lo = (int64_t)blockIdx.x * kSmallChunk;
  {
    const int lane = tid & 63, w = tid >> 6;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int64_t b0 = 64 * w; b0 < n; b0 += 256 * 8) {
      int lev[8];
      int raw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {          // unconditional loads (index clamped): no branches
        const int64_t f = b0 + 256 * u + lane;
        raw[u] = ids[f < n ? f : n - 1];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) lev[u] = b0 + 256 * u + lane < n ? raw[u] - e0 : -1;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int le = lev[u];
        const bool valid = (le >= 0) && (le < n_local);
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
          const bool bit = valid && ((le >> b) & 1);
          const uint64_t bal = __ballot(bit);
          peers &= bit ? bal : ~bal;
        }
        if (valid && (peers & below) == 0) {
          const int c = __popcll(peers);
          atomicAdd(&tot[le], c);
          if (b0 + 256 * u < f_lo) atomicAdd(&pre[le], c);
        }
      }
    }
  }
  __syncthreads();
  // expert starts: thread t scans experts 4t .. 4t+3
  int32_t c4[4], p4[4];
  int64_t s = 0, ps4 = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * tid + j;
    c4[j] = e < n_local ? tot[e] : 0;
    p4[j] = e < n_local ? pre[e] : 0;
    s += c4[j];
    ps4 += (c4[j] + 31) / 32 * 32;
  }
  int64_t total, ptotal;
  int64_t run = block_scan_256(s, total);
  int64_t prun = block_scan_256(ps4, ptotal);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * tid + j;
    if (e < n_local) {
      if (blockIdx.x == 0) {
        offsets[e] = run;
        padded[e] = prun;
      }
      pre[e] = (int32_t)run + p4[j];        // first output row of this workgroup's pairs of e
    }
    run += c4[j];
    prun += (c4[j] + 31) / 32 * 32;
  }
  if (blockIdx.x == 0 && tid == 0) {
    offsets[n_local] = total;
    padded[n_local] = ptotal;
  }
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    const int64_t f = f_lo + lane;
    int le = -1;
    if (f < n) le = ids[f] - e0;
    const bool valid = (le >= 0) && (le < n_local);
    uint64_t peers = __ballot(valid);
    const uint64_t vmask = peers;
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((le >> b) & 1);
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int pos = -1;
    if (valid) {
      pos = pre[le] + __popcll(peers & below);
      const int32_t t = (int32_t)(f / k);
      row_token[pos] = t;
      row_slot[pos] = (int32_t)(f % k);
      const int slot = __popcll(vmask & below);
      list_dst[slot] = pos;
      list_src[slot] = t;
    }
    if (pair_row && f < n) pair_row[f] = pos;
    if (lane == 0) nv_sh = __popcll(vmask);
  }
  __syncthreads();
  copy_rows<SC16>(nv_sh, list_dst, list_src, qc, qs, qo, K, pc, ps, po);
}

__global__ __launch_bounds__(256) void k_hist(const int32_t* __restrict__ ids, int64_t n, int e0,
                                              int n_local, int64_t n_chunks,
                                              int32_t* __restrict__ ws) {
  __shared__ int32_t cnt[1024];
  for (int e = threadIdx.x; e < n_local; e += 256) cnt[e] = 0;
  __syncthreads();
  const int64_t f = (int64_t)blockIdx.x * kChunk + threadIdx.x;
  if (f < n) {
    const int le = ids[f] - e0;
    if (le >= 0 && le < n_local) atomicAdd(&cnt[le], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < n_local; e += 256) ws[(int64_t)e * n_chunks + blockIdx.x] = cnt[e];
}

// Exclusive scan of v over the 1024 threads of the workgroup; returns the
// exclusive prefix and sets total. Ends with a barrier.
__device__ __forceinline__ int64_t block_scan_1024(int64_t v, int64_t& total) {
  __shared__ int64_t sh[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int64_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t u = __shfl_up(incl, d, 64);
    if (lane >= d) incl += u;
  }
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  int64_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t s = sh[i];
    before += i < w ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + incl - v;
}

__global__ __launch_bounds__(1024) void k_scan(int32_t* __restrict__ ws, int64_t n_chunks,
                                               int n_local, int64_t* __restrict__ offsets,
                                               int64_t* __restrict__ padded) {
  __shared__ int64_t start_of[1024];
  const int tid = threadIdx.x;
  const int parts = 1024 / n_local;               // threads per expert (n_local <= 1024)
  const int e = tid / parts, part = tid % parts;
  const bool active = e < n_local;
  const int64_t per = (n_chunks + parts - 1) / parts;
  const int64_t c0 = active ? (int64_t)part * per : 0;
  const int64_t c1 = active ? (c0 + per < n_chunks ? c0 + per : n_chunks) : 0;
  // the thread's chunks of expert e are contiguous in the table; an empty
  // range (c0 >= n_chunks, when parts * per overshoots the chunk count)
  // points at its expert's first entry
  const int cnt_c = (int)(c1 > c0 ? c1 - c0 : 0);
  int32_t* col = ws + (active ? (int64_t)e * n_chunks + (cnt_c > 0 ? c0 : 0) : 0);
  // First kScanRegs entries stay in registers across the block scan (the
  // whole range in the common case: one round of loads); longer ranges
  // re-read the rest in batches. Loads are unconditional: every range starts
  // inside the table and ends at most at its end, so a range plus
  // kScanRegs - 1 entries stays inside the workspace (the table and its 256
  // spare bytes), and entries past the range are masked to zero.
  int32_t a[kScanRegs];
  int32_t s = 0;
#pragma unroll
  for (int u = 0; u < kScanRegs; ++u) a[u] = col[u];
#pragma unroll
  for (int u = 0; u < kScanRegs; ++u) {
    a[u] = u < cnt_c ? a[u] : 0;
    s += a[u];
  }
  for (int b = kScanRegs; b < cnt_c; b += kScanRegs) {
    int32_t t[kScanRegs];
#pragma unroll
    for (int u = 0; u < kScanRegs; ++u) t[u] = col[b + u];
#pragma unroll
    for (int u = 0; u < kScanRegs; ++u) s += b + u < cnt_c ? t[u] : 0;
  }
  int64_t total;
  int64_t run = block_scan_1024(s, total);        // expert-major exclusive prefix
  start_of[tid] = run;
#pragma unroll
  for (int u = 0; u < kScanRegs; ++u) {
    if (u < cnt_c) col[u] = (int32_t)run;
    run += a[u];
  }
  for (int b = kScanRegs; b < cnt_c; b += kScanRegs) {
    int32_t t[kScanRegs];
#pragma unroll
    for (int u = 0; u < kScanRegs; ++u) t[u] = col[b + u];
#pragma unroll
    for (int u = 0; u < kScanRegs; ++u) {
      if (b + u < cnt_c) {
        col[b + u] = (int32_t)run;
        run += t[u];
      }
    }
  }
  __syncthreads();
  int64_t start = 0, cnt = 0;
  if (tid < n_local) {
    start = start_of[tid * parts];
    cnt = (tid + 1 < n_local ? start_of[(tid + 1) * parts] : total) - start;
  }
  int64_t ptotal;
  const int64_t pstart = block_scan_1024(tid < n_local ? (cnt + 31) / 32 * 32 : 0, ptotal);
  if (tid < n_local) {
    offsets[tid] = start;
    padded[tid] = pstart;
  }
  if (tid == 0) {
    offsets[n_local] = total;
    padded[n_local] = ptotal;
  }
}

template <bool SC16>
__global__ __launch_bounds__(256) void k_scatter_copy(
    const int32_t* __restrict__ ids, int64_t n, int k, int e0, int n_local, int nbits,
    int64_t n_chunks, const int32_t* __restrict__ ws, const uint8_t* __restrict__ qc,
    const uint8_t* __restrict__ qs, const float* __restrict__ qo, int64_t K,
    int32_t* __restrict__ row_token, int32_t* __restrict__ row_slot,
    int32_t* __restrict__ pair_row, uint8_t* __restrict__ pc, uint8_t* __restrict__ ps,
    float* __restrict__ po) {
  __shared__ int32_t base[1024];
  __shared__ int32_t wcnt[4][1024];     // pairs per expert in each wavefront
  __shared__ int32_t list_dst[kChunk];  // compacted (output row, token) of routed pairs
  __shared__ int32_t list_src[kChunk];
  __shared__ int32_t wvalid[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int e = tid; e < n_local; e += 256) {
    base[e] = ws[(int64_t)e * n_chunks + blockIdx.x];
    wcnt[0][e] = 0; wcnt[1][e] = 0; wcnt[2][e] = 0; wcnt[3][e] = 0;
  }
  __syncthreads();

  const int64_t f = (int64_t)blockIdx.x * kChunk + tid;
  int le = -1;
  if (f < n) le = ids[f] - e0;
  const bool valid = (le >= 0) && (le < n_local);
  uint64_t peers = __ballot(valid);
  const uint64_t vmask = peers;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = valid && ((le >> b) & 1);
    const uint64_t bal = __ballot(bit);
    peers &= bit ? bal : ~bal;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (valid && (peers & below) == 0) wcnt[w][le] = __popcll(peers);   // lowest lane of its expert
  if (lane == 0) wvalid[w] = __popcll(vmask);
  __syncthreads();
  int pos = -1;
  if (valid) {
    pos = base[le] + __popcll(peers & below);
    for (int i = 0; i < w; ++i) pos += wcnt[i][le];
    const int32_t t = (int32_t)(f / k);
    row_token[pos] = t;
    row_slot[pos] = (int32_t)(f % k);
    int slot = __popcll(vmask & below);
    for (int i = 0; i < w; ++i) slot += wvalid[i];
    list_dst[slot] = pos;
    list_src[slot] = t;
  }
  if (pair_row && f < n) pair_row[f] = pos;
  __syncthreads();

  copy_rows<SC16>(wvalid[0] + wvalid[1] + wvalid[2] + wvalid[3], list_dst, list_src, qc, qs, qo,
                  K, pc, ps, po);
}

// Row gather of already-grouped rows: dst row r (r < offsets[G]) is src row
// row_token[r]; code rows of qbytes (a multiple of 16, 16-byte aligned) and
// scale rows of sbytes. Indices outside the source are skipped.
__global__ __launch_bounds__(256) void k_gather_rows(const int32_t* __restrict__ row_token,
                                                     const int64_t* __restrict__ offsets, int G,
                                                     int64_t src_rows,
                                                     const uint8_t* __restrict__ sq,
                                                     const uint8_t* __restrict__ ss,
                                                     int64_t qbytes, int64_t sbytes,
                                                     uint8_t* __restrict__ dq,
                                                     uint8_t* __restrict__ ds) {
  const int64_t M = offsets[G];
  const int64_t n16 = qbytes / 16;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < M * n16; i += stride) {
    const int64_t r = i / n16, c = i - r * n16;
    const int64_t t = row_token[r];
    if (t < 0 || t >= src_rows) continue;
    *reinterpret_cast<uint4*>(dq + r * qbytes + 16 * c) =
        *reinterpret_cast<const uint4*>(sq + t * qbytes + 16 * c);
  }
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < M * sbytes; i += stride) {
    const int64_t r = i / sbytes, c = i - r * sbytes;
    const int64_t t = row_token[r];
    if (t < 0 || t >= src_rows) continue;
    ds[r * sbytes + c] = ss[t * sbytes + c];
  }
}

}  // namespace

hipError_t launch_gather_rows(const int32_t* row_token, const int64_t* offsets, int G,
                              int64_t m_cap, int64_t src_rows, const uint8_t* src_q,
                              const uint8_t* src_s, int64_t qbytes, int64_t sbytes,
                              uint8_t* dst_q, uint8_t* dst_s, hipStream_t stream) {
  if (m_cap == 0 || G == 0) return hipSuccess;
  int64_t grid = (m_cap * (qbytes / 16) + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  k_gather_rows<<<(unsigned)grid, 256, 0, stream>>>(row_token, offsets, G, src_rows, src_q, src_s,
                                                    qbytes, sbytes, dst_q, dst_s);
  return hipGetLastError();
}

size_t permute_workspace_bytes(int64_t T, int k, int n_local) {
  const int64_t n = T * k;
  const int64_t n_chunks = (n + kChunk - 1) / kChunk;
  return (size_t)((n_chunks > 0 ? n_chunks : 1) * (int64_t)n_local * 4 + 256);
}

// padded[g] = sum over g' < g of round_up(offsets[g'+1] - offsets[g'], align),
// one workgroup, G <= 1024.
__global__ __launch_bounds__(1024) void k_pad_offsets(const int64_t* __restrict__ offsets, int G,
                                                      int64_t align, int64_t* __restrict__ padded) {
  const int g = threadIdx.x;
  const int64_t len = g < G ? offsets[g + 1] - offsets[g] : 0;
  int64_t total;
  const int64_t ex = block_scan_1024((len + align - 1) / align * align, total);
  if (g < G) padded[g] = ex;
  if (g == 0) padded[G] = total;
}

hipError_t launch_padded_offsets(const int64_t* offsets, int G, int64_t align, int64_t* padded,
                                 hipStream_t stream) {
  k_pad_offsets<<<1, 1024, 0, stream>>>(offsets, G, align, padded);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int64_t T, int k, int e0, int n_local,
                          const uint8_t* qc, const uint8_t* qs, const float* qo, int64_t K,
                          int64_t* offsets, int64_t* padded, int32_t* row_token,
                          int32_t* row_slot, int32_t* pair_row, uint8_t* pc, uint8_t* ps,
                          float* po, void* workspace, hipStream_t stream) {
  const int64_t n = T * k;
  int nbits = 0;
  while ((1 << nbits) < n_local) ++nbits;
  const bool sc16 = K % 256 == 0 && ((reinterpret_cast<uintptr_t>(qs) |
                                      reinterpret_cast<uintptr_t>(ps)) & 15u) == 0;
  if (n > 0 && n <= kSmallMax) {
    const unsigned grid = (unsigned)((n + kSmallChunk - 1) / kSmallChunk);
    if (sc16)
      k_permute_small<true><<<grid, 256, 0, stream>>>(ids, n, k, e0, n_local, nbits, qc, qs, qo,
                                                      K, offsets, padded, row_token, row_slot,
                                                      pair_row, pc, ps, po);
    else
      k_permute_small<false><<<grid, 256, 0, stream>>>(ids, n, k, e0, n_local, nbits, qc, qs, qo,
                                                       K, offsets, padded, row_token, row_slot,
                                                       pair_row, pc, ps, po);
    return hipGetLastError();
  }
  const int64_t n_chunks = (n + kChunk - 1) / kChunk;
  int32_t* ws = static_cast<int32_t*>(workspace);
  if (n_chunks > 0) {
    k_hist<<<(unsigned)n_chunks, 256, 0, stream>>>(ids, n, e0, n_local, n_chunks, ws);
  }
  k_scan<<<1, 1024, 0, stream>>>(ws, n_chunks, n_local, offsets, padded);
  if (n_chunks > 0) {
    if (sc16)
      k_scatter_copy<true><<<(unsigned)n_chunks, 256, 0, stream>>>(
          ids, n, k, e0, n_local, nbits, n_chunks, ws, qc, qs, qo, K, row_token, row_slot,
          pair_row, pc, ps, po);
    else
      k_scatter_copy<false><<<(unsigned)n_chunks, 256, 0, stream>>>(
          ids, n, k, e0, n_local, nbits, n_chunks, ws, qc, qs, qo, K, row_token, row_slot,
          pair_row, pc, ps, po);
  }
  return hipGetLastError();
}

// Library-owned scratch for moe_permute_noalloc: the three-launch form's
// per-(expert, chunk) count table lives here instead of in a caller's
// workspace. Every GPU the library runs on holds its own copy for the life of
// the process. The histogram pass writes every table entry a call reads, so
// nothing needs clearing between calls; calls that overlap on one GPU share
// the table and race.
constexpr size_t kPermuteScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) uint8_t scratch[kPermuteScratchBytes];

size_t permute_scratch_bytes() { return kPermuteScratchBytes; }

// Device address of `scratch` on the current device. In host code the
// array's name is only a host-side stand-in, so the address is looked up once
// per device (with that device current) and cached.
hipError_t permute_scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace nvfp4moe
