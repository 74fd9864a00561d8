// Token-to-expert grouping, group-offset scans and the NVFP4 row gather.
//
// Pages: each token is routed to 8 of 384 experts ("Thinking Machines' Inkling
// 2 Small Trains a 594B Model in 68 Hours", section "594B weights, 17B at
// work") and travels to them already in NVFP4 ("Inkling 2 Small uses four-bit
// training ...", section "Quantized NVLink and BBBK"). On one GPU this is a
// stable counting sort of the (token, slot) pairs by local expert plus a gather.
//
// Determinism without atomics on the output order:
//   1. histogram: one workgroup per chunk of 1024 flat pairs counts pairs per
//      local expert (LDS atomics; only the counts, not the order, depend on
//      them) into ws[e][chunk];
//   2. scan: one workgroup turns the counts into offsets, padded offsets and
//      the start of every (expert, chunk) run, in place;
//   3. scatter: one wavefront per chunk walks its pairs in flat order, 64 at a
//      time; lanes holding the same expert find each other with one ballot per
//      bit of the expert index, so each pair's rank among earlier pairs of its
//      expert is a popcount. Row order inside an expert is flat index order.
//   4. gather: one wavefront per routed row copies the token's NVFP4 row
//      (codes, scales, outer scale) with 16-byte vector copies.
#include "codecs.hpp"
#include "internal.hpp"

namespace nvfp4moe {

namespace {

constexpr int kChunk = 1024;

__global__ __launch_bounds__(256) void k_hist(const int32_t* __restrict__ ids, int64_t n, int e0,
                                              int n_local, int64_t n_chunks,
                                              int32_t* __restrict__ ws) {
  __shared__ int32_t cnt[1024];
  for (int e = threadIdx.x; e < n_local; e += 256) cnt[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  for (int i = threadIdx.x; i < kChunk; i += 256) {
    const int64_t f = base + i;
    if (f < n) {
      const int le = ids[f] - e0;
      if (le >= 0 && le < n_local) atomicAdd(&cnt[le], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < n_local; e += 256) ws[(int64_t)e * n_chunks + blockIdx.x] = cnt[e];
}

// One workgroup of 1024 threads; thread e owns expert e.
__global__ __launch_bounds__(1024) void k_scan(int32_t* __restrict__ ws, int64_t n_chunks,
                                               int n_local, int64_t* __restrict__ offsets,
                                               int64_t* __restrict__ padded) {
  __shared__ int64_t tot[1024];
  __shared__ int64_t ptot[1024];
  const int e = threadIdx.x;
  int64_t t = 0;
  if (e < n_local)
    for (int64_t c = 0; c < n_chunks; ++c) t += ws[(int64_t)e * n_chunks + c];
  tot[e] = (e < n_local) ? t : 0;
  ptot[e] = (e < n_local) ? ((t + 31) / 32) * 32 : 0;
  __syncthreads();
  // inclusive Hillis-Steele scans over 1024 entries
  for (int off = 1; off < 1024; off <<= 1) {
    int64_t a = 0, b = 0;
    if (e >= off) {
      a = tot[e - off];
      b = ptot[e - off];
    }
    __syncthreads();
    tot[e] += a;
    ptot[e] += b;
    __syncthreads();
  }
  if (e < n_local) {
    const int64_t start = tot[e] - t;
    offsets[e + 1] = tot[e];
    padded[e + 1] = ptot[e];
    if (e == 0) {
      offsets[0] = 0;
      padded[0] = 0;
    }
    int64_t run = start;
    for (int64_t c = 0; c < n_chunks; ++c) {
      const int64_t i = (int64_t)e * n_chunks + c;
      const int32_t k = ws[i];
      ws[i] = (int32_t)run;
      run += k;
    }
  }
}

__global__ __launch_bounds__(64) void k_scatter(const int32_t* __restrict__ ids, int64_t n, int k,
                                                int e0, int n_local, int nbits, int64_t n_chunks,
                                                const int32_t* __restrict__ ws,
                                                int32_t* __restrict__ row_token,
                                                int32_t* __restrict__ row_slot) {
  __shared__ int32_t base[1024];
  const int lane = threadIdx.x;
  for (int e = lane; e < n_local; e += 64) base[e] = ws[(int64_t)e * n_chunks + blockIdx.x];
  __syncthreads();
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  for (int piece = 0; piece < kChunk; piece += 64) {
    const int64_t f = c0 + piece + lane;
    int le = -1;
    if (f < n) le = ids[f] - e0;
    const bool valid = (le >= 0) && (le < n_local);
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((le >> b) & 1);
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    int pos = 0;
    if (valid) {
      const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      pos = base[le] + __popcll(peers & below);
      row_token[pos] = (int32_t)(f / k);
      row_slot[pos] = (int32_t)(f % k);
    }
    __syncthreads();
    if (valid && (peers & ((lane == 0) ? 0ull : (~0ull >> (64 - lane)))) == 0)
      base[le] += __popcll(peers);  // lowest lane of each expert advances its run
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_gather(const int64_t* __restrict__ offsets, int n_local,
                                                const int32_t* __restrict__ row_token,
                                                const uint8_t* __restrict__ qc,
                                                const uint8_t* __restrict__ qs,
                                                const float* __restrict__ qo, int64_t K,
                                                uint8_t* __restrict__ pc,
                                                uint8_t* __restrict__ ps,
                                                float* __restrict__ po) {
  const int64_t M = offsets[n_local];
  const int lane = threadIdx.x & 63;
  const int64_t n16 = K / 32;       // 16-byte chunks of codes per row
  const int64_t nsb = K / 16;       // scale bytes per row
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < M;
       r += (int64_t)gridDim.x * 4) {
    const int64_t t = row_token[r];
    const uint4* src = reinterpret_cast<const uint4*>(qc + t * (K / 2));
    uint4* dst = reinterpret_cast<uint4*>(pc + r * (K / 2));
    for (int64_t i = lane; i < n16; i += 64) dst[i] = src[i];
    for (int64_t i = lane; i < nsb; i += 64) ps[r * nsb + i] = qs[t * nsb + i];
    if (lane == 0) po[r] = qo[t];
  }
}

}  // namespace

size_t permute_workspace_bytes(int64_t T, int k, int n_local) {
  const int64_t n = T * k;
  const int64_t n_chunks = (n + kChunk - 1) / kChunk;
  return (size_t)((n_chunks > 0 ? n_chunks : 1) * (int64_t)n_local * 4 + 256);
}

hipError_t launch_permute(const int32_t* ids, int64_t T, int k, int e0, int n_local,
                          const uint8_t* qc, const uint8_t* qs, const float* qo, int64_t K,
                          int64_t* offsets, int64_t* padded, int32_t* row_token,
                          int32_t* row_slot, uint8_t* pc, uint8_t* ps, float* po,
                          void* workspace, hipStream_t stream) {
  const int64_t n = T * k;
  const int64_t n_chunks = (n + kChunk - 1) / kChunk;
  int32_t* ws = static_cast<int32_t*>(workspace);
  int nbits = 0;
  while ((1 << nbits) < n_local) ++nbits;
  if (n_chunks > 0) {
    k_hist<<<(unsigned)n_chunks, 256, 0, stream>>>(ids, n, e0, n_local, n_chunks, ws);
  }
  k_scan<<<1, 1024, 0, stream>>>(ws, n_chunks, n_local, offsets, padded);
  if (n_chunks > 0) {
    k_scatter<<<(unsigned)n_chunks, 64, 0, stream>>>(ids, n, k, e0, n_local, nbits, n_chunks,
                                                     ws, row_token, row_slot);
    int64_t grid = (n + 3) / 4;
    const int64_t cap = (int64_t)device_cu_count() * 8;
    if (grid > cap) grid = cap;
    k_gather<<<(unsigned)grid, 256, 0, stream>>>(offsets, n_local, row_token, qc, qs, qo, K, pc,
                                                 ps, po);
  }
  return hipGetLastError();
}

}  // namespace nvfp4moe
