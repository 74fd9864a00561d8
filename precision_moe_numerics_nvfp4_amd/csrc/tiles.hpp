// Grouped tile enumeration shared by the grouped GEMM kernels.
//
// A grouped launch enumerates tiles group by group: group e owns cnt(e)
// consecutive tile indices. The grid is sized for an upper bound and the
// group sizes live on the device, so every workgroup must find which group
// its tile belongs to. Walking the groups one after the other costs one
// dependent memory round trip per group (G of them); here the 256 threads
// read the group sizes in parallel, scan them with wavefront shuffles and
// one LDS exchange, and the thread whose range holds the tile publishes it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4moe {

struct TileLoc {
  int g;          // group, or -1 when the tile index is past the last tile
  int local;      // tile index inside the group
  int total;      // number of tiles over all groups
};

// Call from every thread of a 256-thread workgroup with the same t. cnt(e)
// must be cheap and give the same value whenever called with the same e.
template <class Cnt>
__device__ inline TileLoc locate_tile(int t, int G, Cnt cnt) {
  __shared__ int sh_wave[4];
  __shared__ int sh_out[2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (G + 255) / 256;
  const int e0 = tid * per;
  int own = 0;
  for (int e = e0; e < e0 + per && e < G; ++e) own += cnt(e);
  int incl = own;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) sh_wave[w] = incl;
  if (tid == 0) sh_out[0] = -1;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = sh_wave[i];
    base += i < w ? s : 0;
    total += s;
  }
  int excl = base + incl - own;
  if (t >= excl && t < excl + own) {
    for (int e = e0; e < e0 + per && e < G; ++e) {
      const int c = cnt(e);
      if (t - excl < c) {
        sh_out[0] = e;
        sh_out[1] = t - excl;
        break;
      }
      excl += c;
    }
  }
  __syncthreads();
  TileLoc r;
  r.g = sh_out[0];
  r.local = sh_out[1];
  r.total = total;
  __syncthreads();      // sh_out may be reused by a later call
  return r;
}

}  // namespace nvfp4moe

namespace nvfp4moe {

// Exclusive prefix of cnt(e) over the groups, written to pre[0..G] in LDS
// (pre[G] = total). Call from every thread of the workgroup (blockDim.x a
// multiple of 64, at most 1024); ends with a barrier.
template <class Cnt>
__device__ inline void tile_prefix(int G, Cnt cnt, int* pre) {
  __shared__ int sh_wave[16];
  const int nthr = blockDim.x, nw = nthr >> 6;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (G + nthr - 1) / nthr;
  const int e0 = tid * per;
  int own = 0;
  for (int e = e0; e < e0 + per && e < G; ++e) own += cnt(e);
  int incl = own;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) sh_wave[w] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < nw; ++i) base += i < w ? sh_wave[i] : 0;
  int run = base + incl - own;
  for (int e = e0; e < e0 + per && e < G; ++e) {
    pre[e] = run;
    run += cnt(e);
  }
  if (tid == nthr - 1) pre[G] = base + incl;
  __syncthreads();
}

// LDS rows of 64 bytes (four 16-byte chunks): chunk c of row r sits at
// position c ^ chunk_key(r). For one chunk index, any 8 consecutive rows from
// a multiple of 8 (the 8 lanes of one 128-byte LDS cycle of a 16-byte read)
// and any 16 from a multiple of 16 (16 lanes over 256 bytes) land in distinct
// 16-byte bank groups. The key uses row bits 1-3 only, so rows 32 apart
// share it.
__device__ __forceinline__ int chunk_key(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

// Largest g with pre[g] <= t (t < pre[G]); groups with no tiles are skipped.
__device__ inline int tile_group(const int* pre, int G, int t) {
  int lo = 0, hi = G;            // pre[lo] <= t < pre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Tile loc of an mt x nt grid, ordered in blocks of 4 columns (n-tiles):
// inside a block the n index runs fastest, then m; blocks follow each other.
// A run of 32 consecutive tiles then covers 8 rows x 4 columns of the grid.
__device__ inline void block_order(int loc, int mt, int nt, int& mi, int& ni) {
  const int nb = loc / (mt * 4);                  // block of 4 columns
  const int r = loc - nb * mt * 4;
  const int w = nt - nb * 4 < 4 ? nt - nb * 4 : 4;  // columns in this block
  mi = r / w;
  ni = nb * 4 + r % w;
}

}  // namespace nvfp4moe
