// Expert outputs back to token order, and the backward of that step.
//
// combine:      out[t, :] = sum over slots j of gate[t, j] * y[pair_row[t, j], :]
//               (float32 fused multiply-adds in slot order; pairs whose expert
//               is not local, pair_row = -1, add nothing);
// combine_bwd:  dy[r, :] = gate[t, j] * dout[t, :] for the routed rows, and
//               dgate[t, j] = sum_n dout[t, n] * y[r, n].
// Both are streaming kernels: 16-byte accesses along rows, every load of a
// round issued before its first use. A pair that is not local still issues
// its load, from the first 16 bytes of y for every lane (one cached line per
// wavefront, weight zero), so no branch holds the other loads back.
#include "codecs.hpp"
#include "internal.hpp"

namespace nvfp4moe {

namespace {

template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&v)[8]) {
  if constexpr (BF16) {
    const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    v[0] = u2f(a.x << 16); v[1] = u2f(a.x & 0xFFFF0000u);
    v[2] = u2f(a.y << 16); v[3] = u2f(a.y & 0xFFFF0000u);
    v[4] = u2f(a.z << 16); v[5] = u2f(a.z & 0xFFFF0000u);
    v[6] = u2f(a.w << 16); v[7] = u2f(a.w & 0xFFFF0000u);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + elem);
    const uint4 a = p[0], b = p[1];
    v[0] = u2f(a.x); v[1] = u2f(a.y); v[2] = u2f(a.z); v[3] = u2f(a.w);
    v[4] = u2f(b.x); v[5] = u2f(b.y); v[6] = u2f(b.z); v[7] = u2f(b.w);
  }
}

template <bool BF16>
__device__ __forceinline__ void store8(void* base, int64_t elem, const float (&v)[8]) {
  if constexpr (BF16) {
    uint4 a;
    a.x = pk_bf16(v[0], v[1]);
    a.y = pk_bf16(v[2], v[3]);
    a.z = pk_bf16(v[4], v[5]);
    a.w = pk_bf16(v[6], v[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + elem) = a;
  } else {
    uint4* p = reinterpret_cast<uint4*>(static_cast<float*>(base) + elem);
    p[0] = make_uint4(f2u(v[0]), f2u(v[1]), f2u(v[2]), f2u(v[3]));
    p[1] = make_uint4(f2u(v[4]), f2u(v[5]), f2u(v[6]), f2u(v[7]));
  }
}

// One wavefront per token (the grid walks the tokens), lanes along the
// columns: four 512-column pieces per round. The token's pairs are the same
// for the whole wavefront, so they are taken two at a time, a couple with no
// local pair is skipped by a branch of the whole wavefront, and a non-local
// pair next to a local one loads the first 16 bytes of y (one cached line,
// weight zero) so the couple's loads are in flight together.
template <bool YB, bool OB>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ y, int64_t m_cap,
                                                 int64_t T, int k, int64_t N,
                                                 const int32_t* __restrict__ pair_row,
                                                 const float* __restrict__ gate,
                                                 void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  // the token index is the same for the whole wavefront: scalar loads of its pairs
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int64_t t = (int64_t)blockIdx.x * 4 + w; t < T; t += (int64_t)gridDim.x * 4) {
    for (int64_t base = 0; base < N; base += 2048) {
      const int64_t c0 = base + 8 * lane;
      float acc[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[q][e] = 0.0f;
      for (int j = 0; j < k; j += 2) {
        const int32_t r0 = pair_row[t * k + j];
        const int32_t r1 = j + 1 < k ? pair_row[t * k + j + 1] : -1;
        const bool u0 = r0 >= 0 && r0 < m_cap, u1 = r1 >= 0 && r1 < m_cap;
        if (!u0 && !u1) continue;                // the same for the whole wavefront
        const float g0 = u0 ? (gate ? gate[t * k + j] : 1.0f) : 0.0f;
        const float g1 = u1 ? (gate ? gate[t * k + j + 1] : 1.0f) : 0.0f;
        float v0[4][8], v1[4][8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t c = c0 + 512 * q < N ? c0 + 512 * q : N - 8;
          load8<YB>(y, u0 ? (int64_t)r0 * N + c : 0, v0[q]);
          load8<YB>(y, u1 ? (int64_t)r1 * N + c : 0, v1[q]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc[q][e] = __fmaf_rn(g1, v1[q][e], __fmaf_rn(g0, v0[q][e], acc[q][e]));
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (c0 + 512 * q < N) store8<OB>(out, t * N + c0 + 512 * q, acc[q]);
    }
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// One wavefront per routed row, rows walked by the grid up to offsets[G].
// HASY: y is given and dgate is computed.
template <bool DB, bool YB, bool OB, bool HASY>
__global__ __launch_bounds__(256) void k_combine_bwd(
    const void* __restrict__ dout, int64_t N, int k, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ row_slot, const int64_t* __restrict__ offsets, int G,
    int64_t m_cap, const float* __restrict__ gate, const void* __restrict__ y,
    void* __restrict__ dy, float* __restrict__ dgate) {
  const int lane = threadIdx.x & 63;
  int64_t live = offsets[G];
  live = live < m_cap ? live : m_cap;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < live;
       r += (int64_t)gridDim.x * 4) {
    const int64_t t = row_token[r];
    const int64_t pair = t * k + row_slot[r];
    const float g = gate ? gate[pair] : 1.0f;
    float part = 0.0f;
    // four 512-column pieces per round, all loads of a round in flight together
    for (int64_t c0 = 8 * lane; c0 < N; c0 += 4 * 512) {
      float d[4][8], v[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {            // past the row's end: reload its last chunk
        const int64_t c = c0 + 512 * q < N ? c0 + 512 * q : N - 8;
        load8<DB>(dout, t * N + c, d[q]);
        if constexpr (HASY) load8<YB>(y, r * N + c, v[q]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t c = c0 + 512 * q;
        if (c < N) {
          float o[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = __fmul_rn(g, d[q][e]);
          store8<OB>(dy, r * N + c, o);
          if constexpr (HASY) {
#pragma unroll
            for (int e = 0; e < 8; ++e) part = __fmaf_rn(d[q][e], v[q][e], part);
          }
        }
      }
    }
    if constexpr (HASY) {
      part = wave_sum(part);
      if (lane == 0) dgate[pair] = part;
    }
  }
}

}  // namespace

hipError_t launch_combine(const void* y, bool y_bf16, int64_t m_cap, int64_t T, int k,
                          int64_t N, const int32_t* pair_row, const float* gate, void* out,
                          bool out_bf16, hipStream_t stream) {
  if (T == 0 || N == 0) return hipSuccess;
  int64_t grid = (T + 3) / 4;                   // one wavefront per token
  const int64_t most = (int64_t)device_cu_count() * 64;
  if (grid > most) grid = most;
#define NVFP4MOE_COMBINE(YB, OB) \
  k_combine<YB, OB><<<(unsigned)grid, 256, 0, stream>>>(y, m_cap, T, k, N, pair_row, gate, out)
  if (y_bf16) {
    if (out_bf16) NVFP4MOE_COMBINE(true, true); else NVFP4MOE_COMBINE(true, false);
  } else {
    if (out_bf16) NVFP4MOE_COMBINE(false, true); else NVFP4MOE_COMBINE(false, false);
  }
#undef NVFP4MOE_COMBINE
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const void* dout, bool dout_bf16, int64_t N, int k,
                              const int32_t* row_token, const int32_t* row_slot,
                              const int64_t* offsets, int G, int64_t m_cap, const float* gate,
                              const void* y, bool y_bf16, void* dy, bool dy_bf16, float* dgate,
                              hipStream_t stream) {
  if (m_cap == 0 || N == 0) return hipSuccess;
  int64_t grid = (m_cap + 3) / 4;
  const int64_t most = (int64_t)device_cu_count() * 32;
  if (grid > most) grid = most;
#define NVFP4MOE_CBWD3(DB, YB, OB, HY)                                                       \
  k_combine_bwd<DB, YB, OB, HY><<<(unsigned)grid, 256, 0, stream>>>(                         \
      dout, N, k, row_token, row_slot, offsets, G, m_cap, gate, y, dy, dgate)
#define NVFP4MOE_CBWD(DB, YB, OB)                                                            \
  do {                                                                                       \
    if (y) NVFP4MOE_CBWD3(DB, YB, OB, true);                                                 \
    else NVFP4MOE_CBWD3(DB, true, OB, false);                                                \
  } while (0)
  if (dout_bf16) {
    if (y_bf16) {
      if (dy_bf16) NVFP4MOE_CBWD(true, true, true); else NVFP4MOE_CBWD(true, true, false);
    } else {
      if (dy_bf16) NVFP4MOE_CBWD(true, false, true); else NVFP4MOE_CBWD(true, false, false);
    }
  } else {
    if (y_bf16) {
      if (dy_bf16) NVFP4MOE_CBWD(false, true, true); else NVFP4MOE_CBWD(false, true, false);
    } else {
      if (dy_bf16) NVFP4MOE_CBWD(false, false, true); else NVFP4MOE_CBWD(false, false, false);
    }
  }
#undef NVFP4MOE_CBWD
#undef NVFP4MOE_CBWD3
  return hipGetLastError();
}

}  // namespace nvfp4moe
