// Expert outputs back to token order, and the backward of that step.
//
// combine:      out[t, :] = sum over slots j of gate[t, j] * y[pair_row[t, j], :]
//               (float32 fused multiply-adds in slot order; pairs whose expert
//               is not local, pair_row = -1, add nothing);
// combine_bwd:  dy[r, :] = gate[t, j] * dout[t, :] for the routed rows, and
//               dgate[t, j] = sum_n dout[t, n] * y[r, n].
// Both are streaming kernels: 16-byte accesses along rows, every load of a
// round issued before its first use (indices clamped, weights zeroed), so
// nothing waits on a branch.
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
    a.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
    a.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
    a.z = f32_to_bf16_rne(v[4]) | (f32_to_bf16_rne(v[5]) << 16);
    a.w = f32_to_bf16_rne(v[6]) | (f32_to_bf16_rne(v[7]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + elem) = a;
  } else {
    uint4* p = reinterpret_cast<uint4*>(static_cast<float*>(base) + elem);
    p[0] = make_uint4(f2u(v[0]), f2u(v[1]), f2u(v[2]), f2u(v[3]));
    p[1] = make_uint4(f2u(v[4]), f2u(v[5]), f2u(v[6]), f2u(v[7]));
  }
}

// One thread per 8 consecutive columns of one token; the grid walks
// (token, column chunk) with the chunk fastest. S routed pairs per round of
// loads (2, 4 or 8: the smallest not below k, 8 for larger k).
template <bool YB, bool OB, int S>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ y, int64_t m_cap,
                                                 uint32_t T, int k, uint32_t nc,
                                                 const int32_t* __restrict__ pair_row,
                                                 const float* __restrict__ gate,
                                                 void* __restrict__ out) {
  const uint32_t total = T * nc;
  for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += gridDim.x * 256) {
    const uint32_t t = i / nc, c = i - t * nc;
    const int64_t N = (int64_t)nc * 8;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += S) {
      int32_t r[S];
      float g[S];
#pragma unroll
      for (int u = 0; u < S; ++u) {
        const int j = j0 + u < k ? j0 + u : k - 1;
        r[u] = pair_row[(int64_t)t * k + j];
        g[u] = gate ? gate[(int64_t)t * k + j] : 1.0f;
      }
      float v[S][8];
#pragma unroll
      for (int u = 0; u < S; ++u) {
        const bool use = (j0 + u < k) && r[u] >= 0 && r[u] < m_cap;
        g[u] = use ? g[u] : 0.0f;
        load8<YB>(y, (use ? (int64_t)r[u] : 0) * N + 8 * (int64_t)c, v[u]);
      }
#pragma unroll
      for (int u = 0; u < S; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = __fmaf_rn(g[u], v[u][e], acc[e]);
    }
    store8<OB>(out, (int64_t)t * N + 8 * (int64_t)c, acc);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// One wavefront per routed row, rows walked by the grid up to offsets[G].
template <bool DB, bool YB, bool OB>
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
    for (int64_t c = 8 * lane; c < N; c += 512) {
      float d[8];
      load8<DB>(dout, t * N + c, d);
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = __fmul_rn(g, d[e]);
      store8<OB>(dy, r * N + c, o);
      if (y) {
        float v[8];
        load8<YB>(y, r * N + c, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) part = __fmaf_rn(d[e], v[e], part);
      }
    }
    if (y) {
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
  const uint32_t nc = (uint32_t)(N / 8);
  const int64_t work = T * (int64_t)nc;
  int64_t grid = (work + 255) / 256;
  const int64_t most = (int64_t)device_cu_count() * 16;
  if (grid > most) grid = most;
#define NVFP4MOE_COMBINE_S(YB, OB, S)                                                     \
  k_combine<YB, OB, S><<<(unsigned)grid, 256, 0, stream>>>(y, m_cap, (uint32_t)T, k, nc,   \
                                                           pair_row, gate, out)
#define NVFP4MOE_COMBINE(YB, OB)                                                          \
  do {                                                                                    \
    if (k <= 2) NVFP4MOE_COMBINE_S(YB, OB, 2);                                            \
    else if (k <= 4) NVFP4MOE_COMBINE_S(YB, OB, 4);                                       \
    else NVFP4MOE_COMBINE_S(YB, OB, 8);                                                   \
  } while (0)
  if (y_bf16) {
    if (out_bf16) NVFP4MOE_COMBINE(true, true); else NVFP4MOE_COMBINE(true, false);
  } else {
    if (out_bf16) NVFP4MOE_COMBINE(false, true); else NVFP4MOE_COMBINE(false, false);
  }
#undef NVFP4MOE_COMBINE
#undef NVFP4MOE_COMBINE_S
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const void* dout, bool dout_bf16, int64_t N, int k,
                              const int32_t* row_token, const int32_t* row_slot,
                              const int64_t* offsets, int G, int64_t m_cap, const float* gate,
                              const void* y, bool y_bf16, void* dy, bool dy_bf16, float* dgate,
                              hipStream_t stream) {
  if (m_cap == 0 || N == 0) return hipSuccess;
  int64_t grid = (m_cap + 3) / 4;
  const int64_t most = (int64_t)device_cu_count() * 16;
  if (grid > most) grid = most;
#define NVFP4MOE_CBWD(DB, YB, OB)                                                            \
  k_combine_bwd<DB, YB, OB><<<(unsigned)grid, 256, 0, stream>>>(                             \
      dout, N, k, row_token, row_slot, offsets, G, m_cap, gate, y, dy, dgate)
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
  return hipGetLastError();
}

}  // namespace nvfp4moe
