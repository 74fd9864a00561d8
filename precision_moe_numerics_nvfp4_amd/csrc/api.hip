// C ABI of the NVFP4/MXFP8 expert-layer library: argument validation on the
// host, then kernel launches on the caller's stream. No allocation, no sync.
#include "../../include/nvfp4moe.h"

#include "internal.hpp"

using namespace nvfp4moe;

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The MXFP8 GEMMs address a 256-row operand tile with 32-bit byte offsets.
constexpr int64_t kMaxGemmRowBytes = (int64_t)0xFFFFFFFF / 257;
// wgrad ranks the groups by size in shared memory.
constexpr int kMaxWgradGroups = 16384;

inline int hip_status(hipError_t e) { return e == hipSuccess ? NVFP4MOE_OK : NVFP4MOE_EHIP; }

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

#define REQUIRE(cond, code) \
  do {                      \
    if (!(cond)) return (code); \
  } while (0)

}  // namespace

extern "C" {

int nvfp4moe_abi_version(void) { return NVFP4MOE_ABI_VERSION; }

const char* nvfp4moe_status_string(int status) {
  switch (status) {
    case NVFP4MOE_OK: return "ok";
    case NVFP4MOE_EINVAL: return "invalid argument";
    case NVFP4MOE_EUNSUPPORTED: return "unsupported size or alignment";
    case NVFP4MOE_EWORKSPACE: return "workspace too small";
    case NVFP4MOE_EHIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

int nvfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int outer_mode,
                   int64_t rows_per_group, uint8_t* codes, uint8_t* scales, float* outer,
                   void* stream) {
  REQUIRE(rows >= 0 && cols >= 0, NVFP4MOE_EINVAL);
  REQUIRE(x_dtype == NVFP4MOE_F32 || x_dtype == NVFP4MOE_BF16, NVFP4MOE_EINVAL);
  REQUIRE(outer_mode == NVFP4MOE_OUTER_PER_ROW || outer_mode == NVFP4MOE_OUTER_PER_GROUP,
          NVFP4MOE_EINVAL);
  const bool per_group = outer_mode == NVFP4MOE_OUTER_PER_GROUP;
  if (per_group) REQUIRE(rows_per_group > 0, NVFP4MOE_EINVAL);
  if (rows == 0) return NVFP4MOE_OK;
  REQUIRE(x && codes && scales && outer, NVFP4MOE_EINVAL);
  REQUIRE(cols > 0 && cols % 32 == 0 && cols <= 8192, NVFP4MOE_EUNSUPPORTED);
  if (per_group) REQUIRE(rows % rows_per_group == 0, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(aligned16(x) && aligned16(codes) && aligned16(scales) && aligned16(outer),
          NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_nvfp4_quantize(x, x_dtype == NVFP4MOE_BF16, rows, cols, per_group,
                                          rows_per_group, codes, scales, outer,
                                          as_stream(stream)));
}

size_t nvfp4moe_permute_workspace_size(int64_t T, int k, int n_local) {
  if (T < 0 || k <= 0 || n_local <= 0) return 0;
  return permute_workspace_bytes(T, k, n_local);
}

int moe_permute(const int32_t* topk_ids, int64_t T, int k, int e0, int n_local,
                const uint8_t* xq_codes, const uint8_t* xq_scales, const float* xq_outer,
                int64_t K, int64_t* offsets, int64_t* padded_offsets, int32_t* row_token,
                int32_t* row_slot, int32_t* pair_row, uint8_t* xperm_codes,
                uint8_t* xperm_scales, float* xperm_outer, void* workspace,
                size_t workspace_bytes, void* stream) {
  REQUIRE(T >= 0 && K >= 0 && k > 0 && n_local > 0, NVFP4MOE_EINVAL);
  REQUIRE(offsets && padded_offsets && workspace, NVFP4MOE_EINVAL);
  if (T > 0)
    REQUIRE(topk_ids && xq_codes && xq_scales && xq_outer && row_token && row_slot &&
                xperm_codes && xperm_scales && xperm_outer,
            NVFP4MOE_EINVAL);
  REQUIRE(n_local <= 1024 && k <= 64, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(K % 32 == 0 && K > 0, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(T * (int64_t)k < (int64_t)1 << 31, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(workspace_bytes >= permute_workspace_bytes(T, k, n_local), NVFP4MOE_EWORKSPACE);
  REQUIRE(aligned16(xq_codes) && aligned16(xperm_codes) && aligned16(workspace),
          NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_permute(topk_ids, T, k, e0, n_local, xq_codes, xq_scales, xq_outer,
                                   K, offsets, padded_offsets, row_token, row_slot, pair_row, xperm_codes,
                                   xperm_scales, xperm_outer, workspace, as_stream(stream)));
}

int moe_permute_noalloc(const int32_t* topk_ids, int64_t T, int k, int e0, int n_local,
                        const uint8_t* xq_codes, const uint8_t* xq_scales, const float* xq_outer,
                        int64_t K, int64_t* offsets, int64_t* padded_offsets, int32_t* row_token,
                        int32_t* row_slot, int32_t* pair_row, uint8_t* xperm_codes,
                        uint8_t* xperm_scales, float* xperm_outer, void* stream) {
  REQUIRE(T >= 0 && K >= 0 && k > 0 && n_local > 0, NVFP4MOE_EINVAL);
  REQUIRE(offsets && padded_offsets, NVFP4MOE_EINVAL);
  if (T > 0)
    REQUIRE(topk_ids && xq_codes && xq_scales && xq_outer && row_token && row_slot &&
                xperm_codes && xperm_scales && xperm_outer,
            NVFP4MOE_EINVAL);
  REQUIRE(n_local <= 1024 && k <= 64, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(K % 32 == 0 && K > 0, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(T * (int64_t)k < (int64_t)1 << 31, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(permute_workspace_bytes(T, k, n_local) <= permute_scratch_bytes(), NVFP4MOE_EWORKSPACE);
  REQUIRE(aligned16(xq_codes) && aligned16(xperm_codes), NVFP4MOE_EUNSUPPORTED);
  void* ws = nullptr;
  if (permute_scratch_address(&ws) != hipSuccess) return NVFP4MOE_EHIP;
  return hip_status(launch_permute(topk_ids, T, k, e0, n_local, xq_codes, xq_scales, xq_outer,
                                   K, offsets, padded_offsets, row_token, row_slot, pair_row,
                                   xperm_codes, xperm_scales, xperm_outer, ws, as_stream(stream)));
}

int moe_fwd_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_outer,
                         const uint8_t* b_codes, const uint8_t* b_scales, const float* b_outer,
                         const int64_t* offsets, int G, int64_t m_cap, int64_t N, int64_t K,
                         void* y, int y_dtype, void* stream) {
  REQUIRE(G >= 0 && m_cap >= 0 && N >= 0 && K >= 0, NVFP4MOE_EINVAL);
  REQUIRE(y_dtype == NVFP4MOE_F32 || y_dtype == NVFP4MOE_BF16, NVFP4MOE_EINVAL);
  if (G == 0 || m_cap == 0 || N == 0) return NVFP4MOE_OK;
  REQUIRE(a_codes && a_scales && a_outer && b_codes && b_scales && b_outer && offsets && y,
          NVFP4MOE_EINVAL);
  REQUIRE(N % 128 == 0 && K % 128 == 0 && K > 0, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(aligned16(a_codes) && aligned16(b_codes) && aligned16(y), NVFP4MOE_EUNSUPPORTED);
  REQUIRE(((reinterpret_cast<uintptr_t>(a_scales) | reinterpret_cast<uintptr_t>(b_scales)) & 7u) == 0,
          NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_fwd_grouped_gemm(a_codes, a_scales, a_outer, b_codes, b_scales,
                                            b_outer, offsets, G, m_cap, N, K, y,
                                            y_dtype == NVFP4MOE_BF16, as_stream(stream)));
}

int mxfp8_requant_sr(const uint8_t* codes, const uint8_t* scales, const float* outer,
                     int outer_mode, int64_t rows_per_group, int64_t rows, int64_t cols,
                     const int64_t* offsets, const int64_t* padded_offsets, int G, int64_t P,
                     uint64_t seed, uint32_t tag, uint8_t* out_e4m3, uint8_t* out_e8m0,
                     void* stream) {
  REQUIRE(rows >= 0 && cols >= 0 && G >= 0 && P >= 0, NVFP4MOE_EINVAL);
  REQUIRE(outer_mode == NVFP4MOE_OUTER_PER_ROW || outer_mode == NVFP4MOE_OUTER_PER_GROUP,
          NVFP4MOE_EINVAL);
  const bool per_group = outer_mode == NVFP4MOE_OUTER_PER_GROUP;
  if (per_group) REQUIRE(rows_per_group > 0, NVFP4MOE_EINVAL);
  if (G == 0 || P == 0 || cols == 0) return NVFP4MOE_OK;
  REQUIRE(offsets && padded_offsets && out_e4m3 && out_e8m0, NVFP4MOE_EINVAL);
  if (rows > 0) REQUIRE(codes && scales && outer, NVFP4MOE_EINVAL);
  REQUIRE(cols % 128 == 0 && P % 32 == 0, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(aligned16(codes) && aligned16(out_e4m3), NVFP4MOE_EUNSUPPORTED);
  REQUIRE((reinterpret_cast<uintptr_t>(scales) & 7u) == 0, NVFP4MOE_EUNSUPPORTED);
  // weights (per-group outer scales): each group's block [cols, length]
  // contiguous, the layout dgrad reads
  return hip_status(launch_requant_sr(codes, scales, outer, per_group ? rows_per_group : 0, rows,
                                      cols, offsets, padded_offsets, G, P, per_group, seed, tag,
                                      out_e4m3, out_e8m0, as_stream(stream)));
}

int mxfp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int orientation,
                   const int64_t* offsets, const int64_t* padded_offsets, int G, int64_t P,
                   uint8_t* out_e4m3, uint8_t* out_e8m0, void* stream) {
  REQUIRE(rows >= 0 && cols >= 0, NVFP4MOE_EINVAL);
  REQUIRE(x_dtype == NVFP4MOE_F32 || x_dtype == NVFP4MOE_BF16, NVFP4MOE_EINVAL);
  REQUIRE(orientation == NVFP4MOE_ROWWISE || orientation == NVFP4MOE_COLWISE_GROUPED,
          NVFP4MOE_EINVAL);
  const bool bf16 = x_dtype == NVFP4MOE_BF16;
  if (orientation == NVFP4MOE_ROWWISE) {
    if (rows == 0 || cols == 0) return NVFP4MOE_OK;
    REQUIRE(x && out_e4m3 && out_e8m0, NVFP4MOE_EINVAL);
    REQUIRE(cols % 32 == 0, NVFP4MOE_EUNSUPPORTED);
    REQUIRE(aligned16(x) && aligned16(out_e4m3), NVFP4MOE_EUNSUPPORTED);
    return hip_status(launch_mxfp8_quantize_rowwise(x, bf16, rows, cols, out_e4m3, out_e8m0,
                                                    as_stream(stream)));
  }
  REQUIRE(G >= 0 && P >= 0, NVFP4MOE_EINVAL);
  if (G == 0 || P == 0 || cols == 0) return NVFP4MOE_OK;
  REQUIRE(offsets && padded_offsets && out_e4m3 && out_e8m0, NVFP4MOE_EINVAL);
  if (rows > 0) REQUIRE(x != nullptr, NVFP4MOE_EINVAL);
  REQUIRE(cols % 128 == 0 && P % 32 == 0, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(aligned16(x) && aligned16(out_e4m3), NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_mxfp8_quantize_colwise(x, bf16, rows, cols, offsets, padded_offsets,
                                                  G, P, out_e4m3, out_e8m0,
                                                  as_stream(stream)));
}

int moe_bwd_dgrad(const uint8_t* dy_e4m3, const uint8_t* dy_e8m0, const uint8_t* w_e4m3,
                  const uint8_t* w_e8m0, const int64_t* offsets, int G, int64_t m_cap,
                  int64_t N, int64_t K, void* dx, int dx_dtype, void* stream) {
  REQUIRE(G >= 0 && m_cap >= 0 && N >= 0 && K >= 0, NVFP4MOE_EINVAL);
  REQUIRE(dx_dtype == NVFP4MOE_F32 || dx_dtype == NVFP4MOE_BF16, NVFP4MOE_EINVAL);
  if (G == 0 || m_cap == 0 || K == 0) return NVFP4MOE_OK;
  REQUIRE(dy_e4m3 && dy_e8m0 && w_e4m3 && w_e8m0 && offsets && dx, NVFP4MOE_EINVAL);
  REQUIRE(N % 128 == 0 && K % 128 == 0 && N > 0, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(N <= kMaxGemmRowBytes, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(aligned16(dy_e4m3) && aligned16(w_e4m3) && aligned16(dx), NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_dgrad(dy_e4m3, dy_e8m0, w_e4m3, w_e8m0, offsets, G, m_cap, N, K, dx,
                                 dx_dtype == NVFP4MOE_BF16, as_stream(stream)));
}

int moe_bwd_wgrad(const uint8_t* dyT_e4m3, const uint8_t* dyT_e8m0, const uint8_t* xT_e4m3,
                  const uint8_t* xT_e8m0, const int64_t* padded_offsets, int G, int64_t P,
                  int64_t N, int64_t K, float* dw, void* stream) {
  REQUIRE(G >= 0 && P >= 0 && N >= 0 && K >= 0, NVFP4MOE_EINVAL);
  if (G == 0 || N == 0 || K == 0) return NVFP4MOE_OK;
  REQUIRE(dyT_e4m3 && dyT_e8m0 && xT_e4m3 && xT_e8m0 && padded_offsets && dw, NVFP4MOE_EINVAL);
  REQUIRE(N % 128 == 0 && K % 128 == 0 && P % 32 == 0, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(G <= kMaxWgradGroups && P <= kMaxGemmRowBytes, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(aligned16(dyT_e4m3) && aligned16(xT_e4m3) && aligned16(dw), NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_wgrad(dyT_e4m3, dyT_e8m0, xT_e4m3, xT_e8m0, padded_offsets, G, P, N, K,
                                 dw, as_stream(stream)));
}

int nvfp4_quantize_tile16(const void* x, int x_dtype, int64_t rows, int64_t cols,
                          int64_t rows_per_group, uint8_t* codes, uint8_t* scales, float* outer,
                          void* stream) {
  REQUIRE(rows >= 0 && cols >= 0 && rows_per_group > 0, NVFP4MOE_EINVAL);
  REQUIRE(x_dtype == NVFP4MOE_F32 || x_dtype == NVFP4MOE_BF16, NVFP4MOE_EINVAL);
  if (rows == 0 || cols == 0) return NVFP4MOE_OK;
  REQUIRE(x && codes && scales && outer, NVFP4MOE_EINVAL);
  REQUIRE(rows % 16 == 0 && cols % 16 == 0 && rows_per_group % 16 == 0 &&
              rows % rows_per_group == 0,
          NVFP4MOE_EUNSUPPORTED);
  REQUIRE(rows / 16 <= 65535, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(aligned16(x) && ((reinterpret_cast<uintptr_t>(codes) & 7u) == 0), NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_nvfp4_quantize_tile16(x, x_dtype == NVFP4MOE_BF16, rows, cols,
                                                 rows_per_group, codes, scales, outer,
                                                 as_stream(stream)));
}

int mxfp8_quantize_dual(const void* x, int x_dtype, int64_t rows, int64_t cols,
                        const int64_t* offsets, const int64_t* padded_offsets, int G, int64_t P,
                        uint8_t* row_e4m3, uint8_t* row_e8m0, uint8_t* col_e4m3,
                        uint8_t* col_e8m0, void* stream) {
  REQUIRE(rows >= 0 && cols >= 0 && G >= 0 && P >= 0, NVFP4MOE_EINVAL);
  REQUIRE(x_dtype == NVFP4MOE_F32 || x_dtype == NVFP4MOE_BF16, NVFP4MOE_EINVAL);
  if (G == 0 || P == 0 || cols == 0) return NVFP4MOE_OK;
  REQUIRE(offsets && padded_offsets && row_e4m3 && row_e8m0 && col_e4m3 && col_e8m0,
          NVFP4MOE_EINVAL);
  if (rows > 0) REQUIRE(x != nullptr, NVFP4MOE_EINVAL);
  REQUIRE(cols % 128 == 0 && P % 32 == 0, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(aligned16(x) && aligned16(col_e4m3) && aligned16(row_e4m3), NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_mxfp8_quantize_dual(x, x_dtype == NVFP4MOE_BF16, rows, cols, offsets,
                                               padded_offsets, G, P, row_e4m3, row_e8m0,
                                               col_e4m3, col_e8m0, as_stream(stream)));
}

int moe_fwd_grouped_gemm_mxfp8(const uint8_t* x_e4m3, const uint8_t* x_e8m0,
                               const uint8_t* w_e4m3, const uint8_t* w_e8m0,
                               const int64_t* offsets, int G, int64_t m_cap, int64_t N, int64_t K,
                               void* y, int y_dtype, void* stream) {
  REQUIRE(G >= 0 && m_cap >= 0 && N >= 0 && K >= 0, NVFP4MOE_EINVAL);
  REQUIRE(y_dtype == NVFP4MOE_F32 || y_dtype == NVFP4MOE_BF16, NVFP4MOE_EINVAL);
  if (G == 0 || m_cap == 0 || N == 0) return NVFP4MOE_OK;
  REQUIRE(x_e4m3 && x_e8m0 && w_e4m3 && w_e8m0 && offsets && y, NVFP4MOE_EINVAL);
  REQUIRE(N % 128 == 0 && K % 128 == 0 && K > 0, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(K <= kMaxGemmRowBytes, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(aligned16(x_e4m3) && aligned16(w_e4m3) && aligned16(y), NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_fwd_mxfp8(x_e4m3, x_e8m0, w_e4m3, w_e8m0, offsets, G, m_cap, N, K, y,
                                     y_dtype == NVFP4MOE_BF16, as_stream(stream)));
}

int mxfp8_gather_rows(const int32_t* row_token, const int64_t* offsets, int G, int64_t m_cap,
                      const uint8_t* src_e4m3, const uint8_t* src_e8m0, int64_t src_rows,
                      int64_t K, uint8_t* dst_e4m3, uint8_t* dst_e8m0, void* stream) {
  REQUIRE(G >= 0 && m_cap >= 0 && src_rows >= 0 && K >= 0, NVFP4MOE_EINVAL);
  if (G == 0 || m_cap == 0) return NVFP4MOE_OK;
  REQUIRE(row_token && offsets && src_e4m3 && src_e8m0 && dst_e4m3 && dst_e8m0, NVFP4MOE_EINVAL);
  REQUIRE(K % 32 == 0 && K > 0, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(aligned16(src_e4m3) && aligned16(dst_e4m3), NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_gather_rows(row_token, offsets, G, m_cap, src_rows, src_e4m3, src_e8m0,
                                       K, K / 32, dst_e4m3, dst_e8m0, as_stream(stream)));
}

int nvfp4_quantize_live(const void* x, int x_dtype, int64_t m_cap, int64_t cols,
                        const int64_t* n_live, uint8_t* codes, uint8_t* scales, float* outer,
                        void* stream) {
  REQUIRE(m_cap >= 0 && cols >= 0, NVFP4MOE_EINVAL);
  REQUIRE(x_dtype == NVFP4MOE_F32 || x_dtype == NVFP4MOE_BF16, NVFP4MOE_EINVAL);
  if (m_cap == 0) return NVFP4MOE_OK;
  REQUIRE(x && n_live && codes && scales && outer, NVFP4MOE_EINVAL);
  REQUIRE(cols > 0 && cols % 32 == 0 && cols <= 8192, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(aligned16(x) && aligned16(codes) && aligned16(scales), NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_nvfp4_quantize_live(x, x_dtype == NVFP4MOE_BF16, m_cap, cols, n_live,
                                               codes, scales, outer, as_stream(stream)));
}

int moe_combine(const void* y, int y_dtype, int64_t m_cap, int64_t T, int k, int64_t N,
                const int32_t* pair_row, const float* gate, void* out, int out_dtype,
                void* stream) {
  REQUIRE(m_cap >= 0 && T >= 0 && N >= 0 && k > 0, NVFP4MOE_EINVAL);
  REQUIRE(y_dtype == NVFP4MOE_F32 || y_dtype == NVFP4MOE_BF16, NVFP4MOE_EINVAL);
  REQUIRE(out_dtype == NVFP4MOE_F32 || out_dtype == NVFP4MOE_BF16, NVFP4MOE_EINVAL);
  if (T == 0 || N == 0) return NVFP4MOE_OK;
  REQUIRE(m_cap > 0 && y && pair_row && out, NVFP4MOE_EINVAL);
  REQUIRE(N % 8 == 0 && k <= 64, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(T * (N / 8) < ((int64_t)1 << 31), NVFP4MOE_EUNSUPPORTED);
  REQUIRE(aligned16(y) && aligned16(out), NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_combine(y, y_dtype == NVFP4MOE_BF16, m_cap, T, k, N, pair_row, gate,
                                   out, out_dtype == NVFP4MOE_BF16, as_stream(stream)));
}

int moe_combine_bwd(const void* dout, int dout_dtype, int64_t T, int k, int64_t N,
                    const int32_t* row_token, const int32_t* row_slot, const int64_t* offsets,
                    int G, int64_t m_cap, const float* gate, const void* y, int y_dtype,
                    void* dy, int dy_dtype, float* dgate, void* stream) {
  REQUIRE(T >= 0 && N >= 0 && k > 0 && G >= 0 && m_cap >= 0, NVFP4MOE_EINVAL);
  REQUIRE(dout_dtype == NVFP4MOE_F32 || dout_dtype == NVFP4MOE_BF16, NVFP4MOE_EINVAL);
  REQUIRE(dy_dtype == NVFP4MOE_F32 || dy_dtype == NVFP4MOE_BF16, NVFP4MOE_EINVAL);
  if (y) REQUIRE(y_dtype == NVFP4MOE_F32 || y_dtype == NVFP4MOE_BF16, NVFP4MOE_EINVAL);
  if (G == 0 || m_cap == 0 || N == 0) return NVFP4MOE_OK;
  REQUIRE(dout && row_token && row_slot && offsets && dy, NVFP4MOE_EINVAL);
  if (y) REQUIRE(dgate != nullptr, NVFP4MOE_EINVAL);
  REQUIRE(N % 8 == 0, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(aligned16(dout) && aligned16(dy) && aligned16(y), NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_combine_bwd(dout, dout_dtype == NVFP4MOE_BF16, N, k, row_token,
                                       row_slot, offsets, G, m_cap, gate, y,
                                       y_dtype == NVFP4MOE_BF16, dy, dy_dtype == NVFP4MOE_BF16,
                                       dgate, as_stream(stream)));
}

int moe_padded_offsets(const int64_t* offsets, int G, int align, int64_t* padded_offsets,
                       void* stream) {
  REQUIRE(G >= 0 && align > 0, NVFP4MOE_EINVAL);
  REQUIRE(offsets && padded_offsets, NVFP4MOE_EINVAL);
  REQUIRE(G <= 1024, NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_padded_offsets(offsets, G, align, padded_offsets, as_stream(stream)));
}

int nvfp4_quantize_sr(const void* x, int x_dtype, int64_t rows, int64_t cols, uint64_t seed,
                      uint32_t tag, uint8_t* codes, uint8_t* scales, float* outer,
                      void* stream) {
  REQUIRE(rows >= 0 && cols >= 0, NVFP4MOE_EINVAL);
  REQUIRE(x_dtype == NVFP4MOE_F32 || x_dtype == NVFP4MOE_BF16, NVFP4MOE_EINVAL);
  if (rows == 0) return NVFP4MOE_OK;
  REQUIRE(x && codes && scales && outer, NVFP4MOE_EINVAL);
  REQUIRE(cols > 0 && cols % 32 == 0 && cols <= 8192, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(aligned16(x) && aligned16(codes) && aligned16(scales), NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_nvfp4_quantize_sr(x, x_dtype == NVFP4MOE_BF16, rows, cols, seed, tag,
                                             codes, scales, outer, as_stream(stream)));
}

int nvfp4_requant_sr(const uint8_t* codes, const uint8_t* scales, const float* outer,
                     int outer_mode, int64_t rows_per_group, int64_t rows, int64_t cols,
                     const int64_t* offsets, const int64_t* padded_offsets, int G, int64_t P,
                     int layout, uint64_t seed, uint32_t tag, uint8_t* out_codes,
                     uint8_t* out_scales, float* out_outer, void* stream) {
  REQUIRE(rows >= 0 && cols >= 0 && G >= 0 && P >= 0, NVFP4MOE_EINVAL);
  REQUIRE(outer_mode == NVFP4MOE_OUTER_PER_ROW || outer_mode == NVFP4MOE_OUTER_PER_GROUP,
          NVFP4MOE_EINVAL);
  REQUIRE(layout == NVFP4MOE_LAYOUT_TRANSPOSED || layout == NVFP4MOE_LAYOUT_PER_GROUP,
          NVFP4MOE_EINVAL);
  const bool per_group = outer_mode == NVFP4MOE_OUTER_PER_GROUP;
  if (per_group) REQUIRE(rows_per_group > 0, NVFP4MOE_EINVAL);
  if (G == 0) return NVFP4MOE_OK;
  REQUIRE(offsets && padded_offsets && out_outer, NVFP4MOE_EINVAL);
  if (P == 0 || cols == 0) return hip_status(launch_nvfp4_requant_sr(
      codes, scales, outer, per_group ? rows_per_group : 0, 0, 0, offsets, padded_offsets, G, P,
      false, seed, tag, out_codes, out_scales, out_outer, as_stream(stream)));
  REQUIRE(out_codes && out_scales, NVFP4MOE_EINVAL);
  if (rows > 0) REQUIRE(codes && scales && outer, NVFP4MOE_EINVAL);
  REQUIRE(cols % 128 == 0 && P % 128 == 0, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(aligned16(codes) && aligned16(out_codes), NVFP4MOE_EUNSUPPORTED);
  REQUIRE((reinterpret_cast<uintptr_t>(scales) & 7u) == 0, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(((reinterpret_cast<uintptr_t>(out_scales) | reinterpret_cast<uintptr_t>(outer)) & 3u) == 0,
          NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_nvfp4_requant_sr(
      codes, scales, outer, per_group ? rows_per_group : 0, rows, cols, offsets, padded_offsets,
      G, P, layout == NVFP4MOE_LAYOUT_PER_GROUP, seed, tag, out_codes, out_scales, out_outer,
      as_stream(stream)));
}

int nvfp4_quantize_sr_colwise(const void* x, int x_dtype, int64_t rows, int64_t cols,
                              const int64_t* offsets, const int64_t* padded_offsets, int G,
                              int64_t P, uint64_t seed, uint32_t tag, uint8_t* out_codes,
                              uint8_t* out_scales, float* out_outer, void* stream) {
  REQUIRE(rows >= 0 && cols >= 0 && G >= 0 && P >= 0, NVFP4MOE_EINVAL);
  REQUIRE(x_dtype == NVFP4MOE_F32 || x_dtype == NVFP4MOE_BF16, NVFP4MOE_EINVAL);
  if (G == 0) return NVFP4MOE_OK;
  REQUIRE(offsets && padded_offsets && out_outer, NVFP4MOE_EINVAL);
  if (P > 0 && cols > 0) {
    REQUIRE(out_codes && out_scales, NVFP4MOE_EINVAL);
    if (rows > 0) REQUIRE(x != nullptr, NVFP4MOE_EINVAL);
    REQUIRE(cols % 128 == 0 && P % 128 == 0, NVFP4MOE_EUNSUPPORTED);
    REQUIRE(aligned16(x) && aligned16(out_codes), NVFP4MOE_EUNSUPPORTED);
  }
  return hip_status(launch_nvfp4_quantize_sr_colwise(
      x, x_dtype == NVFP4MOE_BF16, rows, (P > 0 ? cols : 0), offsets, padded_offsets, G, P, seed,
      tag, out_codes, out_scales, out_outer, as_stream(stream)));
}

int moe_bwd_wgrad_nvfp4(const uint8_t* dyT_codes, const uint8_t* dyT_scales,
                        const float* dyT_outer, const uint8_t* xT_codes, const uint8_t* xT_scales,
                        const float* xT_outer, const int64_t* padded_offsets, int G, int64_t P,
                        int64_t N, int64_t K, float* dw, void* stream) {
  REQUIRE(G >= 0 && P >= 0 && N >= 0 && K >= 0, NVFP4MOE_EINVAL);
  if (G == 0 || N == 0 || K == 0) return NVFP4MOE_OK;
  REQUIRE(dyT_codes && dyT_scales && dyT_outer && xT_codes && xT_scales && xT_outer &&
              padded_offsets && dw,
          NVFP4MOE_EINVAL);
  REQUIRE(N % 256 == 0 && K % 256 == 0 && P % 128 == 0, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(256 * (P / 2) < ((int64_t)1 << 32) - 1, NVFP4MOE_EUNSUPPORTED);
  REQUIRE(aligned16(dyT_codes) && aligned16(xT_codes) && aligned16(dw), NVFP4MOE_EUNSUPPORTED);
  REQUIRE(((reinterpret_cast<uintptr_t>(dyT_scales) | reinterpret_cast<uintptr_t>(xT_scales)) &
           7u) == 0,
          NVFP4MOE_EUNSUPPORTED);
  return hip_status(launch_wgrad_nvfp4(dyT_codes, dyT_scales, dyT_outer, xT_codes, xT_scales,
                                       xT_outer, padded_offsets, G, P, N, K, dw,
                                       as_stream(stream)));
}

}  // extern "C"
