// Launchers shared between the C-ABI layer (api.hip) and the kernel files.
// Each launcher assumes its arguments were validated by the C-ABI layer and
// only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4moe {

// quant.hip
hipError_t launch_nvfp4_quantize(const void* x, bool bf16, int64_t rows, int64_t cols,
                                 bool per_group, int64_t rows_per_group, uint8_t* codes,
                                 uint8_t* scales, float* outer, hipStream_t stream);
hipError_t launch_nvfp4_quantize_tile16(const void* x, bool bf16, int64_t rows, int64_t cols,
                                        int64_t rpg, uint8_t* codes, uint8_t* scales,
                                        float* outer, hipStream_t stream);
hipError_t launch_mxfp8_quantize_rowwise(const void* x, bool bf16, int64_t rows, int64_t cols,
                                         uint8_t* out_e4m3, uint8_t* out_e8m0,
                                         hipStream_t stream);

hipError_t launch_nvfp4_quantize_live(const void* x, bool bf16, int64_t rows, int64_t cols,
                                      const int64_t* n_live, uint8_t* codes, uint8_t* scales,
                                      float* outer, hipStream_t stream);

// combine.hip
hipError_t launch_combine(const void* y, bool y_bf16, int64_t m_cap, int64_t T, int k,
                          int64_t N, const int32_t* pair_row, const float* gate, void* out,
                          bool out_bf16, hipStream_t stream);
hipError_t launch_combine_bwd(const void* dout, bool dout_bf16, int64_t N, int k,
                              const int32_t* row_token, const int32_t* row_slot,
                              const int64_t* offsets, int G, int64_t m_cap, const float* gate,
                              const void* y, bool y_bf16, void* dy, bool dy_bf16, float* dgate,
                              hipStream_t stream);

// permute.hip
size_t permute_workspace_bytes(int64_t T, int k, int n_local);
size_t permute_scratch_bytes();
hipError_t permute_scratch_address(void** out);
hipError_t launch_permute(const int32_t* topk_ids, int64_t T, int k, int e0, int n_local,
                          const uint8_t* xq_codes, const uint8_t* xq_scales,
                          const float* xq_outer, int64_t K, int64_t* offsets,
                          int64_t* padded_offsets, int32_t* row_token, int32_t* row_slot,
                          int32_t* pair_row, uint8_t* xperm_codes, uint8_t* xperm_scales,
                          float* xperm_outer,
                          void* workspace, hipStream_t stream);

// requant.hip: grouped-transpose MXFP8 quantizers
hipError_t launch_requant_sr(const uint8_t* codes, const uint8_t* scales, const float* outer,
                             int64_t rows_per_group /* 0 = per row */, int64_t rows,
                             int64_t cols, const int64_t* offsets,
                             const int64_t* padded_offsets, int G, int64_t P,
                             bool blocked /* group g's [cols, length] block at cols * padded[g] */,
                             uint64_t seed, uint32_t tag, uint8_t* out_e4m3, uint8_t* out_e8m0,
                             hipStream_t stream);
hipError_t launch_mxfp8_quantize_colwise(const void* x, bool bf16, int64_t rows, int64_t cols,
                                         const int64_t* offsets,
                                         const int64_t* padded_offsets, int G, int64_t P,
                                         uint8_t* out_e4m3, uint8_t* out_e8m0,
                                         hipStream_t stream);

// permute.hip: copy rows dst[r] = src[row_token[r]] for r < offsets[G]
hipError_t launch_gather_rows(const int32_t* row_token, const int64_t* offsets, int G,
                              int64_t m_cap, int64_t src_rows, const uint8_t* src_q,
                              const uint8_t* src_s, int64_t qbytes, int64_t sbytes,
                              uint8_t* dst_q, uint8_t* dst_s, hipStream_t stream);

// requant.hip: both dY orientations from one read (row-wise for rows < offsets[G])
hipError_t launch_mxfp8_quantize_dual(const void* x, bool bf16, int64_t rows, int64_t cols,
                                      const int64_t* offsets, const int64_t* padded, int G,
                                      int64_t P, uint8_t* row_out, uint8_t* row_e8, uint8_t* out,
                                      uint8_t* out_e8, hipStream_t stream);

hipError_t launch_nvfp4_requant_sr(const uint8_t* codes, const uint8_t* scales,
                                   const float* outer, int64_t rpg, int64_t rows, int64_t cols,
                                   const int64_t* offsets, const int64_t* padded, int G, int64_t P,
                                   bool blocked, uint64_t seed, uint32_t tag, uint8_t* out,
                                   uint8_t* out_sc, float* out_outer, hipStream_t stream);
hipError_t launch_nvfp4_quantize_sr_colwise(const void* x, bool bf16, int64_t rows,
                                            int64_t cols, const int64_t* offsets,
                                            const int64_t* padded, int G, int64_t P,
                                            uint64_t seed, uint32_t tag, uint8_t* out,
                                            uint8_t* out_sc, float* out_outer,
                                            hipStream_t stream);
hipError_t launch_nvfp4_quantize_sr(const void* x, bool bf16, int64_t rows, int64_t cols,
                                    uint64_t seed, uint32_t tag, uint8_t* codes, uint8_t* scales,
                                    float* outer, hipStream_t stream);
hipError_t launch_padded_offsets(const int64_t* offsets, int G, int64_t align, int64_t* padded,
                                 hipStream_t stream);

// gemm_fwd.hip
hipError_t launch_wgrad_nvfp4(const uint8_t* ac, const uint8_t* as, const float* ao,
                              const uint8_t* bc, const uint8_t* bs, const float* bo,
                              const int64_t* padded, int G, int64_t P, int64_t N, int64_t K,
                              float* dw, hipStream_t stream);
hipError_t launch_fwd_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                                   const float* a_outer, const uint8_t* b_codes,
                                   const uint8_t* b_scales, const float* b_outer,
                                   const int64_t* offsets, int G, int64_t m_cap, int64_t N,
                                   int64_t K, void* y, bool y_bf16, hipStream_t stream);

// gemm_bwd.hip
hipError_t launch_dgrad(const uint8_t* dy_e4m3, const uint8_t* dy_e8m0, const uint8_t* w_e4m3,
                        const uint8_t* w_e8m0, const int64_t* offsets, int G, int64_t m_cap,
                        int64_t N, int64_t K, void* dx, bool dx_bf16, hipStream_t stream);
hipError_t launch_fwd_mxfp8(const uint8_t* x_e4m3, const uint8_t* x_e8m0, const uint8_t* w_e4m3,
                            const uint8_t* w_e8m0, const int64_t* offsets, int G, int64_t m_cap,
                            int64_t N, int64_t K, void* y, bool y_bf16, hipStream_t stream);
hipError_t launch_wgrad(const uint8_t* dyT_e4m3, const uint8_t* dyT_e8m0,
                        const uint8_t* xT_e4m3, const uint8_t* xT_e8m0,
                        const int64_t* padded_offsets, int G, int64_t P, int64_t N, int64_t K,
                        float* dw, hipStream_t stream);

// Number of workgroups that fill the device (compute units x wgs_per_cu).
int device_cu_count();

}  // namespace nvfp4moe
