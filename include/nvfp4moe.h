/*
 * nvfp4moe.h -- C ABI of the native 4-bit MoE expert layer for AMD MI355X (gfx950).
 *
 * The method (Thinking Machines, "End-to-End 4-Bit Training"; cited by the title
 * and section of the page that describes each step):
 *   forward:  NVFP4-quantize activations (one FP32 outer scale per token) and
 *             expert weights (one per expert), group routed tokens by expert,
 *             run the expert grouped GEMM on the NVFP4 operands;
 *   backward: dequantize the saved NVFP4 activations and weights, transpose in
 *             float32, re-quantize to MXFP8 with stochastic rounding, quantize
 *             dY to MXFP8, run the dgrad and wgrad grouped GEMMs in MXFP8.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller. The library never
 *     allocates, frees or synchronises; it validates arguments on the host, then
 *     enqueues kernels on `stream` (a hipStream_t; NULL = the default stream) and
 *     returns. Results are ready when the stream reaches that point.
 *   - Row-major everywhere; dimensions are int64_t element counts.
 *   - Argument errors return before any HIP call (NVFP4MOE_EINVAL for null
 *     pointers, negative sizes and bad enums; NVFP4MOE_EUNSUPPORTED for sizes or
 *     alignments the kernels do not handle). Launch failures return
 *     NVFP4MOE_EHIP. Faults inside kernels surface at the caller's next sync.
 *   - Inputs must be finite (no NaN/Inf); this is a precondition, not checked.
 *   - Device pointers must be 16-byte aligned.
 *   - Group offsets (`offsets`, `padded_offsets`) live on the device: they are
 *     produced by moe_permute and never copied to the host, so grids are sized
 *     for the capacity (`m_cap`, `P`) and kernels read the real extents.
 *   - Calls are stateless apart from a per-process device-property cache, and
 *     may be issued concurrently on different streams with disjoint outputs
 *     (moe_permute_noalloc excepted: see there).
 *
 * Where this interface departs from the one first planned for the path:
 *   - `stream` is a `void*` holding a hipStream_t, so the header needs no HIP
 *     include and binds from any language with a C FFI;
 *   - moe_permute takes one more output, `pair_row` (the inverse map, NULL
 *     allowed), which the combine and its backward read;
 *   - sizes are narrower than "multiple of 16": the quantizer takes
 *     cols % 32 == 0 and cols <= 8192 (one wavefront per row), the forward
 *     GEMM N % 128 == 0 and K % 128 == 0, the re-quantization cols % 128 == 0
 *     and P % 32 == 0, the MXFP8 GEMMs N and K multiples of 128 (each returns
 *     NVFP4MOE_EUNSUPPORTED otherwise);
 *   - mxfp8_requant_sr writes a weight (per-expert outer scales) as one
 *     [cols, length] block per expert, [E, K, N] for a weight [E*N, K], so
 *     moe_bwd_dgrad reads each expert's transposed weight as one contiguous
 *     block rather than a column slice of a [K, E*N] matrix;
 *   - entry points beyond the seven of the path: the all-MXFP8 forward, the
 *     routed FFN's combine and intermediate quantizer, the 16x16-tile and
 *     NVFP4-backward variants, the one-pass dual dY quantizer and
 *     moe_permute_noalloc.
 *
 * Formats (NVFP4 and MXFP8 as named on "Inkling 2 Small uses four-bit
 * training ..." (ai-primer), section "Block scales and per-token activations"):
 *   NVFP4  codes  uint8 [rows, cols/2]: E2M1 (sign|2-bit exponent|1-bit
 *                 mantissa), element 2j in bits 3..0, element 2j+1 in bits 7..4;
 *          scales uint8 [rows, cols/16]: OCP E4M3FN, one per 16 consecutive
 *                 elements of a row;
 *          outer  float [rows] (per token) or [groups] (per expert).
 *          value = e2m1 * scale * outer.
 *   MXFP8  elems  uint8 [rows, cols]: OCP E4M3FN;
 *          scales uint8 [rows, cols/32]: E8M0 (2^(c-127)), one per 32
 *                 consecutive elements of a row.
 */
#ifndef NVFP4MOE_H
#define NVFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4MOE_ABI_VERSION 3

#if defined(__GNUC__) || defined(__clang__)
#define NVFP4MOE_API __attribute__((visibility("default")))
#else
#define NVFP4MOE_API
#endif

enum nvfp4moe_status {
    NVFP4MOE_OK = 0,
    NVFP4MOE_EINVAL = 1,        /* null pointer, negative size, unknown enum */
    NVFP4MOE_EUNSUPPORTED = 2,  /* size/alignment not handled by the kernels */
    NVFP4MOE_EWORKSPACE = 3,    /* workspace smaller than required */
    NVFP4MOE_EHIP = 4           /* a HIP launch/runtime call failed */
};

enum nvfp4moe_dtype { NVFP4MOE_F32 = 0, NVFP4MOE_BF16 = 1 };

enum nvfp4moe_outer_mode { NVFP4MOE_OUTER_PER_ROW = 0, NVFP4MOE_OUTER_PER_GROUP = 1 };

enum nvfp4moe_orientation { NVFP4MOE_ROWWISE = 0, NVFP4MOE_COLWISE_GROUPED = 1 };

/* Output layout of the NVFP4 backward's transposes (nvfp4_requant_sr). */
enum nvfp4moe_layout { NVFP4MOE_LAYOUT_TRANSPOSED = 0, NVFP4MOE_LAYOUT_PER_GROUP = 1 };

/* Version of this ABI (NVFP4MOE_ABI_VERSION). */
NVFP4MOE_API int nvfp4moe_abi_version(void);

/* Static string naming a status code; never NULL. */
NVFP4MOE_API const char* nvfp4moe_status_string(int status);

/*
 * NVFP4 quantization of activations (per token) or weights (per expert).
 * Pages: "Inkling 2 Small uses four-bit training ..." (ai-primer), section
 * "Block scales and per-token activations": 16 values share one E4M3 scale;
 * an FP32 outer scale per expert for weights and per token for activations.
 *
 * x        [rows, cols] float32 (x_dtype NVFP4MOE_F32) or bfloat16 (NVFP4MOE_BF16).
 * outer_mode NVFP4MOE_OUTER_PER_ROW: one outer scale per row, outer[rows].
 *          NVFP4MOE_OUTER_PER_GROUP: each run of rows_per_group rows (one
 *          expert of a weight stored [E*N, K] with rows_per_group = N) shares
 *          one, outer[rows/rows_per_group]; outer doubles as scratch.
 * Per group of rows: A = max|x|; s = A/2688; block scale
 * S = E4M3_RNE(max|x_block| / (6*s)) (saturating); code = E2M1_RNE(x * (1/(S*s)))
 * (saturating); A == 0 or S == 0 gives signed-zero codes; outer = s.
 * codes [rows, cols/2], scales [rows, cols/16], outer as above.
 * Requires cols % 32 == 0 (EUNSUPPORTED otherwise); rows may be 0.
 */
NVFP4MOE_API int nvfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols,
                   int outer_mode, int64_t rows_per_group,
                   uint8_t* codes, uint8_t* scales, float* outer, void* stream);

/*
 * NVFP4 with one E4M3 scale per 16x16 tile: the transpose-invariant
 * alternative the pages report trying and rejecting as too sensitive to
 * outliers; kept for the ablation against 16-element blocks.
 * Pages: "Inkling 2 Small uses four-bit training ..." (ai-primer), section
 * "Stochastic rounding across transposes".
 *
 * x [rows, cols] (bf16 | f32), rows and cols multiples of 16; one outer scale
 * per group of rows_per_group rows (a multiple of 16 dividing rows; rows for a
 * single outer scale). A = max|x| over the group, s = A / 2688, tile scale
 * S = E4M3_RNE(max|x_tile| / (6 s)), codes E2M1_RNE(x * (1 / (S s))) (signed
 * zeros for a zero tile).
 * codes [rows, cols/2] (element 2j low nibble), scales [rows/16, cols/16],
 * outer [rows/rows_per_group] (float32, also the group-maximum scratch).
 * Requires x 16-byte and codes 8-byte aligned, rows/16 <= 65535.
 */
NVFP4MOE_API int nvfp4_quantize_tile16(const void* x, int x_dtype, int64_t rows, int64_t cols,
                          int64_t rows_per_group, uint8_t* codes, uint8_t* scales, float* outer,
                          void* stream);

/* Bytes of device workspace moe_permute needs for T tokens, top-k, n_local experts. */
NVFP4MOE_API size_t nvfp4moe_permute_workspace_size(int64_t T, int k, int n_local);

/*
 * Token-to-expert grouping and gather of the NVFP4 activation rows.
 * Pages: "Thinking Machines' Inkling 2 Small Trains a 594B Model in 68 Hours"
 * (hermes-ai), section "594B weights, 17B at work" (8 of 384 experts per token);
 * "Inkling 2 Small uses four-bit training ..." (ai-primer), section "Quantized
 * NVLink and BBBK" (tokens reach their experts already in NVFP4).
 *
 * topk_ids [T, k] int32 expert ids; ids outside [e0, e0+n_local) are not local
 * and are dropped. Outputs (device):
 *   offsets[n_local+1]        int64, exclusive scan of rows per local expert;
 *   padded_offsets[n_local+1] int64, exclusive scan of rows rounded up to 32;
 *   row_token[T*k], row_slot[T*k] int32: row r < offsets[n_local] holds pair
 *     (token, slot); rows of one expert are ordered by t*k+slot ascending;
 *   pair_row[T*k] int32 (may be NULL): the inverse map, pair_row[t*k+slot] =
 *     the row holding that pair, or -1 when its expert is not local;
 *   xperm_codes [T*k, K/2], xperm_scales [T*k, K/16], xperm_outer [T*k]: the
 *     NVFP4 row of row_token[r] copied to row r.
 * Entries at or beyond offsets[n_local] are left untouched.
 * workspace: device memory of at least nvfp4moe_permute_workspace_size() bytes.
 * Requires K % 32 == 0, 1 <= n_local <= 1024, 1 <= k <= 64.
 */
NVFP4MOE_API int moe_permute(const int32_t* topk_ids, int64_t T, int k, int e0, int n_local,
                const uint8_t* xq_codes, const uint8_t* xq_scales, const float* xq_outer,
                int64_t K,
                int64_t* offsets, int64_t* padded_offsets,
                int32_t* row_token, int32_t* row_slot, int32_t* pair_row,
                uint8_t* xperm_codes, uint8_t* xperm_scales, float* xperm_outer,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_permute for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments, results and kernels without the workspace, whose table
 * lives instead in a 4 MiB array the library holds on each GPU it runs on
 * until the process ends. Makes no allocating call.
 *
 * Returns NVFP4MOE_EWORKSPACE, before any HIP call, when the call would need
 * more than 4 MiB of table: nvfp4moe_permute_workspace_size(T, k, n_local) >
 * 4 MiB, i.e. ceil(T*k / 256) * n_local > 1048512 (T*k up to about 5.59 M
 * pairs with 48 local experts, 261,888 with 1024). The other argument rules
 * are moe_permute's. Calls issued on one GPU share its array: calls that
 * overlap in time on one GPU (on different streams, or from different host
 * threads without ordering) race and must not be made. Nothing needs
 * clearing between calls: each call writes every table entry it reads.
 */
NVFP4MOE_API int moe_permute_noalloc(const int32_t* topk_ids, int64_t T, int k, int e0,
                int n_local, const uint8_t* xq_codes, const uint8_t* xq_scales,
                const float* xq_outer, int64_t K,
                int64_t* offsets, int64_t* padded_offsets,
                int32_t* row_token, int32_t* row_slot, int32_t* pair_row,
                uint8_t* xperm_codes, uint8_t* xperm_scales, float* xperm_outer, void* stream);

/*
 * NVFP4 forward grouped GEMM.
 * Pages: "Inkling 2 Small uses four-bit training ..." (ai-primer), section
 * "NVFP4 forward, MXFP8 backward" (expert-layer matmuls in NVFP4).
 *
 * a_*: X_perm NVFP4 [m_cap, K] with per-row outer a_outer[m_cap];
 * b_*: W NVFP4 stored [G, N, K] (K contiguous) with per-expert outer b_outer[G];
 * offsets[G+1] (device): rows [offsets[g], offsets[g+1]) use expert g.
 * y [m_cap, N], y_dtype NVFP4MOE_F32 or NVFP4MOE_BF16 (round to nearest even):
 *   y[r, n] = a_outer[r] * b_outer[g] * sum_k (e2m1*S)_A[r,k] * (e2m1*S)_B[g,n,k]
 * with exact products and float32 accumulation. Rows >= offsets[G] untouched.
 * Requires N % 128 == 0, K % 128 == 0, offsets[G] <= m_cap.
 */
NVFP4MOE_API int moe_fwd_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_outer,
                         const uint8_t* b_codes, const uint8_t* b_scales, const float* b_outer,
                         const int64_t* offsets, int G, int64_t m_cap, int64_t N, int64_t K,
                         void* y, int y_dtype, void* stream);

/*
 * Backward re-quantization of a saved NVFP4 tensor: dequantize (float32) ->
 * grouped transpose -> MXFP8 with stochastic rounding.
 * Pages: "Inkling 2 Small uses four-bit training ..." (ai-primer), section
 * "Stochastic rounding across transposes".
 *
 * codes/scales/outer: NVFP4 [rows, cols]; outer_mode/rows_per_group as in
 *   nvfp4_quantize (per row for activations, per group for weights).
 * offsets[G+1], padded_offsets[G+1] (device int64): input rows
 *   [offsets[g], offsets[g+1]) become output columns starting at
 *   padded_offsets[g]; columns up to the next multiple of 32 are zero. For a
 *   weight [E*N, K] use offsets = padded_offsets = {0, N, 2N, ...} (N % 32 == 0).
 * NVFP4MOE_OUTER_PER_ROW (activations): out_e4m3 [cols, P], out_e8m0
 *   [cols, P/32]; P is the row pitch (P % 32 == 0, P >= padded_offsets[G]);
 *   columns >= padded_offsets[G] are untouched.
 * NVFP4MOE_OUTER_PER_GROUP (weights): one block per group, group g's
 *   [cols, L_g] (L_g = padded_offsets[g+1] - padded_offsets[g]) at element
 *   cols * padded_offsets[g], row pitch L_g, its E8M0 [cols, L_g/32] at
 *   cols * padded_offsets[g] / 32: for a weight [E*N, K] the transposed
 *   weights [E, K, N] that moe_bwd_dgrad reads. Padded offsets must then be
 *   multiples of 32.
 * Block of 32 along the output row: e = smallest exponent with
 *   max|v| <= 448*2^e (clamped to [-127,127]); y = v*2^-e; element rounded to
 *   E4M3 stochastically with the 16-bit draw of Philox4x32-10 keyed by
 *   (seed lo, seed hi), counter (q lo, q hi, tag, 0), q = idx>>3, for the
 *   logical index idx = col*P + p of output column col, padded position p
 *   (half idx&1 of word (idx&7)>>1), in both layouts.
 * Requires cols % 128 == 0.
 */
NVFP4MOE_API int mxfp8_requant_sr(const uint8_t* codes, const uint8_t* scales, const float* outer,
                     int outer_mode, int64_t rows_per_group, int64_t rows, int64_t cols,
                     const int64_t* offsets, const int64_t* padded_offsets, int G, int64_t P,
                     uint64_t seed, uint32_t tag,
                     uint8_t* out_e4m3, uint8_t* out_e8m0, void* stream);

/*
 * MXFP8 quantization of the output gradient dY with round-to-nearest-even.
 * Pages: "Inkling 2 Small uses four-bit training ..." (ai-primer), section
 * "NVFP4 forward, MXFP8 backward" (gradients computed with MXFP8 matmuls).
 *
 * x [rows, cols] float32 or bfloat16.
 * NVFP4MOE_ROWWISE: out_e4m3 [rows, cols], out_e8m0 [rows, cols/32] (blocks along
 *   cols); offsets/padded_offsets/G/P ignored.
 * NVFP4MOE_COLWISE_GROUPED: out_e4m3 [cols, P], out_e8m0 [cols, P/32], the same
 *   grouped transpose and padding as mxfp8_requant_sr.
 * Block exponent as in mxfp8_requant_sr; elements E4M3 round-to-nearest-even.
 * Requires cols % 128 == 0.
 */
NVFP4MOE_API int mxfp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int orientation,
                   const int64_t* offsets, const int64_t* padded_offsets, int G, int64_t P,
                   uint8_t* out_e4m3, uint8_t* out_e8m0, void* stream);

/*
 * Both MXFP8 orientations of dY from one read of it: the NVFP4MOE_ROWWISE and
 * NVFP4MOE_COLWISE_GROUPED results of mxfp8_quantize, byte for byte.
 * Pages: as mxfp8_quantize.
 *
 * row_e4m3 [rows, cols], row_e8m0 [rows, cols/32]: written for the rows that
 * belong to a group (offsets[0] <= r < offsets[G]), other rows untouched;
 * col_e4m3 [cols, P], col_e8m0 [cols, P/32]: as NVFP4MOE_COLWISE_GROUPED.
 * Requires cols % 128 == 0, P % 32 == 0, x, row_e4m3 and col_e4m3 16-byte
 * aligned.
 */
NVFP4MOE_API int mxfp8_quantize_dual(const void* x, int x_dtype, int64_t rows, int64_t cols,
                        const int64_t* offsets, const int64_t* padded_offsets, int G, int64_t P,
                        uint8_t* row_e4m3, uint8_t* row_e8m0, uint8_t* col_e4m3,
                        uint8_t* col_e8m0, void* stream);

/*
 * MXFP8 dgrad grouped GEMM (contraction over N).
 * Pages: "Inkling 2 Small uses four-bit training ..." (ai-primer), sections
 * "NVFP4 forward, MXFP8 backward" and "Stochastic rounding across transposes".
 *
 * dy: MXFP8 [m_cap, N] (blocks along N); w: MXFP8 [G, K, N] (each expert's
 * transposed weight contiguous, blocks along N, as mxfp8_requant_sr writes a
 * weight with NVFP4MOE_OUTER_PER_GROUP); offsets[G+1] (device).
 * dx[r, k] = sum_n dy[r, n] * w[g, k, n] for rows r of group g, float32
 * accumulation; dx [m_cap, K] float32 or bfloat16; rows >= offsets[G] untouched.
 * Requires N % 128 == 0, K % 128 == 0, N <= 16711935 (tile offsets are
 * 32-bit); otherwise NVFP4MOE_EUNSUPPORTED.
 */
NVFP4MOE_API int moe_bwd_dgrad(const uint8_t* dy_e4m3, const uint8_t* dy_e8m0,
                  const uint8_t* w_e4m3, const uint8_t* w_e8m0,
                  const int64_t* offsets, int G, int64_t m_cap, int64_t N, int64_t K,
                  void* dx, int dx_dtype, void* stream);

/*
 * All-MXFP8 forward grouped GEMM: the reference the NVFP4 forward is measured
 * against, and the precision of the last expert layers.
 * Pages: "Inkling 2 Small uses four-bit training ..." (ai-primer), TL;DR
 * (wall-clock savings reported against full MXFP8 training) and section
 * "Expert precision and convolution caches" (expert layers 40-47 kept in
 * MXFP8).
 *
 * x: MXFP8 [m_cap, K] (E4M3 elements, E8M0 scales [m_cap, K/32], blocks along
 * K), rows grouped by expert as moe_permute orders them; w: MXFP8 weights
 * stored [G, N, K] (scales [G, N, K/32]); offsets[G+1] (device).
 * y[r, n] = sum_k x[r, k] * w[g, n, k] for rows r of group g, exact products,
 * float32 accumulation; y [m_cap, N] float32 or bfloat16 (round to nearest
 * even); rows >= offsets[G] untouched.
 * Requires N % 128 == 0, K % 128 == 0, K <= 16711935, x, w, y 16-byte aligned;
 * otherwise NVFP4MOE_EUNSUPPORTED.
 */
NVFP4MOE_API int moe_fwd_grouped_gemm_mxfp8(const uint8_t* x_e4m3, const uint8_t* x_e8m0,
                               const uint8_t* w_e4m3, const uint8_t* w_e8m0,
                               const int64_t* offsets, int G, int64_t m_cap, int64_t N, int64_t K,
                               void* y, int y_dtype, void* stream);

/*
 * Gather of MXFP8 rows into expert order (the MXFP8 counterpart of
 * moe_permute's row copy).
 * Pages: as moe_permute.
 *
 * row_token[r] and offsets[G+1] as written by moe_permute (device); src: MXFP8
 * [src_rows, K] (+ scales [src_rows, K/32]); dst row r (r < offsets[G]) gets
 * src row row_token[r]; dst [m_cap, K] (+ [m_cap, K/32]); rows >= offsets[G]
 * untouched; row indices outside [0, src_rows) are skipped.
 * Requires K % 32 == 0, src and dst elements 16-byte aligned.
 */
NVFP4MOE_API int mxfp8_gather_rows(const int32_t* row_token, const int64_t* offsets, int G,
                      int64_t m_cap, const uint8_t* src_e4m3, const uint8_t* src_e8m0,
                      int64_t src_rows, int64_t K, uint8_t* dst_e4m3, uint8_t* dst_e8m0,
                      void* stream);

/*
 * MXFP8 wgrad grouped GEMM (contraction over the tokens of each expert).
 * Pages: as moe_bwd_dgrad.
 *
 * dyT: MXFP8 [N, P] (grouped transpose of dY); xT: MXFP8 [K, P] (requantized
 * activations); padded_offsets[G+1] (device).
 * dw[g, n, k] = sum over p in [padded_offsets[g], padded_offsets[g+1]) of
 * dyT[n, p] * xT[k, p], float32 accumulation; dw [G, N, K] float32 (the stored
 * weight layout). Groups with no tokens get zeros.
 * Requires N % 128 == 0, K % 128 == 0, P % 32 == 0, P <= 16711935 and
 * G <= 16384; otherwise NVFP4MOE_EUNSUPPORTED.
 */
NVFP4MOE_API int moe_bwd_wgrad(const uint8_t* dyT_e4m3, const uint8_t* dyT_e8m0,
                  const uint8_t* xT_e4m3, const uint8_t* xT_e8m0,
                  const int64_t* padded_offsets, int G, int64_t P, int64_t N, int64_t K,
                  float* dw, void* stream);

/*
 * Per-row NVFP4 quantization of the routed rows of a capacity-sized buffer:
 * the expert FFN's intermediate activation, re-quantized per token before the
 * down-projection. Pages: "Inkling 2 Small uses four-bit training ..."
 * (ai-primer), sections "NVFP4 forward, MXFP8 backward" (expert matmuls in
 * NVFP4) and "Block scales and per-token activations" (one outer scale per
 * token).
 *
 * x [m_cap, cols] float32 or bfloat16; n_live (device, e.g. &offsets[G] of
 * moe_permute): rows r < min(*n_live, m_cap) are quantized exactly as
 * nvfp4_quantize does with NVFP4MOE_OUTER_PER_ROW; later rows untouched.
 * Requires cols % 32 == 0, cols <= 8192, x, codes, scales 16-byte aligned.
 */
NVFP4MOE_API int nvfp4_quantize_live(const void* x, int x_dtype, int64_t m_cap, int64_t cols,
                        const int64_t* n_live, uint8_t* codes, uint8_t* scales, float* outer,
                        void* stream);

/*
 * Expert outputs back to token order: weighted sum over each token's routed
 * pairs (the combine step; with gate == NULL, the un-permute sum of the
 * backward pass). Pages: "Inkling 2 Small uses four-bit training ..."
 * (ai-primer), section "Quantized NVLink and BBBK" (expert outputs are
 * combined back to their tokens; the Hadamard + S2F6 transfer format is a
 * communication step between GPUs, not part of this call).
 *
 * y [m_cap, N] float32 or bfloat16, rows in moe_permute's order; pair_row
 * [T, k] (device) as written by moe_permute; gate [T, k] float32 or NULL
 * (all ones).
 * out[t, n] = sum over j = 0..k-1 with pair_row[t, j] in [0, m_cap) of
 * gate[t, j] * y[pair_row[t, j], n], float32 fused multiply-adds in slot
 * order from 0; out [T, N] float32 or bfloat16 (round to nearest even).
 * Requires m_cap >= 1 when T > 0, N % 8 == 0, k <= 64, T * N / 8 < 2^31, y
 * and out 16-byte aligned.
 */
NVFP4MOE_API int moe_combine(const void* y, int y_dtype, int64_t m_cap, int64_t T, int k,
                int64_t N, const int32_t* pair_row, const float* gate, void* out,
                int out_dtype, void* stream);

/*
 * Backward of moe_combine for the routed rows. Pages: as moe_combine.
 *
 * dout [T, N] float32 or bfloat16; row_token, row_slot, offsets[G+1] (device)
 * as written by moe_permute; gate [T, k] float32 or NULL (ones); y [m_cap, N]
 * (the forward's expert outputs) or NULL.
 * For rows r < min(offsets[G], m_cap), with (t, j) = (row_token[r],
 * row_slot[r]):
 *   dy[r, n]   = gate[t, j] * dout[t, n] (float32 product; dy float32 or
 *                bfloat16, round to nearest even);
 *   dgate[t*k + j] = sum_n dout[t, n] * y[r, n] (float32; only when y is
 *                given; entries of non-local pairs untouched).
 * Requires N % 8 == 0 and dout, y, dy 16-byte aligned.
 */
NVFP4MOE_API int moe_combine_bwd(const void* dout, int dout_dtype, int64_t T, int k, int64_t N,
                    const int32_t* row_token, const int32_t* row_slot,
                    const int64_t* offsets, int G, int64_t m_cap, const float* gate,
                    const void* y, int y_dtype, void* dy, int dy_dtype, float* dgate,
                    void* stream);

/* ---------------------------------------------------------------------------
 * NVFP4 backward: the alternative to the MXFP8 backward, with every gradient
 * matmul operand in NVFP4. Pages: "Inkling 2 Small uses four-bit training ..."
 * (ai-primer), section "NVFP4 forward, MXFP8 backward" (NVFP4 in both passes
 * was tried first and given up) and section "Stochastic rounding across
 * transposes" (the re-quantization recipe kept here); "Thinking Machines
 * details ... 4 bit" (advanceintelligence.ai), section "What to expect next"
 * (a 4-bit backward is being explored).
 * Common rules: E4M3 block scales are rounded up, S = smallest E4M3 value >=
 * max|block| / (6 s), so scaled elements stay within [-6, 6]; E2M1 codes are
 * rounded stochastically with the 16-bit Philox draw of the element's linear
 * output index (as in mxfp8_requant_sr), a magnitude above 6 (float32
 * rounding only) becoming 6; blocks whose scale is 0 hold signed zeros; outer
 * scales s = A / 2688 with A the largest magnitude they cover.
 * dgrad is moe_fwd_grouped_gemm with a = NVFP4 dY (one outer per row) and
 * b = the per-expert transposed weights [G, K, N] (one outer per expert).
 * ------------------------------------------------------------------------- */

/*
 * padded_offsets[g] = sum over g' < g of round_up(offsets[g'+1] - offsets[g'],
 * align), g = 0..G (device arrays). Requires G <= 1024.
 */
NVFP4MOE_API int moe_padded_offsets(const int64_t* offsets, int G, int align,
                       int64_t* padded_offsets, void* stream);

/*
 * Row-wise NVFP4 with stochastic rounding: x [rows, cols] float32 or bfloat16,
 * one outer scale per row (outer[rows]), blocks of 16 along the row; codes
 * [rows, cols/2], scales [rows, cols/16]; the draw of element (r, c) is at
 * index r * cols + c. Requires cols % 32 == 0, cols <= 8192, x, codes, scales
 * 16-byte aligned.
 */
NVFP4MOE_API int nvfp4_quantize_sr(const void* x, int x_dtype, int64_t rows, int64_t cols,
                      uint64_t seed, uint32_t tag, uint8_t* codes, uint8_t* scales,
                      float* outer, void* stream);

/*
 * Saved NVFP4 [rows, cols] (outer per row, or per rows_per_group rows) ->
 * dequantize (float32) -> grouped transpose -> NVFP4 with stochastic
 * rounding along the former rows, one outer scale per group: out_outer[G].
 * Input rows [offsets[g], offsets[g+1]) become output columns
 * [padded_offsets[g], ... + length) of group g, zero up to
 * padded_offsets[g+1]; padded offsets must be multiples of 128 (see
 * moe_padded_offsets) and P >= padded_offsets[G].
 * layout NVFP4MOE_LAYOUT_TRANSPOSED: codes [cols, P/2], scales [cols, P/16],
 *   element (k, p) at linear index k * P + p; columns >= padded_offsets[G]
 *   untouched.
 * layout NVFP4MOE_LAYOUT_PER_GROUP (weights: all groups of one length L):
 *   group g's block [cols, L] at element g * cols * L, element (k, p) at
 *   g * cols * L + k * L + (p - padded_offsets[g]): the transposed weights
 *   [G, K, N] of the dgrad.
 * out_codes and out_outer hold scratch during the call; offsets[G] must not
 * exceed rows. Requires cols % 128 == 0,
 * P % 128 == 0, codes, out_codes 16-byte aligned, scales 8-byte aligned.
 */
NVFP4MOE_API int nvfp4_requant_sr(const uint8_t* codes, const uint8_t* scales, const float* outer,
                     int outer_mode, int64_t rows_per_group, int64_t rows, int64_t cols,
                     const int64_t* offsets, const int64_t* padded_offsets, int G, int64_t P,
                     int layout, uint64_t seed, uint32_t tag, uint8_t* out_codes,
                     uint8_t* out_scales, float* out_outer, void* stream);

/*
 * dY [rows, cols] float32 or bfloat16 -> grouped transpose [cols, P] -> NVFP4
 * with stochastic rounding, one outer scale per group (the wgrad operand).
 * Same grouping, layout and requirements as nvfp4_requant_sr with
 * NVFP4MOE_LAYOUT_TRANSPOSED.
 */
NVFP4MOE_API int nvfp4_quantize_sr_colwise(const void* x, int x_dtype, int64_t rows, int64_t cols,
                              const int64_t* offsets, const int64_t* padded_offsets, int G,
                              int64_t P, uint64_t seed, uint32_t tag, uint8_t* out_codes,
                              uint8_t* out_scales, float* out_outer, void* stream);

/*
 * NVFP4 wgrad grouped GEMM: dyT NVFP4 [N, P] (outer dyT_outer[G]), xT NVFP4
 * [K, P] (outer xT_outer[G]), padded_offsets[G+1] multiples of 128 (device).
 * dw[g, n, k] = dyT_outer[g] * xT_outer[g] * sum over p in group g's columns
 * of (e2m1 * S)_dyT[n, p] * (e2m1 * S)_xT[k, p], exact products (f16 MFMA),
 * float32 accumulation; dw [G, N, K] float32; empty groups get zeros.
 * Requires N % 256 == 0, K % 256 == 0, P % 128 == 0, 128 * P < 2^32.
 */
NVFP4MOE_API int moe_bwd_wgrad_nvfp4(const uint8_t* dyT_codes, const uint8_t* dyT_scales,
                        const float* dyT_outer, const uint8_t* xT_codes,
                        const uint8_t* xT_scales, const float* xT_outer,
                        const int64_t* padded_offsets, int G, int64_t P, int64_t N, int64_t K,
                        float* dw, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4MOE_H */
