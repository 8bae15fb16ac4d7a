/*
 * fp4rollout -- C ABI of the FP4 exploration hot path on MI355X (gfx950).
 *
 * The method (Sol-RL, "FP4 Explore, BF16 Train", project page section
 * "Two-Stage Pipeline"; aitrends summary, Stage-1 and Stage-2 paragraphs):
 * every iteration re-quantizes the current weights to a 4-bit float format,
 * integrates N = 96 noise seeds with a 6-step ODE solver whose linears run as
 * FP4 x FP4 products, scores the candidates with a proxy reward and keeps the
 * K/2 highest- and K/2 lowest-scoring seeds (K = 24) for BF16 regeneration.
 *
 * Conventions shared by every call:
 *   - All data pointers are DEVICE pointers (hipMalloc'ed or torch-owned);
 *     the caller owns and frees every buffer. The library allocates nothing.
 *   - Matrices are row-major; every leading dimension ("ld*") is the distance
 *     between consecutive rows, in ELEMENTS for float/bf16 arrays and in
 *     BYTES for packed codes and scale bytes. The exception is the panel
 *     layout of MXFP4 codes and scales (FP4_LAYOUT_PANEL, below).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on it; nothing synchronizes. A device
 *     fault therefore surfaces at the caller's next synchronization.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     non-OK status no kernel was launched and no output was touched.
 *   - Results are deterministic: repeated calls on the same inputs give
 *     bitwise-identical outputs (no floating-point atomics are used).
 *   - Inputs must be finite; NaN/Inf give unspecified (but memory-safe) output.
 *   - Output buffers must not overlap inputs unless a call says otherwise.
 */
#ifndef FP4ROLLOUT_H
#define FP4ROLLOUT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef FP4_API
#define FP4_API __attribute__((visibility("default")))
#endif

typedef int32_t fp4_status;
#define FP4_OK               0
#define FP4_INVALID_ARGUMENT 1  /* null pointer, bad size/stride/alignment, bad enum */
#define FP4_UNSUPPORTED      2  /* valid but not implemented combination */
#define FP4_DEVICE_ERROR     3  /* the HIP runtime reported an error at launch */
#define FP4_INTERNAL         4  /* unexpected host-side failure */

/* block formats */
#define FP4_FMT_MX 0  /* MXFP4: E2M1 codes, one E8M0 scale byte per 32 elements along K */
#define FP4_FMT_NV 1  /* NVFP4-style: E2M1 codes, one E4M3 scale byte per 16 elements
                         along K, and one fp32 scale for the whole tensor */

/* element types of float arrays */
#define FP4_DT_F32  0
#define FP4_DT_BF16 1

/* fp4_quantize flags */
#define FP4_PRO_RMSNORM        0x1   /* quantize x * (mean_k(x^2) + 1e-6)^(-1/2) (row-wise, unit gain) */
#define FP4_PRO_GELU           0x2   /* quantize x Phi(x) = 0.5 x (1 + erf(x / sqrt 2)). bf16 x: Phi(-|x|)
                                        from a table at every bf16 magnitude in [2^-22, 16]. fp32 x:
                                        the table entry at the bf16 rounding of |x| in [2^-10, 16]
                                        carried to |x| by a 4th-order expansion; erfc evaluated
                                        where |x| > 6. Relative error about 5e-7 either way */
#define FP4_TENSOR_SCALE_GIVEN 0x100 /* NV: read s_g from *tensor_scale instead of computing it */
#define FP4_LAYOUT_PANEL       0x200 /* MX: write codes and scales in the panel layout (below) */

/*
 * Panel layout -- the GEMM-native arrangement of an MXFP4 [rows, k] operand
 * (a storage order only: the codes and scale bytes are those of the
 * row-major layout). Rows are grouped into panels of 256, k into chunks of
 * 128 elements (nc = ceil(k / 128) chunks). The codes of one (panel, chunk)
 * pair form one contiguous 16 KiB block of 256 rows x 64 bytes, row-major
 * inside; the scale bytes one contiguous 1 KiB block of 256 rows x 4 bytes.
 * Blocks are ordered panel-major, chunk-minor:
 *   code byte j (elements 2j, 2j+1) of row r:
 *     ((r / 256 * nc + j / 64) * 256 + r % 256) * 64 + j % 64
 *   scale byte b (elements 32b .. 32b+31) of row r:
 *     ((r / 256 * nc + b / 4) * 256 + r % 256) * 4 + b % 4
 * Rows past `rows` in the last panel and elements past k in the last chunk
 * are padding, written by fp4_quantize as code byte 0 and scale byte 127
 * (2^0). Each load of a GEMM K stage is then one contiguous run, where
 * row-major rows give short pieces of many rows.
 */

/*
 * fp4_quantize -- block-scaled 4-bit quantization of a [rows, k] matrix along k.
 *
 * Used for the per-iteration weight re-quantization (project page,
 * "Two-Stage Pipeline", Stage 2: weights re-quantized for the next
 * iteration; aitrends summary: real-time re-quantization with no compile
 * step) and for the activations entering every FP4 linear of the solver
 * (project page: the FP4 solver's TFLOP rate needs both operands in FP4).
 *
 *   fmt          FP4_FMT_MX or FP4_FMT_NV.
 *   x            [rows, ldx] elements of type x_dtype (FP4_DT_F32 or FP4_DT_BF16);
 *                16-byte aligned, ldx*sizeof(elem) a multiple of 16, ldx >= k.
 *   rows, k      rows >= 1; k >= 32 and a multiple of 32 (MX) or 16 (NV).
 *   codes        out, [rows, ld_codes] bytes (or the panel layout, see flags);
 *                byte j of a row packs elements
 *                2j (low nibble) and 2j+1 (high nibble). Nibble = sign<<3 | m,
 *                magnitude G[m], G = {0, .5, 1, 1.5, 2, 3, 4, 6}; nearest value,
 *                ties to even m, saturating at 6, sign always kept.
 *                4-byte aligned, ld_codes a multiple of 4 and >= k/2.
 *   scales       out, [rows, ld_scales] bytes, one per block; any alignment.
 *                MX: S = max(floor(log2 amax) - 2, -127) + 127 (E8M0, value 2^(S-127)),
 *                    codes of x * 2^(127-S).
 *                NV: E4M3 code of fl(amax_block / fl(6 s_g)), round to nearest even,
 *                    saturating at 448; codes of fl(x / fl(dec(S) s_g)); a block
 *                    whose fl(dec(S) s_g) is 0 gets signed-zero codes.
 *                ld_scales >= k/32 (MX) or k/16 (NV).
 *   tensor_scale MX: must be NULL. NV: device float*, 4-byte aligned; receives
 *                s_g = fl(max|x| / 2688) (1 where that quotient is 0), or
 *                supplies it when flags has FP4_TENSOR_SCALE_GIVEN (it must then
 *                be positive and finite). Without that flag its word is also
 *                used as the amax accumulator while the call runs.
 *   flags        MX: at most one of FP4_PRO_RMSNORM / FP4_PRO_GELU (applied in
 *                fp32 before quantization), optionally FP4_LAYOUT_PANEL: codes
 *                and scales then use the panel layout (sizes from
 *                fp4_panel_bytes; codes 16-byte, scales 4-byte aligned;
 *                ld_codes and ld_scales must be 0).
 *                NV: only FP4_TENSOR_SCALE_GIVEN.
 */
FP4_API fp4_status fp4_quantize(int fmt, const void* x, int x_dtype, int64_t rows, int64_t k, int64_t ldx,
                        uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                        float* tensor_scale, int flags, void* stream);

/*
 * fp4_quantize_lora -- merge a LoRA adapter into a weight and re-quantize the
 * result (MXFP4 or NVFP4-style); the merged weight is never written.
 *
 * The policy is trained with LoRA adapters (rank 32 on the aitrends summary)
 * and after each update the adapted weights are re-quantized at run time for
 * the next FP4 rollout, with no compile step (aitrends summary, Stage-2
 * paragraph; project page, "Two-Stage Pipeline", Stage 2). The merge is the
 * standard LoRA form W' = W + scale * (B A), evaluated in fp32 as
 *     acc = sum over j = 0 .. rank-1, in order, of fmaf(B[n, j], A[j, k], acc)
 *     W'[n, k] = fmaf(scale, acc, W[n, k])
 * and W' is then quantized exactly as fp4_quantize(fmt, W', ...) would.
 * NV without FP4_TENSOR_SCALE_GIVEN takes two passes over W (and the
 * adapter): the first finds max |W'| for the tensor scale, the second
 * recomputes W' bit for bit and quantizes it.
 *
 *   fmt          FP4_FMT_MX or FP4_FMT_NV.
 *   w            [rows, ldw] weight (nn.Linear layout: rows = output features,
 *                k = input features) of type w_dtype, with the alignment and
 *                size rules of fp4_quantize's x.
 *   lora_b       [rows, ld_b] elements (ld_b >= rank), B of the adapter.
 *   lora_a       [rank, ld_a] elements (ld_a >= k), A of the adapter.
 *   ab_dtype     element type of lora_a and lora_b (FP4_DT_F32 or FP4_DT_BF16);
 *                both aligned to their element size.
 *   rank         1 .. 64.
 *   scale        the adapter's scale (alpha / rank in the usual
 *                parametrisation); finite.
 *   codes, ld_codes, scales, ld_scales, tensor_scale
 *                as for fp4_quantize with the same fmt (MX: row-major, or the
 *                panel layout with FP4_LAYOUT_PANEL and ld_codes = ld_scales =
 *                0, tensor_scale NULL; NV: row-major, tensor_scale receives
 *                s_g = fl(max|W'| / 2688), or supplies it with
 *                FP4_TENSOR_SCALE_GIVEN).
 *   flags        MX: 0 or FP4_LAYOUT_PANEL. NV: 0 or FP4_TENSOR_SCALE_GIVEN
 *                (FP4_LAYOUT_PANEL: FP4_UNSUPPORTED).
 *   Errors as for fp4_quantize; rank outside 1 .. 64, a non-finite scale or
 *   misaligned adapters: FP4_INVALID_ARGUMENT.
 */
FP4_API fp4_status fp4_quantize_lora(int fmt, const void* w, int w_dtype, int64_t rows, int64_t k, int64_t ldw,
                        const void* lora_b, int64_t ld_b, const void* lora_a, int64_t ld_a, int ab_dtype,
                        int64_t rank, float scale, uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                        int64_t ld_scales, float* tensor_scale, int flags, void* stream);

/*
 * fp4_quantize_nv_grouped -- fp4_quantize(FP4_FMT_NV, ...) with one tensor
 * scale per group of rows_per_group consecutive rows instead of one for the
 * whole argument: with the rollout's activations grouped per candidate, one
 * candidate's values no longer set another's tensor scale (the NVFP4 format
 * the pages name couples everything under one tensor scale). Group g's rows
 * are quantized exactly as fp4_quantize(FP4_FMT_NV) would quantize those rows
 * alone.
 *   x, x_dtype, rows, k, ldx, codes, ld_codes, scales, ld_scales
 *                   as for fp4_quantize with FP4_FMT_NV (row-major).
 *   rows_per_group  >= 1, dividing rows.
 *   tensor_scales   device float [rows / rows_per_group], 4-byte aligned:
 *                   receives each group's s_g, or supplies them with
 *                   FP4_TENSOR_SCALE_GIVEN (positive and finite); otherwise
 *                   also the groups' amax accumulators while the call runs.
 *   flags           0 or FP4_TENSOR_SCALE_GIVEN.
 */
FP4_API fp4_status fp4_quantize_nv_grouped(const void* x, int x_dtype, int64_t rows, int64_t k, int64_t ldx,
                        int64_t rows_per_group, uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                        int64_t ld_scales, float* tensor_scales, int flags, void* stream);

/*
 * fp4_panel_bytes -- sizes of the panel layout of a [rows, k] MXFP4 operand:
 *   *code_bytes  = ceil(rows / 256) * ceil(k / 128) * 16384,
 *   *scale_bytes = ceil(rows / 256) * ceil(k / 128) * 1024.
 * rows >= 1, k >= 32 and a multiple of 32; both outputs are host pointers.
 */
FP4_API fp4_status fp4_panel_bytes(int64_t rows, int64_t k, int64_t* code_bytes, int64_t* scale_bytes);

/*
 * fp4_gemm -- C[m, n] = sum_k A_hat[m, k] * B_hat[n, k]  (+ residual[m, n]),
 * accumulated in fp32. A is the activation [m, k], B the weight in nn.Linear
 * layout [n, k], both as fp4_quantize outputs of the same format. This is the
 * FP4 x FP4 product of every solver linear (project page, "Two-Stage
 * Pipeline": FP4 solver at up to 4x the BF16 TFLOP rate).
 *
 *   fmt               FP4_FMT_MX (E8M0 scale bytes, a_ts = b_ts = NULL) or
 *                     FP4_FMT_NV (E4M3 scale bytes, a_ts/b_ts = device float*
 *                     tensor scales; A_hat = G dec(S) s_g).
 *   a_codes, lda      [m, lda] bytes, 16-byte aligned, lda multiple of 16, lda >= k/2.
 *   a_scales, ld_as   [m, ld_as] bytes, any alignment, ld_as >= k/32 (MX) or k/16 (NV).
 *   b_codes.. ld_bs   same for B with n rows.
 *   m, n, k           >= 1; k a multiple of 32 (MX) or 16 (NV).
 *   c, c_dtype, ldc   out [m, ldc] of FP4_DT_F32 or FP4_DT_BF16 (fp32 rounded to
 *                     nearest even); 16-byte aligned (fp32) or 8-byte (bf16),
 *                     ldc a multiple of 4 elements, ldc >= n.
 *   residual          NULL, or fp32 [m, ldc] added to the fp32 sum before the
 *                     store (fp32 C only). residual == c (in place) is allowed.
 * Accuracy: |C - C_exact| <= 1e-4 * sum_k |A_hat B_hat| per element for fp32 C.
 */
FP4_API fp4_status fp4_gemm(int fmt,
                    const uint8_t* a_codes, int64_t lda, const uint8_t* a_scales, int64_t ld_as,
                    const float* a_ts,
                    const uint8_t* b_codes, int64_t ldb, const uint8_t* b_scales, int64_t ld_bs,
                    const float* b_ts,
                    int64_t m, int64_t n, int64_t k,
                    void* c, int c_dtype, int64_t ldc, const float* residual, void* stream);

/*
 * fp4_gemm_nv_grouped -- fp4_gemm(FP4_FMT_NV, ...) for an A quantized by
 * fp4_quantize_nv_grouped: row m of C takes the tensor scale of m's group,
 *   C[m, n] = a_ts[m / a_rows_per_group] * b_ts[0] * sum_k (G dec(S))_A (G dec(S))_B  (+ residual)
 * so each group's rows equal an fp4_gemm of that group alone, bit for bit.
 *   a_ts              device float [m / a_rows_per_group] (4-byte aligned).
 *   a_rows_per_group  >= 1, dividing m.
 *   other arguments   as for fp4_gemm with FP4_FMT_NV; scale rows must be
 *                     4-byte aligned (ld_as, ld_bs multiples of 4, as
 *                     fp4_quantize's outputs are), else FP4_UNSUPPORTED.
 */
FP4_API fp4_status fp4_gemm_nv_grouped(const uint8_t* a_codes, int64_t lda, const uint8_t* a_scales, int64_t ld_as,
                        const float* a_ts, int64_t a_rows_per_group, const uint8_t* b_codes, int64_t ldb,
                        const uint8_t* b_scales, int64_t ld_bs, const float* b_ts, int64_t m, int64_t n, int64_t k,
                        void* c, int c_dtype, int64_t ldc, const float* residual, void* stream);

/*
 * fp4_gemm_panel -- fp4_gemm for MXFP4 operands in the panel layout (same
 * product, accumulation, output and accuracy as fp4_gemm).
 *   fmt               FP4_FMT_MX (FP4_FMT_NV: FP4_UNSUPPORTED).
 *   a_codes, a_scales panel layout of A [m, k] as written by fp4_quantize with
 *                     FP4_LAYOUT_PANEL (padding included); codes 16-byte and
 *                     scales 4-byte aligned.
 *   b_codes, b_scales the same for B [n, k].
 *   m, n, k           >= 1; k a multiple of 32, k <= 2^23.
 *   c, c_dtype, ldc,  as in fp4_gemm.
 *   residual
 */
FP4_API fp4_status fp4_gemm_panel(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                          const uint8_t* b_codes, const uint8_t* b_scales,
                          int64_t m, int64_t n, int64_t k,
                          void* c, int c_dtype, int64_t ldc, const float* residual, void* stream);

/*
 * fp4_gemm_panel_gelu -- the first solver linear of a velocity block with the
 * GELU and the MXFP4 quantization of its output in its epilogue, for the
 * reading in which the hidden activation is stored as bf16 between the two
 * linears: the codes and scales of GELU(bf16(A_hat B_hat^T)) in the panel
 * layout of an [m, n] operand, ready for the block's second linear (project
 * page, "Two-Stage Pipeline": every solver linear runs FP4 x FP4; the
 * synthetic velocity block is h + W2 GELU(W1 RMSNorm(h))). Bit-identical to
 * fp4_gemm_panel(..., FP4_DT_BF16) into z followed by
 * fp4_quantize(z, FP4_LAYOUT_PANEL | FP4_PRO_GELU) -- without writing z.
 * The rollout's default is fp4_gemm_panel_gelu_f32; this is its option.
 *   fmt, a_*, b_*, m, n, k  as in fp4_gemm_panel; m and n multiples of 256
 *                           (otherwise FP4_UNSUPPORTED: use the unfused pair).
 *   out_codes, out_scales   the panel layout of [m, n] (fp4_panel_bytes(m, n)
 *                           bytes each), 16-byte and 4-byte aligned.
 */
FP4_API fp4_status fp4_gemm_panel_gelu(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                               const uint8_t* b_codes, const uint8_t* b_scales,
                               int64_t m, int64_t n, int64_t k,
                               uint8_t* out_codes, uint8_t* out_scales, void* stream);

/*
 * fp4_gemm_panel_gelu_f32 -- fp4_gemm_panel_gelu with GELU evaluated on the
 * fp32 sums themselves (no bf16 rounding of the hidden activation): the
 * reading in which the hidden activation stays fp32 between the two linears,
 * and the first linear of the rollout by default. Bit-identical to
 * fp4_gemm_panel(..., FP4_DT_F32) into z followed by
 * fp4_quantize(z, FP4_LAYOUT_PANEL | FP4_PRO_GELU). GELU is z Phi(z): Phi(-|z|)
 * from the workgroup's LDS table of (Phi(-a), phi(a)) at the bf16 magnitudes
 * a in [2^-10, 16], taken at a_c = the bf16 rounding of |z| and carried to |z|
 * by the fourth-order Taylor expansion in d = |z| - a_c (truncation below
 * 6e-8 relative); where |z| > 6 (or z is NaN) the complementary error
 * function is evaluated for that element instead. Relative error about 5e-7
 * overall; the value depends on z alone. Arguments as fp4_gemm_panel_gelu.
 */
FP4_API fp4_status fp4_gemm_panel_gelu_f32(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                                   const uint8_t* b_codes, const uint8_t* b_scales,
                                   int64_t m, int64_t n, int64_t k,
                                   uint8_t* out_codes, uint8_t* out_scales, void* stream);

/*
 * fp4_gemm_panel_euler -- the last block of the velocity network fused with
 * the Euler step that consumes it (aitrends summary, Stage-1 paragraph: a
 * 6-step FP4 ODE solve; the velocity is the residual stream plus the last
 * solver linear):
 *   x_out[i, j] = x[i, j] + (t_next - t_cur) * (residual[i, j] + sum_k A_hat[i, k] B_hat[j, k])
 * evaluated as fmaf(dt, fl(acc + residual), x) with dt = fl32(t_next - t_cur):
 * the same operations as fp4_gemm_panel(..., residual) into an fp32 v
 * followed by euler_step(x_out, x, v), so the result is bit-identical to
 * that pair -- without writing v or reading it back.
 *   fmt, a_*, b_*, m, n, k  as in fp4_gemm_panel (FP4_FMT_MX only).
 *   residual, x, x_out      fp32 [m, ldx], 16-byte aligned, ldx a multiple of 4,
 *                           ldx >= n; x_out may equal x and/or residual (in place).
 *   t_cur, t_next           the step's two times.
 * Accuracy: as fp4_gemm for the product; the update as euler_step.
 */
FP4_API fp4_status fp4_gemm_panel_euler(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                                const uint8_t* b_codes, const uint8_t* b_scales,
                                int64_t m, int64_t n, int64_t k,
                                const float* residual, const float* x, float* x_out, int64_t ldx,
                                float t_cur, float t_next, void* stream);

/*
 * fp4_gemm_panel_euler_reward -- fp4_gemm_panel_euler for the last block of
 * the last solver step, with the candidates' proxy reward (project page,
 * "Two-Stage Pipeline": candidates are scored with proxy rewards) taken from
 * the new state in the same pass, so x_out is not read back:
 *   x_out      exactly as fp4_gemm_panel_euler (bit-identical);
 *   rewards[c] = (1 / rows_per_cand) * sum over the candidate's rows i and all
 *                columns j of x_out[i, j] * u[j], c = 0 .. m / rows_per_cand - 1
 *                (the quantity fp4_proxy_reward computes with u, in another
 *                fp32 summation order: per lane fmas, per 128 x 128 wave a
 *                fixed shuffle tree, then the waves of a candidate in a fixed
 *                order; deterministic).
 *   fmt, a_*, b_*, m, n, k, residual, x, x_out, ldx, t_cur, t_next
 *              as in fp4_gemm_panel_euler.
 *   u          fp32 [n], 16-byte aligned.
 *   rows_per_cand  rows (tokens) per candidate; divides m.
 *   partials   caller workspace, fp32 [(m / 256) * (n / 256) * 4], 4-byte
 *              aligned (per-wave partial sums; contents undefined on return).
 *   rewards    fp32 [m / rows_per_cand] out, 4-byte aligned.
 * FP4_UNSUPPORTED unless m and n are multiples of 256 and rows_per_cand of
 * 128 (the sums cover whole 128 x 128 wave tiles).
 */
FP4_API fp4_status fp4_gemm_panel_euler_reward(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                                const uint8_t* b_codes, const uint8_t* b_scales,
                                int64_t m, int64_t n, int64_t k,
                                const float* residual, const float* x, float* x_out, int64_t ldx,
                                float t_cur, float t_next, const float* u, int64_t rows_per_cand,
                                float* partials, float* rewards, void* stream);

/*
 * fp4_gemm_panel_euler_reward_noalloc -- fp4_gemm_panel_euler_reward without
 * the `partials` workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). The per-wave partial sums go to a library-owned device array
 * of 2^18 floats (1 MiB) per GPU, held until the process ends; the call
 * itself allocates nothing (the first call on a device looks up the array's
 * address once). Arguments, layouts and results are those of
 * fp4_gemm_panel_euler_reward, bit for bit.
 *   Limit: (m / 256) * (n / 256) * 4 <= 262144 (e.g. m = 393216 rows at
 *   n = 3072 uses 73728); larger calls return FP4_INVALID_ARGUMENT.
 *   Every call on one GPU shares that GPU's array, so calls that overlap in
 *   time on one GPU (other streams, other host threads) race; calls ordered
 *   on one stream do not. Nothing in the array needs clearing: each call
 *   writes every partial it reads.
 */
FP4_API fp4_status fp4_gemm_panel_euler_reward_noalloc(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                                               const uint8_t* b_codes, const uint8_t* b_scales, int64_t m,
                                               int64_t n, int64_t k, const float* residual, const float* x,
                                               float* x_out, int64_t ldx, float t_cur, float t_next,
                                               const float* u, int64_t rows_per_cand, float* rewards,
                                               void* stream);

/*
 * euler_step -- one explicit Euler step of the sampler's ODE,
 *   x_out = x + (t_next - t_cur) * v,
 * with dt = fl32(t_next - t_cur) and an fp32 multiply-add per element. The
 * rollout takes 6 such steps from t = 1 to t = 0 (aitrends summary, Stage-1
 * paragraph: 6 FP4 inference steps; project page, "Key Insight": the ODE
 * sampler is deterministic).
 *   x_out, x   fp32 [numel], 16-byte aligned; x_out == x (in place) is allowed.
 *   v          [numel] of v_dtype (FP4_DT_F32 or FP4_DT_BF16), 16-byte aligned.
 *   numel      >= 1.
 */
FP4_API fp4_status euler_step(float* x_out, const float* x, const void* v, int v_dtype, int64_t numel,
                      float t_cur, float t_next, void* stream);

/*
 * fp4_proxy_reward -- per-candidate proxy reward (project page, "Two-Stage
 * Pipeline", Stage 1: candidates are scored with proxy rewards):
 *   u == NULL: reward[c] = mean over the rows_per_cand x dim block of candidate c;
 *   u != NULL: reward[c] = sum_d u[d] * (mean over rows of x[c, :, d]).
 *   x        fp32 [n_cand * rows_per_cand, ldx], 16-byte aligned, ldx multiple of
 *            4, ldx >= dim; dim a multiple of 4.
 *   u        NULL or fp32 [dim], 16-byte aligned.
 *   rewards  out fp32 [n_cand].
 * Summed in fp32 in a fixed order (one workgroup per candidate).
 */
FP4_API fp4_status fp4_proxy_reward(const float* x, int64_t n_cand, int64_t rows_per_cand, int64_t dim,
                            int64_t ldx, const float* u, float* rewards, void* stream);

/*
 * select_topk_bottomk -- the seed filter of Stage 1 (project page, "Two-Stage
 * Pipeline": keep the top/bottom-K most contrastive seeds; aitrends summary:
 * top K/2 and bottom K/2 of the 96 candidates), plus the normalised reward
 * r = 1/2 + 1/2 clip((x - mean)/std, -1, 1) (VeRL-Omni DiffusionNFT docs,
 * "Algorithm", first equation; std over the whole batch, ddof 0; std 0 -> 1/2).
 *
 * One total order ranks the candidates: raw reward descending, equal rewards
 * by ascending index. top_idx[i] is the i-th entry of that order (i < k_top);
 * bottom_idx[i] is the i-th entry from its end (i < k_bottom), i.e. lowest
 * reward first. With k_top + k_bottom <= n the two lists are disjoint.
 * Non-finite rewards are ranked too (the one exception to the finite-input
 * rule above): infinities by value, -0 equal to +0, and every NaN below -inf,
 * NaNs among themselves by ascending index. Every requested slot of top_idx
 * and bottom_idx therefore receives a valid index in 0..n-1; r_norm is NaN
 * everywhere when any reward is NaN.
 *   rewards     fp32 [n], 1 <= n <= 65536.
 *   top_idx     out int32 [k_top] (may be NULL when k_top == 0).
 *   bottom_idx  out int32 [k_bottom] (may be NULL when k_bottom == 0).
 *   r_norm      NULL or out fp32 [n].
 */
FP4_API fp4_status select_topk_bottomk(const float* rewards, int64_t n, int64_t k_top, int64_t k_bottom,
                               int32_t* top_idx, int32_t* bottom_idx, float* r_norm, void* stream);

/*
 * fp4_nft_noise / fp4_nft_loss -- the DiffusionNFT policy update's forward
 * pieces on the regenerated samples (VeRL-Omni DiffusionNFT docs,
 * "Algorithm"; the K seeds the FP4 rollout selects are regenerated in BF16
 * and trained on with DiffusionNFT -- aitrends summary, Stage-2 paragraph).
 * Sample i is a row of d fp32 values of each array (n samples; contiguous).
 *
 * fp4_nft_noise: the forward process on the rectified-flow path of the
 * rollout's sampler, x_t[i] = (1 - t[i]) x0[i] + t[i] eps[i], evaluated as
 * fmaf(t, eps, fl(1 - t) x0). Its velocity, the training target, is
 * v = eps - x0.
 *
 * fp4_nft_loss: with v+ = (1 - beta) v_old + beta v_theta and
 * v- = (1 + beta) v_old - beta v_theta (the implicit positive and negative
 * branches; v_old from the rollout policy, v_theta from the trained one, both
 * at x_t), per sample
 *   terms[i] = r[i] ||v+ - v||^2 + (1 - r[i]) ||v- - v||^2   (squared norm over d),
 * and *loss = mean of terms. r is the optimality probability (the r_norm of
 * select_topk_bottomk). Sums are fp32 in a fixed order (deterministic).
 *   v_old, v_theta, x0, eps  fp32 [n, d], 16-byte aligned; d a multiple of 4.
 *   r                 fp32 [n]; beta finite.
 *   n                 1 .. 65535.
 *   partials          caller workspace, fp32 [n * 128], 4-byte aligned.
 *   terms, loss       out: fp32 [n] and fp32 [1].
 */
FP4_API fp4_status fp4_nft_noise(const float* x0, const float* eps, const float* t, int64_t n, int64_t d,
                        float* x_t, void* stream);
FP4_API fp4_status fp4_nft_loss(const float* v_old, const float* v_theta, const float* x0, const float* eps,
                        const float* r, float beta, int64_t n, int64_t d, float* partials, float* terms,
                        float* loss, void* stream);

/* Human-readable name of a status code (static string). */
FP4_API const char* fp4_status_str(fp4_status s);

/* Version of this ABI (major * 100 + minor). */
FP4_API int fp4_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FP4ROLLOUT_H */
