/*
 * moe_gg.h -- C ABI of the MI355X (gfx950) MoE grouped-GEMM backward library.
 *
 * The library computes the two backward GEMMs of a mixture-of-experts layer
 * whose token rows are bucketed by expert through an offset array:
 *
 *   weight gradient  grad_w[e] = g[o_e:o_{e+1}]^T . x[o_e:o_{e+1}]
 *                    (MXFP8 inputs, f32 accumulation, bf16 output)
 *   data gradient    dx[r]     = g[r] . W_{e(r)}        (f32)
 *
 * plus the MX quantiser that produces the weight gradient's inputs.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or equivalent),
 *     row-major, densely packed, with the layouts stated below.
 *   - Calls enqueue work on `stream` (0 = the null stream) and return without
 *     synchronising.  Errors found on the host come back as a negative
 *     status before anything is enqueued; a device fault shows at the
 *     caller's next synchronisation.
 *   - The caller owns every buffer.  The library allocates no memory and
 *     keeps no mutable global state: calls are reentrant and thread-safe.
 *     Outputs are fully overwritten (no accumulate mode).
 *   - The host never reads `expert_off` (device memory).  Offsets must satisfy
 *     off[0] = 0, off[e] <= off[e+1], off[E] = M; a malformed array yields
 *     unspecified values but no access outside the buffers (each bound is
 *     clamped to [0, M], a decreasing pair counts as empty).
 *   - Empty sizes: a size of 0 is valid (a negative size, or E < 1, is
 *     MOE_GG_EINVAL).  A call whose output has no element returns MOE_GG_OK
 *     and enqueues nothing.  A call whose contraction is empty (no tokens,
 *     M = 0, for the weight gradient; N = 0 for the data gradient; K = 0 for
 *     the grouped GEMM) writes zeros: the empty sum.  A pointer to a buffer of
 *     zero size may be NULL; expert_off may not.
 *   - Debugging aid: with MOE_GG_VALIDATE=1 in the environment (read at each
 *     call), the weight gradient, data gradient and grouped GEMM entry points
 *     copy `expert_off` to the host, synchronising `stream`, and return
 *     MOE_GG_EINVAL before launching if the offsets break those rules.
 */
#ifndef MOE_GG_H
#define MOE_GG_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_GG_API __attribute__((visibility("default")))

enum {
  MOE_GG_OK = 0,
  MOE_GG_EINVAL = -1,       /* null pointer, negative size, misaligned size       */
  MOE_GG_EUNSUPPORTED = -2, /* valid request outside what the kernels tile        */
  MOE_GG_ELAUNCH = -3       /* the HIP runtime refused the launch                 */
};

/*
 * Grouped MXFP8 weight gradient.
 *
 * Source: the tinygrad page "grouped_mxfp8_wgrad.cpp" (kernel signature and
 * its global layouts A = g^T, B = x^T, C = grad_w with the experts stacked;
 * its k-loop over the expert's 128-token blocks; its epilogue, which stores
 * the zero-initialised accumulators of an empty expert as they are).
 *
 *   A        g^T, E4M3 bytes [N][M]   (token axis contiguous)
 *   B        x^T, E4M3 bytes [K][M]
 *   C        grad_w, bf16 bits [E*N][K]; rows e*N..e*N+N-1 hold expert e;
 *            every element is written, an empty expert's rows with +0.0
 *   scale_A  E8M0 bytes [N][M/32]: scale of A[n][32j..32j+31] is 2^(s-127)
 *   scale_B  E8M0 bytes [K][M/32]
 *   expert_off int32 [E+1]: off[0] = 0, nondecreasing, off[E] = M
 *
 *   grad_w[e*N+n][k] = bf16_rne( sum over m in [off[e], off[e+1]) of
 *                        e4m3(A[n][m]) 2^(sA[n][m/32]-127) e4m3(B[k][m]) 2^(sB[k][m/32]-127) )
 *   accumulated in f32.
 *
 * Shapes: M, N, K >= 0, E >= 1, M % 32 == 0 (EINVAL otherwise; M = 0
 * writes +0.0 everywhere); M % 128 == 0,
 * N % 256 == 0, K % 256 == 0, E <= 1024, 256 M < 2^32 and 512 K < 2^31
 * (EUNSUPPORTED otherwise: 32-bit offsets inside an operand panel and an
 * output tile).
 * Expert bounds need not be multiples of 128 (nor of 32): an expert's first
 * and last 128-token steps zero the g^T codes of the tokens outside it, so a
 * scale block shared by two experts contributes its own tokens to each.
 * Offsets are read on the device and clamped to [0, M]; a decreasing pair
 * makes that expert empty.
 *
 * Accuracy: gfx950's block-scaled fp8 MFMA sums each run of 8 consecutive
 * tokens after truncating every product toward zero to a multiple of
 * 2^(floor(log2 p_max) - 13), p_max the largest product magnitude of the run
 * (measured on the hardware).  Where an outlier of g^T meets an outlier of
 * x^T at one token, that run's other products are mostly lost, and no split
 * of the codes into two passes avoids it (several outliers of one row can
 * share a run).  This entry point therefore converts the codes, times their
 * scales, to bf16 (exactly: 4 significant bits, the scale inside bf16's
 * exponent range) and multiplies them on the bf16 MFMA, which adds its 16
 * products to within 2^-22 of the largest of them (measured; the exact sum,
 * rounded once, when they span 2^14 or less) into the f32 accumulator.  The
 * result is thus the exact sum up to f32-level accumulation error and the
 * final bf16 rounding, with or without outliers.  The conversion is exact
 * for every element value bf16 can hold: any code with scale bytes 3..246
 * (all MX quantiser outputs whose block maximum is at least 2^-116), and
 * larger scale bytes with codes below 2^8.  Beyond that, values below
 * bf16's smallest subnormal, 2^-133, round to multiples of it (2^-136 to
 * zero), and values above its largest finite value become infinite
 * (measured); the fast entry point has neither limit.
 */
MOE_GG_API int moe_gg_wgrad_mxfp8(const uint8_t *A, const uint8_t *B, uint16_t *C,
                                  const uint8_t *scale_A, const uint8_t *scale_B,
                                  const int32_t *expert_off, int M, int N, int K, int E,
                                  hipStream_t stream);

/*
 * The same grouped MXFP8 weight gradient on the block-scaled fp8 MFMA
 * (v_mfma_scale_f32_32x32x64_f8f6f4): the hardware's own reduction as
 * described above, at twice the bf16 MFMA's rate.  Same arguments, layouts,
 * shapes and status codes as moe_gg_wgrad_mxfp8.  The result equals the
 * exact sum when every 8-token run's products are within 2^6 of each other,
 * and otherwise can differ by up to 2^-13 of the run's largest product per
 * product.  For callers whose inputs have a moderate in-block range (no
 * outliers) or who accept the hardware's rounding.
 */
MOE_GG_API int moe_gg_wgrad_mxfp8_fast(const uint8_t *A, const uint8_t *B, uint16_t *C,
                                       const uint8_t *scale_A, const uint8_t *scale_B,
                                       const int32_t *expert_off, int M, int N, int K, int E,
                                       hipStream_t stream);

/*
 * Grouped f32 data gradient.
 *
 * Source: the oarust page "grouped_gemm_m_data_backward.slang" (push
 * constants output_gradient, weight, offsets, input_gradient, rows,
 * output_features, input_features, experts; the row -> expert scan
 * expert_for_row; the per-row-expert dot products of tiles that span
 * several experts; the overwriting store).
 *
 *   A   g  (output gradient), f32 [M][N]          N = output_features
 *   B   W  (expert weights),  f32 [E][N][K]        K = input_features
 *   C   dx (input gradient),  f32 [M][K]
 *   expert_off int32 [E+1]; any nondecreasing values (no alignment needed)
 *
 *   dx[r][k] = sum_n g[r][n] W[e(r)][n][k],  e(r) the e with off[e] <= r < off[e+1],
 *   f32 products and f32 accumulation.
 *
 * Shapes: M, N, K >= 0, E >= 1 (EINVAL otherwise; N = 0 writes zeros);
 * K % 4 == 0 and N % 4 == 0 (EUNSUPPORTED otherwise).
 */
MOE_GG_API int moe_gg_dgrad_f32(const float *A, const float *B, float *C,
                                const int32_t *expert_off, int M, int N, int K, int E,
                                hipStream_t stream);

/*
 * Expert-grouped MXFP8 GEMM (the MoE forward, and with transposed weights an
 * MXFP8 data gradient).
 *
 * Source: the tinygrad page's expert_off bucketing of token rows and the
 * Slang page's expert_for_row (each row uses its own expert's weights); the
 * vLLM page's mfma_f8f8 (fp8 weights with one E8M0 scale per 32 along the
 * contraction, times fp8 activations, on the block-scaled MFMA).
 *
 *   A        E4M3 bytes [M][K]      (token rows, contraction contiguous)
 *   B        E4M3 bytes [E][N][K]   (expert e's weights, contraction contiguous)
 *   C        bf16 bits  [M][N], every element written
 *   scale_A  E8M0 [M][K/32]; scale_B  E8M0 [E][N][K/32]
 *   expert_off int32 [E+1]: off[0] = 0, nondecreasing, off[E] = M (any
 *            alignment).  On the device each entry is clamped to [0, M] and
 *            raised to the largest entry before it, which leaves well-formed
 *            offsets as they are and gives any others disjoint row ranges.
 *
 *   C[m][j] = bf16_rne( sum over c of deq(A)[m][c] deq(B[e(m)])[j][c] ),
 *   accumulated in f32, e(m) the expert with off[e] <= m < off[e+1]; rows of
 *   no expert (off[0] > 0 or off[E] < M) are +0.0.
 *
 * Forward y = x W_e^T: A = MX(x) along K, B[e] = MX(W_e) along K.
 * Data gradient dx = g W_e with W_e [N][K]: A = MX(g) along N (this call's K
 * is N), B[e] = moe_gg_mx_quantize_t(W_e) ([K][N] along N).
 *
 * Shapes: M, N, K >= 0, E >= 1 and K % 32 == 0 (EINVAL otherwise; K = 0
 * writes +0.0 everywhere); N % 256 == 0,
 * K % 128 == 0 and E <= 2048 (EUNSUPPORTED otherwise).  Accuracy as for the
 * weight gradient: the codes, times their scales, are converted exactly to
 * bf16 (within the range stated there) and multiplied on the bf16 MFMA with
 * f32 accumulation, so the result is the exact sum up to f32-level
 * accumulation error and the bf16 rounding, also with outliers in either
 * operand or both.
 */
MOE_GG_API int moe_gg_grouped_mxfp8(const uint8_t *A, const uint8_t *B, uint16_t *C,
                                    const uint8_t *scale_A, const uint8_t *scale_B,
                                    const int32_t *expert_off, int M, int N, int K, int E,
                                    hipStream_t stream);

/*
 * The same expert-grouped GEMM in one block-scaled MFMA pass (the hardware's
 * own reduction; see moe_gg_wgrad_mxfp8_fast).  Same arguments and status
 * codes.
 */
MOE_GG_API int moe_gg_grouped_mxfp8_fast(const uint8_t *A, const uint8_t *B, uint16_t *C,
                                         const uint8_t *scale_A, const uint8_t *scale_B,
                                         const int32_t *expert_off, int M, int N, int K, int E,
                                         hipStream_t stream);

/*
 * Expert-grouped GEMM with MXFP4 weights (a8w4): the same as
 * moe_gg_grouped_mxfp8 with B[e] holding E2M1 codes.
 *
 * Source: the decode page's a8w4 MoE stages and mfma_f4f8 (fp4 weights with
 * one E8M0 scale per 32 along k, times MXFP8 activations, on the f8f6f4
 * scaled MFMA with format 4 for the fp4 operand); the token bucketing as for
 * moe_gg_grouped_mxfp8.
 *
 *   A        E4M3 bytes [M][K]        (token rows)
 *   B        E2M1 codes [E][N][K/2]   two per byte along K, element 2i in the
 *            low nibble (moe_gg_mx4_quantize's layout)
 *   C        bf16 bits  [M][N], every element written
 *   scale_A  E8M0 [M][K/32]; scale_B  E8M0 [E][N][K/32]
 *   expert_off int32 [E+1] as for moe_gg_grouped_mxfp8
 *
 *   C[m][j] = bf16_rne( sum over c of deq(A)[m][c] deq4(B[e(m)])[j][c] )
 *
 * The MoE forward y = x W_e^T with A = MX(x) along K and B[e] = MXFP4(W_e)
 * along K.  Shapes, status codes and accuracy as moe_gg_grouped_mxfp8 (an
 * E2M1 value times its E8M0 scale is exactly a bf16 too, for scale bytes up
 * to 252); the _fast entry point makes one block-scaled MFMA pass with
 * format 4 for B.
 */
MOE_GG_API int moe_gg_grouped_a8w4(const uint8_t *A, const uint8_t *B, uint16_t *C,
                                   const uint8_t *scale_A, const uint8_t *scale_B,
                                   const int32_t *expert_off, int M, int N, int K, int E,
                                   hipStream_t stream);
MOE_GG_API int moe_gg_grouped_a8w4_fast(const uint8_t *A, const uint8_t *B, uint16_t *C,
                                        const uint8_t *scale_A, const uint8_t *scale_B,
                                        const int32_t *expert_off, int M, int N, int K, int E,
                                        hipStream_t stream);

/*
 * MX quantiser: f32 [R][L] -> E4M3 codes [R][L] + E8M0 scales [R][L/32],
 * blocks of 32 consecutive elements along L (aligned to the start of a row).
 *
 * Source: the 8192^3 workload's scale rule scale = 2^(floor(log2(blockmax)) - 8)
 * and the decode page's mx8_scale / mx8_q (scale byte clamped to [1, 254];
 * elements clamped to +-448 before the conversion).
 *
 *   s = clamp(floor(log2(max |X[r][32j..32j+31]|)) - 8 + 127, 1, 254), s = 1 for a zero block
 *   Q[r][i] = e4m3_rne_saturate(X[r][i] * 2^(127 - s)); the sign of zero is kept
 *
 * Inputs must be finite (NaN/Inf give unspecified codes).
 * Shapes: R, L >= 0, L % 32 == 0 (EINVAL otherwise).
 */
MOE_GG_API int moe_gg_mx_quantize(const float *X, uint8_t *Q, uint8_t *S, int R, int L,
                                  hipStream_t stream);

/*
 * Transposing MX quantiser: f32 X [R][L] -> E4M3 codes Q [L][R] + E8M0 scales
 * S [L][R/32], blocks of 32 consecutive elements along R.  With X = g [M][N]
 * (token rows) this yields the weight gradient's A operand g^T [N][M] with
 * one scale per 32 tokens, in one pass over g (the producer step before the
 * tinygrad page's A = g^T layout; same scale rule and rounding as
 * moe_gg_mx_quantize):
 *
 *   Q[l][r] and S[l][r/32] equal moe_gg_mx_quantize's output for the
 *   transpose X^T [L][R].
 *
 * Inputs must be finite.  Shapes: R, L >= 0, R % 32 == 0 (EINVAL
 * otherwise); L % 4 == 0 (EUNSUPPORTED otherwise: the loads are float4).
 */
MOE_GG_API int moe_gg_mx_quantize_t(const float *X, uint8_t *Q, uint8_t *S, int R, int L,
                                    hipStream_t stream);

/*
 * The two quantisers with the round-up scale rule instead of the floor rule.
 *
 * Source: the decode page's mx8_scale ("aiter's MXFP8 RoundUp rule"): the
 * scale is ceil_pow2(max / 448), the quotient formed in f32 as the product
 * of the block max and f32(1/448); the byte is that product's exponent field
 * plus one if its mantissa is nonzero, clamped to [1, 254].
 *
 *   t = f32(max |block| * f32(1/448));  s = clamp(ceil(log2 t) + 127, 1, 254)
 *   (s = 1 for a zero block); codes as above: e4m3_rne_saturate(X * 2^(127 - s))
 *
 * The block max lands in (224, 448] after scaling (448 (1 + 2^-22) at the f32
 * edge, saturated), so no element saturates beyond rounding.  Same layouts,
 * shapes and status codes as moe_gg_mx_quantize / moe_gg_mx_quantize_t.
 */
MOE_GG_API int moe_gg_mx_quantize_roundup(const float *X, uint8_t *Q, uint8_t *S, int R, int L,
                                          hipStream_t stream);
MOE_GG_API int moe_gg_mx_quantize_t_roundup(const float *X, uint8_t *Q, uint8_t *S, int R, int L,
                                            hipStream_t stream);

/*
 * MXFP4 quantiser: f32 [R][L] -> E2M1 codes [R][L/2] (two per byte, element
 * 2i in the low nibble) + E8M0 scales [R][L/32], blocks of 32 along L.
 *
 * Source: the decode page's fp4 weights (format 4 of the f8f6f4 MFMA, one
 * E8M0 scale per 32 along k); the page does not print their quantiser, so
 * this is the MX rule with E2M1's largest exponent, 2, in place of E4M3's 8:
 *
 *   s = clamp(floor(log2(max |X[r][32j..32j+31]|)) - 2 + 127, 1, 254), s = 1 for a zero block
 *   code = e2m1_rne_saturate(X * 2^(127 - s)): nearest of 0, 0.5, 1, 1.5, 2,
 *          3, 4, 6, ties to the even code, +-6 beyond; sign bit kept
 *
 * Inputs must be finite.  Shapes: R, L >= 0, L % 32 == 0 (EINVAL
 * otherwise).
 */
MOE_GG_API int moe_gg_mx4_quantize(const float *X, uint8_t *Q, uint8_t *S, int R, int L,
                                   hipStream_t stream);

/*
 * Transposing MXFP4 quantiser: f32 X [R][L] -> E2M1 codes Q [L][R/2] (two per
 * byte along R, the earlier element in the low nibble) + E8M0 scales
 * S [L][R/32]; the same codes and scales as moe_gg_mx4_quantize of X^T.  With
 * X = W_e [N][K] this gives the MXFP4 B[e] = W_e^T [K][N] along N that makes
 * moe_gg_grouped_a8w4 an MXFP4-weight data gradient dx = g W_e.
 *
 * Inputs must be finite.  Shapes: R, L >= 0, R % 32 == 0 (EINVAL
 * otherwise); L % 4 == 0 (EUNSUPPORTED otherwise).
 */
MOE_GG_API int moe_gg_mx4_quantize_t(const float *X, uint8_t *Q, uint8_t *S, int R, int L,
                                     hipStream_t stream);

/*
 * Row -> expert map, the integer step of the data gradient, exposed so that
 * it can be checked exactly: out[r] = the e with off[e] <= r < off[e+1] for r
 * in [0, M), computed by the same device function the data-gradient kernel
 * uses (source: the oarust page's expert_for_row).
 *
 *   expert_off int32 [E+1] (device), out int32 [M] (device).
 * Shapes: M >= 0, E >= 1 (EINVAL otherwise).
 */
MOE_GG_API int moe_gg_row_experts(const int32_t *expert_off, int E, int M, int32_t *out,
                                  hipStream_t stream);

/* Static, never-NULL description of a status code. */
MOE_GG_API const char *moe_gg_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_GG_H */
