/* CPU oracle for the MoE glue path (route -> expand -> SwiGLU -> combine).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code, header, table or helper with the HIP library, and the HIP library never
 * calls it: it exists to say what the right answer is, slowly and plainly.
 *
 * All pointers are host pointers; bf16 values are raw 16-bit patterns.
 * Row-major, contiguous layouts throughout.  Notation: T tokens, H hidden size,
 * E experts, k experts per token, I expert intermediate size, R = T*k expanded
 * rows, slot s = t*k + j.
 *
 * Sources (see moe_oracle.c for the per-function passages):
 *   "CuTeDSL at Perplexity", section "Mixture of Experts (MoE) dispatch/combine",
 *     subsection "Local": per-expert token counts, a unique index for each token
 *     inside its expert's list, the copy into an expert-contiguous buffer and
 *     the weighted accumulation back to token order.
 *   FlashInfer PR analysis "CUTLASS MoE kernel optimisation: vectorisation and
 *     dynamic thread allocation", section 1: expandInputRowsKernel (row copy)
 *     and doActivationKernel (activation on the first GEMM's output).
 *
 * Parity status: every function here is pinned by tests other than itself
 * (brute force on tiny inputs, closed forms, invariants, planted mutants).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Softmax top-k routing, histogram, prefix-sum offsets and permutation maps.
 * logits [T,E] fp32, bias [E] fp32 or NULL.
 * Outputs: topk_ids [T,k], topk_weights [T,k], expert_offsets [E+1],
 * expert_counts [E], dest_of_src [R], src_of_dest [R].
 * Returns 0, or -1 if 1 <= k <= E does not hold or T < 0. */
int moe_ref_route(const float* logits, const float* bias, int T, int E, int k,
                  int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                  int32_t* expert_counts, int32_t* dest_of_src, int32_t* src_of_dest);

/* As moe_ref_route, with each expert's segment padded to a multiple of
 * pad_to rows: expert_offsets are padded, dest_of_src points into the padded
 * layout and src_of_dest (expert_offsets[E] entries, at most
 * T*k + E*(pad_to-1)) holds -1 on padding rows.  Returns 0, or -1 on bad sizes. */
int moe_ref_route_padded(const float* logits, const float* bias, int T, int E, int k, int pad_to,
                         int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                         int32_t* expert_counts, int32_t* dest_of_src, int32_t* src_of_dest);

/* x_exp[dest_of_src[t*k+j], :] = x[t, :] ; x [T,H], x_exp [T*k,H] (bf16 bits). */
void moe_ref_expand_rows(const uint16_t* x, const int32_t* dest_of_src, int T, int H, int k,
                         uint16_t* x_exp);

/* FP8 quantising expand: per token and group of `group` columns, scale =
 * fp32(amax/448), codes = e4m3(fp32(x * fp32(448/amax))) saturating, the two
 * fp32 roundings taken without exponent limits (x and amax scaled by 2^64
 * when amax < 2^-64); codes and scales written to every expanded row of the
 * token.
 * q_out [rows, H] uint8 codes, scales [rows, H/group] fp32. */
void moe_ref_expand_rows_fp8(const uint16_t* x, const int32_t* dest_of_src, int T, int H, int k, int group,
                             uint8_t* q_out, float* scales);

/* MXFP8 quantising expand: per token and block of 32 columns, e =
 * max(floor(log2 amax) - 8, -127) (-127 for an all-zero block), scale byte
 * (E8M0) = e + 127, codes = e4m3(x / 2^e) saturating; codes and scale bytes
 * written to every expanded row of the token.  H must be a multiple of 32.
 * q_out [rows, H] uint8 codes, scales [rows, H/32] uint8. */
void moe_ref_expand_rows_mxfp8(const uint16_t* x, const int32_t* dest_of_src, int T, int H, int k,
                               uint8_t* q_out, uint8_t* scales);

/* The oracle's FP8 E4M3 (OCP, bias 7, max 448) conversions, exported for pinning. */
uint8_t moe_ref_e4m3_from_f32(float v);
double moe_ref_f64_from_e4m3(uint8_t c);

/* act[r,i] = bf16( silu(h[r,i]) * h[r,I+i] ), computed in fp64, rounded once. */
void moe_ref_swiglu(const uint16_t* h, int R, int I, uint16_t* act);

/* out[t,:] = bf16( sum_j w[t,j] * y[dest_of_src[t*k+j], :] ), fp64 sum, rounded once. */
void moe_ref_combine(const uint16_t* y, const float* topk_weights, const int32_t* dest_of_src,
                     int T, int H, int k, uint16_t* out);

/* The oracle's own bf16 conversions (exported so tests can pin them). */
uint16_t moe_ref_bf16_from_f64(double v);
double moe_ref_f64_from_bf16(uint16_t b);
/* Vector form of moe_ref_bf16_from_f64 for tests. */
void moe_ref_bf16_from_f64_n(const double* v, int64_t n, uint16_t* out);

#ifdef __cplusplus
}
#endif
#endif /* MOE_ORACLE_H */
