/* CPU oracle for the MoE glue path.  TEST INFRASTRUCTURE ONLY: see moe_oracle.h
 * for who may call it.  Plain, single-threaded, scalar C; fp64 arithmetic; one
 * rounding to the output type at the end of each computed value.
 *
 * Readings taken where the pages leave a step open (they print no gate
 * function, no tie rule and no order inside an expert's list):
 *   - gate: softmax over the selected k keys (softmax over all E, restricted
 *     to the top k and renormalised, is the same thing);
 *   - selection is on key = fp32(logit + bias), the k largest keys, equal keys
 *     broken toward the lower expert index; slots in descending key order;
 *   - inside an expert's list, rows are in ascending source slot order
 *     (ascending token, since a token never picks an expert twice);
 *   - segments are not padded (expert_offsets[E] = T*k), except in
 *     moe_ref_route_padded, which rounds each segment up to a multiple of
 *     pad_to rows and marks the extra rows -1 in src_of_dest;
 *   - SwiGLU gate is the first I columns of the first GEMM's output, up the
 *     last I; act = silu(gate) * up with silu(g) = g / (1 + exp(-g));
 *   - every conversion to bf16 rounds to nearest, ties to even.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ bf16 */

double moe_ref_f64_from_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 (ties to even) in one step.
 * bf16 keeps 8 significant bits and the fp32 exponent range, so the rounding
 * quantum of a normal value a in [2^(e-1), 2^e) is 2^(e-8); below 2^-126 the
 * quantum is fixed at 2^-133 (bf16 subnormals).  nearbyint() rounds to the
 * nearest integer with ties to even in the default rounding mode.  A rounded
 * magnitude of 2^128 or more is out of range and becomes infinity. */
uint16_t moe_ref_bf16_from_f64(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);               /* a = m * 2^e, m in [0.5, 1) */
    int q = e - 8;
    if (q < -133) q = -133;
    double r = ldexp(nearbyint(ldexp(a, -q)), q);
    if (r >= 0x1p128) return sign | 0x7F80;
    float f = (float)r;               /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

void moe_ref_bf16_from_f64_n(const double* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = moe_ref_bf16_from_f64(v[i]);
}

/* ----------------------------------------------------------------- route */

typedef struct {
    float key;
    int expert;
} keyed_expert;

/* Total order: larger key first; equal keys (as IEEE values, so -0 == +0)
 * put the lower expert index first. */
static int by_key_desc_then_expert(const void* pa, const void* pb) {
    const keyed_expert* a = (const keyed_expert*)pa;
    const keyed_expert* b = (const keyed_expert*)pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    return (a->expert > b->expert) - (a->expert < b->expert);
}

/* "CuTeDSL at Perplexity", MoE dispatch/combine > Local: the dispatch step
 * reads the routing table, counts the tokens of each expert and gives every
 * token a unique index inside its expert's list.  Here:
 *   key[t,e]   = fp32(logit[t,e] + bias[e])      (bias optional)
 *   ids[t,:]   = the k largest keys, ties to the lower e, descending
 *   w[t,j]     = exp(key_j - key_0) / sum_i exp(key_i - key_0)   (fp64 -> fp32)
 *   counts[e]  = number of slots that picked e
 *   offsets    = exclusive prefix sum of counts, offsets[E] = T*k
 *   dest[s]    = offsets[ids[s]] + number of earlier slots with the same expert
 *   src[dest[s]] = s                                                          */
int moe_ref_route(const float* logits, const float* bias, int T, int E, int k,
                  int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                  int32_t* expert_counts, int32_t* dest_of_src, int32_t* src_of_dest) {
    if (T < 0 || E < 1 || k < 1 || k > E) return -1;
    keyed_expert* row = (keyed_expert*)malloc(sizeof(keyed_expert) * (size_t)E);
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    if (!row || !cursor) {
        free(row);
        free(cursor);
        return -2;
    }

    /* top-k selection and weights, token by token */
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            float key = logits[(size_t)t * E + e];
            if (bias) key = key + bias[e];
            row[e].key = key;
            row[e].expert = e;
        }
        qsort(row, (size_t)E, sizeof(keyed_expert), by_key_desc_then_expert);
        double top = (double)row[0].key;
        double denom = 0.0;
        for (int j = 0; j < k; ++j) denom += exp((double)row[j].key - top);
        for (int j = 0; j < k; ++j) {
            topk_ids[(size_t)t * k + j] = row[j].expert;
            topk_weights[(size_t)t * k + j] = (float)(exp((double)row[j].key - top) / denom);
        }
    }

    /* histogram */
    const int64_t R = (int64_t)T * k;
    for (int e = 0; e < E; ++e) expert_counts[e] = 0;
    for (int64_t s = 0; s < R; ++s) expert_counts[topk_ids[s]] += 1;

    /* exclusive prefix sum */
    expert_offsets[0] = 0;
    for (int e = 0; e < E; ++e) expert_offsets[e + 1] = expert_offsets[e] + expert_counts[e];

    /* stable placement: one pass over slots in ascending order */
    for (int e = 0; e < E; ++e) cursor[e] = expert_offsets[e];
    for (int64_t s = 0; s < R; ++s) {
        int e = topk_ids[s];
        dest_of_src[s] = cursor[e];
        cursor[e] += 1;
    }
    for (int64_t s = 0; s < R; ++s) src_of_dest[dest_of_src[s]] = (int32_t)s;

    free(row);
    free(cursor);
    return 0;
}

/* Padded expert segments.  "CuTeDSL at Perplexity", MoE dispatch/combine >
 * Local: after routing, tokens are copied into an optionally padded buffer
 * for the MoE GEMM.  Reading: each expert's segment is rounded up to a
 * multiple of pad_to rows (the grouped GEMM's row tile), the extra rows are
 * padding that no token maps to:
 *   offsets[e+1] = offsets[e] + pad_to * ceil(counts[e] / pad_to)
 *   dest[s]      = offsets[ids[s]] + number of earlier slots with the same expert
 *   src[p]       = s where dest[s] = p, and -1 on padding rows, p < offsets[E]
 * ids, weights and counts are those of moe_ref_route.  pad_to = 1 is the
 * unpadded layout. */
int moe_ref_route_padded(const float* logits, const float* bias, int T, int E, int k, int pad_to,
                         int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                         int32_t* expert_counts, int32_t* dest_of_src, int32_t* src_of_dest) {
    if (pad_to < 1) return -1;
    const int64_t R = (int64_t)T * k;
    int32_t* plain_offsets = (int32_t*)malloc(sizeof(int32_t) * ((size_t)E + 1));
    int32_t* plain_src = (int32_t*)malloc(sizeof(int32_t) * (size_t)(R > 0 ? R : 1));
    int32_t* next_row = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    if (!plain_offsets || !plain_src || !next_row) {
        free(plain_offsets);
        free(plain_src);
        free(next_row);
        return -2;
    }
    int rc = moe_ref_route(logits, bias, T, E, k, topk_ids, topk_weights, plain_offsets, expert_counts,
                           dest_of_src, plain_src);
    if (rc == 0) {
        expert_offsets[0] = 0;
        for (int e = 0; e < E; ++e) {
            const int64_t padded = (int64_t)pad_to * ((expert_counts[e] + pad_to - 1) / pad_to);
            expert_offsets[e + 1] = (int32_t)(expert_offsets[e] + padded);
        }
        for (int e = 0; e < E; ++e) next_row[e] = expert_offsets[e];
        for (int64_t slot = 0; slot < R; ++slot) dest_of_src[slot] = next_row[topk_ids[slot]]++;
        for (int64_t p = 0; p < expert_offsets[E]; ++p) src_of_dest[p] = -1;
        for (int64_t slot = 0; slot < R; ++slot) src_of_dest[dest_of_src[slot]] = (int32_t)slot;
    }
    free(plain_offsets);
    free(plain_src);
    free(next_row);
    return rc;
}

/* ---------------------------------------------------------------- expand */

/* FlashInfer PR analysis, section 1 (expandInputRowsKernel): each source token
 * row is copied unchanged to its expanded rows.  With the placement above the
 * copy of token t for its j-th expert lands in row dest_of_src[t*k + j]. */
void moe_ref_expand_rows(const uint16_t* x, const int32_t* dest_of_src, int T, int H, int k,
                         uint16_t* x_exp) {
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int64_t d = dest_of_src[(size_t)t * k + j];
            for (int c = 0; c < H; ++c) x_exp[(size_t)d * H + c] = x[(size_t)t * H + c];
        }
    }
}

/* ------------------------------------------------------ FP8 quantising expand */

/* Round an fp32 value to FP8 E4M3 (OCP "e4m3fn": 1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, largest finite 448, no infinities), nearest with
 * ties to even, saturating: magnitudes beyond 448 become 448.  Normal values
 * keep 4 significant bits, so the quantum of a in [2^(e-1), 2^e) is 2^(e-4);
 * below 2^-6 (subnormals) the quantum is 2^-9.  Returns the 8-bit code. */
uint8_t moe_ref_e4m3_from_f32(float v) {
    if (isnan(v)) return 0x7F;
    const uint8_t sgn = signbit(v) ? 0x80 : 0x00;
    double mag = fabs((double)v);
    if (mag > 448.0) mag = 448.0;
    if (mag == 0.0) return sgn;
    int ex;
    (void)frexp(mag, &ex);
    const int qe = ex - 4 < -9 ? -9 : ex - 4;                        /* quantum exponent */
    const double rounded = ldexp(nearbyint(ldexp(mag, -qe)), qe);
    if (rounded == 0.0) return sgn;
    if (rounded < 0x1p-6) return sgn | (uint8_t)(rounded / 0x1p-9);  /* subnormal: m * 2^-9 */
    int re;
    const double frac = frexp(rounded, &re);                         /* rounded = frac * 2^re, frac in [0.5, 1) */
    const int mant = (int)((2.0 * frac - 1.0) * 8.0);                /* exact: 3 fraction bits */
    return sgn | (uint8_t)(((re - 1 + 7) << 3) | mant);
}

double moe_ref_f64_from_e4m3(uint8_t c) {
    int ex = (c >> 3) & 0xF, m = c & 0x7;
    double mag = ex == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, ex - 7);
    if (ex == 0xF && m == 0x7) mag = NAN;
    return (c & 0x80) ? -mag : mag;
}

/* Quantising expand.  "CuTeDSL at Perplexity", Blackwell support: kernels
 * were adapted for FP8 blockwise scaling, with absolute maxima over small
 * groups of elements; FlashInfer PR analysis, section 1: expandInputRows
 * applies an operation between its load and its store.  Reading: for each
 * token t and group g of `group` consecutive columns,
 *   amax  = max |x[t, c]| over the group
 *   scale = fp32(amax / 448)
 *   inv   = fp32(448 / amax)   (0 when amax = 0)
 *   q[c]  = e4m3(fp32(x[t, c] * inv))   saturating, nearest-even
 * and every expanded row dest_of_src[t*k + j] receives the token's codes
 * (q_out [rows, H]) and scales (scales [rows, H/group]).  The divisions and
 * the product are single fp32 operations, the precision the kernel decides in,
 * taken without fp32's exponent limits: for amax below 2^-64, 448/amax would
 * overflow, so x and amax are first multiplied by 2^64 (exact for such small
 * values), which gives the significands an unlimited exponent range would. */
void moe_ref_expand_rows_fp8(const uint16_t* x, const int32_t* dest_of_src, int T, int H, int k, int group,
                             uint8_t* q_out, float* scales) {
    const int G = H / group;
    for (int t = 0; t < T; ++t) {
        for (int g = 0; g < G; ++g) {
            float amax = 0.0f;
            for (int c = g * group; c < (g + 1) * group; ++c) {
                float v = fabsf((float)moe_ref_f64_from_bf16(x[(size_t)t * H + c]));
                if (v > amax) amax = v;
            }
            const float scale = amax / 448.0f;
            const float pre = amax < 0x1p-64f ? 0x1p64f : 1.0f;
            const float inv = amax > 0.0f ? 448.0f / (amax * pre) : 0.0f;
            for (int j = 0; j < k; ++j) {
                const int64_t dst_row = dest_of_src[(size_t)t * k + j];
                scales[(size_t)dst_row * G + g] = scale;
                for (int c = g * group; c < (g + 1) * group; ++c) {
                    const float xv = (float)moe_ref_f64_from_bf16(x[(size_t)t * H + c]) * pre;
                    q_out[(size_t)dst_row * H + c] = moe_ref_e4m3_from_f32(xv * inv);
                }
            }
        }
    }
}

/* MXFP8 quantising expand.  "CuTeDSL at Perplexity", Blackwell support,
 * names MXFP8 among the block-scaled formats and takes its absolute maximum
 * over 32 elements.  How the block scale is encoded is not on the pages;
 * reading (the OCP Microscaling formats definition): for each token t and
 * block b of 32 consecutive columns,
 *   amax = max |x[t, c]| over the block
 *   e    = floor(log2 amax) - 8, at least -127 (8 is the exponent of E4M3's
 *          largest normal, 448 = 1.75 * 2^8); e = -127 when amax = 0
 *   scale byte (E8M0) = e + 127, the value 2^e
 *   q[c] = e4m3(x[t, c] / 2^e)   saturating, nearest-even (the division by a
 *          power of two is exact)
 * and every expanded row dest_of_src[t*k + j] receives the token's codes
 * (q_out [rows, H]) and scale bytes (scales [rows, H/32]). */
void moe_ref_expand_rows_mxfp8(const uint16_t* x, const int32_t* dest_of_src, int T, int H, int k,
                               uint8_t* q_out, uint8_t* scales) {
    const int B = H / 32;
    for (int t = 0; t < T; ++t) {
        for (int b = 0; b < B; ++b) {
            double amax = 0.0;
            for (int c = b * 32; c < (b + 1) * 32; ++c) {
                const double v = fabs(moe_ref_f64_from_bf16(x[(size_t)t * H + c]));
                if (v > amax) amax = v;
            }
            int e = -127;
            if (amax > 0.0) {
                int ex;
                (void)frexp(amax, &ex);  /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
                e = ex - 1 - 8;
                if (e < -127) e = -127;
            }
            for (int j = 0; j < k; ++j) {
                const int64_t dst_row = dest_of_src[(size_t)t * k + j];
                scales[(size_t)dst_row * B + b] = (uint8_t)(e + 127);
                for (int c = b * 32; c < (b + 1) * 32; ++c) {
                    const double xv = moe_ref_f64_from_bf16(x[(size_t)t * H + c]);
                    q_out[(size_t)dst_row * H + c] = moe_ref_e4m3_from_f32((float)ldexp(xv, -e));
                }
            }
        }
    }
}

/* ---------------------------------------------------------------- SwiGLU */

/* FlashInfer PR analysis, sections 1-2 (doActivationKernel): the activation
 * applied row by row to the first grouped GEMM's output before the second
 * GEMM.  Gated SiLU: gate g = h[r, i], up u = h[r, I + i]. */
void moe_ref_swiglu(const uint16_t* h, int R, int I, uint16_t* act) {
    for (int64_t r = 0; r < R; ++r) {
        for (int i = 0; i < I; ++i) {
            double g = moe_ref_f64_from_bf16(h[(size_t)r * 2 * I + i]);
            double u = moe_ref_f64_from_bf16(h[(size_t)r * 2 * I + I + i]);
            double silu = g / (1.0 + exp(-g));
            act[(size_t)r * I + i] = moe_ref_bf16_from_f64(silu * u);
        }
    }
}

/* --------------------------------------------------------------- combine */

/* "CuTeDSL at Perplexity", MoE dispatch/combine (opening paragraph and
 * "Local"): after the expert GEMMs, each token's k expert outputs are
 * accumulated with its routing weights, using the positions dispatch
 * computed, and the final token is written to the output buffer. */
void moe_ref_combine(const uint16_t* y, const float* topk_weights, const int32_t* dest_of_src,
                     int T, int H, int k, uint16_t* out) {
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                int64_t row = dest_of_src[(size_t)t * k + j];
                double w = (double)topk_weights[(size_t)t * k + j];
                acc += w * moe_ref_f64_from_bf16(y[(size_t)row * H + c]);
            }
            out[(size_t)t * H + c] = moe_ref_bf16_from_f64(acc);
        }
    }
}
