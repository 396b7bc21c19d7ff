/* moe_glue: the memory-bound data path around the expert GEMMs of a
 * Mixture-of-Experts layer, for AMD Instinct MI355X (gfx950).
 *
 *   moe_route        softmax top-k routing, expert histogram, prefix-sum
 *                    offsets and the token <-> expert-row permutation maps
 *   moe_expand_rows  copy each token row to its k expert-contiguous rows
 *   moe_swiglu       gated SiLU on the first grouped GEMM's output
 *   moe_combine      routing-weighted sum of each token's k expert outputs
 *   moe_route_expand route + expand (one launch for small decode batches,
 *                    the copy folded into the route's last launch for
 *                    mid-size ones, destination-order copy for large ones)
 *   moe_route_padded route with expert segments padded to a row multiple
 *   moe_route_expand_padded  moe_route_padded + expand in one call
 *   moe_expand_rows_fp8  expand with FP8 (E4M3) quantisation per column group
 *   moe_expand_rows_mxfp8 expand with MXFP8 quantisation (E8M0 scale per 32 columns)
 *   moe_route_expand_fp8 moe_route_padded + moe_expand_rows_fp8 in one call
 *   moe_route_expand_mxfp8 moe_route_padded + moe_expand_rows_mxfp8 in one call
 *
 * The problem statement these calls follow:
 *   - "CuTeDSL at Perplexity" (Perplexity blog), section "Mixture of Experts
 *     (MoE) dispatch/combine", subsection "Local": dispatch counts the tokens
 *     of each expert from the routing table and gives each token a unique
 *     index inside its expert's list, then copies the tokens into a buffer for
 *     the MoE GEMM; combine accumulates each token's expert outputs in
 *     registers using those positions and writes the final token.
 *   - FlashInfer PR analysis "CUTLASS MoE kernel optimisation: vectorisation
 *     and dynamic thread allocation": expandInputRowsKernel (section 1),
 *     doActivationKernel (sections 1-2) and the 16-byte row alignment
 *     requirement (section 3).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers, row-major and contiguous.
 *     bf16 tensors are passed as uint16_t* holding raw bf16 bit patterns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on that stream and returns without synchronising.
 *   - The caller allocates and owns every buffer, including the route
 *     workspace.  The library never allocates or frees device memory and
 *     keeps no state between calls, so calls on different streams do not
 *     interfere unless their buffers overlap.  (The one exception is
 *     moe_route_expand_noalloc, whose workspace is a built-in device array.)
 *   - Inputs must not alias outputs.
 *   - Argument errors are detected on the host BEFORE any HIP call: the call
 *     returns a non-OK status, records a message (moe_last_error) and
 *     enqueues nothing.  A launch failure returns MOE_ERR_HIP.
 *   - Notation: T tokens, H hidden size, E experts, k experts per token,
 *     I expert intermediate size, R = T*k expanded rows, slot s = t*k + j.
 */
#ifndef MOE_GLUE_H
#define MOE_GLUE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL                          */
    MOE_ERR_SHAPE = 2,       /* a size is negative, zero where it may not be, or k > E */
    MOE_ERR_ALIGN = 3,       /* a bf16 row is not a multiple of 16 bytes, or a
                                pointer is not 16-byte aligned                     */
    MOE_ERR_UNSUPPORTED = 4, /* beyond a limit below (E, k, element counts)         */
    MOE_ERR_WORKSPACE = 5,   /* route workspace missing or too small                */
    MOE_ERR_HIP = 6          /* the HIP runtime reported an error at launch         */
} moe_status;

#define MOE_E_MAX 512        /* experts                                             */
#define MOE_K_MAX 16         /* experts per token                                   */
#define MOE_PAD_MAX 4096     /* row multiple of padded expert segments              */

/* ------------------------------------------------------------------ route */

/* Bytes of device workspace that moe_route, moe_route_padded and
 * moe_route_expand need for (T, E, k); 0 is never returned for valid
 * arguments, and a negative/invalid argument gives 0.  (moe_route and
 * moe_route_padded use only the front part: the per-workgroup expert
 * histograms; moe_route_expand also keeps T*k row-list entries of 8 bytes,
 * or T*k slot ranks of 4 bytes, there.)  The workspace needs no initialisation and may be reused by later
 * calls on the same stream. */
size_t moe_route_workspace_bytes(int32_t T, int32_t E, int32_t k);

/* Softmax top-k routing plus dispatch bookkeeping ("CuTeDSL at Perplexity",
 * MoE dispatch/combine > Local: per-expert token counts and a unique index for
 * each token inside its expert's list).  The pages print no gate function;
 * this call computes, for every token t:
 *   key[e]      = fp32(logits[t,e] + bias[e])   (bias may be NULL: key = logit)
 *   topk_ids[t,j], j = 0..k-1: the experts of the k largest keys, in
 *                 descending key order; equal keys (-0 == +0) go to the lower
 *                 expert index.
 *   topk_weights[t,j] = exp(key_j - key_0) / sum_i exp(key_i - key_0)
 *                 (softmax over the selected keys; fp32).
 * and for the whole batch:
 *   expert_counts[e]  = number of slots s with topk_ids[s] == e   (may be NULL)
 *   expert_offsets[e] = sum of counts of experts below e; expert_offsets[E] = T*k
 *   dest_of_src[s]    = expert_offsets[topk_ids[s]] + number of slots s' < s
 *                       with the same expert (ascending token order inside
 *                       each expert's segment; no padding)
 *   src_of_dest[dest_of_src[s]] = s.
 * Layouts: logits fp32 [T,E]; bias fp32 [E]; topk_ids int32 [T,k];
 * topk_weights fp32 [T,k]; expert_offsets int32 [E+1]; expert_counts int32 [E];
 * dest_of_src, src_of_dest int32 [T*k].  logits and bias need 4-byte alignment.
 * Limits: 1 <= E <= MOE_E_MAX, 1 <= k <= min(E, MOE_K_MAX), T*E < 2^31.
 * T = 0 is valid: offsets (and counts) become all zeros.
 * Logits and bias must be finite (NaN ordering is unspecified).
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE,
 * MOE_ERR_HIP. */
moe_status moe_route(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                     int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                     int32_t* expert_counts, int32_t* dest_of_src, int32_t* src_of_dest,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Padded expert segments.  "CuTeDSL at Perplexity", MoE dispatch/combine >
 * Local: the routed tokens are copied into an optionally padded buffer for the
 * MoE GEMM.  Same as moe_route except that each expert's segment is rounded up
 * to a multiple of pad_to rows (the grouped GEMM's row tile):
 *   expert_offsets[e+1] = expert_offsets[e] + pad_to * ceil(expert_counts[e] / pad_to)
 *   dest_of_src[s]      = expert_offsets[topk_ids[s]] + number of slots s' < s
 *                         with the same expert
 *   src_of_dest[p]      = s if dest_of_src[s] == p, and -1 on padding rows,
 *                         for p < expert_offsets[E].
 * src_of_dest must have room for moe_route_padded_rows(T, E, k, pad_to) =
 * T*k + E*(pad_to-1) entries (the exact count is expert_offsets[E], on the
 * device).  moe_expand_rows and moe_combine work unchanged on the padded
 * layout with buffers of that many rows; expand does not write padding rows.
 * pad_to = 1 is moe_route.  Limits: 1 <= pad_to <= MOE_PAD_MAX and the row
 * bound below 2^31.  Workspace and errors as moe_route. */
size_t moe_route_padded_rows(int32_t T, int32_t E, int32_t k, int32_t pad_to);
moe_status moe_route_padded(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                            int32_t pad_to, int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                            int32_t* expert_counts, int32_t* dest_of_src, int32_t* src_of_dest,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------- expand */

/* expandInputRows (FlashInfer PR analysis, section 1): the copy of each token
 * row into the expert-contiguous buffer the grouped GEMM reads:
 *   x_expanded[dest_of_src[t*k + j], :] = x[t, :]     for j = 0..k-1
 * x bf16 [T,H]; dest_of_src int32 [T*k] (from moe_route with the same T, k);
 * x_expanded bf16 [T*k, H].
 * Alignment (section 3 of the same page): H*2 bytes must be a multiple of 16
 * (H % 8 == 0) and x, x_expanded 16-byte aligned, else MOE_ERR_ALIGN.
 * dest_of_src must be a permutation of [0, T*k) (not checked).
 * T = 0 is a no-op.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN,
 * MOE_ERR_UNSUPPORTED (T*H/8 >= 2^31), MOE_ERR_HIP. */
moe_status moe_expand_rows(const uint16_t* x, const int32_t* dest_of_src, int32_t T, int32_t H,
                           int32_t k, uint16_t* x_expanded, void* stream);

/* FP8 quantising expand.  expandInputRows (FlashInfer PR analysis, section 1)
 * with a quantisation between its load and its store; "CuTeDSL at
 * Perplexity", Blackwell support: FP8 block-wise scaling with absolute maxima
 * over small groups of elements.  For each token t and each group g of
 * `group` consecutive columns:
 *   amax  = max |x[t, c]| over the group
 *   scale = fp32(amax / 448)
 *   inv   = fp32(448 / amax)  (0 when amax = 0)
 *   code  = E4M3(clamp(fp32(x[t, c] * inv), -448, 448)), nearest-even
 * where inv and the product are fp32 roundings without fp32's exponent
 * limits (for amax < 2^-64, x and amax are scaled by 2^64 first, exactly;
 * scale is then an fp32 subnormal)
 * (OCP FP8 E4M3: bias 7, largest finite 448), and every expanded row
 * dest_of_src[t*k + j] receives the token's codes and scales:
 *   x_expanded uint8 [rows, H] codes, scales fp32 [rows, H/group],
 * rows = T*k (or the padded total of moe_route_padded).  Dequantise with
 * code * scale.  group: a power of two in [8, 512] dividing H.
 * Alignment: x 16 bytes, x_expanded 8 bytes, scales 4 bytes; H % 8 == 0.
 * T = 0 is a no-op.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN,
 * MOE_ERR_UNSUPPORTED (group, sizes), MOE_ERR_HIP. */
moe_status moe_expand_rows_fp8(const uint16_t* x, const int32_t* dest_of_src, int32_t T, int32_t H, int32_t k,
                               int32_t group, uint8_t* x_expanded, float* scales, void* stream);

/* moe_expand_rows with MXFP8 quantisation (OCP microscaling).  "CuTeDSL at
 * Perplexity", section "Blackwell support", names MXFP8 among the
 * block-scaled formats and takes its absolute maximum over 32 elements; the
 * scale encoding follows the OCP Microscaling formats definition, which is
 * also the scale format of gfx950's scaled matrix instructions.  For each
 * token t and block b of 32 consecutive columns:
 *   amax = max |x[t, c]| over the block
 *   e    = max(floor(log2 amax) - 8, -127)   (-127 for an all-zero block)
 *   scales[d, b]        = e + 127            (E8M0 byte: the scale is 2^e)
 *   x_expanded[d, c]    = E4M3(clamp(x[t, c] / 2^e, +-448)), nearest-even
 * for every expanded row d = dest_of_src[t*k + j].  The division by a power
 * of two is exact.
 * x [T, H] bf16; x_expanded [rows, H] uint8 E4M3 codes; scales [rows, H/32]
 * uint8 E8M0 bytes.  Rows not named in dest_of_src are not written.
 * H must be a multiple of 32.  Alignment: x 16 bytes, x_expanded 8 bytes.
 * T = 0 is a no-op.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN,
 * MOE_ERR_UNSUPPORTED (sizes), MOE_ERR_HIP. */
moe_status moe_expand_rows_mxfp8(const uint16_t* x, const int32_t* dest_of_src, int32_t T, int32_t H, int32_t k,
                                 uint8_t* x_expanded, uint8_t* scales, void* stream);

/* ------------------------------------------------ route + expand (dispatch) */

/* The whole dispatch: exactly the results of moe_route followed by
 * moe_expand_rows on the same arguments (all outputs of both calls are
 * written).  "CuTeDSL at Perplexity", sections "Grid synchronization" and
 * MoE dispatch/combine > Local, describes dispatch as routing then copying
 * the tokens into the experts' buffer.  For T <= 64 this call uses one launch
 * in which every workgroup recomputes the routing in LDS and copies its share
 * of the rows (the workspace is not touched and may be NULL).  For larger T
 * the route runs as in moe_route; when there are many expanded rows (T*k of
 * about 24576 and up) it also lists them per token group in the workspace
 * and the copy runs in destination-row order from that list, else in token
 * order --
 * on the two-launch route done by its second launch itself, which then keeps
 * the slot ranks in the workspace instead of in dest_of_src.
 * The workspace must hold moe_route_workspace_bytes(T, E, k) bytes (16-byte
 * aligned) whenever T > 64.
 * Layouts, limits, alignment and errors: the union of moe_route's and
 * moe_expand_rows'. */
moe_status moe_route_expand(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                            const uint16_t* x, int32_t H, int32_t* topk_ids, float* topk_weights,
                            int32_t* expert_offsets, int32_t* expert_counts, int32_t* dest_of_src,
                            int32_t* src_of_dest, uint16_t* x_expanded, void* workspace, size_t workspace_bytes,
                            void* stream);

/* moe_route_padded followed by moe_expand_rows, in one call: exactly their
 * results on the same arguments (all outputs of both calls are written;
 * x_expanded has moe_route_padded_rows rows, its padding rows are not
 * written).  As in moe_route_expand: one launch for T <= 64, mid-size
 * batches copy in the route's last launch, large ones in destination-row
 * order from the route's row list.  The workspace must hold
 * moe_route_workspace_bytes(T, E, k) bytes (16-byte aligned) whenever
 * T > 64; for T <= 64 it may be NULL.  Layouts, limits, alignment and errors:
 * the union of moe_route_padded's and moe_expand_rows'. */
moe_status moe_route_expand_padded(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                                   int32_t pad_to, const uint16_t* x, int32_t H, int32_t* topk_ids,
                                   float* topk_weights, int32_t* expert_offsets, int32_t* expert_counts,
                                   int32_t* dest_of_src, int32_t* src_of_dest, uint16_t* x_expanded,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* moe_route_padded followed by moe_expand_rows_fp8, in one call: exactly their
 * results on the same arguments (pad_to = 1: moe_route; all outputs of both
 * calls are written; padding rows of x_expanded and scales are not written).
 * For T <= 64 routing and quantising copy are one launch (as in
 * moe_route_expand).  On the two-launch route with H <= 8192 and at most
 * ~20 MB of codes the quantising copy runs in the route's place launch;
 * otherwise the route is followed by the quantising expand.
 * The workspace must hold moe_route_workspace_bytes(T, E, k) bytes (16-byte
 * aligned) whenever T > 64; for T <= 64 it may be NULL.  Layouts, limits,
 * alignment and errors: the union of moe_route_padded's and
 * moe_expand_rows_fp8's. */
moe_status moe_route_expand_fp8(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                                int32_t pad_to, const uint16_t* x, int32_t H, int32_t group, int32_t* topk_ids,
                                float* topk_weights, int32_t* expert_offsets, int32_t* expert_counts,
                                int32_t* dest_of_src, int32_t* src_of_dest, uint8_t* x_expanded, float* scales,
                                void* workspace, size_t workspace_bytes, void* stream);

/* moe_route_padded followed by moe_expand_rows_mxfp8, in one call, as
 * moe_route_expand_fp8 is for moe_expand_rows_fp8 (same launch choices;
 * padding rows of x_expanded and scales are not written).  scales is
 * [rows, H/32] E8M0 bytes.  The workspace must hold
 * moe_route_workspace_bytes(T, E, k) bytes (16-byte aligned) whenever T > 64;
 * for T <= 64 it may be NULL.  Layouts, limits, alignment and errors: the
 * union of moe_route_padded's and moe_expand_rows_mxfp8's. */
moe_status moe_route_expand_mxfp8(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                                  int32_t pad_to, const uint16_t* x, int32_t H, int32_t* topk_ids,
                                  float* topk_weights, int32_t* expert_offsets, int32_t* expert_counts,
                                  int32_t* dest_of_src, int32_t* src_of_dest, uint8_t* x_expanded, uint8_t* scales,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* moe_route_expand for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results, launches and errors as
 * moe_route_expand, without the workspace: the library keeps one built-in
 * device scratch array of MOE_NOALLOC_SCRATCH_BYTES per GPU (it exists on
 * each GPU the library runs on until the process ends; its device address is
 * looked up on the first call on each device).  The call allocates nothing.
 * Calls whose moe_route_workspace_bytes(T, E, k) exceeds the scratch return
 * MOE_ERR_UNSUPPORTED before any HIP call.  Every call on one GPU shares that
 * GPU's scratch: calls that can overlap on the device (on different streams,
 * or captured into graphs that run concurrently) race and give wrong results;
 * calls on one stream are safe.  The scratch needs no clearing between calls
 * (the route reads only what the same call wrote). */
#define MOE_NOALLOC_SCRATCH_BYTES (4u << 20)
size_t moe_noalloc_scratch_bytes(void);
moe_status moe_route_expand_noalloc(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                                    const uint16_t* x, int32_t H, int32_t* topk_ids, float* topk_weights,
                                    int32_t* expert_offsets, int32_t* expert_counts, int32_t* dest_of_src,
                                    int32_t* src_of_dest, uint16_t* x_expanded, void* stream);

/* ----------------------------------------------------------------- SwiGLU */

/* doActivation (FlashInfer PR analysis, sections 1-2): gated SiLU on the first
 * grouped GEMM's output, row by row:
 *   act[r, i] = bf16( silu(g) * u ),  g = h[r, i], u = h[r, I + i],
 *   silu(g) = g / (1 + exp(-g)), computed in fp32, rounded to nearest even.
 * h bf16 [R, 2I] (gate columns 0..I-1, up columns I..2I-1); act bf16 [R, I].
 * I % 8 == 0 and h, act 16-byte aligned, else MOE_ERR_ALIGN.
 * R = 0 is a no-op.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN,
 * MOE_ERR_UNSUPPORTED (R*I/8 >= 2^31), MOE_ERR_HIP. */
moe_status moe_swiglu(const uint16_t* h, int32_t R, int32_t I, uint16_t* act, void* stream);

/* ---------------------------------------------------------------- combine */

/* Combine ("CuTeDSL at Perplexity", MoE dispatch/combine, opening paragraph
 * and "Local": weighted accumulation in registers using dispatch's positions):
 *   out[t, :] = bf16( sum_{j=0..k-1} topk_weights[t,j] * y[dest_of_src[t*k+j], :] )
 * accumulated in fp32 in j order, rounded once to nearest even.
 * y bf16 [T*k, H]; topk_weights fp32 [T,k]; dest_of_src int32 [T*k];
 * out bf16 [T, H].  H % 8 == 0 and y, out 16-byte aligned, else MOE_ERR_ALIGN.
 * dest_of_src entries must be rows of y (not checked): in [0, T*k) for the
 * layout of moe_route, in [0, expert_offsets[E]) -- at most
 * moe_route_padded_rows(T, E, k, pad_to) -- for that of moe_route_padded,
 * whose padding rows combine never reads.
 * T = 0 is a no-op.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN,
 * MOE_ERR_UNSUPPORTED (T*H/8 >= 2^31), MOE_ERR_HIP. */
moe_status moe_combine(const uint16_t* y, const float* topk_weights, const int32_t* dest_of_src,
                       int32_t T, int32_t H, int32_t k, uint16_t* out, void* stream);

/* -------------------------------------------------------------- utilities */

/* Plain streaming copy of `bytes` bytes (a multiple of 16; both pointers
 * 16-byte aligned), 16 bytes per lane.  It is the measuring stick for
 * achievable HBM bandwidth and for calibrating traffic counters; it is not
 * part of the MoE path.  Errors: MOE_ERR_NULL, MOE_ERR_ALIGN, MOE_ERR_HIP. */
moe_status moe_copy_probe(const void* src, void* dst, size_t bytes, void* stream);

/* Streaming probe with a read:write mix: `cycles` cycles of reads + writes
 * waves (64 lanes each, `threads` lanes per workgroup: 64, 256 or 1024); in
 * each cycle the first `reads` waves each load vectors_per_lane (1, 2 or 4)
 * KiB of src and the others each store as many KiB to dst, every access of
 * a wave one contiguous KiB, no store depending on a load.  src must hold
 * cycles * reads * vectors_per_lane KiB and dst cycles * writes *
 * vectors_per_lane KiB (+ 1 KiB when writes = 0); device pointers, 16-byte
 * aligned, owned by the caller; src may be NULL when reads = 0, dst never.  It measures
 * what HBM gives a stream with a path kernel's mix of reads and writes; it
 * is not part of the MoE path.  reads, writes <= 64, cycles * (reads +
 * writes) <= 2^24; cycles = 0 or reads = writes = 0 is a no-op.  Errors:
 * MOE_ERR_NULL, MOE_ERR_ALIGN, MOE_ERR_SHAPE, MOE_ERR_HIP. */
moe_status moe_mix_probe(const void* src, void* dst, uint32_t cycles, uint32_t reads, uint32_t writes,
                         int32_t vectors_per_lane, int32_t threads, void* stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status s);

/* Detail text for the last non-OK status returned on the calling thread
 * ("" if none).  Valid until the next call on the same thread. */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_GLUE_H */
