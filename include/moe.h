/*
 * moe.h -- C ABI of the MI355X (gfx950) DeepSeek-V3/R1-style MoE expert layer.
 *
 * One GPU's share of a mixture-of-experts layer: every token is gated to its
 * top-k routed experts plus one shared expert; the token copies are expanded
 * and sorted by expert, the per-expert SwiGLU FFNs run as one ragged grouped
 * GEMM, and the rows are un-permuted and combined with the top-k weights plus
 * the shared-expert output.
 *
 * Sources, cited by short name:
 *   [MND] page "Lower latency and higher throughput with multi-node DeepSeek
 *         deployment" (Perplexity, 2025-04-18).
 *   [R1P] page "CANN/cann-recipes-infer: DeepSeek-R1 prefill optimization"
 *         (DeepSeek-R1 prefill on Atlas A3).
 *   [V32] page "NPU DeepSeek-V3.2-Exp inference optimization practice".
 *
 * Conventions shared by every call
 *   - Tensor pointers are DEVICE pointers, row-major, 16-byte aligned (a non-null
 *     pointer that is not is MOE_EINVAL: the kernels move 16-byte vectors).  The
 *     caller allocates and owns every buffer and the workspace; the library
 *     allocates nothing, frees nothing and keeps no state between calls.
 *   - Every call only enqueues work on `stream`; none synchronizes or reads
 *     device memory on the host (routing counts stay on the device, so a call
 *     sequence can be captured in a HIP graph).  moe_get_error() is the one
 *     call that synchronizes.
 *   - bf16 is passed as raw 16-bit patterns, fp8 as OCP E4M3FN bytes
 *     (max 448), indices as int32.  Weights are [out, in] (the reduction
 *     dimension is contiguous), as both matrix-core operands want them.
 *   - Host-side validation failures return a negative moe_status at once and
 *     enqueue nothing.  A failed kernel launch returns MOE_EHIP.  Bad data found
 *     on the device (an expert id outside [e_base, e_base + E)) is recorded in
 *     the workspace and reported by moe_get_error().
 *   - Calls are reentrant: concurrent calls are fine on different streams with
 *     different workspaces.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* null pointer, bad size, k > E, ... */
  MOE_EUNSUPPORTED = -2,  /* dtype combination or size the kernels do not cover */
  MOE_EWORKSPACE = -3,    /* workspace smaller than the size query returned */
  MOE_EHIP = -4,          /* a HIP launch or runtime call failed */
  MOE_EDEVICE = -5        /* device-detected bad input (see moe_get_error) */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2, MOE_INT8 = 3, MOE_INT4 = 4 } moe_dtype;

/* Problem shape of one call.
 *   T        tokens (for re-routing: received rows)
 *   H        hidden size; a multiple of 128 for bf16/fp8, of 4 for fp32
 *   E        routed experts held by this call (the local experts)
 *   k        routed experts per token, 1 <= k <= E (1 for re-routing)
 *   I        routed SwiGLU intermediate size (multiple of 128 for bf16/fp8)
 *   I_shared shared-expert intermediate size (multiple of 128 for bf16/fp8)
 *   act      activation dtype: MOE_F32 or MOE_BF16
 *   wt       expert-weight dtype: MOE_F32 (with act F32), MOE_BF16 (with act
 *            BF16), MOE_FP8_E4M3 (with act BF16; the expert inputs are then
 *            quantized to fp8 with one fp32 scale per 1x128 vector) or
 *            MOE_INT8 (with act BF16: W8A8, [V32 §quantization strategy]; int8
 *            weights with one fp32 scale per output channel, the expert inputs
 *            and h quantized to int8 with one fp32 scale per row: scale =
 *            amax/127, code = round-half-even(x * 127/amax)) or MOE_INT4
 *            (with act BF16: W4A8; 4-bit two's-complement weight codes with
 *            one fp32 scale per output channel, packed two per byte: per 16
 *            elements of K, byte i holds element i in its low nibble and
 *            element 8 + i in its high nibble, so a weight row of K codes is
 *            K/2 bytes; activations as MOE_INT8)                             */
typedef struct {
  int32_t T, H, E, k, I, I_shared;
  int32_t act, wt;
} moe_shape;

/* Workspace bytes needed by moe_layer and moe_init_routing for shape `s`
 * (0 if the shape is invalid). */
size_t moe_workspace_bytes(const moe_shape* s);

/* Workspace bytes needed by moe_grouped_ffn for G groups (1 .. 1024) and at most R_max
 * rows (0 if the arguments are invalid). */
size_t moe_grouped_ffn_workspace_bytes(const moe_shape* s, int32_t G, int32_t R_max);

/* How moe_layer runs shape `s`: a host-side description of its launch plan, for callers
 * that account work per launch (no device work, no allocation).  The routed experts'
 * GEMMs split their reduction into ffn1_splits / ffn2_splits slices (fp32 partials added
 * by a reduction launch; 1 = no split) only when their grid would leave half the CUs
 * idle ([MND §Quantization]: split-K for small batches).
 *   shared_merged  1: the shared expert is one more group of the routed expert launches
 *   rows_gathered  1: the first expert GEMM reads x through the sort (no expanded copy)
 *   block_m        rows per unit of the routed expert GEMMs
 *   ffn2_tiles_per_wg  output tiles each workgroup of the down projection computes
 *                  one after another (1 for the decode tiles and fp8)
 * Returns MOE_EINVAL / MOE_EUNSUPPORTED for the shapes moe_layer rejects.           */
typedef struct {
  int32_t shared_merged, rows_gathered, ffn1_splits, ffn2_splits, block_m, ffn2_tiles_per_wg;
} moe_layer_plan;
moe_status moe_layer_plan_of(const moe_shape* s, moe_layer_plan* out);

/* Gate and top-k router.  [MND §Expert Parallelism]: each token is sent to k
 * different routed experts whose outputs are weighted-summed; [MND §MoE Router]:
 * a sort that tracks indices yields the top-k expert ids and scores per token.
 *   x       [T, H]  act           tokens
 *   w_gate  [E, H]  act           gate matrix
 *   bias    [E]     fp32 or NULL  added to the logits: z = logit + bias
 *   logits  [T, E]  fp32 or NULL  OUT: x . w_gate^T (fp32 accumulate); NULL: kept in
 *                                 the workspace only
 *   topk_idx[T, k]  int32         OUT: the k largest z, descending; equal z -> lower id
 *   topk_w  [T, k]  fp32          OUT: sigmoid(z) of the selected, renormalized to sum 1
 *   ws      workspace of moe_workspace_bytes(s) bytes                          */
moe_status moe_gate_topk(const moe_shape* s, const void* x, const void* w_gate,
                         const float* bias, float* logits, int32_t* topk_idx,
                         float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream);

/* Router variants.  [MND §MoE Router]: one router serves every MoE model, the
 * ungrouped (Mixtral-style) routing being the case in which the top-K group is
 * every expert.  Experts form n_group groups of E / n_group consecutive ids; a
 * group's score is the sum of its group_topn largest z (added in fp32); the
 * topk_group best groups are kept (equal scores -> lower group id); the k best z
 * of the kept groups' experts are selected (equal z -> lower id).  Weights: the
 * selected sigmoid(z) (MOE_SCORE_SIGMOID) or softmax(z) over all E experts taken
 * at the selected (MOE_SCORE_SOFTMAX); divided by their sum if renormalize; times
 * scale.  z = logit + bias throughout.  A NULL router means {SIGMOID, 1, 1, 1, 1,
 * 1.0f}, the plain router of moe_gate_topk.  Valid: scoring 0 or 1, renormalize 0
 * or 1, 1 <= n_group <= 64 dividing E, 1 <= topk_group <= n_group, group_topn 1 or
 * 2 and at most E / n_group, k <= topk_group * E / n_group, scale finite and > 0;
 * anything else is MOE_EINVAL.                                                     */
typedef enum { MOE_SCORE_SIGMOID = 0, MOE_SCORE_SOFTMAX = 1 } moe_scoring;
typedef struct {
  int32_t scoring;      /* moe_scoring                                              */
  int32_t renormalize;  /* 1: the k weights are divided by their sum                */
  int32_t n_group;      /* expert groups; 1 = no grouping                           */
  int32_t topk_group;   /* groups kept per token                                    */
  int32_t group_topn;   /* a group scores the sum of its group_topn best z (1 or 2) */
  float scale;          /* routed scaling factor applied to the weights             */
} moe_router;

/* moe_gate_topk with a router variant (NULL router: moe_gate_topk). */
moe_status moe_gate_topk_ex(const moe_shape* s, const moe_router* router, const void* x,
                            const void* w_gate, const float* bias, float* logits,
                            int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* Expand-and-sort routing.  [R1P §MoE deployment strategy optimization]:
 * init-routing expands every token once per chosen expert and sorts the copies
 * by expert, giving expanded_x, tokens_per_expert and expanded_row_idx (the
 * map that later restores token order); re-routing is the same sort with k = 1
 * over received, unordered rows.
 *   x                 [T, H] act     tokens (or received rows); may be NULL when
 *                                    expanded_x is NULL (routing only)
 *   ids               [T, k] int32   global expert ids; local id = id - e_base
 *   expanded_x        [T*k, H]       OUT or NULL: row r = x[sorted_src[r] / k];
 *                                    act dtype, or fp8 / int8 codes when s->wt
 *                                    is fp8 / int8 or int4
 *   expanded_scale    OUT fp32: [T*k, H/128] 1x128 scales (fp8), [T*k] row
 *                                    scales (int8, int4), else NULL
 *   expanded_row_idx  [T*k] int32    OUT: slot s = t*k + j -> destination row, -1
 *                                    for an invalid id
 *   sorted_src        [T*k] int32    OUT or NULL: destination row -> slot s
 *                                    (entries past expert_offsets[E] are unspecified)
 *   tokens_per_expert [E] int32      OUT: valid slots per local expert
 *   expert_offsets    [E+1] int32    OUT: exclusive prefix sum of tokens_per_expert
 * Rows of one expert keep ascending slot order, so every output is unique
 * and bit-reproducible.  Slots with an id outside [e_base, e_base + E) are left
 * out and flagged for moe_get_error().                                          */
moe_status moe_init_routing(const moe_shape* s, const void* x, const int32_t* ids,
                            int32_t e_base, void* expanded_x, float* expanded_scale,
                            int32_t* expanded_row_idx, int32_t* sorted_src,
                            int32_t* tokens_per_expert, int32_t* expert_offsets,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Grouped SwiGLU experts.  [MND §Roofline / GroupGEMM]: g groups, group i has
 * m_i rows and multiplies [m_i, k] x [k, n]; here each group runs
 * y = (silu(a W1^T) * (a W3^T)) W2^T with its own weights.  The group sizes
 * are read on the device ([MND §Quantization]: kernels read the routed token
 * counts instead of sizing work by the buffer bound).
 *   G              number of groups (experts), 1 .. 1024 (MOE_EUNSUPPORTED above)
 *   R_max          rows in a and y (>= group_offsets[G], which the kernels read)
 *   a              [R_max, H]  act, or fp8 / int8 codes when s->wt is fp8 / int8 or int4
 *   a_scale        fp32 [R_max, H/128] (fp8), [R_max] (int8), else NULL
 *   group_offsets  [G+1] int32 device array, non-decreasing, offsets[0] = 0
 *   w13            [G, 2I, H]  wt (int4: [G, 2I, H/2] packed bytes): rows 0..I-1 = W1
 *                              (gate), I..2I-1 = W3 (up)
 *   w13_scale      fp32 [G, 2I/128, H/128] (fp8), [G, 2I] per channel (int8, int4), else NULL
 *   w2             [G, H, I]   wt (int4: [G, H, I/2] packed bytes)
 *   w2_scale       fp32 [G, H/128, I/128] (fp8), [G, H] per channel (int8, int4), else NULL
 *   y              [R_max, H]  act  OUT (rows past offsets[G] are not written)
 *   ws             workspace of moe_grouped_ffn_workspace_bytes(s, G, R_max)  */
moe_status moe_grouped_ffn(const moe_shape* s, int32_t G, int32_t R_max, const void* a,
                           const float* a_scale, const int32_t* group_offsets,
                           const void* w13, const float* w13_scale, const void* w2,
                           const float* w2_scale, void* y, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* moe_grouped_ffn on activations that are not in expert order: expert-sorted row r is
 * row row_of[r] / row_div of `a`, read in place by the first GEMM, so the sorted copy of
 * the rows is never written (the row copy of [R1P §MoE deployment strategy optimization]'s
 * re-routing folded into the grouped GEMM).  row_of is typically sorted_src from
 * moe_init_routing: row_div = 1 for re-routed rows (k = 1), row_div = k to read tokens.
 *   a        [a_rows, H]  act, or fp8 / int8 codes as in moe_grouped_ffn, any row order
 *   a_scale  per row of `a`: fp32 [a_rows, H/128] (fp8), [a_rows] (int8, int4), else NULL
 *   row_of   [R_max] int32 device array; every entry r < group_offsets[G] must satisfy
 *            0 <= row_of[r] / row_div < a_rows (the routing's sorted_src does)
 *   row_div  >= 1
 * Everything else as moe_grouped_ffn (same workspace).  y equals moe_grouped_ffn's on the
 * rows gathered into expert order, bit for bit.  MOE_EUNSUPPORTED for fp32 activations
 * and when a_rows * H element bytes reaches 4 GiB (32-bit row offsets).               */
moe_status moe_grouped_ffn_gathered(const moe_shape* s, int32_t G, int32_t R_max, const void* a,
                                    int32_t a_rows, const float* a_scale, const int32_t* row_of,
                                    int32_t row_div, const int32_t* group_offsets,
                                    const void* w13, const float* w13_scale, const void* w2,
                                    const float* w2_scale, void* y, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/* Un-permute and combine.  [R1P §MoE deployment strategy optimization]:
 * finalize-routing restores token order through expanded_row_idx and forms
 * the weighted sum of the routed outputs plus the shared-expert output:
 *   out[t] = skip[t] + sum_j topk_w[t, j] * y[expanded_row_idx[t*k + j]]
 * accumulated in fp32 and rounded once.  With k = 1, topk_w = NULL and
 * skip = NULL this is the plain un-sort of re-routed rows.
 *   y                [R, H]  act  (R >= the largest index used)
 *   skip             [T, H]  act or NULL
 *   topk_w           [T, k]  fp32 or NULL (weights 1)
 *   expanded_row_idx [T*k]   int32; entries < 0 contribute nothing
 *   out              [T, H]  act  OUT                                         */
moe_status moe_finalize_routing(const moe_shape* s, const void* y, const void* skip,
                                const float* topk_w, const int32_t* expanded_row_idx,
                                void* out, hipStream_t stream);

/* Weights of one MoE layer. */
typedef struct {
  const void* w_gate;      /* [E, H] act                                       */
  const void* w13;         /* [E, 2I, H] wt (int4: [E, 2I, H/2] packed bytes)  */
  const void* w2;          /* [E, H, I] wt (int4: [E, H, I/2] packed bytes)    */
  const void* sh_w13;      /* [2*I_shared, H] shared expert: act, or int8 codes when wt
                              is int8 or int4 (then it is W8A8, [V32 §quantization
                              strategy]); never fp8                             */
  const void* sh_w2;       /* [H, I_shared] act, or int8 codes as sh_w13       */
  const float* w13_scale;  /* fp8 [E, 2I/128, H/128]; int8/int4 [E, 2I]; else NULL */
  const float* w2_scale;   /* fp8 [E, H/128, I/128]; int8/int4 [E, H]; else NULL   */
  const float* bias;       /* [E] gate-logit bias or NULL                      */
  const float* sh_w13_scale; /* int8 shared expert: [2*I_shared] per channel; else NULL */
  const float* sh_w2_scale;  /* int8 shared expert: [H] per channel; else NULL          */
} moe_weights;

/* The whole layer: gate + top-k, init-routing, grouped experts, shared expert
 * and finalize-routing, enqueued on one stream with no host synchronization.
 * [MND §Expert Parallelism]: each token goes to k different routed experts, whose
 * outputs are summed with the router's weights, and the shared expert's output is
 * added; [R1P §MoE deployment strategy optimization]: the layer's token path is
 * init-routing (expand and sort by expert), the grouped expert GEMMs, and
 * finalize-routing (un-permute, weighted sum, plus the shared-expert output).
 *   x        [T, H] act
 *   out      [T, H] act  OUT
 *   topk_idx [T, k] int32 OUT or NULL;  topk_w [T, k] fp32 OUT or NULL;
 *   logits   [T, E] fp32  OUT or NULL
 *   ws       workspace of moe_workspace_bytes(s) bytes                         */
moe_status moe_layer(const moe_shape* s, const moe_weights* w, const void* x, void* out,
                     int32_t* topk_idx, float* topk_w, float* logits, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/* moe_layer with the shared expert on a second stream.  [V32 §multi-stream parallel
 * optimization] and [MND §Computation and communication overlap] (Dispatch Overlap):
 * the shared expert needs neither the gate nor the routing, so it can run beside them.
 * When the shared expert runs in launches of its own (fp8, int4 or fp32 experts, or
 * I_shared != I; otherwise it is already a group of the routed launches and `side` is
 * not used), its launches (for the int8 shared expert of int4 layers: the per-token
 * quantization of x, then its two GEMMs) are enqueued on `side` behind an event recorded on `stream`
 * at entry, and `stream` waits for them before finalize.  On return, all of the call's
 * work is ordered before anything enqueued later on `stream`, as with moe_layer; the
 * results are bit-identical to moe_layer's.  side == NULL or side == stream: same as
 * moe_layer.  The call creates two events and releases them before returning.  Both
 * streams must belong to the current device.  An error return after the fork still
 * joins: `stream` waits for whatever was enqueued on `side`.                            */
moe_status moe_layer_overlap(const moe_shape* s, const moe_weights* w, const void* x,
                             void* out, int32_t* topk_idx, float* topk_w, float* logits,
                             void* ws, size_t ws_bytes, hipStream_t stream, hipStream_t side);

/* The most general layer call: moe_layer_overlap with a router variant (NULL
 * router: the plain router; side NULL: one stream). */
moe_status moe_layer_ex(const moe_shape* s, const moe_router* router, const moe_weights* w,
                        const void* x, void* out, int32_t* topk_idx, float* topk_w,
                        float* logits, void* ws, size_t ws_bytes, hipStream_t stream,
                        hipStream_t side);

/* Launch boundaries at which moe_layer_profiled records events. */
enum {
  MOE_EV_START = 0,      /* before the gate projection                          */
  MOE_EV_GATE = 1,       /* after the gate projection                           */
  MOE_EV_TOPK = 2,       /* after the top-k router                              */
  MOE_EV_ROUTE = 3,      /* after the counting sort (count, scan, place)        */
  MOE_EV_EXPAND = 4,     /* after the row expansion (+ fp8 quantization)        */
  MOE_EV_PLAN = 5,       /* after the grouped-GEMM unit table                   */
  MOE_EV_FFN1 = 6,       /* after the routed gate/up GEMM with SwiGLU           */
  MOE_EV_FFN2 = 7,       /* after the routed down GEMM (int8 / int4 experts: and the
                            per-row quantization of h before it)                */
  MOE_EV_SHARED = 8,     /* after both shared-expert GEMMs                      */
  MOE_EV_FINALIZE = 9,   /* after the un-permute + combine                      */
  MOE_EV_COUNT = 10
};

/* moe_layer_overlap (side may be NULL: moe_layer), additionally recording events[i] on
 * `stream` at launch boundary i (i < n_events; NULL entries are skipped), so a
 * profiler can time every kernel class of one layer from the host ([MND §Latency
 * breakdown]: the time of one MoE layer split by kernel class).  When the shared expert
 * runs on `side`, MOE_EV_SHARED follows the wait for it, so the FFN2 -> SHARED
 * interval is the part of the shared expert that the routed work did not hide.  Same
 * arguments and behaviour as moe_layer_overlap otherwise. */
moe_status moe_layer_profiled(const moe_shape* s, const moe_weights* w, const void* x,
                              void* out, int32_t* topk_idx, float* topk_w, float* logits,
                              void* ws, size_t ws_bytes, hipStream_t stream, hipStream_t side,
                              hipEvent_t* events, int32_t n_events);

/* Bytes of the fixed device scratch array behind moe_layer_static (per GPU). */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* moe_layer without a workspace argument and without any allocation, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Its workspace is a file-scope device array of
 * MOE_STATIC_SCRATCH_BYTES (64 MiB) that the library reserves on each GPU it runs on,
 * held until the process ends; shapes whose moe_workspace_bytes() exceeds it are
 * rejected with MOE_EWORKSPACE before anything is enqueued (the DeepSeek-V3 decode shape
 * -- H = 7168, 256 experts of I = 2048, top-8 -- fits up to 365 tokens with bf16 experts,
 * 383 with fp8, 310 with W8A8 and 251 with W4A8 experts).
 * Every call on a GPU shares that GPU's array, whose contents persist from the last call
 * (nothing in it has to start at zero): calls that overlap on one GPU -- on different
 * streams, or on one stream of a graph replayed while another call runs -- race, and the
 * caller must order them.  Arguments, outputs and results as moe_layer (bit for bit);
 * the stream must belong to the current device.  The first call on a device looks up the
 * array's device address (hipGetSymbolAddress); MOE_EHIP if that fails.  No
 * moe_get_error() is possible for this call (the error word lives in the array): its
 * routing ids come from its own top-k and are always in range.                        */
moe_status moe_layer_static(const moe_shape* s, const moe_weights* w, const void* x, void* out,
                            int32_t* topk_idx, float* topk_w, float* logits, hipStream_t stream);

/* Waits for `stream`, then reads and clears the device error word of `ws`:
 * MOE_EDEVICE if a routing call since the last check saw an expert id outside
 * its [e_base, e_base + E) range, else MOE_OK (MOE_EHIP on a runtime error). */
moe_status moe_get_error(void* ws, hipStream_t stream);

/* Static description of a status code. */
const char* moe_status_str(moe_status st);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
