/*
 * moe_int4.h -- C ABI of libmoe_int4.so: the INT4 symmetric group-quantized
 * routed-expert MoE layer on AMD Instinct MI355X (gfx950).
 *
 * The layer (as described in "Running 125B MoE on Three 3090s - vLLM
 * Optimization Edition", section 3.3, "MoE block (decode-05)", with the shapes
 * of "Running 125B MoE on Three 3090s - vLLM Edition", section 1, and the
 * weight format of the model card "Qwen3.8-Flash-Next-INT4-Mixed-AutoRound",
 * table "What is quantized", group A):
 *
 *   logits[t][e] = sum_h x[t][h] * router_w[e][h]         (bf16 in, fp32 sum)
 *   ids[t][0..k) = the k largest logits, descending, ties to the lower id
 *   w[t][j]      = softmax over the k selected logits (equal to the full
 *                  softmax renormalised over the selection)
 *   for each (t, j), e = ids[t][j]:
 *     g = W1_e x_t,  u = W3_e x_t,  a = silu(g) * u,  y = W2_e a
 *   out[t] = sum_j w[t][j] * y_j   (+ sigmoid(x_t . gate_w) * shared(x_t))
 *
 * Conventions shared by every entry point
 *   - bf16 values are passed as their uint16_t bit patterns.
 *   - All tensors are dense, row-major, in DEVICE memory, owned by the caller,
 *     and must be 16-byte aligned.  The library never allocates, frees,
 *     synchronises, or reads device memory from the host.
 *   - Work is enqueued on `hip_stream` (a hipStream_t; NULL = default stream)
 *     and is complete when the stream is.  Calls are capturable into a HIP
 *     graph (no host synchronisation, no memset nodes).
 *   - Weight format (INT4, group G = 128 -- or 64, the finer grouping
 *     weighed in "Running 125B MoE on Three 3090s - vLLM Edition", section 2
 *     -- symmetric, no zero point):
 *       w13_packed int32 [E][2I][H/8]  rows 0..I-1 = gate, rows I..2I-1 = up;
 *       w13_scales bf16  [E][2I][H/G]
 *       w2_packed  int32 [E][H][I/8];   w2_scales bf16 [E][H][I/G]
 *     Element k of a row is nibble k%8 (bits 4(k%8)..4(k%8)+3) of word k/8,
 *     holding code+8 for a code in [-8, 7]; weight = code * scale[row][k/G].
 *   - Workspace: a caller-owned device buffer of at least
 *     moe_int4_workspace_bytes() bytes.  It must be ZERO-FILLED before its
 *     first use.  Its first MOE_INT4_WS_PREFIX_BYTES bytes (the hand-off area
 *     between workgroups of one launch, the same for every shape) are zero
 *     again whenever a call completes, except the sticky status word, so a
 *     workspace can be reused without clearing, also across shapes.  Two
 *     calls in flight at the same time need two workspaces.  A call that did
 *     not complete (a device error, an aborted stream) can leave the area
 *     non-zero: zero the prefix again before reusing such a workspace.
 *   - Status word: the uint32 at byte offset MOE_INT4_WS_STATUS_OFFSET of the
 *     workspace.  The few-token path (T <= 16) hands work between workgroups
 *     of one launch through bounded waits: a workgroup polls data that
 *     workgroups with lower block indices publish.  This relies on the
 *     hardware dispatching a launch's workgroups in increasing block order
 *     (every earlier workgroup is then resident or finished when a later one
 *     waits), which AMD GPUs do but the HIP programming model does not
 *     promise.  A wait that still runs out ORs a MOE_INT4_STATUS_* bit into
 *     the status word; that call's output is then unreliable.  The library
 *     never clears the word: a caller that checks it (after the stream
 *     completes) clears it itself.
 *   - Numerics.  Products are formed exactly and summed in fp32; the output
 *     is rounded once, to nearest even, to bf16.  The SwiGLU activation
 *     a = silu(g) * u is kept in fp16 (round to nearest even, saturating at
 *     +-65504).  For more than 16 tokens (the matrix-core path) x is also
 *     converted to fp16, by rounding toward zero: exact for finite bf16
 *     values of magnitude 2^-17 .. 65504, smaller ones lose low bits (zero
 *     below 2^-24), larger ones saturate at +-65504; and each slot's weighted
 *     down-projection row w * (W2_e a) is rounded to fp16 (saturating) before
 *     a token's rows are added in fp32 in a fixed order.  Up to 16 tokens, x
 *     is used as bf16 unchanged and the weighted slot rows stay in fp32.
 *
 * Errors: every entry point returns 0 on success or a negative code.  All
 * checks run on the host before anything is enqueued, so a failing call has
 * done no work.  moe_int4_last_error() returns a message for the calling
 * thread's last failure.  No C++ exception crosses this boundary.  Failures
 * on the device are reported in the workspace's status word (above).
 */
#ifndef MOE_INT4_H
#define MOE_INT4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_INT4_OK 0
#define MOE_INT4_EINVAL (-1)     /* bad dimension, null pointer, top_k mismatch */
#define MOE_INT4_EALIGN (-2)     /* a pointer is not 16-byte aligned */
#define MOE_INT4_EWORKSPACE (-3) /* workspace smaller than required */
#define MOE_INT4_ELAUNCH (-4)    /* the HIP runtime refused a launch */
#define MOE_INT4_EDEVICE (-5)    /* no usable gfx950 device */

/* Workspace control prefix and status word (see "Workspace" above). */
#define MOE_INT4_WS_PREFIX_BYTES 65792u   /* zero between calls, except the status word */
#define MOE_INT4_WS_STATUS_OFFSET 65536u  /* uint32 sticky status word */
#define MOE_INT4_STATUS_KEY_WAIT 1u       /* routing gave up waiting for router logits */
#define MOE_INT4_STATUS_ROUTE_WAIT 2u     /* an expert workgroup gave up waiting for the routing */
#define MOE_INT4_STATUS_H_WAIT 4u         /* a down-projection workgroup gave up waiting for a */

/* Layer dimensions.  Limits: tokens >= 0 (0 is a no-op); 1 <= top_k <=
 * min(experts, 32); experts <= 1024; group 128 or 64; hidden a multiple of 256,
 * at most 4096; inter a multiple of 128, at most 1024; tokens * hidden and
 * tokens * top_k * inter (and tokens * shared inter) below 2^31. */
typedef struct moe_int4_shape {
    int32_t tokens;  /* T */
    int32_t hidden;  /* H */
    int32_t experts; /* E */
    int32_t inter;   /* I: expert intermediate size */
    int32_t group;   /* G: quantization group along the input dimension */
    int32_t top_k;   /* k */
} moe_int4_shape;

/* Optional always-on shared expert with INT6 weights ("MoE block (decode-05)":
 * it is added as sigmoid(gate logit) * shared output; model card group B:
 * INT6, group 64).  Each run of 32 codes along the input dimension is packed
 * into six int32 words: code i (stored code+32, code in [-32, 31]) occupies
 * bits 6i..6i+5 of the little-endian 192-bit concatenation of the six words.
 *   gate_w     bf16  [H]               (the extra router row)
 *   w13_packed int32 [2*inter][H/32*6]; w13_scales bf16 [2*inter][H/group]
 *   w2_packed  int32 [H][inter/32*6];   w2_scales  bf16 [H][inter/group]
 * group must be 64, inter a multiple of 128 and <= 1024. */
typedef struct moe_shared_int6 {
    const uint16_t *gate_w;
    const int32_t *w13_packed;
    const uint16_t *w13_scales;
    const int32_t *w2_packed;
    const uint16_t *w2_scales;
    int32_t inter;
    int32_t group;
} moe_shared_int6;

/* Bytes of workspace needed for `shape` (and `shared`, may be NULL). */
int32_t moe_int4_workspace_bytes(const moe_int4_shape *shape,
                                 const moe_shared_int6 *shared,
                                 size_t *bytes);

/* Routing only: router GEMV/GEMM, fp32 softmax, top-k, and the stable
 * expert permutation ("MoE block (decode-05)": top-k with ties to the lower
 * id, renormalisation, and the grouping of token slots by expert).
 *   x              bf16 [T][H]        router_w bf16 [E][H]
 *   topk_ids       int32 [T][k]  out  expert ids, descending logit
 *   topk_w         fp32  [T][k]  out  renormalised softmax weights
 *   expert_counts  int32 [E]     out  slots routed to each expert
 *   expert_offsets int32 [E+1]   out  exclusive prefix sum of the counts
 *   sorted_slots   int32 [T*k]   out  slot s = t*k + j, grouped by expert,
 *                                     increasing s within an expert */
int32_t moe_int4_route(const uint16_t *x, const uint16_t *router_w,
                       const moe_int4_shape *shape, int32_t *topk_ids,
                       float *topk_w, int32_t *expert_counts,
                       int32_t *expert_offsets, int32_t *sorted_slots,
                       void *workspace, size_t workspace_bytes,
                       void *hip_stream);

/* Experts under caller-given routing (ids must lie in [0, E); weights are
 * used as given).  `shared` may be NULL; when it is set the shared expert is
 * added with the gate logit x . shared->gate_w.  out bf16 [T][H] is
 * overwritten (round to nearest even once, from fp32) and must not alias x. */
int32_t moe_int4_experts(const uint16_t *x, const int32_t *topk_ids,
                         const float *topk_w, const int32_t *w13_packed,
                         const uint16_t *w13_scales, const int32_t *w2_packed,
                         const uint16_t *w2_scales, const moe_int4_shape *shape,
                         const moe_shared_int6 *shared, uint16_t *out,
                         void *workspace, size_t workspace_bytes,
                         void *hip_stream);

/* The whole layer: routing, routed experts and (optional) shared expert.
 * top_k must equal shape->top_k. */
int32_t moe_int4_forward(const uint16_t *x, const uint16_t *router_w,
                         const int32_t *w13_packed, const uint16_t *w13_scales,
                         const int32_t *w2_packed, const uint16_t *w2_scales,
                         int32_t top_k, uint16_t *out,
                         const moe_int4_shape *shape,
                         const moe_shared_int6 *shared, void *workspace,
                         size_t workspace_bytes, void *hip_stream);

/* moe_int4_forward with stage markers, for measurement: `events` points to
 * four hipEvent_t (created by the caller) that are recorded on hip_stream
 * before routing, after routing, after the routed gate/up projection (for
 * at most 16 tokens this stage also holds the shared expert's gate/up), and
 * after the rest (down projection, shared expert, combine).  Elapsed
 * times between them give each stage's device time.  Otherwise identical to
 * moe_int4_forward. */
int32_t moe_int4_forward_traced(const uint16_t *x, const uint16_t *router_w,
                                const int32_t *w13_packed, const uint16_t *w13_scales,
                                const int32_t *w2_packed, const uint16_t *w2_scales,
                                int32_t top_k, uint16_t *out,
                                const moe_int4_shape *shape,
                                const moe_shared_int6 *shared, void *workspace,
                                size_t workspace_bytes, void *hip_stream,
                                void *const *events);

/* moe_int4_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument; the workspace is a static device array
 * of MOE_INT4_NOALLOC_SCRATCH_BYTES inside the library, one per device, held
 * until the process ends.  Shapes whose moe_int4_workspace_bytes() exceeds
 * that size are rejected with MOE_INT4_EWORKSPACE before anything is
 * enqueued.  The first call on a device also enqueues, ahead of its own
 * kernels, one small kernel that clears the scratch's control prefix.  Every
 * call on a device shares that device's scratch: calls that overlap on one
 * device (two streams, or two threads) race and their results are
 * undefined.  The stream must belong to the current device.
 *   status  uint32 (device memory, 4-byte aligned) or NULL: failed bounded
 *           waits OR their MOE_INT4_STATUS_* bits into it (never cleared by
 *           the library); with NULL they are not reported.
 * Otherwise identical to moe_int4_forward (same kernels, same results). */
#define MOE_INT4_NOALLOC_SCRATCH_BYTES (64u << 20)
int32_t moe_int4_forward_noalloc(const uint16_t *x, const uint16_t *router_w,
                                 const int32_t *w13_packed, const uint16_t *w13_scales,
                                 const int32_t *w2_packed, const uint16_t *w2_scales,
                                 int32_t top_k, uint16_t *out,
                                 const moe_int4_shape *shape,
                                 const moe_shared_int6 *shared, uint32_t *status,
                                 void *hip_stream);

/* Load-time INT4 quantizer ("Running 125B MoE on Three 3090s - vLLM
 * Optimization Edition", section 7, which quantizes the draft head's experts
 * to symmetric INT4 in groups of 128 by rounding to nearest, choosing each
 * group's clipping range as the one with the least squared error):
 *   w       bf16  [rows][cols]        in   weights (finite values)
 *   packed  int32 [rows][cols/8]      out  codes in the layout above
 *   scales  bf16  [rows][cols/group]  out
 * For each group of 128 inputs of a row, with amax its largest magnitude,
 * the candidates are the scales s_j = bf16(fp32(amax * fp32((1 - j/40) / 7)))
 * for j = 0..19 (clips of 1 down to 0.525 of amax, the clip mapped to code
 * 7); a candidate's codes are the nearest integers to w / s_j (ties to even)
 * clamped to [-8, 7], and its error is the sum of (w - code * s_j)^2 in fp32
 * in input order.  The first candidate with the smallest error is written.
 * Scales below 2^-126 are not candidates; a group without any (all zeros)
 * gets scale 0 and codes 0.  group is 128 or 64 (the same search over groups
 * of 64 inputs, for the group-64 weights), cols a multiple of it and
 * rows * cols below 2^31; rows = 0 is a no-op.  Needs no workspace. */
int32_t moe_int4_quantize(const uint16_t *w, int32_t rows, int32_t cols, int32_t group,
                          int32_t *packed, uint16_t *scales, void *hip_stream);

/* INT8 W8A16 linear layer ("Running 125B MoE on Three 3090s - vLLM
 * Optimization Edition", section 3.3, "Hyper-connection (decode-04)": the
 * INT8 pack-quantized weight holds four codes per int32 word, least
 * significant byte first, each stored as code + 128, and is read in place;
 * model card "What is quantized", groups C and D: symmetric, group 64 for the
 * hyper-connection low-rank mixers, 128 for lm_head):
 *   x         bf16  [tokens][k]        in   activations
 *   w_packed  int32 [n][k/4]           in   byte j of word i of row r is the
 *                                           code of input 4 i + j, plus 128
 *   w_scales  bf16  [n][k/group]       in   one per (row, group of inputs)
 *   out       bf16  [tokens][n]        out  overwritten; must not alias x
 * out[t][r] = bf16(sum_i x[t][i] * (byte[r][i] - 128) * scale[r][i / group]),
 * accumulated in fp32 and rounded once (to nearest even).  Activations are
 * taken as fp16 (exact for finite bf16 values of magnitude 2^-14 .. 65504;
 * smaller ones lose low bits, larger ones saturate).  Up to 16 tokens run
 * as GEMVs (while the fp16 activations fit 64 KB of LDS); more run as a
 * matrix-core GEMM whose K may be split over workgroups, the fp32 partials
 * then living in the caller's workspace and being summed in a fixed order
 * (the result does not depend on the split schedule's timing).  group is 64 or 128, k a multiple
 * of it (at most 65536), n in [1, 2^24], tokens in [0, 2^20] with tokens * n
 * and tokens * k below 2^31; tokens = 0 is a no-op.  Pointers must be
 * 16-byte aligned; the workspace may be NULL when
 * moe_int8_linear_workspace_bytes reports 0 for the same shape.
 * Asynchronous on hip_stream; no allocation, no host synchronisation. */
int32_t moe_int8_linear_workspace_bytes(int32_t tokens, int32_t n, int32_t k, int32_t group,
                                        size_t *bytes);
int32_t moe_int8_linear(const uint16_t *x, const int32_t *w_packed, const uint16_t *w_scales,
                        int32_t tokens, int32_t n, int32_t k, int32_t group, uint16_t *out,
                        void *workspace, size_t workspace_bytes, void *hip_stream);

/* Message for the calling thread's most recent failing call ("" if none). */
const char *moe_int4_last_error(void);

/* Library version string. */
const char *moe_int4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_INT4_H */
