/*
 * moe_routed.h -- C ABI of the MI355X (gfx950) routed-experts layer: one GPU's share of a
 * mixture-of-experts layer, forward and backward.
 *
 * The operation (Dist-MoE 0.1.0 PyPI page, "Understand the execution model" and "BF16 Quickstart";
 * TeraMoE README, worker list; MegaMoE ROCm Primus guide, introduction):
 *
 *   caller routing (x, top-k expert ids, top-k scores)
 *     -> plan: group the T*K routed slots by expert (stable)
 *     -> permute: copy each token row into its expert-grouped rows
 *     -> W13 grouped GEMM (gate and up projections) with the SwiGLU activation
 *     -> W2 grouped GEMM (down projection)
 *     -> combine: score-weighted sum of each token's K expert rows, in token order
 *   and the backward of all of it: dscores, DGRAD (input gradients) and WGRAD (weight gradients).
 *
 * Notation: T tokens, D hidden width, F per-expert intermediate width, E experts, K slots per
 * token, N = T*K routed slots; slot i = t*K + k.
 *
 * Data types and layouts (all tensors dense, row-major, contiguous):
 *   bf16 tensors are passed as raw 16-bit patterns (uint16_t).
 *   x[T,D] bf16 ............ token rows
 *   topk_ids[T,K] .......... int32 or int64 (moe_shape.ids_dtype); expert of slot (t,k)
 *   scores[T,K] fp32 ....... routing weight of slot (t,k)
 *   w13[E,2,F,D] bf16 ...... w13[e,0] gate projection, w13[e,1] up projection, each [F,D]
 *                            ([out,in]: g = w13[e,0] . x); the same bytes as [E,2F,D]
 *   w2[E,D,F] bf16 ......... down projection [out,in]
 *   out[T,D] bf16; dout[T,D] bf16; dx[T,D] bf16; dw13[E,2,F,D] bf16; dw2[E,D,F] bf16;
 *   dscores[T,K] fp32.
 *
 * Numerics (Dist-MoE, "Choose a precision and pipeline", BF16): GEMM operands are bf16 and the
 * products accumulate in fp32. Every stored intermediate (the gate/up pre-activations h13 = [g|u],
 * the activation a = silu(g)*u, the expert outputs y, dy, dh13, dxg) and every output except
 * dscores is rounded once to bf16 (nearest-even). The combine and the dX reduction add the K slots
 * of a token in ascending k in fp32; no result depends on atomics or on scheduling, so repeated
 * calls are bitwise identical.
 *
 * Ownership: the caller allocates every buffer (device memory) and owns it; the library holds no
 * device state and allocates nothing. The plan, saved and workspace buffers are sized by the
 * moe_*_bytes queries below, which are closed forms of the shape. x, scores, w13 and w2 must stay
 * unchanged between moe_forward and the matching moe_backward; the plan and saved buffers carry
 * state from moe_plan / moe_forward to later calls until the caller reuses them.
 *
 * Streams and synchronisation: every call only enqueues work on the given stream (0 = the null
 * stream) and returns without waiting, except moe_plan_status, which waits for the stream. No
 * launch size depends on the routing, so a fixed call sequence can be captured in a graph.
 *
 * Errors: a call returns MOE_OK or a negative moe_status. Host-side checks (null or misaligned
 * pointers, bad shapes, unsupported dtypes) happen before anything is enqueued; on such an error
 * nothing is enqueued and no buffer is touched. Expert ids outside [0,E) do not fault: that slot
 * is dropped (no row; adds nothing to out, dx or the weight gradients; its dscore is 0) and
 * counted in the plan's status word, which moe_plan_status reports as MOE_E_BAD_IDS.
 * Duplicate ids within a token are legal: each slot is its own row.
 */
#ifndef MOE_ROUTED_H
#define MOE_ROUTED_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 4

/* moe_shape.ids_dtype */
#define MOE_IDS_I32 0
#define MOE_IDS_I64 1

/* moe_shape.flags: keep the forward intermediates (h13, a, y; xg too with MOE_KEEP_XG or when x
 * spans 4 GiB or more) in the saved buffer so that moe_backward can run. Without it the forward keeps its
 * intermediates in the workspace and stores no h13. */
#define MOE_SAVE_FOR_BACKWARD 1
/* Weight-gradient storage (Dist-MoE, "In-place WGRAD accumulation": gradients accumulate into
 * existing parameter-gradient storage, which is BF16 or FP32, the same dtype for W13 and W2):
 *   MOE_WGRAD_ACCUMULATE: moe_backward adds its dW13, dW2 to the values already in dw13, dw2
 *     (the new contribution, summed in fp32, is added to the old value in fp32 and the sum is
 *     stored: one rounding in bf16 storage); without it dw13, dw2 are overwritten.
 *   MOE_WGRAD_F32: dw13, dw2 are fp32 arrays (float, same shapes); without it bf16. */
#define MOE_WGRAD_ACCUMULATE 2
#define MOE_WGRAD_F32 4
/* Recompute instead of saving (TeraMoE introduction and activation-memory table: the fused
 * kernel trades recomputation for activation memory; Dist-MoE "Use graph and checkpoint
 * features": recompute under a fixed launch sequence). With MOE_SAVE_FOR_BACKWARD | MOE_RECOMPUTE
 * the forward keeps only y (and xg when it is kept at all) in the saved buffer (its a goes to the
 * workspace, which the forward then needs), and moe_backward recomputes h13 and a from x (or xg)
 * with the same kernel before
 * the backward proper: the same bits as the saved ones, so every output is bitwise the one of the
 * saving path, for one more gate/up GEMM. */
#define MOE_RECOMPUTE 8
/* Materialize xg: the forward runs the permute (xg[r] = x[t]) and the gate/up GEMM reads xg;
 * with MOE_SAVE_FOR_BACKWARD xg is kept in the saved buffer and moe_backward reads it instead of
 * x (x may then be NULL there). Without this flag xg is materialized only when x spans 4 GiB or
 * more; otherwise the GEMMs gather x's token rows through the plan. */
#define MOE_KEEP_XG 16

/* Limits checked on the host: 1 <= E <= MOE_MAX_EXPERTS, D and F multiples of 64 with
 * 64 <= D, F <= 2^22 and one expert's gate/up block below 4 GiB (4*F*D <= 2^32 bytes: the GEMM
 * copies address an expert's weight rows and a tile's activation rows by 32-bit byte offsets),
 * 1 <= K <= MOE_MAX_TOPK, T >= 1, T*K <= 2^31 - 2^16, and no grouped-GEMM launch above 2^31 - 1
 * workgroups (256 x 256 output tiles: about (T*K/256 + E) * max(D, 2F) / 256). */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 64

typedef struct moe_shape {
  int64_t T;         /* tokens */
  int64_t D;         /* hidden width */
  int64_t F;         /* per-expert intermediate width */
  int64_t E;         /* experts on this GPU */
  int64_t K;         /* routed slots per token */
  int32_t ids_dtype; /* MOE_IDS_I32 or MOE_IDS_I64 */
  int32_t flags;     /* 0 or an OR of the MOE_SAVE_FOR_BACKWARD ... MOE_KEEP_XG flags above */
} moe_shape;

typedef enum moe_status {
  MOE_OK = 0,
  MOE_E_NULL = -1,    /* a required pointer is NULL */
  MOE_E_SHAPE = -2,   /* shape outside the limits above */
  MOE_E_ALIGN = -3,   /* a pointer is not 16-byte aligned (ids/scores: element aligned) */
  MOE_E_DTYPE = -4,   /* ids_dtype or flags not recognised */
  MOE_E_HIP = -5,     /* a HIP launch or runtime call failed */
  MOE_E_BAD_IDS = -6, /* (moe_plan_status only) the routing held ids outside [0,E) */
  MOE_E_STATE = -7,   /* moe_backward on a shape without MOE_SAVE_FOR_BACKWARD (moe_forward_noalloc:
                         with it) */
  MOE_E_SCRATCH = -8  /* (moe_forward_noalloc only) the shape needs more than
                         MOE_NOALLOC_SCRATCH_BYTES of scratch */
} moe_status;

/* Optional stage timing: when a non-NULL moe_trace is passed, the call records
 * events[0] on the stream before its first kernel and events[s+1] after stage s, for the first
 * n_events events (the caller creates the events). Stages:
 *   moe_plan:     0 block histograms, 1 scan + tile tables, 2 stable scatter
 *   moe_forward:  0 permute (empty when the gate/up GEMM gathers x), 1 W13 GEMM + SwiGLU,
 *                 2 W2 GEMM, 3 combine
 *   moe_backward: 0 combine transpose + dscores, [with MOE_RECOMPUTE: the W13 GEMM + SwiGLU
 *                 again], then DGRAD W2 + SwiGLU derivative and WGRAD W2 (one launch), permute
 *                 of xg (empty when xg was saved), WGRAD W13, DGRAD W13, dX combine              */
#define MOE_TRACE_MAX_EVENTS 16
typedef struct moe_trace {
  int32_t n_events;
  hipEvent_t events[MOE_TRACE_MAX_EVENTS];
} moe_trace;

/* Byte sizes of the caller-allocated buffers (Dist-MoE "Plan memory": the caller learns the
 * device memory a configuration needs before it runs; here every size is a closed form of the
 * shape, so no planner object is kept); 0 for a shape that fails the checks. */
size_t moe_plan_bytes(const moe_shape* shape);
size_t moe_saved_bytes(const moe_shape* shape);     /* 0 unless MOE_SAVE_FOR_BACKWARD */
size_t moe_workspace_bytes(const moe_shape* shape); /* forward without save or with recompute,
                                                      and backward */

/* Routing plan (Dist-MoE, "Understand the execution model": routing metadata is generated on the
 * GPU from caller ids; TeraMoE README: the scheduler forms per-expert batches).
 * From topk_ids[T,K] it builds, in plan (moe_plan_bytes, device):
 *   counts[e] = #slots routed to e;  offsets[e] = sum of counts below e;
 *   pos[i] = offsets[id_i] + #{j < i : id_j = id_i}  (stable expert-grouped row of slot i; -1 when
 *            id_i is out of range);  src[pos[i]] = i;
 *   the row-tile list the grouped GEMMs walk, an expert order by decreasing count,
 *   and the status word (number of out-of-range ids). */
moe_status moe_plan(const moe_shape* shape, const void* topk_ids, void* plan, hipStream_t stream,
                    const moe_trace* trace);

/* Forward (Dist-MoE "Understand the execution model"; TeraMoE compute and combine workers;
 * MegaMoE dispatch grouped GEMM -> SwiGLU -> grouped GEMM combine). With r = pos[t*K+k], e = id:
 *   xg[r]   = x[t]                                           (permute)
 *   g, u    = bf16(w13[e,0] . xg[r]), bf16(w13[e,1] . xg[r])  (gate/up grouped GEMM, fp32 acc)
 *   a[r]    = bf16(silu(g) * u)                              (SwiGLU epilogue)
 *   y[r]    = bf16(w2[e] . a[r])                             (down grouped GEMM)
 *   out[t]  = bf16(sum_k scores[t,k] * y[pos[t*K+k]])        (combine, k ascending, fp32)
 *  plan: from moe_plan with the same shape and ids. saved (moe_saved_bytes) is required with
 * MOE_SAVE_FOR_BACKWARD, workspace (moe_workspace_bytes) without it; the other may be NULL.
 * When x spans less than 4 GiB (T*D*2 < 2^32) the permute is fused into the gate/up GEMM, which
 * reads each routed row's token row of x directly (MoonEP FAQ: tokens go straight to their
 * expert-grouped positions), and xg is never materialized: the backward's W13 weight gradient
 * (and the recompute) read x through the plan the same way. Otherwise xg is written (and saved
 * with MOE_SAVE_FOR_BACKWARD). */
moe_status moe_forward(const moe_shape* shape, const void* plan, const uint16_t* x,
                       const float* scores, const uint16_t* w13, const uint16_t* w2, uint16_t* out,
                       void* saved, void* workspace, hipStream_t stream, const moe_trace* trace);

/* Allocation-free forward, for callers that cannot allocate device memory or pass a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid allocation. It computes
 * exactly what moe_forward computes without MOE_SAVE_FOR_BACKWARD (the same kernels, so the same
 * bits), with the forward's intermediates (a[N,F], y[N,D], and xg[N,D] when materialized) kept in
 * a scratch array that the library holds per GPU (MOE_NOALLOC_SCRATCH_BYTES, loaded with the
 * library's code object and held until the process ends) instead of a caller workspace. The
 * caller passes the inputs (plan from moe_plan, x, scores, w13, w2) and the output out, as for
 * moe_forward. It calls no allocating routine; its first call on a GPU looks up that GPU's copy of
 * the array (hipGetSymbolAddress). Nothing in the scratch has to start at zero: every element a
 * call reads was written earlier in the same call, and each call overwrites what the last one
 * left. Every call on one GPU shares that GPU's scratch: calls that overlap in time on one GPU
 * (other streams, other threads) race and must be ordered by the caller.
 * Errors: as for moe_forward, plus MOE_E_STATE when the shape has MOE_SAVE_FOR_BACKWARD, and
 * MOE_E_SCRATCH when the intermediates exceed MOE_NOALLOC_SCRATCH_BYTES: a and y take 2*N*F and
 * 2*N*D bytes (each rounded up to 256), xg another 2*N*D when it is materialized (MOE_KEEP_XG, or
 * x of 4 GiB or more). Both are host-side checks: nothing is enqueued. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_forward_noalloc(const moe_shape* shape, const void* plan, const uint16_t* x,
                               const float* scores, const uint16_t* w13, const uint16_t* w2,
                               uint16_t* out, hipStream_t stream, const moe_trace* trace);

/* Backward of moe_forward (Dist-MoE: DGRAD and WGRAD; MegaMoE "Design": the down projection's
 * weight gradient is produced before the gate/up one; here the gate/up weight gradient also runs
 * before dxg, so that xg, when it was not saved, is permuted from x into the workspace region
 * that dy no longer needs and dxg takes next), given dout[T,D]:
 *   dy[r]       = bf16(scores[t,k] * dout[t]);   dscores[t,k] = sum_d dout[t,d] * y[r,d]  (fp32)
 *   da[r]       = w2[e]^T . dy[r]   (fp32, not stored);   with s = sigmoid(g):
 *   dg          = bf16(da * u * s * (1 + g*(1 - s)));  du = bf16(da * g * s);  dh13[r] = [dg|du]
 *   dw2[e]      = bf16(sum over e's rows of dy^T a)      (zero for an expert with no rows)
 *   dxg[r]      = bf16(w13[e]^T . dh13[r])                (w13[e] viewed as [2F,D])
 *   dw13[e]     = bf16(sum over e's rows of dh13^T xg)      (xg[r] = x[t], read from x or saved)
 *   dx[t]       = bf16(sum_k dxg[pos[t*K+k]])             (k ascending, fp32)
 * dx is overwritten; dw13 and dw2 are overwritten or accumulated into, bf16 or fp32, as the shape's
 * MOE_WGRAD_* flags say (the accumulation of a call is not atomic with respect to other work on the
 * same buffers: calls that accumulate into one buffer must be ordered, e.g. on one stream).
 * Requires the shape's MOE_SAVE_FOR_BACKWARD, the saved
 * buffer of the matching forward and its x (device, [T,D] bf16, unchanged since the forward; may
 * be NULL when the forward kept xg: MOE_KEEP_XG, or x spanning 4 GiB or more); workspace holds
 * dy/dxg and dh13. */
moe_status moe_backward(const moe_shape* shape, const void* plan, const void* saved,
                        const uint16_t* x, const uint16_t* dout, const float* scores, const uint16_t* w13,
                        const uint16_t* w2, uint16_t* dx, void* dw13, void* dw2,
                        float* dscores, void* workspace, hipStream_t stream,
                        const moe_trace* trace);

/* The row steps on their own, for callers that run the expert GEMMs elsewhere or time the steps
 * apart (TeraMoE README, worker list: dispatch writes the expert inputs, combine applies the
 * weighted accumulation, gather reduces several results of one token locally; Dist-MoE
 * "Understand the execution model": permute -> ... -> combine). Same kernels as inside
 * moe_forward / moe_backward; plan from moe_plan with the same shape and ids; dropped slots
 * (pos = -1) move nothing and add nothing.
 *   moe_permute:          xg[pos[t*K+k]] = x[t]                  (xg [N,D] bf16, rows in grouped order)
 *   moe_combine:          out[t] = bf16(sum_k w_k * rows[pos[t*K+k]]), k ascending in fp32, with
 *                         w_k = scores[t,k], or 1 when scores is NULL (the dX reduction); rows [N,D]
 *   moe_combine_backward: dy[pos[t*K+k]] = bf16(scores[t,k] * dout[t]);
 *                         dscores[t,k] = sum_d dout[t,d] * y[pos[t*K+k], d] (fp32; 0 when dropped)
 * Buffers 16-byte aligned (scores, dscores 4); errors as for moe_forward. */
moe_status moe_permute(const moe_shape* shape, const void* plan, const uint16_t* x, uint16_t* xg,
                       hipStream_t stream);
moe_status moe_combine(const moe_shape* shape, const void* plan, const uint16_t* rows,
                       const float* scores, uint16_t* out, hipStream_t stream);
moe_status moe_combine_backward(const moe_shape* shape, const void* plan, const uint16_t* dout,
                                const uint16_t* y, const float* scores, uint16_t* dy,
                                float* dscores, hipStream_t stream);

/* Copy the plan's integer arrays into caller device buffers (int32): counts[E], offsets[E+1],
 * pos[N], src[N] (src entries past the last routed row are -1). Any of them may be NULL.
 * (Dist-MoE "Understand the execution model": the routing metadata built on the GPU drives the
 * permute, the expert GEMMs and the combine; this exposes it to the caller, e.g. for a
 * dispatcher that sends the grouped rows elsewhere.) Enqueued on stream; errors as for moe_plan. */
moe_status moe_plan_export(const moe_shape* shape, const void* plan, int32_t* counts,
                           int32_t* offsets, int32_t* pos, int32_t* src, hipStream_t stream);

/* Wait for the stream, then report the plan's status word: *bad_ids (host pointer, may be NULL)
 * receives the number of out-of-range ids; returns MOE_E_BAD_IDS when it is non-zero.
 * (Dist-MoE "BF16 Quickstart" and "Understand the execution model" require ids in [0,E) and trap
 * on others; here such slots are dropped and counted, and this call reports the count.) The only
 * call that waits for the stream. */
moe_status moe_plan_status(const moe_shape* shape, const void* plan, int64_t* bad_ids,
                           hipStream_t stream);

/* (TeraMoE README, activation-memory table: what the forward keeps for the backward.)
 * Device pointers to the saved forward intermediates inside saved (for inspection and tests):
 * xg[N,D], h13[N,2F], a[N,F], y[N,D], all bf16. Any output pointer may be NULL. Intermediates that
 * are not saved come back as NULL: h13 and a with MOE_RECOMPUTE, xg unless MOE_KEEP_XG or x
 * spans 4 GiB or more (the GEMMs then read x through the plan). */
moe_status moe_saved_views(const moe_shape* shape, void* saved, uint16_t** xg, uint16_t** h13,
                           uint16_t** a, uint16_t** y);

/* Router (MegaMoE, ROCm Primus guide, introduction: score function + group-limited top-k ahead
 * of the expert path; Primus "Router force load balancing", uniform: routing of random logits).
 * From logits[T,E] fp32 it writes topk_ids[T,K] (shape.ids_dtype) and scores[T,K] fp32, ready for
 * moe_plan / moe_forward:
 *   score: MOE_SCORE_SOFTMAX (softmax over the token's E logits) or MOE_SCORE_SIGMOID (logistic
 *          sigmoid of each logit). Both increase with the logit, so the chosen experts are the K
 *          largest logits, in descending order (ties: lower expert id first; NaN ranks last).
 *   group limit: n_group > 1 splits the experts into n_group groups of E/n_group consecutive ids;
 *          a group ranks by its largest logit (ties: lower group), and only the experts of the
 *          topk_group best groups can be chosen. n_group <= 1 means no group limit.
 *   weights: the chosen experts' scores; with renormalize != 0 divided by their sum over the K
 *          chosen (for softmax: the softmax of the K chosen logits). fp32, expf.
 * Reads shape.T, E, K and ids_dtype only (1 <= E <= MOE_MAX_EXPERTS, 1 <= K <= min(E,
 * MOE_MAX_TOPK)); requires n_group <= 64 dividing E, 1 <= topk_group <= n_group and
 * K <= topk_group * E / n_group. logits and scores 4-byte aligned, topk_ids aligned to its type.
 * Errors as for the other calls; nothing is enqueued on a host-side error. */
#define MOE_SCORE_SOFTMAX 0
#define MOE_SCORE_SIGMOID 1
#define MOE_MAX_GROUPS 64

typedef struct moe_router {
  int32_t score_fn;    /* MOE_SCORE_SOFTMAX or MOE_SCORE_SIGMOID */
  int32_t renormalize; /* != 0: weights divided by their sum over the K chosen experts */
  int32_t n_group;     /* expert groups; <= 1: no group limit */
  int32_t topk_group;  /* groups kept per token when n_group > 1 */
} moe_router;

moe_status moe_route(const moe_shape* shape, const moe_router* router, const float* logits,
                     void* topk_ids, float* scores, hipStream_t stream, const moe_trace* trace);

/* A fixed English description of a moe_status value ("unknown status" for others); static
 * storage, never NULL. */
const char* moe_status_str(int status);
/* The version of this interface (the value of MOE_ABI_VERSION the library was built with). */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTED_H */
