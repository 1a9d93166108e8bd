/*
 * moe.h — C ABI of the MI355X (gfx950) sparse top-k Mixture-of-Experts FFN
 * forward.
 *
 * The layer is the one described by the "moe-training" SKILL page (Quick
 * Start, Basic MoE Architecture): a gate linear over the hidden state, softmax
 * over experts, top-k selection, renormalisation of the k selected scores to
 * sum to 1, a per-expert Linear(H,F) -> GELU -> Linear(F,H) network (F = 4H on
 * that page), and a weighted sum of the selected experts' outputs.  The router
 * also yields the load-balancing loss E * sum_e f_e * P_e and the router
 * z-loss mean(logsumexp(logits)^2) (Core Concepts, 3. Load Balancing), and
 * dispatch honours an expert capacity derived from a capacity factor
 * (Core Concepts, 4. Expert Parallelism: capacity_factor, drop_tokens).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *   buffer; the library never allocates, frees, or keeps a pointer after a
 *   call returns, and holds no state, so calls on distinct streams with
 *   distinct workspaces may run concurrently.  The one exception is
 *   moe_forward_noalloc, whose workspace is a fixed device array of the
 *   library (see there).
 * - Every GPU call is asynchronous on `stream` and never synchronises with
 *   the host, so a call sequence can be captured into a HIP graph.
 * - Row-major storage.  x[T][H]; gate Wg[H][E]; W1[E][H][F]; W2[E][F][H]:
 *   weights are stored [in][out] (the transpose of nn.Linear's [out][in]).
 *   Biases bg[E], b1[E][F], b2[E][H] may be NULL (zero bias).
 * - `dtype` is the storage type of x, weights, biases and of xp, h, y, out.
 *   Arithmetic accumulates in fp32 for both.  logits and topk_w are fp32,
 *   indices int32.
 * - Every argument is validated on the host BEFORE anything is enqueued; on
 *   error nothing is launched and a status other than MOE_OK is returned.
 *   Device faults are asynchronous and surface at the caller's next
 *   synchronisation, as with any stream API.  No C++ exception crosses the ABI.
 * - Kernel envelope: 1 <= E <= 256, 1 <= k <= min(E, 8), T * k < 2^31,
 *   H and F multiples of 8 (bf16) or 4 (fp32), every pointer 16-byte aligned;
 *   for bf16 also T*H*2, H*F*2 and E*H*2 below 2^31 bytes (the 32-bit ranges
 *   of the gathered token rows, one expert's weight block and the gate).
 *   Outside it a call returns MOE_ERR_UNSUPPORTED.
 *
 * Determinism: no floating-point atomics are used; repeated calls on the same
 * inputs produce bitwise-identical outputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,  /* null required pointer, T<1, E<1, k<1, k>E, H<1, F<1, bad dtype or activation */
    MOE_ERR_UNSUPPORTED = 2,  /* valid, but outside the kernel envelope above */
    MOE_ERR_WORKSPACE = 3,    /* ws_bytes smaller than the call needs */
    MOE_ERR_HIP = 4           /* a HIP launch or event call failed */
} moe_status_t;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype_t;

/* Activation between the two expert linears.  MOE_ACT_GELU is the exact
 * (erf) GELU of the basic layer (Quick Start, Basic MoE Architecture);
 * MOE_ACT_SILU, a * sigmoid(a), is the expert of the Mixtral 8x7B block
 * (Advanced Patterns, Mixtral 8x7B Architecture), whose linears, gate
 * included, carry no bias (pass NULL biases) and whose dispatch has no
 * capacity limit (capacity_factor <= 0). */
typedef enum { MOE_ACT_GELU = 0, MOE_ACT_SILU = 1 } moe_activation_t;

typedef struct {
    int64_t T;               /* tokens (batch * sequence, flattened) */
    int32_t H;               /* hidden width */
    int32_t E;               /* number of experts */
    int32_t k;               /* experts chosen per token */
    int32_t F;               /* expert inner width (4H on the pages) */
    double capacity_factor;  /* <= 0: no capacity limit (capacity = T) */
    int32_t dtype;           /* moe_dtype_t */
    int32_t activation;      /* moe_activation_t: the experts' activation */
} moe_problem_t;

/* moe_route flag: read `logits` as an input and skip the gate linear. */
#define MOE_ROUTE_LOGITS_IN 1u

/* Events recorded by moe_forward when `stage_events` is non-NULL: event i is
 * recorded on `stream` just before stage i starts, the last one after the
 * final stage.  MOE_EV_FFN_UP and MOE_EV_FFN_DOWN start the two expert GEMM
 * launches alone; the *_FIXUP stages that follow each sum the K slices of the
 * tiles cut in its last round and apply the epilogue to them (empty when no
 * tile is cut).  A NULL entry skips that point: every recorded event adds a
 * few microseconds between two kernels, so a caller timing one stage records
 * only its two events. */
enum {
    MOE_EV_ROUTE = 0,
    MOE_EV_PERMUTE = 1,
    MOE_EV_FFN_UP = 2,
    MOE_EV_FFN_UP_FIXUP = 3,
    MOE_EV_FFN_DOWN = 4,
    MOE_EV_FFN_DOWN_FIXUP = 5,
    MOE_EV_COMBINE = 6,
    MOE_EV_END = 7,
    MOE_FORWARD_EVENTS = 8
};

/* Expert capacity (host, synchronous): T when capacity_factor <= 0, else
 * ceil(capacity_factor * T * k / E) evaluated in double.  The capacity
 * follows the DeepSpeed MoE config on the "moe-training" SKILL page (Core
 * Concepts, 4. Expert Parallelism): the batch's routed load, scaled by the
 * capacity factor and shared evenly among the experts; here the load counts
 * all k selections of every token. */
moe_status_t moe_capacity(const moe_problem_t* p, int64_t* cap /* host */);

/* Workspace bytes (host, synchronous) that suffice for EVERY call below on
 * this problem, including moe_forward with all its optional outputs NULL. */
moe_status_t moe_workspace_bytes(const moe_problem_t* p, size_t* bytes /* host */);

/* Router: gate linear, softmax, top-k and renormalisation of the reference
 * layer (Quick Start, Basic MoE Architecture), plus the two router losses of
 * Core Concepts, 3. Load Balancing.
 *   logits[T][E]   fp32; gate output x.Wg + bg.  Optional output (NULL to
 *                  skip); with MOE_ROUTE_LOGITS_IN it is a required input.
 *   topk_idx[T][k] int32; the k largest logits of each token in descending
 *                  order, equal logits taken lower expert index first.
 *   topk_w[T][k]   fp32; softmax probabilities of the chosen experts divided
 *                  by their sum (they sum to 1; w == 1 when k == 1).
 *   counts[E]      int32; how many (token, slot) pairs chose each expert,
 *                  before capacity.
 *   losses[2]      fp32; {aux, z}: aux = E * sum_e (counts_e / (T k)) *
 *                  mean_t softmax_e, z = mean_t logsumexp_t^2.  Raw values,
 *                  no loss coefficients applied. */
moe_status_t moe_route(const moe_problem_t* p, const void* x, const void* Wg,
                       const void* bg, float* logits, int32_t* topk_idx, float* topk_w,
                       int32_t* counts, float* losses, uint32_t flags, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/* Dispatch with capacity dropping (the reference layer's per-expert token
 * gather, Quick Start, Basic MoE Architecture, with the capacity and token
 * dropping of the DeepSpeed config in Core Concepts, 4): per expert,
 * the first `capacity` (token, slot) pairs in ascending token order are kept,
 * the rest dropped.  Kept rows are laid out expert-major, token-ascending
 * within an expert.
 *   offsets[E+1]   int32; expert e owns rows [offsets[e], offsets[e+1]);
 *                  A = offsets[E] rows are kept in total.
 *   pos[T][k]      int32; row of the pair in xp, or -1 if dropped.
 *   row_token[T*k] int32; token of each kept row (rows >= A are unspecified).
 *   xp[T*k][H]     gathered copies of x rows (rows >= A are unspecified). */
moe_status_t moe_permute(const moe_problem_t* p, const void* x, const int32_t* topk_idx,
                         int32_t* offsets, int32_t* pos, int32_t* row_token, void* xp,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* Expert FFN (Quick Start, Basic MoE Architecture: Linear(H, F) -> GELU ->
 * Linear(F, H) per expert) on the
 * rows of each expert, as one grouped GEMM pair over unequal groups:
 *   h[r] = GELU(xp[r] . W1[e] + b1[e])   with exact GELU 0.5 a (1 + erf(a/sqrt2)),
 *   y[r] = h[r] . W2[e] + b2[e]          for offsets[e] <= r < offsets[e+1].
 * h[T*k][F] and y[T*k][H] are written for rows < offsets[E] only.
 * ws is optional (may be NULL): with a 16-byte aligned workspace of at least
 * moe_workspace_bytes(p) bytes, the ragged last round of GEMM tiles is split
 * along K for load balance (fp32 partials summed in a fixed order, so results
 * stay reproducible); without it every tile is computed whole. */
moe_status_t moe_expert_ffn(const moe_problem_t* p, const void* xp, const int32_t* offsets,
                            const void* W1, const void* b1, const void* W2, const void* b2,
                            void* h, void* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* Weighted combine (Quick Start, Basic MoE Architecture): for every token
 *   out[t] = sum over s = 0..k-1 with pos[t][s] >= 0 of topk_w[t][s] * y[pos[t][s]],
 * accumulated in fp32 in slot order and rounded once; a token whose slots
 * were all dropped gets a zero row.  Every row of out[T][H] is written. */
moe_status_t moe_combine(const moe_problem_t* p, const void* y, const int32_t* pos,
                         const float* topk_w, void* out, hipStream_t stream);

/* The whole layer: route -> permute -> expert FFN -> combine, with results
 * identical to calling the stages in sequence.  out[T][H] and losses[2] are
 * required; logits, topk_idx, topk_w, counts, offsets and pos are optional
 * outputs (NULL keeps them in the workspace).  stage_events is NULL or an
 * array of MOE_FORWARD_EVENTS created events (see above). */
moe_status_t moe_forward(const moe_problem_t* p, const void* x, const void* Wg,
                         const void* bg, const void* W1, const void* b1, const void* W2,
                         const void* b2, void* out, float* losses, float* logits,
                         int32_t* topk_idx, float* topk_w, int32_t* counts,
                         int32_t* offsets, int32_t* pos, void* ws, size_t ws_bytes,
                         hipStream_t stream, hipEvent_t* stage_events);

/* moe_forward with a workspace the library owns, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments and results as
 * moe_forward without ws / ws_bytes: the workspace is a fixed device array of
 * MOE_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until the
 * process ends (its device address is looked up on the first call on that
 * device).  Problems whose moe_workspace_bytes() exceeds it return
 * MOE_ERR_WORKSPACE before anything is enqueued (64 MiB holds the
 * Mixtral-shaped layer up to 454 tokens).  No call allocates or frees
 * anything.  Every call on one GPU uses the same array: calls that overlap on
 * one GPU (two streams, two threads) race and give undefined results;
 * serialise them.  Nothing needs clearing between calls: each forward writes
 * every scratch region before reading it. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status_t moe_forward_noalloc(const moe_problem_t* p, const void* x, const void* Wg,
                                 const void* bg, const void* W1, const void* b1, const void* W2,
                                 const void* b2, void* out, float* losses, float* logits,
                                 int32_t* topk_idx, float* topk_w, int32_t* counts,
                                 int32_t* offsets, int32_t* pos, hipStream_t stream,
                                 hipEvent_t* stage_events);

/* ------------------------------------------------------------ expert choice
 * Expert-choice routing (Core Concepts, 2. Routing Mechanisms: the experts
 * choose their top tokens instead of each token choosing its top experts,
 * which balances the load exactly).  The T tokens form T / group groups of
 * `group` consecutive tokens (a sequence each; group = T for one group).  In
 * every group each expert takes the C tokens with the largest gate logits
 * l[t][e] (the page ranks the raw router output over the sequence axis);
 * equal logits go to the lower token.  Expert e's selected rows are
 *   r = (e * (T / group) + g) * C + j,  j = 0 .. C-1,
 * token-ascending within each (expert, group), so offsets[e] = e * (T/group) * C
 * and every expert holds the same number of rows.  A token's output is the
 * sum, over the experts that took it in expert order, of its softmax gate
 * probability times that expert's output (no renormalisation; a token no
 * expert took gets a zero row).
 *   C = ceil(capacity_factor * group * k / E) in double, capacity_factor <= 0
 *       read as 1 (each expert takes its balanced share), clamped to [1, group];
 *       here k is the average number of experts per token.
 * Extra errors: group < 1 or T % group != 0 -> MOE_ERR_INVALID_ARG;
 * group > 32768, T * E >= 2^31 or more than 2^31 - 1 selected rows ->
 * MOE_ERR_UNSUPPORTED. */

/* C for this problem and group (host, synchronous). */
moe_status_t moe_ec_capacity(const moe_problem_t* p, int64_t group, int64_t* C /* host */);

/* Workspace bytes (host, synchronous) for both expert-choice calls below. */
moe_status_t moe_ec_workspace_bytes(const moe_problem_t* p, int64_t group,
                                    size_t* bytes /* host */);

/* Gate logits (as moe_route; fp32 [T][E], optional output, or the input when
 * flags has MOE_ROUTE_LOGITS_IN), then expert choice: probs[T][E] fp32 (each
 * token's softmax over the experts), sel[E][T/group][C] int32 (the taken
 * tokens), rowof[T][E] int32 (the row of each taken (token, expert), -1 where
 * not taken) and offsets[E+1] int32.  Selection decides on the fp32 logits. */
moe_status_t moe_route_expert_choice(const moe_problem_t* p, int64_t group, const void* x,
                                     const void* Wg, const void* bg, float* logits,
                                     uint32_t flags, float* probs, int32_t* sel,
                                     int32_t* rowof, int32_t* offsets, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

/* The expert-choice layer: moe_route_expert_choice, the grouped expert FFN
 * (Linear -> activation -> Linear) over the E * (T/group) * C selected rows,
 * gathering x by token inside the first GEMM, and the weighted combine into
 * out[T][H].  logits, probs, sel and rowof are optional outputs (NULL keeps
 * them in the workspace).  stage_events as for moe_forward, with the
 * MOE_EV_PERMUTE stage holding the expert-choice selection. */
moe_status_t moe_forward_expert_choice(const moe_problem_t* p, int64_t group, const void* x,
                                       const void* Wg, const void* bg, const void* W1,
                                       const void* b1, const void* W2, const void* b2,
                                       void* out, float* logits, float* probs, int32_t* sel,
                                       int32_t* rowof, void* ws, size_t ws_bytes,
                                       hipStream_t stream, hipEvent_t* stage_events);

/* ---------------------------------------------------------------- training
 * The backward of the layer (the pages train it: the output's loss plus the
 * weighted load-balancing and z losses, Core Concepts, 3. Load Balancing) for
 *   L = sum_t dout[t] . out[t] + g_aux * aux + g_z * z.
 * For a kept slot s of token t (expert e, weight w = p_e / S, S the sum of the
 * k selected probabilities), with a = x W1[e] + b1[e], h = act(a) and
 * y = h W2[e] + b2[e]:
 *   dy = w dout[t], dw_s = dout[t] . y;  dh = dy W2[e]^T, da = dh * act'(a);
 *   dW2[e] += h^T dy, db2[e] += dy, dW1[e] += x^T da, db1[e] += da,
 *   dx[t] += da W1[e]^T;
 * through the renormalisation dp_j = (dw_j - sum_s dw_s w_s) / S, the aux
 * loss + g_aux E f_e / T (the routed fractions f held constant), the softmax
 * dl = p (dp - p . dp) and the z-loss + g_z 2 lse p / T;
 *   dWg += x^T dl, dbg += dl, dx[t] += dl Wg^T.
 * Dropped slots and the top-k choice pass no gradient.
 * bf16 storage only (fp32 problems -> MOE_ERR_UNSUPPORTED), and T * k *
 * max(H, F) * 2 below 2^31 bytes.  dx is bf16 [T][H]; every parameter
 * gradient is fp32 in the parameter's layout (dWg [H][E], dW1 [E][H][F],
 * dW2 [E][F][H], biases [E], [E][F], [E][H]); the bias gradients are optional.
 * Every gradient is written (not accumulated) and is bitwise reproducible. */

/* Workspace bytes (host) for moe_forward_train and moe_backward. */
moe_status_t moe_train_workspace_bytes(const moe_problem_t* p, size_t* bytes /* host */);

/* moe_forward (out, losses) that keeps in ws what moe_backward needs: the fp32
 * logits, routing, dispatch, the h and y rows, and act'(a), the activation's
 * derivative at the first Linear's pre-activation a (fp32, with bias),
 * evaluated with act(a) and stored as bf16 rows. */
moe_status_t moe_forward_train(const moe_problem_t* p, const void* x, const void* Wg,
                               const void* bg, const void* W1, const void* b1, const void* W2,
                               const void* b2, void* out, float* losses, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/* Events recorded by moe_backward when `stage_events` is non-NULL, event i
 * just before stage i starts, the last after the final stage (a NULL entry
 * skips that point). */
enum {
    MOE_BEV_TOKEN = 0,       /* dw, dy rows, the router's dl */
    MOE_BEV_DGRAD_DA = 1,    /* da = (dy W2^T) * act'(a), act'(a) saved  (one GEMM launch) */
    MOE_BEV_DGRAD_DXE = 2,   /* da W1^T per kept row        (one GEMM launch) */
    MOE_BEV_DX = 3,          /* dx = sum of kept rows + dl Wg^T */
    MOE_BEV_GATHER = 4,      /* the kept rows of x */
    MOE_BEV_WGRAD_W2 = 5,    /* dW2                          (one GEMM launch) */
    MOE_BEV_WGRAD_W1 = 6,    /* dW1                          (one GEMM launch) */
    MOE_BEV_BIAS = 7,        /* db1, db2 (empty when not asked for) */
    MOE_BEV_GATE = 8,        /* dWg, dbg */
    MOE_BEV_END = 9,
    MOE_BACKWARD_EVENTS = 10
};

/* Gradients of L.  ws must hold the state of a moe_forward_train on the same
 * problem and inputs (nothing else may write it in between); biases are not
 * needed (the saved rows already include them).  stage_events is NULL or an
 * array of MOE_BACKWARD_EVENTS created events. */
moe_status_t moe_backward(const moe_problem_t* p, const void* x, const void* Wg, const void* W1,
                          const void* W2, const void* dout, float g_aux, float g_z, void* dx,
                          float* dWg, float* dbg, float* dW1, float* db1, float* dW2,
                          float* db2, void* ws, size_t ws_bytes, hipStream_t stream,
                          hipEvent_t* stage_events);

/* Static description of a status code (host). */
const char* moe_status_string(moe_status_t s);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
