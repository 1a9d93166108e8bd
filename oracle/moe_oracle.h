/*
 * CPU oracle for the sparse top-k MoE FFN forward — TEST INFRASTRUCTURE ONLY.
 *
 * Only tests, the package smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The product path never calls it.
 *
 * It is a plain, slow, per-token fp64 implementation of the layer described
 * by the "moe-training" SKILL page (Quick Start, Basic MoE Architecture:
 * gate Linear -> softmax -> top-k -> renormalise -> per-expert
 * Linear(H,4H) -> GELU -> Linear(4H,H) -> weighted sum; or SiLU in place of
 * GELU, as in the Mixtral block of Advanced Patterns, Mixtral 8x7B
 * Architecture) together with the
 * load-balancing and router z-losses (Core Concepts, 3. Load Balancing) and
 * capacity-factor dropping (Core Concepts, 4. Expert Parallelism; Best
 * Practices, 2. Capacity Factor Tuning).
 *
 * Storage: inputs are read as fp32 values (dtype 0) or bf16 bit patterns
 * (dtype 1, uint16) and widened exactly to double; every sum is in double with
 * no intermediate rounding.  Weight layout is [in][out]: Wg[H][E],
 * W1[E][H][F], W2[E][F][H].  Null bias pointers mean zero bias.
 *
 * All functions return 0 on success and a negative value on a bad argument.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int64_t T;      /* tokens */
    int32_t H;      /* hidden width */
    int32_t E;      /* experts */
    int32_t k;      /* experts per token */
    int32_t F;      /* expert inner width (4H on the pages) */
    double  cf;     /* capacity factor; <= 0 means no capacity limit */
    int32_t dtype;  /* 0: fp32 storage, 1: bf16 storage, 2: fp64 storage */
    int32_t act;    /* expert activation: 0 exact GELU, 1 SiLU */
} orc_problem;

/* Gate logits l[t][e] = bg[e] + sum_i x[t][i] * Wg[i][e]  (double, [T][E]). */
int orc_logits(const orc_problem* p, const void* x, const void* Wg, const void* bg,
               double* logits);

/* Softmax, top-k (descending; equal values: lower expert index first),
 * renormalised weights, pre-capacity counts, aux and z losses, from logits.
 * probs [T][E] and lse [T] are optional (may be NULL). */
int orc_route(const orc_problem* p, const double* logits, int32_t* topk_idx,
              double* topk_w, double* probs, double* lse, int32_t* counts,
              double* aux, double* z);

/* Expert capacity: T when cf <= 0, else ceil(cf * T * k / E). */
int64_t orc_capacity(const orc_problem* p);

/* Token-order dispatch with capacity dropping: offsets [E+1], pos [T][k]
 * (-1 = dropped), row_token [T*k] (entries >= offsets[E] set to -1). */
int orc_dispatch(const orc_problem* p, const int32_t* topk_idx, int32_t* offsets,
                 int32_t* pos, int32_t* row_token);

/* Expert FFN on n rows: rows[r] (storage type, [n][H]) through expert
 * experts[r]; writes GELU outputs h [n][F] (optional) and y [n][H]. */
int orc_expert_rows(const orc_problem* p, const void* rows, int64_t n,
                    const int32_t* experts, const void* W1, const void* b1,
                    const void* W2, const void* b2, double* h, double* y);

/* Layer output for the listed tokens: out[j][o] for token tokens[j], given the
 * routing (topk_idx, topk_w) and dispatch (pos).  out is [ntok][H]. */
int orc_forward_tokens(const orc_problem* p, const void* x, const int32_t* topk_idx,
                       const double* topk_w, const int32_t* pos, const void* W1,
                       const void* b1, const void* W2, const void* b2,
                       const int64_t* tokens, int64_t ntok, double* out);

/* Weighted combine of given expert-output rows y [A][H] (storage type):
 * out[t] = sum over kept slots s, in slot order, of w[t][s] * y[pos[t][s]]. */
int orc_combine(const orc_problem* p, const void* y, const int32_t* pos,
                const double* topk_w, double* out);

/* Expert-choice routing ("moe-training" SKILL page, Core Concepts, 2. Routing
 * Mechanisms: expert choice; experts pick tokens instead of tokens picking
 * experts).  The T tokens form T / group groups of `group` consecutive tokens
 * (a sequence each); in every group each expert takes C = orc_ec_capacity
 * tokens: those with the largest logits[t][e], taken one at a time as the
 * first maximum over the untaken tokens (descending value, equal values lower
 * token first).  Outputs:
 *   sel   [E][T/group][C]  taken tokens of each (expert, group), ascending;
 *   rowof [T][E]           row (e * (T/group) + g) * C + j of token
 *                          sel[e][g][j] in the expert-major row order, else -1;
 *   probs [T][E]           softmax of each token's logits over the experts:
 *                          its weight for each expert that takes it. */
int orc_expert_choice(const orc_problem* p, int64_t group, const double* logits,
                      int32_t* sel, int32_t* rowof, double* probs);

/* Expert-choice capacity: ceil(cf * group * k / E) in double, with cf <= 0
 * read as 1 (each expert takes its balanced share), clamped to [1, group]. */
int64_t orc_ec_capacity(const orc_problem* p, int64_t group);

/* Backward of the layer ("moe-training" SKILL page: training minimises the
 * output loss plus the weighted router losses) for the objective
 *   L = sum_t dout[t] . out[t] + g_aux * aux + g_z * z,
 * dout [T][H] in the storage type.  Routing is decided on logits_in [T][E]
 * when given, else on the gate linear of x.  Outputs (double; any may be
 * NULL): dx [T][H], dWg [H][E], dbg [E], dW1 [E][H][F], db1 [E][F],
 * dW2 [E][F][H], db2 [E][H].  Dropped slots and the top-k selection pass no
 * gradient; the renormalised weights, the softmax and both losses do. */
int orc_backward(const orc_problem* p, const void* x, const void* Wg, const void* bg,
                 const void* W1, const void* b1, const void* W2, const void* b2,
                 const double* logits_in, const void* dout, double g_aux, double g_z,
                 double* dx, double* dWg, double* dbg, double* dW1, double* db1, double* dW2,
                 double* db2);

/* dx rows [ntok][H] of the listed tokens only (the same definition). */
int orc_backward_tokens(const orc_problem* p, const void* x, const void* Wg, const void* bg,
                        const void* W1, const void* b1, const void* W2, const void* b2,
                        const double* logits_in, const void* dout, double g_aux, double g_z,
                        const int64_t* tokens, int64_t ntok, double* dx);

/* The gate gradients dWg [H][E] and dbg [E] alone (either may be NULL): the
 * same definition and summation order as orc_backward, with one forward's
 * work (every kept row's y for dw) and none of the expert-weight terms. */
int orc_backward_gate(const orc_problem* p, const void* x, const void* Wg, const void* bg,
                      const void* W1, const void* b1, const void* W2, const void* b2,
                      const double* logits_in, const void* dout, double g_aux, double g_z,
                      double* dWg, double* dbg);

/* Single entries of the expert-weight gradients: entries [n][4] = (kind, e,
 * i, j) with kind 1: dW1[e][i][j], 2: dW2[e][i][j], 3: db1[e][j], 4: db2[e][j];
 * each is summed over the expert's kept rows in token order. */
int orc_backward_weight_entries(const orc_problem* p, const void* x, const void* Wg,
                                const void* bg, const void* W1, const void* b1, const void* W2,
                                const void* b2, const double* logits_in, const void* dout,
                                const int32_t* entries, int64_t n, double* out);

/* Number of OpenMP threads the oracle uses. */
int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
