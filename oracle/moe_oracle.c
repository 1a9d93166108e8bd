/*
 * CPU oracle for the sparse top-k MoE FFN forward — TEST INFRASTRUCTURE ONLY.
 * Never part of the product path; see moe_oracle.h for the contract.
 *
 * Every step is written as the plain definition, in double, in the order the
 * "moe-training" SKILL page states it (Quick Start, Basic MoE Architecture;
 * Core Concepts, 3. Load Balancing).  No blocking, fusion or reordering of
 * any sum beyond ascending index order.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- storage decoding (the oracle's own; shares nothing with the GPU path) */
static inline double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static inline double load(const void* base, int64_t i, int dtype) {
    if (dtype == 1) return bf16_to_double(((const uint16_t*)base)[i]);
    if (dtype == 2) return ((const double*)base)[i];
    return (double)((const float*)base)[i];
}

/* acc[j] += s * base[off + j] for j < n, in double. */
static void axpy_row(double* acc, double s, const void* base, int64_t off, int64_t n,
                     int dtype) {
    if (dtype == 1) {
        const uint16_t* r = (const uint16_t*)base + off;
        for (int64_t j = 0; j < n; ++j) {
            uint32_t u = (uint32_t)r[j] << 16;
            float f;
            memcpy(&f, &u, sizeof f);
            acc[j] += s * (double)f;
        }
    } else if (dtype == 2) {
        const double* r = (const double*)base + off;
        for (int64_t j = 0; j < n; ++j) acc[j] += s * r[j];
    } else {
        const float* r = (const float*)base + off;
        for (int64_t j = 0; j < n; ++j) acc[j] += s * (double)r[j];
    }
}

static int valid(const orc_problem* p) {
    if (!p) return 0;
    if (p->T < 1 || p->H < 1 || p->E < 1 || p->F < 1) return 0;
    if (p->k < 1 || p->k > p->E) return 0;
    if (p->dtype != 0 && p->dtype != 1 && p->dtype != 2) return 0;
    if (p->act != 0 && p->act != 1) return 0;
    return 1;
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Gate linear: l = x . Wg + bg  (Quick Start, Basic MoE Architecture). */
int orc_logits(const orc_problem* p, const void* x, const void* Wg, const void* bg,
               double* logits) {
    if (!valid(p) || !x || !Wg || !logits) return -1;
    const int64_t T = p->T;
    const int H = p->H, E = p->E, dt = p->dtype;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double* l = logits + t * E;
        for (int e = 0; e < E; ++e) l[e] = 0.0;
        for (int i = 0; i < H; ++i) {
            const double xi = load(x, t * H + i, dt);
            axpy_row(l, xi, Wg, (int64_t)i * E, E, dt);
        }
        if (bg)
            for (int e = 0; e < E; ++e) l[e] += load(bg, e, dt);
    }
    return 0;
}

/* Softmax over experts, top-k, renormalisation of the k scores, expert counts,
 * the load-balancing loss E * sum_e f_e P_e and the z-loss mean(lse^2)
 * (Quick Start, Basic MoE Architecture; Core Concepts, 3. Load Balancing). */
int orc_route(const orc_problem* p, const double* logits, int32_t* topk_idx,
              double* topk_w, double* probs, double* lse, int32_t* counts, double* aux,
              double* z) {
    if (!valid(p) || !logits || !topk_idx || !topk_w) return -1;
    const int64_t T = p->T;
    const int E = p->E, k = p->k;
    double* P = probs ? probs : (double*)malloc(sizeof(double) * (size_t)(T * E));
    double* L = lse ? lse : (double*)malloc(sizeof(double) * (size_t)T);
    if (!P || !L) return -2;

#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double* l = logits + t * E;
        double* pt = P + t * E;
        /* softmax, shifted by the row maximum */
        double m = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > m) m = l[e];
        double Z = 0.0;
        for (int e = 0; e < E; ++e) {
            pt[e] = exp(l[e] - m);
            Z += pt[e];
        }
        for (int e = 0; e < E; ++e) pt[e] = pt[e] / Z;
        L[t] = m + log(Z);

        /* top-k: k passes of "first maximum" over the logits, skipping experts
         * already taken; descending order, equal values lower index first.
         * Softmax is strictly increasing, so the order on l equals that on p. */
        int32_t* idx = topk_idx + t * k;
        for (int s = 0; s < k; ++s) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                int taken = 0;
                for (int q = 0; q < s; ++q)
                    if (idx[q] == e) taken = 1;
                if (taken) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            idx[s] = best;
        }
        /* renormalise the selected probabilities to sum to 1 */
        double S = 0.0;
        for (int s = 0; s < k; ++s) S += pt[idx[s]];
        for (int s = 0; s < k; ++s) topk_w[t * k + s] = pt[idx[s]] / S;
    }

    if (counts) {
        for (int e = 0; e < E; ++e) counts[e] = 0;
        for (int64_t j = 0; j < T * k; ++j) counts[topk_idx[j]] += 1;
    }
    if (aux) {
        /* f_e: fraction of all T*k selections that chose e (before capacity);
         * P_e: mean softmax probability of e over tokens. */
        double acc = 0.0;
        for (int e = 0; e < E; ++e) {
            int64_t c = 0;
            for (int64_t j = 0; j < T * k; ++j) c += (topk_idx[j] == e);
            double pe = 0.0;
            for (int64_t t = 0; t < T; ++t) pe += P[t * E + e];
            acc += ((double)c / (double)(T * k)) * (pe / (double)T);
        }
        *aux = (double)E * acc;
    }
    if (z) {
        double acc = 0.0;
        for (int64_t t = 0; t < T; ++t) acc += L[t] * L[t];
        *z = acc / (double)T;
    }
    if (!probs) free(P);
    if (!lse) free(L);
    return 0;
}

/* capacity = ceil(cf * T * k / E); no limit (T) when cf <= 0. */
int64_t orc_capacity(const orc_problem* p) {
    if (!valid(p)) return -1;
    if (!(p->cf > 0.0)) return p->T;
    double c = ceil(p->cf * (double)(p->T * (int64_t)p->k) / (double)p->E);
    return (int64_t)c;
}

/* Per expert, keep the first `cap` (token, slot) pairs in ascending token
 * order; lay the kept rows out expert-major. */
int orc_dispatch(const orc_problem* p, const int32_t* topk_idx, int32_t* offsets,
                 int32_t* pos, int32_t* row_token) {
    if (!valid(p) || !topk_idx || !offsets || !pos || !row_token) return -1;
    const int64_t T = p->T;
    const int E = p->E, k = p->k;
    const int64_t cap = orc_capacity(p);
    int64_t* fill = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    int64_t* rank = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T * k));
    if (!fill || !rank) return -2;
    for (int64_t t = 0; t < T; ++t) {
        for (int s = 0; s < k; ++s) {
            const int e = topk_idx[t * k + s];
            if (e < 0 || e >= E) { free(fill); free(rank); return -3; }
            if (fill[e] < cap) {
                rank[t * k + s] = fill[e];
                fill[e] += 1;
            } else {
                rank[t * k + s] = -1;
            }
        }
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + (int32_t)fill[e];
    for (int64_t j = 0; j < T * k; ++j) row_token[j] = -1;
    for (int64_t t = 0; t < T; ++t) {
        for (int s = 0; s < k; ++s) {
            const int64_t j = t * k + s;
            if (rank[j] < 0) {
                pos[j] = -1;
            } else {
                const int32_t r = offsets[topk_idx[j]] + (int32_t)rank[j];
                pos[j] = r;
                row_token[r] = (int32_t)t;
            }
        }
    }
    free(fill);
    free(rank);
    return 0;
}

/* One expert row: a = xr . W1[e] + b1[e];  g = act(a);  y = g . W2[e] + b2[e]
 * (Basic MoE Architecture: Linear(H, 4H) -> nn.GELU() -> Linear(4H, H)), act
 * the exact erf GELU 0.5 a (1 + erf(a / sqrt 2)); or SiLU a / (1 + exp(-a))
 * (nn.SiLU of the Mixtral block, Advanced Patterns, Mixtral 8x7B Architecture). */
static double act_grad(const orc_problem* p, double a) {
    if (p->act == 1) {
        const double s = 1.0 / (1.0 + exp(-a));
        return s * (1.0 + a * (1.0 - s));
    }
    return 0.5 * (1.0 + erf(a * M_SQRT1_2)) + a * exp(-0.5 * a * a) / sqrt(2.0 * M_PI);
}

static double act_val(const orc_problem* p, double a) {
    return p->act == 1 ? a / (1.0 + exp(-a)) : 0.5 * a * (1.0 + erf(a * M_SQRT1_2));
}

/* One row through expert e: pre-activation a = x W1[e] + b1[e] [F] and
 * y = act(a) W2[e] + b2[e] [H]. */
static void row_forward(const orc_problem* p, const double* xr, int e, const void* W1,
                        const void* b1, const void* W2, const void* b2, double* a, double* y) {
    const int H = p->H, F = p->F, dt = p->dtype;
    for (int j = 0; j < F; ++j) a[j] = 0.0;
    for (int i = 0; i < H; ++i) axpy_row(a, xr[i], W1, ((int64_t)e * H + i) * F, F, dt);
    if (b1)
        for (int j = 0; j < F; ++j) a[j] += load(b1, (int64_t)e * F + j, dt);
    for (int o = 0; o < H; ++o) y[o] = 0.0;
    for (int j = 0; j < F; ++j) axpy_row(y, act_val(p, a[j]), W2, ((int64_t)e * F + j) * H, H, dt);
    if (b2)
        for (int o = 0; o < H; ++o) y[o] += load(b2, (int64_t)e * H + o, dt);
}

/* As row_forward, with the activation h = act(a) left in a. */
static void expert_row(const orc_problem* p, const double* xr, int e, const void* W1,
                       const void* b1, const void* W2, const void* b2, double* a,
                       double* y) {
    row_forward(p, xr, e, W1, b1, W2, b2, a, y);
    for (int j = 0; j < p->F; ++j) a[j] = act_val(p, a[j]);
}

int orc_expert_rows(const orc_problem* p, const void* rows, int64_t n,
                    const int32_t* experts, const void* W1, const void* b1,
                    const void* W2, const void* b2, double* h, double* y) {
    if (!valid(p) || n < 0 || (n > 0 && (!rows || !experts || !y)) || !W1 || !W2)
        return -1;
    const int H = p->H, F = p->F, dt = p->dtype;
    int bad = 0;
#pragma omp parallel
    {
        double* xr = (double*)malloc(sizeof(double) * (size_t)H);
        double* a = (double*)malloc(sizeof(double) * (size_t)F);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n; ++r) {
            const int e = experts[r];
            if (e < 0 || e >= p->E) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            for (int i = 0; i < H; ++i) xr[i] = load(rows, r * H + i, dt);
            expert_row(p, xr, e, W1, b1, W2, b2, a, y + r * H);
            if (h) memcpy(h + r * F, a, sizeof(double) * (size_t)F);
        }
        free(xr);
        free(a);
    }
    return bad ? -3 : 0;
}

/* Weighted sum over the k slots, in slot order, starting from zero
 * (Quick Start, Basic MoE Architecture).  A dropped
 * slot contributes nothing and the other weights are not renormalised. */
int orc_forward_tokens(const orc_problem* p, const void* x, const int32_t* topk_idx,
                       const double* topk_w, const int32_t* pos, const void* W1,
                       const void* b1, const void* W2, const void* b2,
                       const int64_t* tokens, int64_t ntok, double* out) {
    if (!valid(p) || !x || !topk_idx || !topk_w || !pos || !W1 || !W2 || ntok < 0 ||
        (ntok > 0 && (!tokens || !out)))
        return -1;
    const int H = p->H, F = p->F, k = p->k, dt = p->dtype;
    int bad = 0;
#pragma omp parallel
    {
        double* xr = (double*)malloc(sizeof(double) * (size_t)H);
        double* a = (double*)malloc(sizeof(double) * (size_t)F);
        double* y = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
        for (int64_t j = 0; j < ntok; ++j) {
            const int64_t t = tokens[j];
            double* o = out + j * H;
            for (int c = 0; c < H; ++c) o[c] = 0.0;
            if (t < 0 || t >= p->T) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            for (int i = 0; i < H; ++i) xr[i] = load(x, t * H + i, dt);
            for (int s = 0; s < k; ++s) {
                if (pos[t * k + s] < 0) continue;
                const int e = topk_idx[t * k + s];
                expert_row(p, xr, e, W1, b1, W2, b2, a, y);
                const double w = topk_w[t * k + s];
                for (int c = 0; c < H; ++c) o[c] += w * y[c];
            }
        }
        free(xr);
        free(a);
        free(y);
    }
    return bad ? -3 : 0;
}

int orc_combine(const orc_problem* p, const void* y, const int32_t* pos,
                const double* topk_w, double* out) {
    if (!valid(p) || !y || !pos || !topk_w || !out) return -1;
    const int64_t T = p->T;
    const int H = p->H, k = p->k, dt = p->dtype;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double* o = out + t * H;
        for (int c = 0; c < H; ++c) o[c] = 0.0;
        for (int s = 0; s < k; ++s) {
            const int32_t r = pos[t * k + s];
            if (r < 0) continue;
            axpy_row(o, topk_w[t * k + s], y, (int64_t)r * H, H, dt);
        }
    }
    return 0;
}

int64_t orc_ec_capacity(const orc_problem* p, int64_t group) {
    const double cf = p->cf > 0.0 ? p->cf : 1.0;
    double c = ceil(cf * (double)group * (double)p->k / (double)p->E);
    if (c < 1.0) c = 1.0;
    if (c > (double)group) c = (double)group;
    return (int64_t)c;
}

int orc_expert_choice(const orc_problem* p, int64_t group, const double* logits,
                      int32_t* sel, int32_t* rowof, double* probs) {
    if (!valid(p) || group < 1 || p->T % group != 0 || !logits || !sel || !rowof || !probs)
        return -1;
    const int64_t T = p->T, G = group, ng = T / group;
    const int E = p->E;
    const int64_t C = orc_ec_capacity(p, group);

    /* each token's softmax over the experts, shifted by its maximum logit */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double* l = logits + t * E;
        double m = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > m) m = l[e];
        double Z = 0.0;
        for (int e = 0; e < E; ++e) Z += exp(l[e] - m);
        for (int e = 0; e < E; ++e) {
            probs[t * E + e] = exp(l[e] - m) / Z;
            rowof[t * E + e] = -1;
        }
    }

    /* each (expert, group): C passes of "first maximum" over the untaken
     * tokens of the group, then the taken tokens listed in token order */
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < (int64_t)E * ng; ++q) {
        const int e = (int)(q / ng);
        const int64_t g = q % ng;
        char* taken = (char*)calloc((size_t)G, 1);
        if (!taken) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        for (int64_t s = 0; s < C; ++s) {
            int64_t best = -1;
            for (int64_t i = 0; i < G; ++i) {
                if (taken[i]) continue;
                if (best < 0 || logits[(g * G + i) * E + e] > logits[(g * G + best) * E + e])
                    best = i;
            }
            taken[best] = 1;
        }
        int64_t j = 0;
        for (int64_t i = 0; i < G; ++i) {
            if (!taken[i]) continue;
            const int64_t t = g * G + i;
            const int64_t row = (e * ng + g) * C + j;
            sel[row] = (int32_t)t;
            rowof[t * E + e] = (int32_t)row;
            ++j;
        }
        free(taken);
    }
    return bad ? -2 : 0;
}

/* ---------------------------------------------------------------- backward
 * The backward of the layer for the objective
 *   L = sum_t dout[t] . out[t] + g_aux * aux + g_z * z,
 * written from the chain rule on the forward's definition, in its order:
 *   kept slot s of token t, expert e, weight w = p_e / S (S: the sum of the k
 *   selected probabilities), pre-activation a = x W1[e] + b1[e], h = act(a),
 *   y = h W2[e] + b2[e], out[t] = sum over kept s of w y:
 *     dy = w dout[t];  dw_s = dout[t] . y  (0 for a dropped slot)
 *     dW2[e] += h^T dy;  db2[e] += dy;  dh = dy W2[e]^T;  da = dh * act'(a)
 *     dW1[e] += x^T da;  db1[e] += da;  dx[t] += da W1[e]^T
 *   through the renormalisation: dp_j = (dw_j - sum_s dw_s w_s) / S for the
 *   k selected experts j; the aux loss adds g_aux * E * f_e / T to every dp_e
 *   (f_e, the routed fraction, does not depend on the logits); the softmax
 *   gives dl_e = p_e (dp_e - sum_j p_j dp_j); the z-loss adds
 *   g_z * 2 lse p_e / T;  dWg += x^T dl;  dbg += dl;  dx[t] += dl Wg^T.
 * act'(a): GELU 0.5 (1 + erf(a / sqrt 2)) + a exp(-a^2 / 2) / sqrt(2 pi);
 * SiLU s (1 + a (1 - s)) with s = 1 / (1 + e^-a). */
/* Routing state shared by the backward functions. */
typedef struct {
    double* L;        /* [T][E] logits */
    double* P;        /* [T][E] probabilities */
    double* lse;      /* [T] */
    int32_t* idx;     /* [T][k] */
    double* w;        /* [T][k] renormalised weights */
    int32_t* counts;  /* [E] pre-capacity */
    int32_t* pos;     /* [T][k] row or -1 */
} bwd_route;

static void bwd_route_free(bwd_route* r) {
    free(r->L); free(r->P); free(r->lse); free(r->idx); free(r->w); free(r->counts); free(r->pos);
}

static int bwd_route_make(const orc_problem* p, const void* x, const void* Wg, const void* bg,
                          const double* logits_in, bwd_route* r) {
    const int64_t T = p->T;
    const int E = p->E, k = p->k;
    memset(r, 0, sizeof *r);
    r->L = (double*)malloc(sizeof(double) * (size_t)(T * E));
    r->P = (double*)malloc(sizeof(double) * (size_t)(T * E));
    r->lse = (double*)malloc(sizeof(double) * (size_t)T);
    r->idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k));
    r->w = (double*)malloc(sizeof(double) * (size_t)(T * k));
    r->counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    r->pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k));
    int32_t* off = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t* rt = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k));
    if (!r->L || !r->P || !r->lse || !r->idx || !r->w || !r->counts || !r->pos || !off || !rt) {
        free(off); free(rt); bwd_route_free(r);
        return -2;
    }
    int rc = 0;
    if (logits_in)
        memcpy(r->L, logits_in, sizeof(double) * (size_t)(T * E));
    else
        rc = orc_logits(p, x, Wg, bg, r->L);
    if (!rc) rc = orc_route(p, r->L, r->idx, r->w, r->P, r->lse, r->counts, NULL, NULL);
    if (!rc) rc = orc_dispatch(p, r->idx, off, r->pos, rt);
    free(off);
    free(rt);
    if (rc) bwd_route_free(r);
    return rc;
}

/* da [F] of one kept row from dy [H] and the pre-activation a [F]. */
static void row_da(const orc_problem* p, int e, const void* W2, const double* a,
                   const double* dy, double* da) {
    const int H = p->H, F = p->F, dt = p->dtype;
    for (int j = 0; j < F; ++j) {
        double dh = 0.0;
        for (int o = 0; o < H; ++o) dh += load(W2, ((int64_t)e * F + j) * H + o, dt) * dy[o];
        da[j] = dh * act_grad(p, a[j]);
    }
}

/* dl [E] of token t from dw [k] (dropped slots 0). */
static void token_dl(const orc_problem* p, const bwd_route* r, int64_t t, const double* dw,
                     double g_aux, double g_z, double* dp, double* dl) {
    const int64_t T = p->T;
    const int E = p->E, k = p->k;
    const double* pt = r->P + t * E;
    const int32_t* idx = r->idx + t * k;
    double S = 0.0, sw = 0.0;
    for (int s = 0; s < k; ++s) S += pt[idx[s]];
    for (int s = 0; s < k; ++s) sw += dw[s] * r->w[t * k + s];
    for (int e = 0; e < E; ++e)
        dp[e] = g_aux * (double)E * ((double)r->counts[e] / (double)(T * k)) / (double)T;
    for (int s = 0; s < k; ++s) dp[idx[s]] += (dw[s] - sw) / S;
    double pdp = 0.0;
    for (int e = 0; e < E; ++e) pdp += pt[e] * dp[e];
    for (int e = 0; e < E; ++e)
        dl[e] = pt[e] * (dp[e] - pdp) + g_z * 2.0 * r->lse[t] * pt[e] / (double)T;
}

int orc_backward(const orc_problem* p, const void* x, const void* Wg, const void* bg,
                 const void* W1, const void* b1, const void* W2, const void* b2,
                 const double* logits_in, const void* dout, double g_aux, double g_z,
                 double* dx, double* dWg, double* dbg, double* dW1, double* db1, double* dW2,
                 double* db2) {
    if (!valid(p) || !x || !Wg || !W1 || !W2 || !dout) return -1;
    const int64_t T = p->T;
    const int H = p->H, E = p->E, k = p->k, F = p->F, dt = p->dtype;
    bwd_route r;
    int rc = bwd_route_make(p, x, Wg, bg, logits_in, &r);
    if (rc) return rc;
    /* per (token, slot): pre-activation, dy and da of kept slots */
    double* A = (double*)calloc((size_t)(T * k * F), sizeof(double));
    double* DA = (double*)calloc((size_t)(T * k * F), sizeof(double));
    double* DY = (double*)calloc((size_t)(T * k * H), sizeof(double));
    double* DL = (double*)calloc((size_t)(T * E), sizeof(double));
    double* X = (double*)malloc(sizeof(double) * (size_t)(T * H));
    if (!A || !DA || !DY || !DL || !X) {
        free(A); free(DA); free(DY); free(DL); free(X); bwd_route_free(&r);
        return -2;
    }
    for (int64_t t = 0; t < T; ++t)
        for (int i = 0; i < H; ++i) X[t * H + i] = load(x, t * H + i, dt);

#pragma omp parallel
    {
        double* y = (double*)malloc(sizeof(double) * (size_t)H);
        double* dw = (double*)malloc(sizeof(double) * (size_t)k);
        double* dp = (double*)malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < T; ++t) {
            const double* xr = X + t * H;
            for (int s = 0; s < k; ++s) {
                dw[s] = 0.0;
                if (r.pos[t * k + s] < 0) continue;
                const int e = r.idx[t * k + s];
                double* a = A + (t * k + s) * F;
                double* dy = DY + (t * k + s) * H;
                row_forward(p, xr, e, W1, b1, W2, b2, a, y);
                const double wts = r.w[t * k + s];
                for (int o = 0; o < H; ++o) {
                    const double g = load(dout, t * H + o, dt);
                    dy[o] = wts * g;
                    dw[s] += g * y[o];
                }
                row_da(p, e, W2, a, dy, DA + (t * k + s) * F);
            }
            token_dl(p, &r, t, dw, g_aux, g_z, dp, DL + t * E);
        }
        free(y); free(dw); free(dp);
    }

    if (dx) {
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            double* o = dx + t * H;
            for (int i = 0; i < H; ++i) o[i] = 0.0;
            for (int s = 0; s < k; ++s) {
                if (r.pos[t * k + s] < 0) continue;
                const int e = r.idx[t * k + s];
                const double* da = DA + (t * k + s) * F;
                for (int i = 0; i < H; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < F; ++j) acc += load(W1, ((int64_t)e * H + i) * F + j, dt) * da[j];
                    o[i] += acc;
                }
            }
            for (int i = 0; i < H; ++i) {
                double acc = 0.0;
                for (int e = 0; e < E; ++e) acc += load(Wg, (int64_t)i * E + e, dt) * DL[t * E + e];
                o[i] += acc;
            }
        }
    }
    /* weight gradients: per expert, kept rows in ascending token order */
#pragma omp parallel for schedule(dynamic, 1)
    for (int e = 0; e < E; ++e) {
        if (dW1) memset(dW1 + (int64_t)e * H * F, 0, sizeof(double) * (size_t)H * F);
        if (db1) memset(db1 + (int64_t)e * F, 0, sizeof(double) * (size_t)F);
        if (dW2) memset(dW2 + (int64_t)e * F * H, 0, sizeof(double) * (size_t)F * H);
        if (db2) memset(db2 + (int64_t)e * H, 0, sizeof(double) * (size_t)H);
        for (int64_t t = 0; t < T; ++t) {
            for (int s = 0; s < k; ++s) {
                if (r.pos[t * k + s] < 0 || r.idx[t * k + s] != e) continue;
                const double* xr = X + t * H;
                const double* a = A + (t * k + s) * F;
                const double* da = DA + (t * k + s) * F;
                const double* dy = DY + (t * k + s) * H;
                if (dW1)
                    for (int i = 0; i < H; ++i)
                        for (int j = 0; j < F; ++j) dW1[((int64_t)e * H + i) * F + j] += xr[i] * da[j];
                if (db1)
                    for (int j = 0; j < F; ++j) db1[(int64_t)e * F + j] += da[j];
                if (dW2)
                    for (int j = 0; j < F; ++j) {
                        const double h = act_val(p, a[j]);
                        for (int o = 0; o < H; ++o) dW2[((int64_t)e * F + j) * H + o] += h * dy[o];
                    }
                if (db2)
                    for (int o = 0; o < H; ++o) db2[(int64_t)e * H + o] += dy[o];
            }
        }
    }
    if (dWg || dbg) {
        for (int e = 0; e < E; ++e) {
            if (dbg) {
                double acc = 0.0;
                for (int64_t t = 0; t < T; ++t) acc += DL[t * E + e];
                dbg[e] = acc;
            }
            if (dWg)
                for (int i = 0; i < H; ++i) {
                    double acc = 0.0;
                    for (int64_t t = 0; t < T; ++t) acc += X[t * H + i] * DL[t * E + e];
                    dWg[(int64_t)i * E + e] = acc;
                }
        }
    }
    free(A); free(DA); free(DY); free(DL); free(X);
    bwd_route_free(&r);
    return 0;
}

int orc_backward_tokens(const orc_problem* p, const void* x, const void* Wg, const void* bg,
                        const void* W1, const void* b1, const void* W2, const void* b2,
                        const double* logits_in, const void* dout, double g_aux, double g_z,
                        const int64_t* tokens, int64_t ntok, double* dx) {
    if (!valid(p) || !x || !Wg || !W1 || !W2 || !dout || ntok < 0 || (ntok > 0 && (!tokens || !dx)))
        return -1;
    const int64_t T = p->T;
    const int H = p->H, E = p->E, k = p->k, F = p->F, dt = p->dtype;
    bwd_route r;
    int rc = bwd_route_make(p, x, Wg, bg, logits_in, &r);
    if (rc) return rc;
    int bad = 0;
#pragma omp parallel
    {
        double* xr = (double*)malloc(sizeof(double) * (size_t)H);
        double* a = (double*)malloc(sizeof(double) * (size_t)(k * F));
        double* da = (double*)malloc(sizeof(double) * (size_t)F);
        double* y = (double*)malloc(sizeof(double) * (size_t)H);
        double* dy = (double*)malloc(sizeof(double) * (size_t)H);
        double* dw = (double*)malloc(sizeof(double) * (size_t)k);
        double* dp = (double*)malloc(sizeof(double) * (size_t)E);
        double* dl = (double*)malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < ntok; ++n) {
            const int64_t t = tokens[n];
            double* o = dx + n * H;
            for (int i = 0; i < H; ++i) o[i] = 0.0;
            if (t < 0 || t >= T) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            for (int i = 0; i < H; ++i) xr[i] = load(x, t * H + i, dt);
            for (int s = 0; s < k; ++s) {
                dw[s] = 0.0;
                if (r.pos[t * k + s] < 0) continue;
                const int e = r.idx[t * k + s];
                row_forward(p, xr, e, W1, b1, W2, b2, a + s * F, y);
                for (int q = 0; q < H; ++q) {
                    const double g = load(dout, t * H + q, dt);
                    dy[q] = r.w[t * k + s] * g;
                    dw[s] += g * y[q];
                }
                row_da(p, e, W2, a + s * F, dy, da);
                for (int i = 0; i < H; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < F; ++j) acc += load(W1, ((int64_t)e * H + i) * F + j, dt) * da[j];
                    o[i] += acc;
                }
            }
            token_dl(p, &r, t, dw, g_aux, g_z, dp, dl);
            for (int i = 0; i < H; ++i) {
                double acc = 0.0;
                for (int e = 0; e < E; ++e) acc += load(Wg, (int64_t)i * E + e, dt) * dl[e];
                o[i] += acc;
            }
        }
        free(xr); free(a); free(da); free(y); free(dy); free(dw); free(dp); free(dl);
    }
    bwd_route_free(&r);
    return bad ? -3 : 0;
}

/* The gate gradients dWg and dbg alone, by the definition orc_backward uses
 * and in its order: every token's kept rows run forward for dw_s = dout . y,
 * token_dl gives dl, then dbg[e] = sum_t dl[t][e] and dWg[i][e] =
 * sum_t x[t][i] dl[t][e] over ascending t.  No expert-weight or dx term is
 * formed, so it needs one forward's work and memory for dl only. */
int orc_backward_gate(const orc_problem* p, const void* x, const void* Wg, const void* bg,
                      const void* W1, const void* b1, const void* W2, const void* b2,
                      const double* logits_in, const void* dout, double g_aux, double g_z,
                      double* dWg, double* dbg) {
    if (!valid(p) || !x || !Wg || !W1 || !W2 || !dout) return -1;
    const int64_t T = p->T;
    const int H = p->H, E = p->E, k = p->k, F = p->F, dt = p->dtype;
    bwd_route r;
    int rc = bwd_route_make(p, x, Wg, bg, logits_in, &r);
    if (rc) return rc;
    double* DL = (double*)calloc((size_t)(T * E), sizeof(double));
    if (!DL) {
        bwd_route_free(&r);
        return -2;
    }
    int bad = 0;
#pragma omp parallel
    {
        double* xr = (double*)malloc(sizeof(double) * (size_t)H);
        double* a = (double*)malloc(sizeof(double) * (size_t)F);
        double* y = (double*)malloc(sizeof(double) * (size_t)H);
        double* dw = (double*)malloc(sizeof(double) * (size_t)k);
        double* dp = (double*)malloc(sizeof(double) * (size_t)E);
        if (!xr || !a || !y || !dw || !dp) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < T; ++t) {
            if (!xr || !a || !y || !dw || !dp) continue;
            for (int i = 0; i < H; ++i) xr[i] = load(x, t * H + i, dt);
            for (int s = 0; s < k; ++s) {
                dw[s] = 0.0;
                if (r.pos[t * k + s] < 0) continue;
                row_forward(p, xr, r.idx[t * k + s], W1, b1, W2, b2, a, y);
                for (int o = 0; o < H; ++o) dw[s] += load(dout, t * H + o, dt) * y[o];
            }
            token_dl(p, &r, t, dw, g_aux, g_z, dp, DL + t * E);
        }
        free(xr); free(a); free(y); free(dw); free(dp);
    }
    if (!bad) {
        for (int e = 0; e < E; ++e) {
            if (dbg) {
                double acc = 0.0;
                for (int64_t t = 0; t < T; ++t) acc += DL[t * E + e];
                dbg[e] = acc;
            }
            if (dWg)
                for (int i = 0; i < H; ++i) {
                    double acc = 0.0;
                    for (int64_t t = 0; t < T; ++t) acc += load(x, t * H + i, dt) * DL[t * E + e];
                    dWg[(int64_t)i * E + e] = acc;
                }
        }
    }
    free(DL);
    bwd_route_free(&r);
    return bad ? -2 : 0;
}

int orc_backward_weight_entries(const orc_problem* p, const void* x, const void* Wg,
                                const void* bg, const void* W1, const void* b1, const void* W2,
                                const void* b2, const double* logits_in, const void* dout,
                                const int32_t* entries, int64_t n, double* out) {
    if (!valid(p) || !x || !Wg || !W1 || !W2 || !dout || n < 0 || (n > 0 && (!entries || !out)))
        return -1;
    (void)b2;                                  /* no weight gradient depends on b2 */
    const int64_t T = p->T;
    const int H = p->H, E = p->E, k = p->k, F = p->F, dt = p->dtype;
    bwd_route r;
    int rc = bwd_route_make(p, x, Wg, bg, logits_in, &r);
    if (rc) return rc;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < n; ++q) {
        const int kind = entries[4 * q], e = entries[4 * q + 1], i = entries[4 * q + 2],
                  j = entries[4 * q + 3];
        /* kind 1: dW1[e][i][j]; 2: dW2[e][i][j]; 3: db1[e][j]; 4: db2[e][j] */
        const int fcol = kind == 1 || kind == 3 ? j : i;   /* the column f of a that is needed */
        if (kind < 1 || kind > 4 || e < 0 || e >= E || fcol < 0 || fcol >= F ||
            (kind == 1 && (i < 0 || i >= H)) || (kind == 2 && (j < 0 || j >= H)) ||
            (kind == 4 && (j < 0 || j >= H))) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        double acc = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            for (int s = 0; s < k; ++s) {
                if (r.pos[t * k + s] < 0 || r.idx[t * k + s] != e) continue;
                const double wts = r.w[t * k + s];
                if (kind == 4) {
                    acc += wts * load(dout, t * H + j, dt);
                    continue;
                }
                /* pre-activation column fcol of this row */
                double a = b1 ? load(b1, (int64_t)e * F + fcol, dt) : 0.0;
                for (int h = 0; h < H; ++h)
                    a += load(x, t * H + h, dt) * load(W1, ((int64_t)e * H + h) * F + fcol, dt);
                if (kind == 2) {
                    acc += act_val(p, a) * wts * load(dout, t * H + j, dt);
                    continue;
                }
                double dh = 0.0;
                for (int o = 0; o < H; ++o)
                    dh += load(W2, ((int64_t)e * F + fcol) * H + o, dt) * wts * load(dout, t * H + o, dt);
                const double da = dh * act_grad(p, a);
                acc += kind == 1 ? load(x, t * H + i, dt) * da : da;
            }
        }
        out[q] = acc;
    }
    bwd_route_free(&r);
    return bad ? -3 : 0;
}
