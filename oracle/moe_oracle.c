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
    } else {
        const float* r = (const float*)base + off;
        for (int64_t j = 0; j < n; ++j) acc[j] += s * (double)r[j];
    }
}

static int valid(const orc_problem* p) {
    if (!p) return 0;
    if (p->T < 1 || p->H < 1 || p->E < 1 || p->F < 1) return 0;
    if (p->k < 1 || p->k > p->E) return 0;
    if (p->dtype != 0 && p->dtype != 1) return 0;
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
static void expert_row(const orc_problem* p, const double* xr, int e, const void* W1,
                       const void* b1, const void* W2, const void* b2, double* a,
                       double* y) {
    const int H = p->H, F = p->F, dt = p->dtype;
    for (int j = 0; j < F; ++j) a[j] = 0.0;
    for (int i = 0; i < H; ++i) axpy_row(a, xr[i], W1, ((int64_t)e * H + i) * F, F, dt);
    for (int j = 0; j < F; ++j) {
        if (b1) a[j] += load(b1, (int64_t)e * F + j, dt);
        a[j] = p->act == 1 ? a[j] / (1.0 + exp(-a[j]))
                           : 0.5 * a[j] * (1.0 + erf(a[j] * M_SQRT1_2));
    }
    for (int o = 0; o < H; ++o) y[o] = 0.0;
    for (int j = 0; j < F; ++j) axpy_row(y, a[j], W2, ((int64_t)e * F + j) * H, H, dt);
    if (b2)
        for (int o = 0; o < H; ++o) y[o] += load(b2, (int64_t)e * H + o, dt);
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
