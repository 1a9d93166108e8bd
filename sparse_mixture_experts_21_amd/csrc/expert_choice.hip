// Expert-choice routing ("moe-training" SKILL page, Core Concepts, 2. Routing
// Mechanisms: experts choose their top tokens instead of tokens choosing
// experts, which balances the load exactly).  The T tokens form T / G groups
// of G consecutive tokens (a sequence each); in every group each expert takes
// the C tokens with the largest gate logits, equal logits going to the lower
// token.  Expert e's rows are e * ng * C .. (e + 1) * ng * C - 1 (ng = T / G),
// group-major and token-ascending inside a group, so every expert holds
// exactly ng * C rows and the grouped GEMMs run on them unchanged.
//
//   ec_probs    each token's softmax over the experts (its weight for every
//               expert that takes it) and the fixed row offsets;
//   ec_select   one workgroup per (expert, group): the group's column of
//               logits as order-preserving integer keys in LDS, an MSB-first
//               radix select of the C-th largest key (four 8-bit passes with
//               per-wave LDS histograms), then two block scans in token order
//               that settle the ties at the threshold and assign rows.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// Order-preserving map from fp32 to uint32 (larger float -> larger key).  -0
// is folded into +0 first, so the two tie as they compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t b = f == 0.0f ? 0u : __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Exclusive scan of one value per thread over the workgroup (token order =
// thread order); also returns the workgroup total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wtot, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(incl, d);
        if (lane >= d) incl += u;
    }
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const int t = wtot[w];
        base += w < wave ? t : 0;
        tot += t;
    }
    __syncthreads();                                   // wtot reusable
    total = tot;
    return base + incl - v;
}

__global__ __launch_bounds__(256) void ec_probs(const float* __restrict__ logits, int64_t T,
                                                int E, float* __restrict__ probs,
                                                int32_t* __restrict__ offsets, int64_t rows_per_e) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (blockIdx.x == 0)
        for (int q = threadIdx.x; q <= E; q += 256) offsets[q] = (int32_t)(q * rows_per_e);
    if (t >= T) return;
    const float* l = logits + t * E;
    float m = l[0];
    for (int e = 1; e < E; ++e) m = fmaxf(m, l[e]);
    float Z = 0.f;
    for (int e = 0; e < E; ++e) Z += expf(l[e] - m);
    const float r = 1.0f / Z;
    for (int e = 0; e < E; ++e) probs[t * E + e] = expf(l[e] - m) * r;
}

// Workgroup b = e * ng + g.  Dynamic LDS: G keys.
__global__ __launch_bounds__(kSelThreads) void ec_select(const float* __restrict__ logits, int E,
                                                         int64_t G, int ng, int C,
                                                         int32_t* __restrict__ sel,
                                                         int32_t* __restrict__ rowof) {
    extern __shared__ uint32_t keys[];
    __shared__ int hist[kSelWaves][256];
    __shared__ int wtot[kSelWaves];
    __shared__ uint32_t s_prefix;
    __shared__ int s_need;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x;
    const int e = b / ng, g = b % ng;
    const int64_t t0 = (int64_t)g * G;

    for (int64_t i = tid; i < G; i += kSelThreads) keys[i] = order_key(logits[(t0 + i) * E + e]);
    if (tid == 0) {
        s_prefix = 0u;
        s_need = C;
    }
    __syncthreads();

    // ---- radix select: after pass p the top 8 (p + 1) bits of the C-th
    // largest key are known, and `need` counts how many keys equal to that
    // prefix are still to be taken (all larger ones are taken).
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int q = lane; q < 256; q += 64) hist[wave][q] = 0;
        __syncthreads();
        const uint32_t prefix = s_prefix;
        for (int64_t i = tid; i < G; i += kSelThreads) {
            const uint32_t k = keys[i];
            // 64-bit shift: in pass 0 every key is a candidate (shift by 32)
            const bool cand = ((uint64_t)k >> (shift + 8)) == (uint64_t)prefix;
            if (cand) atomicAdd(&hist[wave][(k >> shift) & 255u], 1);
        }
        __syncthreads();
        if (wave == 0) {
            const int need = s_need;
            // lane l owns digits 4l .. 4l + 3; counts summed over the waves
            int c[4], cl = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int s = 0;
                for (int w = 0; w < kSelWaves; ++w) s += hist[w][4 * lane + j];
                c[j] = s;
                cl += s;
            }
            // inclusive suffix sum over lanes: keys in digits >= 4l
            int suf = cl;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int u = __shfl_down(suf, d);
                if (lane + d < 64) suf += u;
            }
            // the threshold digit lies in the highest lane whose suffix reaches need
            const uint64_t ok = __ballot(suf >= need);
            const int L = 63 - __builtin_clzll(ok);
            if (lane == L) {
                int above = suf - cl;                  // keys in higher lanes' digits
                int dig = 4 * lane;
                for (int j = 3; j >= 0; --j) {
                    if (above + c[j] >= need) {
                        dig = 4 * lane + j;
                        break;
                    }
                    above += c[j];
                }
                s_need = need - above;
                s_prefix = (prefix << 8) | (uint32_t)dig;
            }
        }
        __syncthreads();
    }
    const uint32_t kth = s_prefix;                     // the C-th largest key
    const int need = s_need;                           // ties at kth still to take

    // ---- assignment in token order: thread tid owns tokens [tid*per, tid*per + per)
    const int per = (int)((G + kSelThreads - 1) / kSelThreads);
    const int64_t i0 = (int64_t)tid * per, i1 = min((int64_t)(tid + 1) * per, G);
    int n_eq = 0;
    for (int64_t i = i0; i < i1; ++i) n_eq += keys[i] == kth;
    int tot;
    const int eq_base = block_exclusive_scan(n_eq, wtot, tot);
    int n_take = 0, eq_seen = 0;
    for (int64_t i = i0; i < i1; ++i) {
        const uint32_t k = keys[i];
        const bool eq = k == kth;
        n_take += k > kth || (eq && eq_base + eq_seen < need);
        eq_seen += eq;
    }
    const int row_base = block_exclusive_scan(n_take, wtot, tot);
    int j = row_base;
    eq_seen = 0;
    const int64_t row0 = (int64_t)b * C;
    for (int64_t i = i0; i < i1; ++i) {
        const uint32_t k = keys[i];
        const bool eq = k == kth;
        const bool take = k > kth || (eq && eq_base + eq_seen < need);
        eq_seen += eq;
        const int64_t t = t0 + i;
        if (take) {
            sel[row0 + j] = (int32_t)t;
            rowof[t * E + e] = (int32_t)(row0 + j);
            ++j;
        } else {
            rowof[t * E + e] = -1;
        }
    }
}

}  // namespace

hipError_t launch_expert_choice(const moe_problem_t& p, int64_t group, int64_t C,
                                const float* logits, float* probs, int32_t* sel,
                                int32_t* rowof, int32_t* offsets, hipStream_t s) {
    const int64_t ng = p.T / group;
    ec_probs<<<dim3((unsigned)((p.T + 255) / 256)), dim3(256), 0, s>>>(logits, p.T, p.E, probs,
                                                                      offsets, ng * C);
    const size_t lds = (size_t)group * 4;                 // group <= 32768: at most 128 KB
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ec_select),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
    }
    ec_select<<<dim3((unsigned)(p.E * ng)), dim3(kSelThreads), lds, s>>>(
        logits, p.E, group, (int)ng, (int)C, sel, rowof);
    return hipGetLastError();
}

}  // namespace moe
