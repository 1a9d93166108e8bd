// Reduction of the router's per-block partials to the expert counts and the
// two router losses ("moe-training" SKILL page, Core Concepts, 3. Load
// Balancing):
//   aux = E * sum_e (counts_e / (T k)) * (psum_e / T),   z = sum_t lse_t^2 / T.
// Each column (expert e, or e == E for the lse^2 partials) is summed by one
// 256-thread workgroup, so the columns are read by many CUs at once: thread t
// adds blocks 4t .. 4t + 3 of each round of 1024 in order in fp64, then a
// butterfly over the wave and the 4 wave sums in order.  The order is fixed,
// so the losses are bitwise reproducible without floating-point atomics.  The
// column sums go to the workspace; one wave then forms the losses.  Used by
// the router's own finalize kernels and, inside the fused forward, by the
// dispatch scan and rank kernels.
#pragma once

#include "moe_internal.h"

namespace moe {

constexpr int kColThreads = 256;      // threads of a column workgroup
constexpr int kColPer = 4;            // consecutive elements per thread and round

struct FinArgs {
    const float* psum;     // [E][nblk] per-block sums of softmax probabilities
    const float* lse2;     // [nblk]    per-block sums of lse^2
    const int32_t* cnt;    // [E][nblk] per-block expert histograms
    int64_t nblk;
    int64_t T;
    int k;
    double* col_sum;       // [E + 1] workspace: column sums
    long long* col_cnt;    // [E]     workspace: expert counts
    int32_t* counts;       // [E] out
    float* losses;         // [2] out: aux, z
};

// Column c (0 <= c <= E) summed by the calling kColThreads-thread workgroup.
__device__ inline void fin_column_block(const FinArgs& f, int E, int c) {
    __shared__ double wsum[kColThreads / 64];
    __shared__ long long wcnt[kColThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* pv = c < E ? f.psum + (int64_t)c * f.nblk : f.lse2;
    const int32_t* pc = f.cnt + (int64_t)(c < E ? c : 0) * f.nblk;
    const int64_t n = f.nblk;
    double a = 0.0;
    long long m = 0;
    for (int64_t j0 = (int64_t)tid * kColPer; j0 < n; j0 += kColThreads * kColPer) {
        // unconditional loads at clamped indices (a predicated load would be
        // compiled into a branch and a wait per element), masked afterwards
        float v[kColPer];
        int32_t q[kColPer];
#pragma unroll
        for (int i = 0; i < kColPer; ++i) {
            const int64_t j = j0 + i < n ? j0 + i : n - 1;
            v[i] = pv[j];
            q[i] = pc[j];
        }
#pragma unroll
        for (int i = 0; i < kColPer; ++i) {
            if (j0 + i < n) {
                a += (double)v[i];
                if (c < E) m += q[i];
            }
        }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        a += __shfl_xor(a, d);
        m += __shfl_xor(m, d);
    }
    if (lane == 0) {
        wsum[wave] = a;
        wcnt[wave] = m;
    }
    __syncthreads();
    if (tid == 0) {
        double s = wsum[0];
        long long t = wcnt[0];
        for (int w = 1; w < kColThreads / 64; ++w) {
            s += wsum[w];
            t += wcnt[w];
        }
        f.col_sum[c] = s;
        if (c < E) f.col_cnt[c] = t;
    }
}

// One whole wave (64 lanes, all calling), once every column sum is in the
// workspace: lane l takes experts l, l + 64, ... (E <= 256), all loads issued
// together, its terms added in expert order, then a butterfly over the wave
// (each level adds the same two operands on both lanes, so every lane ends
// with the same bits); lane 0 writes the losses.
__device__ inline void fin_losses(const FinArgs& f, int E) {
    const int lane = threadIdx.x & 63;
    long long cnt[4];
    double sum[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {                 // unconditional loads at clamped indices
        const int e = min(lane + 64 * i, E - 1);
        cnt[i] = f.col_cnt[e];
        sum[i] = f.col_sum[e];
    }
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
            f.counts[e] = (int32_t)cnt[i];
            acc += ((double)cnt[i] / (double)(f.T * f.k)) * (sum[i] / (double)f.T);
        }
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) acc += __shfl_xor(acc, d);
    if (lane == 0) {
        f.losses[0] = (float)((double)E * acc);
        f.losses[1] = (float)(f.col_sum[E] / (double)f.T);
    }
}

}  // namespace moe
