// Weighted combine back to token order ("moe-training" SKILL page, Quick
// Start, Basic MoE Architecture: the output starts at zero and each selected
// expert's output, scaled by its renormalised score, is added to the token's
// row).  Token-major gather instead of a scatter-add: every output element is
// produced by exactly one thread, summed in fp32 in slot order and rounded
// once, so there are no atomics and results are bitwise reproducible.
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

#ifndef MOE_COMBINE_NT
#define MOE_COMBINE_NT 1
#endif
// y is read once and out written once: nontemporal, so neither allocates in
// (nor first has to write back dirty lines of) the last-level cache.
template <typename V>
__device__ __forceinline__ V ld_stream(const V* p) {
    return MOE_COMBINE_NT ? __builtin_nontemporal_load(p) : *p;
}
template <typename V>
__device__ __forceinline__ void st_stream(V* p, V v) {
    if (MOE_COMBINE_NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// TPT threads (1 to 4 waves) per token row, sized to the row so that a row
// of up to TPT * kCombVec 16-byte vectors (8 bf16 or 4 fp32 each) goes in one
// pass and narrow rows do not leave most of a workgroup idle; a workgroup
// holds 256 / TPT tokens.  The token's (row, weight) pairs are uniform over
// its threads and taken kMaxK slots at a time (one chunk for top-k routing;
// expert choice passes one slot per expert); every kept slot's vectors of a
// chunk are loaded before they are added, in fp32 and in slot order, and the
// sum is rounded once.
constexpr int kCombThreads = 256;
constexpr int kCombVec = 2;

template <bool BF16, int TPT>
__global__ __launch_bounds__(kCombThreads) void combine_rows(const u32x4_t* __restrict__ y,
                                                             const int32_t* __restrict__ pos,
                                                             const float* __restrict__ topk_w,
                                                             int k, int64_t T, int64_t vec,
                                                             u32x4_t* __restrict__ out) {
    const int lane = threadIdx.x % TPT;
    const int64_t t = (int64_t)blockIdx.x * (kCombThreads / TPT) + threadIdx.x / TPT;
    if (t >= T) return;                                   // whole waves
    for (int64_t v0 = lane; v0 < vec; v0 += TPT * kCombVec) {
        float acc[kCombVec][8];
#pragma unroll
        for (int u = 0; u < kCombVec; ++u)
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[u][q] = 0.f;
        for (int s0 = 0; s0 < k; s0 += kMaxK) {
            int32_t row[kMaxK];
            float w[kMaxK];
#pragma unroll
            for (int s = 0; s < kMaxK; ++s) {
                row[s] = s0 + s < k ? pos[t * k + s0 + s] : -1;
                w[s] = s0 + s < k ? topk_w[t * k + s0 + s] : 0.f;
            }
            u32x4_t d[kMaxK][kCombVec];
#pragma unroll
            for (int s = 0; s < kMaxK; ++s) {
                if (row[s] < 0) continue;              // uniform: no divergence
#pragma unroll
                for (int u = 0; u < kCombVec; ++u) {
                    const int64_t v = v0 + (int64_t)u * TPT;
                    if (v < vec) d[s][u] = ld_stream(&y[(int64_t)row[s] * vec + v]);
                }
            }
#pragma unroll
            for (int u = 0; u < kCombVec; ++u) {
#pragma unroll
                for (int s = 0; s < kMaxK; ++s) {
                    if (row[s] < 0) continue;
                    if (BF16) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            acc[u][2 * q] = fmaf(w[s], bf16_lo(d[s][u][q]), acc[u][2 * q]);
                            acc[u][2 * q + 1] = fmaf(w[s], bf16_hi(d[s][u][q]), acc[u][2 * q + 1]);
                        }
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[u][q] = fmaf(w[s], __uint_as_float(d[s][u][q]), acc[u][q]);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kCombVec; ++u) {
            const int64_t v = v0 + (int64_t)u * TPT;
            if (v >= vec) continue;
            u32x4_t o;
            if (BF16) {
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[u][2 * q], acc[u][2 * q + 1]);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[u][q]);
            }
            st_stream(&out[t * vec + v], o);
        }
    }
}

template <bool BF16>
hipError_t launch_rows(const moe_problem_t& p, const void* y, const int32_t* pos,
                       const float* topk_w, void* out, int64_t vec, hipStream_t s) {
    auto* yv = static_cast<const u32x4_t*>(y);
    auto* ov = static_cast<u32x4_t*>(out);
    auto go = [&](auto tpt) {
        constexpr int TPT = decltype(tpt)::value;
        const unsigned nb = (unsigned)((p.T + (kCombThreads / TPT) - 1) / (kCombThreads / TPT));
        combine_rows<BF16, TPT><<<dim3(nb), dim3(kCombThreads), 0, s>>>(yv, pos, topk_w, p.k, p.T,
                                                                         vec, ov);
    };
    if (vec > 128 * kCombVec) go(std::integral_constant<int, 256>{});
    else if (vec > 64 * kCombVec) go(std::integral_constant<int, 128>{});
    else go(std::integral_constant<int, 64>{});
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const moe_problem_t& p, const void* y, const int32_t* pos,
                          const float* topk_w, void* out, hipStream_t s) {
    const bool bf16 = p.dtype == MOE_DTYPE_BF16;
    const int64_t vec = (int64_t)p.H * (bf16 ? 2 : 4) / 16;
    return bf16 ? launch_rows<true>(p, y, pos, topk_w, out, vec, s)
                : launch_rows<false>(p, y, pos, topk_w, out, vec, s);
}

}  // namespace moe
