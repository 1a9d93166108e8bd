// Weighted combine back to token order ("moe-training" SKILL page, Quick
// Start, Basic MoE Architecture: the output starts at zero and each selected
// expert's output, scaled by its renormalised score, is added to the token's
// row).  Token-major gather instead of a scatter-add: every output element is
// produced by exactly one thread, summed in fp32 in slot order and rounded
// once, so there are no atomics and results are bitwise reproducible.
#include <type_traits>

#include "moe_internal.h"
#include "gemm_common.h"

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

// The combine of a top-k forward whose second GEMM left its cut last round as
// K-slice partials (launch_ffn_down with fixup = false), so that the forward
// needs no fixup launch for it.  Row r of expert e lies in row tile
// tb[e] + (r - offsets[e]) / BM; with the 256-column tile of a vector, the
// launch's tile order (dense_position) tells whether that tile was cut, and
// which of the tail tiles it is.  Such a vector is finished from its S slices
// exactly as ffn_gemm_fixup finishes it (slices summed in order, then + b2,
// one rounding to bf16), so the output equals the unfused combine's bit for
// bit; every other vector is read from y.  Per token as combine_rows (k <=
// kMaxK slots): every kept slot's vectors loaded first, then summed in slot
// order in fp32.  The token's slot entries are loaded before the workgroup's
// tile counts are reduced, so the two round trips overlap.  KM >= k slots are
// held in registers (2 for top-1 and top-2, else kMaxK), which keeps the
// kernel at several waves per SIMD.  CV vectors per thread and pass; a token
// row may span TPT / 256 workgroups (a few tokens: one vector per thread, so
// that the slices of the whole row are loaded by many threads at once).
// A cut vector's first slice and the next BATCH ones are loaded together.
template <int BM, int KM, int TPT, int CV>
__global__ __launch_bounds__(kCombThreads) void combine_rows_cut(
    const u32x4_t* __restrict__ y, const int32_t* __restrict__ pos,
    const float* __restrict__ topk_w, const int32_t* __restrict__ topk_idx, int k, int64_t T,
    int64_t vec, u32x4_t* __restrict__ out, const int32_t* __restrict__ offsets, int E,
    const uint16_t* __restrict__ bias, const float* __restrict__ part, GemmCut gc) {
    constexpr int UNIT = BM * 256;                        // floats of one partial tile
    constexpr int BATCH = CV == 1 ? 8 : 4;                // slice loads in flight
    constexpr int WPT = TPT > kCombThreads ? TPT / kCombThreads : 1;   // workgroups per token
    __shared__ int tb[kMaxE];                             // row tiles of the experts before e
    __shared__ int ofs[kMaxE];                            // the experts' first rows
    __shared__ int s_real_mt;
    const int lane = WPT > 1 ? (int)(blockIdx.x % WPT) * kCombThreads + (int)threadIdx.x
                             : (int)threadIdx.x % TPT;
    const int64_t t = WPT > 1 ? (int64_t)(blockIdx.x / WPT)
                              : (int64_t)blockIdx.x * (kCombThreads / TPT) + threadIdx.x / TPT;
    const bool live = t < T;
    int32_t row[KM], ex[KM];
    float w[KM];
#pragma unroll
    for (int s = 0; s < KM; ++s) {
        row[s] = live && s < k ? pos[t * k + s] : -1;
        w[s] = live && s < k ? topk_w[t * k + s] : 0.f;
        ex[s] = live && s < k ? topk_idx[t * k + s] : 0;
    }
    if (threadIdx.x < 64) {
        const int ln = threadIdx.x;
        int base = 0;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + ln;
            const int b = e < E ? offsets[e] : 0;
            const int tiles = e < E ? (offsets[e + 1] - b + BM - 1) / BM : 0;
            int incl = tiles;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int v = __shfl_up(incl, d);
                if (ln >= d) incl += v;
            }
            if (e < E) {
                tb[e] = base + incl - tiles;
                ofs[e] = b;
            }
            base += __shfl(incl, 63);
        }
        if (ln == 0) s_real_mt = base;
    }
    __syncthreads();
    if (!live) return;                                    // whole waves
    const TailPlan pl = plan_tail(s_real_mt, gc.Nt, gc.ncu, gc.nk, gc.ns, true);
    const int lg = gc.SBN == 16 ? 4 : gc.SBN == 8 ? 3 : 2;
    int32_t mt[KM], m[KM];
#pragma unroll
    for (int s = 0; s < KM; ++s) {
        mt[s] = m[s] = 0;
        if (row[s] >= 0 && pl.S > 1) {
            const int lr = row[s] - ofs[ex[s]];
            mt[s] = lr / BM;
            m[s] = lr - mt[s] * BM;
            mt[s] += tb[ex[s]];
        }
    }
    const int64_t H = vec * 8;
    for (int64_t v0 = lane; v0 < vec; v0 += TPT * CV) {
        float acc[CV][8];
#pragma unroll
        for (int u = 0; u < CV; ++u)
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[u][q] = 0.f;
        // float offset of the vector's first slice in part, or -1: read y
        int32_t cut[KM][CV];
        u32x4_t d[KM][CV];
#pragma unroll
        for (int s = 0; s < KM; ++s) {
            if (row[s] < 0) continue;                     // uniform: no divergence
#pragma unroll
            for (int u = 0; u < CV; ++u) {
                const int64_t v = v0 + (int64_t)u * TPT;
                cut[s][u] = -1;
                if (v >= vec) continue;
                if (pl.S > 1) {
                    const int p = dense_position(mt[s], (int)(v >> 5), pl.real_mt, gc.Nt, lg);
                    if (p >= pl.full)
                        cut[s][u] = (p - pl.full) * pl.S * UNIT + m[s] * 256 + 8 * (int)(v & 31);
                }
                if (cut[s][u] < 0) d[s][u] = ld_stream(&y[(int64_t)row[s] * vec + v]);
            }
        }
#pragma unroll
        for (int s = 0; s < KM; ++s) {
            if (row[s] < 0) continue;
#pragma unroll
            for (int u = 0; u < CV; ++u) {
                if (cut[s][u] < 0) continue;
                const float* src = part + cut[s][u];
                f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(src);
                f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(src + 4);
                for (int sb = 1; sb < pl.S; sb += BATCH) {
                    // (independent of slice 0's loads, so both are in flight together)
                    // unconditional loads at clamped slice indices, masked in the sum
                    f32x4_t t0[BATCH], t1[BATCH];
#pragma unroll
                    for (int b = 0; b < BATCH; ++b) {
                        const float* q = src + (int64_t)min(sb + b, pl.S - 1) * UNIT;
                        t0[b] = *reinterpret_cast<const f32x4_t*>(q);
                        t1[b] = *reinterpret_cast<const f32x4_t*>(q + 4);
                    }
#pragma unroll
                    for (int b = 0; b < BATCH; ++b) {
                        if (sb + b < pl.S) {
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                a0[q] += t0[b][q];
                                a1[q] += t1[b][q];
                            }
                        }
                    }
                }
                float bv[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) bv[q] = 0.f;
                if (bias) {
                    const int64_t c = (v0 + (int64_t)u * TPT) << 3;
                    const u32x4_t bb =
                        *reinterpret_cast<const u32x4_t*>(bias + (int64_t)ex[s] * H + c);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        bv[2 * q] = bf16_lo(bb[q]);
                        bv[2 * q + 1] = bf16_hi(bb[q]);
                    }
                }
                d[s][u] = u32x4_t{pack_bf16x2(a0[0] + bv[0], a0[1] + bv[1]),
                                  pack_bf16x2(a0[2] + bv[2], a0[3] + bv[3]),
                                  pack_bf16x2(a1[0] + bv[4], a1[1] + bv[5]),
                                  pack_bf16x2(a1[2] + bv[6], a1[3] + bv[7])};
            }
        }
#pragma unroll
        for (int u = 0; u < CV; ++u) {
            const int64_t v = v0 + (int64_t)u * TPT;
            if (v >= vec) continue;
#pragma unroll
            for (int s = 0; s < KM; ++s) {
                if (row[s] < 0) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[u][2 * q] = fmaf(w[s], bf16_lo(d[s][u][q]), acc[u][2 * q]);
                    acc[u][2 * q + 1] = fmaf(w[s], bf16_hi(d[s][u][q]), acc[u][2 * q + 1]);
                }
            }
            u32x4_t o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[u][2 * q], acc[u][2 * q + 1]);
            st_stream(&out[t * vec + v], o);
        }
    }
}

}  // namespace

hipError_t launch_combine_cut(const moe_problem_t& p, const void* y, const int32_t* pos,
                              const float* topk_w, const int32_t* topk_idx,
                              const int32_t* offsets, const void* b2, const float* part,
                              void* out, hipStream_t s) {
    const GemmCut gc = down_gemm_cut(p);
    const int64_t vec = (int64_t)p.H * 2 / 16;
    auto* yv = static_cast<const u32x4_t*>(y);
    auto* ov = static_cast<u32x4_t*>(out);
    auto* bb = static_cast<const uint16_t*>(b2);
    auto go = [&](auto bm, auto km, auto tpt, auto cv) {
        constexpr int BM = decltype(bm)::value, KM = decltype(km)::value;
        constexpr int TPT = decltype(tpt)::value, CV = decltype(cv)::value;
        const unsigned nb = TPT > kCombThreads
            ? (unsigned)(p.T * (TPT / kCombThreads))
            : (unsigned)((p.T + (kCombThreads / TPT) - 1) / (kCombThreads / TPT));
        combine_rows_cut<BM, KM, TPT, CV><<<dim3(nb), dim3(kCombThreads), 0, s>>>(
            yv, pos, topk_w, topk_idx, p.k, p.T, vec, ov, offsets, p.E, bb, part, gc);
    };
    using I = std::integral_constant<int, 1>;
    using II = std::integral_constant<int, kCombVec>;
    auto pick_tpt = [&](auto bm, auto km) {
        if (p.T < kCombineCutWideBelow) {
            // a few tokens: one vector per thread, the row over up to 4 workgroups
            if (vec > 512) go(bm, km, std::integral_constant<int, 1024>{}, I{});
            else if (vec > 256) go(bm, km, std::integral_constant<int, 512>{}, I{});
            else if (vec > 128) go(bm, km, std::integral_constant<int, 256>{}, I{});
            else go(bm, km, std::integral_constant<int, 128>{}, I{});
        } else if (vec > 128 * kCombVec) go(bm, km, std::integral_constant<int, 256>{}, II{});
        else if (vec > 64 * kCombVec) go(bm, km, std::integral_constant<int, 128>{}, II{});
        else go(bm, km, std::integral_constant<int, 64>{}, II{});
    };
    auto pick_km = [&](auto bm) {
        if (p.k <= 2) pick_tpt(bm, std::integral_constant<int, 2>{});
        else pick_tpt(bm, std::integral_constant<int, kMaxK>{});
    };
    if (gc.bm == 256) pick_km(std::integral_constant<int, 256>{});
    else if (gc.bm == 128) pick_km(std::integral_constant<int, 128>{});
    else pick_km(std::integral_constant<int, 64>{});
    return hipGetLastError();
}

hipError_t launch_combine(const moe_problem_t& p, const void* y, const int32_t* pos,
                          const float* topk_w, void* out, hipStream_t s) {
    const bool bf16 = p.dtype == MOE_DTYPE_BF16;
    const int64_t vec = (int64_t)p.H * (bf16 ? 2 : 4) / 16;
    return bf16 ? launch_rows<true>(p, y, pos, topk_w, out, vec, s)
                : launch_rows<false>(p, y, pos, topk_w, out, vec, s);
}

}  // namespace moe
