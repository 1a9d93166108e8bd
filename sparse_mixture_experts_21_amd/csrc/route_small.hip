// Routing and dispatch of a tiny batch in one workgroup ("moe-training" SKILL
// page: Core Concepts, 2. Routing Mechanisms (top-k gate) and 3. Load
// Balancing (the two router losses); Quick Start, Basic MoE Architecture (the
// per-expert token gather) with the capacity rule of 4. Expert Parallelism).
//
// For T * E <= kSmallPairs (a decode step: a few tokens), the whole of what
// the router and the two dispatch kernels do is one launch:
//   1. logits l[t][e] = x[t] . Wg[:, e] (+ bg[e]) in fp32.  x and the gate
//      columns are staged in LDS (all of H at once when T + E rows of it fit
//      in 130 KB, else in blocks); with few pairs, 32 or more threads per
//      (token, expert) pair add 8-element chunks, the partial sums added in a
//      fixed order; with 32 pairs or more, 16 x 16 tiles of them on MFMA,
//      the 16 waves taking every 16th 32-wide k-step of each block, then the
//      waves' partial tiles added in wave order;
//   2. per token (one wave, a lane per expert): softmax, top-k on the logits
//      (descending, equal logits to the lower expert), the k probabilities
//      renormalised to sum to one, lse;
//   3. per expert (a lane of wave 0 each): the routed count, the kept count
//      min(count, cap), the sum of probabilities over the tokens in token
//      order; the exclusive scan of the kept counts -> offsets; the two
//      losses  aux = E sum_e (count_e / (T k)) (psum_e / T),  z = sum_t lse_t^2 / T
//      (butterfly sums over the lanes);
//   4. per expert (the same lane): its (token, slot) pairs in token order,
//      rank r -> pos = offsets[e] + r while r < cap (else -1), row_token.
// The same outputs as launch_route + launch_permute with a fused row gather,
// computed in a different (fixed) floating-point order.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kSmallThreads = 1024;
constexpr int kSmallLds = 66560;       // bf16 elements of the x / gate staging (130 KB)
constexpr int kSmallMfmaPairs = 32;    // from this many (token, expert) pairs on, MFMA logits

template <bool MFMA>
__global__ __launch_bounds__(kSmallThreads) void route_small(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wg,
    const uint16_t* __restrict__ bg, int T, int H, int E, int k, int32_t cap,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ counts, float* __restrict__ losses, int32_t* __restrict__ offsets,
    int32_t* __restrict__ pos, int32_t* __restrict__ row_token) {
    // x block [T][HB] and, after it, the gate block transposed to [E][HB], bf16,
    // rows PITCH = HB + 8 apart (so the rows of different pairs start in
    // different banks).  HB: all of H when the T + E rows fit, else blocks.
    __shared__ __attribute__((aligned(16))) uint16_t xs[kSmallLds];
    __shared__ float part[kSmallThreads / 64][kSmallPairs];
    __shared__ float lg[kSmallPairs];          // logits, then probabilities
    __shared__ float lse2[kSmallPairs];
    __shared__ int32_t sel[kSmallPairs * kMaxK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int NP = T * E;                      // (token, expert) pairs, <= kSmallPairs
    const int HB = min(H, (kSmallLds / (T + E) - 8) & ~7);
    const int PITCH = HB + 8;
    uint16_t* ws = xs + T * PITCH;
    // Fewer than kSmallMfmaPairs pairs: TP >= 32 threads per pair each add
    // 8-element chunks c = hp, hp + TP, ... of every block, then a butterfly
    // within the wave and the waves in order.  More: logit tiles of 16 tokens
    // x 16 experts on v_mfma_f32_16x16x32_bf16 (A: lane l holds 8 consecutive
    // h of token row l % 16, B: of expert column l % 16, both straight from the
    // staged rows; T * E <= 64 makes at most four tiles), the 16 waves taking
    // every 16th 32-wide k-step of each block, then their partial tiles added
    // in wave order.
    constexpr bool mfma = MFMA;              // the host picks it: NP >= kSmallMfmaPairs
    int TP = kSmallThreads;
    while (TP * NP > kSmallThreads) TP >>= 1;
    const int p = tid / TP, hp = tid % TP;     // pair p = t * E + e (p < NP when active)
    const bool active = !mfma && p < NP;
    float fac = 0.f;
    const int TT = (T + 15) / 16, ET = (E + 15) / 16, NTL = TT * ET;
    const int l16 = lane & 15, kg = lane >> 4;
    f32x4_t acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int h0 = 0; h0 < H; h0 += HB) {
        const int hb = min(HB, H - h0);        // a multiple of 8
        const int nch = hb / 8;
        if (h0) __syncthreads();               // the previous block has been read
        // x rows: 16-byte vectors, (row, chunk) pairs dealt to the threads
        // row-major (the loop is unrolled so several loads are in flight)
        {
            const int rpi = max(1, kSmallThreads / nch);          // rows per pass
            const int r0 = tid / nch, c0 = tid % nch;
            if (r0 < rpi) {
#pragma unroll 4
                for (int r = r0; r < T; r += rpi)
                    for (int c = c0; c < nch; c += kSmallThreads)
                        *reinterpret_cast<u32x4_t*>(xs + r * PITCH + 8 * c) =
                            *reinterpret_cast<const u32x4_t*>(x + (int64_t)r * H + h0 + 8 * c);
            }
        }
        // gate row h (E values) by one thread, scattered to ws[e][h]: 16-byte
        // vectors when E % 8 == 0, else element by element
#pragma unroll 4
        for (int hh = tid; hh < hb; hh += kSmallThreads) {
            const uint16_t* row = Wg + (int64_t)(h0 + hh) * E;
            if (E % 8 == 0) {
                for (int e8 = 0; e8 < E; e8 += 8) {
                    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(row + e8);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        ws[(e8 + 2 * q) * PITCH + hh] = (uint16_t)(v[q] & 0xffffu);
                        ws[(e8 + 2 * q + 1) * PITCH + hh] = (uint16_t)(v[q] >> 16);
                    }
                }
            } else {
                for (int ee = 0; ee < E; ++ee) ws[ee * PITCH + hh] = row[ee];
            }
        }
        __syncthreads();
        if (active) {
            const int t = p / E, e = p % E;
            for (int c = hp; c < nch; c += TP) {
                const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xs + t * PITCH + 8 * c);
                const u32x4_t wv = *reinterpret_cast<const u32x4_t*>(ws + e * PITCH + 8 * c);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    fac = fmaf(bf16_lo(xv[q]), bf16_lo(wv[q]), fac);
                    fac = fmaf(bf16_hi(xv[q]), bf16_hi(wv[q]), fac);
                }
            }
        }
        const int nks = mfma ? (hb + 31) / 32 : 0;
        for (int ks = wave; ks < nks; ks += kSmallThreads / 64) {
            const int kc = ks * 32 + kg * 8;              // this lane's 8 h of the block
            const bool kin = kc < hb;                     // hb % 8 == 0: all 8 or none
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q >= NTL) break;                      // uniform
                const int tr = (q / ET) * 16 + l16, er = (q % ET) * 16 + l16;
                const u32x4_t z = {0u, 0u, 0u, 0u};
                const u32x4_t av =
                    (kin && tr < T) ? *reinterpret_cast<const u32x4_t*>(xs + tr * PITCH + kc) : z;
                const u32x4_t bv =
                    (kin && er < E) ? *reinterpret_cast<const u32x4_t*>(ws + er * PITCH + kc) : z;
                acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv), acc[q],
                    0, 0, 0);
            }
        }
    }
    if (!mfma) {
        // the pair's TP partials: butterfly over min(TP, 64) lanes, then waves in order
        const int TW = min(TP, 64);
        for (int d = TW >> 1; d >= 1; d >>= 1) fac += __shfl_xor(fac, d);
        if (active && (lane % TW) == 0) part[wave][p] = fac;   // one value per (wave, pair)
    } else {
        // each wave's partial of every pair (lane l holds tokens 4 (l / 16) + i
        // of expert column l % 16 of each tile)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q >= NTL) break;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tq = (q / ET) * 16 + 4 * kg + i, eq = (q % ET) * 16 + l16;
                if (tq < T && eq < E) part[wave][tq * E + eq] = acc[q][i];
            }
        }
    }
    __syncthreads();
    if (tid < NP) {
        // the waves that hold the pair's partials, in order
        const int w0 = mfma ? 0 : tid * TP / 64;
        const int nw = mfma ? kSmallThreads / 64 : (TP > 64 ? TP / 64 : 1);
        float sum = part[w0][tid];
        for (int w = 1; w < nw; ++w) sum += part[w0 + w][tid];
        if (bg) sum += bf16_lo((uint32_t)bg[tid % E]);
        lg[tid] = sum;
        if (logits) logits[tid] = sum;
    }
    __syncthreads();
    // per token (wave w takes tokens w, w + 16, ...; lane q = expert q):
    // softmax, top-k on the logits (descending, equal logits to the lower
    // expert), renormalised weights, lse^2; the probabilities replace the logits
    for (int tt = wave; tt < T; tt += kSmallThreads / 64) {
        const bool in = lane < E;
        const float l = in ? lg[tt * E + lane] : -INFINITY;
        float m = l;
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
        const float ex = in ? expf(l - m) : 0.f;
        float Z = ex;
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) Z += __shfl_xor(Z, d);
        bool taken = !in;
        float S = 0.f;
        int sv = -1;              // lane s < k: the s-th choice
        float pvs = 0.f;
        for (int s = 0; s < k; ++s) {
            // the largest logit not yet taken; ties to the lower expert
            float bv = taken ? -INFINITY : l;
            int bi = taken ? 0x7fffffff : lane;
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) {
                const float ov = __shfl_xor(bv, d);
                const int oi = __shfl_xor(bi, d);
                if (ov > bv || (ov == bv && oi < bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (lane == bi) taken = true;
            const float pv = expf(bv - m) / Z;
            S += pv;
            if (lane == s) {
                sv = bi;
                pvs = pv;
            }
        }
        if (lane < k) {
            topk_idx[tt * k + lane] = sv;
            topk_w[tt * k + lane] = pvs / S;
            sel[tt * k + lane] = sv;
        }
        if (lane == 0) {
            const float lse = m + logf(Z);
            lse2[tt] = lse * lse;
        }
        if (in) lg[tt * E + lane] = ex / Z;
    }
    __syncthreads();
    // wave 0, lane e: routed and kept counts, probability sums in token order,
    // the exclusive scan of kept counts -> offsets, the losses; then the ranks
    if (wave == 0) {
        const bool in = lane < E;
        int c = 0;
        float ps = 0.f;
        if (in) {
            for (int tt = 0; tt < T; ++tt) {
                ps += lg[tt * E + lane];
                for (int s = 0; s < k; ++s) c += sel[tt * k + s] == lane;
            }
            counts[lane] = c;
        }
        const int kept = in ? min(c, cap) : 0;
        int incl = kept;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(incl, d);
            if (lane >= d) incl += u;
        }
        const int o = incl - kept;
        if (in) offsets[lane] = o;
        if (lane == 63) offsets[E] = incl;
        // aux = E sum_e (c_e / (T k)) (psum_e / T); z = sum_t lse_t^2 / T
        float a = (float)c * ps;
        float zz = lane < T ? lse2[lane] : 0.f;
        for (int tt = 64 + lane; tt < T; tt += 64) zz += lse2[tt];
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            a += __shfl_xor(a, d);
            zz += __shfl_xor(zz, d);
        }
        if (lane == 0 && losses) {
            losses[0] = (float)E * a / ((float)T * (float)T * (float)k);
            losses[1] = zz / (float)T;
        }
        if (in) {
            int r = 0;
            for (int j = 0; j < T * k; ++j) {
                if (sel[j] != lane) continue;
                if (r < cap) {
                    pos[j] = o + r;
                    row_token[o + r] = j / k;
                } else {
                    pos[j] = -1;
                }
                ++r;
            }
        }
    }
}

}  // namespace

bool route_small_fits(const moe_problem_t& p) {
    return p.dtype == MOE_DTYPE_BF16 && p.T * (int64_t)p.E <= kSmallPairs && p.k <= kMaxK;
}

hipError_t launch_route_small(const moe_problem_t& p, int64_t cap, const void* x, const void* Wg,
                              const void* bg, float* logits, int32_t* topk_idx, float* topk_w,
                              int32_t* counts, float* losses, int32_t* offsets, int32_t* pos,
                              int32_t* row_token, hipStream_t s) {
    const int32_t c = (int32_t)std::min<int64_t>(cap, INT32_MAX);
    auto* xb = static_cast<const uint16_t*>(x);
    auto* wb = static_cast<const uint16_t*>(Wg);
    auto* bb = static_cast<const uint16_t*>(bg);
    if (p.T * (int64_t)p.E >= kSmallMfmaPairs)
        route_small<true><<<dim3(1), dim3(kSmallThreads), 0, s>>>(
            xb, wb, bb, (int)p.T, p.H, p.E, p.k, c, logits, topk_idx, topk_w, counts, losses,
            offsets, pos, row_token);
    else
        route_small<false><<<dim3(1), dim3(kSmallThreads), 0, s>>>(
            xb, wb, bb, (int)p.T, p.H, p.E, p.k, c, logits, topk_idx, topk_w, counts, losses,
            offsets, pos, row_token);
    return hipGetLastError();
}

}  // namespace moe
