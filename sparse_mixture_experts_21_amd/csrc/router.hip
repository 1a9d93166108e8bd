// Router: gate linear, softmax over experts, top-k, renormalisation of the k
// selected scores, and per-block partial sums for the load-balancing loss and
// the router z-loss ("moe-training" SKILL page, Quick Start, Basic MoE
// Architecture; Core Concepts, 3. Load Balancing).
//
// bf16: route_bf16 (below) streams x and the gate through LDS and computes the
// gate tile of TM tokens on MFMA, then the routing epilogue.  fp32: plain FMA
// dot products and a 4-lanes-per-token epilogue.  Per-block partials (sum of
// softmax probabilities per expert, sum of lse^2, expert histogram, per 16
// tokens) are reduced in a fixed order by one workgroup per column, so the
// losses are bitwise reproducible without floating-point atomics.
#include "moe_internal.h"
#include "lds_dma.h"
#include "route_finalize.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

// ---------------------------------------------------------------- routing epilogue
// logit_s: [16][E] fp32 logits of the block's tokens (bias already added).
// Wave 0 runs 4 lanes per token; lanes q = 0..3 of a token own experts
// e = q, q+4, q+8, ...  The probabilities overwrite logit_s.
struct RouteOut {
    int32_t* topk_idx;
    float* topk_w;
    float* blk_psum;
    float* blk_lse2;
    int32_t* blk_cnt;
};

__device__ void route_epilogue(float* logit_s, int32_t* idx_s, float* lse_s, int64_t t0,
                               int64_t T, int E, int k, const RouteOut& o) {
    const int tid = threadIdx.x;
    if (tid < 64) {
        const int r = tid >> 2, q = tid & 3;
        const bool valid = (t0 + r) < T;
        float* lr = logit_s + r * E;
        // row maximum
        float m = -INFINITY;
        for (int e = q; e < E; e += 4) m = fmaxf(m, lr[e]);
        m = fmaxf(m, __shfl_xor(m, 1));
        m = fmaxf(m, __shfl_xor(m, 2));
        float Z = 0.f;
        for (int e = q; e < E; e += 4) Z += expf(lr[e] - m);
        // fixed pairing order: (q0+q1) + (q2+q3), identical on all four lanes
        Z += __shfl_xor(Z, 1);
        Z += __shfl_xor(Z, 2);
        // top-k on the logits: descending, equal values -> lower expert index
        uint64_t taken = 0;     // bit j <=> expert q + 4 j taken
        int sel[kMaxK];
        float pv[kMaxK];
        for (int s = 0; s < k; ++s) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            int j = 0;
            for (int e = q; e < E; e += 4, ++j) {
                if ((taken >> j) & 1ull) continue;
                float v = lr[e];
                if (bi == 0x7fffffff || v > bv) { bv = v; bi = e; }
            }
#pragma unroll
            for (int d = 1; d <= 2; d <<= 1) {
                float ov = __shfl_xor(bv, d);
                int oi = __shfl_xor(bi, d);
                if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) {
                    bv = ov;
                    bi = oi;
                }
            }
            sel[s] = bi;
            pv[s] = expf(bv - m) / Z;
            if ((bi & 3) == q) taken |= 1ull << (bi >> 2);
        }
        // probabilities of all experts (needed by the load-balancing loss)
        for (int e = q; e < E; e += 4) lr[e] = valid ? expf(lr[e] - m) / Z : 0.f;
        if (q == 0) {
            float S = 0.f;
            for (int s = 0; s < k; ++s) S += pv[s];
            for (int s = 0; s < k; ++s) {
                idx_s[r * kMaxK + s] = valid ? sel[s] : -1;
                if (valid) {
                    o.topk_idx[(t0 + r) * k + s] = sel[s];
                    o.topk_w[(t0 + r) * k + s] = pv[s] / S;
                }
            }
            float lse = m + logf(Z);
            lse_s[r] = valid ? lse * lse : 0.f;
        }
    }
    __syncthreads();
    const int64_t blk = blockIdx.x, nblk = gridDim.x;
    for (int e = tid; e < E; e += kThreads) {
        float ps = 0.f;
        int c = 0;
        for (int r = 0; r < kRouteTok; ++r) {
            ps += logit_s[r * E + e];
            for (int s = 0; s < k; ++s) c += (idx_s[r * kMaxK + s] == e);
        }
        o.blk_psum[e * nblk + blk] = ps;        // column-major: [E][nblk]
        o.blk_cnt[e * nblk + blk] = c;
    }
    if (tid == 0) {
        float a = 0.f;
        for (int r = 0; r < kRouteTok; ++r) a += lse_s[r];
        o.blk_lse2[blk] = a;
    }
}

// ---------------------------------------------------------------- bf16 router
// One workgroup (4 waves) owns TM consecutive tokens and computes their gate
// tile [TM][E] = x[TM][H] . Wg[H][E] on v_mfma_f32_16x16x32_bf16 (A = 16 token
// rows, B = 16 experts, 32 hidden units per k-step), streaming x and the gate
// through a ring of NS LDS stages of BK hidden units by direct DMA (1 KB per
// wave instruction, x nontemporal: it is read once, and a plain load would
// first write back the dirty lines earlier kernels left in the last-level
// cache).  x rows keep whole contiguous row segments per DMA; the gate slab
// Wg[h0 .. h0 + BK)[0 .. E) is contiguous in the [H][E] layout, so neither
// needs a copy.  In LDS, 16-byte chunk c of token row r sits at slot
// c ^ f(r) (f below), so the 16 rows of an A fragment hit 16 distinct bank
// slots.  A B fragment (8 consecutive h of one expert per lane) comes from
// the slab with two transposing reads (ds_read_b64_tr_b16: in each 16-lane
// group, source lane s reads 4 experts of row h0 + s / 4 and lane i receives
// rows h0 .. h0 + 3 of expert i) when E % 4 == 0 (8-byte aligned rows), else
// from eight 16-bit reads.
//
// Work split: with E <= 64 the waves split each stage's k-steps (every wave
// accumulates the whole [TM][E] tile over its own k-steps) and the four
// partial tiles are added in the fixed order ((w0 + w1) + w2) + w3; with
// wider gates each wave owns every fourth 16-expert tile over all k-steps.
//
// Routing epilogue.  E <= 16 (16 tokens per workgroup): one thread per
// (token, expert), the 16 lanes of a token an aligned group: max and softmax
// sum by butterflies (the same operands on every lane of the group), top-k
// slot = the expert's rank among the token's logits (descending, equal
// logits -> lower expert).  Wider gates: LPT = 256 / TM lanes per token, lane
// q taking experts q, q + LPT, ..., top-k by k passes of a first-maximum
// argmax over the untaken experts.  Both renormalise the k selected
// probabilities.  Per 16-token block (the dispatch chunk): the sums of
// softmax probabilities and the expert counts (tokens in a fixed order) and
// the sum of lse^2, column-major [E][nblk], for the fixed-order loss
// reduction.
// EB: 16-expert tiles (E <= 16 EB); TM tokens per workgroup; BK hidden units
// per stage; NS stages; WE gate columns reserved per stage (E <= WE); SE:
// waves own expert tiles (else they split the k-steps).
template <int EB, int TM_, int BK_, int NS_, int WE, bool SE>
struct RouteCfg {
    static constexpr bool kSplitE = SE;
    static constexpr int TM = TM_;
    static constexpr int BK = BK_;
    static constexpr int NS = NS_;
    static constexpr int E16 = 16 * EB;
    static constexpr int P = BK * 2;                      // bytes of a token row per stage
    static constexpr int CPR = P / 16;                    // 16-byte chunks per row
    static constexpr int XU = TM * P / 1024;              // 1 KB DMAs for the token rows
    static constexpr int WUMAX = (BK * WE * 2 + 1023) / 1024;    // ... for the gate slab
    static constexpr int ND = (XU + WUMAX + 3) / 4;       // DMAs per wave per stage
    static constexpr int STAGE = (XU + WUMAX) * 1024;
    static constexpr int KS = BK / 32;                    // k-steps per stage
    static constexpr int KW = kSplitE ? KS : KS / 4;      // k-steps per wave per stage
    static constexpr int TT = TM / 16;                    // token tiles
    static constexpr int ET = kSplitE ? EB / 4 : EB;      // expert tiles per wave
    static constexpr int LPT = 256 / TM;                  // epilogue lanes per token
    static constexpr bool kLane16 = EB == 1 && TM == 16;  // one lane per (token, expert)
    // epilogue LDS: split-K partial tiles [4][TM][E16] (or none), logits
    // [TM][E16], selection flags [TM][E16], lse^2 [TM]
    static constexpr int RED = kSplitE ? 0 : 4 * TM * E16 * 4;
    static constexpr int EPI = RED + TM * E16 * 4 + TM * E16 + TM * 4;
    static constexpr int RING = NS * STAGE + 1024;        // + a sink for padding DMAs
    static constexpr int LDS = RING > EPI ? RING : EPI;
    static_assert(TM * P % 1024 == 0 && 1024 % P == 0, "whole rows per DMA");
    static_assert(kSplitE ? (EB % 4 == 0) : (KS % 4 == 0), "work split");
    static_assert(TM == 16 || TM == 32 || TM == 64, "epilogue lane groups");
    static_assert(WE >= 16 * EB - 15 && WE <= 16 * EB, "gate columns");
};

typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// swizzle of token row r: 16 consecutive rows land on 16 distinct bank slots
template <int CPR>
__device__ __forceinline__ int row_swz(int r) {
    if constexpr (CPR >= 16) return r & 15;
    else if constexpr (CPR == 8) return (r >> 1) & 7;
    else return (r >> 2) & 3;
}

template <int EB, int TM_, int BK_, int NS_, int WE, bool SE>
__global__ __launch_bounds__(kThreads) void route_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wg,
    const uint16_t* __restrict__ bg, float* __restrict__ logits_io, int logits_in, int64_t T,
    int H, int E, int k, RouteOut o) {
    using C = RouteCfg<EB, TM_, BK_, NS_, WE, SE>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t t0 = (int64_t)blockIdx.x * C::TM;
    const int ntok = (T - t0 < C::TM) ? (int)(T - t0) : C::TM;
    float* red = reinterpret_cast<float*>(lds);                      // [4][TM][E16]
    float* lg = reinterpret_cast<float*>(lds + C::RED);              // [TM][E16]
    uint8_t* flag = lds + C::RED + C::TM * C::E16 * 4;               // [TM][E16]
    float* lse_s = reinterpret_cast<float*>(flag + C::TM * C::E16);  // [TM]
    const int row = lane & 15, g = lane >> 4;

    if (!logits_in) {
        const uint32_t ring0 = (uint32_t)(uintptr_t)lds;
        const __amdgpu_buffer_rsrc_t xr =
            make_rsrc(uniform_ptr(x + t0 * H), (uint32_t)ntok * (uint32_t)H * 2u);
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(uniform_ptr(Wg), (uint32_t)(E * H * 2));
        const int nst = (H + C::BK - 1) / C::BK;
        const int wu = (C::BK * E * 2 + 1023) / 1024;            // gate DMAs actually needed
        // DMA q of this wave fills 1 KB unit j = wave + 4 q of the stage: the
        // token rows first, then the gate slab; units past XU + wu go to the
        // sink (every wave issues ND per stage: static vmcnt bookkeeping).
        auto issue = [&](int st) {
            const uint32_t slot = ring0 + (uint32_t)((st % C::NS) * C::STAGE);
#pragma unroll
            for (int q = 0; q < C::ND; ++q) {
                const int j = wave + 4 * q;
                uint32_t dst = ring0 + (uint32_t)(C::NS * C::STAGE);
                if (j < C::XU) {
                    constexpr int LPR = C::CPR < 64 ? C::CPR : 64;      // lanes per row
                    const int r = j * (64 / LPR) + lane / LPR;
                    const int cs = lane % LPR;                           // slot chunk
                    const int h = st * C::BK + 8 * (cs ^ row_swz<C::CPR>(r));
                    const uint32_t off = (st < nst && h < H)
                        ? ((uint32_t)r * (uint32_t)H + (uint32_t)h) * 2u : kOob;
                    dst = slot + (uint32_t)(j * 1024);
                    dma16_nt(xr, off, __builtin_amdgcn_readfirstlane(dst));
                } else {
                    // slab bytes past E * H * 2 (h >= H) are outside the resource: zero
                    uint32_t off = kOob;
                    if (j < C::XU + wu) {
                        dst = slot + (uint32_t)(j * 1024);
                        if (st < nst)
                            off = (uint32_t)st * (uint32_t)(C::BK * E * 2) +
                                  (uint32_t)((j - C::XU) * 1024) + (uint32_t)lane * 16u;
                    }
                    dma16(wr, off, __builtin_amdgcn_readfirstlane(dst));
                }
            }
        };

        f32x4_t acc[C::TT][C::ET];
#pragma unroll
        for (int a = 0; a < C::TT; ++a)
#pragma unroll
            for (int b = 0; b < C::ET; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // B-fragment addresses (bytes into the slab, + the k-step's 32 E rows).
        // Transposing reads (E % 4 == 0): source lane row = lane % 16 / 4 of
        // its 4-row group, 4 experts from 16 t + 4 (lane % 4); experts past E
        // read valid slab bytes of another column (those D columns are unused).
        // 16-bit reads: expert min(16 t + lane % 16, E - 1).
        const bool tr = (E & 3) == 0;
        uint32_t boff[C::ET];
#pragma unroll
        for (int b = 0; b < C::ET; ++b) {
            const int t = C::kSplitE ? wave + 4 * b : b;
            if (tr) {
                const int e4 = min(16 * t + 4 * (lane & 3), E - 4);
                boff[b] = (uint32_t)(((8 * g + ((lane & 15) >> 2)) * E + e4) * 2);
            } else {
                boff[b] = (uint32_t)((8 * g * E + min(16 * t + row, E - 1)) * 2);
            }
        }
#pragma unroll
        for (int st = 0; st < C::NS - 1; ++st) issue(st);
        for (int st = 0; st < nst; ++st) {
            wait_vmcnt<(C::NS - 2) * C::ND>();
            lds_barrier();
            issue(st + C::NS - 1);
            const uint32_t slot = ring0 + (uint32_t)((st % C::NS) * C::STAGE);
            const uint32_t slab = slot + (uint32_t)(C::XU * 1024);
#pragma unroll
            for (int kq = 0; kq < C::KW; ++kq) {
                const int kk = C::kSplitE ? kq : wave * C::KW + kq;   // k-step of the stage
                const int c = 4 * kk + g;                             // chunk of the row
                const uint32_t kbase = slab + (uint32_t)(kk * 32 * E * 2);
                bf16x8_t bfr[C::ET];
#pragma unroll
                for (int b = 0; b < C::ET; ++b) {
                    if (tr) {
                        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_v4i16_t*)(uintptr_t)(kbase + boff[b]));
                        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_v4i16_t*)(uintptr_t)(kbase + boff[b] + (uint32_t)(8 * E)));
                        const v8i16_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        bfr[b] = __builtin_bit_cast(bf16x8_t, v);
                    } else {
                        const lds_u16_t* pw =
                            reinterpret_cast<const lds_u16_t*>((uintptr_t)(kbase + boff[b]));
                        u32x4_t v;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            v[i] = (uint32_t)pw[(2 * i) * E] | ((uint32_t)pw[(2 * i + 1) * E] << 16);
                        bfr[b] = __builtin_bit_cast(bf16x8_t, v);
                    }
                }
#pragma unroll
                for (int a = 0; a < C::TT; ++a) {
                    const int r = 16 * a + row;
                    const u32x4_t xa = *reinterpret_cast<const lds_u32x4_t*>(
                        (uintptr_t)(slot + (uint32_t)(r * C::P + ((c ^ row_swz<C::CPR>(r)) << 4))));
#pragma unroll
                    for (int b = 0; b < C::ET; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, xa), bfr[b], acc[a][b], 0, 0, 0);
                }
            }
        }
        wait_vmcnt<0>();
        lds_barrier();
        // D[token][expert]: lane holds tokens 16 a + 4 (lane / 16) + i of expert
        // column 16 t + lane % 16
        if constexpr (C::kSplitE) {
#pragma unroll
            for (int a = 0; a < C::TT; ++a)
#pragma unroll
                for (int b = 0; b < C::ET; ++b) {
                    const int e = 16 * (wave + 4 * b) + row;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        lg[(16 * a + 4 * g + i) * C::E16 + e] = acc[a][b][i];
                }
        } else {
#pragma unroll
            for (int a = 0; a < C::TT; ++a)
#pragma unroll
                for (int b = 0; b < C::ET; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        red[(wave * C::TM + 16 * a + 4 * g + i) * C::E16 + 16 * b + row] =
                            acc[a][b][i];
        }
    }
    __syncthreads();

    if constexpr (C::kLane16) {
        // ---- one thread per (token r, expert e); 16 tokens
        const int r = tid >> 4, e = tid & 15, grp = lane & ~15, wv = tid >> 6;
        const bool ev = e < E, tv = r < ntok;
        float l;
        if (!logits_in) {
            l = ((red[(0 * 16 + r) * 16 + e] + red[(1 * 16 + r) * 16 + e]) +
                 red[(2 * 16 + r) * 16 + e]) + red[(3 * 16 + r) * 16 + e];
            if (ev && bg) l += __uint_as_float((uint32_t)bg[e] << 16);
            if (ev && tv && logits_io) logits_io[(t0 + r) * E + e] = l;
        } else {
            l = (ev && tv) ? logits_io[(t0 + r) * E + e] : 0.f;
        }
        float m = ev ? l : -INFINITY;
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d));
        const float pu = ev ? expf(l - m) : 0.f;                // unnormalised probability
        float Z = pu;
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) Z += __shfl_xor(Z, d);
        int rank = 0;
        for (int j = 0; j < E; ++j) {
            const float lj = __shfl(l, grp | j);
            rank += (lj > l) || (lj == l && j < e);
        }
        const bool sel = ev && rank < k;
        // renormalised top-k weight: exp(l_e - m) / sum over the selected of exp(l - m)
        float S = sel ? pu : 0.f;
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) S += __shfl_xor(S, d);
        if (sel && tv) {
            o.topk_idx[(t0 + r) * k + rank] = e;
            o.topk_w[(t0 + r) * k + rank] = pu / S;
        }
        // block partials: the 4 tokens of a wave by butterflies, then the
        // waves in order
        float ps = (ev && tv) ? pu / Z : 0.f;
        int cnt = (sel && tv) ? 1 : 0;
        float l2 = 0.f;
        if (e == 0 && tv) {
            const float lse = m + logf(Z);
            l2 = lse * lse;
        }
#pragma unroll
        for (int d = 16; d < 64; d <<= 1) {
            ps += __shfl_xor(ps, d);
            cnt += __shfl_xor(cnt, d);
            l2 += __shfl_xor(l2, d);
        }
        __syncthreads();                         // every lane has read red
        float* part = red;                       // [4 waves][16] probability sums
        int* part_c = reinterpret_cast<int*>(red + 4 * 16);
        float* part_l = red + 8 * 16;            // [4 waves]
        if (lane < 16) {
            part[wv * 16 + lane] = ps;
            part_c[wv * 16 + lane] = cnt;
            if (lane == 0) part_l[wv] = l2;
        }
        __syncthreads();
        const int64_t blk = blockIdx.x, nblk = gridDim.x;
        if (tid < E) {
            o.blk_psum[tid * nblk + blk] =
                ((part[tid] + part[16 + tid]) + part[32 + tid]) + part[48 + tid];
            o.blk_cnt[tid * nblk + blk] =
                part_c[tid] + part_c[16 + tid] + part_c[32 + tid] + part_c[48 + tid];
        }
        if (tid == 0) o.blk_lse2[blk] = ((part_l[0] + part_l[1]) + part_l[2]) + part_l[3];
    } else {
        // ---- logits tile [TM][E16]: the split-K sum, bias, optional output
        for (int j = tid; j < C::TM * C::E16; j += kThreads) {
            const int r = j / C::E16, e = j % C::E16;
            float v = 0.f;
            if (!logits_in) {
                if constexpr (!C::kSplitE)
                    v = ((red[j] + red[C::TM * C::E16 + j]) + red[2 * C::TM * C::E16 + j]) +
                        red[3 * C::TM * C::E16 + j];
                else
                    v = lg[j];
                if (e < E && bg) v += __uint_as_float((uint32_t)bg[e] << 16);
                if (e < E && r < ntok && logits_io) logits_io[(t0 + r) * E + e] = v;
            } else if (e < E && r < ntok) {
                v = logits_io[(t0 + r) * E + e];
            }
            flag[j] = 0;
            lg[j] = v;        // the split-K layout reads red[j] only for this j
        }
        __syncthreads();
        // ---- LPT lanes per token
        constexpr int LPT = C::LPT;
        const int r = tid / LPT, q = tid % LPT;
        const bool valid = r < ntok;
        float* lr = lg + r * C::E16;
        float m = -INFINITY;
        for (int e = q; e < E; e += LPT) m = fmaxf(m, lr[e]);
#pragma unroll
        for (int d = 1; d < LPT; d <<= 1) m = fmaxf(m, __shfl_xor(m, d));
        float Z = 0.f;
        for (int e = q; e < E; e += LPT) Z += expf(lr[e] - m);
#pragma unroll
        for (int d = 1; d < LPT; d <<= 1) Z += __shfl_xor(Z, d);
        uint64_t taken = 0;                 // bit j <=> expert q + LPT j taken
        int sel[kMaxK];
        float pv[kMaxK];
        for (int s = 0; s < k; ++s) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            int j = 0;
            for (int e = q; e < E; e += LPT, ++j) {
                if ((taken >> j) & 1ull) continue;
                const float v = lr[e];
                if (bi == 0x7fffffff || v > bv) { bv = v; bi = e; }
            }
#pragma unroll
            for (int d = 1; d < LPT; d <<= 1) {
                const float ov = __shfl_xor(bv, d);
                const int oi = __shfl_xor(bi, d);
                if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) {
                    bv = ov;
                    bi = oi;
                }
            }
            sel[s] = bi;
            pv[s] = expf(bv - m) / Z;
            if (bi % LPT == q) taken |= 1ull << (bi / LPT);
        }
        // every lane of the group holds the same sel / pv; lane 0 writes them
        if (q == 0) {
            float S = 0.f;
            for (int s = 0; s < k; ++s) S += pv[s];
            for (int s = 0; s < k; ++s) {
                if (valid) {
                    flag[r * C::E16 + sel[s]] = 1;
                    o.topk_idx[(t0 + r) * k + s] = sel[s];
                    o.topk_w[(t0 + r) * k + s] = pv[s] / S;
                }
            }
            const float lse = m + logf(Z);
            lse_s[r] = valid ? lse * lse : 0.f;
        }
        // probabilities of all experts (for the load-balancing loss)
        for (int e = q; e < E; e += LPT) lr[e] = valid ? expf(lr[e] - m) / Z : 0.f;
        __syncthreads();
        // ---- per 16-token block partials, tokens in order (independent loads)
        const int64_t nblk = (T + kRouteTok - 1) / kRouteTok;
        constexpr int NB = C::TM / kRouteTok;
        for (int j = tid; j < NB * E; j += kThreads) {
            const int b = j / E, e = j % E;
            const int64_t blk = t0 / kRouteTok + b;
            if (blk >= nblk) continue;
            float pr[kRouteTok];
            int fl[kRouteTok];
#pragma unroll
            for (int rr = 0; rr < kRouteTok; ++rr) {
                pr[rr] = lg[(b * kRouteTok + rr) * C::E16 + e];
                fl[rr] = flag[(b * kRouteTok + rr) * C::E16 + e];
            }
            float ps = 0.f;
            int c = 0;
#pragma unroll
            for (int rr = 0; rr < kRouteTok; ++rr) {
                ps += pr[rr];
                c += fl[rr];
            }
            o.blk_psum[e * nblk + blk] = ps;            // column-major: [E][nblk]
            o.blk_cnt[e * nblk + blk] = c;
        }
        if (tid < NB) {
            const int64_t blk = t0 / kRouteTok + tid;
            if (blk < nblk) {
                float a = 0.f;
#pragma unroll
                for (int rr = 0; rr < kRouteTok; ++rr) a += lse_s[tid * kRouteTok + rr];
                o.blk_lse2[blk] = a;
            }
        }
    }
}

template <int EB, int TM, int BK, int NS, int WE, bool SE>
static void launch_route_bf16(hipStream_t s, const uint16_t* x, const uint16_t* Wg,
                              const uint16_t* bg, float* logits, int logits_in, int64_t T, int H,
                              int E, int k, RouteOut o) {
    const int64_t nwg = (T + TM - 1) / TM;
    route_bf16<EB, TM, BK, NS, WE, SE><<<dim3((unsigned)nwg), dim3(kThreads), 0, s>>>(
        x, Wg, bg, logits, logits_in, T, H, E, k, o);
}

// ---------------------------------------------------------------- fp32 router
// Plain fp32 FMA dot products (small fp32 layers).  Dynamic LDS: logit_s[16][E].
__global__ __launch_bounds__(kThreads) void route_f32(
    const float* __restrict__ x, const float* __restrict__ Wg, const float* __restrict__ bg,
    float* __restrict__ logits_io, int logits_in, int64_t T, int H, int E, int k, RouteOut o) {
    extern __shared__ float smem[];
    __shared__ int32_t idx_s[kRouteTok * kMaxK];
    __shared__ float lse_s[kRouteTok];
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * kRouteTok;
    float* logit_s = smem;
    for (int j = tid; j < kRouteTok * E; j += kThreads) {
        const int r = j / E, e = j % E;
        const int64_t t = t0 + r;
        float v = 0.f;
        if (t < T) {
            if (logits_in) {
                v = logits_io[t * E + e];
            } else {
                const float* xr = x + t * H;
                for (int i = 0; i < H; ++i) v = fmaf(xr[i], Wg[(int64_t)i * E + e], v);
                if (bg) v += bg[e];
                if (logits_io) logits_io[t * E + e] = v;
            }
        }
        logit_s[j] = v;
    }
    __syncthreads();
    route_epilogue(logit_s, idx_s, lse_s, t0, T, E, k, o);
}

// ---------------------------------------------------------------- finalize
// E + 1 column workgroups, then one wave for the losses.
__global__ __launch_bounds__(kColThreads) void route_fin_columns(FinArgs f, int E) {
    fin_column_block(f, E, blockIdx.x);
}

__global__ __launch_bounds__(64) void route_fin_losses(FinArgs f, int E) {
    fin_losses(f, E);
}

}  // namespace

hipError_t launch_route(const moe_problem_t& p, const WsLayout& L, char* ws, const void* x,
                        const void* Wg, const void* bg, float* logits, bool logits_in,
                        int32_t* topk_idx, float* topk_w, int32_t* counts, float* losses,
                        bool finalize, hipStream_t s) {
    const int64_t T = p.T;
    const int H = p.H, E = p.E, k = p.k;
    RouteOut o;
    o.topk_idx = topk_idx;
    o.topk_w = topk_w;
    o.blk_psum = reinterpret_cast<float*>(ws + L.blk_psum);
    o.blk_lse2 = reinterpret_cast<float*>(ws + L.blk_lse2);
    o.blk_cnt = reinterpret_cast<int32_t*>(ws + L.blk_cnt);
    const int64_t nblk = L.nblk_route;
    if (p.dtype == MOE_DTYPE_BF16) {
        auto* xb = static_cast<const uint16_t*>(x);
        auto* wb = static_cast<const uint16_t*>(Wg);
        auto* bb = static_cast<const uint16_t*>(bg);
        const int li = logits_in ? 1 : 0;
        // shapes per gate width, from a sweep on one MI355X: with E <= 8 the
        // 37 KB ring lets 4 workgroups share a CU, so the Mixtral-shaped batch
        // (1024 workgroups) runs in one round; wide gates are bound by
        // re-streaming the whole gate through every workgroup
        if (E <= 8)
            launch_route_bf16<1, 16, 256, 3, 8, false>(s, xb, wb, bb, logits, li, T, H, E, k, o);
        else if (E <= 16)
            launch_route_bf16<1, 16, 256, 3, 16, false>(s, xb, wb, bb, logits, li, T, H, E, k, o);
        else if (E <= 32)
            launch_route_bf16<2, 32, 128, 3, 32, false>(s, xb, wb, bb, logits, li, T, H, E, k, o);
        else if (E <= 64)
            launch_route_bf16<4, 32, 64, 4, 64, true>(s, xb, wb, bb, logits, li, T, H, E, k, o);
        else if (E <= 128)
            launch_route_bf16<8, 16, 64, 2, 128, true>(s, xb, wb, bb, logits, li, T, H, E, k, o);
        else
            launch_route_bf16<16, 32, 64, 2, 256, true>(s, xb, wb, bb, logits, li, T, H, E, k, o);
    } else {
        const size_t lds = sizeof(float) * (size_t)kRouteTok * E;
        route_f32<<<dim3((unsigned)nblk), dim3(kThreads), lds, s>>>(
            static_cast<const float*>(x), static_cast<const float*>(Wg),
            static_cast<const float*>(bg), logits, logits_in ? 1 : 0, T, H, E, k, o);
    }
    if (finalize) {
        const FinArgs f{o.blk_psum, o.blk_lse2, o.blk_cnt, nblk, T, k,
                        reinterpret_cast<double*>(ws + L.fin_sum),
                        reinterpret_cast<long long*>(ws + L.fin_cnt), counts, losses};
        route_fin_columns<<<dim3(E + 1), dim3(kColThreads), 0, s>>>(f, E);
        route_fin_losses<<<dim3(1), dim3(64), 0, s>>>(f, E);
    }
    return hipGetLastError();
}

}  // namespace moe
