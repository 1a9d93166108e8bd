// Router: gate linear, softmax over experts, top-k, renormalisation of the k
// selected scores, and per-block partial sums for the load-balancing loss and
// the router z-loss ("moe-training" SKILL page, Quick Start, Basic MoE
// Architecture; Core Concepts, 3. Load Balancing).
//
// One workgroup (4 waves) owns 16 tokens.  The gate linear is a skinny GEMM
// [16 x H] . [H x E] on v_mfma_f32_16x16x32_bf16; the 4 waves split the H axis
// and wave 0 adds the other waves' partial tiles, parked in LDS, in a fixed
// order.  With E <= 16 (route_bf16_ring) x and the gate stream through an LDS
// ring by direct DMA; wider gates (route_bf16) load 16-byte fragments straight
// into registers from x and from a per-call [E][H] copy of the gate.  The
// routing epilogue runs 4 lanes per token.  Per-block partials (sum of softmax
// probabilities per expert, sum of lse^2, expert histogram) are reduced in a
// fixed order by one workgroup per column, so the losses are bitwise
// reproducible without floating-point atomics.
#include "moe_internal.h"
#include "lds_dma.h"
#include "route_finalize.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
// cache-policy operand of a buffer load: nontemporal (x is read once here)
constexpr int kNtLoad = 2;

// ---------------------------------------------------------------- gate transpose
__global__ void gate_transpose_bf16(const uint16_t* __restrict__ Wg, uint16_t* __restrict__ WgT,
                                    int H, int E) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)H * E) return;
    int h = (int)(i / E), e = (int)(i % E);
    WgT[(int64_t)e * H + h] = Wg[i];
}

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

// ---------------------------------------------------------------- routing epilogue, E <= 16
// Thread t owns (token r = t / 16, expert e = t % 16): the 16 lanes of a token
// are one aligned group of a wave.  red[w][r][e] holds wave w's partial gate
// tile; the logit is ((w0 + w1) + w2) + w3 (+ bias).  Max, softmax sum and the
// renormalisation sum are butterflies within the group: every lane adds the
// same two operands at every level (in either order, which is exact), so all
// 16 lanes agree bit for bit.  The top-k slot of an expert is its rank among
// the token's logits, descending, equal values -> lower index first.  Block
// partials: per expert over the block's tokens (4 per wave by shuffles, then
// waves 0..3 in order through LDS), written column-major [E][nblk].
__device__ __forceinline__ void route_epilogue16(float* red, int64_t t0, int ntok, int E, int k,
                                                 const uint16_t* __restrict__ bg,
                                                 float* __restrict__ logits_out,
                                                 const RouteOut& o) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = tid >> 4, e = tid & 15, grp = lane & ~15;
    const bool ev = e < E, tv = r < ntok;
    float l = ((red[(0 * kRouteTok + r) * 16 + e] + red[(1 * kRouteTok + r) * 16 + e]) +
               red[(2 * kRouteTok + r) * 16 + e]) + red[(3 * kRouteTok + r) * 16 + e];
    if (ev && bg) l += __uint_as_float((uint32_t)bg[e] << 16);
    if (ev && tv && logits_out) logits_out[(t0 + r) * E + e] = l;
    float m = ev ? l : -INFINITY;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d));
    const float pu = ev ? expf(l - m) : 0.f;                    // unnormalised probability
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
    // block partials
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
        part[wave * 16 + lane] = ps;
        part_c[wave * 16 + lane] = cnt;
        if (lane == 0) part_l[wave] = l2;
    }
    __syncthreads();
    const int64_t blk = blockIdx.x, nblk = gridDim.x;
    if (tid < E) {
        o.blk_psum[tid * nblk + blk] = ((part[tid] + part[16 + tid]) + part[32 + tid]) + part[48 + tid];
        o.blk_cnt[tid * nblk + blk] = part_c[tid] + part_c[16 + tid] + part_c[32 + tid] + part_c[48 + tid];
    }
    if (tid == 0) o.blk_lse2[blk] = ((part_l[0] + part_l[1]) + part_l[2]) + part_l[3];
}

// ---------------------------------------------------------------- bf16 router
// NT = number of 16-expert tiles (E <= 16 NT).  Waves 1..3 park their partial
// tiles in LDS red[3][16][16 NT]; wave 0 adds them to its own registers in the
// fixed order ((w0 + w1) + w2) + w3 and writes logit_s[16][E].
template <int NT>
__global__ __launch_bounds__(kThreads) void route_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ WgT,
    const uint16_t* __restrict__ bg, float* __restrict__ logits_io, int logits_in, int64_t T,
    int H, int E, int k, RouteOut o) {
    constexpr int E16 = NT * 16;
    __shared__ float logit_s[kRouteTok * E16];          // [16][E] (row stride E)
    __shared__ float red[3 * kRouteTok * E16];          // [3][16][E16]
    __shared__ int32_t idx_s[kRouteTok * kMaxK];
    __shared__ float lse_s[kRouteTok];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t t0 = (int64_t)blockIdx.x * kRouteTok;

    if (!logits_in) {
        const int row = lane & 15, g = lane >> 4;
        // x through a raw buffer resource based at the block's first token
        // (loads at offsets past the end return zero) and the transposed gate
        // likewise; every lane owns 8 consecutive h of token min(t0+row, T-1).
        const uint32_t xrow = (uint32_t)(min(t0 + row, T - 1) - t0) * (uint32_t)H * 2u;
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            uniform_ptr(x + t0 * H), (short)0,
            (T - t0 < kRouteTok ? (int)(T - t0) : kRouteTok) * H * 2,
            0x00020000);
        const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
            uniform_ptr(WgT), (short)0, E * H * 2, 0x00020000);
        f32x4_t acc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // wave w reduces the contiguous k-steps [ks0, ks1) of 32 h each, UNR at a
        // time with all of their loads in flight before the MFMAs
        const int nks = (H + 31) >> 5;
        const int wv = __builtin_amdgcn_readfirstlane(wave);   // uniform loop bounds
        const int ks0 = (wv * nks) / kWaves, ks1 = ((wv + 1) * nks) / kWaves;
        constexpr int UNR = NT <= 2 ? 8 : (NT <= 4 ? 4 : 2);
        for (int ks = ks0; ks < ks1; ks += UNR) {
            u32x4_t av[UNR], bv[UNR][NT];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int h0 = (ks + u) * 32 + g * 8;
                // H % 8 == 0, so a lane's 8 h are all in range or all past the end
                const bool ok = (ks + u) < ks1 && h0 < H;
                av[u] = __builtin_amdgcn_raw_buffer_load_b128(
                    xr, ok ? xrow + (uint32_t)h0 * 2u : 0x80000000u, 0, kNtLoad);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int e = nt * 16 + row;
                    const uint32_t off = (ok && e < E) ? ((uint32_t)e * (uint32_t)H + (uint32_t)h0) * 2u
                                                       : 0x80000000u;
                    bv[u][nt] = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 0);
                }
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, av[u]), __builtin_bit_cast(bf16x8_t, bv[u][nt]),
                        acc[nt], 0, 0, 0);
        }
        // D[token][expert]: lane holds tokens 4*(lane/16)+i of expert nt*16 + lane%16
        if (wave > 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    red[((wave - 1) * kRouteTok + (lane >> 4) * 4 + i) * E16 + nt * 16 +
                        (lane & 15)] = acc[nt][i];
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int e = nt * 16 + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = (lane >> 4) * 4 + i;
                    float v = acc[nt][i];
                    v += red[(0 * kRouteTok + r) * E16 + e];
                    v += red[(1 * kRouteTok + r) * E16 + e];
                    v += red[(2 * kRouteTok + r) * E16 + e];
                    if (e < E) {
                        if (bg) v += __uint_as_float((uint32_t)bg[e] << 16);
                        logit_s[r * E + e] = v;
                        if (logits_io && t0 + r < T) logits_io[(t0 + r) * E + e] = v;
                    }
                }
            }
        }
    } else {
        for (int j = tid; j < kRouteTok * E; j += kThreads) {
            const int r = j / E;
            logit_s[j] = (t0 + r < T) ? logits_io[(t0 + r) * E + (j % E)] : 0.f;
        }
    }
    __syncthreads();
    route_epilogue(logit_s, idx_s, lse_s, t0, T, E, k, o);
}

// ---------------------------------------------------------------- bf16 router, E <= 16
// The block's 16 token rows stream through an LDS ring of kRingStages stages of
// kStageH hidden units, next to the matching slab Wg[h0 .. h0 + kStageH)[0 .. E)
// of the gate (E KB, contiguous in the [H][E] layout, so no transposed copy is
// needed).  One direct-to-LDS DMA moves 1 KB, so x leaves HBM in whole
// contiguous row segments: fragment-shaped register loads touch 16 rows x 64 B
// per instruction, which HBM serves well below its streaming rate.  x is read
// with the nontemporal hint: it is streamed once here, and a normal load would
// first have to write back the dirty lines earlier kernels left in the
// last-level cache.  The 16-byte chunk c of token row r sits at slot c ^ r, so
// the 16 rows of a fragment read land on distinct banks; a lane assembles its
// gate fragment (8 consecutive h of one expert) from 16-bit reads of the slab.
// The waves split each stage's 16 k-steps.  Stage bookkeeping: before
// computing stage s a wave waits until only the DMAs of the (kRingStages - 2)
// younger stages are outstanding; a barrier then publishes every wave's part of
// stage s and frees the slot of stage s - 1, which the DMAs of stage
// s + kRingStages - 1 overwrite.
#ifndef MOE_RING_RB
#define MOE_RING_RB 512
#endif
#ifndef MOE_RING_NS
#define MOE_RING_NS 4
#endif
constexpr int kRingStages = MOE_RING_NS;
constexpr int kRowBytes = MOE_RING_RB;    // bytes of one token row per stage

template <int EC>   // gate columns reserved per stage (E <= EC)
struct RingCfg {
    static constexpr int RB = kRowBytes, NS = kRingStages;
    static constexpr int SH = RB / 2;                       // hidden units per stage
    static constexpr int RPU = 1024 / RB;                   // token rows per 1 KB DMA
    static constexpr int XU = kRouteTok / RPU;              // DMAs for the token rows
    static constexpr int WU = EC * RB / 1024;               // DMAs for the gate slab (max)
    static constexpr int ND = (XU + WU) / kWaves;           // DMAs per wave per stage
    static constexpr int STAGE = (XU + WU) * 1024;
    static constexpr int LDS = NS * STAGE + 1024;           // + a sink for padding DMAs
    static constexpr int KW = SH / 32 / kWaves;             // k-steps per wave per stage
    static_assert((XU + WU) % kWaves == 0 && KW >= 1, "ring shape");
    static_assert(NS >= 3, "the wait count assumes two younger stages may be in flight");
};

typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;

template <int EC>
__global__ __launch_bounds__(kThreads) void route_bf16_ring(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wg,
    const uint16_t* __restrict__ bg, float* __restrict__ logits_out, int64_t T, int H, int E,
    int k, RouteOut o) {
    using C = RingCfg<EC>;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[C::LDS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t t0 = (int64_t)blockIdx.x * kRouteTok;
    const int ntok = (T - t0 < kRouteTok) ? (int)(T - t0) : kRouteTok;
    const uint32_t ring0 = (uint32_t)(uintptr_t)ring;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(uniform_ptr(x + t0 * H), (uint32_t)(ntok * H * 2));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(uniform_ptr(Wg), (uint32_t)(E * H * 2));
    const int nst = (H + C::SH - 1) / C::SH;
    const int wu = (E * C::RB + 1023) / 1024;          // gate-slab DMAs actually needed

    // DMA q of this wave fills 1 KB unit j = wave + 4 q of the stage: token rows
    // (RPU per unit) first, then the gate slab; units past XU + wu are padding
    // DMAs into the sink (every wave issues C::ND per stage, which keeps the
    // vmcnt bookkeeping static).
    auto issue = [&](int st) {
        const uint32_t slot = ring0 + (uint32_t)((st % C::NS) * C::STAGE);
#pragma unroll
        for (int q = 0; q < C::ND; ++q) {
            const int j = wave + kWaves * q;
            uint32_t dst = ring0 + (uint32_t)(C::NS * C::STAGE);
            if (j < C::XU) {
                const int r = j * C::RPU + lane / (64 / C::RPU);
                const int cl = lane % (64 / C::RPU);
                const int h = st * C::SH + 8 * (cl ^ (r & 15));
                const uint32_t off = (st < nst && h < H)
                    ? ((uint32_t)r * (uint32_t)H + (uint32_t)h) * 2u : kOob;
                dst = slot + (uint32_t)(j * 1024);
                dma16_nt(xr, off, __builtin_amdgcn_readfirstlane(dst));
            } else {
                // slab bytes past E * H * 2 (h >= H) are out of the resource: zero
                uint32_t off = kOob;
                if (j < C::XU + wu) {
                    dst = slot + (uint32_t)(j * 1024);
                    if (st < nst)
                        off = (uint32_t)st * (uint32_t)(E * C::RB) +
                              (uint32_t)((j - C::XU) * 1024) + (uint32_t)lane * 16u;
                }
                dma16(wr, off, __builtin_amdgcn_readfirstlane(dst));
            }
        }
    };

    const int row = lane & 15, g = lane >> 4;
    const int er = row < E ? row : E - 1;            // columns >= E are discarded
    const bool row_ok = row < ntok;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
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
            const int kk = wave * C::KW + kq;
            const int c = 4 * kk + g;                 // 16-byte chunk of the stage row
            const bool h_ok = st * C::SH + 8 * c < H;
            u32x4_t a = *reinterpret_cast<const lds_u32x4_t*>(
                (uintptr_t)(slot + (uint32_t)(row * C::RB + ((c ^ row) << 4))));
            const lds_u16_t* pw = reinterpret_cast<const lds_u16_t*>(
                (uintptr_t)(slab + (uint32_t)((8 * c * E + er) * 2)));
            u32x4_t b;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                b[i] = (uint32_t)pw[(2 * i) * E] | ((uint32_t)pw[(2 * i + 1) * E] << 16);
            const u32x4_t z = {0u, 0u, 0u, 0u};
            if (!(h_ok && row_ok)) a = z;
            if (!h_ok) b = z;
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                          __builtin_bit_cast(bf16x8_t, b), acc,
                                                          0, 0, 0);
        }
    }
    wait_vmcnt<0>();
    lds_barrier();
    float* red = reinterpret_cast<float*>(ring);                 // [4 waves][16][16]
#pragma unroll
    for (int i = 0; i < 4; ++i)
        red[(wave * kRouteTok + (lane >> 4) * 4 + i) * 16 + (lane & 15)] = acc[i];
    __syncthreads();
    route_epilogue16(red, t0, ntok, E, k, bg, logits_out, o);
}


template <int NT>
static void launch_route_bf16_nt(int64_t nblk, hipStream_t s, const uint16_t* x,
                                 const uint16_t* WgT, const uint16_t* bg, float* logits,
                                 int logits_in, int64_t T, int H, int E, int k, RouteOut o) {
    route_bf16<NT><<<dim3((unsigned)nblk), dim3(kThreads), 0, s>>>(x, WgT, bg, logits,
                                                                     logits_in, T, H, E, k, o);
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
// E + 1 column workgroups, then one thread for the losses.
__global__ __launch_bounds__(kColThreads) void route_fin_columns(FinArgs f, int E) {
    fin_column_block(f, E, blockIdx.x);
}

__global__ void route_fin_losses(FinArgs f, int E) {
    if (threadIdx.x == 0) fin_losses(f, E);
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
        if (!logits_in && E <= 16) {
            if (E <= 8)
                route_bf16_ring<8><<<dim3((unsigned)nblk), dim3(kThreads), 0, s>>>(
                    xb, wb, bb, logits, T, H, E, k, o);
            else
                route_bf16_ring<16><<<dim3((unsigned)nblk), dim3(kThreads), 0, s>>>(
                    xb, wb, bb, logits, T, H, E, k, o);
        } else {
            uint16_t* WgT = reinterpret_cast<uint16_t*>(ws + L.wgt);
            if (!logits_in) {
                const int64_t n = (int64_t)H * E;
                gate_transpose_bf16<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(
                    wb, WgT, H, E);
            }
            const int NT = (E + 15) / 16;
            const int NTp = NT <= 1 ? 1 : NT <= 2 ? 2 : NT <= 4 ? 4 : NT <= 8 ? 8 : 16;
            const int li = logits_in ? 1 : 0;
            switch (NTp) {
                case 1: launch_route_bf16_nt<1>(nblk, s, xb, WgT, bb, logits, li, T, H, E, k, o); break;
                case 2: launch_route_bf16_nt<2>(nblk, s, xb, WgT, bb, logits, li, T, H, E, k, o); break;
                case 4: launch_route_bf16_nt<4>(nblk, s, xb, WgT, bb, logits, li, T, H, E, k, o); break;
                case 8: launch_route_bf16_nt<8>(nblk, s, xb, WgT, bb, logits, li, T, H, E, k, o); break;
                default: launch_route_bf16_nt<16>(nblk, s, xb, WgT, bb, logits, li, T, H, E, k, o); break;
            }
        }
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
