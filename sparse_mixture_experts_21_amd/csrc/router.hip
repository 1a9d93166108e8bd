// Router: gate linear, softmax over experts, top-k, renormalisation of the k
// selected scores, and per-block partial sums for the load-balancing loss and
// the router z-loss ("moe-training" SKILL page, Quick Start, Basic MoE
// Architecture; Core Concepts, 3. Load Balancing).
//
// One workgroup (4 waves) owns 16 tokens.  The gate linear is a skinny GEMM
// [16 x H] . [H x E]: the H axis is split over the 4 waves, each wave issues
// v_mfma_f32_16x16x32_bf16 on 16-byte fragments loaded straight from HBM (x)
// and L2 (the gate weights, transposed once per call to [E][H] so that a lane
// reads 8 consecutive H values); wave 0 adds the other waves' partial tiles,
// parked in LDS, in a fixed order.  The routing epilogue runs 4 lanes per token.  Per-block
// partials (sum of softmax probabilities per expert, sum of lse^2, expert
// histogram) are reduced by two small kernels in a fixed order, so the losses
// are bitwise reproducible without floating-point atomics.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

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
    const int64_t blk = blockIdx.x;
    for (int e = tid; e < E; e += kThreads) {
        float ps = 0.f;
        int c = 0;
        for (int r = 0; r < kRouteTok; ++r) {
            ps += logit_s[r * E + e];
            for (int s = 0; s < k; ++s) c += (idx_s[r * kMaxK + s] == e);
        }
        o.blk_psum[blk * E + e] = ps;
        o.blk_cnt[blk * E + e] = c;
    }
    if (tid == 0) {
        float a = 0.f;
        for (int r = 0; r < kRouteTok; ++r) a += lse_s[r];
        o.blk_lse2[blk] = a;
    }
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
        const int64_t t = min(t0 + row, T - 1);
        const uint16_t* xr = x + t * H;
        f32x4_t acc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int nks = (H + 31) >> 5;
        // wave w takes k-steps w, w+4, ...; a lane owns 8 consecutive h values
#pragma unroll 2
        for (int ks = wave; ks < nks; ks += kWaves) {
            const int h0 = ks * 32 + g * 8;
            u32x4_t av = u32x4_t{0u, 0u, 0u, 0u};
            if (h0 < H) av = *reinterpret_cast<const u32x4_t*>(xr + h0);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int e = nt * 16 + row;
                u32x4_t bv = u32x4_t{0u, 0u, 0u, 0u};
                if (e < E && h0 < H)
                    bv = *reinterpret_cast<const u32x4_t*>(WgT + (int64_t)e * H + h0);
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv), acc[nt],
                    0, 0, 0);
            }
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
// Block e < E: column e of the block partials (probability sum, histogram);
// block E: the lse^2 partials.  Fixed-order double tree -> deterministic.
__global__ __launch_bounds__(256) void route_reduce(const float* __restrict__ blk_psum,
                                                    const float* __restrict__ blk_lse2,
                                                    const int32_t* __restrict__ blk_cnt,
                                                    int64_t nblk, int E, double* fin,
                                                    int32_t* counts) {
    __shared__ double sd[256];
    __shared__ int64_t si[256];
    const int tid = threadIdx.x, col = blockIdx.x;
    double a = 0.0;
    int64_t c = 0;
    for (int64_t j = tid; j < nblk; j += 256) {
        if (col < E) {
            a += (double)blk_psum[j * E + col];
            c += blk_cnt[j * E + col];
        } else {
            a += (double)blk_lse2[j];
        }
    }
    sd[tid] = a;
    si[tid] = c;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) {
            sd[tid] += sd[tid + w];
            si[tid] += si[tid + w];
        }
        __syncthreads();
    }
    if (tid == 0) {
        fin[col] = sd[0];
        if (col < E) counts[col] = (int32_t)si[0];
    }
}

// aux = E * sum_e (counts_e / (T k)) * (psum_e / T);  z = sum lse^2 / T.
__global__ void route_losses(const double* __restrict__ fin, const int32_t* __restrict__ counts,
                             int64_t T, int E, int k, float* losses) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    double acc = 0.0;
    for (int e = 0; e < E; ++e)
        acc += ((double)counts[e] / (double)(T * k)) * (fin[e] / (double)T);
    losses[0] = (float)((double)E * acc);
    losses[1] = (float)(fin[E] / (double)T);
}

}  // namespace

hipError_t launch_route(const moe_problem_t& p, const WsLayout& L, char* ws, const void* x,
                        const void* Wg, const void* bg, float* logits, bool logits_in,
                        int32_t* topk_idx, float* topk_w, int32_t* counts, float* losses,
                        hipStream_t s) {
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
        uint16_t* WgT = reinterpret_cast<uint16_t*>(ws + L.wgt);
        if (!logits_in) {
            const int64_t n = (int64_t)H * E;
            gate_transpose_bf16<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(
                static_cast<const uint16_t*>(Wg), WgT, H, E);
        }
        const int NT = (E + 15) / 16;
        const int NTp = NT <= 1 ? 1 : NT <= 2 ? 2 : NT <= 4 ? 4 : NT <= 8 ? 8 : 16;
        auto* xb = static_cast<const uint16_t*>(x);
        auto* bb = static_cast<const uint16_t*>(bg);
        const int li = logits_in ? 1 : 0;
        switch (NTp) {
            case 1: launch_route_bf16_nt<1>(nblk, s, xb, WgT, bb, logits, li, T, H, E, k, o); break;
            case 2: launch_route_bf16_nt<2>(nblk, s, xb, WgT, bb, logits, li, T, H, E, k, o); break;
            case 4: launch_route_bf16_nt<4>(nblk, s, xb, WgT, bb, logits, li, T, H, E, k, o); break;
            case 8: launch_route_bf16_nt<8>(nblk, s, xb, WgT, bb, logits, li, T, H, E, k, o); break;
            default: launch_route_bf16_nt<16>(nblk, s, xb, WgT, bb, logits, li, T, H, E, k, o); break;
        }
    } else {
        const size_t lds = sizeof(float) * (size_t)kRouteTok * E;
        route_f32<<<dim3((unsigned)nblk), dim3(kThreads), lds, s>>>(
            static_cast<const float*>(x), static_cast<const float*>(Wg),
            static_cast<const float*>(bg), logits, logits_in ? 1 : 0, T, H, E, k, o);
    }
    double* fin = reinterpret_cast<double*>(ws + L.fin);
    route_reduce<<<dim3(E + 1), dim3(256), 0, s>>>(o.blk_psum, o.blk_lse2, o.blk_cnt, nblk, E,
                                                   fin, counts);
    route_losses<<<dim3(1), dim3(64), 0, s>>>(fin, counts, T, E, k, losses);
    return hipGetLastError();
}

}  // namespace moe
