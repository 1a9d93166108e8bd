// Device helpers shared by the grouped GEMM kernels of the forward and the
// backward: the expert activations and their derivatives, and the lookup of
// an expert's row tile from the row offsets.
#pragma once

#include "moe_internal.h"

namespace moe {

enum Act { kActNone = 0, kActGelu = 1, kActSilu = 2 };

// Exact (erf) GELU, 0.5 a (1 + erf(a / sqrt 2)) = max(a, 0) - 0.5 |a| q with
// q = 1 - erf(|a| / sqrt 2) (erf is odd; no cancellation for a < 0, where the
// result is the small 0.5 a q), erf evaluated by formula 7.1.26 of Abramowitz & Stegun,
// Handbook of Mathematical Functions:
//   erf(u) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-u^2),
//   t = 1 / (1 + p u), u >= 0, |error| <= 1.5e-7,
// i.e. below fp32 rounding of GELU's output scale and far below bf16.  With
// u = |a| / sqrt 2 the factor 1/sqrt 2 folds into p, and exp(-u^2) is
// 2^(a^2 * (-1 / (2 ln 2))).  One reciprocal and one exponential, no branches.
// The coefficients are halved (exactly: a power of two), so the polynomial
// gives h = q / 2 directly.
__device__ __forceinline__ float gelu_half_q(float a, float& ex) {
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752440f, fabsf(a), 1.0f));
    float poly = fmaf(t, 0.5f * 1.061405429f, 0.5f * -1.453152027f);
    poly = fmaf(t, poly, 0.5f * 1.421413741f);
    poly = fmaf(t, poly, 0.5f * -0.284496736f);
    poly = fmaf(t, poly, 0.5f * 0.254829592f);
    ex = __builtin_amdgcn_exp2f(a * (a * -0.72134752044448170368f));
    return t * poly * ex;                                 // (1 - erf(|a| / sqrt 2)) / 2
}
__device__ __forceinline__ float gelu_erf(float a) {
    float ex;
    const float h = gelu_half_q(a, ex);
    return fmaf(-fabsf(a), h, fmaxf(a, 0.0f));
}

// SiLU, a * sigmoid(a) = a / (1 + e^-a) with e^-a = 2^(-a log2 e).  For very
// negative a the denominator overflows to +inf and the result is -0; for very
// positive a it is 1 and the result is a.
__device__ __forceinline__ float silu(float a) {
    return a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * -1.44269504088896340736f));
}

template <int ACT>
__device__ __forceinline__ float activate(float v) {
    if constexpr (ACT == kActGelu) return gelu_erf(v);
    else if constexpr (ACT == kActSilu) return silu(v);
    else return v;
}

// Locate the expert and row tile of row-tile index mt.  Returns false when mt
// is beyond the last real tile.  The whole wave walks 64 experts at a time
// (tile counts, a shuffle scan, a ballot), so the cost grows with E / 64.
template <int BM>
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int E, int mt,
                                          int& e_out, int& m0, int& row_begin, int& n_rows) {
    const int lane = threadIdx.x & 63;
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        const int b = e < E ? offsets[e] : 0;
        const int n = e < E ? offsets[e + 1] - b : 0;
        const int tiles = (n + BM - 1) / BM;
        int incl = tiles;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(incl, d);
            if (lane >= d) incl += t;
        }
        const int excl = incl - tiles;
        const uint64_t hit = __ballot(e < E && mt >= base + excl && mt < base + incl);
        if (hit) {
            // wave-uniform results, pinned to scalar registers
            const int src = __ffsll((unsigned long long)hit) - 1;
            e_out = __builtin_amdgcn_readfirstlane(__shfl(e, src));
            m0 = __builtin_amdgcn_readfirstlane((mt - base - __shfl(excl, src)) * BM);
            row_begin = __builtin_amdgcn_readfirstlane(__shfl(b, src));
            n_rows = __builtin_amdgcn_readfirstlane(__shfl(n, src));
            return true;
        }
        base += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
    }
    return false;
}

// Tile order.  Real tiles get the dense positions 0 .. R-1 (R = real row tiles
// x Nt; the real row-tile count is computed on the device from `offsets`).
// Full super-block rows come first: super-blocks of 256 tiles (SBM = 256/SBN
// row tiles x SBN column tiles, one tile per CU), walked row-major.  The
// hardware deals workgroups to the 8 XCDs round-robin, so position p runs on
// XCD p % 8; in each super-block every XCD gets an 8 x 4 sub-block (rotating
// with the super-block index), so the ~32 tiles resident on one XCD share
// their row and weight slabs in its L2, and slabs another XCD already pulled
// come from the memory-side cache.  The remaining (< SBM) row tiles follow,
// XCD x taking the column tiles nt = x (mod 8) when Nt % 8 == 0.
__device__ __forceinline__ void dense_coords(int p, int real_mt, int Nt, int SBN, int& mt,
                                             int& nt) {
    const int SBM = 256 / SBN;
    if (Nt % SBN != 0) {                                  // no super-blocks (narrow N)
        mt = p / Nt;
        nt = p % Nt;
        return;
    }
    const int F = real_mt / SBM;                          // full super-block rows
    const int nfull = F * SBM * Nt;
    if (p < nfull) {
        const int sb = p >> 8, q = p & 255;
        const int x = q & 7, j = q >> 3;                  // XCD, slot on the XCD
        const int nsbn = Nt / SBN;
        const int sbm = sb / nsbn, sbn = sb % nsbn;
        // XCD x takes sub-block (x + sb) % 8
        const int s8 = (x + sb) & 7;
        const int xm = s8 % (SBM / 8), xn = s8 / (SBM / 8);
        mt = sbm * SBM + xm * 8 + (j & 7);
        nt = sbn * SBN + xn * 4 + (j >> 3);
        return;
    }
    const int q = p - nfull, rem = real_mt - F * SBM;
    if (Nt % 8 == 0) {
        const int x = q & 7, j = q >> 3;
        nt = 8 * (j / rem) + x;
        mt = F * SBM + j % rem;
    } else {
        mt = F * SBM + q / Nt;
        nt = q % Nt;
    }
}

// Position p of tile (mt, nt) in the order above: the inverse of dense_coords
// for 0 <= mt < real_mt, 0 <= nt < Nt, with SBN = 1 << lg (every division a
// shift).
__device__ __forceinline__ int dense_position(int mt, int nt, int real_mt, int Nt, int lg) {
    const int SBN = 1 << lg, lm = 8 - lg;                 // SBM = 256 / SBN = 1 << lm
    if (Nt & (SBN - 1)) return mt * Nt + nt;
    const int F = real_mt >> lm;
    if (mt < (F << lm)) {
        const int sb = (mt >> lm) * (Nt >> lg) + (nt >> lg);
        const int s8 = ((mt & ((1 << lm) - 1)) >> 3) + (((nt & (SBN - 1)) >> 2) << (lm - 3));
        const int x = (s8 - sb) & 7;                                    // XCD of the sub-block
        const int j = (mt & 7) + 8 * (nt & 3);                          // slot on the XCD
        return (sb << 8) + x + 8 * j;
    }
    const int q0 = (F << lm) * Nt, rm = mt - (F << lm), rem = real_mt - (F << lm);
    if ((Nt & 7) == 0) return q0 + (nt & 7) + 8 * ((nt >> 3) * rem + rm);
    return q0 + rm * Nt + nt;
}

// How a grouped GEMM launch cuts its last round.  The R = real_mt * Nt real
// tiles leave tail = R mod ncu tiles for a ragged last round; when those are
// at most half of it, each is cut along K into S = ncu / tail slices (at most
// kMaxUnits slices in all, each at least ns k-tiles deep), which write fp32
// partial tiles; the positions [0, full) are computed whole.  The GEMM, its
// fixup and the combine that finishes the second GEMM's cut tiles all take
// the plan from here.
constexpr int kMaxUnits = 256;

struct TailPlan {
    int real_mt;      // real row tiles
    int full;         // tiles computed whole: positions [0, full)
    int tail;         // tiles cut into S slices: positions [full, full + tail S)
    int S;            // slices per tail tile (1: no cut)
};

__host__ __device__ __forceinline__ TailPlan plan_tail(int real_mt, int Nt, int ncu, int nk,
                                                       int ns, bool allow) {
    TailPlan pl;
    pl.real_mt = real_mt;
    const int R = real_mt * Nt;
    pl.tail = R % ncu;
    int S = pl.tail > 0 ? (ncu < kMaxUnits ? ncu : kMaxUnits) / pl.tail : 1;
    if (nk / ns < S) S = nk / ns;
    if (!allow || S < 2) {
        pl.S = 1;
        pl.tail = 0;
    } else {
        pl.S = S;
    }
    pl.full = R - pl.tail;
    return pl;
}

// Real row tiles over all experts (every lane gets the same value).
template <int BM>
__device__ __forceinline__ int real_row_tiles(const int32_t* __restrict__ offsets, int E) {
    const int lane = threadIdx.x & 63;
    int t = 0;
    for (int e = lane; e < E; e += 64) t += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) t += __shfl_xor(t, d);
    return t;
}

// Derivatives for the backward.  GELU'(a) = Phi(a) + a phi(a): with q as in
// gelu_erf, Phi(a) = 1 - q/2 for a >= 0 and q/2 below, and phi(a) =
// exp(-a^2 / 2) / sqrt(2 pi) is the same exponential times 1 / sqrt(2 pi).
__device__ __forceinline__ float gelu_erf_grad(float a) {
    float ex;
    const float h = gelu_half_q(a, ex);                   // q / 2
    const float Phi = a >= 0.0f ? 1.0f - h : h;
    return fmaf(a * 0.39894228040143267794f, ex, Phi);
}

// SiLU'(a) = s (1 + a (1 - s)), s = sigmoid(a) (0 for very negative a).
__device__ __forceinline__ float silu_grad(float a) {
    const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * -1.44269504088896340736f));
    return s * fmaf(a, 1.0f - s, 1.0f);
}

template <int ACT>
__device__ __forceinline__ float activate_grad(float v) {
    if constexpr (ACT == kActGelu) return gelu_erf_grad(v);
    else if constexpr (ACT == kActSilu) return silu_grad(v);
    else return 1.0f;
}

// act(a), and act'(a) in g, from one evaluation of the shared terms (the
// reciprocal, polynomial and exponential of the erf form; the sigmoid).
template <int ACT>
__device__ __forceinline__ float activate_with_grad(float a, float& g) {
    if constexpr (ACT == kActGelu) {
        float ex;
        const float h = gelu_half_q(a, ex);               // q / 2
        g = fmaf(a * 0.39894228040143267794f, ex, a >= 0.0f ? 1.0f - h : h);
        return fmaf(-fabsf(a), h, fmaxf(a, 0.0f));
    } else if constexpr (ACT == kActSilu) {
        const float s =
            __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * -1.44269504088896340736f));
        g = s * fmaf(a, 1.0f - s, 1.0f);
        return a * s;
    } else {
        g = 1.0f;
        return a;
    }
}

}  // namespace moe
