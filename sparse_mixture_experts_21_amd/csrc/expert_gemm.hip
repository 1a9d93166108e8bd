// Expert FFN as a grouped GEMM over unequal expert groups ("moe-training"
// SKILL page, Quick Start, Basic MoE Architecture: per expert Linear(H, 4H)
// -> GELU -> Linear(4H, H); the page's explainer on efficient training notes
// that batched matmuls assume equal group sizes, which this kernel does not).
//
//   up:   h[r] = GELU(X[r] . W1[e] + b1[e])     (K = H, N = F)
//   down: y[r] = h[r] . W2[e] + b2[e]           (K = F, N = H)
// for the rows offsets[e] <= r < offsets[e+1] of every expert e.
//
// Tiles never straddle experts and are never padded to capacity: the grid is
// sized for the worst case (T k / BM + E row tiles) and each workgroup finds
// its expert and row tile from `offsets` on the device, so no host
// synchronisation is needed; surplus workgroups return at once and experts
// with no rows cost nothing (their weights are never read).
//
// bf16 kernel (gfx950): 256 threads, tile BN = 256 output columns x BM rows,
// BK = 64, v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  The MFMA is
// issued as D[n][m] = W^T[n][k] . X^T[k][m], so both LDS tiles are stored
// K-contiguous ([n][k] and [m][k], 128-byte rows, 16-byte chunks XOR-swizzled
// by row to spread banks) and each lane of the epilogue owns 4 consecutive
// output columns -> 8-byte stores.  The weights arrive [k][n] (N-contiguous):
// each thread loads an 8 x 8 block (8 rows of 16 bytes), transposes it in
// registers and writes 8 K-contiguous 16-byte chunks.  Two LDS stages: the
// global loads of tile k+1 are in flight while tile k is multiplied.
#include "moe_internal.h"

namespace moe {
namespace {

enum Act { kActNone = 0, kActGelu = 1 };

__device__ __forceinline__ float gelu_erf(float a) {
    return 0.5f * a * (1.0f + erff(a * 0.70710678118654752440f));
}

// Locate the expert and row tile of row-tile index mt.  Returns false when mt
// is beyond the last real tile.
template <int BM>
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int E, int mt,
                                          int& e_out, int& m0, int& row_begin, int& n_rows) {
    int base = 0;
    for (int e = 0; e < E; ++e) {
        const int b = offsets[e], n = offsets[e + 1] - b;
        const int tiles = (n + BM - 1) / BM;
        if (mt < base + tiles) {
            e_out = e;
            m0 = (mt - base) * BM;
            row_begin = b;
            n_rows = n;
            return true;
        }
        base += tiles;
    }
    return false;
}

// ---------------------------------------------------------------- bf16 MFMA
template <int BM>
struct Cfg {
    static constexpr int BN = 256, BK = 64;
    static constexpr int WM = (BM == 256) ? 2 : 1;   // waves along m
    static constexpr int WN = 4 / WM;                // waves along n
    static constexpr int TN = BN / WN, TM = BM / WM; // per-wave extent
    static constexpr int FN = TN / 32, FM = TM / 32; // 32x32 MFMA tiles per wave
    static constexpr int XCH = BM * 8 / 256;         // X 16-byte chunks per thread per k-tile
    static constexpr int STAGE = (BN + BM) * BK;     // bf16 elements per LDS stage
};

__device__ __forceinline__ int swz(int row, int chunk) { return (chunk ^ (row & 7)) << 3; }

template <int BM, int ACT>
__global__ __launch_bounds__(256) void ffn_gemm_bf16(
    const uint16_t* __restrict__ X, const int32_t* __restrict__ rowmap,
    const int32_t* __restrict__ offsets, int E, const uint16_t* __restrict__ W,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ C, int K, int N, int Mt_max) {
    using G = Cfg<BM>;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * G::STAGE];

    const int mt = blockIdx.x % Mt_max;
    const int nt = blockIdx.x / Mt_max;
    int e, m0, row_begin, n_rows;
    if (!find_tile<BM>(offsets, E, mt, e, m0, row_begin, n_rows)) return;
    const int n0 = nt * G::BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave % G::WN, wm = wave / G::WN;

    // ---- per-thread global source addresses
    const uint16_t* xsrc[G::XCH];
    int xrow[G::XCH], xchk[G::XCH];
#pragma unroll
    for (int i = 0; i < G::XCH; ++i) {
        const int lin = tid + 256 * i;
        xrow[i] = lin >> 3;
        xchk[i] = lin & 7;
        const int r = row_begin + min(m0 + xrow[i], n_rows - 1);
        const int64_t src = rowmap ? (int64_t)rowmap[r] : (int64_t)r;
        xsrc[i] = X + src * K + xchk[i] * 8;
    }
    const int kb = tid >> 5, nb = tid & 31;            // this thread's 8x8 weight block
    const bool wcol_ok = (n0 + nb * 8) < N;
    const uint16_t* wsrc = W + (int64_t)e * K * N + (int64_t)(kb * 8) * N + n0 + nb * 8;

    u32x4_t xr[G::XCH];
    u32x4_t wr[8];

    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < G::XCH; ++i) {
            xr[i] = u32x4_t{0u, 0u, 0u, 0u};
            if (k0 + xchk[i] * 8 < K) xr[i] = *reinterpret_cast<const u32x4_t*>(xsrc[i] + k0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            wr[i] = u32x4_t{0u, 0u, 0u, 0u};
            if (wcol_ok && k0 + kb * 8 + i < K)
                wr[i] = *reinterpret_cast<const u32x4_t*>(wsrc + (int64_t)(k0 + i) * N);
        }
    };
    auto store_tile = [&](int stage) {
        uint16_t* ws_ = lds + stage * G::STAGE;            // [BN][BK]
        uint16_t* xs_ = ws_ + G::BN * G::BK;               // [BM][BK]
#pragma unroll
        for (int i = 0; i < G::XCH; ++i)
            *reinterpret_cast<u32x4_t*>(xs_ + xrow[i] * G::BK + swz(xrow[i], xchk[i])) = xr[i];
        // 8x8 transpose: column j of the block = k values kb*8..kb*8+7 of n = nb*8 + j
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int d = j >> 1;
            u32x4_t o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t lo = wr[2 * q][d], hi = wr[2 * q + 1][d];
                o[q] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                               : ((lo & 0xffffu) | (hi << 16));
            }
            const int n = nb * 8 + j;
            *reinterpret_cast<u32x4_t*>(ws_ + n * G::BK + swz(n, kb)) = o;
        }
    };

    f32x16_t acc[G::FN][G::FM];
#pragma unroll
    for (int i = 0; i < G::FN; ++i)
#pragma unroll
        for (int j = 0; j < G::FM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = (K + G::BK - 1) / G::BK;
    load_tile(0);
    store_tile(0);
    __syncthreads();

    const int half = lane >> 5, l32 = lane & 31;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_tile((kt + 1) * G::BK);
        const uint16_t* ws_ = lds + cur * G::STAGE;
        const uint16_t* xs_ = ws_ + G::BN * G::BK;
#pragma unroll
        for (int kk = 0; kk < G::BK / 16; ++kk) {
            const int chunk = 2 * kk + half;
            bf16x8_t a[G::FN], b[G::FM];
#pragma unroll
            for (int i = 0; i < G::FN; ++i) {
                const int n = wn * G::TN + 32 * i + l32;
                a[i] = *reinterpret_cast<const bf16x8_t*>(ws_ + n * G::BK + swz(n, chunk));
            }
#pragma unroll
            for (int j = 0; j < G::FM; ++j) {
                const int m = wm * G::TM + 32 * j + l32;
                b[j] = *reinterpret_cast<const bf16x8_t*>(xs_ + m * G::BK + swz(m, chunk));
            }
#pragma unroll
            for (int i = 0; i < G::FN; ++i)
#pragma unroll
                for (int j = 0; j < G::FM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j],
                                                                        0, 0, 0);
        }
        if (kt + 1 < nk) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: D[n][m]; lane owns m = l32 and n = 8 g + 4 half + 0..3
    const uint16_t* be = bias ? bias + (int64_t)e * N : nullptr;
#pragma unroll
    for (int i = 0; i < G::FN; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n = n0 + wn * G::TN + 32 * i + 8 * g + 4 * half;
            if (n >= N) continue;
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if (be) {
                const u32x2_t bb = *reinterpret_cast<const u32x2_t*>(be + n);
                bv[0] = bf16_lo(bb[0]);
                bv[1] = bf16_hi(bb[0]);
                bv[2] = bf16_lo(bb[1]);
                bv[3] = bf16_hi(bb[1]);
            }
#pragma unroll
            for (int j = 0; j < G::FM; ++j) {
                const int m = m0 + wm * G::TM + 32 * j + l32;
                if (m >= n_rows) continue;
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[q] = acc[i][j][4 * g + q] + bv[q];
                    if (ACT == kActGelu) v[q] = gelu_erf(v[q]);
                }
                u32x2_t o;
                o[0] = pack_bf16x2(v[0], v[1]);
                o[1] = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<u32x2_t*>(C + (int64_t)(row_begin + m) * N + n) = o;
            }
        }
    }
}

// ---------------------------------------------------------------- fp32
// Plain LDS-tiled fp32 FMA kernel for fp32 layers: 64 x 64 tile, BK = 16,
// each of 256 threads computes a 4 x 4 block.
template <int ACT>
__global__ __launch_bounds__(256) void ffn_gemm_f32(const float* __restrict__ X,
                                                    const int32_t* __restrict__ rowmap,
                                                    const int32_t* __restrict__ offsets, int E,
                                                    const float* __restrict__ W,
                                                    const float* __restrict__ bias,
                                                    float* __restrict__ C, int K, int N,
                                                    int Mt_max) {
    constexpr int BM = 64, BN = 64, BK = 16;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[BK][BN + 4];
    const int mt = blockIdx.x % Mt_max;
    const int nt = blockIdx.x / Mt_max;
    int e, m0, row_begin, n_rows;
    if (!find_tile<BM>(offsets, E, mt, e, m0, row_begin, n_rows)) return;
    const int n0 = nt * BN;
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const float* We = W + (int64_t)e * K * N;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int lin = tid + 256 * i;
            const int r = lin >> 4, kk = lin & 15;
            const int row = row_begin + min(m0 + r, n_rows - 1);
            const int64_t src = rowmap ? (int64_t)rowmap[row] : (int64_t)row;
            As[kk][r] = (k0 + kk < K) ? X[src * K + k0 + kk] : 0.f;
            const int kb = lin >> 6, c = lin & 63;
            Bs[kb][c] = (k0 + kb < K && n0 + c < N) ? We[(int64_t)(k0 + kb) * N + n0 + c] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty * 4 + i;
        if (m >= n_rows) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= N) continue;
            float v = acc[i][j] + (bias ? bias[(int64_t)e * N + n] : 0.f);
            if (ACT == kActGelu) v = gelu_erf(v);
            C[(int64_t)(row_begin + m) * N + n] = v;
        }
    }
}

// Row tile height for the bf16 kernel: large tiles when experts hold many
// rows (compute bound), shorter ones when the average expert holds few rows
// (weight streaming; a tall tile would mostly multiply padding).
int pick_bm(const moe_problem_t& p) {
    int64_t cap = p.T;
    if (p.capacity_factor > 0) {
        const double c = std::ceil(p.capacity_factor * (double)(p.T * p.k) / (double)p.E);
        cap = (int64_t)std::min<double>(c, (double)p.T);
    }
    const int64_t avg = std::min<int64_t>((p.T * p.k + p.E - 1) / p.E, cap);
    if (avg <= 64) return 64;
    if (avg <= 128) return 128;
    return 256;
}

template <int ACT>
hipError_t launch_gemm(const moe_problem_t& p, const void* X, const int32_t* rowmap,
                       const int32_t* offsets, const void* W, const void* bias, void* Cout,
                       int K, int N, hipStream_t s) {
    const int64_t rows = p.T * p.k;
    if (p.dtype == MOE_DTYPE_BF16) {
        const int bm = pick_bm(p);
        const int Mt = (int)((rows + bm - 1) / bm + p.E);
        const int Nt = (N + 255) / 256;
        const dim3 grid((unsigned)((int64_t)Mt * Nt)), block(256);
        auto* x = static_cast<const uint16_t*>(X);
        auto* w = static_cast<const uint16_t*>(W);
        auto* b = static_cast<const uint16_t*>(bias);
        auto* c = static_cast<uint16_t*>(Cout);
        if (bm == 256)
            ffn_gemm_bf16<256, ACT><<<grid, block, 0, s>>>(x, rowmap, offsets, p.E, w, b, c, K, N, Mt);
        else if (bm == 128)
            ffn_gemm_bf16<128, ACT><<<grid, block, 0, s>>>(x, rowmap, offsets, p.E, w, b, c, K, N, Mt);
        else
            ffn_gemm_bf16<64, ACT><<<grid, block, 0, s>>>(x, rowmap, offsets, p.E, w, b, c, K, N, Mt);
    } else {
        const int Mt = (int)((rows + 63) / 64 + p.E);
        const int Nt = (N + 63) / 64;
        ffn_gemm_f32<ACT><<<dim3((unsigned)((int64_t)Mt * Nt)), dim3(256), 0, s>>>(
            static_cast<const float*>(X), rowmap, offsets, p.E, static_cast<const float*>(W),
            static_cast<const float*>(bias), static_cast<float*>(Cout), K, N, Mt);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_up(const moe_problem_t& p, const void* xp, const int32_t* rowmap,
                         const int32_t* offsets, const void* W1, const void* b1, void* h,
                         hipStream_t s) {
    return launch_gemm<kActGelu>(p, xp, rowmap, offsets, W1, b1, h, p.H, p.F, s);
}

hipError_t launch_ffn_down(const moe_problem_t& p, const void* h, const int32_t* offsets,
                           const void* W2, const void* b2, void* y, hipStream_t s) {
    return launch_gemm<kActNone>(p, h, nullptr, offsets, W2, b2, y, p.F, p.H, s);
}

}  // namespace moe
