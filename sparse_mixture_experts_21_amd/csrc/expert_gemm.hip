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
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation, issued as
// D[n][m] = W^T[n][k] . X^T[k][m] so each lane of the epilogue owns 4
// consecutive output columns (8-byte stores).  Operands move HBM -> LDS with
// buffer_load ... lds (no VGPR staging) through 4 LDS stages of a 32-deep
// k-tile, issued 3 k-tiles ahead of the MFMAs.  The weights stay in their
// natural [k][n] layout in LDS and are turned into K-contiguous MFMA
// fragments by ds_read_b64_tr_b16; the rows of X are [m][k] in LDS.  LDS
// fragment reads for the next k-substep are interleaved with the MFMAs of
// the current one, and one barrier per k-tile orders DMA and reads.
#include "moe_internal.h"
#include "lds_dma.h"

namespace moe {
namespace {

enum Act { kActNone = 0, kActGelu = 1 };

// Exact (erf) GELU, 0.5 a (1 + erf(a / sqrt 2)), with erf evaluated by formula
// 7.1.26 of Abramowitz & Stegun, Handbook of Mathematical Functions:
//   erf(u) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-u^2),
//   t = 1 / (1 + p u), u >= 0, |error| <= 1.5e-7,
// i.e. below fp32 rounding of GELU's output scale and far below bf16.  One
// reciprocal and one exponential, no branches.
__device__ __forceinline__ float gelu_erf(float a) {
    const float u = fabsf(a) * 0.70710678118654752440f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, u, 1.0f));
    float poly = fmaf(t, 1.061405429f, -1.453152027f);
    poly = fmaf(t, poly, 1.421413741f);
    poly = fmaf(t, poly, -0.284496736f);
    poly = fmaf(t, poly, 0.254829592f);
    const float q = t * poly * __expf(-u * u);          // 1 - erf(|a| / sqrt 2)
    return 0.5f * a * ((a >= 0.0f) ? 2.0f - q : q);
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
#ifndef MOE_GEMM_BK
#define MOE_GEMM_BK 32
#endif
#ifndef MOE_GEMM_NS
#define MOE_GEMM_NS 4
#endif
template <int BM>
struct Cfg {
    static constexpr int BN = 256, BK = MOE_GEMM_BK;  // k-tile depth
    static constexpr int NS = MOE_GEMM_NS;            // LDS stages
    static constexpr int WM = (BM == 256) ? 2 : 1;   // waves along m
    static constexpr int WN = 4 / WM;                // waves along n
    static constexpr int TN = BN / WN, TM = BM / WM; // per-wave extent
    static constexpr int FN = TN / 32, FM = TM / 32; // 32x32 MFMA tiles per wave
    static constexpr int W_BYTES = BK * BN * 2;      // weight tile [BK][BN], 512-byte rows
    static constexpr int X_BYTES = BM * BK * 2;      // row tile [BM][BK], 2 BK-byte rows
    static constexpr int CPR = BK / 8;               // 16-byte chunks per X row
    static constexpr int RPB = 64 / CPR;             // X rows per 1 KB DMA block
    static constexpr int RSH = (CPR == 4) ? 2 : 1;   // X swizzle: chunk ^= (m >> RSH) % CPR
    static constexpr int STAGE = W_BYTES + X_BYTES;
    static constexpr int WI = W_BYTES / 4096;        // 1 KB DMA blocks per wave (weights)
    static constexpr int XI = X_BYTES / 4096;        // 1 KB DMA blocks per wave (rows)
    static_assert(BK == 32 || BK == 64, "k-tile depth");
    static_assert(NS >= 2, "stages");
    static constexpr int OP = BN * 2 + 16;           // output staging row pitch (bytes)
    static constexpr int BM_ROWS = BM;
    static constexpr int LDS_BYTES = (NS * STAGE > BM * OP) ? NS * STAGE : BM * OP;
};

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;

// Workgroup -> (row tile, column tile).  The grid is a sequence of
// super-blocks of 256 tiles (SBM row tiles x SBN column tiles, one tile per
// CU), walked row-major.  The hardware deals workgroups to the 8 XCDs
// round-robin, so position p of a super-block runs on XCD p % 8; each XCD
// gets an 8 x 4 sub-block of it (rotating with the super-block index).  Inside an XCD the ~32 resident tiles share
// their row and weight slabs in its L2; across XCDs the whole chip works on
// one super-block at a time, so slabs another XCD already pulled are served
// from the memory-side cache instead of HBM.  Positions past the last real
// tile return at once.
__device__ __forceinline__ void tile_coords(int b, int SBN, int nsbn, int nsbm, int& mt, int& nt) {
    const int sb = b >> 8, p = b & 255;
    const int x = p & 7, j = p >> 3;                     // XCD, slot on the XCD
#ifdef MOE_GEMM_SB_COLMAJOR
    const int sbm = sb % nsbm, sbn = sb / nsbm;
#else
    const int sbm = sb / nsbn, sbn = sb % nsbn;
    (void)nsbm;
#endif
    // XCD x takes sub-block (x + sb) % 8: the rotation spreads the tiles of a
    // partial (ragged) super-block over all XCDs instead of a fixed few
    const int s8 = (x + sb) & 7;
    const int xm = s8 % (256 / SBN / 8), xn = s8 / (256 / SBN / 8);  // sub-block
    mt = sbm * (256 / SBN) + xm * 8 + (j & 7);
    nt = sbn * SBN + xn * 4 + (j >> 3);
}

// LDS layouts (per stage):
//   weights [k][n]: 32 rows of 512 bytes; 16-byte chunk c of row k is stored
//     at chunk c ^ (4 (k & 3)).  A-fragments are read with ds_read_b64_tr_b16:
//     in each 16-lane group, source lane s reads 4 consecutive n of row
//     k0 + s/4 and lane i receives k0..k0+3 of column n0 + i, i.e. the
//     K-contiguous operand the MFMA wants, from an N-contiguous tile.
//   rows [m][k]: rows of 2 BK bytes; chunk c of row m is stored at
//     c ^ ((m >> RSH) % CPR), RSH = log2(16 / CPR).
// Both swizzles make every fragment read land in 16 distinct 16-byte bank
// slots per 16 lanes; the DMA writes are 1 KB contiguous per instruction.
template <int BM, int ACT>
__global__ __launch_bounds__(256) void ffn_gemm_bf16(
    const uint16_t* __restrict__ X, uint32_t x_bytes, const int32_t* __restrict__ rowmap,
    const int32_t* __restrict__ offsets, int E, const uint16_t* __restrict__ W,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ C, int K, int N, int Mt, int Nt,
    int SBN) {
    using G = Cfg<BM>;
    __shared__ __attribute__((aligned(1024))) char lds[G::LDS_BYTES];

    int mt, nt;
    tile_coords(blockIdx.x, SBN, (Nt + SBN - 1) / SBN, (Mt + 256 / SBN - 1) / (256 / SBN), mt, nt);
    int e, m0, row_begin, n_rows;
    if (nt >= Nt || mt >= Mt) return;
    if (!find_tile<BM>(offsets, E, mt, e, m0, row_begin, n_rows)) return;
    const int n0 = nt * G::BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave % G::WN, wm = wave / G::WN;
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;

    // ---- DMA sources (byte offsets; fixed for the whole k loop except + k0)
    const __amdgpu_buffer_rsrc_t x_rsrc = make_rsrc(X, x_bytes);
    const __amdgpu_buffer_rsrc_t w_rsrc =
        make_rsrc(W + (int64_t)e * K * N, (uint32_t)K * (uint32_t)N * 2u);
    uint32_t woff[G::WI];
#pragma unroll
    for (int q = 0; q < G::WI; ++q) {
        const int blk = 4 * q + wave;                       // 1 KB block = 2 weight rows
        const int k = 2 * blk + (lane >> 5);
        const int c = (lane & 31) ^ (4 * (k & 3));           // logical 16-byte chunk
        woff[q] = (uint32_t)k * (uint32_t)N * 2u + (uint32_t)(n0 + 8 * c) * 2u;
    }
    uint32_t xoff[G::XI];
    int xk[G::XI];
#pragma unroll
    for (int q = 0; q < G::XI; ++q) {
        const int blk = 4 * q + wave;                       // 1 KB block = RPB rows
        const int row = G::RPB * blk + lane / G::CPR;
        const int c = (lane % G::CPR) ^ ((row >> G::RSH) % G::CPR);
        const int r = row_begin + min(m0 + row, n_rows - 1);
        const uint32_t src = rowmap ? (uint32_t)rowmap[r] : (uint32_t)r;
        xoff[q] = src * (uint32_t)K * 2u + (uint32_t)c * 16u;
        xk[q] = 8 * c;
    }
    const uint32_t wstep = (uint32_t)G::BK * (uint32_t)N * 2u;

    // DMA number q (0 <= q < WI + XI) of k-tile t, into stage t % NS.  k-tiles
    // past the end read at out-of-range offsets and fill the stage with zeros.
    auto issue_one = [&](int t, int q) {
        const uint32_t st = lds0 + (uint32_t)((t % G::NS) * G::STAGE);
        const int k0 = t * G::BK;
        if (q < G::WI) {
            dma16(w_rsrc, woff[q] + (uint32_t)t * wstep,
                  __builtin_amdgcn_readfirstlane(st + (uint32_t)((4 * q + wave) * 1024)));
        } else {
            const int qx = q - G::WI;
            const uint32_t o = (k0 + xk[qx] < K) ? xoff[qx] + (uint32_t)k0 * 2u : kOob;
            dma16(x_rsrc, o,
                  __builtin_amdgcn_readfirstlane(st + (uint32_t)(G::W_BYTES + (4 * qx + wave) * 1024)));
        }
    };

    // ---- fragment read addresses (bytes, relative to a stage base)
    const int l32 = lane & 31, half = lane >> 5;
    uint32_t aoff[G::FN], boff[G::FM];
    {
        const int grp = lane >> 4, s16 = lane & 15;
        const int k = 8 * (grp >> 1) + (s16 >> 2);          // + 16 kk, + 4 for the 2nd read
#pragma unroll
        for (int i = 0; i < G::FN; ++i) {
            const int n = wn * G::TN + 32 * i + 16 * (grp & 1) + 4 * (s16 & 3);
            const int pc = (n >> 3) ^ (4 * (k & 3));
            aoff[i] = (uint32_t)(k * 512 + pc * 16 + (n & 4) * 2);
        }
#pragma unroll
        for (int j = 0; j < G::FM; ++j) {
            const int m = wm * G::TM + 32 * j + l32;
            boff[j] = (uint32_t)(m * G::BK * 2);             // + chunk, swizzled per kk
        }
    }
    bf16x8_t fa[2][G::FN], fb[2][G::FM];
    // fragment f (f < FN: weights via two transposed reads; else rows) of
    // k-substep kk of k-tile t into register buffer buf
    auto read_frag = [&](int t, int kk, int buf, int f) {
        const uint32_t st = lds0 + (uint32_t)((t % G::NS) * G::STAGE);
        if (f < G::FN) {
            const uint32_t a = st + aoff[f] + (uint32_t)(kk * 16 * 512);
            const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16_t*)(uintptr_t)a);
            const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16_t*)(uintptr_t)(a + 4 * 512));
            const v8i16_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            fa[buf][f] = __builtin_bit_cast(bf16x8_t, v);
        } else {
            const int j = f - G::FN;
            const int m = wm * G::TM + 32 * j + l32;
            const int pc = (2 * kk + half) ^ ((m >> G::RSH) % G::CPR);
            const uint32_t b = st + G::W_BYTES + boff[j] + (uint32_t)(pc * 16);
            fb[buf][j] = *(const lds_bf16x8_t*)(uintptr_t)b;
        }
    };
    // Fragments in the order the next substep's MFMAs consume them (row-major
    // over the accumulator tiles): A0, B0..B(FM-1), A1..A(FN-1).
    auto frag_id = [](int o) { return o == 0 ? 0 : (o <= G::FM ? G::FN + o - 1 : o - G::FM); };
    auto read_frags = [&](int t, int kk, int buf) {
#pragma unroll
        for (int o = 0; o < G::FN + G::FM; ++o) read_frag(t, kk, buf, frag_id(o));
    };

    f32x16_t acc[G::FN][G::FM];
#pragma unroll
    for (int i = 0; i < G::FN; ++i)
#pragma unroll
        for (int j = 0; j < G::FM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    // MFMAs number lo..hi-1 (row-major over the FN x FM accumulator tiles)
    auto mfma_range = [&](int buf, int lo, int hi) {
#pragma unroll
        for (int x = 0; x < G::FN * G::FM; ++x) {
            if (x < lo || x >= hi) continue;
            const int i = x / G::FM, j = x % G::FM;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j],
                                                                acc[i][j], 0, 0, 0);
        }
    };
    auto mfma = [&](int buf) { mfma_range(buf, 0, G::FN * G::FM); };
    constexpr int NMF = G::FN * G::FM;
    constexpr int NRD = 2 * G::FN + G::FM;   // LDS read instructions per substep
    constexpr int NDMA = G::WI + G::XI;      // DMA instructions per wave per k-tile

    // ---- pipeline: DMA runs NS-1 k-tiles ahead of the MFMAs.  The DMAs of a
    // k-tile are spread over two substeps (H1 of them in the last substep of
    // k-tile kt, after the barrier that frees their stage, the other H2 in the
    // first substep of k-tile kt+1), one at a time between MFMAs, so the
    // address units never see a burst that would stall the wave's issue.
    constexpr int H1 = (NDMA + 1) / 2, H2 = NDMA - H1;
    constexpr int NSUB = G::BK / 16;         // 16-deep MFMA k-substeps per k-tile
    constexpr int NF = G::FN + G::FM;        // fragments per substep
    // the fragment reads of a substep go into its first half of MFMA groups,
    // so they land well before the next substep's first MFMA needs them
    constexpr int RG2 = H2 > 1 ? H2 / 2 : 1, RG1 = H1 > 1 ? H1 / 2 : 1;
    const int nk = (K + G::BK - 1) / G::BK;
#pragma unroll
    for (int t = 0; t + 1 < G::NS; ++t)
#pragma unroll
        for (int q = 0; q < NDMA; ++q) issue_one(t, q);
#pragma unroll
    for (int q = 0; q < H1; ++q) issue_one(G::NS - 1, q);
    wait_vmcnt<(G::NS - 2) * NDMA + H1>();
    lds_barrier();
    read_frags(0, 0, 0);

    for (int kt = 0; kt < nk; ++kt) {
        // substep 0: MFMAs of substep 0 || fragments of substep 1 || the rest
        // of k-tile kt+NS-1's DMAs (its stage was freed one barrier ago)
#pragma unroll
        for (int g = 0; g < H2; ++g) {
            __builtin_amdgcn_sched_barrier(0);
            issue_one(kt + G::NS - 1, H1 + g);
            mfma_range(0, g * NMF / H2, (g + 1) * NMF / H2);
            if (g < RG2) {
#pragma unroll
                for (int o = g * NF / RG2; o < (g + 1) * NF / RG2; ++o)
                    read_frag(kt, 1, 1, frag_id(o));
            }
#pragma unroll
            for (int q = 0; q < NMF; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (q < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
        }
        if (H2 == 0) {
            __builtin_amdgcn_sched_barrier(0);
            read_frags(kt, 1, 1);
            mfma(0);
#pragma unroll
            for (int q = 0; q < NMF; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (q < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
        // substeps 1..NSUB-2 (deeper k-tiles only)
#pragma unroll
        for (int sub = 1; sub + 1 < NSUB; ++sub) {
            __builtin_amdgcn_sched_barrier(0);
            read_frags(kt, sub + 1, (sub + 1) & 1);
            mfma(sub & 1);
#pragma unroll
            for (int q = 0; q < NMF; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (q < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // tile kt+1 complete in every wave's view; nobody reads stage kt % NS any more
        wait_vmcnt<(G::NS - 2) * NDMA>();
        wait_lgkm0();
        lds_barrier();
        // last substep: MFMAs || first fragments of tile kt+1 || DMAs of tile kt+NS
#pragma unroll
        for (int g = 0; g < H1; ++g) {
            __builtin_amdgcn_sched_barrier(0);
            issue_one(kt + G::NS, g);
            mfma_range((NSUB - 1) & 1, g * NMF / H1, (g + 1) * NMF / H1);
            if (g < RG1) {
#pragma unroll
                for (int o = g * NF / RG1; o < (g + 1) * NF / RG1; ++o)
                    read_frag(kt + 1, 0, 0, frag_id(o));
            }
#pragma unroll
            for (int q = 0; q < NMF; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (q < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();

    // ---- epilogue.  D[n][m]: a lane owns m = l32 and n = 8 g + 4 half + 0..3 of
    // each 32x32 tile.  Bias and activation in fp32, one rounding to bf16, then
    // the whole output tile is staged in LDS ([m][n], 528-byte pitch: the
    // 8-byte writes of 16 consecutive rows and the 16-byte reads of one row are
    // both bank-conflict free) and written out as full contiguous row
    // segments, so every 128-byte line of the output is written once.
    wait_lgkm0();
    lds_barrier();
    const uint16_t* be = bias ? bias + (int64_t)e * N : nullptr;
#pragma unroll
    for (int i = 0; i < G::FN; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int nl = wn * G::TN + 32 * i + 8 * g + 4 * half;
            const int n = min(n0 + nl, N - 4);
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
                const int ml = wm * G::TM + 32 * j + l32;
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[q] = acc[i][j][4 * g + q] + bv[q];
                    if (ACT == kActGelu) v[q] = gelu_erf(v[q]);
                }
                u32x2_t o;
                o[0] = pack_bf16x2(v[0], v[1]);
                o[1] = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<u32x2_t*>(lds + ml * G::OP + nl * 2) = o;
            }
        }
    }
    lds_barrier();
    const int rows = min(G::BM_ROWS, n_rows - m0);
    const int chunks = min(G::BN, N - n0) / 8;            // 16-byte chunks per row (N % 8 == 0)
    uint16_t* cbase = C + (int64_t)(row_begin + m0) * N + n0;
    for (int idx = tid; idx < G::BM_ROWS * (G::BN / 8); idx += 256) {
        const int r = idx / (G::BN / 8), c = idx % (G::BN / 8);
        if (r < rows && c < chunks)
            *reinterpret_cast<u32x4_t*>(cbase + (int64_t)r * N + c * 8) =
                *reinterpret_cast<const u32x4_t*>(lds + r * G::OP + c * 16);
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
        // super-block width in column tiles: the widest of 16/8/4 that divides Nt
#ifdef MOE_GEMM_SBN
        const int SBN = MOE_GEMM_SBN;
#else
        const int SBN = (Nt % 16 == 0) ? 16 : (Nt % 8 == 0) ? 8 : 4;
#endif
        const int64_t nsb = (int64_t)((Mt + 256 / SBN - 1) / (256 / SBN)) * ((Nt + SBN - 1) / SBN);
        const dim3 grid((unsigned)(nsb * 256)), block(256);
        auto* x = static_cast<const uint16_t*>(X);
        auto* w = static_cast<const uint16_t*>(W);
        auto* b = static_cast<const uint16_t*>(bias);
        auto* c = static_cast<uint16_t*>(Cout);
        // bytes addressable through X: the token rows (gather) or the kept rows
        const int64_t xrows = rowmap ? p.T : rows;
        const uint32_t xb = (uint32_t)(xrows * K * 2);
        if (bm == 256)
            ffn_gemm_bf16<256, ACT><<<grid, block, 0, s>>>(x, xb, rowmap, offsets, p.E, w, b, c, K, N, Mt, Nt, SBN);
        else if (bm == 128)
            ffn_gemm_bf16<128, ACT><<<grid, block, 0, s>>>(x, xb, rowmap, offsets, p.E, w, b, c, K, N, Mt, Nt, SBN);
        else
            ffn_gemm_bf16<64, ACT><<<grid, block, 0, s>>>(x, xb, rowmap, offsets, p.E, w, b, c, K, N, Mt, Nt, SBN);
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
