// Expert FFN as a grouped GEMM over unequal expert groups ("moe-training"
// SKILL page, Quick Start, Basic MoE Architecture: per expert Linear(H, 4H)
// -> GELU -> Linear(4H, H); the page's explainer on efficient training notes
// that batched matmuls assume equal group sizes, which this kernel does not).
//
//   up:   h[r] = act(X[r] . W1[e] + b1[e])      (K = H, N = F)
//   down: y[r] = h[r] . W2[e] + b2[e]           (K = F, N = H)
// for the rows offsets[e] <= r < offsets[e+1] of every expert e, with act the
// exact GELU, or SiLU for the Mixtral 8x7B expert (same page, Advanced
// Patterns: bias-free Linear -> SiLU -> Linear experts).
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
// buffer_load ... lds (no VGPR staging) through a ring of LDS stages (2 of
// 64-deep k-tiles for 256-row tiles, 4 of 32-deep ones for the narrower
// layouts, or 3 when two workgroups share a CU), issued NS - 1 k-tiles ahead
// of the MFMAs.  The weights stay in their
// natural [k][n] layout in LDS and are turned into K-contiguous MFMA
// fragments by ds_read_b64_tr_b16; the rows of X are [m][k] in LDS.  LDS
// fragment reads for the next k-substep are interleaved with the MFMAs of
// the current one, and one barrier per k-tile orders DMA and reads.
//
// Load balance: when the real tiles leave a ragged last round of at most half
// the workgroup slots, those tiles are cut along K into slices that fill one whole round
// and write fp32 partials; ffn_gemm_fixup sums them in slice order and applies
// the epilogue (bias, activation, bf16).  In the inference forward the second
// GEMM's partials go to the combine instead, which does the same for the
// rows it reads (launch_ffn_down with fixup = false).
#include <type_traits>

#include "moe_internal.h"
#include "lds_dma.h"
#include "gemm_common.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- bf16 MFMA
// k-tile depth and LDS stages: the 256-row layout takes 64-deep k-tiles in 2
// stages (one barrier per 64 k, 128 KB of LDS); the narrower layouts, which
// stream weights, keep 32-deep k-tiles in 4 stages (prefetch 3 k-tiles ahead),
// or NSV stages where a kernel overrides it (3 stages, 72 KB at 128 rows, so
// that two workgroups share a CU).
template <int BM, int NSV = 0>
struct Cfg {
    static constexpr int BN = 256;
    static constexpr int BK = BM == 256 ? 64 : 32;    // k-tile depth
    static constexpr int NS = NSV ? NSV : (BM == 256 ? 2 : 4);   // LDS stages
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
    static constexpr int UNIT = BM * BN;             // floats of one fp32 partial tile
};

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;

// The last (R mod ncu) tiles would leave most CUs idle in a final, ragged
// round: plan_tail cuts them along K when they are at most half a round.  Few
// tiles (a few tokens per expert) are the same case: every tile is a tail
// tile, and the partials cover only the tiles' real rows.
template <int BM, int NSV>
__device__ __forceinline__ TailPlan tail_plan(const int32_t* __restrict__ offsets, int E, int Nt,
                                              int ncu, int nk, bool allow) {
    const int mtiles = __builtin_amdgcn_readfirstlane(real_row_tiles<BM>(offsets, E));
    return plan_tail(mtiles, Nt, ncu, nk, Cfg<BM, NSV>::NS, allow);
}

// Expert, row range and column offset of tile (mt, nt).
struct TileRef {
    int e, m0, row_begin, n_rows, n0;
};

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
// DMA pipeline and MFMA loop over the k-tiles [kb, kb + nkr) of tile `tr`,
// accumulating into acc (the caller zeroes it).  `lds` holds Cfg<BM>::LDS_BYTES.
// NTW: weight loads carry the nontemporal hint (see ffn_gemm_bf16).
template <int BM, bool NTW, int NSV>
__device__ __forceinline__ void gemm_mainloop(
    const TileRef& tr, int kb, int nkr, char* lds, const uint16_t* __restrict__ X,
    uint32_t x_bytes, const int32_t* __restrict__ rowmap, const uint16_t* __restrict__ W, int K,
    int N, f32x16_t (&acc)[Cfg<BM>::FN][Cfg<BM>::FM]) {
    using G = Cfg<BM, NSV>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave % G::WN, wm = wave / G::WN;
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;

    // ---- DMA sources (byte offsets; fixed for the whole k loop except + k0).
    // Contiguous rows: the resource starts at the tile's first row, so only one
    // tile has to fit the 32-bit offsets.  Gathered rows (rowmap): it spans X.
    const int tile_rows = min(BM, tr.n_rows - tr.m0);
    const __amdgpu_buffer_rsrc_t x_rsrc =
        rowmap ? make_rsrc(X, x_bytes)
               : make_rsrc(X + (int64_t)(tr.row_begin + tr.m0) * K,
                           (uint32_t)tile_rows * (uint32_t)K * 2u);
    const __amdgpu_buffer_rsrc_t w_rsrc =
        make_rsrc(W + (int64_t)tr.e * K * N, (uint32_t)K * (uint32_t)N * 2u);
    uint32_t woff[G::WI];
#pragma unroll
    for (int q = 0; q < G::WI; ++q) {
        const int blk = 4 * q + wave;                       // 1 KB block = 2 weight rows
        const int k = 2 * blk + (lane >> 5);
        const int c = (lane & 31) ^ (4 * (k & 3));           // logical 16-byte chunk
        woff[q] = (uint32_t)k * (uint32_t)N * 2u + (uint32_t)(tr.n0 + 8 * c) * 2u;
    }
    uint32_t xoff[G::XI];
    int xk[G::XI];
#pragma unroll
    for (int q = 0; q < G::XI; ++q) {
        const int blk = 4 * q + wave;                       // 1 KB block = RPB rows
        const int row = G::RPB * blk + lane / G::CPR;
        const int c = (lane % G::CPR) ^ ((row >> G::RSH) % G::CPR);
        const int rr = min(row, tile_rows - 1);             // row within the tile
        const uint32_t src =
            rowmap ? (uint32_t)rowmap[tr.row_begin + tr.m0 + rr] : (uint32_t)rr;
        xoff[q] = src * (uint32_t)K * 2u + (uint32_t)c * 16u;
        xk[q] = 8 * c;
    }
    const uint32_t wstep = (uint32_t)G::BK * (uint32_t)N * 2u;

    // DMA number q (0 <= q < WI + XI) of k-tile kb + t, into stage t % NS.
    // k-tiles past K read at out-of-range offsets and fill the stage with zeros.
    auto issue_one = [&](int t, int q) {
        const uint32_t st = lds0 + (uint32_t)((t % G::NS) * G::STAGE);
        const int k0 = (kb + t) * G::BK;
        if (q < G::WI) {
            const uint32_t o = woff[q] + (uint32_t)(kb + t) * wstep;
            const uint32_t l = __builtin_amdgcn_readfirstlane(st + (uint32_t)((4 * q + wave) * 1024));
            if constexpr (NTW) dma16_nt(w_rsrc, o, l);
            else dma16(w_rsrc, o, l);
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
    const int nk = nkr;
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
}

// The staged tile (LDS [m][n], pitch Cfg<BM>::OP) to out as full rows.  The
// caller has passed an LDS barrier after writing it.
template <int BM>
__device__ __forceinline__ void store_staged(const TileRef& tr, const char* lds,
                                             uint16_t* __restrict__ out, int N) {
    using G = Cfg<BM>;
    const int rows = min(G::BM_ROWS, tr.n_rows - tr.m0);
    const int chunks = min(G::BN, N - tr.n0) / 8;         // 16-byte chunks per row (N % 8 == 0)
    uint16_t* cbase = out + (int64_t)(tr.row_begin + tr.m0) * N + tr.n0;
    for (int idx = threadIdx.x; idx < G::BM_ROWS * (G::BN / 8); idx += 256) {
        const int r = idx / (G::BN / 8), c = idx % (G::BN / 8);
        if (r < rows && c < chunks)
            *reinterpret_cast<u32x4_t*>(cbase + (int64_t)r * N + c * 8) =
                *reinterpret_cast<const u32x4_t*>(lds + r * G::OP + c * 16);
    }
}

// Bias, activation, bf16 and the store of tile `tr` from the accumulators.
// D[n][m]: a lane owns m = l32 and n = 8 g + 4 half + 0..3 of each 32x32 tile.
// The tile is staged in LDS ([m][n], 528-byte pitch: the 8-byte writes of 16
// consecutive rows and the 16-byte reads of one row are both bank-conflict
// free) and written out as full contiguous row segments, so every 128-byte
// line of the output is written once.  Bias and activation are applied in
// fp32 with one rounding to bf16.  SAVE (training): the activation's
// derivative act'(a) at the same fp32 pre-activation, from the same
// evaluation, is rounded to bf16 and written to Cpre; the backward multiplies
// by it.  Then the tile goes out in two halves of its rows (each wave's
// accumulator rows j < FM/2, then the rest), h and act' staged side by side in
// the same LDS, so both are written as full rows.
template <int BM, int ACT, bool SAVE>
__device__ __forceinline__ void gemm_epilogue(const TileRef& tr,
                                              f32x16_t (&acc)[Cfg<BM>::FN][Cfg<BM>::FM],
                                              char* lds, const uint16_t* __restrict__ bias,
                                              uint16_t* __restrict__ C, uint16_t* __restrict__ Cpre,
                                              int N) {
    using G = Cfg<BM>;
    wait_lgkm0();
    lds_barrier();
    const uint16_t* be = bias ? bias + (int64_t)tr.e * N : nullptr;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wn = wave % G::WN, wm = wave / G::WN;
    const int l32 = lane & 31, half = lane >> 5;
    // bias of the lane's columns 32 i + 8 g + 4 half + 0..3
    auto bias4 = [&](int nl, float (&bv)[4]) {
        bv[0] = bv[1] = bv[2] = bv[3] = 0.f;
        if (be) {
            const u32x2_t bb = *reinterpret_cast<const u32x2_t*>(be + min(tr.n0 + nl, N - 4));
            bv[0] = bf16_lo(bb[0]);
            bv[1] = bf16_hi(bb[0]);
            bv[2] = bf16_lo(bb[1]);
            bv[3] = bf16_hi(bb[1]);
        }
    };
    if constexpr (!SAVE) {
        // with and without bias (the bias-free layers skip the add)
        auto stage = [&](auto HB) {
            constexpr bool kBias = decltype(HB)::value != 0;
#pragma unroll
            for (int i = 0; i < G::FN; ++i) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int nl = wn * G::TN + 32 * i + 8 * g + 4 * half;
                    float bv[4] = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (kBias) bias4(nl, bv);
#pragma unroll
                    for (int j = 0; j < G::FM; ++j) {
                        const int ml = wm * G::TM + 32 * j + l32;
                        float v[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            v[q] = activate<ACT>(kBias ? acc[i][j][4 * g + q] + bv[q]
                                                       : acc[i][j][4 * g + q]);
                        const u32x2_t o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                        *reinterpret_cast<u32x2_t*>(lds + ml * G::OP + nl * 2) = o;
                    }
                }
            }
        };
        if (be) stage(std::integral_constant<int, 1>{});
        else stage(std::integral_constant<int, 0>{});
        lds_barrier();
        store_staged<BM>(tr, lds, C, N);
    } else {
        constexpr int HJ = G::FM / 2;                  // accumulator rows per half
        constexpr int HR = G::TM / 2;                  // a wave's rows per half
        constexpr int HROWS = G::WM * HR;              // staged rows per half
        constexpr int GOFF = HROWS * G::OP;            // act' region after the h region
        static_assert(2 * GOFF <= G::LDS_BYTES, "two half tiles fit the staging LDS");
        const int rows = min(G::BM_ROWS, tr.n_rows - tr.m0);
        const int chunks = min(G::BN, N - tr.n0) / 8;
        const int64_t origin = (int64_t)(tr.row_begin + tr.m0) * N + tr.n0;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            if (hh) lds_barrier();                     // the first half has been copied out
#pragma unroll
            for (int i = 0; i < G::FN; ++i) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int nl = wn * G::TN + 32 * i + 8 * g + 4 * half;
                    float bv[4];
                    bias4(nl, bv);
#pragma unroll
                    for (int jj = 0; jj < HJ; ++jj) {
                        const int j = hh * HJ + jj;
                        const int lr = wm * HR + 32 * jj + l32;      // staged row
                        float v[4], d[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            v[q] = activate_with_grad<ACT>(acc[i][j][4 * g + q] + bv[q], d[q]);
                        const u32x2_t o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                        const u32x2_t gd = {pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3])};
                        *reinterpret_cast<u32x2_t*>(lds + lr * G::OP + nl * 2) = o;
                        *reinterpret_cast<u32x2_t*>(lds + GOFF + lr * G::OP + nl * 2) = gd;
                    }
                }
            }
            lds_barrier();
            for (int idx = threadIdx.x; idx < HROWS * (G::BN / 8); idx += 256) {
                const int lr = idx / (G::BN / 8), c = idx % (G::BN / 8);
                const int r = (lr / HR) * G::TM + hh * HR + lr % HR;  // row of the tile
                if (r < rows && c < chunks) {
                    const int64_t at = origin + (int64_t)r * N + c * 8;
                    *reinterpret_cast<u32x4_t*>(C + at) =
                        *reinterpret_cast<const u32x4_t*>(lds + lr * G::OP + c * 16);
                    *reinterpret_cast<u32x4_t*>(Cpre + at) =
                        *reinterpret_cast<const u32x4_t*>(lds + GOFF + lr * G::OP + c * 16);
                }
            }
        }
    }
}

// fp32 partial tile of one K slice, row-major [BM][BN] (Cfg<BM>::UNIT floats
// per slice); only the tile's real rows are written (and later read), so a
// slice of a tile with a few rows costs a few KB.  A lane holds columns
// 8 g + 4 half + 0..3 of row l32 of each 32x32 MFMA tile (acc[i][j][4 g + q]).
template <int BM>
__device__ __forceinline__ void store_partial(const f32x16_t (&acc)[Cfg<BM>::FN][Cfg<BM>::FM],
                                              float* __restrict__ dst, int rows) {
    using G = Cfg<BM>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wn = wave % G::WN, wm = wave / G::WN;
    const int l32 = lane & 31, half = lane >> 5;
#pragma unroll
    for (int j = 0; j < G::FM; ++j) {
        const int m = wm * G::TM + 32 * j + l32;
        if (m >= rows) continue;
#pragma unroll
        for (int i = 0; i < G::FN; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = wn * G::TN + 32 * i + 8 * g + 4 * half;
                const f32x4_t v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                   acc[i][j][4 * g + 3]};
                *reinterpret_cast<f32x4_t*>(dst + m * G::BN + n) = v;
            }
    }
}

template <int BM>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[Cfg<BM>::FN][Cfg<BM>::FM]) {
#pragma unroll
    for (int i = 0; i < Cfg<BM>::FN; ++i)
#pragma unroll
        for (int j = 0; j < Cfg<BM>::FM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

template <int BM>
__device__ __forceinline__ bool tile_ref(const int32_t* __restrict__ offsets, int E, int mt,
                                         int nt, TileRef& tr) {
    tr.n0 = nt * Cfg<BM>::BN;
    return find_tile<BM>(offsets, E, mt, tr.e, tr.m0, tr.row_begin, tr.n_rows);
}

// One whole tile with the row layout of Cfg<TB> (TB <= the kernel's BM).
template <int TB, int ACT, bool NTW, bool SAVE, int NSV>
__device__ __forceinline__ void whole_tile(const TileRef& tr, char* lds,
                                           const uint16_t* __restrict__ X, uint32_t x_bytes,
                                           const int32_t* __restrict__ rowmap,
                                           const uint16_t* __restrict__ W,
                                           const uint16_t* __restrict__ bias,
                                           uint16_t* __restrict__ C, uint16_t* __restrict__ Cpre,
                                           int K, int N) {
    // k-tiles of this layout's own depth (the layouts differ in k-tile depth)
    const int nk = (K + Cfg<TB>::BK - 1) / Cfg<TB>::BK;
    f32x16_t acc[Cfg<TB>::FN][Cfg<TB>::FM];
    zero_acc<TB>(acc);
    gemm_mainloop<TB, NTW, NSV>(tr, 0, nk, lds, X, x_bytes, rowmap, W, K, N, acc);
    gemm_epilogue<TB, ACT, SAVE>(tr, acc, lds, bias, C, Cpre, N);
}

// Workgroup p: whole tile p (p < full), or one K slice of a tail tile.  `part`
// (nullable) is the fp32 slice buffer; without it no tile is cut.  The last
// row tile of an expert is usually short: with at most 128 (64) real rows it
// runs the 128-row (64-row) layout, whose four waves split the columns instead
// of idling on rows that do not exist.  NSV (0: the layout's own stage count)
// overrides the LDS stages of every layout the kernel runs; with NSV the
// kernel is built for two resident workgroups per CU, and `ncu` counts
// workgroup slots (two per CU) for the round of tiles.
template <int BM, int ACT, bool SAVE, int NSV>
__global__ __launch_bounds__(256, NSV ? 2 : 1) void ffn_gemm_bf16(
    const uint16_t* __restrict__ X, uint32_t x_bytes, const int32_t* __restrict__ rowmap,
    const int32_t* __restrict__ offsets, int E, const uint16_t* __restrict__ W,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ C, uint16_t* __restrict__ Cpre,
    int K, int N, int Nt, int SBN, int ncu, float* __restrict__ part) {
    using G = Cfg<BM, NSV>;
    __shared__ __attribute__((aligned(1024))) char lds[G::LDS_BYTES];
    static_assert(BM < 128 || Cfg<64, NSV>::LDS_BYTES <= G::LDS_BYTES, "64-row layout fits");
    static_assert(BM < 256 || Cfg<128, NSV>::LDS_BYTES <= G::LDS_BYTES, "128-row layout fits");
    // With at most 128 rows per tile (few rows per expert) an expert's weights
    // are read about once, so they stream past the last-level cache instead of
    // evicting (and writing back) other kernels' lines; the 256-row layout
    // re-reads weight tiles across row tiles and keeps the default policy.
    constexpr bool kNtW = BM <= 128;
    const int nk = (K + G::BK - 1) / G::BK;
    const TailPlan pl = tail_plan<BM, NSV>(offsets, E, Nt, ncu, nk, part != nullptr);
    const int p = blockIdx.x;
    int tile = p, kb = 0, nkr = nk, unit = -1;
    if (p >= pl.full) {
        const int u = p - pl.full;
        if (u >= pl.tail * pl.S) return;
        tile = pl.full + u / pl.S;
        const int s = u % pl.S;
        kb = s * nk / pl.S;
        nkr = (s + 1) * nk / pl.S - kb;
        unit = u;
    }
    int mt, nt;
    dense_coords(tile, pl.real_mt, Nt, SBN, mt, nt);
    TileRef tr;
    if (!tile_ref<BM>(offsets, E, mt, nt, tr)) return;
    if (unit < 0) {
        const int rows = tr.n_rows - tr.m0;
        if constexpr (BM >= 128) {
            if (rows <= 64) {
                whole_tile<64, ACT, kNtW, SAVE, NSV>(tr, lds, X, x_bytes, rowmap, W, bias, C, Cpre, K,
                                                  N);
                return;
            }
        }
        if constexpr (BM >= 256) {
            if (rows <= 128) {
                whole_tile<128, ACT, kNtW, SAVE, NSV>(tr, lds, X, x_bytes, rowmap, W, bias, C, Cpre, K,
                                                   N);
                return;
            }
        }
        whole_tile<BM, ACT, kNtW, SAVE, NSV>(tr, lds, X, x_bytes, rowmap, W, bias, C, Cpre, K, N);
        return;
    }
    f32x16_t acc[G::FN][G::FM];
    zero_acc<BM>(acc);
    gemm_mainloop<BM, kNtW, NSV>(tr, kb, nkr, lds, X, x_bytes, rowmap, W, K, N, acc);
    store_partial<BM>(acc, part + (int64_t)unit * G::UNIT, tr.n_rows - tr.m0);
}

// Tail tiles: workgroup (tile i, chunk c) takes rows 16 c .. 16 c + 15 of the
// tile, 4 rows per pass (one per wave), 4 columns per lane: the S slices of
// each 16-byte vector loaded 8 at a time and summed in slice order, then bias,
// activation, one rounding to bf16 and an 8-byte store.  Rows past the tile's
// real rows were never written and are not read.
template <int BM>
struct FixCfg {
    static constexpr int ROWS = 16;                       // rows per workgroup
    static constexpr int CHUNKS = BM / ROWS;              // workgroups per tile
    static constexpr int BATCH = 8;                       // slice loads in flight
};

template <int BM, int ACT, int NSV>
__global__ __launch_bounds__(256) void ffn_gemm_fixup(
    const int32_t* __restrict__ offsets, int E, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ C, uint16_t* __restrict__ Cpre, int K, int N, int Nt, int SBN, int ncu,
    const float* __restrict__ part) {
    using G = Cfg<BM, NSV>;
    const int nk = (K + G::BK - 1) / G::BK;
    const TailPlan pl = tail_plan<BM, NSV>(offsets, E, Nt, ncu, nk, true);
    const int i = blockIdx.x / FixCfg<BM>::CHUNKS, c = blockIdx.x % FixCfg<BM>::CHUNKS;
    if (pl.S < 2 || i >= pl.tail) return;
    int mt, nt;
    dense_coords(pl.full + i, pl.real_mt, Nt, SBN, mt, nt);
    TileRef tr;
    if (!tile_ref<BM>(offsets, E, mt, nt, tr)) return;
    const int rows = min(BM, tr.n_rows - tr.m0);
    const int col = 4 * (threadIdx.x & 63);
    if (tr.n0 + col >= N) return;                         // N % 4 == 0: all 4 columns valid
    const int wave = threadIdx.x >> 6;
    const float* src = part + (int64_t)i * pl.S * G::UNIT + col;
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias) {
        const u32x2_t bb = *reinterpret_cast<const u32x2_t*>(bias + (int64_t)tr.e * N + tr.n0 + col);
        bv[0] = bf16_lo(bb[0]);
        bv[1] = bf16_hi(bb[0]);
        bv[2] = bf16_lo(bb[1]);
        bv[3] = bf16_hi(bb[1]);
    }
    for (int r = c * FixCfg<BM>::ROWS + wave; r < min(rows, (c + 1) * FixCfg<BM>::ROWS); r += 4) {
        const float* p = src + r * G::BN;
        f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
        for (int s0 = 1; s0 < pl.S; s0 += FixCfg<BM>::BATCH) {
            // unconditional loads at clamped slice indices, masked in the sum
            f32x4_t t[FixCfg<BM>::BATCH];
#pragma unroll
            for (int u = 0; u < FixCfg<BM>::BATCH; ++u)
                t[u] = *reinterpret_cast<const f32x4_t*>(
                    p + (int64_t)min(s0 + u, pl.S - 1) * G::UNIT);
#pragma unroll
            for (int u = 0; u < FixCfg<BM>::BATCH; ++u) {
                if (s0 + u < pl.S) {
                    a[0] += t[u][0]; a[1] += t[u][1]; a[2] += t[u][2]; a[3] += t[u][3];
                }
            }
        }
        float o[4];
        const int64_t at = (int64_t)(tr.row_begin + tr.m0 + r) * N + tr.n0 + col;
        u32x2_t w;
        if (Cpre) {                                       // act'(a), kept for the backward
            float d[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = activate_with_grad<ACT>(a[q] + bv[q], d[q]);
            w[0] = pack_bf16x2(d[0], d[1]);
            w[1] = pack_bf16x2(d[2], d[3]);
            *reinterpret_cast<u32x2_t*>(Cpre + at) = w;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = activate<ACT>(a[q] + bv[q]);
        }
        w[0] = pack_bf16x2(o[0], o[1]);
        w[1] = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<u32x2_t*>(C + at) = w;
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
            const float v = activate<ACT>(acc[i][j] + (bias ? bias[(int64_t)e * N + n] : 0.f));
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
    // Few rows per expert: the GEMMs stream weights from HBM, and a row tile
    // that holds a whole expert reads its weights once per column tile.  The
    // 64-row layout only pays off below half a tile on average.
    if (avg <= 32) return 64;
    if (avg <= 128) return 128;
    return 256;
}

int gemm_nt(int N) { return (N + 255) / 256; }

// Every real tile, plus room for one round of K slices; the fixup covers at
// most half a round of tail tiles (each is cut in 2 or more).  `slots`:
// workgroups resident at once (CUs, or twice that with NSV).
template <int BM, int ACT, int NSV>
hipError_t launch_bf16(const uint16_t* x, uint32_t xb, const int32_t* rowmap, const int32_t* offsets,
                 int E, const uint16_t* w, const uint16_t* b, uint16_t* c, uint16_t* cpre, int K,
                 int N, int Mt, int Nt, int SBN, int slots, float* part, hipEvent_t mid,
                 hipStream_t s, bool fixup) {
    const int units = std::min(slots, kMaxUnits);
    const dim3 block(256), grid((unsigned)((int64_t)Mt * Nt + units));
    if (cpre)
        ffn_gemm_bf16<BM, ACT, true, NSV><<<grid, block, 0, s>>>(x, xb, rowmap, offsets, E, w, b,
                                                                 c, cpre, K, N, Nt, SBN, slots,
                                                                 part);
    else
        ffn_gemm_bf16<BM, ACT, false, NSV><<<grid, block, 0, s>>>(x, xb, rowmap, offsets, E, w, b,
                                                                  c, nullptr, K, N, Nt, SBN, slots,
                                                                  part);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && mid) e = hipEventRecord(mid, s);
    if (e != hipSuccess) return e;
    if (part && fixup)
        ffn_gemm_fixup<BM, ACT, NSV>
            <<<dim3((unsigned)(units / 2 * FixCfg<BM>::CHUNKS)), block, 0, s>>>(
                offsets, E, b, c, cpre, K, N, Nt, SBN, slots, part);
    return hipGetLastError();
}

// Two resident workgroups per CU (3 LDS stages each, 72 KB) for the first
// GEMM when its tiles have 128 rows: with a few dozen rows per expert it
// streams weights, and two workgroups keep twice the DMAs in flight per CU
// while each other's epilogue runs (10 % off that launch on a 128-expert top-1
// layer, 5 % on a 256-token decode batch).  The second GEMM, and the 64-row
// layout, measured slower or unchanged that way.  MOE_GEMM_DUAL (a build
// switch for such comparisons) 0: never; 1: this rule; 2: the first GEMM at
// 64 or 128 rows; 3: both GEMMs at 64 or 128 rows.
#ifndef MOE_GEMM_DUAL
#define MOE_GEMM_DUAL 1
#endif
bool gemm_dual(int bm, bool first) {
    switch (MOE_GEMM_DUAL) {
    case 1: return first && bm == 128;
    case 2: return first && bm <= 128;
    case 3: return bm <= 128;
    default: return false;
    }
}

template <int ACT>
hipError_t launch_gemm(const moe_problem_t& p, const void* X, const int32_t* rowmap,
                       const int32_t* offsets, const void* W, const void* bias, void* Cout,
                       void* Cpre, int K, int N, float* part, hipEvent_t mid, hipStream_t s,
                       bool fixup = true) {
    const int64_t rows = p.T * p.k;
    if (p.dtype == MOE_DTYPE_BF16) {
        const int bm = pick_bm(p);
        const int Mt = (int)((rows + bm - 1) / bm + p.E);     // row tiles, worst case
        const int Nt = gemm_nt(N);
        // super-block width in column tiles: the widest of 16/8/4 that divides Nt
        const int SBN = (Nt % 16 == 0) ? 16 : (Nt % 8 == 0) ? 8 : 4;
        const int ncu = device_cus();
        auto* x = static_cast<const uint16_t*>(X);
        auto* w = static_cast<const uint16_t*>(W);
        auto* b = static_cast<const uint16_t*>(bias);
        auto* c = static_cast<uint16_t*>(Cout);
        auto* cp = static_cast<uint16_t*>(Cpre);
        // bytes addressable through X: the token rows (gather) or the kept rows
        const int64_t xrows = rowmap ? p.T : rows;
        const uint32_t xb = (uint32_t)(xrows * K * 2);
        hipError_t e;
        const bool dual = gemm_dual(bm, ACT != kActNone);
        if (bm == 256)
            e = launch_bf16<256, ACT, 0>(x, xb, rowmap, offsets, p.E, w, b, c, cp, K, N, Mt, Nt,
                                         SBN, ncu, part, mid, s, fixup);
        else if (bm == 128 && dual)
            e = launch_bf16<128, ACT, 3>(x, xb, rowmap, offsets, p.E, w, b, c, cp, K, N, Mt, Nt,
                                         SBN, 2 * ncu, part, mid, s, fixup);
        else if (bm == 128)
            e = launch_bf16<128, ACT, 0>(x, xb, rowmap, offsets, p.E, w, b, c, cp, K, N, Mt, Nt,
                                         SBN, ncu, part, mid, s, fixup);
        else if (dual)
            e = launch_bf16<64, ACT, 3>(x, xb, rowmap, offsets, p.E, w, b, c, cp, K, N, Mt, Nt, SBN,
                                        2 * ncu, part, mid, s, fixup);
        else
            e = launch_bf16<64, ACT, 0>(x, xb, rowmap, offsets, p.E, w, b, c, cp, K, N, Mt, Nt, SBN,
                                        ncu, part, mid, s, fixup);
        return e;
    } else {
        const int Mt = (int)((rows + 63) / 64 + p.E);
        const int Nt = (N + 63) / 64;
        ffn_gemm_f32<ACT><<<dim3((unsigned)((int64_t)Mt * Nt)), dim3(256), 0, s>>>(
            static_cast<const float*>(X), rowmap, offsets, p.E, static_cast<const float*>(W),
            static_cast<const float*>(bias), static_cast<float*>(Cout), K, N, Mt);
        const hipError_t e = hipGetLastError();
        return (e == hipSuccess && mid) ? hipEventRecord(mid, s) : e;
    }
}

}  // namespace

hipError_t launch_ffn_up(const moe_problem_t& p, const void* xp, const int32_t* rowmap,
                         const int32_t* offsets, const void* W1, const void* b1, void* h,
                         void* hgrad, float* part, hipEvent_t mid, hipStream_t s) {
    if (p.activation == MOE_ACT_SILU)
        return launch_gemm<kActSilu>(p, xp, rowmap, offsets, W1, b1, h, hgrad, p.H, p.F, part,
                                     mid, s);
    return launch_gemm<kActGelu>(p, xp, rowmap, offsets, W1, b1, h, hgrad, p.H, p.F, part, mid,
                                 s);
}

hipError_t launch_ffn_down(const moe_problem_t& p, const void* h, const int32_t* offsets,
                           const void* W2, const void* b2, void* y, float* part, hipEvent_t mid,
                           hipStream_t s, bool fixup) {
    return launch_gemm<kActNone>(p, h, nullptr, offsets, W2, b2, y, nullptr, p.F, p.H, part, mid,
                                 s, fixup);
}

GemmCut down_gemm_cut(const moe_problem_t& p) {
    // as launch_gemm picks them for the second GEMM (K = F, N = H)
    GemmCut g;
    g.bm = pick_bm(p);
    const bool dual = g.bm <= 128 && gemm_dual(g.bm, false);
    g.ns = dual ? 3 : g.bm == 256 ? Cfg<256>::NS : g.bm == 128 ? Cfg<128>::NS : Cfg<64>::NS;
    const int bk = g.bm == 256 ? Cfg<256>::BK : g.bm == 128 ? Cfg<128>::BK : Cfg<64>::BK;
    g.nk = (p.F + bk - 1) / bk;
    g.Nt = gemm_nt(p.H);
    g.SBN = (g.Nt % 16 == 0) ? 16 : (g.Nt % 8 == 0) ? 8 : 4;
    g.ncu = dual ? 2 * device_cus() : device_cus();
    return g;
}

size_t gemm_partial_bytes(const moe_problem_t& p) {
    if (p.dtype != MOE_DTYPE_BF16) return 0;
    // at most kMaxUnits K slices of one BM x 256 fp32 tile each
    return (size_t)kMaxUnits * (size_t)pick_bm(p) * 256u * sizeof(float);
}

}  // namespace moe
