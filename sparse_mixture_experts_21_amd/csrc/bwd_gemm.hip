// Grouped GEMMs of the backward ("moe-training" SKILL page: training the
// layer; the gradients of its expert FFNs by the chain rule).  For the kept
// rows r of expert e (offsets[e] <= r < offsets[e+1]):
//
//   dgrad   C[r][n] = sum_k X[r][k] B[e][n][k]      both operands K-contiguous
//           (da = (dy . W2[e]^T) * act'(a), act'(a) saved by the forward:
//                                            X = dy, B = W2[e] = [F][H], K = H;
//            dxe = da . W1[e]^T:            X = da, B = W1[e] = [H][F], K = F)
//   wgrad   C[e][i][j] = sum_r P[r][i] Q[r][j]       both operands row-major over r
//           (dW2[e] = h^T dy:  P = h, Q = dy;  dW1[e] = xp^T da:  P = xp, Q = da)
//
// The tile machinery is the forward's (256 x 256 output tiles on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation), but with 8 waves (2 per
// SIMD) of 128 rows x 64 columns where the forward runs 4; operands moved
// HBM -> LDS by buffer_load ... lds through a 128 KB ring (dgrad: 2 stages of
// 64-deep k-tiles; wgrad: 4 stages of 32-deep ones).  An
// operand is either K-contiguous ("row" layout: LDS [idx][k], 64-byte rows,
// plain 16-byte fragment reads) or row-major over k ("k-major": LDS [k][idx],
// 512-byte rows, ds_read_b64_tr_b16 transposed fragment reads).  dgrad uses
// row/row, wgrad k-major/k-major.  The MFMA's first operand is the side whose
// index runs along the output row, so every lane owns 4 consecutive output
// columns of one output row.  Out-of-range rows, columns and k read as zero
// through the buffer resources' ranges or an out-of-range offset.
#include "moe_internal.h"
#include "lds_dma.h"
#include "gemm_common.h"

namespace moe {
namespace {

constexpr int kT = 256;                 // tile edge (both output dimensions)
constexpr int kLds = 128 * 1024;        // the DMA ring: 2 stages of 64-deep or 4 of 32-deep k-tiles

// k-tile depth BK and what follows from it: LDS stages, bytes of one operand
// tile per stage, and the row layout's 16-byte chunks per row, rows per 1 KB
// block and swizzle shift.
template <int BK_>
struct KT {
    static constexpr int BK = BK_;
    static constexpr int NS = BK == 64 ? 2 : 4;
    static constexpr int OP = kT * BK * 2;
    static constexpr int STAGE = 2 * OP;
    static constexpr int CPR = BK / 8, RPB = 64 / CPR, RSH = CPR == 4 ? 2 : 1;
    static_assert(BK == 32 || BK == 64, "k-tile depth");
    static_assert(NS * STAGE == kLds, "ring size");
};

enum Layout { kRow = 0, kKmaj = 1 };

// Waves of a workgroup over the 256 x 256 tile: 2 along the output rows (B
// side) and NW / 2 along the output columns (A side).  4 waves: 128 x 128 per
// wave; 8 waves (2 per SIMD): 128 rows x 64 columns per wave.
template <int NW_>
struct WaveLayout {
    static constexpr int NW = NW_;
    static constexpr int WN = NW / 2;                  // waves along the columns
    static constexpr int TA = kT / WN, TB = kT / 2;    // per-wave extent: columns, rows
    static constexpr int FA = TA / 32, FB = TB / 32;   // 32 x 32 MFMA tiles per wave
    static_assert(NW == 4 || NW == 8, "waves");
};
template <int NW>
using BAcc = f32x16_t[WaveLayout<NW>::FA][WaveLayout<NW>::FB];

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;

// One operand of a tile: a buffer resource whose byte 0 is element (idx0, k0)
// of the tile's block, the row stride in bytes, the number of valid indices
// (along the tile edge) and of valid k.
struct Operand {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t ld;        // bytes between consecutive rows of the source
    int n_idx;          // valid indices from idx0 (rows for kRow, columns for kKmaj)
    int n_k;            // valid k from k0
};

// Byte offset (within the operand's resource) of DMA q's 16 bytes for k-tile
// t, and the LDS byte offset it lands at, for this lane.
template <int L, class Q, int NW>
__device__ __forceinline__ uint32_t dma_src(const Operand& o, int q, int t) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int blk = NW * q + wave;                      // 1 KB block of the stage tile
    if constexpr (L == kRow) {
        // RPB rows of 2 BK bytes per block; chunk c of row idx stored at
        // c ^ ((idx >> RSH) % CPR)
        const int idx = Q::RPB * blk + lane / Q::CPR;
        const int c = (lane % Q::CPR) ^ ((idx >> Q::RSH) % Q::CPR);
        const int k = t * Q::BK + 8 * c;
        if (idx >= o.n_idx || k >= o.n_k) return kOob;
        return (uint32_t)idx * o.ld + (uint32_t)k * 2u;
    } else {
        // 2 rows of 512 bytes per block; chunk c of row k stored at c ^ (4 (k & 3))
        const int kr = 2 * blk + (lane >> 5);
        const int c = (lane & 31) ^ (4 * (kr & 3));
        const int k = t * Q::BK + kr;
        if (8 * c >= o.n_idx || k >= o.n_k) return kOob;
        return (uint32_t)k * o.ld + (uint32_t)(8 * c) * 2u;
    }
}

// LDS byte offset (relative to the operand's tile in a stage) of fragment f of
// the wave's 128-wide half `w0` for k-substep kk; kRow returns one 16-byte
// read, kKmaj the first of two 8-byte transposed reads (the second is 4 rows on).
template <int L, class Q>
__device__ __forceinline__ uint32_t frag_addr(int w0, int f, int kk) {
    const int lane = threadIdx.x & 63;
    if constexpr (L == kRow) {
        const int idx = w0 + 32 * f + (lane & 31);
        const int pc = (2 * kk + (lane >> 5)) ^ ((idx >> Q::RSH) % Q::CPR);
        return (uint32_t)(idx * Q::BK * 2 + pc * 16);
    } else {
        const int grp = lane >> 4, s16 = lane & 15;
        const int k = 8 * (grp >> 1) + (s16 >> 2);
        const int idx = w0 + 32 * f + 16 * (grp & 1) + 4 * (s16 & 3);
        const int pc = (idx >> 3) ^ (4 * (k & 3));
        return (uint32_t)((k + 16 * kk) * 512 + pc * 16 + (idx & 4) * 2);
    }
}

template <int L>
__device__ __forceinline__ bf16x8_t read_frag(uint32_t a) {
    if constexpr (L == kRow) {
        return *(const lds_bf16x8_t*)(uintptr_t)a;
    } else {
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(uintptr_t)a);
        const v4i16_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(uintptr_t)(a + 4 * 512));
        const v8i16_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8_t, v);
    }
}

// acc[i][j] += A-side fragments i (wave column half) x B-side fragments j
// (wave row half) over nk k-tiles.  A: first MFMA operand (output columns),
// B: second (output rows).  The schedule is the forward GEMM's: DMA runs
// kNS - 1 k-tiles ahead, a k-tile's DMAs are spread one at a time between
// MFMA groups over two substeps (H1 after the barrier that frees their stage,
// H2 in the next substep), and the fragments of the next substep are read
// between the current substep's MFMAs (scheduling groups), with one barrier
// per k-tile.
template <int LA, int LB, int BK, int NW>
__device__ __forceinline__ void bwd_mainloop(const Operand& A, const Operand& B, int nk,
                                             char* lds, BAcc<NW>& acc) {
    using Q = KT<BK>;
    using WL = WaveLayout<NW>;
    constexpr int FA = WL::FA, FB = WL::FB;
    constexpr int kNS = Q::NS, kStage = Q::STAGE, kOpBytes = Q::OP;
    constexpr int kDmaPerOp = kOpBytes / (1024 * NW);  // 1 KB DMA blocks per wave per operand
    static_assert(kDmaPerOp * 1024 * NW == kOpBytes, "operand tile splits over the waves");
    const int wave = threadIdx.x >> 6;
    const int wn = wave % WL::WN, wm = wave / WL::WN;
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
    constexpr int NDMA = 2 * kDmaPerOp;
    auto issue_one = [&](int t, int q) {
        const uint32_t st = lds0 + (uint32_t)((t % kNS) * kStage);
        if (q < kDmaPerOp) {
            const uint32_t l = __builtin_amdgcn_readfirstlane(st + (uint32_t)((NW * q + wave) * 1024));
            dma16(A.rsrc, dma_src<LA, Q, NW>(A, q, t), l);
        } else {
            const int qb = q - kDmaPerOp;
            const uint32_t l = __builtin_amdgcn_readfirstlane(
                st + (uint32_t)(kOpBytes + (NW * qb + wave) * 1024));
            dma16(B.rsrc, dma_src<LB, Q, NW>(B, qb, t), l);
        }
    };
    bf16x8_t fa[2][FA], fb[2][FB];
    // fragment f (f < FA: A side, else B side) of substep kk of k-tile t
    auto read_one = [&](int t, int kk, int buf, int f) {
        const uint32_t st = lds0 + (uint32_t)((t % kNS) * kStage);
        if (f < FA) fa[buf][f] = read_frag<LA>(st + frag_addr<LA, Q>(WL::TA * wn, f, kk));
        else fb[buf][f - FA] = read_frag<LB>(st + kOpBytes + frag_addr<LB, Q>(WL::TB * wm, f - FA, kk));
    };
    // fragments in the order the MFMAs consume them: A0, B0..B(FB-1), A1..
    auto frag_id = [](int o) { return o == 0 ? 0 : (o <= FB ? FA + o - 1 : o - FB); };
    auto read_all = [&](int t, int kk, int buf) {
#pragma unroll
        for (int o = 0; o < FA + FB; ++o) read_one(t, kk, buf, frag_id(o));
    };
    auto mfma_range = [&](int buf, int lo, int hi) {
#pragma unroll
        for (int x = 0; x < FA * FB; ++x) {
            if (x < lo || x >= hi) continue;
            const int i = x / FB, j = x % FB;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j],
                                                                acc[i][j], 0, 0, 0);
        }
    };
    constexpr int NMF = FA * FB;
    constexpr int NRD = (LA == kKmaj ? 2 : 1) * FA + (LB == kKmaj ? 2 : 1) * FB;
    constexpr int NF = FA + FB;
    constexpr int H1 = (NDMA + 1) / 2, H2 = NDMA - H1;
    constexpr int NSUB = BK / 16;
    constexpr int RG2 = H2 > 1 ? H2 / 2 : 1, RG1 = H1 > 1 ? H1 / 2 : 1;
#pragma unroll
    for (int t = 0; t + 1 < kNS; ++t)
#pragma unroll
        for (int q = 0; q < NDMA; ++q) issue_one(t, q);
#pragma unroll
    for (int q = 0; q < H1; ++q) issue_one(kNS - 1, q);
    wait_vmcnt<(kNS - 2) * NDMA + H1>();
    lds_barrier();
    read_all(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        // substep 0: MFMAs || fragments of substep 1 || the rest of k-tile kt+NS-1's DMAs
#pragma unroll
        for (int g = 0; g < H2; ++g) {
            __builtin_amdgcn_sched_barrier(0);
            issue_one(kt + kNS - 1, H1 + g);
            mfma_range(0, g * NMF / H2, (g + 1) * NMF / H2);
            if (g < RG2) {
#pragma unroll
                for (int o = g * NF / RG2; o < (g + 1) * NF / RG2; ++o)
                    read_one(kt, 1, 1, frag_id(o));
            }
#pragma unroll
            for (int q = 0; q < NMF; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (q < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
        }
        // substeps 1..NSUB-2
#pragma unroll
        for (int sub = 1; sub + 1 < NSUB; ++sub) {
            __builtin_amdgcn_sched_barrier(0);
            read_all(kt, sub + 1, (sub + 1) & 1);
            mfma_range(sub & 1, 0, NMF);
#pragma unroll
            for (int q = 0; q < NMF; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (q < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // k-tile kt+1 has landed for every wave; stage kt % NS is free again
        wait_vmcnt<(kNS - 2) * NDMA>();
        wait_lgkm0();
        lds_barrier();
        // last substep: MFMAs || first fragments of k-tile kt+1 || DMAs of k-tile kt+NS
#pragma unroll
        for (int g = 0; g < H1; ++g) {
            __builtin_amdgcn_sched_barrier(0);
            issue_one(kt + kNS, g);
            mfma_range((NSUB - 1) & 1, g * NMF / H1, (g + 1) * NMF / H1);
            if (g < RG1) {
#pragma unroll
                for (int o = g * NF / RG1; o < (g + 1) * NF / RG1; ++o)
                    read_one(kt + 1, 0, 0, frag_id(o));
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
    wait_lgkm0();
}

template <int NW>
__device__ __forceinline__ void zero(BAcc<NW>& acc) {
#pragma unroll
    for (int i = 0; i < WaveLayout<NW>::FA; ++i)
#pragma unroll
        for (int j = 0; j < WaveLayout<NW>::FB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// ---------------------------------------------------------------- dgrad
// Workgroup p: a row tile (over the experts' kept rows, 256 rows each, never
// straddling experts) x a column tile, in the forward GEMM's tile order.
// EPI_DA: multiply by gp[r][n] = act'(a[r][n]), saved by the training
// forward's first GEMM; EPI_PLAIN: store as is.  Output bf16 [rows][N].
// The epilogue stages the tile in LDS ([m][n] bf16, 528-byte pitch, as the
// forward's) and writes it out by whole rows; with EPI_DA each lane first
// multiplies its values by the act' values at the same positions, loaded
// straight from global memory (8 bytes per lane and accumulator row).
// Both run 8 waves (2 per SIMD, 128 x 64 each), so one wave's MFMAs cover
// the other's LDS reads.
enum { kEpiPlain = 0, kEpiDa = 1 };
constexpr int kBwdWaves = 8;
constexpr int kOutPitch = kT * 2 + 16;
constexpr int kDgradLds = kLds > kT * kOutPitch ? kLds : kT * kOutPitch;

template <int EPI>
__global__ __launch_bounds__(64 * kBwdWaves) void bwd_dgrad(const uint16_t* __restrict__ X,
                                                 const int32_t* __restrict__ offsets, int E,
                                                 const uint16_t* __restrict__ Bw,
                                                 const uint16_t* __restrict__ gp,
                                                 uint16_t* __restrict__ C, int K, int N, int Nt,
                                                 int SBN) {
    __shared__ __attribute__((aligned(1024))) char lds[kDgradLds];
    const int p = blockIdx.x;
    // the forward GEMM's XCD-aware order over the real tiles
    const int real_mt = __builtin_amdgcn_readfirstlane(real_row_tiles<kT>(offsets, E));
    if (p >= real_mt * Nt) return;
    int mt, nt;
    dense_coords(p, real_mt, Nt, SBN, mt, nt);
    int e, m0, row_begin, n_rows;
    if (!find_tile<kT>(offsets, E, mt, e, m0, row_begin, n_rows)) return;
    const int n0 = nt * kT;
    const int rows = min(kT, n_rows - m0);
    Operand a, b;
    // A (output columns): B[e][n0 ..][k], K-contiguous rows of the expert's weights
    a.rsrc = make_rsrc(uniform_ptr(Bw + ((int64_t)e * N + n0) * K), (uint32_t)min(kT, N - n0) * K * 2u);
    a.ld = (uint32_t)K * 2u;
    a.n_idx = min(kT, N - n0);
    a.n_k = K;
    // B (output rows): X[row_begin + m0 ..][k]
    b.rsrc = make_rsrc(uniform_ptr(X + (int64_t)(row_begin + m0) * K), (uint32_t)rows * K * 2u);
    b.ld = (uint32_t)K * 2u;
    b.n_idx = rows;
    b.n_k = K;
    constexpr int NW = kBwdWaves;
    using WL = WaveLayout<NW>;
    BAcc<NW> acc;
    zero<NW>(acc);
    // dgrad: 64-deep k-tiles in 2 stages
    bwd_mainloop<kRow, kRow, 64, NW>(a, b, (K + 63) / 64, lds, acc);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave % WL::WN, wm = wave / WL::WN;
    const int l32 = lane & 31, half = lane >> 5;
    const int chunks = min(kT, N - n0) / 8;             // 16-byte chunks per row (N % 8 == 0)
    const int64_t base = (int64_t)(row_begin + m0) * N + n0;
    lds_barrier();
    const int cols = min(kT, N - n0);
#pragma unroll
    for (int j = 0; j < WL::FB; ++j) {
        const int m = WL::TB * wm + 32 * j + l32;
#pragma unroll
        for (int i = 0; i < WL::FA; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int nl = WL::TA * wn + 32 * i + 8 * g + 4 * half;
                char* slot = lds + m * kOutPitch + nl * 2;
                float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                              acc[i][j][4 * g + 3]};
                if constexpr (EPI == kEpiDa) {
                    // the lane's own 4 act' values, straight from global memory
                    u32x2_t pa = {0u, 0u};
                    if (m < rows && nl < cols)
                        pa = *reinterpret_cast<const u32x2_t*>(gp + base + (int64_t)m * N + nl);
                    v[0] *= bf16_lo(pa[0]);
                    v[1] *= bf16_hi(pa[0]);
                    v[2] *= bf16_lo(pa[1]);
                    v[3] *= bf16_hi(pa[1]);
                }
                u32x2_t o;
                o[0] = pack_bf16x2(v[0], v[1]);
                o[1] = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<u32x2_t*>(slot) = o;
            }
    }
    lds_barrier();
    for (int idx = tid; idx < kT * (kT / 8); idx += 64 * NW) {
        const int r = idx / (kT / 8), c = idx % (kT / 8);
        if (r < rows && c < chunks)
            *reinterpret_cast<u32x4_t*>(C + base + (int64_t)r * N + c * 8) =
                *reinterpret_cast<const u32x4_t*>(lds + r * kOutPitch + c * 16);
    }
}

// ---------------------------------------------------------------- wgrad
// Workgroup p: expert p / (It Jt), output tile (i, j) of C[e] [I][J] (fp32):
// C[e][i][j] = sum over the expert's rows r of P[r][i] Q[r][j].  An expert
// without rows gets zeros.
__global__ __launch_bounds__(64 * kBwdWaves) void bwd_wgrad(const uint16_t* __restrict__ P,
                                                 const uint16_t* __restrict__ Q,
                                                 const int32_t* __restrict__ offsets, int I,
                                                 int J, int It, int Jt, int E, int SBN,
                                                 float* __restrict__ C) {
    __shared__ __attribute__((aligned(1024))) char lds[kLds];
    // tile rows are (expert, i) pairs, expert-major; the forward GEMM's
    // XCD-aware order over them and the j tiles
    int mt, nt;
    dense_coords(blockIdx.x, E * It, Jt, SBN, mt, nt);
    const int e = mt / It;
    const int i0 = (mt % It) * kT, j0 = nt * kT;
    const int r0 = __builtin_amdgcn_readfirstlane(offsets[e]);
    const int nr = __builtin_amdgcn_readfirstlane(offsets[e + 1]) - r0;
    Operand a, b;
    // A (output columns j): Q[r0 + k][j0 ..]
    a.rsrc = make_rsrc(uniform_ptr(Q + (int64_t)r0 * J + j0), (uint32_t)nr * J * 2u);
    a.ld = (uint32_t)J * 2u;
    a.n_idx = min(kT, J - j0);
    a.n_k = nr;
    // B (output rows i): P[r0 + k][i0 ..]
    b.rsrc = make_rsrc(uniform_ptr(P + (int64_t)r0 * I + i0), (uint32_t)nr * I * 2u);
    b.ld = (uint32_t)I * 2u;
    b.n_idx = min(kT, I - i0);
    b.n_k = nr;
    BAcc<kBwdWaves> acc;
    zero<kBwdWaves>(acc);
    // wgrad: 32-deep k-tiles in 4 stages (measured a little faster here)
    bwd_mainloop<kKmaj, kKmaj, 32, kBwdWaves>(a, b, (nr + 31) / 32, lds, acc);
    using WL = WaveLayout<kBwdWaves>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wn = wave % WL::WN, wm = wave / WL::WN;
    const int l32 = lane & 31, half = lane >> 5;
    float* Ce = C + (int64_t)e * I * J;
#pragma unroll
    for (int jj = 0; jj < WL::FB; ++jj) {
        const int i = i0 + WL::TB * wm + 32 * jj + l32;
        if (i >= I) continue;
#pragma unroll
        for (int ii = 0; ii < WL::FA; ++ii)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int j = j0 + WL::TA * wn + 32 * ii + 8 * g + 4 * half;
                if (j >= J) continue;
                const f32x4_t v = {acc[ii][jj][4 * g], acc[ii][jj][4 * g + 1],
                                   acc[ii][jj][4 * g + 2], acc[ii][jj][4 * g + 3]};
                *reinterpret_cast<f32x4_t*>(Ce + (int64_t)i * J + j) = v;
            }
    }
}

}  // namespace

hipError_t launch_bwd_dgrad(const moe_problem_t& p, bool da, const void* X, const int32_t* offsets,
                            const void* Bw, const void* gp, void* C, int K, int N,
                            hipStream_t s) {
    const int64_t rows = p.T * p.k;
    const int Mt = (int)((rows + kT - 1) / kT + p.E);          // row tiles, worst case
    const int Nt = (N + kT - 1) / kT;
    const int SBN = (Nt % 16 == 0) ? 16 : (Nt % 8 == 0) ? 8 : 4;
    const dim3 grid((unsigned)((int64_t)Mt * Nt));
    auto* x = static_cast<const uint16_t*>(X);
    auto* b = static_cast<const uint16_t*>(Bw);
    auto* pr = static_cast<const uint16_t*>(gp);
    auto* c = static_cast<uint16_t*>(C);
    if (da)
        bwd_dgrad<kEpiDa><<<grid, dim3(64 * kBwdWaves), 0, s>>>(x, offsets, p.E, b, pr, c, K, N,
                                                                 Nt, SBN);
    else
        bwd_dgrad<kEpiPlain><<<grid, dim3(64 * kBwdWaves), 0, s>>>(x, offsets, p.E, b, pr, c, K,
                                                                    N, Nt, SBN);
    return hipGetLastError();
}

hipError_t launch_bwd_wgrad(const moe_problem_t& p, const void* P, const void* Q,
                            const int32_t* offsets, int I, int J, float* C, hipStream_t s) {
    const int It = (I + kT - 1) / kT, Jt = (J + kT - 1) / kT;
    const int SBN = (Jt % 16 == 0) ? 16 : (Jt % 8 == 0) ? 8 : 4;
    bwd_wgrad<<<dim3((unsigned)(p.E * It * Jt)), dim3(64 * kBwdWaves), 0, s>>>(
        static_cast<const uint16_t*>(P), static_cast<const uint16_t*>(Q), offsets, I, J, It, Jt,
        p.E, SBN, C);
    return hipGetLastError();
}

}  // namespace moe
