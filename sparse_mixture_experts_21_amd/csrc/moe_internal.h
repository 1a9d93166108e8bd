// Internal declarations shared by the HIP sources of libmoe.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

#include "moe.h"

namespace moe {

// ---------------------------------------------------------------- types
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kMaxE = 256;
constexpr int kMaxK = 8;

// bf16 <-> fp32 on raw 16-bit patterns.  Widening is exact; narrowing rounds to
// nearest even in hardware (v_cvt_pk_bf16_f32, one instruction per pair).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ---------------------------------------------------------------- workspace
// Byte offsets of every scratch region inside the caller's workspace; all
// regions are 256-byte aligned.  Regions a call does not use are still laid
// out so that one layout serves every entry point.
struct WsLayout {
    size_t blk_psum;     // [E][nblk_route] fp32: per-block sums of softmax probs
    size_t blk_lse2;     // [nblk_route]    fp32: per-block sums of lse^2
    size_t blk_cnt;      // [E][nblk_route] int32: per-block expert histograms
    size_t fin_sum;      // [E + 1] fp64: column sums of the router partials
    size_t fin_cnt;      // [E] int64: expert counts from the router partials
    size_t small_disp;   // [E + 1 + 2 T k] int32: offsets, pos, row_token that moe_route
                         // drops when a few tokens route in one launch (route_small)
    size_t chunk_hist;   // [E][nchunk] int32 expert histogram per chunk
    size_t chunk_base;   // [E][nchunk] int32 pairs routed to e before the chunk
    size_t col_tot;      // [E] int32: pairs routed to each expert
    size_t gemm_part;    // fp32 K-slice partial tiles of the expert GEMMs' last round
    // moe_forward intermediates, used when the caller passes NULL
    size_t logits, topk_idx, topk_w, counts, offsets, pos, row_token, xp, h, y;
    size_t route_bytes, permute_bytes, ffn_bytes, total;
    int64_t nblk_route, nchunk;
};

constexpr int kRouteTok = 16;      // tokens per router workgroup
constexpr int kChunkTok = 16;      // tokens per dispatch chunk: one router block, so the
                                   // router's per-block histograms are the chunk histograms
static_assert(kChunkTok == kRouteTok, "dispatch chunks are router blocks");

WsLayout ws_layout(const moe_problem_t& p);
// Compute units of the current device (looked up once per device).
int device_cus();

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; none synchronises.
// finalize = false leaves the per-block partials in the workspace for the next
// launch_permute (given fin_counts / fin_losses) to reduce.
hipError_t launch_route(const moe_problem_t& p, const WsLayout& L, char* ws, const void* x,
                        const void* Wg, const void* bg, float* logits, bool logits_in,
                        int32_t* topk_idx, float* topk_w, int32_t* counts, float* losses,
                        bool finalize, hipStream_t s);
// fin_counts / fin_losses (both or neither): also reduce the router partials
// that a launch_route with finalize = false left in the workspace.
hipError_t launch_permute(const moe_problem_t& p, const WsLayout& L, char* ws, int64_t cap,
                          const void* x, const int32_t* topk_idx, int32_t* offsets,
                          int32_t* pos, int32_t* row_token, void* xp, int32_t* fin_counts,
                          float* fin_losses, hipStream_t s);
// Routing and dispatch of a batch with T * E <= kSmallPairs (bf16) in one
// launch: what launch_route and launch_permute (with the row gather fused into
// the first GEMM) produce, in another fixed floating-point order.
constexpr int kSmallPairs = 64;
bool route_small_fits(const moe_problem_t& p);
hipError_t launch_route_small(const moe_problem_t& p, int64_t cap, const void* x, const void* Wg,
                              const void* bg, float* logits, int32_t* topk_idx, float* topk_w,
                              int32_t* counts, float* losses, int32_t* offsets, int32_t* pos,
                              int32_t* row_token, hipStream_t s);
// rowmap (nullable): when set, row r of the first GEMM reads x[rowmap[r]]
// instead of xp[r] (the gather fused into the operand load).
// part (nullable): fp32 buffer of gemm_partial_bytes(p) for the K slices of
// the ragged last round of tiles; without it no tile is cut.
// mid (nullable): event recorded between the GEMM launch and its fixup.
// hgrad (nullable, bf16 only): also store act'(a) at the pre-activation rows
// a (with bias), for the backward.
hipError_t launch_ffn_up(const moe_problem_t& p, const void* xp, const int32_t* rowmap,
                         const int32_t* offsets, const void* W1, const void* b1, void* h,
                         void* hgrad, float* part, hipEvent_t mid, hipStream_t s);
// fixup = false (bf16): the K-slice partials of the cut last round are left in
// part for launch_combine_cut, and the cut tiles' rows of y are not written.
hipError_t launch_ffn_down(const moe_problem_t& p, const void* h, const int32_t* offsets,
                           const void* W2, const void* b2, void* y, float* part, hipEvent_t mid,
                           hipStream_t s, bool fixup = true);
size_t gemm_partial_bytes(const moe_problem_t& p);
// How the second (bf16) expert GEMM of p lays out its tiles and cuts its last
// round: row tile height, LDS stages and k-tiles of the row layout, column
// tiles, super-block width, workgroup slots.
struct GemmCut {
    int bm, ns, nk, Nt, SBN, ncu;
};
GemmCut down_gemm_cut(const moe_problem_t& p);
// out[t] = sum over the k slots s of row t, in order, with pos[t][s] >= 0 of
// topk_w[t][s] * y[pos[t][s]]; any k (expert choice passes k = E).
hipError_t launch_combine(const moe_problem_t& p, const void* y, const int32_t* pos,
                          const float* topk_w, void* out, hipStream_t s);
// The same for top-k routing (bf16) after launch_ffn_down(..., fixup = false):
// a row of a cut tile is finished here from the K-slice partials in part (summed
// in slice order, plus b2, rounded to bf16: the values the fixup would have
// written to y), the other rows are read from y.  topk_idx gives each slot's
// expert, offsets the experts' row ranges.
constexpr int64_t kCombineCutWideBelow = 8;   // below this, one vector per thread (wide rows)
hipError_t launch_combine_cut(const moe_problem_t& p, const void* y, const int32_t* pos,
                              const float* topk_w, const int32_t* topk_idx,
                              const int32_t* offsets, const void* b2, const float* part,
                              void* out, hipStream_t s);
// ---- backward (bf16)
hipError_t launch_gather(const moe_problem_t& p, const void* x, const int32_t* pos, void* xp,
                         hipStream_t s);
// dgrad: C[r][n] = sum_k X[r][k] Bw[e][n][k] over each expert's rows; da: times
// gp[r][n] (act'(a), saved by the training forward).  wgrad: C[e][i][j] = sum
// over the rows of e of P[r][i] Q[r][j].
hipError_t launch_bwd_dgrad(const moe_problem_t& p, bool da, const void* X, const int32_t* offsets,
                            const void* Bw, const void* gp, void* C, int K, int N,
                            hipStream_t s);
hipError_t launch_bwd_wgrad(const moe_problem_t& p, const void* P, const void* Q,
                            const int32_t* offsets, int I, int J, float* C, hipStream_t s);
hipError_t launch_bwd_token(const moe_problem_t& p, const void* dout, const void* y,
                            const int32_t* pos, const int32_t* topk_idx, const float* topk_w,
                            const float* logits, const int32_t* counts, float g_aux, float g_z,
                            void* dy, float* dl, hipStream_t s);
hipError_t launch_bwd_dx(const moe_problem_t& p, const void* dxe, const int32_t* pos,
                         const float* dl, const void* Wg, void* dx, hipStream_t s);
hipError_t launch_bwd_colsum(const moe_problem_t& p, const void* rows, const int32_t* offsets,
                             int N, float* out, hipStream_t s);
int64_t bwd_gate_chunks(const moe_problem_t& p);
hipError_t launch_bwd_gate(const moe_problem_t& p, const void* x, const float* dl, float* part,
                           float* pb, float* dWg, float* dbg, hipStream_t s);
// Expert choice on fp32 logits [T][E]: probs [T][E], sel [E][T/group][C],
// rowof [T][E] (-1 where not taken) and offsets [E+1] (e * (T/group) * C).
hipError_t launch_expert_choice(const moe_problem_t& p, int64_t group, int64_t C,
                                const float* logits, float* probs, int32_t* sel,
                                int32_t* rowof, int32_t* offsets, hipStream_t s);

}  // namespace moe
