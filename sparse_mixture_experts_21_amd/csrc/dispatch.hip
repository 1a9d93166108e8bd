// Token dispatch with capacity dropping: a per-expert histogram, a prefix-sum
// permutation, and a row gather ("moe-training" SKILL page, Quick Start, Basic
// MoE Architecture: the per-expert token gather; Core Concepts, 4. Expert
// Parallelism: capacity factor and dropping tokens over capacity).
//
// Per expert the first `cap` (token, slot) pairs in ascending token order are
// kept.  The pairs are cut into chunks of kChunkTok tokens (one router block):
//   1. chunk_hist   per-chunk expert histogram, column-major [E][nchunk] (LDS
//                   integer atomics; order independent, hence deterministic).
//                   The fused forward skips it: the router already wrote
//                   exactly this table as its per-block expert counts;
//   2. scan_columns per expert (one workgroup each), exclusive scan over
//                   chunks -> the number of earlier pairs routed to e before
//                   each chunk, and the expert's total;
//   3. chunk_rank   kept counts min(total, cap) and their exclusive scan ->
//                   offsets (every workgroup forms them from the E totals);
//                   then one wave walks its chunk 64 pairs at a time in token
//                   order; lanes routed to the same expert find each other
//                   with 8 ballots over the expert id bits, and the rank is
//                   the running per-expert count plus the number of matching
//                   lower lanes;  pos = offsets[e] + rank when rank < cap;
//   4. gather_tokens  xp[pos[t][s]] = x[t], one workgroup per token (skipped
//                   when the first expert GEMM reads x through row_token itself).
#include "moe_internal.h"
#include "route_finalize.h"

namespace moe {
namespace {

__global__ __launch_bounds__(64) void chunk_hist(const int32_t* __restrict__ topk_idx,
                                                 int64_t T, int E, int k,
                                                 int32_t* __restrict__ hist) {
    __shared__ int32_t h[kMaxE];
    const int tid = threadIdx.x;
    const int64_t c = blockIdx.x, nchunk = gridDim.x;
    for (int e = tid; e < E; e += 64) h[e] = 0;
    __syncthreads();
    const int64_t j0 = c * kChunkTok * k;
    const int64_t j1 = min((c + 1) * kChunkTok, T) * k;
    for (int64_t j = j0 + tid; j < j1; j += 64) {
        const int e = topk_idx[j];
        if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);   // invalid ids are dropped
    }
    __syncthreads();
    for (int e = tid; e < E; e += 64) hist[e * nchunk + c] = h[e];
}

// Workgroup e < E scans expert column e: thread t takes kColPer consecutive
// chunks of each round (one round of loads), the thread totals get an
// exclusive scan (shuffles within each wave, the 4 wave totals through LDS),
// and each thread writes its chunks' running prefix; the column total goes to
// col_tot[e].  With FIN the workgroups E .. 2E sum the router's per-block
// partials (one column each), which saves the fused forward two launches.
template <bool FIN>
__global__ __launch_bounds__(kColThreads) void scan_columns(const int32_t* __restrict__ hist,
                                                           int64_t nchunk, int E,
                                                           int32_t* __restrict__ base,
                                                           int32_t* __restrict__ col_tot,
                                                           FinArgs fin) {
    __shared__ int32_t wtot[kColThreads / 64];
    const int col = blockIdx.x;
    if (FIN && col >= E) {
        fin_column_block(fin, E, col - E);
        return;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t* src = hist + (int64_t)col * nchunk;
    int32_t* dst = base + (int64_t)col * nchunk;
    int32_t carry = 0;
    for (int64_t s0 = 0; s0 < nchunk; s0 += kColThreads * kColPer) {
        const int64_t c0 = s0 + (int64_t)tid * kColPer;
        int32_t v[kColPer];
#pragma unroll
        for (int i = 0; i < kColPer; ++i)          // clamped, masked: no per-load branch
            v[i] = src[c0 + i < nchunk ? c0 + i : nchunk - 1];
        int32_t tot = 0;
#pragma unroll
        for (int i = 0; i < kColPer; ++i) {
            if (c0 + i >= nchunk) v[i] = 0;
            tot += v[i];
        }
        int32_t incl = tot;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t t = __shfl_up(incl, d);
            if (lane >= d) incl += t;
        }
        if (lane == 63) wtot[wave] = incl;
        __syncthreads();
        int32_t before = 0, round = 0;
#pragma unroll
        for (int w = 0; w < kColThreads / 64; ++w) {
            if (w < wave) before += wtot[w];
            round += wtot[w];
        }
        __syncthreads();                           // wtot is rewritten next round
        int32_t run = carry + before + incl - tot;
#pragma unroll
        for (int i = 0; i < kColPer; ++i) {
            if (c0 + i < nchunk) dst[c0 + i] = run;
            run += v[i];
        }
        carry += round;
    }
    if (tid == 0) col_tot[col] = carry;
}

// Every workgroup derives offsets[] from the column totals itself (kept count
// min(total, cap), exclusive scan over the experts); workgroup 0 publishes
// them and, with FIN, the router's expert counts and losses.
template <bool FIN>
__global__ __launch_bounds__(64) void chunk_rank(const int32_t* __restrict__ topk_idx,
                                                 const int32_t* __restrict__ base,
                                                 const int32_t* __restrict__ col_tot, int64_t T,
                                                 int E, int k, int32_t cap,
                                                 int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ pos,
                                                 int32_t* __restrict__ row_token, FinArgs fin) {
    __shared__ int32_t run[kMaxE];
    __shared__ int32_t off[kMaxE + 1];
    const int lane = threadIdx.x;
    const int64_t c = blockIdx.x, nchunk = gridDim.x;
    {
        // lane l owns experts 4l .. 4l + 3 (E <= 256)
        int32_t kv[4], tot = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            kv[i] = min(col_tot[e < E ? e : E - 1], cap);   // unconditional load, masked
            if (e >= E) kv[i] = 0;
            tot += kv[i];
        }
        int32_t incl = tot;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t t = __shfl_up(incl, d);
            if (lane >= d) incl += t;
        }
        int32_t o = incl - tot;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            if (e < E) off[e] = o;
            o += kv[i];
        }
        if (lane == 63) off[E] = incl;
    }
    for (int e = lane; e < E; e += 64) run[e] = base[e * nchunk + c];
    __syncthreads();
    if (c == 0) {
        for (int e = lane; e <= E; e += 64) offsets[e] = off[e];
        if (FIN) fin_losses(fin, E);
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int64_t j0 = c * kChunkTok * k;
    const int64_t j1 = min((c + 1) * kChunkTok, T) * k;
    for (int64_t jb = j0; jb < j1; jb += 64) {
        const int64_t j = jb + lane;
        const bool valid = j < j1;
        int e = valid ? topk_idx[j] : 0;
        const bool in_range = (unsigned)e < (unsigned)E;
        if (!in_range) e = 0;
        uint64_t same = __ballot(valid && in_range);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t m = __ballot(bit);
            same &= bit ? m : ~m;
        }
        const int32_t before = (int32_t)__popcll(same & below);
        int32_t r = 0;
        if (valid && in_range) r = run[e] + before;
        // all lanes have read run[] before any lane updates it: the update is
        // issued by the highest lane of each group after its own read
        __builtin_amdgcn_wave_barrier();
        if (valid && in_range && (same >> lane) == 1ull) run[e] = r + 1;
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            if (in_range && r < cap) {
                const int32_t p = off[e] + r;
                pos[j] = p;
                row_token[p] = (int32_t)(j / k);
            } else {
                pos[j] = -1;
            }
        }
    }
}

// xp[pos[t][s]] = x[t] for every kept slot: one workgroup per token, whose
// destination rows are workgroup-uniform, so each x row is read exactly once
// and each kept row written once (the minimum traffic), both nontemporally.
constexpr int kGatherThreads = 256;
constexpr int kGatherVec = 4;          // 16-byte vectors per thread and pass

__global__ __launch_bounds__(kGatherThreads) void gather_tokens(
    const u32x4_t* __restrict__ x, const int32_t* __restrict__ pos, int k, int64_t vec,
    u32x4_t* __restrict__ xp) {
    const int64_t t = blockIdx.x;
    int32_t dst[kMaxK];
#pragma unroll
    for (int s = 0; s < kMaxK; ++s) dst[s] = s < k ? pos[t * k + s] : -1;
    const u32x4_t* src = x + t * vec;
    for (int64_t v0 = threadIdx.x; v0 < vec; v0 += kGatherThreads * kGatherVec) {
        u32x4_t d[kGatherVec];
#pragma unroll
        for (int u = 0; u < kGatherVec; ++u) {
            const int64_t v = v0 + (int64_t)u * kGatherThreads;
            if (v < vec) d[u] = __builtin_nontemporal_load(&src[v]);
        }
#pragma unroll
        for (int s = 0; s < kMaxK; ++s) {
            if (dst[s] < 0) continue;                  // uniform: dropped or past k
#pragma unroll
            for (int u = 0; u < kGatherVec; ++u) {
                const int64_t v = v0 + (int64_t)u * kGatherThreads;
                if (v < vec) __builtin_nontemporal_store(d[u], &xp[(int64_t)dst[s] * vec + v]);
            }
        }
    }
}

}  // namespace

hipError_t launch_permute(const moe_problem_t& p, const WsLayout& L, char* ws, int64_t cap,
                          const void* x, const int32_t* topk_idx, int32_t* offsets,
                          int32_t* pos, int32_t* row_token, void* xp, int32_t* fin_counts,
                          float* fin_losses, hipStream_t s) {
    const int64_t T = p.T;
    const int E = p.E, k = p.k;
    const int64_t nchunk = L.nchunk;
    int32_t* hist = reinterpret_cast<int32_t*>(ws + L.chunk_hist);
    int32_t* base = reinterpret_cast<int32_t*>(ws + L.chunk_base);
    int32_t* tot = reinterpret_cast<int32_t*>(ws + L.col_tot);
    const int32_t cap32 = (int32_t)std::min<int64_t>(cap, (int64_t)0x7fffffff);
    if (fin_counts && fin_losses) {
        // fused forward: the router's per-block expert counts are the chunk
        // histogram, and its partials are reduced alongside the scan
        const FinArgs f{reinterpret_cast<const float*>(ws + L.blk_psum),
                        reinterpret_cast<const float*>(ws + L.blk_lse2),
                        reinterpret_cast<const int32_t*>(ws + L.blk_cnt), L.nblk_route, T, k,
                        reinterpret_cast<double*>(ws + L.fin_sum),
                        reinterpret_cast<long long*>(ws + L.fin_cnt), fin_counts, fin_losses};
        hist = reinterpret_cast<int32_t*>(ws + L.blk_cnt);
        scan_columns<true><<<dim3(2 * E + 1), dim3(kColThreads), 0, s>>>(hist, nchunk, E, base,
                                                                         tot, f);
        chunk_rank<true><<<dim3((unsigned)nchunk), dim3(64), 0, s>>>(
            topk_idx, base, tot, T, E, k, cap32, offsets, pos, row_token, f);
    } else {
        chunk_hist<<<dim3((unsigned)nchunk), dim3(64), 0, s>>>(topk_idx, T, E, k, hist);
        scan_columns<false><<<dim3(E), dim3(kColThreads), 0, s>>>(hist, nchunk, E, base, tot,
                                                                  FinArgs{});
        chunk_rank<false><<<dim3((unsigned)nchunk), dim3(64), 0, s>>>(
            topk_idx, base, tot, T, E, k, cap32, offsets, pos, row_token, FinArgs{});
    }
    if (xp) {
        const int64_t row_bytes = (int64_t)p.H * (p.dtype == MOE_DTYPE_BF16 ? 2 : 4);
        gather_tokens<<<dim3((unsigned)T), dim3(kGatherThreads), 0, s>>>(
            static_cast<const u32x4_t*>(x), pos, k, row_bytes / 16, static_cast<u32x4_t*>(xp));
    }
    return hipGetLastError();
}

hipError_t launch_gather(const moe_problem_t& p, const void* x, const int32_t* pos, void* xp,
                         hipStream_t s) {
    const int64_t row_bytes = (int64_t)p.H * (p.dtype == MOE_DTYPE_BF16 ? 2 : 4);
    gather_tokens<<<dim3((unsigned)p.T), dim3(kGatherThreads), 0, s>>>(
        static_cast<const u32x4_t*>(x), pos, p.k, row_bytes / 16, static_cast<u32x4_t*>(xp));
    return hipGetLastError();
}

}  // namespace moe
