// Token dispatch with capacity dropping: a per-expert histogram, a prefix-sum
// permutation, and a row gather ("moe-training" SKILL page, Quick Start, Basic
// MoE Architecture: the per-expert token gather; Core Concepts, 4. Expert
// Parallelism: capacity factor and dropping tokens over capacity).
//
// Per expert the first `cap` (token, slot) pairs in ascending token order are
// kept.  The pairs are cut into chunks of kChunkTok tokens:
//   1. chunk_hist   per-chunk expert histogram (LDS integer atomics; the
//                   result is order independent, hence deterministic);
//   2. chunk_scan   per expert, exclusive scan over chunks -> the number of
//                   earlier pairs routed to e before each chunk; kept counts
//                   min(count, cap) and their exclusive scan -> offsets;
//   3. chunk_rank   one wave walks its chunk 64 pairs at a time in token
//                   order; lanes routed to the same expert find each other
//                   with 8 ballots over the expert id bits, and the rank is
//                   the running per-expert count plus the number of matching
//                   lower lanes;  pos = offsets[e] + rank when rank < cap;
//   4. gather_rows  xp[r] = x[row_token[r]] with 16-byte copies (skipped when
//                   the first expert GEMM reads x through row_token itself).
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void chunk_hist(const int32_t* __restrict__ topk_idx,
                                                  int64_t T, int E, int k,
                                                  int32_t* __restrict__ hist) {
    __shared__ int32_t h[kMaxE];
    const int tid = threadIdx.x;
    const int64_t c = blockIdx.x;
    for (int e = tid; e < E; e += 256) h[e] = 0;
    __syncthreads();
    const int64_t j0 = c * kChunkTok * k;
    const int64_t j1 = min((c + 1) * kChunkTok, T) * k;
    for (int64_t j = j0 + tid; j < j1; j += 256) {
        const int e = topk_idx[j];
        if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);   // invalid ids are dropped
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) hist[c * E + e] = h[e];
}

__global__ __launch_bounds__(256) void chunk_scan(const int32_t* __restrict__ hist,
                                                  int64_t nchunk, int E, int32_t cap,
                                                  int32_t* __restrict__ base,
                                                  int32_t* __restrict__ offsets) {
    __shared__ int32_t kept[kMaxE];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 256) {
        int32_t run = 0;
        for (int64_t c = 0; c < nchunk; ++c) {
            base[c * E + e] = run;
            run += hist[c * E + e];
        }
        kept[e] = min(run, cap);
    }
    __syncthreads();
    if (tid == 0) {
        int32_t acc = 0;
        for (int e = 0; e < E; ++e) {
            offsets[e] = acc;
            acc += kept[e];
        }
        offsets[E] = acc;
    }
}

__global__ __launch_bounds__(64) void chunk_rank(const int32_t* __restrict__ topk_idx,
                                                 const int32_t* __restrict__ base,
                                                 const int32_t* __restrict__ offsets, int64_t T,
                                                 int E, int k, int32_t cap,
                                                 int32_t* __restrict__ pos,
                                                 int32_t* __restrict__ row_token) {
    __shared__ int32_t run[kMaxE];
    __shared__ int32_t off[kMaxE];
    const int lane = threadIdx.x;
    const int64_t c = blockIdx.x;
    for (int e = lane; e < E; e += 64) {
        run[e] = base[c * E + e];
        off[e] = offsets[e];
    }
    __syncthreads();
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

// xp[r] = x[row_token[r]] for r < offsets[E]; `vec` 16-byte vectors per row.
__global__ __launch_bounds__(256) void gather_rows(const u32x4_t* __restrict__ x,
                                                   const int32_t* __restrict__ row_token,
                                                   const int32_t* __restrict__ offsets, int E,
                                                   int64_t vec, int64_t rows_per_block,
                                                   u32x4_t* __restrict__ xp) {
    const int64_t A = offsets[E];
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
    if (r0 >= A) return;
    const int64_t r1 = min(r0 + rows_per_block, A);
    for (int64_t r = r0; r < r1; ++r) {
        const u32x4_t* src = x + (int64_t)row_token[r] * vec;
        u32x4_t* dst = xp + r * vec;
        for (int64_t v = threadIdx.x; v < vec; v += 256) dst[v] = src[v];
    }
}

}  // namespace

hipError_t launch_permute(const moe_problem_t& p, const WsLayout& L, char* ws, int64_t cap,
                          const void* x, const int32_t* topk_idx, int32_t* offsets,
                          int32_t* pos, int32_t* row_token, void* xp, hipStream_t s) {
    const int64_t T = p.T;
    const int E = p.E, k = p.k;
    const int64_t nchunk = L.nchunk;
    int32_t* hist = reinterpret_cast<int32_t*>(ws + L.chunk_hist);
    int32_t* base = reinterpret_cast<int32_t*>(ws + L.chunk_base);
    const int32_t cap32 = (int32_t)std::min<int64_t>(cap, (int64_t)0x7fffffff);
    chunk_hist<<<dim3((unsigned)nchunk), dim3(256), 0, s>>>(topk_idx, T, E, k, hist);
    chunk_scan<<<dim3(1), dim3(256), 0, s>>>(hist, nchunk, E, cap32, base, offsets);
    chunk_rank<<<dim3((unsigned)nchunk), dim3(64), 0, s>>>(topk_idx, base, offsets, T, E, k,
                                                          cap32, pos, row_token);
    if (xp) {
        const int64_t row_bytes = (int64_t)p.H * (p.dtype == MOE_DTYPE_BF16 ? 2 : 4);
        const int64_t vec = row_bytes / 16;
        const int64_t rpb = vec >= 256 ? 4 : 16;
        const int64_t nb = (T * k + rpb - 1) / rpb;
        gather_rows<<<dim3((unsigned)nb), dim3(256), 0, s>>>(
            static_cast<const u32x4_t*>(x), row_token, offsets, E, vec, rpb,
            static_cast<u32x4_t*>(xp));
    }
    return hipGetLastError();
}

}  // namespace moe
