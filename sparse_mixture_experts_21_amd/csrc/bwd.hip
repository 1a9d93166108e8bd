// The memory-bound kernels of the backward ("moe-training" SKILL page:
// training the layer with its load-balancing and z losses), for the objective
//   L = sum_t dout[t] . out[t] + g_aux * aux + g_z * z:
//
//   bwd_token    per token: dw_s = dout . y[pos_s] and dy[pos_s] = w_s dout for
//                every kept slot; then the router: the softmax of the saved
//                logits, dp through the renormalised top-k weights
//                (dp_j = (dw_j - sum_s dw_s w_s) / S), the aux loss
//                (+ g_aux E f_e / T, the routed fractions held constant), the
//                softmax (dl = p (dp - p . dp)) and the z-loss
//                (+ g_z 2 lse p / T).  Dropped slots pass nothing.
//   bwd_dx       dx[t] = sum over kept slots of dxe[pos_s] + dl[t] . Wg^T
//   bwd_colsum   bias gradients: per expert, the column sums of its rows
//   bwd_gate_*   dWg = x^T dl and dbg = sum_t dl over chunks of tokens, then
//                the chunk partials summed in chunk order
// Every reduction runs in a fixed order, so the gradients are bitwise
// reproducible.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBT = 256;       // threads of the per-token kernels

// Sum over the workgroup in a fixed order (wave butterflies, then the wave sums
// in order); every thread gets the result.  `red` holds kBT / 64 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float s = red[0];
#pragma unroll
    for (int w = 1; w < kBT / 64; ++w) s += red[w];
    return s;
}

__device__ __forceinline__ float block_max(float v, float* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float s = red[0];
#pragma unroll
    for (int w = 1; w < kBT / 64; ++w) s = fmaxf(s, red[w]);
    return s;
}

// One workgroup per token.  dout, y, dy: bf16 rows of H (vec 16-byte vectors).
__global__ __launch_bounds__(kBT) void bwd_token(
    const u32x4_t* __restrict__ dout, const u32x4_t* __restrict__ y,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, const float* __restrict__ logits,
    const int32_t* __restrict__ counts, int64_t T, int E, int k, int64_t vec, float g_aux,
    float g_z, u32x4_t* __restrict__ dy, float* __restrict__ dl) {
    __shared__ float red[kBT / 64];
    __shared__ float s_dw[kMaxK];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    // ---- expert side: dw_s and dy rows of the kept slots
    for (int s = 0; s < k; ++s) {
        const int32_t r = pos[t * k + s];                  // uniform
        float part = 0.f;
        if (r >= 0) {
            const float w = topk_w[t * k + s];
            for (int64_t v = tid; v < vec; v += kBT) {
                const u32x4_t g = dout[t * vec + v];
                const u32x4_t yy = y[(int64_t)r * vec + v];
                u32x4_t o;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float g0 = bf16_lo(g[q]), g1 = bf16_hi(g[q]);
                    part = fmaf(g0, bf16_lo(yy[q]), part);
                    part = fmaf(g1, bf16_hi(yy[q]), part);
                    o[q] = pack_bf16x2(w * g0, w * g1);
                }
                dy[(int64_t)r * vec + v] = o;
            }
        }
        const float dw = block_sum(part, red);         // 0 for a dropped slot
        if (tid == 0) s_dw[s] = dw;
    }
    __syncthreads();
    // ---- router side: thread e < E owns expert e
    const int e = tid;
    const float l = e < E ? logits[t * E + e] : -INFINITY;
    const float m = block_max(l, red);
    const float ex = e < E ? expf(l - m) : 0.f;
    const float Z = block_sum(ex, red);
    const float p = ex / Z;
    const float lse = m + logf(Z);
    float S = 0.f, sw = 0.f;
    for (int s = 0; s < k; ++s) {
        const int j = topk_idx[t * k + s];
        S += expf(logits[t * E + j] - m) / Z;
        sw += s_dw[s] * topk_w[t * k + s];
    }
    float dp = 0.f;
    if (e < E) {
        dp = g_aux * (float)E * ((float)counts[e] / (float)(T * k)) / (float)T;
        for (int s = 0; s < k; ++s)
            if (topk_idx[t * k + s] == e) dp += (s_dw[s] - sw) / S;
    }
    const float pdp = block_sum(e < E ? p * dp : 0.f, red);
    if (e < E) dl[t * E + e] = p * (dp - pdp) + g_z * 2.0f * lse * p / (float)T;
}

// dx[t] = sum over kept slots (slot order) of dxe rows + sum_e dl[t][e]
// Wg[h][e] (Wg [H][E] bf16), fp32, rounded once.  kDxTok tokens per
// workgroup, so the gate rows a thread needs are loaded once for all of them:
// into registers when E % 8 == 0 and E <= 16 (REG), else re-read per token
// (they stay in the cache).  Per token and 8 hidden
// units h = 8 v .. 8 v + 7: the kept slots' dxe rows in slot order, plus the
// gate term sum_e dl[t][e] Wg[h][e] in e order.
constexpr int kDxTok = 16;

template <bool REG>
__global__ __launch_bounds__(kBT) void bwd_dx(const u32x4_t* __restrict__ dxe,
                                              const int32_t* __restrict__ pos,
                                              const float* __restrict__ dl,
                                              const uint16_t* __restrict__ Wg, int E, int k,
                                              int64_t vec, int64_t T, u32x4_t* __restrict__ dx) {
    __shared__ float s_dl[kDxTok][kMaxE];
    const int64_t t0 = (int64_t)blockIdx.x * kDxTok;
    const int nt = (int)min((int64_t)kDxTok, T - t0);
    for (int i = threadIdx.x; i < nt * E; i += kBT) s_dl[i / E][i % E] = dl[t0 * E + i];
    __syncthreads();
    for (int64_t v = threadIdx.x; v < vec; v += kBT) {
        // REG: the 8 gate rows of this vector's hidden units (8 E contiguous bf16)
        u32x4_t wreg[8][2];
        if constexpr (REG) {
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    if (8 * c < E)
                        wreg[u][c] = *reinterpret_cast<const u32x4_t*>(Wg + (8 * v + u) * E + 8 * c);
        }
        for (int j = 0; j < nt; ++j) {
            const int64_t t = t0 + j;
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < k; ++s) {
                const int32_t r = pos[t * k + s];
                if (r < 0) continue;
                const u32x4_t d = dxe[(int64_t)r * vec + v];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] += bf16_lo(d[q]);
                    acc[2 * q + 1] += bf16_hi(d[q]);
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                float g = 0.f;
                if constexpr (REG) {
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        if (8 * c >= E) break;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            g = fmaf(s_dl[j][8 * c + 2 * q], bf16_lo(wreg[u][c][q]), g);
                            g = fmaf(s_dl[j][8 * c + 2 * q + 1], bf16_hi(wreg[u][c][q]), g);
                        }
                    }
                } else {
                    const uint16_t* wr = Wg + (8 * v + u) * E;
                    for (int e = 0; e < E; ++e)
                        g = fmaf(s_dl[j][e], __uint_as_float((uint32_t)wr[e] << 16), g);
                }
                acc[u] += g;
            }
            u32x4_t o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
            dx[t * vec + v] = o;
        }
    }
}

// Column sums of each expert's rows: workgroup (e, column block of 256):
// out[e][n] = sum over rows r of expert e (ascending) of rows[r][n] (bf16).
__global__ __launch_bounds__(256) void bwd_colsum(const uint16_t* __restrict__ rows,
                                                  const int32_t* __restrict__ offsets, int N,
                                                  int nb, float* __restrict__ out) {
    const int e = blockIdx.x / nb, n = (blockIdx.x % nb) * 256 + threadIdx.x;
    if (n >= N) return;
    const int r0 = offsets[e], r1 = offsets[e + 1];
    float acc = 0.f;
    for (int r = r0; r < r1; ++r) acc += __uint_as_float((uint32_t)rows[(int64_t)r * N + n] << 16);
    out[(int64_t)e * N + n] = acc;
}

// dWg partials: workgroup (block of 512 hidden units, token chunk c, expert
// block of kGateE): part[c][h][e] = sum over the chunk's tokens (ascending) of
// x[t][h] dl[t][e], two hidden units per thread.  The chunk's dl rows go
// through LDS in sub-blocks of kGateSub tokens, padded with zeros past the
// last token and the last expert, so the products run with fixed trip counts
// and no branches (the padding adds exact zeros); each thread loads the x
// values of kGateTok tokens before adding their products.  The first
// hidden-unit block also writes pb[c][e] = sum of dl[t][e] over the chunk.
constexpr int kGateE = 16;
constexpr int kGateTok = 16;
constexpr int kGateSub = 128;               // tokens per LDS sub-block
constexpr int kGateMaxChunks = 1024;

__global__ __launch_bounds__(256) void bwd_gate_partial(const uint16_t* __restrict__ x,
                                                        const float* __restrict__ dl, int64_t T,
                                                        int H, int E, int64_t chunk,
                                                        float* __restrict__ part,
                                                        float* __restrict__ pb) {
    __shared__ __attribute__((aligned(16))) float sdl[kGateSub][kGateE];
    const int tid = threadIdx.x;
    const int h = 2 * (blockIdx.x * 256 + tid);            // H % 8 == 0: h + 1 < H with h
    const bool hv = h < H;
    const int c = blockIdx.y, e0 = blockIdx.z * kGateE;
    const int ne = min(kGateE, E - e0);
    const int64_t t0 = (int64_t)c * chunk, t1 = min(t0 + chunk, T);
    float acc0[kGateE], acc1[kGateE], bsum = 0.f;
#pragma unroll
    for (int j = 0; j < kGateE; ++j) acc0[j] = acc1[j] = 0.f;
    for (int64_t sb = t0; sb < t1; sb += kGateSub) {
        const int n = (int)min<int64_t>(kGateSub, t1 - sb);
        __syncthreads();                                   // the previous sub-block is read
        for (int i = tid; i < kGateSub * kGateE; i += 256) {
            const int r = i / kGateE, j = i % kGateE;
            sdl[r][j] = (r < n && j < ne) ? dl[(sb + r) * E + e0 + j] : 0.f;
        }
        __syncthreads();
        // bias gradient: thread j < ne of the first hidden-unit block sums column j
        if (blockIdx.x == 0 && tid < ne)
            for (int r = 0; r < n; ++r) bsum += sdl[r][tid];
        for (int tb = 0; tb < kGateSub; tb += kGateTok) {
            uint32_t xv[kGateTok];
#pragma unroll
            for (int u = 0; u < kGateTok; ++u) {
                // rows past the chunk read its last row; their dl is zero
                const int64_t t = sb + min(tb + u, n - 1);
                xv[u] = hv ? *reinterpret_cast<const uint32_t*>(x + t * H + h) : 0u;
            }
#pragma unroll
            for (int u = 0; u < kGateTok; ++u) {
                const float x0 = bf16_lo(xv[u]), x1 = bf16_hi(xv[u]);
                const f32x4_t* d = reinterpret_cast<const f32x4_t*>(sdl[tb + u]);
#pragma unroll
                for (int q = 0; q < kGateE / 4; ++q) {
                    const f32x4_t dv = d[q];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        acc0[4 * q + r] = fmaf(x0, dv[r], acc0[4 * q + r]);
                        acc1[4 * q + r] = fmaf(x1, dv[r], acc1[4 * q + r]);
                    }
                }
            }
        }
    }
    if (hv) {
        float* o = part + ((int64_t)c * H + h) * E + e0;
#pragma unroll
        for (int j = 0; j < kGateE; ++j)
            if (j < ne) {
                o[j] = acc0[j];
                o[E + j] = acc1[j];
            }
    }
    if (blockIdx.x == 0 && tid < ne) pb[(int64_t)c * E + e0 + tid] = bsum;
}

__global__ __launch_bounds__(256) void bwd_gate_reduce(const float* __restrict__ part,
                                                       const float* __restrict__ pb, int H, int E,
                                                       int nchunk, float* __restrict__ dWg,
                                                       float* __restrict__ dbg) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < (int64_t)H * E) {
        float a = 0.f;
        for (int c = 0; c < nchunk; ++c) a += part[(int64_t)c * H * E + i];
        dWg[i] = a;
    }
    if (dbg && blockIdx.x == 0 && threadIdx.x < (unsigned)E) {
        float b = 0.f;
        for (int c = 0; c < nchunk; ++c) b += pb[(int64_t)c * E + threadIdx.x];
        dbg[threadIdx.x] = b;
    }
}

}  // namespace

int64_t bwd_gate_chunks(const moe_problem_t& p) {
    return std::min<int64_t>(kGateMaxChunks, (p.T + kGateSub - 1) / kGateSub);
}

hipError_t launch_bwd_token(const moe_problem_t& p, const void* dout, const void* y,
                            const int32_t* pos, const int32_t* topk_idx, const float* topk_w,
                            const float* logits, const int32_t* counts, float g_aux, float g_z,
                            void* dy, float* dl, hipStream_t s) {
    const int64_t vec = (int64_t)p.H * 2 / 16;
    bwd_token<<<dim3((unsigned)p.T), dim3(kBT), 0, s>>>(
        static_cast<const u32x4_t*>(dout), static_cast<const u32x4_t*>(y), pos, topk_idx, topk_w,
        logits, counts, p.T, p.E, p.k, vec, g_aux, g_z, static_cast<u32x4_t*>(dy), dl);
    return hipGetLastError();
}

hipError_t launch_bwd_dx(const moe_problem_t& p, const void* dxe, const int32_t* pos,
                         const float* dl, const void* Wg, void* dx, hipStream_t s) {
    const int64_t vec = (int64_t)p.H * 2 / 16;
    const dim3 grid((unsigned)((p.T + kDxTok - 1) / kDxTok));
    auto* d = static_cast<const u32x4_t*>(dxe);
    auto* w = static_cast<const uint16_t*>(Wg);
    auto* o = static_cast<u32x4_t*>(dx);
    if (p.E % 8 == 0 && p.E <= 16)
        bwd_dx<true><<<grid, dim3(kBT), 0, s>>>(d, pos, dl, w, p.E, p.k, vec, p.T, o);
    else
        bwd_dx<false><<<grid, dim3(kBT), 0, s>>>(d, pos, dl, w, p.E, p.k, vec, p.T, o);
    return hipGetLastError();
}

hipError_t launch_bwd_colsum(const moe_problem_t& p, const void* rows, const int32_t* offsets,
                             int N, float* out, hipStream_t s) {
    const int nb = (N + 255) / 256;
    bwd_colsum<<<dim3((unsigned)(p.E * nb)), dim3(256), 0, s>>>(
        static_cast<const uint16_t*>(rows), offsets, N, nb, out);
    return hipGetLastError();
}

hipError_t launch_bwd_gate(const moe_problem_t& p, const void* x, const float* dl, float* part,
                           float* pb, float* dWg, float* dbg, hipStream_t s) {
    const int64_t nchunk = bwd_gate_chunks(p);
    const int64_t chunk = (p.T + nchunk - 1) / nchunk;
    const dim3 g1((unsigned)((p.H + 511) / 512), (unsigned)nchunk,
                  (unsigned)((p.E + kGateE - 1) / kGateE));
    bwd_gate_partial<<<g1, dim3(256), 0, s>>>(static_cast<const uint16_t*>(x), dl, p.T, p.H, p.E,
                                               chunk, part, pb);
    const int64_t n = (int64_t)p.H * p.E;
    bwd_gate_reduce<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(
        part, pb, p.H, p.E, (int)nchunk, dWg, dbg);
    return hipGetLastError();
}

}  // namespace moe
