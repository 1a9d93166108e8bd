// Weighted combine back to token order ("moe-training" SKILL page, Quick
// Start, Basic MoE Architecture: the output starts at zero and each selected
// expert's output, scaled by its renormalised score, is added to the token's
// row).  Token-major gather instead of a scatter-add: every output element is
// produced by exactly one thread, summed in fp32 in slot order and rounded
// once, so there are no atomics and results are bitwise reproducible.
#include "moe_internal.h"

namespace moe {
namespace {

// One thread = one 16-byte vector of one token row (8 bf16 or 4 fp32).
template <bool BF16>
__global__ __launch_bounds__(256) void combine_rows(const u32x4_t* __restrict__ y,
                                                    const int32_t* __restrict__ pos,
                                                    const float* __restrict__ topk_w,
                                                    int64_t T, int k, int64_t vec,
                                                    u32x4_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= T * vec) return;
    const int64_t t = i / vec, v = i % vec;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < k; ++s) {
        const int32_t r = pos[t * k + s];
        if (r < 0) continue;
        const float w = topk_w[t * k + s];
        const u32x4_t d = y[(int64_t)r * vec + v];
        if (BF16) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = fmaf(w, bf16_lo(d[q]), acc[2 * q]);
                acc[2 * q + 1] = fmaf(w, bf16_hi(d[q]), acc[2 * q + 1]);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] = fmaf(w, __uint_as_float(d[q]), acc[q]);
        }
    }
    u32x4_t o;
    if (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[q]);
    }
    out[i] = o;
}

}  // namespace

hipError_t launch_combine(const moe_problem_t& p, const void* y, const int32_t* pos,
                          const float* topk_w, void* out, hipStream_t s) {
    const bool bf16 = p.dtype == MOE_DTYPE_BF16;
    const int64_t vec = (int64_t)p.H * (bf16 ? 2 : 4) / 16;
    const int64_t n = p.T * vec;
    const unsigned nb = (unsigned)((n + 255) / 256);
    if (bf16)
        combine_rows<true><<<dim3(nb), dim3(256), 0, s>>>(static_cast<const u32x4_t*>(y), pos,
                                                          topk_w, p.T, p.k, vec,
                                                          static_cast<u32x4_t*>(out));
    else
        combine_rows<false><<<dim3(nb), dim3(256), 0, s>>>(static_cast<const u32x4_t*>(y), pos,
                                                           topk_w, p.T, p.k, vec,
                                                           static_cast<u32x4_t*>(out));
    return hipGetLastError();
}

}  // namespace moe
