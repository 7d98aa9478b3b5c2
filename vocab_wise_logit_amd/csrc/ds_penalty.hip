// ds_penalty.hip -- the repetition penalty of the autoregressive mode.
//
// [ISSUE]: the existing sampler draws one token per request and applies a
// repetition penalty over seen-token masks.  The pages name the penalty but give
// no formula; it is read as the multiplicative penalty: a seen id's logit x
// becomes x / theta when x > 0 and x * theta otherwise, computed in binary32 and
// stored back in place in the logits' own type (bf16 rounded to nearest even).
// The token is then drawn by the sampler like a cell with guidance 0.
//
// One thread per 32-bit mask word: the words are read once, coalesced, and each
// set bit updates its logit in place.  Seen ids are a small part of a row, so the
// kernel touches the mask (V / 8 bytes per row) and a few scattered logits.
#include <stdint.h>

#include "ds_device.h"
#include "ds_kernels.h"

namespace ds {
namespace {

// binary32 -> bf16 pattern, round to nearest even: adding 0x7FFF plus the
// pattern's lowest kept bit carries into the kept half exactly when the dropped
// half is above the tie, or at it with an odd kept half.  Infinities pass
// through; finite values past the largest bf16 carry into infinity.
__device__ __forceinline__ uint16_t bf16_rne(float y) {
    const uint32_t b = __float_as_uint(y);
    if ((b & 0x7F800000u) == 0x7F800000u) return (uint16_t)(b >> 16);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

template <bool BF16>
__global__ __launch_bounds__(kPenaltyThreads) void k_repetition_penalty(PenaltyArgs a) {
    const int64_t g = (int64_t)blockIdx.x * kPenaltyThreads + threadIdx.x;
    if (g >= a.n_rows * a.W) return;
    const int64_t row = g / a.W;
    const int32_t w = (int32_t)(g - row * a.W);
    uint32_t m = __builtin_nontemporal_load(a.seen + g);
    const int32_t tail = a.V - w * 32;  // ids of this word inside the row (>= 1)
    if (tail < 32) m &= (1u << tail) - 1u;
    if (m == 0u) return;
    const float theta = a.penalty[row];
    // a row whose theta is not finite and positive is left as it is
    if (!(theta > 0.0f && theta < __builtin_huge_valf())) return;
    const int64_t base = row * (int64_t)a.V + (int64_t)w * 32;
    while (m) {
        const int b = __builtin_ctz(m);
        m &= m - 1u;
        if (BF16) {
            uint16_t* p = static_cast<uint16_t*>(a.logits) + base + b;
            const float x = __uint_as_float((uint32_t)*p << 16);
            *p = bf16_rne(x > 0.0f ? x / theta : x * theta);
        } else {
            float* p = static_cast<float*>(a.logits) + base + b;
            const float x = *p;
            *p = x > 0.0f ? x / theta : x * theta;
        }
    }
}

}  // namespace

hipError_t launch_repetition_penalty(bool bf16, const PenaltyArgs& a, hipStream_t st) {
    const int64_t words = a.n_rows * a.W;
    if (words <= 0) return hipSuccess;
    const int64_t blocks = (words + kPenaltyThreads - 1) / kPenaltyThreads;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (bf16)
        hipLaunchKernelGGL(k_repetition_penalty<true>, dim3((unsigned)blocks), dim3(kPenaltyThreads), 0, st, a);
    else
        hipLaunchKernelGGL(k_repetition_penalty<false>, dim3((unsigned)blocks), dim3(kPenaltyThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace ds
