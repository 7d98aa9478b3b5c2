// ds_penalty.hip -- the repetition penalty of the autoregressive mode.
//
// [ISSUE]: the existing sampler draws one token per request and applies a
// repetition penalty over seen-token masks.  The pages name the penalty but give
// no formula; it is read as the multiplicative penalty: a seen id's logit x
// becomes x / theta when x > 0 and x * theta otherwise, computed in binary32 and
// stored back in place in the logits' own type (bf16 rounded to nearest even).
// The token is then drawn by the sampler like a cell with guidance 0.
//
// One thread per kPenaltyWords mask words: the words and the row's theta are
// loaded together, then the logits of up to kPenaltyBatch set bits are all read
// before any is penalised and written back in place.  Seen ids are a small part
// of a row, so the kernel reads the mask (V / 8 bytes per row) and a few
// scattered logits: it is bound by those scattered reads and writes and by the
// latency of the two dependent reads.  (256 rows of V = 248320 with 256 to 1280
// seen ids each: 13.7 us with one word per thread and one read at a time, 11.0
// with two words and four reads; four words per thread take longer, 12.3 us.)
#include <stdint.h>

#include "ds_device.h"
#include "ds_kernels.h"

namespace ds {
namespace {

template <bool BF16>
__global__ __launch_bounds__(kPenaltyThreads) void k_repetition_penalty(PenaltyArgs a) {
    static_assert(kPenaltyWords == 2 || kPenaltyWords == 4, "two or four mask words per thread");
    const int64_t groups = (a.W + kPenaltyWords - 1) / kPenaltyWords;  // per row
    const int64_t g = (int64_t)blockIdx.x * kPenaltyThreads + threadIdx.x;
    if (g >= a.n_rows * groups) return;
    const int64_t row = g / groups;
    const int32_t w0 = (int32_t)(g - row * groups) * kPenaltyWords;
    const uint32_t* words = a.seen + row * (int64_t)a.W;
    // the thread's ids w0 * 32 .. as one or two 64-bit masks, ids past V cleared
    uint64_t m[kPenaltyWords / 2];
#pragma unroll
    for (int h = 0; h < kPenaltyWords / 2; ++h) {
        uint32_t lo = 0u, hi = 0u;
        const int32_t w = w0 + 2 * h;
        if (w < a.W) lo = __builtin_nontemporal_load(words + w);
        if (w + 1 < a.W) hi = __builtin_nontemporal_load(words + w + 1);
        m[h] = (uint64_t)hi << 32 | lo;
        const int32_t tail = a.V - w * 32;  // ids of these two words inside the row
        if (tail < 64) m[h] &= tail > 0 ? (1ull << tail) - 1ull : 0ull;
    }
    const float theta = a.penalty[row];
    // a row whose theta is not finite and positive is left as it is
    if (!(theta > 0.0f && theta < __builtin_huge_valf())) return;
    const int64_t base = row * (int64_t)a.V + (int64_t)w0 * 32;
    // kPenaltyBatch seen ids at a time: every read issued before any write
    while (m[0] != 0ull || (kPenaltyWords == 4 && m[kPenaltyWords / 2 - 1] != 0ull)) {
        int64_t at[kPenaltyBatch];
        bool ok[kPenaltyBatch];
#pragma unroll
        for (int k = 0; k < kPenaltyBatch; ++k) {
            ok[k] = true;
            if (m[0]) {
                at[k] = base + __builtin_ctzll(m[0]);
                m[0] &= m[0] - 1ull;
            } else if (kPenaltyWords == 4 && m[kPenaltyWords / 2 - 1]) {
                at[k] = base + 64 + __builtin_ctzll(m[kPenaltyWords / 2 - 1]);
                m[kPenaltyWords / 2 - 1] &= m[kPenaltyWords / 2 - 1] - 1ull;
            } else {
                ok[k] = false;
                at[k] = base;
            }
        }
        if (BF16) {
            uint16_t* x = static_cast<uint16_t*>(a.logits);
            uint16_t v[kPenaltyBatch];
#pragma unroll
            for (int k = 0; k < kPenaltyBatch; ++k) v[k] = ok[k] ? x[at[k]] : (uint16_t)0;
#pragma unroll
            for (int k = 0; k < kPenaltyBatch; ++k)
                if (ok[k]) x[at[k]] = bf16_rne(penalized(__uint_as_float((uint32_t)v[k] << 16), theta));
        } else {
            float* x = static_cast<float*>(a.logits);
            float v[kPenaltyBatch];
#pragma unroll
            for (int k = 0; k < kPenaltyBatch; ++k) v[k] = ok[k] ? x[at[k]] : 0.0f;
#pragma unroll
            for (int k = 0; k < kPenaltyBatch; ++k)
                if (ok[k]) x[at[k]] = penalized(v[k], theta);
        }
    }
}

}  // namespace

hipError_t launch_repetition_penalty(bool bf16, const PenaltyArgs& a, hipStream_t st) {
    const int64_t threads = a.n_rows * ((a.W + kPenaltyWords - 1) / kPenaltyWords);
    if (threads <= 0) return hipSuccess;
    const int64_t blocks = (threads + kPenaltyThreads - 1) / kPenaltyThreads;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (bf16)
        hipLaunchKernelGGL(k_repetition_penalty<true>, dim3((unsigned)blocks), dim3(kPenaltyThreads), 0, st, a);
    else
        hipLaunchKernelGGL(k_repetition_penalty<false>, dim3((unsigned)blocks), dim3(kPenaltyThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace ds
