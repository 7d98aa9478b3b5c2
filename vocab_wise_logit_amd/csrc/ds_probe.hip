// ds_probe.hip -- measurement aid: the HBM read ceiling at a given launch shape.
//
// One workgroup reads one row of 16-byte pieces once, with the same nontemporal
// loads and the same four pieces in flight per thread as the streaming sampler
// kernels, folds every word with xor (so no load can be dropped) and writes one
// word per row.  Timing it next to a sampler kernel of the same shape and bytes
// separates what the memory system delivers from what the kernel's arithmetic
// costs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ds_device.h"
#include "ds_kernels.h"

namespace ds {
namespace {

template <int NT>
__global__ __launch_bounds__(NT) void k_read_rows(const void* x, int64_t row_pieces, uint32_t* sink) {
    __shared__ uint32_t s_acc;
    const gptr<u32x4> p = as_global<u32x4>(x) + (int64_t)blockIdx.x * row_pieces;
    if (threadIdx.x == 0) s_acc = 0u;
    u32x4 acc = u32x4{0u, 0u, 0u, 0u};
    int64_t j = threadIdx.x;
    for (; j + 3 * NT < row_pieces; j += 4 * NT) {
        const u32x4 a = stream_load(p + j);
        const u32x4 b = stream_load(p + j + NT);
        const u32x4 c = stream_load(p + j + 2 * NT);
        const u32x4 d = stream_load(p + j + 3 * NT);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; j < row_pieces; j += NT) acc ^= stream_load(p + j);
    __syncthreads();
    __hip_atomic_fetch_xor(&s_acc, acc.x ^ acc.y ^ acc.z ^ acc.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = s_acc;
}

}  // namespace

hipError_t launch_read_probe(const void* x, int64_t n_rows, int64_t row_pieces, int threads, uint32_t* sink,
                             hipStream_t st) {
    const dim3 g((unsigned)n_rows);
    switch (threads) {
        case 256:
            hipLaunchKernelGGL(k_read_rows<256>, g, dim3(256), 0, st, x, row_pieces, sink);
            break;
        case 512:
            hipLaunchKernelGGL(k_read_rows<512>, g, dim3(512), 0, st, x, row_pieces, sink);
            break;
        case 1024:
            hipLaunchKernelGGL(k_read_rows<1024>, g, dim3(1024), 0, st, x, row_pieces, sink);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ds
