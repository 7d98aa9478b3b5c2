// ds_pins.hip -- TEST-ONLY kernels that run the sampler library's device
// building blocks (ds_device.h) over large input ranges, so that tests can
// compare them value by value with the CPU oracle: Philox4x32-10 words, the
// per-id noise word, the Gumbel map over every value of its uniform lattice, bf16
// widening of every bit pattern and the order-preserving float key.  Built next to
// this file by tests/gpu_pins/build_pins.py; nothing in the library loads it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ds_device.h"

namespace {

constexpr int kThreads = 256;

__global__ void k_philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1, int64_t n,
                         uint32_t* out) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    const ds::Words4 w = ds::philox4x32_10(c0 + (uint32_t)i, c1, c2, c3, k0, k1);
    out[4 * i + 0] = w.w0;
    out[4 * i + 1] = w.w1;
    out[4 * i + 2] = w.w2;
    out[4 * i + 3] = w.w3;
}

__global__ void k_noise(ds::NoiseKey nk, uint32_t v0, int64_t n, uint32_t* out) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    out[i] = ds::noise_word(nk, v0 + (uint32_t)i);
}

// G of the word whose top 23 bits are j, for j = 0 .. n - 1 (the low 9 bits, which
// the map drops, are set to a pattern of their own)
__global__ void k_gumbel(int64_t n, float* out) {
    const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (j >= n) return;
    out[j] = ds::gumbel_from_word(((uint32_t)j << 9) | ((uint32_t)j & 0x1FFu));
}

// dword p | ((65535 - p) << 16): its low half widens pattern p, its high half
// pattern 65535 - p
__global__ void k_bf16(uint32_t* lo, uint32_t* hi) {
    const uint32_t p = blockIdx.x * kThreads + threadIdx.x;
    if (p >= 65536u) return;
    const uint32_t w = p | ((65535u - p) << 16);
    lo[p] = __float_as_uint(ds::bf16_lo(w));
    hi[65535u - p] = __float_as_uint(ds::bf16_hi(w));
}

__global__ void k_order_key(const uint32_t* bits, int64_t n, uint32_t* key, uint32_t* back) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    key[i] = ds::order_key(__uint_as_float(bits[i]));
    back[i] = __float_as_uint(ds::key_value(key[i]));
}

unsigned blocks(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

int finish() {
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipDeviceSynchronize();
    return (int)e;
}

}  // namespace

// Each entry point launches on the null stream, waits for the result and returns
// the HIP status.  Output pointers are device memory sized as stated.
extern "C" {

// out [n][4]: Philox blocks of the counters (c0 + i, c1, c2, c3), key (k0, k1).
int pins_philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1, int64_t n,
                uint32_t* out) {
    if (n < 1 || n > ((int64_t)1 << 30) || !out) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_philox, dim3(blocks(n)), dim3(kThreads), 0, 0, c0, c1, c2, c3, k0, k1, n, out);
    return finish();
}

// out [n]: noise words of ids v0 .. v0 + n - 1 of one cell.
int pins_noise(uint32_t k0, uint32_t k1, uint32_t t, uint32_t row_iter, uint32_t rid, uint32_t v0, int64_t n,
               uint32_t* out) {
    if (n < 1 || n > ((int64_t)1 << 30) || !out) return (int)hipErrorInvalidValue;
    const ds::NoiseKey nk{k0, k1, t, row_iter, rid};
    hipLaunchKernelGGL(k_noise, dim3(blocks(n)), dim3(kThreads), 0, 0, nk, v0, n, out);
    return finish();
}

// out [2^23]: G for every top-23-bit value of the noise word.
int pins_gumbel_lattice(float* out) {
    if (!out) return (int)hipErrorInvalidValue;
    const int64_t n = (int64_t)1 << 23;
    hipLaunchKernelGGL(k_gumbel, dim3(blocks(n)), dim3(kThreads), 0, 0, n, out);
    return finish();
}

// lo, hi [65536]: the binary32 bits that bf16 pattern p widens to, through the
// low-half and the high-half decoder.
int pins_bf16_all(uint32_t* lo, uint32_t* hi) {
    if (!lo || !hi) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_bf16, dim3(blocks(65536)), dim3(kThreads), 0, 0, lo, hi);
    return finish();
}

// key, back [n]: the order key of each binary32 bit pattern, and the bits it maps back to.
int pins_order_key(const uint32_t* bits, int64_t n, uint32_t* key, uint32_t* back) {
    if (n < 1 || n > ((int64_t)1 << 30) || !bits || !key || !back) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_order_key, dim3(blocks(n)), dim3(kThreads), 0, 0, bits, n, key, back);
    return finish();
}

}  // extern "C"
