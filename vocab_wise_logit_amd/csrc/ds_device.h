// ds_device.h -- device building blocks shared by the sampler kernels (gfx950).
//
// Sources, by page title and section:
//   [ISSUE] mstar issue "Sampler support for discrete diffusion", comment on the API
//           shape: CFG combine, top-ratio filter to ceil(0.1 V) ids, Gumbel noise.
//   [DRAFT] LightLLM PR "perf: avoid full-vocab all-gather for draft greedy
//           sampling", "Design and invariants": max / log-sum-exp / argmax triples,
//           smallest id on ties.
//   [PHILOX] Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
//           1, 2, 3", SC'11: Philox4x32 round function and Weyl key schedule.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds {

constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Largest Gumbel value the noise map can produce is -log(-log(1 - 2^-24)) =
// 16.6355...; the bound used to prune ids that cannot win adds a margin for the
// fp32 rounding of G and of h / tau.
constexpr float kGumbelBound = 16.75f;
// Smallest value, -log(-log(2^-24)) = -2.8116..., with margin.
constexpr float kGumbelFloor = -2.82f;

// ------------------------------------------------------ global-memory views

// Kernel arguments arrive as generic pointers; casting them to the global
// address space lets the compiler emit global_load instead of flat_load.
template <typename T>
using gptr = const __attribute__((address_space(1))) T*;

// 16-byte load unit of the streaming kernels.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ gptr<T> as_global(const void* p) {
    return (gptr<T>)p;
}

// Logits are read once per call: loads carry the nontemporal hint, which on
// this GPU streams them past the caches' normal retention (measured: a
// one-workgroup-per-row reduction of 127 MB, 23.8 -> 22.3 us).
__device__ __forceinline__ u32x4 stream_load(gptr<u32x4> p) { return __builtin_nontemporal_load(p); }
// Cache-policy operand of the buffer loads: the nontemporal bit.
constexpr int kBufferNontemporal = 2;

// Word 3 of a gfx9 buffer resource for raw 32-bit loads (no swizzle, no stride):
// the hardware returns 0 for any dword outside [0, num_records).
constexpr int kBufferRsrcWord3 = 0x00020000;

// ------------------------------------------------------------ element decode

// bf16 is the upper half of a binary32, so widening is a shift (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// binary32 -> bf16 pattern, round to nearest even: adding 0x7FFF plus the
// pattern's lowest kept bit carries into the kept half exactly when the dropped
// half is above the tie, or at it with an odd kept half.  Infinities pass
// through; finite values past the largest bf16 carry into infinity.
__device__ __forceinline__ uint16_t bf16_rne(float y) {
    const uint32_t b = __float_as_uint(y);
    if ((b & 0x7F800000u) == 0x7F800000u) return (uint16_t)(b >> 16);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// [ISSUE] repetition penalty over seen-token masks (the pages give no formula):
// read as the multiplicative penalty, a seen id's logit x becomes x / theta when
// x > 0 and x * theta otherwise, in binary32 (IEEE division, correctly rounded).
__device__ __forceinline__ float penalized(float x, float theta) { return x > 0.0f ? x / theta : x * theta; }

// [ISSUE] CFG combine in fp32 with one rounding of s*(c-u)+c.  At a masked id
// (c = u = -inf) the difference is NaN.  `guided` maps it back to -inf (IEEE
// maxNum returns the non-NaN operand; every other input passes through
// unchanged).  `guided_raw` leaves it: max, argmax and every >= / == test skip a
// NaN, so a streaming pass only has to check its exp-sum, which a NaN turns into
// NaN, and redo the sum with `guided` in that (masked, guided) case.
__device__ __forceinline__ float guided_raw(float c, float u, float s) { return __builtin_fmaf(s, c - u, c); }
__device__ __forceinline__ float guided(float c, float u, float s) {
    return __builtin_fmaxf(guided_raw(c, u, s), kNegInf);
}

// Order-preserving map binary32 -> uint32 (negative values: all bits flipped,
// others: sign bit set).  Callers never feed -0 where it could differ from +0.
__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t b = __float_as_uint(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ------------------------------------------------------------------- noise

// [PHILOX] Philox4x32 with ten rounds.  Each round multiplies words 0 and 2 by
// the two Philox constants, swaps the halves and xors in the round key; the key
// advances by the Weyl increments.  The key words are wave-uniform, so the
// schedule runs on the scalar unit.
struct Words4 {
    uint32_t w0, w1, w2, w3;
};

// a ^ b ^ c in one gfx950 three-input bitwise instruction (truth table 0x96).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return (uint32_t)__builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ Words4 philox4x32_10(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                                uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t pa = (uint64_t)0xD2511F53u * x0;
        const uint64_t pb = (uint64_t)0xCD9E8D57u * x2;
        const uint32_t y0 = xor3((uint32_t)(pb >> 32), x1, k0);
        const uint32_t y2 = xor3((uint32_t)(pa >> 32), x3, k1);
        x1 = (uint32_t)pb;
        x3 = (uint32_t)pa;
        x0 = y0;
        x2 = y2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return Words4{x0, x1, x2, x3};
}

// Per-cell noise stream: the counter words that do not depend on the id.
struct NoiseKey {
    uint32_t k0, k1;    // seed halves
    uint32_t t;         // position inside the request
    uint32_t row_iter;  // (row & 0xFFFF) | (iteration << 16)
    uint32_t rid;       // low 32 bits of the request id
};

__device__ __forceinline__ uint32_t noise_word(const NoiseKey& nk, uint32_t v) {
    const Words4 w = philox4x32_10(v >> 2, nk.t, nk.row_iter, nk.rid, nk.k0, nk.k1);
    const uint32_t sel = v & 3u;
    uint32_t x = w.w0;
    x = sel == 1u ? w.w1 : x;
    x = sel == 2u ? w.w2 : x;
    x = sel == 3u ? w.w3 : x;
    return x;
}

// G = -log(-log U), U = ((x >> 9) * 2 + 1) * 2^-24 (exact in fp32).  The inner
// w = -ln U takes two routes, both cheap and accurate in relative terms:
//   U < 1/2:  w = -ln2 * log2(U), with |log2 U| >= 1;
//   U >= 1/2: d = 1 - U is exact, and -ln(1 - d) = 2 atanh(r), r = d / (2 - d)
//             <= 1/3, summed as 2r (1 + r^2/3 + ... + r^12/13) (next term below
//             2e-8 relative).
// Then G = -ln2 * log2(w).  Over all 2^23 values of U, w is within 3e-7 relative
// and G within 2e-6 absolute of the exact values (fp32 spacing near G = 14 is
// 1e-6).
__device__ __forceinline__ float gumbel_from_word(uint32_t x) {
    const uint32_t j = x >> 9;
    const float U = (float)(j * 2u + 1u) * 0x1p-24f;
    const float wa = -__builtin_amdgcn_logf(U) * kLn2;
    const float d = (float)((1u << 24) - 2u * j - 1u) * 0x1p-24f;
    const float r = d * __builtin_amdgcn_rcpf(2.0f - d);
    const float s = r * r;
    float p = 1.0f / 13.0f;
    p = __builtin_fmaf(p, s, 1.0f / 11.0f);
    p = __builtin_fmaf(p, s, 1.0f / 9.0f);
    p = __builtin_fmaf(p, s, 1.0f / 7.0f);
    p = __builtin_fmaf(p, s, 1.0f / 5.0f);
    p = __builtin_fmaf(p, s, 1.0f / 3.0f);
    p = __builtin_fmaf(p, s, 1.0f);
    const float wb = 2.0f * r * p;
    const float w = j < (1u << 22) ? wa : wb;
    return -__builtin_amdgcn_logf(w) * kLn2;
}

// Pruning bounds of the Gumbel race.  An id whose h lies below win_bound(z, tau)
// scores h/tau + G < (z - kGumbelBound) + G <= z - 0.11, so it loses to any id
// scoring z.  The term |z| * 2^-20 covers the fp32 roundings of h * (1/tau) + G,
// of z and of the bound itself (each within a few units of 2^-24 |z|), so the
// bound stays valid for scores far from zero (small temperatures).
__device__ __forceinline__ float win_bound(float z, float tau) {
    return (z - kGumbelBound - __builtin_fabsf(z) * 0x1p-20f) * tau;
}
// The same bound from an id known only by its value m: its score is at least
// m/tau + kGumbelFloor, whatever its noise.
__device__ __forceinline__ float max_bound(float m, float inv_tau, float tau) {
    return win_bound(__builtin_fmaf(m, inv_tau, kGumbelFloor), tau);
}

// ---------------------------------------------------------- wave reductions
//
// All-lane reductions use DPP inside each row of 16 lanes (xor 1, xor 2, half
// mirror, mirror) and then combine the four row results read into scalar
// registers, so the result is wave-uniform and no LDS round trip is involved.

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within 16

__device__ __forceinline__ float readlane_f(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// The maximum is taken on order keys: an unsigned max with the DPP operand fused
// into it is one instruction per step, where a float max needs the DPP value
// canonicalised first; the four row results combine on the scalar unit.  A NaN
// counts as -inf, as fmaxf would ignore it.
__device__ __forceinline__ float wave_max(float x) {
    uint32_t k = order_key(__builtin_fmaxf(x, kNegInf));
    k = max(k, (uint32_t)dpp_i<kDppXor1>((int)k));
    k = max(k, (uint32_t)dpp_i<kDppXor2>((int)k));
    k = max(k, (uint32_t)dpp_i<kDppHalfMirror>((int)k));
    k = max(k, (uint32_t)dpp_i<kDppMirror>((int)k));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)k, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)k, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)k, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)k, 48);
    return key_value(max(max(r0, r1), max(r2, r3)));
}
__device__ __forceinline__ float wave_min(float x) {
    x = __builtin_fminf(x, dpp_f<kDppXor1>(x));
    x = __builtin_fminf(x, dpp_f<kDppXor2>(x));
    x = __builtin_fminf(x, dpp_f<kDppHalfMirror>(x));
    x = __builtin_fminf(x, dpp_f<kDppMirror>(x));
    return __builtin_fminf(__builtin_fminf(readlane_f(x, 0), readlane_f(x, 16)),
                           __builtin_fminf(readlane_f(x, 32), readlane_f(x, 48)));
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_f<kDppXor1>(x);
    x += dpp_f<kDppXor2>(x);
    x += dpp_f<kDppHalfMirror>(x);
    x += dpp_f<kDppMirror>(x);
    return (readlane_f(x, 0) + readlane_f(x, 16)) + (readlane_f(x, 32) + readlane_f(x, 48));
}
__device__ __forceinline__ int wave_sum_i(int x) {
    x += dpp_i<kDppXor1>(x);
    x += dpp_i<kDppXor2>(x);
    x += dpp_i<kDppHalfMirror>(x);
    x += dpp_i<kDppMirror>(x);
    return (__builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16)) +
           (__builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48));
}
__device__ __forceinline__ int wave_min_i(int x) {
    x = min(x, dpp_i<kDppXor1>(x));
    x = min(x, dpp_i<kDppXor2>(x));
    x = min(x, dpp_i<kDppHalfMirror>(x));
    x = min(x, dpp_i<kDppMirror>(x));
    return min(min(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
               min(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// The same reductions inside each row of 16 lanes (every lane of a row gets its
// row's result).
__device__ __forceinline__ float row16_max(float x) {
    x = __builtin_fmaxf(x, dpp_f<kDppXor1>(x));
    x = __builtin_fmaxf(x, dpp_f<kDppXor2>(x));
    x = __builtin_fmaxf(x, dpp_f<kDppHalfMirror>(x));
    return __builtin_fmaxf(x, dpp_f<kDppMirror>(x));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<kDppXor1>(x);
    x += dpp_f<kDppXor2>(x);
    x += dpp_f<kDppHalfMirror>(x);
    return x + dpp_f<kDppMirror>(x);
}
__device__ __forceinline__ int row16_min_i(int x) {
    x = min(x, dpp_i<kDppXor1>(x));
    x = min(x, dpp_i<kDppXor2>(x));
    x = min(x, dpp_i<kDppHalfMirror>(x));
    return min(x, dpp_i<kDppMirror>(x));
}

// The same inside each group of 8 lanes (xor 1, xor 2, half mirror), or of 16.
template <int G>
__device__ __forceinline__ float grp_max(float x) {
    static_assert(G == 8 || G == 16, "groups of 8 or 16 lanes");
    x = __builtin_fmaxf(x, dpp_f<kDppXor1>(x));
    x = __builtin_fmaxf(x, dpp_f<kDppXor2>(x));
    x = __builtin_fmaxf(x, dpp_f<kDppHalfMirror>(x));
    if (G == 16) x = __builtin_fmaxf(x, dpp_f<kDppMirror>(x));
    return x;
}
template <int G>
__device__ __forceinline__ float grp_sum(float x) {
    static_assert(G == 8 || G == 16, "groups of 8 or 16 lanes");
    x += dpp_f<kDppXor1>(x);
    x += dpp_f<kDppXor2>(x);
    x += dpp_f<kDppHalfMirror>(x);
    if (G == 16) x += dpp_f<kDppMirror>(x);
    return x;
}
template <int G>
__device__ __forceinline__ int grp_min_i(int x) {
    static_assert(G == 8 || G == 16, "groups of 8 or 16 lanes");
    x = min(x, dpp_i<kDppXor1>(x));
    x = min(x, dpp_i<kDppXor2>(x));
    x = min(x, dpp_i<kDppHalfMirror>(x));
    if (G == 16) x = min(x, dpp_i<kDppMirror>(x));
    return x;
}

// Wave argmax of (z, id): larger z wins, equal z keeps the smaller id.  Returns
// the winning lane's (z, id) in every lane, and the winning lane index.  The
// id reduction runs only when several lanes hold the maximum.
__device__ __forceinline__ int wave_argmax(float& z, int& id) {
    const float zm = wave_max(z);
    uint64_t m = __ballot(z == zm);
    if (__popcll(m) > 1) {
        const int im = wave_min_i(z == zm ? id : 0x7FFFFFFF);
        m = __ballot(z == zm && id == im);
    }
    const int l = (int)__builtin_ctzll(m);
    z = zm;
    id = __builtin_amdgcn_readlane(id, l);
    return l;
}

// Inclusive prefix sum over lanes 0..lane: four shifted adds inside each row of
// 16 lanes (a lane with no source lane reads 0), then each row adds the totals
// of the rows below it, read into scalar registers.
constexpr int kDppWaveShl1 = 0x130;   // lane i takes lane i + 1 (lane 63 reads 0)
constexpr int kDppWaveShr1 = 0x138;   // lane i takes lane i - 1 (lane 0 reads 0)
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr1, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr2, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr4, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr8, 0xF, 0xF, true);
    const int r0 = __builtin_amdgcn_readlane(x, 15);
    const int r01 = r0 + __builtin_amdgcn_readlane(x, 31);
    const int r012 = r01 + __builtin_amdgcn_readlane(x, 47);
    const int row = lane_id() >> 4;
    return x + (row == 0 ? 0 : row == 1 ? r0 : row == 2 ? r01 : r012);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }
// Number of set bits of m in lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// ------------------------------------------------------ per-launch requests

// Per-request parameters of the requests covered by one launch, passed by value
// in the kernel argument segment ([PR]: per-request guidance and temperature,
// broadcast to every position of the request).
constexpr int kMaxReqPerLaunch = 64;

// One request's parameters, read by a cell's wave with a single scalar load.
struct ReqParams {
    int32_t start;        // first position, relative to the launch's pos0
    float scale;          // guidance
    float tau;
    float inv_tau;        // 1 / tau (correctly rounded), 0 for greedy requests
    int32_t uoff;         // u position of the request's first position
    uint32_t row_iter_hi; // iteration << 16
    uint32_t rid;         // low 32 bits of the request id
    int32_t pad;
};

struct ReqTable {
    int32_t n;        // requests in this launch
    int32_t pos0;     // first packed position covered
    int32_t npos;     // positions covered
    int32_t P;        // total packed positions of the call
    int32_t Pu;       // positions of the u layout: P, or the guided positions when u is compacted
    int32_t all_guided;  // every request of the launch reads u at its own position (no compaction)
    int32_t offs[kMaxReqPerLaunch + 1];  // request starts, relative to pos0 (searched by position)
    int32_t pad[2];
    ReqParams req[kMaxReqPerLaunch];
};

// Per-request parameters read from device memory when the launch runs (the
// fixed-shape entry point), instead of from the kernel-argument table.
struct DevReq {
    const int64_t* request_ids;  // [n]
    const int32_t* seq_lens;     // [n]
    const int32_t* iterations;   // [n]
    const float* guidance;       // [n], read only when u is present
    const float* temperature;    // [n]
    int32_t n;                   // requests (<= kWave unless one_per_request)
    int32_t P;                   // positions of the packed layout: row stride and grid extent
    int32_t one_per_request;     // position r is request r's only position (seq_lens unread)
};

// 1 / tau for sampled requests (correctly rounded, as the host computes it), 0
// for greedy ones.
__device__ __forceinline__ float inv_temperature(float tau) { return tau > 0.0f ? 1.0f / tau : 0.0f; }

// What a cell takes from its request under DevReq.
struct DevCell {
    float s, tau, inv_tau;
    uint32_t t;        // position inside the request
    uint32_t iter_hi;  // iteration << 16
    uint32_t rid;      // low 32 bits of the request id
};

// The request holding position pl, from DevReq's arrays; false when pl is
// padding.  Every wave calls it whole: lane r holds request r's length (a
// negative length counts as 0; lengths are clamped to d.P so the sums stay
// below 2^31), a wave prefix sum gives the request starts and the positions in
// use, min(sum, d.P).  A guidance scale that is not finite, or any scale when u
// is absent, counts as 0; a temperature that is not a positive finite number
// samples greedily.
__device__ __forceinline__ bool dev_cell(const DevReq& d, bool have_u, int pl, DevCell& o) {
    int r, start;
    if (d.one_per_request) {
        // one position per request (the autoregressive step): no lengths to scan
        if (pl >= d.n) return false;
        r = pl;
        start = pl;
    } else {
        const int lane = lane_id();
        int T = 0;
        if (lane < d.n) T = min(max(d.seq_lens[lane], 0), d.P);
        const int incl = wave_incl_scan(T);
        const int used = min(__builtin_amdgcn_readlane(incl, kWave - 1), d.P);
        if (pl >= used) return false;
        // the first request whose inclusive end passes pl (r < d.n, since pl is
        // below the sum of the lengths)
        r = popc(ballot(incl <= pl));
        start = __builtin_amdgcn_readlane(incl - T, r);
    }
    // guidance is read only where u is: without u every scale is 0
    float s = 0.0f;
    if (have_u) {
        s = d.guidance[r];
        if (!__builtin_isfinite(s)) s = 0.0f;
    }
    const float tau = d.temperature[r];
    o.s = s;
    o.tau = (tau > 0.0f && tau < __builtin_huge_valf()) ? tau : 0.0f;
    o.inv_tau = inv_temperature(o.tau);
    o.t = (uint32_t)(pl - start);
    o.iter_hi = (uint32_t)d.iterations[r] << 16;
    o.rid = (uint32_t)d.request_ids[r];
    return true;
}

// Request r's parameters as one 32-byte scalar load (a field-by-field read is
// split by the compiler into loads at each field's first use, each waiting
// for its own memory latency).
__device__ __forceinline__ ReqParams req_params(const ReqTable& rq, int r) {
    typedef int32_t i32x8 __attribute__((ext_vector_type(8), aligned(4)));
    const i32x8 v = *reinterpret_cast<const i32x8*>(&rq.req[r]);
    ReqParams q;
    q.start = v[0];
    q.scale = __int_as_float(v[1]);
    q.tau = __int_as_float(v[2]);
    q.inv_tau = __int_as_float(v[3]);
    q.uoff = v[4];
    q.row_iter_hi = (uint32_t)v[5];
    q.rid = (uint32_t)v[6];
    q.pad = 0;
    return q;
}

// The request owning launch-relative position pl: the last r with offs[r] <= pl,
// by a binary search of scalar loads from the kernel arguments (they hit the
// scalar cache; one vector load of every start per wave measured no faster, its
// memory round trip delaying a guided cell's u loads).
__device__ __forceinline__ int find_request(const ReqTable& rq, int pl) {
    int lo = 0, hi = rq.n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (rq.offs[mid] <= pl)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

}  // namespace ds
