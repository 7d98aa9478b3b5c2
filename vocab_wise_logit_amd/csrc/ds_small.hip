// ds_small.hip -- one wavefront per cell for vocabularies that fit in registers.
//
// Each 64-lane wave owns one cell (row, position) of the packed [C, P, V] logits
// and holds the whole guided row h[0..V) in VGPRs (dword slots of two bf16 or one
// f32 per lane).  Everything after the load is register / LDS work:
//   1. h = CFG combine ([ISSUE] comment on the API shape; [PR] "What does this PR
//      do?": guidance 0 never reads u), row max, smallest-id argmax, log-sum-exp;
//   2. greedy cells (temperature 0): token = argmax, logprob = max - LSE;
//   3. sampled cells: the exact top_k-th largest h ([ISSUE] top-ratio filter),
//      found by counting ids above pivots with wave ballots; the ids above the
//      final pivot are compacted into a per-wave LDS list, so refinement runs on a
//      few registers instead of the whole row;
//   4. Gumbel-max ([ISSUE]) over the kept ids that can still win: an id whose
//      h/tau + max-noise is below the argmax's h/tau + min-noise never wins, so
//      only ids with h >= max(t, M - tau * (Gmax - Gmin)) draw Philox noise.
// Ties: smallest id for the greedy argmax and for exact Gumbel ties ([DRAFT]
// "Design and invariants" rule, applied to every decision).
#include <stdint.h>

#include "ds_device.h"
#include "ds_kernels.h"

namespace ds {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kListCap = 512;
constexpr int kListRegs = kListCap / kWave;

// Wave argmax of (z, id) that also carries the winner's h.
__device__ __forceinline__ void wave_argmax3(float& z, int& id, float& hv) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float oz = __shfl_xor(z, o);
        const int oi = __shfl_xor(id, o);
        const float oh = __shfl_xor(hv, o);
        const bool take = (oz > z) || (oz == z && oi < id);
        z = take ? oz : z;
        id = take ? oi : id;
        hv = take ? oh : hv;
    }
}

template <bool BF16, int NS>
struct Row {
    static constexpr int NE = BF16 ? 2 * NS : NS;
    float h[NE];
    int par;  // bf16: 1 if the row starts in the high half of a dword

    // Row-relative id of register element i of this lane.
    __device__ __forceinline__ int id_of(int i, int lane) const {
        if (BF16) return 2 * ((i >> 1) * kWave + lane) + (i & 1) - par;
        return i * kWave + lane;
    }

    // Number of ids in h that are >= x (x > -inf), counted with ballots.
    __device__ __forceinline__ int count_ge(float x) const {
        int n = 0;
#pragma unroll
        for (int i = 0; i < NE; ++i) n += popc(ballot(h[i] >= x));
        return n;
    }
};

// Count ids >= x and write every such (h, id) to the wave's LDS list (entries
// beyond the capacity are dropped; the caller checks the returned count).
template <bool BF16, int NS>
__device__ __forceinline__ int count_and_compact(const Row<BF16, NS>& R, float x, int lane,
                                                 float* lh, int* le) {
    int base = 0;
#pragma unroll
    for (int i = 0; i < Row<BF16, NS>::NE; ++i) {
        const bool pred = R.h[i] >= x;
        const uint64_t m = ballot(pred);
        if (m) {
            const int o = base + lanes_below(m);
            if (pred && o < kListCap) {
                lh[o] = R.h[i];
                le[o] = R.id_of(i, lane);
            }
            base += popc(m);
        }
    }
    __builtin_amdgcn_wave_barrier();
    return base;
}

// Exact k-th largest over all valid ids, by key-space bisection on the full
// registers (bounded by 32 rounds).  Used only when the pivot search fails.
template <bool BF16, int NS>
__device__ float kth_by_bisection(const Row<BF16, NS>& R, int k, int V, float M) {
    uint32_t lo = order_key(kNegInf);  // count(lo) = V >= k
    uint32_t hi = order_key(M) + 1u;   // count = 0 < k
    if (R.count_ge(M) >= k) return M;
    hi = order_key(M);
    while (hi - lo > 1u) {
        const uint32_t mid = lo + ((hi - lo) >> 1);
        const int c = (mid == order_key(kNegInf)) ? V : R.count_ge(key_value(mid));
        if (c >= k)
            lo = mid;
        else
            hi = mid;
    }
    return key_value(lo);
}

template <bool BF16, int NS>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void k_sample_small(SampleArgs a, ReqTable rq) {
    using R_t = Row<BF16, NS>;
    constexpr int NE = R_t::NE;
    __shared__ float s_h[kWavesPerBlock][kListCap];
    __shared__ int s_e[kWavesPerBlock][kListCap];

    const int wv = threadIdx.x >> 6;
    const int lane = lane_id();
    const int64_t wid = (int64_t)blockIdx.x * kWavesPerBlock + wv;
    if (wid >= (int64_t)a.rows * rq.npos) return;  // whole wave leaves together
    const int row = (int)(wid / rq.npos);
    const int pl = (int)(wid - (int64_t)row * rq.npos);
    const int r = find_request(rq, pl);
    const int64_t cell = (int64_t)row * rq.P + rq.pos0 + pl;
    const int V = a.V;
    const float s = rq.scale[r];
    const float tau = rq.tau[r];
    float* lh = s_h[wv];
    int* le = s_e[wv];

    // ---------------------------------------------------------------- load
    R_t R;
    if (BF16) {
        const uintptr_t cb = (uintptr_t)a.c;
        const uint32_t* c32 = (const uint32_t*)(cb & ~(uintptr_t)3);
        const int64_t g = (int64_t)((cb & 3) >> 1) + cell * V;
        R.par = (int)(g & 1);
        const int64_t d0 = g >> 1;
        const int ndw = (R.par + V + 1) >> 1;
        uint32_t cw[NS];
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int d = j * kWave + lane;
            cw[j] = 0xFF80FF80u;  // two bf16 -inf
            if (d < ndw) cw[j] = c32[d0 + d];
        }
        if (s != 0.0f) {
            const uint32_t* u32 = (const uint32_t*)((uintptr_t)a.u & ~(uintptr_t)3);
            uint32_t uw[NS];
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const int d = j * kWave + lane;
                uw[j] = 0xFF80FF80u;
                if (d < ndw) uw[j] = u32[d0 + d];
            }
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                R.h[2 * j] = guided(bf16_lo(cw[j]), bf16_lo(uw[j]), s);
                R.h[2 * j + 1] = guided(bf16_hi(cw[j]), bf16_hi(uw[j]), s);
            }
        } else {
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                R.h[2 * j] = bf16_lo(cw[j]);
                R.h[2 * j + 1] = bf16_hi(cw[j]);
            }
        }
        // the two half-dwords that belong to the neighbouring rows
        if (R.par && lane == 0) R.h[0] = kNegInf;
        if ((R.par + V) & 1) {
            const int dl = ndw - 1;
#pragma unroll
            for (int j = 0; j < NS; ++j)
                if (j == (dl >> 6) && lane == (dl & 63)) R.h[2 * j + 1] = kNegInf;
        }
    } else {
        R.par = 0;
        const float* c = (const float*)a.c + cell * V;
        float cv[NS];
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int e = j * kWave + lane;
            cv[j] = kNegInf;
            if (e < V) cv[j] = c[e];
        }
        if (s != 0.0f) {
            const float* u = (const float*)a.u + cell * V;
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const int e = j * kWave + lane;
                float uv = kNegInf;
                if (e < V) uv = u[e];
                R.h[j] = guided(cv[j], uv, s);
            }
        } else {
#pragma unroll
            for (int j = 0; j < NS; ++j) R.h[j] = cv[j];
        }
    }

    // ------------------------------------------------ max, argmax, log-sum-exp
    float mx = R.h[0];
#pragma unroll
    for (int i = 1; i < NE; ++i) mx = __builtin_fmaxf(mx, R.h[i]);
    const float M = wave_max(mx);

    // smallest id attaining M: ids grow with the register index inside a lane,
    // so the first register slot (across lanes) holding M decides.
    int am = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        if (BF16) {
            const uint64_t m0 = ballot(R.h[2 * j] == M);
            const uint64_t m1 = ballot(R.h[2 * j + 1] == M);
            if (m0 | m1) {
                const int a0 = m0 ? 2 * (j * kWave + (int)__builtin_ctzll(m0)) - R.par : 0x7FFFFFFF;
                const int a1 = m1 ? 2 * (j * kWave + (int)__builtin_ctzll(m1)) + 1 - R.par : 0x7FFFFFFF;
                am = a0 < a1 ? a0 : a1;
                break;
            }
        } else {
            const uint64_t m0 = ballot(R.h[j] == M);
            if (m0) {
                am = j * kWave + (int)__builtin_ctzll(m0);
                break;
            }
        }
    }

    const float mL = M * kLog2e;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < NE; ++i) acc += __builtin_amdgcn_exp2f(__builtin_fmaf(R.h[i], kLog2e, -mL));
    const float S = wave_sum(acc);
    // exact residual of the rounded M*log2(e) shifts every exponent equally
    const float err = __builtin_fmaf(M, kLog2e, -mL);
    const float lse = M + (log2f(S) - err) * kLn2;

    if (tau == 0.0f) {
        if (lane == 0) {
            a.tokens[cell] = am;
            a.logprobs[cell] = M - lse;
            if (a.thresholds) a.thresholds[cell] = __builtin_nanf("");
        }
        return;
    }

    // ------------------------------------------------ top-k threshold (exact)
    const int k = a.top_k;
    // first pivot: mean + z0 * sd of (h - M) over the first slots, clamped
    float sum = 0.0f, sq = 0.0f;
    constexpr int NSTAT = NE < 4 ? NE : 4;
#pragma unroll
    for (int i = 0; i < NSTAT; ++i) {
        const float d = __builtin_fmaxf(R.h[i] - M, -64.0f);
        sum += d;
        sq = __builtin_fmaf(d, d, sq);
    }
    const float nstat = (float)(NSTAT * kWave);
    const float mean = wave_sum(sum) / nstat;
    const float var = __builtin_fmaxf(wave_sum(sq) / nstat - mean * mean, 0.0f);
    const float sd = __builtin_sqrtf(var) + 1e-3f;

    float t = kNegInf;
    bool have_t = false;     // t is exact
    bool list_ok = false;    // the LDS list holds every id >= lo
    float lo = M + mean + a.z0 * sd;
    if (!(lo < M)) lo = M - sd;
    float hi = M;
    int c_hi = -1;
    int c_lo = 0;
    for (int tries = 0; tries < 8; ++tries) {
        c_lo = count_and_compact(R, lo, lane, lh, le);
        if (c_lo >= k && c_lo <= kListCap) {
            list_ok = true;
            break;
        }
        if (c_lo < k) {
            hi = lo;
            c_hi = c_lo;
            if (tries < 3) {
                lo = lo - (2.0f + 2.0f * tries) * sd;
            } else {
                // smallest finite h of the row
                float mn = __builtin_huge_valf();
#pragma unroll
                for (int i = 0; i < NE; ++i) mn = R.h[i] > kNegInf ? __builtin_fminf(mn, R.h[i]) : mn;
                lo = wave_min(mn);
                if (R.count_ge(lo) < k) {  // fewer than k finite ids: t = -inf
                    t = kNegInf;
                    have_t = true;
                    break;
                }
            }
        } else {
            // too many ids for the list: move the pivot up towards hi
            const float target = 0.5f * (float)kListCap;
            const float chi = (float)(c_hi < 0 ? 1 : c_hi);
            float p = lo + (hi - lo) * (((float)c_lo - target) / ((float)c_lo - chi));
            if (!(p > lo && p < hi)) p = 0.5f * lo + 0.5f * hi;
            if (!(p > lo && p < hi)) {
                // lo and hi are adjacent floats: every id in [lo, hi) equals lo
                t = lo;
                have_t = true;
                break;
            }
            const int cp = R.count_ge(p);
            if (cp >= k) {
                lo = p;
            } else {
                hi = p;
                c_hi = cp;
            }
        }
    }

    // list registers (all ids >= lo), refined on a few registers per lane
    float xl[kListRegs];
    int el[kListRegs];
    const int nl = list_ok ? (c_lo + kWave - 1) / kWave : 0;
    if (list_ok) {
#pragma unroll
        for (int i = 0; i < kListRegs; ++i) {
            const int o = i * kWave + lane;
            xl[i] = kNegInf;
            el[i] = 0x7FFFFFFF;
            if (i < nl && o < c_lo) {
                xl[i] = lh[o];
                el[i] = le[o];
            }
        }
        auto cnt_l = [&](float x) {
            int n = 0;
#pragma unroll
            for (int i = 0; i < kListRegs; ++i)
                if (i < nl) n += popc(ballot(xl[i] >= x));
            return n;
        };
        hi = M;
        c_hi = cnt_l(M);
        int clo = c_lo;
        if (c_hi >= k) {
            t = M;
        } else {
            for (int it = 0; it < 48; ++it) {
                const int nw = clo - c_hi;
                if (nw <= 4 || k - c_hi <= 1) break;
                float p = lo + (hi - lo) * (((float)(clo - k) + 0.5f) / (float)nw);
                if (!(p > lo && p < hi)) p = 0.5f * lo + 0.5f * hi;
                if (!(p > lo && p < hi)) break;
                const int c = cnt_l(p);
                if (c >= k) {
                    lo = p;
                    clo = c;
                } else {
                    hi = p;
                    c_hi = c;
                }
            }
            // take distinct values from the top of [lo, hi) until the count reaches k
            for (int it = 0; it <= kListCap; ++it) {
                float m2 = kNegInf;
#pragma unroll
                for (int i = 0; i < kListRegs; ++i)
                    if (i < nl) m2 = xl[i] < hi ? __builtin_fmaxf(m2, xl[i]) : m2;
                const float xm = wave_max(m2);
                const int c = cnt_l(xm);
                if (c >= k) {
                    t = xm;
                    break;
                }
                hi = xm;
                c_hi = c;
            }
        }
        have_t = true;
    }
    if (!have_t) t = kth_by_bisection(R, k, V, M);

    // ------------------------------------------------------------ Gumbel-max
    NoiseKey nk;
    nk.k0 = a.k0;
    nk.k1 = a.k1;
    nk.t = (uint32_t)(pl - rq.offs[r]);  // offs are launch-relative
    nk.row_iter = ((uint32_t)row & 0xFFFFu) | rq.row_iter_hi[r];
    nk.rid = rq.rid[r];
    const float inv_tau = rq.inv_tau[r];
    // ids below cthr cannot beat the argmax (see the header comment)
    const float prune = M - tau * (kGumbelBound - kGumbelFloor);
    const float cthr = __builtin_fmaxf(t, prune);

    float bz = kNegInf, bh = kNegInf;
    int be = 0x7FFFFFFF;
    if (list_ok && cthr >= lo) {
        // recompact the survivors from the list registers
        int base = 0;
#pragma unroll
        for (int i = 0; i < kListRegs; ++i) {
            if (i < nl) {
                const bool pred = xl[i] >= cthr;
                const uint64_t m = ballot(pred);
                if (m) {
                    const int o = base + lanes_below(m);
                    if (pred) {
                        lh[o] = xl[i];
                        le[o] = el[i];
                    }
                    base += popc(m);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        for (int b0 = 0; b0 < base; b0 += kWave) {
            const int o = b0 + lane;
            if (o < base) {
                const float hv = lh[o];
                const int ev = le[o];
                const float z = __builtin_fmaf(hv, inv_tau, gumbel_from_word(noise_word(nk, (uint32_t)ev)));
                if (z > bz || (z == bz && ev < be)) {
                    bz = z;
                    be = ev;
                    bh = hv;
                }
            }
        }
    } else {
        // every valid id with h >= cthr, straight from the row registers
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const int ev = R.id_of(i, lane);
            const bool pred = R.h[i] >= cthr && ev >= 0 && ev < V;
            if (ballot(pred)) {
                if (pred) {
                    const float z =
                        __builtin_fmaf(R.h[i], inv_tau, gumbel_from_word(noise_word(nk, (uint32_t)ev)));
                    if (z > bz || (z == bz && ev < be)) {
                        bz = z;
                        be = ev;
                        bh = R.h[i];
                    }
                }
            }
        }
    }
    wave_argmax3(bz, be, bh);
    if (lane == 0) {
        a.tokens[cell] = be;
        a.logprobs[cell] = bh - lse;
        if (a.thresholds) a.thresholds[cell] = t + 0.0f;
    }
}

template <bool BF16, int NS>
hipError_t launch_ns(const SampleArgs& a, const ReqTable& rq, hipStream_t st) {
    const int64_t cells = (int64_t)a.rows * rq.npos;
    const int64_t blocks = (cells + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL((k_sample_small<BF16, NS>), dim3((unsigned)blocks), dim3(kWavesPerBlock * kWave), 0,
                       st, a, rq);
    return hipGetLastError();
}

// Register-slot counts that get an instantiation (bf16 rows stop at 16 slots,
// beyond which the compiler spills; those vocabularies use the row kernel).
template <bool BF16>
hipError_t dispatch(int ns, const SampleArgs& a, const ReqTable& rq, hipStream_t st) {
    if (ns <= 2) return launch_ns<BF16, 2>(a, rq, st);
    if (ns <= 4) return launch_ns<BF16, 4>(a, rq, st);
    if (ns <= 6) return launch_ns<BF16, 6>(a, rq, st);
    if (ns <= 9) return launch_ns<BF16, 9>(a, rq, st);
    if (ns <= 12) return launch_ns<BF16, 12>(a, rq, st);
    if (ns <= 16 || BF16) return launch_ns<BF16, 16>(a, rq, st);
    if constexpr (!BF16) {
        if (ns <= 24) return launch_ns<BF16, 24>(a, rq, st);
        return launch_ns<BF16, 32>(a, rq, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int small_slots_needed(bool bf16, int V) {
    // bf16: a row may start in the high half of a dword
    const int dw = bf16 ? (V + 2) / 2 : V;
    return (dw + kWave - 1) / kWave;
}

hipError_t launch_sample_small(bool bf16, const SampleArgs& a, const ReqTable& rq, hipStream_t st) {
    const int ns = small_slots_needed(bf16, a.V);
    if (ns > (bf16 ? kSmallMaxSlotsBf16 : kSmallMaxSlotsF32)) return hipErrorInvalidValue;
    return bf16 ? dispatch<true>(ns, a, rq, st) : dispatch<false>(ns, a, rq, st);
}

}  // namespace ds
