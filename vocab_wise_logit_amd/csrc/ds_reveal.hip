// ds_reveal.hip -- the confidence reveal after sampling.
//
// [ISSUE] comment on the API shape: each step scores every position of the
// canvas, ranks them by confidence and commits the best few, as a top-k over the
// request's [C, T] scores flattened row-major.  Per request this kernel returns
// the reveal_count best cells, best first, the smaller flattened index first on
// equal scores ([DRAFT]'s smallest-id rule, applied to this decision too).
//
// One 1024-thread workgroup per request:
//   1. the reveal_count-th largest score key, by a 4 x 8-bit LDS radix select over
//      the request's cells (held in registers when there are at most 16 per
//      thread, otherwise read again on every pass), which also gives the number
//      of cells tied at that key that must be taken;
//   2. one pass in flattened order collects every cell above that key, and the
//      first tied cells in index order (a block prefix count per 1024 cells);
//   3. a bitonic sort of the selected cells on the 64-bit key (order key << 32 |
//      ~index), descending: in one wave's registers when at most 128 are
//      selected (no block barrier), otherwise in LDS; then the write-out; -0 and
//      +0 rank as equal scores.
#include <stdint.h>

#include "ds_device.h"
#include "ds_kernels.h"

namespace ds {
namespace {

constexpr int NTR = kRevealThreads;
constexpr int NWR = NTR / kWave;

struct RevealLDS {
    unsigned long long sel[kRevealCap];
    uint32_t hist[256];
    int wsum[NWR];
    int nsel;
    uint32_t bcast_u;
    int bcast_i;
};

__device__ __forceinline__ uint32_t score_key(float x) { return order_key(x + 0.0f); }

// The bin holding the kk-th largest key of sh.hist[0, 256) (1 <= kk <= total);
// kk becomes the rank inside it.  Wave 0 scans the bins from the top, four per
// lane.
__device__ uint32_t pick_bin(RevealLDS& sh, int& kk) {
    if (threadIdx.x < kWave) {
        const int lane = lane_id();
        int own = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) own += (int)sh.hist[255 - (lane * 4 + i)];
        int x = own;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        const int excl = x - own;
        if (excl < kk && kk <= x) {
            int above = excl;
            for (int i = 0; i < 4; ++i) {
                const int bin = 255 - (lane * 4 + i);
                const int c = (int)sh.hist[bin];
                if (above + c >= kk) {
                    sh.bcast_u = (uint32_t)bin;
                    sh.bcast_i = above;
                    break;
                }
                above += c;
            }
        }
    }
    __syncthreads();
    const uint32_t d = sh.bcast_u;
    kk -= sh.bcast_i;
    __syncthreads();
    return d;
}

// Cells of one request, either held in registers (KPT > 0: cell f = tid + j * NTR
// for j < KPT, at most KPT * NTR cells) or read from memory on every visit.
template <int KPT>
struct Cells {
    const float* scores;
    int64_t P, off;
    int C, T, n;
    uint32_t key[KPT > 0 ? KPT : 1];

    __device__ void load() {
        if (KPT == 0) return;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int f = (int)threadIdx.x + j * NTR;
            key[j] = 0u;
            if (f < n) {
                const int c = f / T;
                key[j] = score_key(scores[(int64_t)c * P + off + (f - c * T)]);
            }
        }
    }
    // f(index, key, valid) over the cells this thread visits, in chunks of NTR
    // consecutive flattened indices (chunk by chunk, in increasing order)
    template <typename F>
    __device__ __forceinline__ void chunks(F&& fn) const {
        if (KPT > 0) {
#pragma unroll
            for (int j = 0; j < (KPT > 0 ? KPT : 1); ++j) {
                if (j * NTR >= n) break;  // uniform
                const int f = (int)threadIdx.x + j * NTR;
                fn(f, key[j], f < n);
            }
        } else {
            for (int c = 0; c < C; ++c) {
                const float* row = scores + (int64_t)c * P + off;
                for (int t0 = 0; t0 < T; t0 += NTR) {
                    const int t = t0 + (int)threadIdx.x;
                    fn(c * T + t, t < T ? score_key(row[t]) : 0u, t < T);
                }
            }
        }
    }
};

template <int KPT>
__device__ void reveal_body(const RevealArgs& a, const RevealTable& rt, RevealLDS& sh) {
    const int r = blockIdx.x;
    const int T = rt.T[r];
    const int k = rt.k[r];
    const int64_t off = rt.off[r];
    const int lane = lane_id();
    const int wv = threadIdx.x >> 6;
    Cells<KPT> cells;
    cells.scores = a.scores;
    cells.P = a.P;
    cells.off = off;
    cells.C = a.C;
    cells.T = T;
    cells.n = a.C * T;
    cells.load();

    // ---- 1. radix select of the k-th largest key
    uint32_t prefix = 0, pmask = 0;
    int kk = k;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = threadIdx.x; i < 256; i += NTR) sh.hist[i] = 0;
        __syncthreads();
        cells.chunks([&](int, uint32_t key, bool valid) {
            if (valid && (key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
        });
        __syncthreads();
        prefix |= pick_bin(sh, kk) << shift;
        pmask |= 255u << shift;
    }
    const uint32_t tkey = prefix;  // kk cells at this key are taken, in index order

    // ---- 2. collect: every cell above tkey, then the first kk cells at tkey
    if (threadIdx.x == 0) sh.nsel = 0;
    int taken = 0;  // tied cells taken so far (uniform)
    cells.chunks([&](int f, uint32_t key, bool valid) {
        const bool tie = valid && key == tkey;
        const uint64_t m = ballot(tie);
        __syncthreads();  // the previous chunk's counts have been read
        if (lane == 0) sh.wsum[wv] = popc(m);
        __syncthreads();
        int before = taken + lanes_below(m);
        int chunk = 0;
        for (int w2 = 0; w2 < NWR; ++w2) {
            if (w2 < wv) before += sh.wsum[w2];
            chunk += sh.wsum[w2];
        }
        const bool take = (valid && key > tkey) || (tie && before < kk);
        const uint64_t tm = ballot(take);
        if (tm) {
            int base = 0;
            const int leader = (int)__builtin_ctzll(tm);
            if (lane == leader) base = atomicAdd(&sh.nsel, popc(tm));
            base = __builtin_amdgcn_readlane(base, leader);
            if (take) sh.sel[base + lanes_below(tm)] = ((unsigned long long)key << 32) | (unsigned long long)(~(uint32_t)f);
        }
        taken += chunk;
    });
    __syncthreads();

    // ---- 3. bitonic sort of the k selected keys, descending (pad with 0)
    if (k <= 2 * kWave) {
        // one wave sorts 128 keys in registers, two per lane (key e = lane + 64 h):
        // the partner of e at a stride below 64 is in lane ^ stride, read with a
        // shuffle, at stride 64 it is the lane's other key; no block barrier
        if (wv == 0) {
            unsigned long long x[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) x[h] = lane + kWave * h < k ? sh.sel[lane + kWave * h] : 0ull;
            for (int size = 2; size <= 2 * kWave; size <<= 1) {
                for (int stride = size >> 1; stride > 0; stride >>= 1) {
                    if (stride == kWave) {
                        // e = lane is the lower of the pair; (lane & size) == 0 here
                        const bool desc = (lane & size) == 0;
                        const unsigned long long hi = x[0] > x[1] ? x[0] : x[1];
                        const unsigned long long lo = x[0] > x[1] ? x[1] : x[0];
                        x[0] = desc ? hi : lo;
                        x[1] = desc ? lo : hi;
                    } else {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int e = lane + kWave * h;
                            const unsigned long long y = __shfl_xor(x[h], stride);
                            const bool lower = (e & stride) == 0;
                            const bool desc = (e & size) == 0;  // the same for both keys of the pair
                            const bool take_max = lower == desc;
                            x[h] = take_max ? (x[h] > y ? x[h] : y) : (x[h] > y ? y : x[h]);
                        }
                    }
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
                if (lane + kWave * h < k) sh.sel[lane + kWave * h] = x[h];
        }
        __syncthreads();
    }
    int N = 1;
    while (N < k) N <<= 1;
    if (k <= 2 * kWave) N = 1;  // sorted above
    for (int i = k + (int)threadIdx.x; i < N; i += NTR) sh.sel[i] = 0ull;
    __syncthreads();
    for (int size = 2; size <= N; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < (N >> 1); i += NTR) {
                const int lo = (i / stride) * 2 * stride + (i % stride);
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const unsigned long long x = sh.sel[lo], y = sh.sel[hi];
                if ((x < y) == desc) {
                    sh.sel[lo] = y;
                    sh.sel[hi] = x;
                }
            }
            __syncthreads();
        }
    }

    // ---- 4. write-out (the score as the caller gave it, -0 included)
    const int64_t o = rt.out[r];
    for (int j = threadIdx.x; j < k; j += NTR) {
        const int f = (int)(~(uint32_t)sh.sel[j]);
        a.index_out[o + j] = f;
        if (a.score_out) {
            const int c = f / T;
            a.score_out[o + j] = a.scores[(int64_t)c * a.P + off + (f - c * T)];
        }
    }
}

// Requests of up to 16 * 1024 cells keep their keys in registers (one load each);
// larger ones read their cells on every pass.
__global__ __launch_bounds__(NTR) void k_reveal_topk(RevealArgs a, RevealTable rt) {
    __shared__ RevealLDS sh;
    const int r = blockIdx.x;
    if (rt.k[r] == 0) return;
    const int n = a.C * rt.T[r];
    if (n <= NTR)
        reveal_body<1>(a, rt, sh);
    else if (n <= 4 * NTR)
        reveal_body<4>(a, rt, sh);
    else if (n <= 16 * NTR)
        reveal_body<16>(a, rt, sh);
    else
        reveal_body<0>(a, rt, sh);
}

}  // namespace

hipError_t launch_reveal_topk(const RevealArgs& a, const RevealTable& rt, hipStream_t st) {
    if (rt.n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_reveal_topk, dim3((unsigned)rt.n), dim3(NTR), 0, st, a, rt);
    return hipGetLastError();
}

}  // namespace ds
