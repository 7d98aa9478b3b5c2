// ds_row.hip -- streaming kernels for large vocabularies.
//
// A row is cut into contiguous vocabulary chunks ([DRAFT] "Design and
// invariants": each tensor-parallel shard reduces its part of the vocabulary to
// (max, log-sum-exp, argmax); here the shards are chunks of one row on one GPU),
// and each chunk into `ppc` parts.  One 512-thread workgroup streams one part
// once from HBM in 16-byte pieces, four pieces per thread per group, keeping an
// online max and exp-sum per thread, and writes a partial record to the
// workspace.  A second, small kernel merges each row's partial records in
// order: larger max wins, equal maxima keep the smaller id, sums add in
// probability space.  The kernel boundary is the only synchronisation; no
// workgroup ever waits for another.
//
// Sampling ([ISSUE] comment on the API shape: top-ratio filter plus Gumbel).
// While it streams, a part keeps a bound below which no id can win the Gumbel
// race: after its first group every lane scores its own maximum so far and the
// block adopts the bound of the best score (an id whose h is below
// (z - Gmax) * tau loses to the id that scored z); every later batch of scores
// raises it.  Pieces, then ids, at or above the bound are queued in LDS and
// scored 64 at a time, one per lane, so the noise costs one Philox block per
// queued id and nothing for the rest.  The part records its best (score, id, h)
// and how many ids it queued.  Every id that can win the row's race was queued
// by its part, so if the parts queued at most top_k ids in all, every id that
// can win lies inside the top-ratio set and the best of the part winners is the
// row's winner.  Otherwise (a flat row), when the fallback is forced, or for the
// threshold output, the merge runs a radix select of the threshold (two passes
// over the row when the threshold's first-digit bin fits in LDS).  The race's
// winner is the argmax over every id, kept or not, so once it is known to be
// kept it is the row's winner; only when it is not, or without a race, does a
// Gumbel pass over every kept id follow.
#include <stdint.h>

#include "ds_device.h"
#include "ds_kernels.h"

#include <type_traits>

namespace ds {
namespace {

constexpr int NT = kRowThreads;
constexpr int U = kRowU;
// The parts kernel with the threshold window runs smaller workgroups: its
// per-wave work at the ends of a part (the first group's race bound, the queue
// drains) is then spread over four times as many groups.
template <bool WIN>
constexpr int kPartThreads = WIN ? kRowThreadsWin : kRowThreads;
template <bool WIN>
constexpr int kPartWaves = kPartThreads<WIN> / kWave;

// One wave's share of a part: (max, exp-sum, argmax) and its race winner.
struct WaveRec {
    float m, s;
    int id;
    float bz, bh;
    int be, nq;
    int above;  // keys above the row's threshold window
};

// Cross-wave reduction slots of a block of NW_ waves.
template <int NW_>
struct RedT {
    float f[NW_];
    float f2[NW_];
    int i[NW_];
    WaveRec w[NW_];
    uint32_t bcast_u;
    int bcast_i;
};

// A sampled part's Gumbel race queues, per wave: pieces holding an id at or
// above the bound (their decoded h and first id), and ids at or above the bound.
// Each is drained once it holds 64 entries, and one step adds at most 64, so 128
// entries never overflow.  The pieces' h are stored element-major ([element]
// [entry]): a drain reads element i of 64 consecutive entries, one per lane, and
// with the entries contiguous per element those reads (and the writes) fall on
// distinct banks.
template <bool BF16, bool SAMPLE, bool WIN = false>
struct PartLDS {
    static constexpr int EPP = BF16 ? 8 : 4;
    static constexpr int kQ = SAMPLE ? 2 * kWave : 1;
    static constexpr int NW = kPartWaves<WIN>;
    float ph[NW][EPP][kQ];
    int pv[NW][kQ];
    Cand q[NW][kQ];
    // threshold window: pieces holding an id inside it (up to 64 per wave, ids
    // outside the part as NaN), and the h (raw bits) of those ids, staged per wave
    // and written to the row's key buffer 64 at a time
    float wq[NW][EPP][WIN ? kWave : 1];
    uint32_t wk[NW][WIN ? 2 * kWave : 1];
    uint32_t bkey;  // order key of the block's race bound (only grows)
    RedT<NW> r;
};

// What a part needs to know about its row's threshold window.
struct WinCtx {
    bool on;          // the row has a window
    float lo, hi;     // its bounds as floats
    uint32_t* keys;   // the row's buffer [kWinKeysPerRow] of h (raw bits) inside the window
    int32_t* count;   // keys appended to it by all of the row's parts
};

// The exact threshold select: digits of 11, 11 and 10 bits of the order key;
// the keys sharing the first digit with the answer are kept in LDS when they fit.
constexpr int kDigitShift[3] = {21, 10, 0};
constexpr int kDigitBits[3] = {11, 11, 10};
constexpr int kHistBins = 2048;

// The merge runs in one of two shapes.  When the call asks for no threshold, a
// row's merge almost always only folds its part records, so the kernel is
// latency-bound: small blocks with little LDS let every row of a launch run at
// once.  When every row needs the exact select over the row (the threshold
// without a window, or the forced fallback), larger blocks keep more keys of the
// threshold's first-digit bin in LDS, which saves passes over the row.
constexpr int kMergeStage = 64;    // part records staged in LDS at a time
constexpr int kMergeThreadsFast = 256;
constexpr int kKeyCapFast = 2048;
constexpr int kMergeThreadsExact = 512;
// 8064, not 8192: with it a 512-thread block's LDS (keys, the 2048-bin
// histogram, the reduction slots) stays under 40 KB, so four blocks fit a CU.
constexpr int kKeyCapExact = 8064;
// With the threshold window the merge selects among the window's keys in global
// memory and needs LDS keys only when the window misses, so it takes the small
// shape: eight of its blocks share a compute unit and a 2048-row launch runs in
// one round (29.4 -> 25.8 us on the large-vocabulary step).
constexpr int kMergeThreadsWin = kMergeThreadsFast;
constexpr int kKeyCapWin = kKeyCapFast;
// The window kernel: one workgroup per row, a sample of the row histogrammed in
// LDS.  Its sample of up to kWindowSample ids (30 runs of 512 bf16 ids): the
// window's width goes as 1 / sqrt(sampled share), and the parts' and the merge's
// work with it, against the sample's reads here.  On the large-vocabulary step
// (thresholds included) 7168 ids: window 25 us, parts 500, merge 37; 15360: 42,
// 467, 30 (28 us less in all); 31744: 126, 443, 27.  Each wave of a 256-thread
// workgroup takes its eight runs four at a time (kWindowBatch): 36 us for the
// 15360-id sample, against 41 us with every run of a 512-thread workgroup's
// waves in registers at once (two rounds of 1024 rows).  The sample's 123 MB of
// 1 KB pieces scattered over the rows read at about 3.4 TB/s, which is most of
// that time.
constexpr int kWindowThreads = 256;
constexpr int kWindowSample = 16128;
constexpr int kWindowBatch = 4;

// The merge's staged part records (or the threshold select's keys) and histogram.
template <int MT_, int KCAP>
struct MergeLDS {
    static constexpr int kThreads = MT_;
    static constexpr int kKeyCap = KCAP;
    union {
        PartRec rec[kMergeStage];
        uint32_t keys[KCAP];
    } u;
    uint32_t hist[kHistBins];
    int nkeys;
    int nabove;
    RedT<MT_ / kWave> r;
};

// The window kernel's LDS: the sample's histogram and the reduction slots.
template <int BT_>
struct WindowLDS {
    static constexpr int kThreads = BT_;
    uint32_t hist[kHistBins];
    RedT<BT_ / kWave> r;
};

// Block argmax of (z, id, h): larger z, then smaller id.
template <int NW_>
__device__ __forceinline__ void block_argmax3(float& z, int& id, float& hv, RedT<NW_>& r) {
    const int wl = wave_argmax(z, id);
    hv = readlane_f(hv, wl);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if (lane_id() == 0) {
        r.f[w] = z;
        r.i[w] = id;
        r.f2[w] = hv;
    }
    __syncthreads();
    z = r.f[0];
    id = r.i[0];
    hv = r.f2[0];
#pragma unroll
    for (int i = 1; i < NW_; ++i) {
        const bool take = (r.f[i] > z) || (r.f[i] == z && r.i[i] < id);
        z = take ? r.f[i] : z;
        id = take ? r.i[i] : id;
        hv = take ? r.f2[i] : hv;
    }
}

// ------------------------------------------------------------- row geometry

template <bool BF16>
struct Piece {
    static constexpr int EPP = BF16 ? 8 : 4;  // ids per 16-byte piece
    float h[EPP];
};

// FIX = false leaves the NaN of a masked id under guidance in h (see guided_raw).
template <bool BF16, bool FIX = true>
__device__ __forceinline__ void decode_piece(const u32x4 cw, const u32x4 uw, float s, bool use_u,
                                             Piece<BF16>& P) {
    if (BF16) {
        const uint32_t cc[4] = {cw.x, cw.y, cw.z, cw.w};
        if (use_u) {
            const uint32_t uu[4] = {uw.x, uw.y, uw.z, uw.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                P.h[2 * i] = FIX ? guided(bf16_lo(cc[i]), bf16_lo(uu[i]), s)
                                 : guided_raw(bf16_lo(cc[i]), bf16_lo(uu[i]), s);
                P.h[2 * i + 1] = FIX ? guided(bf16_hi(cc[i]), bf16_hi(uu[i]), s)
                                     : guided_raw(bf16_hi(cc[i]), bf16_hi(uu[i]), s);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                P.h[2 * i] = bf16_lo(cc[i]);
                P.h[2 * i + 1] = bf16_hi(cc[i]);
            }
        }
    } else {
        const float cf[4] = {__uint_as_float(cw.x), __uint_as_float(cw.y), __uint_as_float(cw.z),
                             __uint_as_float(cw.w)};
        if (use_u) {
            const float uf[4] = {__uint_as_float(uw.x), __uint_as_float(uw.y), __uint_as_float(uw.z),
                                 __uint_as_float(uw.w)};
#pragma unroll
            for (int i = 0; i < 4; ++i) P.h[i] = FIX ? guided(cf[i], uf[i], s) : guided_raw(cf[i], uf[i], s);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) P.h[i] = cf[i];
        }
    }
}

// One row inside the 16-byte-aligned views of c and u.
struct RowGeom {
    gptr<u32x4> c16;
    gptr<u32x4> u16;
    int64_t gbase;  // element index of id 0 in the aligned view
    int V;
    int L;          // chunk length ceil(V / nch)
    int nch;
    int ppc;        // parts per chunk
};

// Pieces [q0, q1] (q1 < q0 when empty) holding part `q` of chunk `j`, whose ids are
// [lo, hi).
template <bool BF16>
struct PartRange {
    int lo, hi;
    int64_t q0, q1;
    __device__ PartRange(const RowGeom& G, int j, int q) {
        constexpr int EPP = Piece<BF16>::EPP;
        lo = min(G.V, j * G.L);
        hi = min(G.V, lo + G.L);
        q0 = 0;
        q1 = -1;
        if (hi > lo) {
            const int64_t c0 = (G.gbase + lo) / EPP;
            const int64_t c1 = (G.gbase + hi - 1) / EPP;
            const int64_t per = (c1 - c0 + G.ppc) / G.ppc;
            q0 = c0 + (int64_t)q * per;
            q1 = min(c1, q0 + per - 1);
        }
    }
};

// Visit every id of the row: f(v, h).  Used by the exact multi-pass path; four
// pieces per thread are loaded before any is decoded, so that a single
// workgroup keeps enough loads in flight to stream its row.
template <bool BF16, int BT, typename F>
__device__ __forceinline__ void for_each_id(const RowGeom& G, float s, bool use_u, F&& f) {
    constexpr int EPP = Piece<BF16>::EPP;
    constexpr int UF = 4;
    const int64_t q0 = G.gbase / EPP;
    const int64_t q1 = (G.gbase + G.V - 1) / EPP;
    for (int64_t qb = q0 + threadIdx.x; qb <= q1; qb += (int64_t)BT * UF) {
        u32x4 cw[UF], uw[UF];
#pragma unroll
        for (int i = 0; i < UF; ++i) {
            const int64_t q = qb + (int64_t)i * BT;
            cw[i] = u32x4{0u, 0u, 0u, 0u};
            uw[i] = cw[i];
            if (q <= q1) {
                cw[i] = stream_load(G.c16 + q);
                if (use_u) uw[i] = stream_load(G.u16 + q);
            }
        }
#pragma unroll
        for (int i = 0; i < UF; ++i) {
            const int64_t q = qb + (int64_t)i * BT;
            if (q > q1) break;
            Piece<BF16> P;
            decode_piece<BF16>(cw[i], uw[i], s, use_u, P);
            const int64_t v0 = q * EPP - G.gbase;
#pragma unroll
            for (int e = 0; e < EPP; ++e)
                if (v0 + e >= 0 && v0 + e < G.V) f((int)(v0 + e), P.h[e]);
        }
    }
}

// The digit (histogram bin) holding the kk-th largest key among those counted
// in sh.hist[0, nbins), with 1 <= kk <= their number; kk becomes the rank inside
// that bin.  Thread j owns bins nbins-1-j*b .. nbins-b-j*b (b = nbins / threads),
// so a block prefix sum over the threads counts the keys in higher bins.
template <typename SH>
__device__ uint32_t find_digit(SH& sh, int nbins, int& kk) {
    const int bpt = nbins / SH::kThreads;
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // wave-uniform, in a scalar register
    int own = 0;
    for (int i = 0; i < bpt; ++i) own += (int)sh.hist[nbins - 1 - ((int)threadIdx.x * bpt + i)];
    int x = own;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == kWave - 1) sh.r.i[wv] = x;
    __syncthreads();
    int base = 0;
    for (int w2 = 0; w2 < wv; ++w2) base += sh.r.i[w2];
    const int incl = base + x;
    const int excl = incl - own;
    if (excl < kk && kk <= incl) {
        int above = excl;
        for (int i = 0; i < bpt; ++i) {
            const int bin = nbins - 1 - ((int)threadIdx.x * bpt + i);
            const int c = (int)sh.hist[bin];
            if (above + c >= kk) {
                sh.r.bcast_u = (uint32_t)bin;
                sh.r.bcast_i = above;
                break;
            }
            above += c;
        }
    }
    __syncthreads();
    const uint32_t d = sh.r.bcast_u;
    kk -= sh.r.bcast_i;
    __syncthreads();
    return d;
}

// Wave-aggregated append to an LDS counter; returns this lane's slot or -1.
__device__ __forceinline__ int wave_append(bool pred, int* counter) {
    const uint64_t m = ballot(pred);
    if (!m) return -1;
    int base = 0;
    const int leader = (int)__builtin_ctzll(m);
    if (lane_id() == leader) base = atomicAdd(counter, popc(m));
    base = __builtin_amdgcn_readlane(base, leader);
    return pred ? base + lanes_below(m) : -1;
}

// One pass of an LDS radix select: histogram the digit `dg` of the keys that
// share the selected prefix (from LDS, or over the whole row), then fix that
// digit (the bin holding the kk-th largest; kk becomes the rank inside it).
template <bool BF16, typename SH>
__device__ __forceinline__ void select_pass(const RowGeom& G, float s, bool use_u, SH& sh, int dg, bool from_lds, int n,
                                            uint32_t& prefix, uint32_t& pmask, int& kk) {
    constexpr int BT = SH::kThreads;
    const int shift = kDigitShift[dg];
    const uint32_t dmask = (1u << kDigitBits[dg]) - 1u;
    for (int i = threadIdx.x; i < kHistBins; i += BT) sh.hist[i] = 0;
    __syncthreads();
    if (from_lds) {
        for (int i = threadIdx.x; i < n; i += BT) {
            const uint32_t key = sh.u.keys[i];
            if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dmask], 1u);
        }
    } else {
        for_each_id<BF16, BT>(G, s, use_u, [&](int, float h) {
            const uint32_t key = order_key(h + 0.0f);
            if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dmask], 1u);
        });
    }
    __syncthreads();
    const uint32_t d = find_digit(sh, 1 << kDigitBits[dg], kk);
    prefix |= d << shift;
    pmask |= dmask << shift;
}

// The rank-th largest of the n keys in sh.u.keys (1 <= rank <= n), exactly.
template <bool BF16, typename SH>
__device__ __forceinline__ uint32_t lds_kth(const RowGeom& G, SH& sh, int n, int rank) {
    uint32_t prefix = 0, pmask = 0;
    int kk = rank;
    select_pass<BF16>(G, 0.0f, false, sh, 0, true, n, prefix, pmask, kk);
    select_pass<BF16>(G, 0.0f, false, sh, 1, true, n, prefix, pmask, kk);
    select_pass<BF16>(G, 0.0f, false, sh, 2, true, n, prefix, pmask, kk);
    return prefix;
}

// A window of order keys that holds the row's top_k-th largest key with high
// probability, from a sample of the row: the ids of every `every`-th run of 64
// pieces (at most SCAP ids), one histogram of their h over kHistBins equal bins,
// and the bins holding the sample's order statistics at ranks k * n / V -+
// (sigmas standard deviations + 4).  The window [key_lo, key_hi] runs from the
// lower edge of the one bin to the upper edge of the other (open at an end bin),
// and is expected to hold about 2 (sigmas sqrt(k f) + 4) / f row ids (f the
// sampled share) plus a bin's width at either end; whether it holds the answer
// is checked by whoever uses it.  The bins are a non-decreasing function of h,
// so ranks counted over them bracket the sample's order statistics.
//
// Each wave takes its runs RB at a time (all of them at once by default),
// loading a batch's runs before it decodes any.  The bins span the finite range
// of the first batch; with later batches that range is widened by a quarter on
// either side and what lies beyond it goes to the end bins.  Returns false (no
// window) when the row is too short for a sample to pay, the expected window
// would not leave room in `cap` keys, or the first batch's finite values are all
// equal.
template <bool BF16, int SCAP, int RB_ = 0, typename SH>
__device__ __forceinline__ bool sample_window(const RowGeom& G, float s, bool use_u, int k, SH& sh, float sigmas,
                                              int cap, uint32_t& key_lo, uint32_t& key_hi) {
    constexpr int BT = SH::kThreads;
    constexpr int NW = BT / kWave;
    constexpr int EPP = Piece<BF16>::EPP;
    constexpr int kRunIds = kWave * EPP;
    constexpr int kSampleRuns = SCAP / kRunIds - 1;
    constexpr int RPW = (kSampleRuns + NW - 1) / NW;  // runs per wave
    constexpr int RB = RB_ > 0 && RB_ < RPW ? RB_ : RPW;  // runs per batch
    constexpr int NB = (RPW + RB - 1) / RB;
    static_assert(kSampleRuns >= 1, "a sample of at least one run");
    const int64_t q0 = G.gbase / EPP;
    const int64_t q1 = (G.gbase + G.V - 1) / EPP;
    const int64_t runs = (q1 - q0) / kWave + 1;
    const int every = (int)((runs + kSampleRuns - 1) / kSampleRuns);
    const int nsr = (int)((runs + every - 1) / every);  // runs in the sample, at most kSampleRuns
    // the window's expected width in row ids, 2 m / f with f the sampled share,
    // must leave room in `cap` keys (checked again on the sample actually drawn)
    const float f_exp = (float)(nsr * kRunIds) / (float)G.V;
    const float m_exp = sigmas * __builtin_sqrtf((float)k * f_exp) + 4.0f;
    if (!(every >= 4 && 2.0f * m_exp < 0.7f * (float)cap * f_exp)) return false;
    const int wv = threadIdx.x / kWave;
    const int lane = lane_id();
    for (int i = threadIdx.x; i < kHistBins; i += BT) sh.hist[i] = 0;
    float lo_f = 0.0f, scale = 0.0f;  // bin of h: trunc(fma(h, scale, -lo_f * scale)), clamped to the bins
    int nv = 0;                       // sampled ids of this lane (every one is binned once)
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) {
        // run wv + j * NW of the sample is run (wv + j * NW) * every of the row
        u32x4 cw[RB], uw[RB];
#pragma unroll
        for (int jj = 0; jj < RB; ++jj) {
            const int i = wv + (bt * RB + jj) * NW;
            const int64_t q = q0 + (int64_t)i * every * kWave + lane;
            cw[jj] = u32x4{0u, 0u, 0u, 0u};
            uw[jj] = cw[jj];
            if (bt * RB + jj < RPW && i < nsr && q <= q1) {
                cw[jj] = stream_load(G.c16 + q);
                if (use_u) uw[jj] = stream_load(G.u16 + q);
            }
        }
        // h of the batch's ids (NaN where a slot holds none, and for a masked id
        // under guidance: such ids are counted as sampled but binned nowhere,
        // which ranks them below every bin, where a masked id belongs), and of
        // the first batch the range
        float h[RB][EPP];
        float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
        for (int jj = 0; jj < RB; ++jj) {
            const int i = wv + (bt * RB + jj) * NW;
            const int64_t q = q0 + (int64_t)i * every * kWave + lane;
            const int64_t v0 = q * EPP - G.gbase;
            const bool pv = bt * RB + jj < RPW && i < nsr && q <= q1;  // a piece was loaded
            Piece<BF16> P;
            decode_piece<BF16, false>(cw[jj], uw[jj], s, use_u, P);
            // a missing piece, or one reaching past the row (a row's first and
            // last pieces only): its ids outside the row as NaN
            int nvp = EPP;
            if (!(pv && v0 >= 0 && v0 + EPP <= G.V)) {
                nvp = 0;
#pragma unroll
                for (int e = 0; e < EPP; ++e) {
                    const bool in = pv && v0 + e >= 0 && v0 + e < G.V;
                    if (!in) P.h[e] = __builtin_nanf("");
                    nvp += in ? 1 : 0;
                }
            }
            nv += nvp;
#pragma unroll
            for (int e = 0; e < EPP; ++e) {
                h[jj][e] = P.h[e];
                if (bt == 0) {  // (a NaN changes neither)
                    mn = __builtin_fminf(mn, P.h[e]);
                    mx = __builtin_fmaxf(mx, P.h[e]);
                }
            }
        }
        if (bt == 0) {
            // the block's min and max of the lanes' values (every read done
            // before the slots are written again)
            auto block_range = [&](float a, float b, float& lo, float& hi) {
                const float wa = wave_min(a), wb = wave_max(b);
                if (lane == 0) {
                    sh.r.f[wv] = wa;
                    sh.r.f2[wv] = wb;
                }
                __syncthreads();
                lo = __builtin_inff();
                hi = -__builtin_inff();
#pragma unroll
                for (int w2 = 0; w2 < NW; ++w2) {
                    lo = __builtin_fminf(lo, sh.r.f[w2]);
                    hi = __builtin_fmaxf(hi, sh.r.f2[w2]);
                }
                __syncthreads();
            };
            float bmn, bmx;
            block_range(mn, mx, bmn, bmx);
            if (!(bmn > -__builtin_inff() && bmx < __builtin_inff())) {
                // an infinite h in the first batch (a masked id, or an overflow):
                // the finite range instead
                mn = __builtin_inff();
                mx = -__builtin_inff();
#pragma unroll
                for (int jj = 0; jj < RB; ++jj)
#pragma unroll
                    for (int e = 0; e < EPP; ++e)
                        if (__builtin_fabsf(h[jj][e]) < __builtin_inff()) {
                            mn = __builtin_fminf(mn, h[jj][e]);
                            mx = __builtin_fmaxf(mx, h[jj][e]);
                        }
                block_range(mn, mx, bmn, bmx);
            }
            const float pad = NB > 1 ? 0.25f * (bmx - bmn) : 0.0f;
            lo_f = bmn - pad;
            scale = (float)kHistBins / ((bmx + pad) - lo_f);
            if (!(bmx > bmn && scale < __builtin_inff())) return false;
        }
        // a non-decreasing function of h (-inf to the lowest bin, +inf to the
        // highest, NaN to none)
        const float off = -lo_f * scale;
#pragma unroll
        for (int jj = 0; jj < RB; ++jj)
#pragma unroll
            for (int e = 0; e < EPP; ++e) {
                const float x = h[jj][e];
                if (x == x) {
                    const float t = __builtin_amdgcn_fmed3f(__builtin_fmaf(x, scale, off), 0.0f, (float)(kHistBins - 1));
                    atomicAdd(&sh.hist[(int)t], 1u);
                }
            }
    }
    {
        const int wn = wave_sum_i(nv);
        if (lane == 0) sh.r.i[wv] = wn;
    }
    __syncthreads();
    int ns = 0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) ns += sh.r.i[w2];
    __syncthreads();  // every read of the counts before find_digit reuses their slots
    // expected sample rank of the answer and a margin of `sigmas` standard deviations
    const float f = (float)ns / (float)G.V;
    const float r = (float)k * f;
    const float m = sigmas * __builtin_sqrtf(r) + 4.0f;
    if (!(ns > 0 && 2.0f * m < 0.7f * (float)cap * f)) return false;
    const int r_hi = (int)__builtin_floorf(r - m);
    const int r_lo = (int)__builtin_ceilf(r + m);
    const float width = __builtin_amdgcn_rcpf(scale);  // of a bin, the edges lo_f + b * width
    key_hi = 0xFFFFFFFFu;  // open above
    key_lo = 0u;           // open below
    if (r_hi >= 1) {
        int kh = r_hi;
        const int b = (int)find_digit(sh, kHistBins, kh);
        if (b + 1 < kHistBins) key_hi = order_key(__builtin_fmaf((float)(b + 1), width, lo_f) + 0.0f);
    }
    if (r_lo <= ns) {
        int kl = r_lo;
        const int b = (int)find_digit(sh, kHistBins, kl);
        if (b > 0) key_lo = order_key(__builtin_fmaf((float)b, width, lo_f) + 0.0f);
    }
    return true;
}

// The rank-th largest (1 <= rank <= n) order key of the n h values (raw bits,
// keys of h + 0) in global memory at hb, all with keys in [base, base + span]: a
// radix select on key - base with as many 11-bit digits as the span needs (a
// narrow span would otherwise put every key of the first digit into one bin),
// each pass reading the values again (they are few, and cached after the first).
template <typename SH>
__device__ __forceinline__ uint32_t window_kth(SH& sh, const uint32_t* hb, int n, int rank, uint32_t base,
                                               uint32_t span) {
    constexpr int BT = SH::kThreads;
    constexpr int kBits = 11;
    static_assert((1 << kBits) == kHistBins, "one digit per histogram");
    const gptr<uint32_t> g = as_global<uint32_t>(hb);
    const int span_bits = span ? 32 - __builtin_clz(span) : 1;
    const int passes = (span_bits + kBits - 1) / kBits;
    uint32_t prefix = 0, pmask = 0;
    int kk = rank;
    for (int pidx = passes - 1; pidx >= 0; --pidx) {
        const int shift = kBits * pidx;
        const uint32_t dmask = (1u << kBits) - 1u;
        for (int i = threadIdx.x; i < kHistBins; i += BT) sh.hist[i] = 0;
        __syncthreads();
        auto add = [&](uint32_t bits) {
            const uint32_t rel = order_key(__uint_as_float(bits) + 0.0f) - base;
            if ((rel & pmask) == prefix) atomicAdd(&sh.hist[(rel >> shift) & dmask], 1u);
        };
        int i = threadIdx.x;
        for (; i + 3 * BT < n; i += 4 * BT) {  // four loads in flight per thread
            const uint32_t a = g[i], b = g[i + BT], c = g[i + 2 * BT], d = g[i + 3 * BT];
            add(a);
            add(b);
            add(c);
            add(d);
        }
        for (; i < n; i += BT) add(g[i]);
        __syncthreads();
        const uint32_t d = find_digit(sh, kHistBins, kk);
        prefix |= d << shift;
        pmask |= shift + kBits >= 32 ? ~0u << shift : dmask << shift;
    }
    return base + prefix;
}

// The float bounds of a key window, for comparing h directly (the key order is
// the order of h + 0, and h is never NaN where this is used); the open ends,
// keys 0xFFFFFFFF and 0 (which decode to NaN), become +-inf.
__device__ __forceinline__ float window_hi(uint32_t key_hi) {
    return key_hi == 0xFFFFFFFFu ? __builtin_inff() : key_value(key_hi);
}
__device__ __forceinline__ float window_lo(uint32_t key_lo) {
    return key_lo == 0u ? -__builtin_inff() : key_value(key_lo);
}

// Exact top_k-th largest h of the row (an LDS radix select on order keys), by
// passes over the row.
//
// On long rows a sample comes first (sample_window), then one pass over the row
// counts the keys above the window and collects those inside it; when the k-th
// largest falls inside and the window fits in LDS, it is selected there
// exactly.  Otherwise (an unlucky sample, or too many keys in the window) the
// full path runs: one pass histograms the first 11-bit digit, a second collects
// the keys in the chosen bin into LDS, where the last two digits are selected,
// and if that bin holds more than kKeyCap keys the last digits take a pass over
// the row each.  The result is exact either way; the sample only saves a pass.
template <bool BF16, typename SH>
__device__ __forceinline__ float radix_select_row(const RowGeom& G, float s, bool use_u, int k, SH& sh) {
    constexpr int BT = SH::kThreads;
    uint32_t key_lo, key_hi;
    if (sample_window<BF16, SH::kKeyCap>(G, s, use_u, k, sh, 3.0f, SH::kKeyCap, key_lo, key_hi)) {
        if (threadIdx.x == 0) {
            sh.nkeys = 0;
            sh.nabove = 0;
        }
        __syncthreads();
        const float f_hi = window_hi(key_hi);
        const float f_lo = window_lo(key_lo);
        int above = 0;
        for_each_id<BF16, BT>(G, s, use_u, [&](int, float h) {
            above += h > f_hi ? 1 : 0;
            const int at = wave_append(h >= f_lo && h <= f_hi, &sh.nkeys);
            if (at >= 0 && at < SH::kKeyCap) sh.u.keys[at] = order_key(h + 0.0f);
        });
        if (above) atomicAdd(&sh.nabove, above);
        __syncthreads();
        const int n = sh.nkeys;
        const int A = sh.nabove;
        __syncthreads();
        if (n <= SH::kKeyCap && A < k && k <= A + n) return key_value(lds_kth<BF16>(G, sh, n, k - A));
    }

    // ---- full path
    uint32_t prefix = 0, pmask = 0;
    int kk = k;
    select_pass<BF16>(G, s, use_u, sh, 0, false, 0, prefix, pmask, kk);
    // keep the keys that share the first digit with the answer
    if (threadIdx.x == 0) sh.nkeys = 0;
    __syncthreads();
    for_each_id<BF16, BT>(G, s, use_u, [&](int, float h) {
        const uint32_t key = order_key(h + 0.0f);
        const int at = wave_append((key & pmask) == prefix, &sh.nkeys);
        if (at >= 0 && at < SH::kKeyCap) sh.u.keys[at] = key;
    });
    __syncthreads();
    const int n = sh.nkeys;
    const bool fit = n <= SH::kKeyCap;
    select_pass<BF16>(G, s, use_u, sh, 1, fit, n, prefix, pmask, kk);
    select_pass<BF16>(G, s, use_u, sh, 2, fit, n, prefix, pmask, kk);
    return key_value(prefix);
}

// ----------------------------------------------------------- one part

// Per-cell parameters of one sampled (or greedy) row.
struct CellParams {
    int64_t cell;   // index into the [C, P] outputs; times V, into c
    int64_t ucell;  // times V, into u (cell unless u is compacted; then V * b is a multiple of 16)
    float s, tau, inv_tau;
    NoiseKey nk;
};

struct PartOut {
    float m, s;
    int id;
    bool nan;  // (all threads) some wave's exp-sum is NaN: redo the part with FIX
    // Gumbel race of a sampled part: best (score, id, h) among the queued ids and
    // how many ids were queued
    float bz, bh;
    int be, nq;
    int above;  // keys above the threshold window (WIN)
};

// Stream one part: online max / exp-sum per thread, block-reduced to (m, s,
// smallest argmax).  A thread notes the id of its maximum while the group that
// raised it is still in registers, so no re-read is needed at the end.  With
// `race`, each wave also runs the Gumbel race over the ids that can still win
// (queued in LDS, scored 64 at a time).  At most 64 VGPRs: four workgroups per CU
// keep enough loads in flight.
// With WIN (the threshold output requested) each thread also counts the ids
// whose h lies above the row's threshold window and appends the order keys of
// those inside it to the row's key buffer, through a per-wave LDS stage.
template <bool BF16, bool SAMPLE, bool FIX, bool WIN>
__device__ PartOut stream_part(const RowGeom& G, const PartRange<BF16>& pr, const CellParams& cp, bool use_u,
                               bool race, PartLDS<BF16, SAMPLE, WIN>& sh, const WinCtx& wc) {
    constexpr int EPP = Piece<BF16>::EPP;
    constexpr int NT = kPartThreads<WIN>;
    constexpr int NWAVES = kPartWaves<WIN>;
    const float s = cp.s;
    float m = kNegInf, acc = 0.0f;
    int mid = 0x7FFFFFFF;  // smallest id of this thread attaining m
    const int64_t nq = pr.q1 - pr.q0 + 1;
    const int its = nq > 0 ? (int)((nq + (int64_t)NT * U - 1) / ((int64_t)NT * U)) : 0;
    // piece j of this part is c16[q0 + j]; thread t takes j = it*NT*U + uu*NT + t
    const gptr<u32x4> pc = G.c16 + pr.q0;
    const gptr<u32x4> pu = G.u16 + pr.q0;
    const int nqi = (int)nq;
    const int vbase = (int)(pr.q0 * EPP - G.gbase);  // row id of element 0 of piece 0
    const int lane = lane_id();

    // Gumbel race state: wave-uniform bound, queue lengths and queued count; the
    // lane's best (score, id, h)
    const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // wave-uniform, in a scalar register
    float Bw = kNegInf;
    int pn = 0, qn = 0, qtot = 0;
    float bz = kNegInf, bh = kNegInf;
    int be = 0x7FFFFFFF;
    if (SAMPLE && race) {
        if (threadIdx.x == 0) sh.bkey = order_key(kNegInf);
        __syncthreads();
    }
    // score 64 queued ids, one per lane, and raise the bound
    auto flush_ids = [&]() {
        qn -= kWave;
        const Cand c = sh.q[wv][qn + lane];
        const float z = __builtin_fmaf(c.h, cp.inv_tau, gumbel_from_word(noise_word(cp.nk, (uint32_t)c.e)));
        if (z > bz || (z == bz && c.e < be)) {
            bz = z;
            be = c.e;
            bh = c.h;
        }
        const float nb = win_bound(wave_max(bz), cp.tau);
        if (nb > Bw) {
            Bw = nb;
            if (lane == 0) atomicMax(&sh.bkey, order_key(nb));
        }
    };
    // move the ids at or above the bound of 64 queued pieces to the id queue
    auto expand = [&](float Bq) {
        pn -= kWave;
        const int pi = pn + lane;
        const int v0 = sh.pv[wv][pi];
#pragma unroll 1
        for (int i = 0; i < EPP; ++i) {
            const float h = sh.ph[wv][i][pi];
            const bool pred = h >= Bq;
            const uint64_t mk = ballot(pred);
            if (mk) {
                if (pred) sh.q[wv][qn + lanes_below(mk)] = Cand{h, v0 + i};
                qn += popc(mk);
                qtot += popc(mk);
                if (qn >= kWave) {
                    __builtin_amdgcn_wave_barrier();
                    flush_ids();
                    __builtin_amdgcn_wave_barrier();
                    Bq = __builtin_fmaxf(Bq, Bw);
                }
            }
        }
    };

    // threshold window: ids above it, queued pieces and staged keys (all counted
    // per wave, wave-uniform)
    int wabove = 0, wqn = 0, wn = 0;
    // write the newest n (<= 64) staged keys to the row's buffer (keys past its
    // capacity are dropped; the count still grows, which marks the row's window
    // as unusable)
    auto win_flush = [&](int n) {
        int base = 0;
        if (lane == 0) base = atomicAdd(wc.count, n);
        base = __builtin_amdgcn_readlane(base, 0);
        wn -= n;
        if (lane < n && base + lane < kWinKeysPerRow) wc.keys[base + lane] = sh.wk[wv][wn + lane];
    };
    // (keys in [lo, wc.hi]; masks straight from the compares, and the lane
    // predicate from the same compares, so no mask is rebuilt from a bool)
    auto win_push = [&](float h, float lo) {
        const bool ge = h >= lo, le = h <= wc.hi;
        const uint64_t mk = __builtin_amdgcn_ballot_w64(ge) & __builtin_amdgcn_ballot_w64(le);
        if (mk) {
            if (ge & le) sh.wk[wv][wn + lanes_below(mk)] = __float_as_uint(h);
            wn += popc(mk);
            if (wn >= kWave) {
                __builtin_amdgcn_wave_barrier();
                win_flush(kWave);
                __builtin_amdgcn_wave_barrier();
            }
        }
    };
    // the ids inside the window from the queued pieces, one piece per lane
    // (a rolled loop, so that its pushes and flushes are emitted once per call)
    auto win_expand = [&]() {
        const int n = wqn;
        wqn = 0;
        // slots past the queue hold stale values: a NaN bound keeps them out (no
        // comparison with it holds)
        const float lo = lane < n ? wc.lo : __builtin_nanf("");
#pragma unroll 1
        for (int i = 0; i < EPP; ++i) win_push(sh.wq[wv][i][lane], lo);
    };

    // ids [lo, hi) cover every element of pieces 1 .. nq-2; only the first and the
    // last iteration can hold a partial or missing piece
    // raw 16-byte pieces of one group (u only when it is read)
    struct Raw {
        u32x4 c[U];
        u32x4 u[U];
    };
    auto load = [&](int it, Raw& R, bool edge) {
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
            const int j = it * NT * U + uu * NT + (int)threadIdx.x;
            if (!edge) {
                R.c[uu] = stream_load(pc + j);
                if (use_u) R.u[uu] = stream_load(pu + j);
            } else {
                const uint32_t ninf = BF16 ? 0xFF80FF80u : 0xFF800000u;
                R.c[uu] = u32x4{ninf, ninf, ninf, ninf};
                R.u[uu] = R.c[uu];
                if (j < nqi) {
                    R.c[uu] = stream_load(pc + j);
                    if (use_u) R.u[uu] = stream_load(pu + j);
                }
            }
        }
    };
    auto group = [&](int it, auto edge_tag) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        Raw raw;
        load(it, raw, EDGE);
        Piece<BF16> P[U];
        float pm[U];
        float gm = kNegInf;
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
            const int j = it * NT * U + uu * NT + (int)threadIdx.x;
            decode_piece<BF16, FIX>(raw.c[uu], raw.u[uu], s, use_u, P[uu]);
            if (EDGE) {
                const int v0 = vbase + j * EPP;
                if (v0 < pr.lo || v0 + EPP > pr.hi) {
#pragma unroll
                    for (int i = 0; i < EPP; ++i)
                        if (v0 + i < pr.lo || v0 + i >= pr.hi) P[uu].h[i] = kNegInf;
                }
            }
            pm[uu] = P[uu].h[0];
#pragma unroll
            for (int i = 1; i < EPP; ++i) pm[uu] = __builtin_fmaxf(pm[uu], P[uu].h[i]);
            gm = __builtin_fmaxf(gm, pm[uu]);
        }
        if constexpr (WIN) {
            if (wc.on) {
                // ids above the window are counted per wave; a piece with an id
                // inside it is queued whole (ids outside the part as NaN) and its
                // ids are sorted out 64 pieces at a time, which keeps the per-id
                // work to two compares
#pragma unroll
                for (int uu = 0; uu < U; ++uu) {
                    const int j = it * NT * U + uu * NT + (int)threadIdx.x;
                    const int v0 = vbase + j * EPP;
                    // lane masks straight from the compares (a bool taken through
                    // ballot() would be turned into a 0/1 value and compared again)
                    uint64_t any = 0;
#pragma unroll
                    for (int i = 0; i < EPP; ++i) {
                        const float h = P[uu].h[i];
                        const uint64_t gt = __builtin_amdgcn_ballot_w64(h > wc.hi);
                        wabove += popc(gt);
                        uint64_t in = __builtin_amdgcn_ballot_w64(h >= wc.lo) & ~gt;
                        // ids outside the part hold -inf here: never inside
                        if (EDGE) in &= __builtin_amdgcn_ballot_w64(j < nqi && v0 + i >= pr.lo && v0 + i < pr.hi);
                        any |= in;
                    }
                    // the count taken now (an empty statement that reads it): left
                    // to the compiler, the popcounts of a whole group sink to its end
                    // and keep 32 masks live, and the scalar registers they take are
                    // spilled and reloaded on every group
                    asm volatile("" : "+s"(wabove));
                    if (any) {
                        const int add = popc(any);
                        if (wqn + add > kWave) {
                            __builtin_amdgcn_wave_barrier();
                            win_expand();
                            __builtin_amdgcn_wave_barrier();
                        }
                        if (__builtin_amdgcn_inverse_ballot_w64(any)) {
                            const int at = wqn + lanes_below(any);
#pragma unroll
                            for (int i = 0; i < EPP; ++i) {
                                const bool ok = !EDGE || (j < nqi && v0 + i >= pr.lo && v0 + i < pr.hi);
                                sh.wq[wv][i][at] = ok ? P[uu].h[i] : __builtin_nanf("");
                            }
                        }
                        wqn += add;
                    }
                }
            }
        }
        if (gm > m) {
            // first piece, then first id, holding the new maximum (ids grow with
            // the piece index inside a group and with the element inside a piece)
            int id = 0x7FFFFFFF;
#pragma unroll
            for (int uu = U - 1; uu >= 0; --uu) {
                if (pm[uu] == gm) {
                    int e = EPP - 1;
#pragma unroll
                    for (int i = EPP - 1; i >= 0; --i)
                        if (P[uu].h[i] == gm) e = i;
                    id = vbase + (it * NT * U + uu * NT + (int)threadIdx.x) * EPP + e;
                }
            }
            acc *= __builtin_amdgcn_exp2f((m - gm) * kLog2e);
            m = gm;
            mid = id;
        }
        // queue bound: no id below it can win (a bound of -inf means the wave has
        // seen no finite h yet, and then nothing is queued)
        float Bq = __builtin_inff();
        if (SAMPLE && race) {
            if (EDGE && it == 0) {
                // after the first group, every lane scores its own maximum so far
                // (one Philox batch per wave, as for a single id) and the block
                // adopts the bound of the best score; these ids stay in the race
                // but are not counted, the counted queue still sees every id above
                // the bound
                if (m > kNegInf) {
                    const float z = __builtin_fmaf(m, cp.inv_tau, gumbel_from_word(noise_word(cp.nk, (uint32_t)mid)));
                    if (z > bz || (z == bz && mid < be)) {
                        bz = z;
                        be = mid;
                        bh = m;
                    }
                }
                const float nb = win_bound(wave_max(bz), cp.tau);
                if (lane == 0) atomicMax(&sh.bkey, order_key(nb));
                __syncthreads();
                Bw = key_value(sh.bkey);
            } else {
                Bw = __builtin_fmaxf(Bw, key_value(__hip_atomic_load(&sh.bkey, __ATOMIC_RELAXED,
                                                                     __HIP_MEMORY_SCOPE_WORKGROUP)));
            }
            if (Bw > kNegInf) Bq = Bw;
        }
        // a thread that has seen only -inf keeps acc = 0 (exp2(-inf) = 0)
        const float mL = (m > kNegInf) ? m * kLog2e : 0.0f;
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
#pragma unroll
            for (int i = 0; i < EPP; ++i) acc += __builtin_amdgcn_exp2f(__builtin_fmaf(P[uu].h[i], kLog2e, -mL));
            if (SAMPLE && race) {
                const bool pred = pm[uu] >= Bq;
                const uint64_t mk = ballot(pred);
                if (mk) {
                    if (pred) {
                        const int at = pn + lanes_below(mk);
#pragma unroll
                        for (int i = 0; i < EPP; ++i) sh.ph[wv][i][at] = P[uu].h[i];
                        sh.pv[wv][at] = vbase + (it * NT * U + uu * NT + (int)threadIdx.x) * EPP;
                    }
                    pn += popc(mk);
                    if (pn >= kWave) {
                        __builtin_amdgcn_wave_barrier();
                        expand(Bq);
                        __builtin_amdgcn_wave_barrier();
                        Bq = __builtin_fmaxf(Bq, Bw);
                    }
                }
            }
        }
    };
    for (int it = 0; it < its; ++it) {
        if (it == 0 || it == its - 1)
            group(it, std::true_type{});
        else
            group(it, std::false_type{});
    }
    // undo the rounding of m * log2(e) for this thread's partial sum
    if (m > kNegInf) acc *= __builtin_amdgcn_exp2f(-__builtin_fmaf(m, kLog2e, -(m * kLog2e)));
    if (SAMPLE && race) {
        // drain the queues: the last pieces (fewer than 64), then the last ids
        __builtin_amdgcn_wave_barrier();
        if (pn > 0) {
            const int take = pn;
            pn = kWave;  // expand() takes entries [pn - 64, pn): pad to a full step
            if (lane >= take) sh.pv[wv][lane] = 0;
            if (lane >= take)
#pragma unroll
                for (int i = 0; i < EPP; ++i) sh.ph[wv][i][lane] = kNegInf;
            __builtin_amdgcn_wave_barrier();
            expand(Bw);
            __builtin_amdgcn_wave_barrier();
        }
        if (lane < qn) {
            const Cand c = sh.q[wv][lane];
            const float z = __builtin_fmaf(c.h, cp.inv_tau, gumbel_from_word(noise_word(cp.nk, (uint32_t)c.e)));
            if (z > bz || (z == bz && c.e < be)) {
                bz = z;
                be = c.e;
                bh = c.h;
            }
        }
    }
    if (WIN && wc.on) {
        __builtin_amdgcn_wave_barrier();
        if (wqn > 0) win_expand();
        __builtin_amdgcn_wave_barrier();
        if (wn > 0) win_flush(wn);
    }
    // wave shares, then one exchange through LDS; thread 0 combines them
    const float wm = wave_max(m);
    const float ws = wave_sum((m > kNegInf) ? acc * __builtin_amdgcn_exp2f((m - wm) * kLog2e) : 0.0f);
    const int wid = wave_min_i((wm > kNegInf && m == wm) ? mid : 0x7FFFFFFF);
    if (SAMPLE && race) {
        const int wl = wave_argmax(bz, be);
        bh = readlane_f(bh, wl);
    }
    const int wab = WIN ? wabove : 0;
    if (lane == 0) sh.r.w[wv] = WaveRec{wm, ws, wid, bz, bh, be, qtot, wab};
    __syncthreads();
    PartOut o;
    o.nan = false;
    if (!FIX && use_u) {
#pragma unroll
        for (int i = 0; i < NWAVES; ++i) o.nan |= sh.r.w[i].s != sh.r.w[i].s;
    }
    o.m = kNegInf;
    o.s = 0.0f;
    o.id = 0x7FFFFFFF;
    o.bz = kNegInf;
    o.bh = kNegInf;
    o.be = 0x7FFFFFFF;
    o.nq = 0;
    o.above = 0;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 0; i < NWAVES; ++i) o.m = __builtin_fmaxf(o.m, sh.r.w[i].m);
#pragma unroll
        for (int i = 0; i < NWAVES; ++i) {
            const WaveRec r = sh.r.w[i];
            if (r.m > kNegInf) {
                o.s += r.s * __builtin_amdgcn_exp2f((r.m - o.m) * kLog2e);
                if (r.m == o.m) o.id = min(o.id, r.id);
            }
            if (SAMPLE && race) {
                if (r.bz > o.bz || (r.bz == o.bz && r.be < o.be)) {
                    o.bz = r.bz;
                    o.be = r.be;
                    o.bh = r.bh;
                }
                o.nq += r.nq;
            }
            o.above += r.above;
        }
    }
    return o;
}

// --------------------------------------------------------------- kernels

template <bool BF16>
__device__ __forceinline__ RowGeom row_geom(const void* cptr, const void* uptr, bool use_u, int64_t cell, int V,
                                             int nch, int ppc) {
    constexpr int ES = BF16 ? 2 : 4;
    const uintptr_t cb = (uintptr_t)cptr;
    RowGeom G;
    G.c16 = as_global<u32x4>((const char*)cptr - (cb & 15));
    G.u16 = use_u ? as_global<u32x4>((const char*)uptr - (cb & 15)) : G.c16;
    G.gbase = (int64_t)((cb & 15) / ES) + cell * V;
    G.V = V;
    G.nch = nch;
    G.L = (V + nch - 1) / nch;
    G.ppc = ppc;
    return G;
}

// The u pointer that puts the cell's u row where its c row is (the identity
// unless u is compacted, when the row-to-row shift keeps the 16-byte alignment).
__device__ __forceinline__ const void* cell_u(const void* uptr, const CellParams& cp, int V, bool bf16) {
    return uptr ? (const void*)((const char*)uptr + (cp.ucell - cp.cell) * (int64_t)V * (bf16 ? 2 : 4)) : uptr;
}

// The repetition penalty of one part's ids [v0, v1), in place, ahead of the
// part's stream (the autoregressive step; the same arithmetic as
// k_repetition_penalty: x / theta for x > 0, else x * theta, in binary32, stored
// in the logits' type).  Each thread loads up to four of the part's seen-mask
// words at once, then reads the logits of kPenaltyBatch set ids before writing
// any back; a barrier ends it, after which the workgroup's stream, and the merge
// launched later, read the penalised values.  The parts of a row own disjoint
// id ranges that cover it, so each seen id is penalised once, and the lines a
// part writes are those its own stream reads next: the step reads the row once
// instead of a separate pass reading a whole line for each seen id.
template <bool BF16, int NT>
__device__ void penalize_part(void* xrow, const uint32_t* seen, float theta, int v0, int v1) {
    if (v1 > v0 && theta > 0.0f && theta < __builtin_huge_valf()) {
        const int w0 = v0 >> 5, w1 = (v1 - 1) >> 5;  // the part's words, inclusive
        // word w of the mask, only the part's bits [v0 - 32 w, v1 - 32 w) kept
        auto word = [&](int w) {
            uint32_t x = w <= w1 ? __builtin_nontemporal_load(seen + w) : 0u;
            const int b0 = v0 - w * 32, b1 = v1 - w * 32;
            if (b0 > 0) x &= ~0u << b0;
            if (b1 < 32) x &= b1 > 0 ? (1u << b1) - 1u : 0u;
            return x;
        };
        for (int wb = w0 + (int)threadIdx.x; wb <= w1; wb += NT * 4) {
            // four words per thread (scalars, not an array, so that they stay in
            // registers)
            uint32_t m0 = word(wb), m1 = word(wb + NT), m2 = word(wb + 2 * NT), m3 = word(wb + 3 * NT);
            // the next set id of the thread's words, lowest word first
            auto next = [&](int& v) {
                const bool s0 = m0 != 0u, s1 = !s0 && m1 != 0u, s2 = !s0 && !s1 && m2 != 0u;
                const uint32_t cur = s0 ? m0 : s1 ? m1 : s2 ? m2 : m3;
                const int k = s0 ? 0 : s1 ? 1 : s2 ? 2 : 3;
                v = (wb + k * NT) * 32 + __builtin_ctz(cur | (cur == 0u ? 1u : 0u));
                const uint32_t rest = cur & (cur - 1u);
                m0 = s0 ? rest : m0;
                m1 = s1 ? rest : m1;
                m2 = s2 ? rest : m2;
                m3 = (s0 || s1 || s2) ? m3 : rest;
                return cur != 0u;
            };
            while ((m0 | m1 | m2 | m3) != 0u) {
                int at[kPenaltyBatch];
                bool ok[kPenaltyBatch];
#pragma unroll
                for (int b = 0; b < kPenaltyBatch; ++b) ok[b] = next(at[b]);
                if constexpr (BF16) {
                    uint16_t* x = static_cast<uint16_t*>(xrow);
                    uint16_t hv[kPenaltyBatch];
#pragma unroll
                    for (int b = 0; b < kPenaltyBatch; ++b) hv[b] = ok[b] ? x[at[b]] : (uint16_t)0;
#pragma unroll
                    for (int b = 0; b < kPenaltyBatch; ++b)
                        if (ok[b]) x[at[b]] = bf16_rne(penalized(__uint_as_float((uint32_t)hv[b] << 16), theta));
                } else {
                    float* x = static_cast<float*>(xrow);
                    float fv[kPenaltyBatch];
#pragma unroll
                    for (int b = 0; b < kPenaltyBatch; ++b) fv[b] = ok[b] ? x[at[b]] : 0.0f;
#pragma unroll
                    for (int b = 0; b < kPenaltyBatch; ++b)
                        if (ok[b]) x[at[b]] = penalized(fv[b], theta);
                }
            }
        }
    }
    __syncthreads();
}

// Kernel 1 body: stream part `part` of the row and write its partial record.
// With WIN the part also takes its share of the row's threshold window; it then
// streams with masked ids already mapped to -inf (FIX), since appended keys
// cannot be taken back by a second pass.
// With `seen` (the autoregressive step) the part first applies the repetition
// penalty to its own ids (penalize_part).
template <bool BF16, bool SAMPLE, bool WIN = false>
__device__ void part_body(const void* cptr, const void* uptr, int V, int nch, bool force_fallback,
                          const RowWork& w, const CellParams& cp, int64_t slot, int part,
                          const uint32_t* seen = nullptr, const float* penalty = nullptr, int W = 0) {
    __shared__ PartLDS<BF16, SAMPLE, WIN> sh;
    const int j = part / w.ppc;
    const int q = part - j * w.ppc;
    const bool use_u = SAMPLE && cp.s != 0.0f;
    const bool race = SAMPLE && cp.tau != 0.0f && !force_fallback;
    const RowGeom G = row_geom<BF16>(cptr, cell_u(uptr, cp, V, BF16), use_u, cp.cell, V, nch, w.ppc);
    const PartRange<BF16> pr(G, j, q);
    if (seen) {
        // the part's ids: its pieces, clipped to its chunk
        constexpr int EPP = Piece<BF16>::EPP;
        int v0 = 0, v1 = 0;
        if (pr.q1 >= pr.q0) {
            v0 = (int)max((int64_t)pr.lo, pr.q0 * EPP - G.gbase);
            v1 = (int)min((int64_t)pr.hi, (pr.q1 + 1) * EPP - G.gbase);
        }
        void* xrow = const_cast<char*>(static_cast<const char*>(cptr)) + cp.cell * (int64_t)V * (BF16 ? 2 : 4);
        penalize_part<BF16, kPartThreads<WIN>>(xrow, seen + cp.cell * (int64_t)W, penalty[cp.cell], v0, v1);
    }
    WinCtx wc{false, 0.0f, 0.0f, nullptr, nullptr};
    PartOut po;
    if constexpr (WIN) {
        const WinRec wr = w.win[slot];
        wc.on = wr.lo <= wr.hi;
        wc.lo = window_lo(wr.lo);
        wc.hi = window_hi(wr.hi);
        wc.keys = w.keys + slot * kWinKeysPerRow;
        wc.count = &w.win[slot].count;
        po = stream_part<BF16, SAMPLE, true, true>(G, pr, cp, use_u, race, sh, wc);
    } else {
        po = stream_part<BF16, SAMPLE, false, false>(G, pr, cp, use_u, race, sh, wc);
        if (po.nan) {
            // a masked id under guidance: stream the part again with h = -inf there
            __syncthreads();
            po = stream_part<BF16, SAMPLE, true, false>(G, pr, cp, use_u, race, sh, wc);
        }
    }
    if (threadIdx.x == 0) {
        PartRec* rec = w.part + slot * w.nparts + part;
        rec->m = po.m;
        rec->s = po.s;
        rec->id = po.id;
        rec->nq = race ? po.nq : -1;
        rec->bz = po.bz;
        rec->be = po.be;
        rec->bh = po.bh;
        rec->above = po.above;
    }
}

// The window kernel's body: the threshold window of a sampled row from a sample
// of the row (sample_window); greedy rows, and rows too short for a sample to
// pay, get none.  The row's key count starts at 0.
template <bool BF16>
__device__ void window_body(const void* cptr, const void* uptr, int V, int k, const RowWork& w, const CellParams& cp,
                            int64_t slot) {
    __shared__ WindowLDS<kWindowThreads> sh;
    uint32_t lo = 1u, hi = 0u;  // no window
    if (cp.tau != 0.0f) {
        const bool use_u = cp.s != 0.0f;
        const RowGeom G = row_geom<BF16>(cptr, cell_u(uptr, cp, V, BF16), use_u, cp.cell, V, 1, 1);
        uint32_t a, b;
        // five standard deviations: with thousands of rows per launch, one row
        // whose window misses costs its merge a pass over the row, and the launch
        // waits for its slowest row
        if (sample_window<BF16, kWindowSample, kWindowBatch>(G, cp.s, use_u, k, sh, 5.0f, kWinKeysPerRow, a, b)) {
            lo = a;
            hi = b;
        }
    }
    if (threadIdx.x == 0) w.win[slot] = WinRec{lo, hi, 0, 0};
}

// Kernel 2 body: merge the row's partial records ([DRAFT]: larger max wins,
// equal maxima keep the smaller id, sums add in probability space), then finish
// the greedy or sampled decision.
template <bool BF16, bool SAMPLE, int MT_, int KCAP, bool WIN = false>
__device__ __forceinline__ void merge_body(const void* cptr, const void* uptr, int V, int nch, int top_k, bool force_fallback,
                           const RowWork& w, const CellParams& cp, int64_t slot, int* tokens, float* logprobs,
                           float* lse_out, float* thresholds, float* triples, int64_t n_rows) {
    __shared__ MergeLDS<MT_, KCAP> sh;
    const bool use_u = SAMPLE && cp.s != 0.0f;
    const bool sampled = SAMPLE && cp.tau != 0.0f;
    const PartRec* recs = w.part + slot * w.nparts;
    float M = kNegInf, S = 0.0f;
    int id = 0x7FFFFFFF;
    // race winners of the parts
    float bz = kNegInf, bh = kNegInf;
    int be = 0x7FFFFFFF;
    int64_t queued = 0, above = 0;
    bool raced = sampled && !force_fallback;
    // records in chunk-major order, staged through LDS kMergeStage at a time
    float mj = kNegInf, sj = 0.0f;
    int idj = 0x7FFFFFFF;
    for (int t0 = 0; t0 < w.nparts; t0 += kMergeStage) {
        const int n = min(kMergeStage, w.nparts - t0);
        __syncthreads();
        if ((int)threadIdx.x < n) sh.u.rec[threadIdx.x] = recs[t0 + threadIdx.x];
        __syncthreads();
        for (int i = 0; i < n; ++i) {
            const int p = t0 + i;
            const PartRec r = sh.u.rec[i];
            if (WIN) above += r.above;
            if (sampled) {
                raced &= r.nq >= 0;
                queued += r.nq;
                if (r.bz > bz || (r.bz == bz && r.be < be)) {
                    bz = r.bz;
                    be = r.be;
                    bh = r.bh;
                }
            }
            if (r.m > kNegInf) {
                const float mn = __builtin_fmaxf(mj, r.m);
                sj = ((mj > kNegInf) ? sj * __builtin_amdgcn_exp2f((mj - mn) * kLog2e) : 0.0f) +
                     r.s * __builtin_amdgcn_exp2f((r.m - mn) * kLog2e);
                if (r.m > mj || (r.m == mj && r.id < idj)) idj = r.id;
                mj = mn;
            }
            if ((p + 1) % w.ppc != 0) continue;
            // chunk jj complete: its triple, then fold it into the row
            const int jj = p / w.ppc;
            if (triples && threadIdx.x == 0) {
                float* o = triples + ((int64_t)jj * n_rows + cp.cell) * 3;
                o[0] = mj;
                o[1] = (mj > kNegInf) ? mj + __builtin_logf(sj) : kNegInf;
                o[2] = __int_as_float(idj);
            }
            if (mj > kNegInf) {
                const float mn = __builtin_fmaxf(M, mj);
                S = ((M > kNegInf) ? S * __builtin_amdgcn_exp2f((M - mn) * kLog2e) : 0.0f) +
                    sj * __builtin_amdgcn_exp2f((mj - mn) * kLog2e);
                if (mj > M || (mj == M && idj < id)) id = idj;
                M = mn;
            }
            mj = kNegInf;
            sj = 0.0f;
            idj = 0x7FFFFFFF;
        }
    }
    const float lse = M + __builtin_logf(S);
    if (!sampled) {
        if (threadIdx.x == 0) {
            tokens[cp.cell] = id;
            if (lse_out) lse_out[cp.cell] = lse;
            logprobs[cp.cell] = M - lse;
            if (thresholds) thresholds[cp.cell] = __builtin_nanf("");
        }
        return;
    }

    // ---- Gumbel-max over the top-ratio set.  Every id that can win was queued by
    // its part; when at most top_k ids were queued they all lie inside the set.
    const int k = top_k;
    // Past that, the race's winner is still the argmax over all ids (an id it did
    // not score has a smaller key), so it is the answer as soon as it is kept.
    bool done = raced && queued <= (int64_t)k;
    float t = kNegInf;
    const RowGeom G = row_geom<BF16>(cptr, cell_u(uptr, cp, V, BF16), use_u, cp.cell, V, nch, w.ppc);
    bool have_t = false;
    if constexpr (WIN) {
        // the parts counted the keys above the row's window and appended those
        // inside it: when the top_k-th largest falls inside and every key was
        // kept, it is selected among them in LDS, with no pass over the row
        const WinRec wr = w.win[slot];
        const int n = wr.count;
        if (wr.lo <= wr.hi && n <= kWinKeysPerRow && above < (int64_t)k && (int64_t)k <= above + n) {
            t = key_value(window_kth(sh, w.keys + slot * kWinKeysPerRow, n, k - (int)above, wr.lo, wr.hi - wr.lo));
            have_t = true;
        }
    }
    if (!have_t && (!done || thresholds)) t = radix_select_row<BF16>(G, cp.s, use_u, k, sh);
    done = done || (raced && bz > kNegInf && bh >= t);
    if (!done) {
        // exact pass over the kept ids that can beat the argmax
        const float cthr = __builtin_fmaxf(t, max_bound(M, cp.inv_tau, cp.tau));
        bz = kNegInf;
        be = 0x7FFFFFFF;
        bh = kNegInf;
        for_each_id<BF16, MT_>(G, cp.s, use_u, [&](int v, float hv) {
            if (!(hv >= cthr)) return;
            const float z = __builtin_fmaf(hv, cp.inv_tau, gumbel_from_word(noise_word(cp.nk, (uint32_t)v)));
            if (z > bz || (z == bz && v < be)) {
                bz = z;
                be = v;
                bh = hv;
            }
        });
        block_argmax3(bz, be, bh, sh.r);
    }
    if (threadIdx.x == 0) {
        tokens[cp.cell] = be;
        logprobs[cp.cell] = bh - lse;
        if (thresholds) thresholds[cp.cell] = t + 0.0f;
    }
}

__device__ __forceinline__ CellParams sample_cell(const SampleArgs& a, const ReqTable& rq, int64_t slot) {
    const int64_t lin = a.w.cell_base + slot;  // launch-relative cell
    const int row = (int)(lin / rq.npos);
    const int pl = (int)(lin - (int64_t)row * rq.npos);
    const ReqParams q = req_params(rq, find_request(rq, pl));
    CellParams cp;
    cp.cell = (int64_t)row * rq.P + rq.pos0 + pl;
    cp.ucell = (int64_t)row * rq.Pu + q.uoff + (pl - q.start);
    cp.s = q.scale;
    cp.tau = q.tau;
    cp.inv_tau = q.inv_tau;
    cp.nk.k0 = a.k0;
    cp.nk.k1 = a.k1;
    cp.nk.t = (uint32_t)(pl - q.start);
    cp.nk.row_iter = ((uint32_t)row & 0xFFFFu) | q.row_iter_hi;
    cp.nk.rid = q.rid;
    return cp;
}

// The cell of workspace slot `slot` under device-resident parameters; false
// when it is padding (the whole workgroup leaves together).
__device__ __forceinline__ bool sample_cell_dev(const SampleArgs& a, const DevReq& d, int64_t slot, CellParams& cp) {
    const int64_t lin = a.w.cell_base + slot;  // row * d.P + position
    const int row = (int)(lin / d.P);
    const int pl = (int)(lin - (int64_t)row * d.P);
    DevCell dc;
    if (!dev_cell(d, a.u != nullptr, pl, dc)) return false;
    cp.cell = lin;
    cp.ucell = lin;
    cp.s = dc.s;
    cp.tau = dc.tau;
    cp.inv_tau = dc.inv_tau;
    cp.nk.k0 = a.k0;
    cp.nk.k1 = a.k1;
    cp.nk.t = dc.t;
    cp.nk.row_iter = ((uint32_t)row & 0xFFFFu) | dc.iter_hi;
    cp.nk.rid = dc.rid;
    return true;
}

__device__ __forceinline__ CellParams greedy_cell(const GreedyArgs& a, int64_t slot) {
    CellParams cp;
    cp.cell = a.w.cell_base + slot;
    cp.ucell = cp.cell;
    cp.s = 0.0f;
    cp.tau = 0.0f;
    cp.inv_tau = 0.0f;
    cp.nk = NoiseKey{0, 0, 0, 0, 0};
    return cp;
}

// Block b is part (b % nparts) of row slot (b / nparts), so neighbouring
// workgroups stream neighbouring memory.  The greedy parts kernel keeps to 64
// VGPRs (four workgroups per CU); the sampled one may take 80 (three), which the
// race's noise code needs without spilling.
// The parts kernels keep to 80 VGPRs (six waves per SIMD, three workgroups per
// compute unit); with the threshold window they may take 128 (two workgroups),
// which its per-id tests need without spilling.
template <bool BF16, bool WIN>
__global__ __launch_bounds__(kPartThreads<WIN>) __attribute__((amdgpu_waves_per_eu(WIN ? 4 : 6, 8))) void k_sample_parts(SampleArgs a, ReqTable rq) {
    const int64_t slot = blockIdx.x / a.w.nparts;
    const int part = (int)(blockIdx.x - slot * a.w.nparts);
    part_body<BF16, true, WIN>(a.c, a.u, a.V, a.vocab_chunks, a.force_fallback != 0, a.w, sample_cell(a, rq, slot),
                               slot, part);
}
// With the threshold window the bf16 merge is held to 64 VGPRs, so that eight of
// its 256-thread blocks share a compute unit (four spilled registers; the f32 one
// would spill many more).
template <bool BF16, int MT_, int KCAP, bool WIN>
__global__ __launch_bounds__(MT_) __attribute__((amdgpu_waves_per_eu(WIN && BF16 ? 8 : 1, 8))) void k_sample_merge(SampleArgs a, ReqTable rq) {
    const int64_t slot = blockIdx.x;
    merge_body<BF16, true, MT_, KCAP, WIN>(a.c, a.u, a.V, a.vocab_chunks, a.top_k, a.force_fallback != 0, a.w,
                                           sample_cell(a, rq, slot), slot, a.tokens, a.logprobs, nullptr,
                                           a.thresholds, nullptr, 0);
}
template <bool BF16>
__global__ __launch_bounds__(kWindowThreads) void k_sample_window(SampleArgs a, ReqTable rq) {
    const int64_t slot = blockIdx.x;
    window_body<BF16>(a.c, a.u, a.V, a.top_k, a.w, sample_cell(a, rq, slot), slot);
}
// The same kernels with the per-request parameters in device memory.
template <bool BF16, bool WIN>
__global__ __launch_bounds__(kPartThreads<WIN>) __attribute__((amdgpu_waves_per_eu(WIN ? 4 : 6, 8))) void k_sample_parts_dev(SampleArgs a, DevReq d) {
    const int64_t slot = blockIdx.x / a.w.nparts;
    const int part = (int)(blockIdx.x - slot * a.w.nparts);
    CellParams cp;
    if (!sample_cell_dev(a, d, slot, cp)) return;
    part_body<BF16, true, WIN>(a.c, a.u, a.V, a.vocab_chunks, a.force_fallback != 0, a.w, cp, slot, part, a.seen,
                               a.penalty, a.W);
}
template <bool BF16, int MT_, int KCAP, bool WIN>
__global__ __launch_bounds__(MT_) __attribute__((amdgpu_waves_per_eu(WIN && BF16 ? 8 : 1, 8))) void k_sample_merge_dev(SampleArgs a, DevReq d) {
    const int64_t slot = blockIdx.x;
    CellParams cp;
    if (!sample_cell_dev(a, d, slot, cp)) return;
    merge_body<BF16, true, MT_, KCAP, WIN>(a.c, a.u, a.V, a.vocab_chunks, a.top_k, a.force_fallback != 0, a.w, cp,
                                           slot, a.tokens, a.logprobs, nullptr, a.thresholds, nullptr, 0);
}
template <bool BF16>
__global__ __launch_bounds__(kWindowThreads) void k_sample_window_dev(SampleArgs a, DevReq d) {
    const int64_t slot = blockIdx.x;
    CellParams cp;
    if (!sample_cell_dev(a, d, slot, cp)) return;  // padding: its parts and merge leave too
    window_body<BF16>(a.c, a.u, a.V, a.top_k, a.w, cp, slot);
}
template <bool BF16>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8, 8))) void k_greedy_parts(GreedyArgs a) {
    const int64_t slot = blockIdx.x / a.w.nparts;
    const int part = (int)(blockIdx.x - slot * a.w.nparts);
    part_body<BF16, false>(a.x, nullptr, a.V, a.vocab_chunks, false, a.w, greedy_cell(a, slot), slot, part);
}
// Greedy rows need no pass over the row after the parts, so one wave merges a
// row: lane i loads record i of each 64, and the fold walks them in order with
// the record broadcast from its lane.
__global__ __launch_bounds__(kWave) void k_greedy_merge(GreedyArgs a) {
    const int64_t cell = a.w.cell_base + blockIdx.x;
    const PartRec* recs = a.w.part + (int64_t)blockIdx.x * a.w.nparts;
    const int lane = lane_id();
    float M = kNegInf, S = 0.0f, mj = kNegInf, sj = 0.0f;
    int id = 0x7FFFFFFF, idj = 0x7FFFFFFF;
    for (int t0 = 0; t0 < a.w.nparts; t0 += kWave) {
        const int n = min(kWave, a.w.nparts - t0);
        float rm = kNegInf, rs = 0.0f;
        int rid = 0x7FFFFFFF;
        if (lane < n) {
            const PartRec r = recs[t0 + lane];
            rm = r.m;
            rs = r.s;
            rid = r.id;
        }
        for (int i = 0; i < n; ++i) {
            const int p = t0 + i;
            const float m = readlane_f(rm, i);
            const float sm = readlane_f(rs, i);
            const int im = __builtin_amdgcn_readlane(rid, i);
            if (m > kNegInf) {
                const float mn = __builtin_fmaxf(mj, m);
                sj = ((mj > kNegInf) ? sj * __builtin_amdgcn_exp2f((mj - mn) * kLog2e) : 0.0f) +
                     sm * __builtin_amdgcn_exp2f((m - mn) * kLog2e);
                if (m > mj || (m == mj && im < idj)) idj = im;
                mj = mn;
            }
            if ((p + 1) % a.w.ppc != 0) continue;
            // chunk jj complete: its triple, then fold it into the row
            const int jj = p / a.w.ppc;
            if (a.triples && lane == 0) {
                float* o = a.triples + ((int64_t)jj * a.n_rows + cell) * 3;
                o[0] = mj;
                o[1] = (mj > kNegInf) ? mj + __builtin_logf(sj) : kNegInf;
                o[2] = __int_as_float(idj);
            }
            if (mj > kNegInf) {
                const float mn = __builtin_fmaxf(M, mj);
                S = ((M > kNegInf) ? S * __builtin_amdgcn_exp2f((M - mn) * kLog2e) : 0.0f) +
                    sj * __builtin_amdgcn_exp2f((mj - mn) * kLog2e);
                if (mj > M || (mj == M && idj < id)) id = idj;
                M = mn;
            }
            mj = kNegInf;
            sj = 0.0f;
            idj = 0x7FFFFFFF;
        }
    }
    if (lane == 0) {
        const float lse = M + __builtin_logf(S);
        a.token[cell] = id;
        a.lse[cell] = lse;
        a.logprob[cell] = M - lse;
    }
}

// One workgroup per row for the draft path when the rows alone fill the GPU:
// no second kernel and no workspace.  Each thread streams its pieces of one
// vocabulary chunk after another, four 16-byte pieces in flight per group; at
// the end of a chunk each wave reduces its lanes' (max, exp-sum, smallest
// argmax) and writes one record to LDS, with no barrier, so the loads of the
// next chunk follow at once.  After the row, the first wave folds each chunk's
// wave records into its triple ([DRAFT] "Design and invariants"), and the
// triples into the row.  Chunk boundaries fall on piece
// boundaries (the host checks V and ceil(V / chunks) are multiples of the ids
// per piece and that rows start 16-byte aligned).
template <bool BF16>
__global__ __launch_bounds__(kGreedyRowThreads) void k_greedy_rows(GreedyArgs a) {
    constexpr int EPP = Piece<BF16>::EPP;
    constexpr int NTR = kGreedyRowThreads;
    constexpr int NW = NTR / kWave;
    constexpr int UR = kGreedyRowU;
    __shared__ float s_m[kGreedyRowMaxChunks][NW];
    __shared__ float s_s[kGreedyRowMaxChunks][NW];
    __shared__ int s_id[kGreedyRowMaxChunks][NW];
    const int64_t row = blockIdx.x;
    const int V = a.V;
    const int nch = a.vocab_chunks;
    const int L = (V + nch - 1) / nch;
    const gptr<u32x4> x16 = as_global<u32x4>((const char*)a.x + row * (int64_t)V * (BF16 ? 2 : 4));
    const int t = (int)threadIdx.x;
    const int lane = lane_id();
    const int wv = t >> 6;
    const uint32_t ninf = BF16 ? 0xFF80FF80u : 0xFF800000u;
    for (int j = 0; j < nch; ++j) {
        const int lo = min(V, j * L);
        const int hi = min(V, lo + L);
        const gptr<u32x4> xc = x16 + lo / EPP;
        const int nq = (hi - lo) / EPP;
        float m = kNegInf, acc = 0.0f;
        // the first piece holding the thread's maximum: its index and raw
        // dwords, searched for the first id only once the chunk is done (the
        // maximum rises in most groups of random rows, in some lane of every wave)
        int mq = 0;
        u32x4 mraw = u32x4{ninf, ninf, ninf, ninf};
        // Whole groups load without any test, so all their loads are in flight
        // together, and the next whole group's loads are issued before this
        // group is reduced (with one workgroup per compute unit there are two
        // waves per SIMD, too few to hide the reduction behind other waves'
        // loads); the chunk's last, partial group clamps its indices and selects
        // -inf past the end (a load under a branch would make the compiler wait
        // for the loads before it).
        auto load_full = [&](int base, u32x4(&raw)[UR]) {
#pragma unroll
            for (int u = 0; u < UR; ++u) raw[u] = stream_load(xc + base + u * NTR + t);
        };
        auto load_tail = [&](int base, u32x4(&raw)[UR]) {
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int jp = base + u * NTR + t;
                raw[u] = stream_load(xc + min(jp, nq - 1));
                if (jp >= nq) raw[u] = u32x4{ninf, ninf, ninf, ninf};
            }
        };
        auto group = [&](int base, const u32x4(&raw)[UR]) {
            Piece<BF16> P[UR];
            float pm[UR];
            float gm = kNegInf;
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                decode_piece<BF16>(raw[u], raw[u], 0.0f, false, P[u]);
                pm[u] = P[u].h[0];
#pragma unroll
                for (int e = 1; e < EPP; ++e) pm[u] = __builtin_fmaxf(pm[u], P[u].h[e]);
                gm = __builtin_fmaxf(gm, pm[u]);
            }
            if (gm > m) {
                // first piece holding the new maximum (ids grow with u)
                int pu = UR - 1;
                u32x4 r = raw[UR - 1];
#pragma unroll
                for (int u = UR - 2; u >= 0; --u) {
                    if (pm[u] == gm) {
                        pu = u;
                        r = raw[u];
                    }
                }
                mq = base + pu * NTR + t;
                mraw = r;
                acc *= __builtin_amdgcn_exp2f((m - gm) * kLog2e);
                m = gm;
            }
            const float mL = (m > kNegInf) ? m * kLog2e : 0.0f;
#pragma unroll
            for (int u = 0; u < UR; ++u)
#pragma unroll
                for (int e = 0; e < EPP; ++e) acc += __builtin_amdgcn_exp2f(__builtin_fmaf(P[u].h[e], kLog2e, -mL));
        };
        constexpr int GP = NTR * UR;  // pieces per group
        const int nfull = nq / GP;
        int base = 0;
        if (nfull > 0) {
            u32x4 cur[UR], nxt[UR];
            load_full(0, cur);
            for (int g = 1; g < nfull; ++g) {
                load_full(g * GP, nxt);
                group(base, cur);
                base += GP;
#pragma unroll
                for (int u = 0; u < UR; ++u) cur[u] = nxt[u];
            }
            group(base, cur);
            base += GP;
        }
        if (base < nq) {
            u32x4 raw[UR];
            load_tail(base, raw);
            group(base, raw);
        }
        // undo the rounding of m * log2(e), then the wave's share of the chunk
        if (m > kNegInf) acc *= __builtin_amdgcn_exp2f(-__builtin_fmaf(m, kLog2e, -(m * kLog2e)));
        const float wm = wave_max(m);
        const float ws = wave_sum((m > kNegInf) ? acc * __builtin_amdgcn_exp2f((m - wm) * kLog2e) : 0.0f);
        // the first id of the maximum's piece, in the lanes that hold the wave's maximum
        int mid = 0x7FFFFFFF;
        if (wm > kNegInf && m == wm) {
            Piece<BF16> P;
            decode_piece<BF16>(mraw, mraw, 0.0f, false, P);
            int e = EPP - 1;
#pragma unroll
            for (int i = EPP - 1; i >= 0; --i)
                if (P.h[i] == m) e = i;
            mid = lo + mq * EPP + e;
        }
        const int wid = wave_min_i(mid);
        if (lane == 0) {
            s_m[j][wv] = wm;
            s_s[j][wv] = ws;
            s_id[j][wv] = wid;
        }
    }
    __syncthreads();
    if (wv != 0) return;
    // The first wave folds the records: in groups of NW lanes, lane l takes wave
    // (l % NW)'s record of chunk g + l / NW, each group reduces one chunk to its
    // triple, and the triples fold into the row (larger max wins, equal maxima
    // keep the smaller id, sums add in probability space).
    constexpr int CPP = kWave / NW;  // chunks per pass of the wave
    float M = kNegInf, S = 0.0f;
    int id = 0x7FFFFFFF;
    for (int g = 0; g < nch; g += CPP) {
        const int c = g + lane / NW;
        const int w = lane % NW;
        float rm = kNegInf, rs = 0.0f;
        int ri = 0x7FFFFFFF;
        if (c < nch) {
            rm = s_m[c][w];
            rs = s_s[c][w];
            ri = s_id[c][w];
        }
        const float mj = grp_max<NW>(rm);
        const float sj = grp_sum<NW>((rm > kNegInf) ? rs * __builtin_amdgcn_exp2f((rm - mj) * kLog2e) : 0.0f);
        const int idj = grp_min_i<NW>((mj > kNegInf && rm == mj) ? ri : 0x7FFFFFFF);
        if (a.triples && w == 0 && c < nch) {
            float* o = a.triples + ((int64_t)c * a.n_rows + row) * 3;
            o[0] = mj;
            o[1] = (mj > kNegInf) ? mj + __builtin_logf(sj) : kNegInf;
            o[2] = __int_as_float(idj);
        }
        // fold this pass's chunk triples (the first lane of each group) into the row
        const bool lead = w == 0;
        const float gm = wave_max(lead ? mj : kNegInf);
        const float mn = __builtin_fmaxf(M, gm);
        const float gs = wave_sum((lead && mj > kNegInf) ? sj * __builtin_amdgcn_exp2f((mj - mn) * kLog2e) : 0.0f);
        const int gi = wave_min_i((lead && gm > kNegInf && mj == gm) ? idj : 0x7FFFFFFF);
        if (mn > kNegInf) {
            S = ((M > kNegInf) ? S * __builtin_amdgcn_exp2f((M - mn) * kLog2e) : 0.0f) + gs;
            if (gm > M || (gm == M && gi < id)) id = gi;
            M = mn;
        }
    }
    if (lane == 0) {
        const float lse = M + __builtin_logf(S);
        a.token[row] = id;
        a.lse[row] = lse;
        a.logprob[row] = M - lse;
    }
}

}  // namespace

int row_parts_per_chunk(bool bf16, int V, int chunks, int64_t cells, bool window) {
    const int epp = bf16 ? 8 : 4;
    const int64_t L = ((int64_t)V + chunks - 1) / chunks;
    const int64_t pieces = L / epp + 2;
    // enough waves to cover the GPU several times over (12288: two rounds of 6
    // waves per SIMD for the plain parts kernel), parts of >= 1024 pieces; for a
    // 256-row autoregressive step that is six parts per row, 5% faster than four
    const int64_t target = 12288 / (window ? kPartWaves<true> : kPartWaves<false>);
    int64_t p = (target + cells * chunks - 1) / (cells * chunks);
    const int64_t p_cap = pieces / 1024 > 1 ? pieces / 1024 : 1;
    if (p > p_cap) p = p_cap;
    if (p * chunks > kWorkParts) p = kWorkParts / chunks > 0 ? kWorkParts / chunks : 1;
    return (int)(p < 1 ? 1 : p);
}

namespace {

// The kernels of one streaming launch: with the threshold output and a window
// workspace, the window kernel first and the parts and merge kernels with the
// window; otherwise parts and merge, the merge in its exact shape whenever every
// row selects its threshold.
template <bool BF16, typename Src, typename KW, typename KP, typename KPW, typename KM, typename KME, typename KMEW>
hipError_t launch_row(const SampleArgs& a, const Src& src, hipStream_t st, KW kwin, KP kparts, KPW kparts_win,
                      KM kmerge, KME kmerge_exact, KMEW kmerge_exact_win) {
    const int64_t parts = (int64_t)a.w.ncells * a.w.nparts;
    if (parts == 0) return hipSuccess;
    const dim3 mg((unsigned)a.w.ncells);
    const bool exact = a.thresholds != nullptr || a.force_fallback != 0;  // every row selects its threshold
    const bool win = a.thresholds != nullptr && a.force_fallback == 0 && a.w.win != nullptr && a.w.keys != nullptr;
    if (win) {
        hipLaunchKernelGGL(kwin, mg, dim3(kWindowThreads), 0, st, a, src);
        hipLaunchKernelGGL(kparts_win, dim3((unsigned)parts), dim3(kPartThreads<true>), 0, st, a, src);
        hipLaunchKernelGGL(kmerge_exact_win, mg, dim3(kMergeThreadsWin), 0, st, a, src);
    } else {
        hipLaunchKernelGGL(kparts, dim3((unsigned)parts), dim3(NT), 0, st, a, src);
        if (exact)
            hipLaunchKernelGGL(kmerge_exact, mg, dim3(kMergeThreadsExact), 0, st, a, src);
        else
            hipLaunchKernelGGL(kmerge, mg, dim3(kMergeThreadsFast), 0, st, a, src);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sample_row(bool bf16, const SampleArgs& a, const ReqTable& rq, hipStream_t st) {
    if (bf16)
        return launch_row<true>(a, rq, st, k_sample_window<true>, k_sample_parts<true, false>,
                                k_sample_parts<true, true>, k_sample_merge<true, kMergeThreadsFast, kKeyCapFast, false>,
                                k_sample_merge<true, kMergeThreadsExact, kKeyCapExact, false>,
                                k_sample_merge<true, kMergeThreadsWin, kKeyCapWin, true>);
    return launch_row<false>(a, rq, st, k_sample_window<false>, k_sample_parts<false, false>,
                             k_sample_parts<false, true>, k_sample_merge<false, kMergeThreadsFast, kKeyCapFast, false>,
                             k_sample_merge<false, kMergeThreadsExact, kKeyCapExact, false>,
                             k_sample_merge<false, kMergeThreadsWin, kKeyCapWin, true>);
}

hipError_t launch_sample_row_dev(bool bf16, const SampleArgs& a, const DevReq& d, hipStream_t st) {
    if (d.n < 1 || (d.n > kWave && !d.one_per_request) || d.P < 1) return hipErrorInvalidValue;
    if (bf16)
        return launch_row<true>(a, d, st, k_sample_window_dev<true>, k_sample_parts_dev<true, false>,
                                k_sample_parts_dev<true, true>,
                                k_sample_merge_dev<true, kMergeThreadsFast, kKeyCapFast, false>,
                                k_sample_merge_dev<true, kMergeThreadsExact, kKeyCapExact, false>,
                                k_sample_merge_dev<true, kMergeThreadsWin, kKeyCapWin, true>);
    return launch_row<false>(a, d, st, k_sample_window_dev<false>, k_sample_parts_dev<false, false>,
                             k_sample_parts_dev<false, true>,
                             k_sample_merge_dev<false, kMergeThreadsFast, kKeyCapFast, false>,
                             k_sample_merge_dev<false, kMergeThreadsExact, kKeyCapExact, false>,
                             k_sample_merge_dev<false, kMergeThreadsWin, kKeyCapWin, true>);
}

bool greedy_rows_fits(bool bf16, int V, int chunks, const void* x) {
    const int epp = bf16 ? 8 : 4;
    if (V < 1 || chunks < 1 || chunks > kGreedyRowMaxChunks) return false;
    const int L = (V + chunks - 1) / chunks;
    return V % epp == 0 && L % epp == 0 && ((uintptr_t)x & 15u) == 0;
}

hipError_t launch_greedy_rows(bool bf16, const GreedyArgs& a, hipStream_t st) {
    if (a.n_rows < 1 || a.n_rows > INT32_MAX || !greedy_rows_fits(bf16, a.V, a.vocab_chunks, a.x))
        return hipErrorInvalidValue;
    if (bf16)
        hipLaunchKernelGGL(k_greedy_rows<true>, dim3((unsigned)a.n_rows), dim3(kGreedyRowThreads), 0, st, a);
    else
        hipLaunchKernelGGL(k_greedy_rows<false>, dim3((unsigned)a.n_rows), dim3(kGreedyRowThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_greedy_lse(bool bf16, const GreedyArgs& a, hipStream_t st) {
    const int64_t parts = (int64_t)a.w.ncells * a.w.nparts;
    if (parts == 0) return hipSuccess;
    if (bf16) {
        hipLaunchKernelGGL(k_greedy_parts<true>, dim3((unsigned)parts), dim3(NT), 0, st, a);
    } else {
        hipLaunchKernelGGL(k_greedy_parts<false>, dim3((unsigned)parts), dim3(NT), 0, st, a);
    }
    hipLaunchKernelGGL(k_greedy_merge, dim3((unsigned)a.w.ncells), dim3(kWave), 0, st, a);
    return hipGetLastError();
}

}  // namespace ds
