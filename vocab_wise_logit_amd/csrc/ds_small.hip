// ds_small.hip -- one wavefront per cell for vocabularies that fit in registers.
//
// Each 64-lane wave owns one cell (row, position) of the packed [C, P, V] logits
// and holds the whole guided row h[0..V) in VGPRs (dword slots of two bf16 or one
// f32 per lane).  The row's loads (c, and u for guided cells) go out before any
// of their data is used; everything after them is register / LDS work:
//   1. h = CFG combine ([ISSUE] comment on the API shape; [PR] "What does this PR
//      do?": guidance 0 never reads u), row max, log-sum-exp;
//   2. greedy cells (temperature 0): token = smallest-id argmax, logprob =
//      max - LSE;
//   3. sampled cells, Gumbel-max ([ISSUE]) over the top-ratio set: an id whose
//      h/tau + max-noise is below the argmax's h/tau + min-noise never wins, so
//      only ids with h >= M - tau * (Gmax - Gmin) are candidates.  They are
//      compacted into a per-wave LDS list (per-lane counts and a wave prefix sum)
//      and raced, 64 Philox draws at a time.  If at most top_k ids are
//      candidates they all lie inside the top-ratio set; otherwise the winner
//      stands when fewer than top_k ids have a larger h.
//   4. rows with many candidates (flat rows) first narrow them: a per-wave LDS
//      histogram over [M - tau * (Gmax - Gmin), M] yields the exact float edge
//      of a top set holding the top-ratio set with a few ids to spare, which is
//      listed and raced as in 3.  The exact top_k-th largest h ([ISSUE]
//      top-ratio filter) is located on that list only when the race's winner is
//      not kept or the caller asks for the threshold.
// Ties: smallest id for the greedy argmax and for exact Gumbel ties ([DRAFT]
// "Design and invariants" rule, applied to every decision).
#include <stdint.h>

#include "ds_device.h"
#include "ds_kernels.h"

#include <type_traits>

namespace ds {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kListCap = 512;
constexpr int kListRegs = kListCap / kWave;
// Sampled cells with at most this many ids that can win race them all; beyond
// it, the top-ratio set is first narrowed with a histogram.
constexpr int kRaceAll = 256;
// Per-wave histogram of the narrowing step: kHistLow spill bins (one per lane,
// for ids below the range) and then kHistBins bins over the range.
constexpr int kHistLow = kWave;
constexpr int kHistBins = 256;
constexpr float kHistTop = (float)(kHistLow + kHistBins) - 0.5f;

struct Entry {
    float h;
    int e;
};

// Register-slot counts that get an instantiation, in increasing order; a row is
// launched with the smallest that holds it.
constexpr int kSlotSizes[] = {2, 4, 6, 9, 12, 16, 24, 32};
// Slots of an NS-slot instantiation that every row it is launched for fills
// completely: those of the next smaller instantiation (which the row did not fit,
// so its dwords reach past them: for bf16, (V + 2) / 2 > 64 * prev implies
// V >= 128 * prev, so even a row starting on a dword boundary has
// (V + 1) / 2 >= 64 * prev dwords; for f32 V > 64 * prev).
template <bool BF16, int NS>
constexpr int kFullSlots = [] {
    int prev = 0;
    for (int n : kSlotSizes)
        if (n < NS) prev = n;
    return prev;
}();

template <bool BF16, int NS>
struct Row {
    static constexpr int NE = BF16 ? 2 * NS : NS;
    float h[NE];
    int ebase;  // id of register element 0 in this lane (bf16: 2 * lane - parity)

    // Row-relative id of register element i of this lane.
    __device__ __forceinline__ int id_of(int i) const {
        if (BF16) return ebase + 2 * kWave * (i >> 1) + (i & 1);
        return ebase + kWave * i;
    }

    // Number of ids whose h is >= x (x > -inf), counted with ballots.
    __device__ __forceinline__ int count_ge(float x) const {
        int n = 0;
#pragma unroll
        for (int i = 0; i < NE; ++i) n += popc(__builtin_amdgcn_ballot_w64(h[i] >= x));
        return n;
    }

    // Write the ids whose h is >= x to `list` as (h, id) in slot order (slot i's
    // ids after those of slot i - 1, in lane order within a slot): one ballot per
    // slot gives its count, and mbcnt on it, started at the running count, each
    // id's place.  A slot that would take the list past `cap` (<= kListCap)
    // entries is not written, so the list holds every such id exactly when the
    // returned count is <= cap.
    __device__ __forceinline__ int write_ge(float x, Entry* list, int cap) const {
        int base = 0;  // wave-uniform
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const bool p = h[i] >= x;
            const uint64_t m = __builtin_amdgcn_ballot_w64(p);
            const int nm = popc(m);
            if (base + nm <= cap && p) {
                const uint32_t at = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)base));
                list[at] = Entry{h[i], id_of(i)};
            }
            base += nm;
        }
        __builtin_amdgcn_wave_barrier();
        return base;
    }

    // Count the ids whose h is >= x and, if there are at most `cap` (<= kListCap)
    // of them, write them to `list` (write_ge).  Returns the count.
    __device__ __forceinline__ int count_compact(float x, Entry* list, int cap = kListCap) const {
        const int total = count_ge(x);
        if (total <= cap) write_ge(x, list, cap);
        __builtin_amdgcn_wave_barrier();
        return total;
    }

    // Add every id to a per-wave LDS histogram: bin b = trunc(clamp(fma(h,
    // scale, off), low, kHistTop)).  The caller places the range of interest on
    // bins [kHistLow, kHistLow + kHistBins); `low` = kHistLow - 1 - lane sends
    // the ids below it to a bin of the lane's own, so they do not pile onto one
    // address.
    __device__ __forceinline__ void histogram(uint32_t* hist, float scale, float off, float low) const {
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const float x = __builtin_amdgcn_fmed3f(__builtin_fmaf(h[i], scale, off), low, kHistTop);
            __hip_atomic_fetch_add(&hist[(uint32_t)x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        }
    }
};

// Exact k-th largest over all valid ids, by key-space bisection on the full
// registers (bounded by 32 rounds).  Used only when the pivot search fails.
template <bool BF16, int NS>
__device__ float kth_by_bisection(const Row<BF16, NS>& R, int k, int V, float M) {
    if (R.count_ge(M) >= k) return M;
    uint32_t lo = order_key(kNegInf);  // count(lo) = V >= k
    uint32_t hi = order_key(M);        // count(hi) < k
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

// Smallest finite h of the row (rare path).  The empty volatile asm pins the
// computation inside the branch that needs it; otherwise the compiler hoists this
// loop-invariant reduction into the common path.
template <bool BF16, int NS>
__device__ __forceinline__ float min_finite(const Row<BF16, NS>& R) {
    float mn = __builtin_huge_valf();
    asm volatile("" : "+v"(mn));
#pragma unroll
    for (int i = 0; i < Row<BF16, NS>::NE; ++i) mn = R.h[i] > kNegInf ? __builtin_fminf(mn, R.h[i]) : mn;
    return wave_min(mn);
}

// A top set of the row that holds the top-ratio set: the smallest float c such
// that at least k ids have h >= c, up to the resolution of a histogram of the ids
// at or above `lo` (lo < M).  kHistBins bins span [lo, M]; the bin holding the
// k-th largest h is found from suffix counts, and c is the exact float at which
// the binning predicate fma(h, scale, off) >= that bin's index turns true (it is
// monotone in h), so count(h >= c) is that bin's suffix count, returned in n.
// Returns false when the histogram cannot resolve the range (no finite scale)
// or fewer than k ids reach it.  The histogram lives in the wave's list memory,
// which the caller overwrites only after this returns.
template <bool BF16, int NS>
__device__ bool top_set_by_histogram(const Row<BF16, NS>& R, Entry* list, int k, float lo, float M, int lane,
                                     float& c_out, int& n_out) {
    const float scale = (float)kHistBins * __builtin_amdgcn_rcpf(M - lo);
    const float off = __builtin_fmaf(-lo, scale, (float)kHistLow);
    if (!(scale > 0.0f && scale < 1e30f) || !(__builtin_fabsf(off) < 1e30f)) return false;
    uint32_t* hist = reinterpret_cast<uint32_t*>(list);
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    // clear the range's bins (the spill bins below it are never read)
    reinterpret_cast<u32x4_t*>(hist + kHistLow)[lane] = u32x4_t{0u, 0u, 0u, 0u};
    asm volatile("" ::: "memory");
    R.histogram(hist, scale, off, (float)(kHistLow - 1 - lane));
    asm volatile("" ::: "memory");
    // lane l holds bins 4l .. 4l+3 of the range; suffix counts from the top
    const u32x4_t b = reinterpret_cast<const u32x4_t*>(hist + kHistLow)[lane];
    asm volatile("" ::: "memory");
    const int T = (int)(b.x + b.y + b.z + b.w);
    const int incl = wave_incl_scan(T);
    const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
    if (total < k) return false;
    const int above = total - incl;  // ids in the bins of higher lanes
    // the lane whose bins hold the k-th largest, then the bin inside it
    const uint64_t m = ballot(above < k && above + T >= k);
    const int ls = (int)__builtin_ctzll(m);
    int jl = 0, nl = above + T;
    if (above + (int)b.w >= k) {
        jl = 3;
        nl = above + (int)b.w;
    } else if (above + (int)(b.w + b.z) >= k) {
        jl = 2;
        nl = above + (int)(b.w + b.z);
    } else if (above + (int)(b.w + b.z + b.y) >= k) {
        jl = 1;
        nl = above + (int)(b.w + b.z + b.y);
    }
    const int j = 4 * ls + __builtin_amdgcn_readlane(jl, ls);
    n_out = __builtin_amdgcn_readlane(nl, ls);
    // smallest float c with fma(c, scale, off) >= kHistLow + j
    const float J = (float)(kHistLow + j);
    auto in_set = [&](uint32_t key) { return __builtin_fmaf(key_value(key), scale, off) >= J; };
    uint32_t kc = order_key((J - off) * __builtin_amdgcn_rcpf(scale) + 0.0f);
    int steps = 0;
    while (in_set(kc - 1u) && steps < 64) {
        --kc;
        ++steps;
    }
    while (!in_set(kc) && steps < 64) {
        ++kc;
        ++steps;
    }
    if (steps >= 64 || !in_set(kc) || in_set(kc - 1u)) return false;
    c_out = key_value(kc);
    return true;
}

// Exact k-th largest of a wave's LDS list, given that the list holds every id
// whose h is >= lo and n >= k of them (lo < M).  Interpolation on the count
// narrows [lo, hi); distinct values are then taken from the top until the count
// reaches k.
__device__ __forceinline__ float list_kth(const Entry* list, int n, int k, float lo, float M,
                                                    int lane) {
    float xl[kListRegs];
    const int nl = (n + kWave - 1) / kWave;
#pragma unroll
    for (int i = 0; i < kListRegs; ++i) {
        const int o = i * kWave + lane;
        xl[i] = kNegInf;
        if (i < nl && o < n) xl[i] = list[o].h;
    }
    auto cnt = [&](float x) {
        int c = 0;
#pragma unroll
        for (int i = 0; i < kListRegs; ++i)
            if (i < nl) c += popc(ballot(xl[i] >= x));
        return c;
    };
    float hi = M;
    int c_hi = cnt(M);
    if (c_hi >= k) return M;
    int clo = n;
    for (int it = 0; it < 48; ++it) {
        const int nw = clo - c_hi;
        if (nw <= 4 || k - c_hi <= 1) break;
        float p = lo + (hi - lo) * ((float)(clo - k) + 0.5f) * __builtin_amdgcn_rcpf((float)nw);
        if (!(p > lo && p < hi)) p = 0.5f * lo + 0.5f * hi;
        if (!(p > lo && p < hi)) break;
        const int c = cnt(p);
        if (c >= k) {
            lo = p;
            clo = c;
        } else {
            hi = p;
            c_hi = c;
        }
    }
    for (int it = 0; it <= kListCap; ++it) {
        float m2 = kNegInf;
#pragma unroll
        for (int i = 0; i < kListRegs; ++i)
            if (i < nl) m2 = xl[i] < hi ? __builtin_fmaxf(m2, xl[i]) : m2;
        const float xm = wave_max(m2);
        const int c = cnt(xm);
        if (c >= k) return xm;
        hi = xm;
    }
    return lo;  // not reached: the count at the smallest list value is n >= k
}

// Gumbel race over the list entries with h >= cthr: each lane keeps its best
// (z, id, h) with z = h / tau + G, larger z first, smaller id on ties.
__device__ __forceinline__ void gumbel_list(Entry* list, int n, float cthr, bool filter, float inv_tau,
                                            const NoiseKey& nk, int lane, float& bz, int& be, float& bh) {
    // keep only the entries that can win, in order
    int base = filter ? 0 : n;
    for (int b0 = 0; filter && b0 < n; b0 += kWave) {
        const int o = b0 + lane;
        Entry en{kNegInf, 0};
        if (o < n) en = list[o];
        const bool pred = o < n && en.h >= cthr;
        const uint64_t m = ballot(pred);
        __builtin_amdgcn_wave_barrier();
        if (pred) list[base + lanes_below(m)] = en;
        base += popc(m);
        __builtin_amdgcn_wave_barrier();
    }
    for (int b0 = 0; b0 < base; b0 += kWave) {
        const int o = b0 + lane;
        if (o < base) {
            const Entry en = list[o];
            const float z = __builtin_fmaf(en.h, inv_tau, gumbel_from_word(noise_word(nk, (uint32_t)en.e)));
            if (z > bz || (z == bz && en.e < be)) {
                bz = z;
                be = en.e;
                bh = en.h;
            }
        }
    }
}

// Number of list entries whose h is above x.  The list has kWave spare entries
// past kListCap, so every lane reads in bounds; entries past n are ignored.
__device__ __forceinline__ int count_list_above(const Entry* list, int n, float x, int lane) {
    int c = 0;
    for (int b0 = 0; b0 < n; b0 += kWave) {
        const float hv = list[b0 + lane].h;
        c += popc(ballot(b0 + lane < n && hv > x));
    }
    return c;
}

// u's dwords loaded in u's own dword frame, moved into c's: when the two rows
// start at different halves of a dword, each c-frame dword takes one element
// from this own-frame dword and one from its neighbour (the next one when c's
// row starts on a dword boundary, `next`, else the previous one).  The
// neighbour is the adjacent lane's (a DPP wave shift), or at the wave's edge the
// adjacent slot's edge lane; past the first or last slot it reads 0, which only
// reaches positions outside the row.
template <int NS>
__device__ __forceinline__ void realign_u(uint32_t (&uw)[NS], bool next, int lane) {
    if (next) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {  // uw[j + 1] is still in its own frame here
            const uint32_t nb = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)uw[j], kDppWaveShl1, 0xF, 0xF, true);
            const uint32_t edge = j + 1 < NS ? (uint32_t)__builtin_amdgcn_readlane((int)uw[j + 1], 0) : 0u;
            uw[j] = __builtin_amdgcn_alignbit(lane == kWave - 1 ? edge : nb, uw[j], 16);
        }
    } else {
#pragma unroll
        for (int j = NS - 1; j >= 0; --j) {  // uw[j - 1] is still in its own frame here
            const uint32_t nb = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)uw[j], kDppWaveShr1, 0xF, 0xF, true);
            const uint32_t edge = j > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)uw[j - 1], kWave - 1) : 0u;
            uw[j] = __builtin_amdgcn_alignbit(uw[j], lane == 0 ? edge : nb, 16);
        }
    }
}

// Load one row's dwords through a buffer resource that covers exactly the row:
// the hardware range check returns 0 for dwords past it, so no load is branched
// or masked.  Slot j of lane l is dword 64 j + l.
template <int NS>
__device__ __forceinline__ void load_slots(const void* base, int lane, int ndw, uint32_t (&w)[NS]) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, ndw * 4, kBufferRsrcWord3);
#pragma unroll
    for (int j = 0; j < NS; ++j)
        w[j] = __builtin_amdgcn_raw_buffer_load_b32(r, lane * 4, j * kWave * 4, kBufferNontemporal);
}

// What a wave needs to know about its cell (all wave-uniform).
struct CellInfo {
    int64_t cell;       // index into the [C, P] outputs; times V, into c
    int64_t ucell;      // times V, into u (cell unless u is compacted)
    float s, tau, inv_tau;
    uint32_t t;         // position inside the request
    uint32_t row_iter;  // (row & 0xFFFF) | (iteration << 16)
    uint32_t rid;       // low 32 bits of the request id
};

// The cell at launch-relative position pl of `row`, from the kernel-argument
// table; false past the launch's positions.
__device__ __forceinline__ bool locate(const ReqTable& rq, int pl, int row, CellInfo& ci) {
    if (pl >= rq.npos) return false;  // (the kernel checks first)
    const ReqParams q = req_params(rq, find_request(rq, pl));
    ci.cell = (int64_t)row * rq.P + rq.pos0 + pl;
    ci.t = (uint32_t)(pl - q.start);  // starts are launch-relative
    ci.ucell = (int64_t)row * rq.Pu + q.uoff + ci.t;
    ci.s = q.scale;
    ci.tau = q.tau;
    ci.inv_tau = q.inv_tau;
    ci.row_iter = ((uint32_t)row & 0xFFFFu) | q.row_iter_hi;
    ci.rid = q.rid;
    return true;
}

// The same from per-request arrays in device memory, read as the wave starts.
__device__ __forceinline__ bool locate(const DevReq& d, bool have_u, int pl, int row, CellInfo& ci) {
    DevCell dc;
    if (!dev_cell(d, have_u, pl, dc)) return false;
    ci.cell = (int64_t)row * d.P + pl;
    ci.ucell = ci.cell;
    ci.s = dc.s;
    ci.tau = dc.tau;
    ci.inv_tau = dc.inv_tau;
    ci.t = dc.t;
    ci.row_iter = ((uint32_t)row & 0xFFFFu) | dc.iter_hi;
    ci.rid = dc.rid;
    return true;
}

template <bool BF16, int NS, typename Src>
__device__ __forceinline__ void sample_small_body(const SampleArgs& a, const Src& src) {
    using R_t = Row<BF16, NS>;
    constexpr int NE = R_t::NE;
    // + one spare entry per lane; 16-byte aligned for the histogram's vector accesses
    __shared__ __attribute__((aligned(16))) Entry s_list[kWavesPerBlock][kListCap + kWave];

    // every per-cell quantity below is wave-uniform (scalar registers); the grid
    // is (positions / 4, rows) with rows beyond 65535 folded into z
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = lane_id();
    const int pl = (int)blockIdx.x * kWavesPerBlock + wv;
    const int row = (int)(blockIdx.z * gridDim.y + blockIdx.y);
    if (row >= a.rows) return;  // whole wave leaves together
    constexpr bool kTable = !std::is_same<Src, DevReq>::value;
    // With the table, a cell's rows are known before its request is: c's loads,
    // and u's when every request of the launch reads u at its own position, go
    // out before the request lookup.
    bool early_u = false;
    int64_t cell;
    if constexpr (kTable) {
        if (pl >= src.npos) return;  // past the launch's positions: the whole wave leaves
        cell = (int64_t)row * src.P + src.pos0 + pl;
        early_u = src.all_guided != 0;
    } else {
        if (pl >= src.P) return;  // past the fixed layout (the grid rounds up to whole blocks)
        cell = (int64_t)row * src.P + pl;
    }
    const int V = a.V;
    Entry* list = s_list[wv];

    // ---------------------------------------------------------------- load
    // Both rows' loads are issued before any of their data is used, so a guided
    // cell waits for one memory latency, not two.  Dwords past a row read as 0
    // (buffer range check); only the slots from kFullSlots<NS> on can hold them.
    constexpr int FS = kFullSlots<BF16, NS>;
    uint32_t cw[NS], uw[NS];
    // bf16: the row in c's dword frame (its first id in the high half when par)
    int par = 0, ndw = V;
    if (BF16) {
        const uintptr_t cb = (uintptr_t)a.c;
        const int64_t g = (int64_t)((cb & 3) >> 1) + cell * V;
        par = (int)(g & 1);
        const int64_t off = (g >> 1) * 4 - (int64_t)(cb & 3);  // byte offset of the row's first dword
        ndw = (par + V + 1) >> 1;
        load_slots<NS>((const char*)a.c + off, lane, ndw, cw);
    } else {
        load_slots<NS>((const float*)a.c + cell * V, lane, V, cw);
    }
    // u's row (its own cell: a compacted u layout moves it), in its own dword frame
    // for bf16: the same as c's unless its start is on the other half
    int upar = par;
    auto load_u = [&](int64_t ucell) {
        if (BF16) {
            const uintptr_t ub = (uintptr_t)a.u + (uintptr_t)(ucell * V) * 2u;
            upar = (int)((ub >> 1) & 1u);
            load_slots<NS>((const char*)(ub - 2u * (uintptr_t)upar), lane, (upar + V + 1) >> 1, uw);
        } else {
            load_slots<NS>((const float*)a.u + ucell * V, lane, V, uw);
        }
    };
    if (early_u) load_u(cell);
    CellInfo ci;
    bool here;
    if constexpr (kTable)
        here = locate(src, pl, row, ci);
    else
        here = locate(src, a.u != nullptr, pl, row, ci);
    if (!here) return;  // padding position of the fixed layout: the whole wave leaves
    const float s = ci.s;
    const float tau = ci.tau;
    const bool use_u = s != 0.0f;
    if (use_u && !early_u) load_u(ci.ucell);

    R_t R;
    if (BF16) {
        R.ebase = 2 * lane - par;
        // c becomes -inf past the row, which makes h -inf whatever u reads there
        // (guided maps the NaN of -inf - -inf back to -inf)
#pragma unroll
        for (int j = FS; j < NS; ++j) cw[j] = (lane + j * kWave < ndw) ? cw[j] : 0xFF80FF80u;
        if (use_u) {
            if (upar != par) realign_u<NS>(uw, par == 0, lane);
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                R.h[2 * j] = guided_raw(bf16_lo(cw[j]), bf16_lo(uw[j]), s);
                R.h[2 * j + 1] = guided_raw(bf16_hi(cw[j]), bf16_hi(uw[j]), s);
            }
        } else {
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                R.h[2 * j] = bf16_lo(cw[j]);
                R.h[2 * j + 1] = bf16_hi(cw[j]);
            }
        }
        // the two half-dwords that belong to the neighbouring rows (the last
        // dword lies in a slot from FS on)
        if (par && lane == 0) R.h[0] = kNegInf;
        if ((par + V) & 1) {
            const int dl = ndw - 1;
#pragma unroll
            for (int j = FS; j < NS; ++j)
                if (j == (dl >> 6) && lane == (dl & 63)) R.h[2 * j + 1] = kNegInf;
        }
    } else {
        R.ebase = lane;
#pragma unroll
        for (int j = FS; j < NS; ++j) cw[j] = (lane + j * kWave < V) ? cw[j] : 0xFF800000u;
        if (use_u) {
#pragma unroll
            for (int j = 0; j < NS; ++j) R.h[j] = guided_raw(__uint_as_float(cw[j]), __uint_as_float(uw[j]), s);
        } else {
#pragma unroll
            for (int j = 0; j < NS; ++j) R.h[j] = __uint_as_float(cw[j]);
        }
    }

    // ---------------------------------------------------- max, log-sum-exp
    float mx = R.h[0];
#pragma unroll
    for (int i = 1; i < NE; ++i) mx = __builtin_fmaxf(mx, R.h[i]);
    const float M = wave_max(mx);

    const float mL = M * kLog2e;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < NE; ++i) acc += __builtin_amdgcn_exp2f(__builtin_fmaf(R.h[i], kLog2e, -mL));
    float S = wave_sum(acc);
    if (S != S) {
        // a masked id under guidance left a NaN h: make it -inf and sum again
#pragma unroll
        for (int i = 0; i < NE; ++i) R.h[i] = __builtin_fmaxf(R.h[i], kNegInf);
        acc = 0.0f;
#pragma unroll
        for (int i = 0; i < NE; ++i) acc += __builtin_amdgcn_exp2f(__builtin_fmaf(R.h[i], kLog2e, -mL));
        S = wave_sum(acc);
    }
    // exact residual of the rounded M*log2(e) shifts every exponent equally
    const float err = __builtin_fmaf(M, kLog2e, -mL);
    // S >= 1 - 2^-23 (the maximum's own term), so the hardware log2 needs no
    // denormal scaling
    const float lse = M + (__builtin_amdgcn_logf(S) - err) * kLn2;

    if (tau == 0.0f) {
        // Only greedy cells need the argmax of h (sampled cells take the Gumbel
        // winner): the smallest id attaining M.  Ids grow with the register index
        // inside a lane, so the first register slot (across lanes) holding M
        // decides.
        int am = 0x7FFFFFFF;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            if (BF16) {
                const uint64_t m0 = ballot(R.h[2 * j] == M);
                const uint64_t m1 = ballot(R.h[2 * j + 1] == M);
                if (m0 | m1) {
                    const int a0 = m0 ? 2 * (j * kWave + (int)__builtin_ctzll(m0)) : 0x7FFFFFFF;
                    const int a1 = m1 ? 2 * (j * kWave + (int)__builtin_ctzll(m1)) + 1 : 0x7FFFFFFF;
                    am = (a0 < a1 ? a0 : a1) - (R.ebase & 1);  // ebase & 1 == parity
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
        am = __builtin_amdgcn_readfirstlane(am);
        if (lane == 0) {
            a.tokens[cell] = am;
            a.logprobs[cell] = M - lse;
            if (a.thresholds) a.thresholds[cell] = __builtin_nanf("");
        }
        return;
    }

    // ------------------------------------------------------------ sampling
    const int k = a.top_k;
    NoiseKey nk;
    nk.k0 = a.k0;
    nk.k1 = a.k1;
    nk.t = ci.t;
    nk.row_iter = ci.row_iter;
    nk.rid = ci.rid;
    const float inv_tau = ci.inv_tau;
    // No id with h below `prune` can beat the argmax: its h/tau plus the largest
    // possible noise stays below M/tau plus the smallest possible noise.
    const float prune = max_bound(M, inv_tau, tau);
    const bool want_t = a.thresholds != nullptr;

    float t = kNegInf;
    float cthr = prune;  // draw noise for list entries with h >= cthr
    int n_list = -1;     // entries in the LDS list (all ids >= the list floor), or -1
    float bz = kNegInf, bh = kNegInf;
    int be = 0x7FFFFFFF;
    bool decided = false;  // (bz, be, bh) is the row's winner, wave-uniform
    // Race every id of a listed top set of n ids that holds the top-ratio set
    // (all ids with h >= floor).  The winner is then the argmax over the kept
    // ids as soon as it is kept itself, that is when fewer than top_k ids have a
    // larger h (those all lie above it, so all are listed).  Only when it is not
    // is the threshold found on the list, for a second race over the kept ids.
    auto race_listed = [&](int n, float floor) {
        gumbel_list(list, n, prune, false, inv_tau, nk, lane, bz, be, bh);
        const int wl = wave_argmax(bz, be);
        bh = readlane_f(bh, wl);
        if (count_list_above(list, n, bh, lane) < k) {
            decided = true;
        } else {
            bz = kNegInf;
            bh = kNegInf;
            be = 0x7FFFFFFF;
            t = list_kth(list, n, k, floor, M, lane);
            cthr = __builtin_fmaxf(t, prune);
        }
    };
    // Fast path: the ids that can still win.  If at most top_k of them reach
    // `prune`, they all lie inside the top-ratio set (fewer than top_k ids are
    // larger than any of them), so the filter is satisfied without locating its
    // exact threshold.  Up to kRaceAll of them are all raced (race_listed: the
    // race's winner is the argmax over every id, and it stands when it is kept).
    // A count of the ids above `prune` among the first four register elements of
    // every lane (a quarter to a ninth of the row, by ballots) tells rows with
    // far more than `cap` of them apart; those skip the full count and go
    // straight to the histogram, which handles any row.
    const int cap = min(max(k, kRaceAll), kListCap);
    int sub = 0;
#pragma unroll
    for (int i = 0; i < (NE < 4 ? NE : 4); ++i) sub += popc(ballot(R.h[i] >= prune));
    const bool flat = sub * NE > 6 * cap;  // about 1.5 * cap ids expected
    if (!want_t && !flat) {
        // (written straight away: a row that is not flat rarely has more)
        const int nb = R.write_ge(prune, list, cap);
        if (nb <= cap) {
            n_list = nb;
            if (nb > k) race_listed(nb, prune);
        }
    }
    // More ids can still win (rows flat next to tau * (Gmax - Gmin)), or the
    // threshold is wanted: a histogram of the ids above `prune` gives a top set
    // of a little more than top_k ids, exactly, which is listed and raced (or
    // searched for the threshold).
    if (n_list < 0) {
        float c;
        int n;
        if (top_set_by_histogram(R, list, k, prune, M, lane, c, n) && n <= kListCap) {
            // n ids have h >= c, so the list is written without counting first
            const int nc = R.write_ge(c, list, kListCap);
            if (nc <= kListCap) {
                n_list = nc;
                if (!want_t) {
                    race_listed(nc, c);
                } else {
                    t = list_kth(list, nc, k, c, M, lane);
                    cthr = __builtin_fmaxf(t, prune);
                }
            }
        }
    }
    if (n_list < 0) {
        // Exact threshold over the whole row: pivot from the row's spread, count
        // and compact the ids above the pivot, refine on the compacted list.
        bool have_t = false;
        float sum = 0.0f, sq = 0.0f;
        constexpr int NSTAT = NE < 4 ? NE : 4;
#pragma unroll
        for (int i = 0; i < NSTAT; ++i) {
            const float d = __builtin_fmaxf(R.h[i] - M, -64.0f);
            sum += d;
            sq = __builtin_fmaf(d, d, sq);
        }
        constexpr float inv_n = 1.0f / (float)(NSTAT * kWave);
        const float mean = wave_sum(sum) * inv_n;
        const float var = __builtin_fmaxf(wave_sum(sq) * inv_n - mean * mean, 0.0f);
        const float sd = __builtin_amdgcn_sqrtf(var) + 1e-3f;
        float lo = M + mean + a.z0 * sd;
        if (!(lo < M)) lo = M - sd;
        float hi = M;
        int c_hi = -1;
        // the search below keeps count(>= hi) < k, which fails at hi = M when at
        // least k ids tie with the maximum: then the threshold is M itself
        if (R.count_ge(M) >= k) {
            t = M;
            have_t = true;
        }
        for (int tries = 0; tries < 8 && !have_t; ++tries) {
            const int c_lo = R.count_compact(lo, list);
            if (c_lo >= k && c_lo <= kListCap) {
                t = list_kth(list, c_lo, k, lo, M, lane);
                n_list = c_lo;
                have_t = true;
                break;
            }
            if (c_lo < k) {
                hi = lo;
                c_hi = c_lo;
                if (tries < 3) {
                    lo = lo - (2.0f + 2.0f * tries) * sd;
                } else {
                    lo = min_finite(R);
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
                float p = lo + (hi - lo) * ((float)c_lo - target) * __builtin_amdgcn_rcpf((float)c_lo - chi);
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
        if (!have_t) t = kth_by_bisection(R, k, V, M);
        cthr = __builtin_fmaxf(t, prune);
    }

    // ------------------------------------------------------------ Gumbel-max
    if (decided) {
        // the race above settled it
    } else if (n_list >= 0) {
        gumbel_list(list, n_list, cthr, cthr > prune, inv_tau, nk, lane, bz, be, bh);
    } else {
        // every valid id with h >= cthr, straight from the row registers (rare:
        // fewer than top_k finite ids, massive ties, or a failed pivot search);
        // the slot loop stays rolled so the noise code is emitted once
#pragma unroll 1
        for (int i = 0; i < NE; ++i) {
            float hv = R.h[0];
#pragma unroll
            for (int j = 1; j < NE; ++j) hv = (i == j) ? R.h[j] : hv;
            const int ev = BF16 ? R.ebase + 2 * kWave * (i >> 1) + (i & 1) : R.ebase + kWave * i;
            const bool pred = hv >= cthr && ev >= 0 && ev < V;
            if (ballot(pred)) {
                if (pred) {
                    const float z = __builtin_fmaf(hv, inv_tau, gumbel_from_word(noise_word(nk, (uint32_t)ev)));
                    if (z > bz || (z == bz && ev < be)) {
                        bz = z;
                        be = ev;
                        bh = hv;
                    }
                }
            }
        }
    }
    if (!decided) {
        const int wl = wave_argmax(bz, be);
        bh = readlane_f(bh, wl);
    }
    if (lane == 0) {
        a.tokens[cell] = be;
        a.logprobs[cell] = bh - lse;
        if (want_t) a.thresholds[cell] = t + 0.0f;
    }
}

// Rows of up to 9 register slots (bf16) or 16 (f32) are held to 7 waves per SIMD
// or more (at most 73 VGPRs) without spilling, so a 6.5k-cell step fits in one
// round of the GPU's 1024 SIMDs; wider rows take what the compiler needs.
template <bool BF16, int NS>
__global__ __launch_bounds__(kWavesPerBlock * kWave) __attribute__((amdgpu_waves_per_eu(7, 8)))
void k_sample_small(SampleArgs a, ReqTable rq) {
    sample_small_body<BF16, NS>(a, rq);
}
template <bool BF16, int NS>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void k_sample_small_wide(SampleArgs a, ReqTable rq) {
    sample_small_body<BF16, NS>(a, rq);
}
// The same kernels with the per-request parameters in device memory.
template <bool BF16, int NS>
__global__ __launch_bounds__(kWavesPerBlock * kWave) __attribute__((amdgpu_waves_per_eu(7, 8)))
void k_sample_small_dev(SampleArgs a, DevReq d) {
    sample_small_body<BF16, NS>(a, d);
}
template <bool BF16, int NS>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void k_sample_small_dev_wide(SampleArgs a, DevReq d) {
    sample_small_body<BF16, NS>(a, d);
}

// Grid (positions / 4, rows), rows beyond 65535 folded into z.
inline dim3 small_grid(int64_t positions, int rows) {
    return dim3((unsigned)((positions + kWavesPerBlock - 1) / kWavesPerBlock), (unsigned)(rows < 65535 ? rows : 65535),
                (unsigned)((rows + 65534) / 65535));
}

template <bool BF16, int NS>
hipError_t launch_ns(const SampleArgs& a, const ReqTable& rq, hipStream_t st) {
    const dim3 g = small_grid(rq.npos, a.rows);
    constexpr bool kOcc = BF16 ? NS <= 9 : NS <= 16;
    if constexpr (kOcc)
        hipLaunchKernelGGL((k_sample_small<BF16, NS>), g, dim3(kWavesPerBlock * kWave), 0, st, a, rq);
    else
        hipLaunchKernelGGL((k_sample_small_wide<BF16, NS>), g, dim3(kWavesPerBlock * kWave), 0, st, a, rq);
    return hipGetLastError();
}
template <bool BF16, int NS>
hipError_t launch_ns(const SampleArgs& a, const DevReq& d, hipStream_t st) {
    const dim3 g = small_grid(d.P, a.rows);
    constexpr bool kOcc = BF16 ? NS <= 9 : NS <= 16;
    if constexpr (kOcc)
        hipLaunchKernelGGL((k_sample_small_dev<BF16, NS>), g, dim3(kWavesPerBlock * kWave), 0, st, a, d);
    else
        hipLaunchKernelGGL((k_sample_small_dev_wide<BF16, NS>), g, dim3(kWavesPerBlock * kWave), 0, st, a, d);
    return hipGetLastError();
}

// Register-slot counts that get an instantiation (bf16 rows stop at 16 slots,
// beyond which the compiler spills; those vocabularies use the row kernel).
template <bool BF16, typename Src>
hipError_t dispatch(int ns, const SampleArgs& a, const Src& src, hipStream_t st) {
    if (ns <= 2) return launch_ns<BF16, 2>(a, src, st);
    if (ns <= 4) return launch_ns<BF16, 4>(a, src, st);
    if (ns <= 6) return launch_ns<BF16, 6>(a, src, st);
    if (ns <= 9) return launch_ns<BF16, 9>(a, src, st);
    if (ns <= 12) return launch_ns<BF16, 12>(a, src, st);
    if (ns <= 16 || BF16) return launch_ns<BF16, 16>(a, src, st);
    if constexpr (!BF16) {
        if (ns <= 24) return launch_ns<BF16, 24>(a, src, st);
        return launch_ns<BF16, 32>(a, src, st);
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

hipError_t launch_sample_small_dev(bool bf16, const SampleArgs& a, const DevReq& d, hipStream_t st) {
    const int ns = small_slots_needed(bf16, a.V);
    if (ns > (bf16 ? kSmallMaxSlotsBf16 : kSmallMaxSlotsF32) || d.n < 1 || (d.n > kWave && !d.one_per_request) ||
        d.P < 1)
        return hipErrorInvalidValue;
    return bf16 ? dispatch<true>(ns, a, d, st) : dispatch<false>(ns, a, d, st);
}

}  // namespace ds
