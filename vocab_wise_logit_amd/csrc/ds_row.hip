// ds_row.hip -- one 1024-thread workgroup per row for large vocabularies.
//
// The row is streamed once from HBM in 16-byte pieces.  Each thread keeps an
// online (max, sum of exp) pair ([DRAFT] "Design and invariants": per-shard max,
// log-sum-exp and argmax), and the vocabulary is cut into `vocab_chunks`
// contiguous chunks, each reduced to a (max, lse, argmax) triple that is merged
// with the smallest-id tie rule -- the page's tensor-parallel shards, here as
// chunks of one row inside one workgroup.
//
// Sampling ([ISSUE] comment on the API shape: top-ratio filter plus Gumbel) needs
// the few ids that can still win the Gumbel race.  While streaming, each thread
// records the maximum of every group of 4 pieces it loaded in LDS.  After the
// pass the argmax's own noise G_a fixes a bound b = (M/tau + G_a - Gmax) * tau
// below which no id can win; only groups whose maximum reaches b are re-read
// (typically a few hundred of the row's ids), their ids with h >= b become
// candidates, and:
//   - if at most top_k ids reach b, all of them are inside the top-ratio set;
//   - otherwise the exact top_k-th largest h is among the candidates and is
//     selected there (radix select on the LDS list).
// When the lists overflow, when the caller asks for the threshold and it lies
// below b, or when the fallback is forced, the exact multi-pass path runs: a
// radix select of the threshold over re-reads of the row and a Gumbel pass over
// every kept id.  Both paths return the same token.
#include <stdint.h>

#include "ds_device.h"
#include "ds_kernels.h"

namespace ds {
namespace {

constexpr int NT = 1024;
constexpr int NWAVES = NT / kWave;
constexpr int U = 4;          // pieces per group
constexpr int GCAP = 8192;    // group maxima kept in LDS
constexpr int GLCAP = 2048;   // groups re-read
constexpr int CCAP = 2048;    // candidate (h, id) pairs

enum Mode { kModeGreedy = 0, kModeSample = 1 };

struct Shared {
    float gmax[GCAP];
    int glist[GLCAP];
    float ch[CCAP];
    int ce[CCAP];
    uint32_t hist[256];
    float red_f[NWAVES];
    float red_f2[NWAVES];
    int red_i[NWAVES];
    int cnt_g;
    int cnt_c;
    int flag;
    uint32_t bcast_u;
    float bcast_f;
};

__device__ __forceinline__ float block_max(float x, Shared& sh) {
    x = wave_max(x);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if (lane_id() == 0) sh.red_f[w] = x;
    __syncthreads();
    float r = sh.red_f[0];
#pragma unroll
    for (int i = 1; i < NWAVES; ++i) r = __builtin_fmaxf(r, sh.red_f[i]);
    return r;
}

__device__ __forceinline__ float block_sum(float x, Shared& sh) {
    x = wave_sum(x);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if (lane_id() == 0) sh.red_f[w] = x;
    __syncthreads();
    float r = 0.0f;
#pragma unroll
    for (int i = 0; i < NWAVES; ++i) r += sh.red_f[i];
    return r;
}

__device__ __forceinline__ int block_min_i(int x, Shared& sh) {
    x = wave_min_i(x);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if (lane_id() == 0) sh.red_i[w] = x;
    __syncthreads();
    int r = sh.red_i[0];
#pragma unroll
    for (int i = 1; i < NWAVES; ++i) r = min(r, sh.red_i[i]);
    return r;
}

// Block argmax of (z, id, h): larger z, then smaller id.
__device__ __forceinline__ void block_argmax3(float& z, int& id, float& hv, Shared& sh) {
    const int wl = wave_argmax(z, id);
    hv = readlane_f(hv, wl);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if (lane_id() == 0) {
        sh.red_f[w] = z;
        sh.red_i[w] = id;
        sh.red_f2[w] = hv;
    }
    __syncthreads();
    z = sh.red_f[0];
    id = sh.red_i[0];
    hv = sh.red_f2[0];
#pragma unroll
    for (int i = 1; i < NWAVES; ++i) {
        const bool take = (sh.red_f[i] > z) || (sh.red_f[i] == z && sh.red_i[i] < id);
        z = take ? sh.red_f[i] : z;
        id = take ? sh.red_i[i] : id;
        hv = take ? sh.red_f2[i] : hv;
    }
}

// Elements of one 16-byte piece, widened and guided.
template <bool BF16>
struct Piece {
    static constexpr int EPP = BF16 ? 8 : 4;
    float h[EPP];
};

template <bool BF16>
__device__ __forceinline__ void decode_piece(const u32x4 cw, const u32x4 uw, float s, bool use_u,
                                             Piece<BF16>& P) {
    if (BF16) {
        const uint32_t cc[4] = {cw.x, cw.y, cw.z, cw.w};
        if (use_u) {
            const uint32_t uu[4] = {uw.x, uw.y, uw.z, uw.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                P.h[2 * i] = guided(bf16_lo(cc[i]), bf16_lo(uu[i]), s);
                P.h[2 * i + 1] = guided(bf16_hi(cc[i]), bf16_hi(uu[i]), s);
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
            for (int i = 0; i < 4; ++i) P.h[i] = guided(cf[i], uf[i], s);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) P.h[i] = cf[i];
        }
    }
}

template <bool BF16>
__device__ __forceinline__ void load_piece(gptr<u32x4> c16, gptr<u32x4> u16, int64_t q, float s,
                                           bool use_u, Piece<BF16>& P) {
    const u32x4 cw = c16[q];
    const u32x4 uw = use_u ? u16[q] : cw;
    decode_piece<BF16>(cw, uw, s, use_u, P);
}

// Geometry of one row inside the 16-byte-aligned view of the tensors.
struct RowGeom {
    gptr<u32x4> c16;
    gptr<u32x4> u16;
    int64_t gbase;  // element index of id 0 in the aligned view
    int V;
    int L;          // chunk length ceil(V / nch)
    int nch;
    int gpc;        // group ids reserved per chunk
};

template <bool BF16>
struct ChunkRange {
    int lo, hi;          // row ids [lo, hi)
    int64_t q0, q1;      // first / last piece index (q1 < q0 when empty)
    __device__ ChunkRange(const RowGeom& G, int j) {
        constexpr int EPP = Piece<BF16>::EPP;
        lo = min(G.V, j * G.L);
        hi = min(G.V, lo + G.L);
        if (hi > lo) {
            q0 = (G.gbase + lo) / EPP;
            q1 = (G.gbase + hi - 1) / EPP;
        } else {
            q0 = 0;
            q1 = -1;
        }
    }
};

// Mask the ids of a piece that fall outside [lo, hi) (row-relative).
template <bool BF16>
__device__ __forceinline__ void mask_piece(Piece<BF16>& P, int64_t q, const RowGeom& G, int lo, int hi) {
    constexpr int EPP = Piece<BF16>::EPP;
    const int64_t v0 = q * EPP - G.gbase;
    if (v0 < lo || v0 + EPP > hi) {
#pragma unroll
        for (int i = 0; i < EPP; ++i) {
            const int64_t v = v0 + i;
            if (v < lo || v >= hi) P.h[i] = kNegInf;
        }
    }
}

// Visit every id of the row (all chunks): f(v, h).  Used by the exact paths.
template <bool BF16, typename F>
__device__ __forceinline__ void for_each_id(const RowGeom& G, float s, bool use_u, F&& f) {
    constexpr int EPP = Piece<BF16>::EPP;
    const int64_t q0 = G.gbase / EPP;
    const int64_t q1 = (G.gbase + G.V - 1) / EPP;
    for (int64_t q = q0 + threadIdx.x; q <= q1; q += NT) {
        Piece<BF16> P;
        load_piece<BF16>(G.c16, G.u16, q, s, use_u, P);
        mask_piece<BF16>(P, q, G, 0, G.V);
        const int64_t v0 = q * EPP - G.gbase;
#pragma unroll
        for (int i = 0; i < EPP; ++i)
            if (v0 + i >= 0 && v0 + i < G.V) f((int)(v0 + i), P.h[i]);
    }
}

// Exact top_k-th largest h of the row: four 8-bit radix passes over re-reads.
template <bool BF16>
__device__ float radix_select_row(const RowGeom& G, float s, bool use_u, int k, Shared& sh) {
    uint32_t prefix = 0, pmask = 0;
    int kk = k;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = threadIdx.x; i < 256; i += NT) sh.hist[i] = 0;
        __syncthreads();
        for_each_id<BF16>(G, s, use_u, [&](int, float h) {
            const uint32_t key = order_key(h + 0.0f);
            if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
        });
        __syncthreads();
        if (threadIdx.x == 0) {
            int above = 0;
            int d = 255;
            for (; d > 0; --d) {
                const int c = (int)sh.hist[d];
                if (above + c >= kk) break;
                above += c;
            }
            sh.bcast_u = (uint32_t)d | ((uint32_t)above << 8);
        }
        __syncthreads();
        const uint32_t d = sh.bcast_u & 255u;
        kk -= (int)(sh.bcast_u >> 8);
        prefix |= d << shift;
        pmask |= 255u << shift;
        __syncthreads();
    }
    return key_value(prefix);
}

// Exact top_k-th largest among the first n candidates in LDS (n >= k).
__device__ float radix_select_list(int n, int k, Shared& sh) {
    uint32_t prefix = 0, pmask = 0;
    int kk = k;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = threadIdx.x; i < 256; i += NT) sh.hist[i] = 0;
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += NT) {
            const uint32_t key = order_key(sh.ch[i] + 0.0f);
            if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            int above = 0;
            int d = 255;
            for (; d > 0; --d) {
                const int c = (int)sh.hist[d];
                if (above + c >= kk) break;
                above += c;
            }
            sh.bcast_u = (uint32_t)d | ((uint32_t)above << 8);
        }
        __syncthreads();
        const uint32_t d = sh.bcast_u & 255u;
        kk -= (int)(sh.bcast_u >> 8);
        prefix |= d << shift;
        pmask |= 255u << shift;
        __syncthreads();
    }
    return key_value(prefix);
}

// Wave-aggregated append of this lane's item to an LDS counter; returns the slot
// (or -1 when the lane has nothing).
__device__ __forceinline__ int wave_append(bool pred, int* counter) {
    const uint64_t m = ballot(pred);
    if (!m) return -1;
    int base = 0;
    const int leader = (int)__builtin_ctzll(m);
    if (lane_id() == leader) base = atomicAdd(counter, popc(m));
    base = __builtin_amdgcn_readlane(base, leader);
    return pred ? base + lanes_below(m) : -1;
}

struct RowResult {
    float M;       // row max of h
    float lse;     // log-sum-exp of h
    int id;        // smallest argmax
};

// The single streaming pass: per-chunk triples merged into the row result.
// Optionally writes each group's maximum to sh.gmax and each chunk's triple.
template <bool BF16>
__device__ RowResult stream_row(const RowGeom& G, float s, bool use_u, bool keep_groups,
                                float* triples, int64_t n_rows, int64_t row_index, Shared& sh) {
    constexpr int EPP = Piece<BF16>::EPP;
    float Mrow = kNegInf, Srow = 0.0f;
    int idrow = 0x7FFFFFFF;
    for (int j = 0; j < G.nch; ++j) {
        const ChunkRange<BF16> cr(G, j);
        float m = kNegInf, acc = 0.0f;
        int bg = -1;  // group (within chunk) holding this thread's max
        const int64_t nq = cr.q1 - cr.q0 + 1;
        const int its = (int)((nq + (int64_t)NT * U - 1) / ((int64_t)NT * U));
        // one group: U raw 16-byte pieces of c (and u); two groups are in flight
        // at a time (ping-pong) so the loads of the next group overlap the math
        // on the current one
        struct Raw {
            u32x4 c[U], u[U];
        };
        auto load = [&](Raw& R, int it) {
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
                const int64_t q = cr.q0 + (int64_t)it * NT * U + (int64_t)uu * NT + threadIdx.x;
                const uint32_t ninf = BF16 ? 0xFF80FF80u : 0xFF800000u;
                R.c[uu] = u32x4{ninf, ninf, ninf, ninf};
                R.u[uu] = R.c[uu];
                if (q <= cr.q1) {
                    R.c[uu] = G.c16[q];
                    if (use_u) R.u[uu] = G.u16[q];
                }
            }
        };
        auto process = [&](const Raw& R, int it) {
            Piece<BF16> P[U];
            float gm = kNegInf;
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
                const int64_t q = cr.q0 + (int64_t)it * NT * U + (int64_t)uu * NT + threadIdx.x;
                decode_piece<BF16>(R.c[uu], R.u[uu], s, use_u, P[uu]);
                mask_piece<BF16>(P[uu], q, G, cr.lo, cr.hi);
#pragma unroll
                for (int i = 0; i < EPP; ++i) gm = __builtin_fmaxf(gm, P[uu].h[i]);
            }
            const int gid = it * NT + (int)threadIdx.x;
            if (gm > m) {
                acc *= __builtin_amdgcn_exp2f((m - gm) * kLog2e);
                m = gm;
                bg = gid;
            }
            // a thread that has seen only -inf keeps acc = 0 (exp2(-inf) = 0)
            const float mL = (m > kNegInf) ? m * kLog2e : 0.0f;
#pragma unroll
            for (int uu = 0; uu < U; ++uu)
#pragma unroll
                for (int i = 0; i < EPP; ++i) acc += __builtin_amdgcn_exp2f(__builtin_fmaf(P[uu].h[i], kLog2e, -mL));
            if (keep_groups) sh.gmax[j * G.gpc + gid] = gm;
        };
        Raw A, B;
        if (its > 0) load(A, 0);
        for (int it = 0; it < its; it += 2) {
            if (it + 1 < its) load(B, it + 1);
            process(A, it);
            if (it + 1 < its) {
                if (it + 2 < its) load(A, it + 2);
                process(B, it + 1);
            }
        }
        // undo the rounding of m * log2(e) for this thread's partial sum
        if (m > kNegInf) acc *= __builtin_amdgcn_exp2f(-__builtin_fmaf(m, kLog2e, -(m * kLog2e)));
        const float Mj = block_max(m, sh);
        const float part = (m > kNegInf) ? acc * __builtin_amdgcn_exp2f((m - Mj) * kLog2e) : 0.0f;
        const float Sj = block_sum(part, sh);
        // smallest id attaining Mj: only threads whose max equals Mj look again
        int idj = 0x7FFFFFFF;
        if (Mj > kNegInf && m == Mj && bg >= 0) {
            const int it = bg / NT;
#pragma unroll
            for (int uu = 0; uu < U && idj == 0x7FFFFFFF; ++uu) {
                const int64_t q = cr.q0 + (int64_t)it * NT * U + (int64_t)uu * NT + threadIdx.x;
                if (q > cr.q1) break;
                Piece<BF16> P1;
                load_piece<BF16>(G.c16, G.u16, q, s, use_u, P1);
                mask_piece<BF16>(P1, q, G, cr.lo, cr.hi);
                const int64_t v0 = q * EPP - G.gbase;
#pragma unroll
                for (int i = EPP - 1; i >= 0; --i)
                    if (P1.h[i] == Mj) idj = (int)(v0 + i);
            }
        }
        idj = block_min_i(idj, sh);
        if (triples && threadIdx.x == 0) {
            float* o = triples + ((int64_t)j * n_rows + row_index) * 3;
            o[0] = Mj;
            o[1] = (Mj > kNegInf) ? Mj + __builtin_logf(Sj) : kNegInf;
            o[2] = __int_as_float(idj);
        }
        // merge the chunk triple into the row ([DRAFT]: larger max wins, equal
        // maxima keep the smaller id, sums add in probability space)
        if (Mj > kNegInf) {
            const float Mn = __builtin_fmaxf(Mrow, Mj);
            Srow = ((Mrow > kNegInf) ? Srow * __builtin_amdgcn_exp2f((Mrow - Mn) * kLog2e) : 0.0f) +
                   Sj * __builtin_amdgcn_exp2f((Mj - Mn) * kLog2e);
            if (Mj > Mrow || (Mj == Mrow && idj < idrow)) idrow = idj;
            Mrow = Mn;
        }
    }
    RowResult r;
    r.M = Mrow;
    r.lse = Mrow + __builtin_logf(Srow);
    r.id = idrow;
    return r;
}

template <bool BF16>
__global__ __launch_bounds__(NT) void k_greedy_lse(GreedyArgs a) {
    __shared__ Shared sh;
    const int64_t row = blockIdx.x;
    if (row >= a.n_rows) return;
    constexpr int ES = BF16 ? 2 : 4;
    const uintptr_t xb = (uintptr_t)a.x;
    RowGeom G;
    G.c16 = as_global<u32x4>((const char*)a.x - (xb & 15));
    G.u16 = G.c16;
    G.gbase = (int64_t)((xb & 15) / ES) + row * a.V;
    G.V = a.V;
    G.nch = a.vocab_chunks;
    G.L = (a.V + a.vocab_chunks - 1) / a.vocab_chunks;
    G.gpc = 0;
    const RowResult r = stream_row<BF16>(G, 0.0f, false, false, a.triples, a.n_rows, row, sh);
    if (threadIdx.x == 0) {
        a.token[row] = r.id;
        a.lse[row] = r.lse;
        a.logprob[row] = r.M - r.lse;
    }
}

template <bool BF16>
__global__ __launch_bounds__(NT) void k_sample_row(SampleArgs a, ReqTable rq) {
    __shared__ Shared sh;
    constexpr int EPP = Piece<BF16>::EPP;
    constexpr int ES = BF16 ? 2 : 4;
    const int64_t wid = blockIdx.x;
    if (wid >= (int64_t)a.rows * rq.npos) return;
    const int row = (int)(wid / rq.npos);
    const int pl = (int)(wid - (int64_t)row * rq.npos);
    const int r = find_request(rq, pl);
    const int64_t cell = (int64_t)row * rq.P + rq.pos0 + pl;
    const float s = rq.scale[r];
    const float tau = rq.tau[r];
    const bool use_u = s != 0.0f;

    const uintptr_t cb = (uintptr_t)a.c;
    RowGeom G;
    G.c16 = as_global<u32x4>((const char*)a.c - (cb & 15));
    G.u16 = use_u ? as_global<u32x4>((const char*)a.u - (cb & 15)) : G.c16;
    G.gbase = (int64_t)((cb & 15) / ES) + cell * a.V;
    G.V = a.V;
    G.nch = a.vocab_chunks;
    G.L = (a.V + a.vocab_chunks - 1) / a.vocab_chunks;
    {
        const int64_t qmax = (int64_t)G.L / EPP + 2;
        G.gpc = (int)(((qmax + (int64_t)NT * U - 1) / ((int64_t)NT * U)) * NT);
    }
    const bool sampled = tau != 0.0f;
    const bool groups_fit = (int64_t)G.gpc * G.nch <= GCAP;
    const bool fast = sampled && groups_fit && !a.force_fallback;
    if (fast)
        for (int i = threadIdx.x; i < GCAP; i += NT) sh.gmax[i] = kNegInf;
    __syncthreads();

    const RowResult rr = stream_row<BF16>(G, s, use_u, fast, nullptr, 0, 0, sh);
    if (!sampled) {
        if (threadIdx.x == 0) {
            a.tokens[cell] = rr.id;
            a.logprobs[cell] = rr.M - rr.lse;
            if (a.thresholds) a.thresholds[cell] = __builtin_nanf("");
        }
        return;
    }

    NoiseKey nk;
    nk.k0 = a.k0;
    nk.k1 = a.k1;
    nk.t = (uint32_t)(pl - rq.offs[r]);
    nk.row_iter = ((uint32_t)row & 0xFFFFu) | rq.row_iter_hi[r];
    nk.rid = rq.rid[r];
    const float inv_tau = rq.inv_tau[r];
    const int k = a.top_k;
    // the argmax's own draw bounds every id that could still win
    const float za = __builtin_fmaf(rr.M, inv_tau, gumbel_from_word(noise_word(nk, (uint32_t)rr.id)));
    const float b = (za - kGumbelBound) * tau;

    float t = kNegInf;
    bool have_t = false;
    bool done = false;
    float bz = kNegInf, bh = kNegInf;
    int be = 0x7FFFFFFF;

    if (fast) {
        if (threadIdx.x == 0) {
            sh.cnt_g = 0;
            sh.cnt_c = 0;
        }
        __syncthreads();
        const int ng = G.gpc * G.nch;
        for (int g0 = 0; g0 < ng; g0 += NT) {
            const int g = g0 + (int)threadIdx.x;
            const bool pred = g < ng && sh.gmax[g] >= b;
            const int slot = wave_append(pred, &sh.cnt_g);
            if (slot >= 0 && slot < GLCAP) sh.glist[slot] = g;
        }
        __syncthreads();
        const int nglist = sh.cnt_g;
        if (nglist <= GLCAP) {
            for (int i0 = 0; i0 < nglist; i0 += NT) {
                const int i = i0 + (int)threadIdx.x;
                Piece<BF16> P[U];
                int64_t qs[U];
                bool any = false;
                if (i < nglist) {
                    const int g = sh.glist[i];
                    const int j = g / G.gpc;
                    const int rem = g - j * G.gpc;
                    const int it = rem / NT;
                    const int tt = rem - it * NT;
                    const ChunkRange<BF16> cr(G, j);
#pragma unroll
                    for (int uu = 0; uu < U; ++uu) {
                        qs[uu] = cr.q0 + (int64_t)it * NT * U + (int64_t)uu * NT + tt;
                        if (qs[uu] <= cr.q1) {
                            load_piece<BF16>(G.c16, G.u16, qs[uu], s, use_u, P[uu]);
                            mask_piece<BF16>(P[uu], qs[uu], G, cr.lo, cr.hi);
                            any = true;
                        } else {
#pragma unroll
                            for (int e = 0; e < EPP; ++e) P[uu].h[e] = kNegInf;
                        }
                    }
                } else {
#pragma unroll
                    for (int uu = 0; uu < U; ++uu) {
                        qs[uu] = 0;
#pragma unroll
                        for (int e = 0; e < EPP; ++e) P[uu].h[e] = kNegInf;
                    }
                }
                (void)any;
#pragma unroll
                for (int uu = 0; uu < U; ++uu)
#pragma unroll
                    for (int e = 0; e < EPP; ++e) {
                        const bool pred = P[uu].h[e] >= b;
                        const int slot = wave_append(pred, &sh.cnt_c);
                        if (slot >= 0 && slot < CCAP) {
                            sh.ch[slot] = P[uu].h[e];
                            sh.ce[slot] = (int)(qs[uu] * EPP + e - G.gbase);
                        }
                    }
            }
            __syncthreads();
            const int nb = sh.cnt_c;
            if (nb <= CCAP) {
                // every id with h >= b is in the list
                float cthr = b;
                if (nb >= k) {
                    t = radix_select_list(nb, k, sh);
                    have_t = true;
                    cthr = __builtin_fmaxf(t, b);
                }
                for (int i = threadIdx.x; i < nb; i += NT) {
                    const float hv = sh.ch[i];
                    const int ev = sh.ce[i];
                    if (hv >= cthr) {
                        const float z = __builtin_fmaf(hv, inv_tau, gumbel_from_word(noise_word(nk, (uint32_t)ev)));
                        if (z > bz || (z == bz && ev < be)) {
                            bz = z;
                            be = ev;
                            bh = hv;
                        }
                    }
                }
                done = true;
            }
        }
    }
    // uniform: `done` depends only on LDS counters read after a barrier
    if (!done || (a.thresholds && !have_t)) {
        t = radix_select_row<BF16>(G, s, use_u, k, sh);
        have_t = true;
    }
    if (!done) {
        const float cthr = __builtin_fmaxf(t, b);
        bz = kNegInf;
        be = 0x7FFFFFFF;
        for_each_id<BF16>(G, s, use_u, [&](int v, float hv) {
            if (!(hv >= cthr)) return;
            const float z = __builtin_fmaf(hv, inv_tau, gumbel_from_word(noise_word(nk, (uint32_t)v)));
            if (z > bz || (z == bz && v < be)) {
                bz = z;
                be = v;
                bh = hv;
            }
        });
    }
    block_argmax3(bz, be, bh, sh);
    if (threadIdx.x == 0) {
        a.tokens[cell] = be;
        a.logprobs[cell] = bh - rr.lse;
        if (a.thresholds) a.thresholds[cell] = t + 0.0f;
    }
}

}  // namespace

hipError_t launch_sample_row(bool bf16, const SampleArgs& a, const ReqTable& rq, hipStream_t st) {
    const int64_t cells = (int64_t)a.rows * rq.npos;
    if (bf16)
        hipLaunchKernelGGL(k_sample_row<true>, dim3((unsigned)cells), dim3(NT), 0, st, a, rq);
    else
        hipLaunchKernelGGL(k_sample_row<false>, dim3((unsigned)cells), dim3(NT), 0, st, a, rq);
    return hipGetLastError();
}

hipError_t launch_greedy_lse(bool bf16, const GreedyArgs& a, hipStream_t st) {
    if (a.n_rows == 0) return hipSuccess;
    if (bf16)
        hipLaunchKernelGGL(k_greedy_lse<true>, dim3((unsigned)a.n_rows), dim3(NT), 0, st, a);
    else
        hipLaunchKernelGGL(k_greedy_lse<false>, dim3((unsigned)a.n_rows), dim3(NT), 0, st, a);
    return hipGetLastError();
}

}  // namespace ds
