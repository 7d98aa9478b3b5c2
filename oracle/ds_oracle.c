/*
 * ds_oracle.c -- plain, slow, obviously-correct CPU oracle for the per-position
 * full-vocabulary sampling reduction.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may include, link,
 * load or call this file.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * Sources (the pages; cited by title and section):
 *   [ISSUE]  mstar issue "Sampler support for discrete diffusion":
 *            the opening request (return log-probabilities for every sampled
 *            position) and the comment on the API shape (greedy token = argmax of
 *            the log-probabilities, confidence = their max; CFG combine of two
 *            logit tensors and top-ratio filtering to ceil(0.1 * V) entries with
 *            Gumbel noise; both per request, like temperature).
 *   [PR]     mstar PR "Add a sampler resource for discrete diffusion", section
 *            "What does this PR do?": the contract sample(request_ids, c_logits,
 *            u_logits, seq_lens, iterations) over logits packed as
 *            [rows, positions, vocab], returning (tokens, logprobs) per position;
 *            guidance scale and temperature per request, broadcast per position;
 *            guidance scale 0 means no unconditional logits are built.
 *   [DRAFT]  LightLLM PR "perf: avoid full-vocab all-gather for draft greedy
 *            sampling", section "Design and invariants": per-shard max,
 *            log-sum-exp and argmax, three 32-bit words per token, ties resolve to
 *            the smallest global id, the id travels bit-for-bit in a float word,
 *            and the selected probability is exp(selected_logit - full LSE).
 *   [PHILOX] Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 *            1, 2, 3", SC'11: the Philox4x32 round function and key schedule.
 *
 * Readings where the pages are silent (each restated in the design doc):
 *   - CFG convention: guided = lc + s * (lc - lu) on log-softmaxed c and u, then
 *     renormalised; log-probabilities are of that distribution over the full
 *     vocabulary, before temperature and before the top-ratio filter.
 *   - Selection (argmax, threshold, Gumbel) uses the fp32 guided logit
 *     h = fmaf(s, c - u, c) (h = c when s == 0, u unread), which orders the
 *     vocabulary exactly like the renormalised CFG log-probabilities up to fp32
 *     rounding.  A c of -inf (masked id) gives h = -inf.
 *   - Temperature divides h; temperature 0 is greedy; the filter keeps every id
 *     whose h is >= the k-th largest h (ties kept), k = ceil(V / 10) by default.
 *   - Gumbel noise: Philox4x32-10 keyed by the 64-bit seed; counter
 *     (v >> 2, t, (row & 0xFFFF) | (iteration << 16), (uint32)request_id), word
 *     v & 3; U = ((x >> 9) * 2 + 1) * 2^-24; G = -log(-log U); the token
 *     maximises h / tau + G over the kept ids, smallest id on exact ties.
 *   - Autoregressive mode ([ISSUE]: the existing sampler draws one token per
 *     request and applies a repetition penalty over seen-token masks; the pages
 *     give no formula): a seen id's logit x becomes x / theta when x > 0 and
 *     x * theta otherwise, in binary32, stored back in the logits' own type
 *     (bf16 by round-to-nearest-even); the token is then drawn like a cell with
 *     guidance 0, with the top-ratio filter chosen by the caller's top_k.
 *   - Confidence reveal ([ISSUE], the top-k over the flattened [C, T] scores):
 *     per request, the reveal_count largest scores of its [C, T] block flattened
 *     row-major, best first, the smaller flattened index first on equal scores.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off, no fast-math, so that
 * float expressions round exactly as written (IEEE-754 binary32 / binary64,
 * round-to-nearest-even, denormals kept).
 */

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define DSO_F32 0
#define DSO_BF16 1

static char g_err[256];

const char *dso_last_error(void) { return g_err; }

static int fail(const char *msg) {
    snprintf(g_err, sizeof g_err, "%s", msg);
    return 1;
}

/* ---------------------------------------------------------------- encoding */

static float f32_from_bits(uint32_t b) {
    float f;
    memcpy(&f, &b, sizeof f);
    return f;
}

static uint32_t bits_from_f32(float f) {
    uint32_t b;
    memcpy(&b, &f, sizeof b);
    return b;
}

/* bf16 is the upper half of an IEEE binary32: widening is exact. */
float dso_bf16_to_f32(uint16_t b) { return f32_from_bits((uint32_t)b << 16); }

void dso_bf16_to_f32_array(const uint16_t *src, float *dst, int64_t n) {
    for (int64_t i = 0; i < n; i++) dst[i] = dso_bf16_to_f32(src[i]);
}

static float load_elem(const void *base, int dtype, int64_t i) {
    if (dtype == DSO_BF16) return dso_bf16_to_f32(((const uint16_t *)base)[i]);
    return ((const float *)base)[i];
}

/* Order-preserving map from binary32 to uint32 (negative: all bits flipped;
 * non-negative: sign bit set).  -0 and +0 map to different keys, which is why
 * guided logits are canonicalised to +0 before any key is taken. */
uint32_t dso_order_key(float x) {
    uint32_t b = bits_from_f32(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

float dso_key_to_f32(uint32_t k) {
    uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return f32_from_bits(b);
}

/* ------------------------------------------------- guided selection logit */

/* [ISSUE] CFG combine, [PR] guidance 0 means u is never built or read.
 * h = c + s * (c - u) with one rounding of the product-sum (fmaf), then +0.0f
 * to turn a -0 into +0.  A masked id (c == -inf) stays masked. */
float dso_guided_logit(float c, float u, float s) {
    float h;
    if (s == 0.0f)
        h = c;
    else if (c == -INFINITY)
        h = -INFINITY;
    else
        h = fmaf(s, c - u, c);
    return h + 0.0f;
}

/* Valid inputs: c finite or -inf (a masked id); when s != 0, u is finite, or -inf
 * at an id whose c is -inf too. */
static int check_inputs(float c, float u, float s) {
    if (isnan(c) || c == INFINITY) return 0;
    if (s != 0.0f) {
        if (isnan(u) || u == INFINITY) return 0;
        if (c != -INFINITY && u == -INFINITY) return 0;
    }
    return 1;
}

/* ---------------------------------------------------------- log-sum-exp */

static double lse_d(const double *x, int64_t n) {
    double m = -INFINITY;
    for (int64_t i = 0; i < n; i++)
        if (x[i] > m) m = x[i];
    if (m == -INFINITY) return -INFINITY;
    double s = 0.0;
    for (int64_t i = 0; i < n; i++) s += exp(x[i] - m);
    return m + log(s);
}

double dso_lse(const double *x, int64_t n) { return lse_d(x, n); }

/* [ISSUE]/[PR] log-probabilities of the guided distribution for one row.
 * lc = c - LSE(c), lu = u - LSE(u), g = lc + s * (lc - lu), lp = g - LSE(g).
 * When s == 0, g = lc and u is not read.  Masked ids (c == -inf) get -inf.
 * work must hold 2 * V doubles.  Returns 0 on success. */
int dso_row_logprobs(int dtype, const void *c_row, const void *u_row, float s, int32_t V,
                     double *lp, double *work) {
    double *cd = work, *ud = work + V;
    for (int32_t v = 0; v < V; v++) {
        float c = load_elem(c_row, dtype, v);
        float u = (s != 0.0f) ? load_elem(u_row, dtype, v) : 0.0f;
        if (!check_inputs(c, u, s)) return fail("unsupported non-finite logit");
        cd[v] = (double)c;
        ud[v] = (double)u;
    }
    double Lc = lse_d(cd, V);
    if (Lc == -INFINITY) return fail("row has no finite logit");
    double Lu = (s != 0.0f) ? lse_d(ud, V) : 0.0;
    for (int32_t v = 0; v < V; v++) {
        if (cd[v] == -INFINITY) {
            lp[v] = -INFINITY;
            continue;
        }
        double lc = cd[v] - Lc;
        double g = lc;
        if (s != 0.0f) {
            double lu = ud[v] - Lu;
            g = lc + (double)s * (lc - lu);
        }
        lp[v] = g;
    }
    double Lg = lse_d(lp, V);
    for (int32_t v = 0; v < V; v++) lp[v] -= Lg;
    return 0;
}

/* --------------------------------------------------------------- Philox */

/* [PHILOX] Philox4x32 with 10 rounds.  One round maps (x0, x1, x2, x3) with key
 * (k0, k1) to (hi(B*x2) ^ x1 ^ k0, lo(B*x2), hi(A*x0) ^ x3 ^ k1, lo(A*x0)),
 * A = 0xD2511F53, B = 0xCD9E8D57; the key is bumped by the Weyl constants
 * (0x9E3779B9, 0xBB67AE85) between rounds. */
void dso_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; round++) {
        uint64_t pa = (uint64_t)0xD2511F53u * (uint64_t)x0;
        uint64_t pb = (uint64_t)0xCD9E8D57u * (uint64_t)x2;
        uint32_t y0 = (uint32_t)(pb >> 32) ^ x1 ^ k0;
        uint32_t y1 = (uint32_t)pb;
        uint32_t y2 = (uint32_t)(pa >> 32) ^ x3 ^ k1;
        uint32_t y3 = (uint32_t)pa;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* The 32-bit noise word for vocabulary id v of one cell. */
uint32_t dso_noise_word(uint64_t seed, int64_t request_id, int32_t iteration, int32_t row,
                        int32_t t, int32_t v) {
    uint32_t ctr[4], key[2], out[4];
    ctr[0] = (uint32_t)v >> 2;
    ctr[1] = (uint32_t)t;
    ctr[2] = ((uint32_t)row & 0xFFFFu) | ((uint32_t)iteration << 16);
    ctr[3] = (uint32_t)request_id;
    key[0] = (uint32_t)seed;
    key[1] = (uint32_t)(seed >> 32);
    dso_philox4x32_10(ctr, key, out);
    return out[(uint32_t)v & 3u];
}

/* U in (0, 1): the top 23 bits of the word on the odd lattice of step 2^-23. */
double dso_uniform(uint32_t x) { return (double)((x >> 9) * 2u + 1u) * 0x1p-24; }

/* G = -log(-log U), with -log U = -log1p(U - 1) (U - 1 is exact). */
double dso_gumbel(uint32_t x) {
    double U = dso_uniform(x);
    return -log(-log1p(U - 1.0));
}

/* ------------------------------------------------------------ selection */

static int cmp_key_desc(const void *a, const void *b) {
    uint32_t x = *(const uint32_t *)a, y = *(const uint32_t *)b;
    return (x < y) - (x > y);
}

/* The k-th largest of n binary32 values (1 <= k <= n), by a full sort of their
 * order keys.  Values must already be canonical (+0, never -0). */
float dso_kth_largest(const float *h, int64_t n, int64_t k) {
    uint32_t *keys = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)n);
    for (int64_t i = 0; i < n; i++) keys[i] = dso_order_key(h[i]);
    qsort(keys, (size_t)n, sizeof(uint32_t), cmp_key_desc);
    float t = dso_key_to_f32(keys[k - 1]);
    free(keys);
    return t;
}

/* One cell of the diffusion sampler, given its guided logits h (fp32, canonical)
 * and its log-probabilities lp.  temperature 0: greedy.  Otherwise top-ratio
 * filter then Gumbel-max.  Writes token, logprob, threshold (NaN when greedy),
 * the z gap between the best and second-best kept id, and near_tie. */
static void sample_cell(const float *h, const double *lp, int32_t V, int32_t top_k, float tau,
                        uint64_t seed, int64_t request_id, int32_t iteration, int32_t row,
                        int32_t t, int32_t *token, float *logprob, float *threshold,
                        double *gap, uint8_t *near_tie) {
    /* greedy argmax: the smallest id attaining the maximum ([DRAFT] tie rule,
     * applied to every greedy decision) */
    int32_t am = 0;
    for (int32_t v = 1; v < V; v++)
        if (h[v] > h[am]) am = v;

    if (tau == 0.0f) {
        *token = am;
        *logprob = (float)lp[am];
        *threshold = NAN;
        *gap = INFINITY;
        *near_tie = 0;
        return;
    }

    /* [ISSUE] top-ratio filter: keep ids whose h is >= the k-th largest */
    float thr = dso_kth_largest(h, V, top_k);
    uint32_t tkey = dso_order_key(thr);

    /* [ISSUE] Gumbel-max over the kept ids */
    int32_t best = -1;
    double z1 = -INFINITY, z2 = -INFINITY;
    for (int32_t v = 0; v < V; v++) {
        if (dso_order_key(h[v]) < tkey) continue;
        double G = dso_gumbel(dso_noise_word(seed, request_id, iteration, row, t, v));
        double z = (double)h[v] / (double)tau + G;
        if (best < 0 || z > z1) {
            if (best >= 0) z2 = z1;
            z1 = z;
            best = v;
        } else if (z > z2) {
            z2 = z;
        }
    }
    *token = best;
    *logprob = (float)lp[best];
    *threshold = thr;
    *gap = z1 - z2;
    double scale = fabs(z1) > 1.0 ? fabs(z1) : 1.0;
    *near_tie = (z1 - z2) < 1e-5 * scale;
}

/* --------------------------------------------------------- sampler call */

/* [PR] The whole call for a list of cells.  c, u: [rows, P, V] (dtype DSO_F32 or
 * DSO_BF16); u may be NULL iff every guidance scale is 0.  Request r covers the
 * packed positions [off_r, off_r + seq_lens[r]) in argument order; cell index is
 * row * P + p.  Outputs are indexed like `cells`.  Returns 0 on success. */
int dso_sample(int dtype, int32_t V, int32_t top_k, const void *c, const void *u, int32_t R,
               const int32_t *seq_lens, const int64_t *request_ids, const int32_t *iterations,
               const float *guidance, const float *temperature, int32_t rows, uint64_t seed,
               const int64_t *cells, int64_t n_cells, int32_t *tokens, float *logprobs,
               float *thresholds, double *gaps, uint8_t *near_tie, float *max_h, double *lse_h) {
    if (V < 1 || R < 1 || rows < 1) return fail("bad sizes");
    if (top_k == 0) top_k = (V + 9) / 10;
    if (top_k < 1 || top_k > V) return fail("bad top_k");
    int64_t P = 0;
    for (int32_t r = 0; r < R; r++) {
        if (seq_lens[r] < 0) return fail("negative seq_len");
        if (guidance[r] != 0.0f && u == NULL) return fail("u missing");
        if (!(temperature[r] >= 0.0f) || isinf(temperature[r])) return fail("bad temperature");
        if (!isfinite(guidance[r])) return fail("bad guidance");
        P += seq_lens[r];
    }
    float *h = (float *)malloc(sizeof(float) * (size_t)V);
    double *lp = (double *)malloc(sizeof(double) * (size_t)V);
    double *work = (double *)malloc(sizeof(double) * 2 * (size_t)V);
    double *hd = (double *)malloc(sizeof(double) * (size_t)V);
    int rc = 0;
    for (int64_t i = 0; i < n_cells && rc == 0; i++) {
        int64_t cell = cells[i];
        if (cell < 0 || cell >= (int64_t)rows * P) {
            rc = fail("cell out of range");
            break;
        }
        int32_t row = (int32_t)(cell / P);
        int64_t p = cell % P;
        int32_t r = 0;
        int64_t off = 0;
        while (p >= off + seq_lens[r]) off += seq_lens[r++];
        int32_t t = (int32_t)(p - off);
        float s = guidance[r];
        int64_t base = cell * (int64_t)V;
        for (int32_t v = 0; v < V; v++) {
            float cv = load_elem(c, dtype, base + v);
            float uv = (s != 0.0f) ? load_elem(u, dtype, base + v) : 0.0f;
            if (!check_inputs(cv, uv, s)) {
                rc = fail("unsupported non-finite logit");
                break;
            }
            h[v] = dso_guided_logit(cv, uv, s);
        }
        if (rc) break;
        const void *c_row = (dtype == DSO_BF16) ? (const void *)((const uint16_t *)c + base)
                                                : (const void *)((const float *)c + base);
        const void *u_row = NULL;
        if (s != 0.0f)
            u_row = (dtype == DSO_BF16) ? (const void *)((const uint16_t *)u + base)
                                        : (const void *)((const float *)u + base);
        rc = dso_row_logprobs(dtype, c_row, u_row, s, V, lp, work);
        if (rc) break;
        sample_cell(h, lp, V, top_k, temperature[r], seed, request_ids[r], iterations[r], row, t,
                    &tokens[i], &logprobs[i], &thresholds[i], &gaps[i], &near_tie[i]);
        if (max_h || lse_h) {
            float m = -INFINITY;
            for (int32_t v = 0; v < V; v++) {
                hd[v] = (double)h[v];
                if (h[v] > m) m = h[v];
            }
            if (max_h) max_h[i] = m;
            if (lse_h) lse_h[i] = lse_d(hd, V);
        }
    }
    free(h);
    free(lp);
    free(work);
    free(hd);
    return rc;
}

/* ------------------------------------------------ autoregressive mode */

/* binary32 -> bf16 rounded to nearest, ties to the even pattern.  The two
 * candidates are the bf16 values on either side (the upper half of the pattern,
 * and that plus one unit in the last place, away from zero); the nearer one is
 * taken, distances measured exactly in binary64.  Past the largest finite bf16
 * the next pattern is infinity, whose distance is that of 2^128 (an unbounded
 * exponent), so only values from the largest finite plus half a unit round to
 * it.  Infinities map to themselves; NaN is not an input. */
uint16_t dso_f32_to_bf16(float f) {
    uint32_t b = bits_from_f32(f);
    if ((b & 0x7FFFFFFFu) >= 0x7F800000u) return (uint16_t)(b >> 16);
    uint32_t lo = b & 0xFFFF0000u, hi = lo + 0x10000u;
    double vlo = (double)f32_from_bits(lo);
    double vhi = ((hi & 0x7FFFFFFFu) == 0x7F800000u) ? copysign(ldexp(1.0, 128), (double)f)
                                                        : (double)f32_from_bits(hi);
    double dlo = fabs((double)f - vlo), dhi = fabs(vhi - (double)f);
    if (dlo < dhi) return (uint16_t)(lo >> 16);
    if (dhi < dlo) return (uint16_t)(hi >> 16);
    return ((lo >> 16) & 1u) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);
}

/* [ISSUE] repetition penalty of the autoregressive sampler (reading: the
 * multiplicative penalty, see the header). */
float dso_penalized(float x, float theta) { return x > 0.0f ? x / theta : x * theta; }

/* In place over n_rows rows of V logits: every id whose bit is set in the row's
 * seen mask (bit v & 31 of word v >> 5, ceil(V / 32) words per row; bits past V
 * ignored) takes the penalised value of its row's theta (finite, > 0). */
int dso_repetition_penalty(int dtype, int32_t V, void *logits, const uint32_t *seen,
                           const float *theta, int64_t n_rows) {
    if (V < 1 || n_rows < 0) return fail("bad sizes");
    int64_t W = ((int64_t)V + 31) / 32;
    for (int64_t i = 0; i < n_rows; i++) {
        if (!(theta[i] > 0.0f) || isinf(theta[i])) return fail("bad penalty");
        for (int32_t v = 0; v < V; v++) {
            if (!((seen[i * W + (v >> 5)] >> (v & 31)) & 1u)) continue;
            int64_t at = i * (int64_t)V + v;
            float x = load_elem(logits, dtype, at);
            if (isnan(x) || x == INFINITY) return fail("unsupported non-finite logit");
            float y = dso_penalized(x, theta[i]);
            if (dtype == DSO_BF16)
                ((uint16_t *)logits)[at] = dso_f32_to_bf16(y);
            else
                ((float *)logits)[at] = y;
        }
    }
    return 0;
}

/* ---------------------------------------------------- draft greedy path */

/* [DRAFT] per-chunk triple: (max, log-sum-exp, smallest argmax) over the ids of
 * one contiguous vocabulary chunk.  An empty chunk is the identity
 * (-inf, -inf, INT32_MAX). */
typedef struct {
    double m;
    double lse;
    int32_t id;
} dso_triple;

static dso_triple chunk_triple(const void *x_row, int dtype, int32_t lo, int32_t hi,
                               double *work) {
    dso_triple tr = {-INFINITY, -INFINITY, INT32_MAX};
    if (hi <= lo) return tr;
    for (int32_t v = lo; v < hi; v++) {
        float xv = load_elem(x_row, dtype, v);
        work[v - lo] = (double)xv;
        if (tr.id == INT32_MAX || xv > (float)tr.m) {
            tr.m = xv;
            tr.id = v;
        }
    }
    tr.lse = lse_d(work, hi - lo);
    return tr;
}

/* [DRAFT] merge of two triples: larger max wins, equal maxima keep the smaller
 * id, log-sum-exps add in probability space. */
static dso_triple merge(dso_triple a, dso_triple b) {
    dso_triple r;
    if (a.m > b.m || (a.m == b.m && a.id < b.id)) {
        r.m = a.m;
        r.id = a.id;
    } else {
        r.m = b.m;
        r.id = b.id;
    }
    double hi = a.lse > b.lse ? a.lse : b.lse;
    double lo = a.lse > b.lse ? b.lse : a.lse;
    r.lse = (hi == -INFINITY) ? -INFINITY : hi + log1p(exp(lo - hi));
    return r;
}

void dso_merge_triples(const double *a, const double *b, double *out) {
    dso_triple x = {a[0], a[1], (int32_t)a[2]}, y = {b[0], b[1], (int32_t)b[2]};
    dso_triple r = merge(x, y);
    out[0] = r.m;
    out[1] = r.lse;
    out[2] = (double)r.id;
}

/* [DRAFT] greedy draft path over n_rows rows of V logits.  token = smallest
 * argmax, lse = full-vocabulary log-sum-exp, logprob = x[token] - lse.
 * With n_chunks >= 1 the row is cut into contiguous chunks of ceil(V / n_chunks)
 * ids (the last may be shorter or empty); the per-chunk triples are written to
 * triples[(j * n_rows + i) * 3 + {0,1,2}] when triples != NULL, and token / lse
 * come from folding the chunk triples with `merge` in chunk order.  The dense
 * values (one chunk) are written to dense_token / dense_lse when non-NULL. */
int dso_greedy_lse(int dtype, int32_t V, const void *x, const int64_t *rows, int64_t n_rows,
                   int32_t n_chunks, int32_t *token, double *lse, double *logprob,
                   double *triples, int32_t *dense_token, double *dense_lse) {
    if (V < 1 || n_chunks < 1) return fail("bad sizes");
    double *work = (double *)malloc(sizeof(double) * (size_t)V);
    int64_t L = ((int64_t)V + n_chunks - 1) / n_chunks;
    for (int64_t i = 0; i < n_rows; i++) {
        const void *row = (dtype == DSO_BF16)
                              ? (const void *)((const uint16_t *)x + rows[i] * (int64_t)V)
                              : (const void *)((const float *)x + rows[i] * (int64_t)V);
        for (int32_t v = 0; v < V; v++) {
            float xv = load_elem(row, dtype, v);
            if (isnan(xv) || xv == INFINITY) {
                free(work);
                return fail("unsupported non-finite logit");
            }
        }
        dso_triple acc = {-INFINITY, -INFINITY, INT32_MAX};
        for (int32_t j = 0; j < n_chunks; j++) {
            int64_t lo = (int64_t)j * L, hi = lo + L;
            if (lo > V) lo = V;
            if (hi > V) hi = V;
            dso_triple tr = chunk_triple(row, dtype, (int32_t)lo, (int32_t)hi, work);
            if (triples) {
                double *o = triples + ((int64_t)j * n_rows + i) * 3;
                o[0] = tr.m;
                o[1] = tr.lse;
                o[2] = (double)tr.id;
            }
            acc = merge(acc, tr);
        }
        token[i] = acc.id;
        lse[i] = acc.lse;
        logprob[i] = (double)load_elem(row, dtype, acc.id) - acc.lse;
        if (dense_token || dense_lse) {
            dso_triple d = chunk_triple(row, dtype, 0, V, work);
            if (dense_token) dense_token[i] = d.id;
            if (dense_lse) dense_lse[i] = d.lse;
        }
    }
    free(work);
    return 0;
}

/* ---------------------------------------------------- confidence reveal */

/* The step after the sampler on the issue page ([ISSUE], comment on the API
 * shape): every position of a request is scored by a confidence, and the caller
 * commits the reveal_count best, as a top-k over the request's [C, T] scores
 * flattened row-major (f = c * T + t).  Order: the larger score first; equal
 * scores keep the smaller flattened index first ([DRAFT]'s smallest-id rule,
 * applied to this decision as to every other). */
typedef struct {
    float s;
    int64_t f;
} dso_ranked;

static int cmp_ranked(const void *pa, const void *pb) {
    const dso_ranked *a = (const dso_ranked *)pa, *b = (const dso_ranked *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->f < b->f) ? -1 : (a->f > b->f);
}

/* scores: [C, P] row-major with the requests packed along positions in argument
 * order; reveal[r] in [0, C * seq_lens[r]].  Writes sum(reveal) entries, request
 * by request in argument order: the flattened index and the score of each
 * revealed cell, best first. */
int dso_reveal_topk(const float *scores, int32_t C, int64_t P, const int32_t *seq_lens,
                    const int32_t *reveal, int32_t R, int64_t *idx_out, float *val_out) {
    int64_t off = 0, out = 0;
    for (int32_t r = 0; r < R; r++) {
        const int64_t T = seq_lens[r];
        const int64_t n = (int64_t)C * T;
        if (T < 0 || off + T > P) return fail("seq_lens exceed the positions of scores");
        if (reveal[r] < 0 || reveal[r] > n) return fail("reveal count outside [0, C * T]");
        dso_ranked *buf = (dso_ranked *)malloc(sizeof(dso_ranked) * (size_t)(n > 0 ? n : 1));
        if (!buf) return fail("out of memory");
        for (int32_t c = 0; c < C; c++) {
            for (int64_t t = 0; t < T; t++) {
                const float s = scores[(int64_t)c * P + off + t];
                if (isnan(s)) {
                    free(buf);
                    return fail("NaN score");
                }
                buf[c * T + t].s = s;
                buf[c * T + t].f = c * T + t;
            }
        }
        qsort(buf, (size_t)n, sizeof(dso_ranked), cmp_ranked);
        for (int32_t j = 0; j < reveal[r]; j++) {
            idx_out[out + j] = buf[j].f;
            val_out[out + j] = buf[j].s;
        }
        out += reveal[r];
        off += T;
        free(buf);
    }
    return 0;
}

/* ------------------------------------------- array forms (test helpers) */

/* Loops over the functions above, for checks that need millions of values:
 * Philox blocks of the counters (ctr[0] + i, ctr[1], ctr[2], ctr[3]),
 * i = 0 .. n - 1 (the first word wraps modulo 2^32), four words each. */
void dso_philox_range(const uint32_t ctr[4], const uint32_t key[2], int64_t n, uint32_t *out) {
    for (int64_t i = 0; i < n; i++) {
        uint32_t c[4] = {ctr[0] + (uint32_t)i, ctr[1], ctr[2], ctr[3]};
        dso_philox4x32_10(c, key, out + 4 * i);
    }
}

/* Noise words of ids v0 .. v0 + n - 1 of one cell. */
void dso_noise_words(uint64_t seed, int64_t request_id, int32_t iteration, int32_t row, int32_t t,
                     int32_t v0, int64_t n, uint32_t *out) {
    for (int64_t i = 0; i < n; i++)
        out[i] = dso_noise_word(seed, request_id, iteration, row, t, v0 + (int32_t)i);
}

/* Gumbel values of n noise words. */
void dso_gumbel_array(const uint32_t *x, int64_t n, double *out) {
    for (int64_t i = 0; i < n; i++) out[i] = dso_gumbel(x[i]);
}
