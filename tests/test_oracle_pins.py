"""Pins of the CPU oracle against things other than itself.

Each test checks one oracle function against a closed form, a brute-force
computation in a different formulation, an independent library routine
(torch's bf16 widening, scipy's logsumexp and Gumbel quantile, rocRAND's Philox),
a published known-answer vector, or an invariant of the mathematics.  The pages
print no worked example of the sampler; the one number they print that touches
our data layout (the draft path's 48-byte per-token payload) is pinned too.
"""

from __future__ import annotations

import json
import math
import os
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import scipy.stats

import near_tie_pin
import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ helpers

def f32(x) -> np.float32:
    return np.float32(x)


def round_to_f32(q: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) binary32 of an exact rational."""
    approx = np.float32(float(q))  # may be off by one ulp (double rounding)
    best = None
    for cand in (np.nextafter(approx, np.float32(-np.inf)), approx,
                 np.nextafter(approx, np.float32(np.inf))):
        if not np.isfinite(cand):
            continue
        d = abs(Fraction(float(cand)) - q)
        key = (d, int(np.array(cand).view(np.uint32)) & 1)  # tie -> even mantissa
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def bits(x) -> int:
    return int(np.array(x, dtype=np.float32).view(np.uint32))


# ------------------------------------------------------------ bf16 widening

def test_bf16_widening_exhaustive_vs_torch():
    import torch

    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f32(allbits)
    ref = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_encoder_round_trip():
    # the generator's encoder and the oracle's decoder agree on every finite bf16
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_to_f32(allbits)
    fin = np.isfinite(vals)
    assert np.array_equal(synth.bf16_from_f32(vals[fin]), allbits[fin])


# ------------------------------------------------------- guided logit (fp32)

def test_guided_logit_is_one_rounding_of_exact_value():
    rng = np.random.default_rng(11)
    n_double_round_cases = 0
    for i in range(4000):
        c = f32(rng.normal() * 8)
        u = f32(rng.normal() * 8)
        s = f32(rng.choice([2.0, 1.5, 0.3, -0.7, 3.1]) if i % 3 else rng.normal())
        if s == 0:
            continue
        d = f32(c - u)  # one IEEE subtraction, then one rounding of s*d + c
        exact = Fraction(float(s)) * Fraction(float(d)) + Fraction(float(c))
        want = round_to_f32(exact) + f32(0.0)
        got = oracle.guided_logit(float(c), float(u), float(s))
        assert bits(got) == bits(want), (c, u, s)
        two_roundings = f32(f32(s * d) + c)
        n_double_round_cases += bits(two_roundings) != bits(want)
    # the sample must contain cases where a separate multiply and add would differ
    assert n_double_round_cases > 20


def test_guided_logit_special_cases():
    # s == 0: h is c bit for bit, and u is not looked at (NaN / inf allowed)
    for c in (1.25, -3.5, 0.0, 7e-3):
        for u in (np.nan, np.inf, -np.inf, 4.0):
            assert bits(oracle.guided_logit(c, u, 0.0)) == bits(f32(c))
    # -0 is canonicalised to +0
    assert bits(oracle.guided_logit(-0.0, 5.0, 0.0)) == 0
    assert bits(oracle.guided_logit(-0.0, 0.0, 2.0)) == 0
    # s == -1 gives u when c - u is exact
    for c, u in ((3.0, -1.5), (0.25, 8.0), (-6.0, -6.5)):
        assert oracle.guided_logit(c, u, -1.0) == u
    # masked id: c == -inf stays -inf for any s and finite or -inf u
    for s in (2.0, -0.5, 1.5):
        for u in (3.0, -np.inf):
            assert oracle.guided_logit(-np.inf, u, s) == -np.inf


# ------------------------------------------------------------- LSE / logprob

def test_lse_brute_force_and_closed_forms():
    rng = np.random.default_rng(3)
    for V in (1, 2, 5, 16):
        x = rng.uniform(-20, 20, V)
        want = math.log(math.fsum(math.exp(v) for v in x))
        assert abs(oracle.lse(x) - want) < 1e-12 * max(1, abs(want))
    for V in (1, 7, 1024, 248320):
        assert abs(oracle.lse(np.full(V, 2.5)) - (2.5 + math.log(V))) < 1e-9
    # two-level row: n ids at a, the rest at b
    V, n, a, b = 1000, 13, 4.0, -1.0
    x = np.full(V, b)
    x[:n] = a
    want = math.log(n * math.exp(a) + (V - n) * math.exp(b))
    assert abs(oracle.lse(x) - want) < 1e-12
    assert oracle.lse(np.array([-np.inf, -np.inf])) == -np.inf
    assert abs(oracle.lse(np.array([-np.inf, 0.0])) - 0.0) < 1e-15


def _bf16_row(rng, V, sigma):
    return synth.bf16_from_f32((rng.normal(size=V) * sigma).astype(np.float32))


@pytest.mark.parametrize("s", [0.0, 2.0, 1.5, -1.0, 0.37])
def test_row_logprobs_normalised_and_equal_to_h_space(s):
    rng = np.random.default_rng(int(abs(s) * 100) + 5)
    V = 1025
    c = _bf16_row(rng, V, 3.0)
    u = _bf16_row(rng, V, 3.0) if s != 0 else np.full(V, 0x7FC0, np.uint16)  # NaN, unread
    lp = oracle.row_logprobs(c, u if s != 0 else None, s)
    # probabilities sum to one
    assert abs(math.fsum(np.exp(lp)) - 1.0) < 1e-12
    # renormalised CFG on log-softmaxed inputs == log-softmax of (1+s)c - s*u
    cd = oracle.bf16_to_f32(c).astype(np.float64)
    ud = oracle.bf16_to_f32(u).astype(np.float64) if s != 0 else np.zeros(V)
    s32 = float(np.float32(s))  # the oracle takes the scale as binary32
    h64 = (1.0 + s32) * cd - s32 * ud
    want = h64 - scipy.special.logsumexp(h64)
    assert np.max(np.abs(lp - want)) < 1e-9


def test_row_logprobs_brute_force_in_probability_space():
    # guided distribution p_c^(1+s) / p_u^s, renormalised, in pure Python (V <= 16)
    rng = np.random.default_rng(8)
    for V in (2, 3, 8, 16):
        for s in (2.0, 0.5, -0.25, 0.3):
            s = float(np.float32(s))
            c = (rng.normal(size=V) * 2).astype(np.float32)
            u = (rng.normal(size=V) * 2).astype(np.float32)
            zc = math.fsum(math.exp(float(v)) for v in c)
            zu = math.fsum(math.exp(float(v)) for v in u)
            w = [(math.exp(float(a)) / zc) ** (1 + s) / (math.exp(float(b)) / zu) ** s
                 for a, b in zip(c, u)]
            zw = math.fsum(w)
            want = np.array([math.log(x / zw) for x in w])
            got = oracle.row_logprobs(c, u, s)
            assert np.max(np.abs(got - want)) < 1e-10


def test_row_logprobs_closed_forms():
    V = 1024
    c = np.full(V, 1.75, np.float32)
    u = np.full(V, -0.5, np.float32)
    for s in (0.0, 2.0, -1.0):
        lp = oracle.row_logprobs(c, u if s else None, s)
        assert np.max(np.abs(lp + math.log(V))) < 1e-12
    # s == -1 gives the unconditional log-softmax
    rng = np.random.default_rng(2)
    c = rng.normal(size=64).astype(np.float32)
    u = rng.normal(size=64).astype(np.float32)
    lp = oracle.row_logprobs(c, u, -1.0)
    assert np.max(np.abs(lp - (u - scipy.special.logsumexp(u.astype(np.float64))))) < 1e-12
    # masked ids get zero probability, the rest renormalise
    c[[0, 7, 63]] = -np.inf
    u[[0, 7, 63]] = -np.inf
    lp = oracle.row_logprobs(c, u, 2.0)
    assert np.all(np.isneginf(lp[[0, 7, 63]]))
    assert abs(math.fsum(np.exp(lp)) - 1.0) < 1e-12


def test_row_logprobs_rejects_unsupported_values():
    c = np.zeros(4, np.float32)
    u = np.zeros(4, np.float32)
    c[1] = np.nan
    with pytest.raises(ValueError):
        oracle.row_logprobs(c, u, 2.0)
    c[1] = 0
    u[2] = -np.inf  # u masked where c is not
    with pytest.raises(ValueError):
        oracle.row_logprobs(c, u, 2.0)


# ------------------------------------------------------------------- Philox

def test_philox_known_answer_vectors():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for case in kat["cases"]:
        ctr = [int(x, 16) for x in case["counter"]]
        key = [int(x, 16) for x in case["key"]]
        want = [int(x, 16) for x in case["out"]]
        assert list(oracle.philox4x32_10(ctr, key)) == want


def _hipcc():
    for p in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""):
        if p and os.path.exists(p):
            return p
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available to build the rocRAND probe")
def test_philox_matches_rocrand_host_implementation():
    src = os.path.join(os.path.dirname(__file__), "rocrand_philox_probe.cpp")
    rng = np.random.default_rng(99)
    n = 20000
    seeds = rng.integers(0, 2**63, n, dtype=np.uint64) * 2 + rng.integers(0, 2, n).astype(np.uint64)
    c0 = rng.integers(0, 2**32, n, dtype=np.uint64)
    c1 = rng.integers(0, 2**30, n, dtype=np.uint64)
    c2 = rng.integers(0, 2**32, n, dtype=np.uint64)
    c3 = rng.integers(0, 2**32, n, dtype=np.uint64)
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "probe")
        subprocess.run([_hipcc(), "-O1", "-o", exe, src], check=True, capture_output=True)
        inp = "\n".join(f"{a} {b} {c} {e} {f}" for a, b, c, e, f in zip(seeds, c0, c1, c2, c3))
        out = subprocess.run([exe], input=inp, text=True, check=True, capture_output=True).stdout
    ref = np.array([[int(x) for x in line.split()] for line in out.strip().splitlines()],
                   dtype=np.uint64)
    assert ref.shape == (n, 4)
    for i in range(n):
        key = [int(seeds[i]) & 0xFFFFFFFF, int(seeds[i]) >> 32]
        got = oracle.philox4x32_10([c0[i], c1[i], c2[i], c3[i]], key)
        assert list(got) == [int(x) for x in ref[i]], i


def test_noise_word_depends_on_every_key_field():
    base = dict(seed=42, request_id=1000, iteration=3, row=5, t=17, v=1234)
    w0 = oracle.noise_word(**base)
    for field, alt in (("seed", 43), ("seed", 42 + (1 << 32)), ("request_id", 1001),
                       ("iteration", 4), ("row", 6), ("t", 18), ("v", 1235), ("v", 1238)):
        assert oracle.noise_word(**{**base, field: alt}) != w0, field
    # ids sharing v >> 2 come from one Philox call, one word each
    words = [oracle.noise_word(**{**base, "v": 1232 + j}) for j in range(4)]
    full = oracle.philox4x32_10([1232 >> 2, 17, (5 & 0xFFFF) | (3 << 16), 1000], [42, 0])
    assert words == [int(x) for x in full]


def test_array_forms_equal_the_scalar_functions():
    # the array helpers used by the GPU pins are loops over the pinned scalars
    rng = np.random.default_rng(8)
    for _ in range(20):
        ctr = rng.integers(0, 2**32, 4, dtype=np.uint64).astype(np.uint32)
        ctr[0] = np.uint32(0xFFFFFFF0) if _ % 5 == 0 else ctr[0]  # wraps inside the range
        key = rng.integers(0, 2**32, 2, dtype=np.uint64).astype(np.uint32)
        blk = oracle.philox_range(ctr, key, 40)
        for i in (0, 7, 15, 16, 39):
            c = ctr.copy()
            c[0] = np.uint32((int(ctr[0]) + i) & 0xFFFFFFFF)
            assert blk[i].tolist() == oracle.philox4x32_10(c, key).tolist()
    words = oracle.noise_words(42, 1000, 3, 5, 17, 1230, 9)
    assert words.tolist() == [oracle.noise_word(42, 1000, 3, 5, 17, v) for v in range(1230, 1239)]
    xs = rng.integers(0, 2**32, 50, dtype=np.uint64).astype(np.uint32)
    assert oracle.gumbel_array(xs).tolist() == [oracle.gumbel(int(x)) for x in xs]


# ---------------------------------------------------------- uniform / Gumbel

def test_uniform_lattice_and_gumbel_quantile():
    assert oracle.uniform(0) == 2.0 ** -24
    assert oracle.uniform(0xFFFFFFFF) == 1.0 - 2.0 ** -24
    assert oracle.uniform(0x1FF) == 2.0 ** -24          # low 9 bits are dropped
    assert oracle.uniform(0x200) == 3 * 2.0 ** -24
    rng = np.random.default_rng(4)
    xs = rng.integers(0, 2**32, 5000, dtype=np.uint64)
    xs = np.concatenate([xs, np.array([0, 1 << 31, 0xFFFFFFFF, 0xFFFFFE00], np.uint64)])
    for x in xs:
        U = oracle.uniform(int(x))
        ref = scipy.stats.gumbel_r.ppf(U)
        G = oracle.gumbel(int(x))
        assert abs(G - ref) <= 1e-9 * max(1.0, abs(ref)), (x, G, ref)
    # the largest possible noise value, used as an exact pruning bound
    gmax = oracle.gumbel(0xFFFFFFFF)
    assert abs(gmax - 24 * math.log(2)) < 1e-6
    assert oracle.gumbel(0) < -2.8


# ---------------------------------------------------------------- threshold

def test_kth_largest_against_sorting_and_invariants():
    rng = np.random.default_rng(5)
    for V, k in ((1, 1), (10, 1), (10, 10), (1025, 103), (1025, 1), (1025, 1025), (5000, 500)):
        h = (rng.normal(size=V) * 3).astype(np.float32)
        # plant ties straddling the threshold
        if V >= 10:
            h[:4] = h[4]
        t = oracle.kth_largest(h, k)
        want = sorted(h.tolist(), reverse=True)[k - 1]
        assert t == want
        assert np.count_nonzero(h > t) < k <= np.count_nonzero(h >= t)
        if k == 1:
            assert t == h.max()
        if k == V:
            assert t == h.min()
    h = np.array([-np.inf, -np.inf, 1.0, 2.0], np.float32)
    assert oracle.kth_largest(h, 3) == -np.inf


# ------------------------------------------------------ whole sampler cells

def _cells_from_rows(c_rows, u_rows, s, tau, top_k=0, seed=7, V=None):
    """One request whose positions are the given rows (one row of cells)."""
    c_rows = np.asarray(c_rows)
    n, V = c_rows.shape
    c = c_rows.reshape(1, n, V)
    u = None if u_rows is None else np.asarray(u_rows).reshape(1, n, V)
    return oracle.sample(c=c, u=u, seq_lens=[n], request_ids=[1000], iterations=[0],
                         guidance=[s], temperature=[tau], rows=1, seed=seed, top_k=top_k)


def test_greedy_brute_force_with_planted_ties():
    rng = np.random.default_rng(21)
    V = 16
    rows_c, rows_u, want = [], [], []
    for i in range(300):
        c = (rng.integers(-6, 7, V) * 0.5).astype(np.float32)  # coarse grid: many ties
        u = (rng.integers(-6, 7, V) * 0.5).astype(np.float32)
        if i % 3 == 0:
            c[0] = c[V - 1] = 9.0
            u[0] = u[V - 1] = 1.0
        rows_c.append(c)
        rows_u.append(u)
        s = Fraction(2)
        h = [round_to_f32(Fraction(float(a)) + s * Fraction(float(f32(a - b)))) for a, b in zip(c, u)]
        m = max(h)
        want.append(min(v for v in range(V) if h[v] == m))
    res = _cells_from_rows(np.stack(rows_c), np.stack(rows_u), 2.0, 0.0)
    assert res.tokens.tolist() == want
    assert np.all(np.isnan(res.thresholds))


def test_gumbel_max_frequencies_follow_softmax_over_kept_ids():
    V, tau, n = 8, 0.7, 120000
    c = np.array([1.0, 0.5, -0.25, 0.75, 0.0, -1.0, 0.3, 0.9], np.float32)
    rows = np.broadcast_to(c, (n, V))
    for k in (V, 3):
        res = _cells_from_rows(rows, None, 0.0, tau, top_k=k)
        counts = np.bincount(res.tokens, minlength=V)
        kept = np.argsort(-c, kind="stable")[:k]
        p = np.zeros(V)
        p[kept] = scipy.special.softmax(c[kept].astype(np.float64) / tau)
        assert counts[p == 0].sum() == 0
        stat = scipy.stats.chisquare(counts[p > 0], n * p[p > 0])
        assert stat.pvalue > 1e-3, (k, counts, n * p)
        assert np.all(res.thresholds == np.sort(c)[::-1][k - 1])


def test_top_k_one_is_greedy_and_ties_keep_all():
    rng = np.random.default_rng(31)
    V, n = 64, 400
    c = (rng.normal(size=(n, V)) * 2).astype(np.float32)
    res = _cells_from_rows(c, None, 0.0, 1.3, top_k=1)
    assert np.array_equal(res.tokens, np.argmax(c, axis=1))
    # ties at the k-th value are all kept: with k=1 and a 3-way tie at the max,
    # every tied id must be drawn sometimes and no other id ever
    row = np.zeros(V, np.float32)
    row[[0, 21, 42]] = 5.0
    c2 = np.broadcast_to(row, (3000, V))
    res2 = _cells_from_rows(c2, None, 0.0, 1.0, top_k=1)
    assert set(np.unique(res2.tokens).tolist()) == {0, 21, 42}


def test_small_temperature_recovers_greedy():
    rng = np.random.default_rng(41)
    V, n = 256, 300
    c = np.round(rng.normal(size=(n, V)) * 4 * 16) / 16  # grid of 1/16
    c = c.astype(np.float32)
    top2 = np.sort(c, axis=1)[:, -2:]
    ok = (top2[:, 1] - top2[:, 0]) >= 1 / 16
    greedy = _cells_from_rows(c, None, 0.0, 0.0)
    cold = _cells_from_rows(c, None, 0.0, 1e-3)
    assert np.array_equal(cold.tokens[ok], greedy.tokens[ok])


def test_sampled_logprob_is_full_vocab_pre_temperature():
    rng = np.random.default_rng(51)
    V, n, s = 1025, 40, 2.0
    c = _bf16_row(rng, n * V, 3).reshape(n, V)
    u = _bf16_row(rng, n * V, 3).reshape(n, V)
    res = _cells_from_rows(c, u, s, 0.9)
    for i in range(n):
        lp = oracle.row_logprobs(c[i], u[i], s)
        assert res.logprobs[i] == np.float32(lp[res.tokens[i]])
        assert res.thresholds[i] == sorted(
            [oracle.guided_logit(float(a), float(b), s) for a, b in
             zip(oracle.bf16_to_f32(c[i]), oracle.bf16_to_f32(u[i]))], reverse=True)[102]


def test_changing_iteration_or_seed_changes_draws_and_repeats_are_identical():
    w = synth.omnivoice(n_requests=2)
    a = oracle.sample_workload(w)
    b = oracle.sample_workload(w)
    assert np.array_equal(a.tokens, b.tokens)
    w.iterations[:] = 1
    c = oracle.sample_workload(w)
    assert np.mean(a.tokens != c.tokens) > 0.1  # concentrated rows: about 1 - sum(p^2)
    w.iterations[:] = 0
    w.seed = 43
    d = oracle.sample_workload(w)
    assert np.mean(a.tokens != d.tokens) > 0.1


def test_near_tie_flag_and_gap_recomputed_from_pinned_noise():
    # The flag that excuses a sampled cell from token equality, recomputed in
    # Python double from the pinned noise word and Gumbel map: about 1200 random
    # cells plus races built to land just inside and just outside the band, with
    # scores near 1, 100 and 1000 (where the band is relative).
    checked, near, (inside, outside) = near_tie_pin.check()
    assert checked >= 1200
    assert inside >= 6 and outside >= 6
    assert near >= inside


def test_unread_u_rows_may_hold_nan():
    w = synth.mixed(n_requests=6)
    assert np.any(w.guidance == 0) and np.any(w.guidance != 0)
    res = oracle.sample_workload(w)
    assert np.all(np.isfinite(res.logprobs))
    assert np.all(res.logprobs <= 0)


# ------------------------------------------------------ draft path / chunks

@pytest.mark.parametrize("V", [9, 16, 1025])
def test_chunked_triples_fold_to_dense(V):
    rng = np.random.default_rng(V)
    n = 50
    x = (rng.integers(-8, 9, (n, V)) * 0.25).astype(np.float32)  # many ties
    for chunks in sorted({1, 2, 3, 4, 7, V}):
        r = oracle.greedy_lse(x, vocab_chunks=chunks)
        assert np.array_equal(r.token, r.dense_token)
        assert np.array_equal(r.token, np.argmax(x, axis=1))
        assert np.max(np.abs(r.lse - r.dense_lse)) < 1e-12
        assert np.max(np.abs(r.lse - scipy.special.logsumexp(x.astype(np.float64), axis=1))) < 1e-12
        assert np.allclose(r.logprob, x[np.arange(n), r.token] - r.lse, atol=0, rtol=1e-15)
        # each triple is its own chunk's reduction; empty chunks are the identity
        L = -(-V // chunks)
        for j in range(chunks):
            lo, hi = min(j * L, V), min((j + 1) * L, V)
            t = r.triples[j]
            if hi == lo:
                assert np.all(t[:, 0] == -np.inf) and np.all(t[:, 2] == 2**31 - 1)
                continue
            seg = x[:, lo:hi]
            assert np.array_equal(t[:, 0], seg.max(axis=1))
            assert np.array_equal(t[:, 2], lo + np.argmax(seg, axis=1))


def test_triple_merge_algebra():
    rng = np.random.default_rng(77)
    ident = [-np.inf, -np.inf, 2**31 - 1]
    for _ in range(2000):
        a, b, c = ([float(rng.integers(-3, 3)), float(rng.normal()), float(rng.integers(0, 50))]
                   for _ in range(3))
        ab = oracle.merge_triples(a, b)
        ba = oracle.merge_triples(b, a)
        assert ab[0] == ba[0] and ab[2] == ba[2] and abs(ab[1] - ba[1]) < 1e-12
        l = oracle.merge_triples(ab, c)
        r = oracle.merge_triples(a, oracle.merge_triples(b, c))
        assert l[0] == r[0] and l[2] == r[2] and abs(l[1] - r[1]) < 1e-12
        assert list(oracle.merge_triples(a, ident)) == a
        want_lse = scipy.special.logsumexp([a[1], b[1]])
        assert abs(ab[1] - want_lse) < 1e-12
        if a[0] == b[0]:
            assert ab[2] == min(a[2], b[2])


def test_draft_closed_forms_and_ties():
    V = 248320
    x = np.full((3, V), 2.0, np.float32)
    x[1, [5, V - 1]] = 9.0
    x[2, [62079, 62080, 124160]] = 9.0  # straddles chunk boundaries at 4 chunks
    r = oracle.greedy_lse(x, vocab_chunks=4)
    assert r.token.tolist() == [0, 5, 62079]
    assert abs(r.lse[0] - (2.0 + math.log(V))) < 1e-9
    assert abs(r.logprob[0] + math.log(V)) < 1e-9
    bx = synth.bf16_from_f32(x)
    rb = oracle.greedy_lse(bx, vocab_chunks=3)
    assert np.array_equal(rb.token, r.token)


def test_draft_payload_matches_page_figures():
    with open(os.path.join(GOLDEN, "draft_payload.json")) as f:
        g = json.load(f)
    V, ranks = g["vocab"], g["ranks"]
    x = synth.bf16_from_f32(np.zeros((1, V), np.float32))
    assert x[0].nbytes == g["bytes_before"]
    r = oracle.greedy_lse(x, vocab_chunks=ranks)
    words = r.triples.astype(np.float32)  # three 32-bit words per chunk per token
    assert words[:, 0, :].nbytes == g["bytes_after"]
    assert round(g["bytes_before"] / g["bytes_after"], 1) == g["reduction_factor_1dp"]
    assert round(100 * (1 - g["bytes_after"] / g["bytes_before"]), 4) == g["reduction_percent_4dp"]


def test_validation_errors():
    w = synth.tiny(0.9)
    with pytest.raises(ValueError):
        oracle.sample(c=w.c, u=None, seq_lens=w.seq_lens, request_ids=w.request_ids,
                      iterations=w.iterations, guidance=w.guidance, temperature=w.temperature,
                      rows=w.rows, seed=1)
    with pytest.raises(ValueError):
        oracle.sample(c=w.c, u=w.u, seq_lens=w.seq_lens, request_ids=w.request_ids,
                      iterations=w.iterations, guidance=w.guidance, temperature=[-1.0],
                      rows=w.rows, seed=1)
    with pytest.raises(ValueError):
        oracle.sample(c=w.c, u=w.u, seq_lens=w.seq_lens, request_ids=w.request_ids,
                      iterations=w.iterations, guidance=w.guidance, temperature=w.temperature,
                      rows=w.rows, seed=1, top_k=w.vocab + 1)


# ------------------------------------------------------ confidence reveal

def _reveal_case(seed, C, seq, grid):
    rng = np.random.default_rng(seed)
    P = int(np.sum(seq))
    s = (np.round(rng.normal(size=(C, P)) * grid) / grid).astype(np.float32)
    s[rng.random((C, P)) < 0.05] = -np.inf
    return s


def test_reveal_closed_forms():
    # increasing scores in flattened order: the best are the last cells, last first
    C, seq = 3, [4, 0, 5]
    P = sum(seq)
    s = np.zeros((C, P), np.float32)
    off = 0
    for T in seq:
        for c in range(C):
            s[c, off:off + T] = c * T + np.arange(T)
        off += T
    idx, val = oracle.reveal_topk(s, seq, [5, 0, 15])
    assert idx.tolist() == [11, 10, 9, 8, 7] + list(range(14, -1, -1))
    assert val.tolist() == [float(i) for i in idx]
    # equal scores: the smallest flattened indices, in order
    idx, _ = oracle.reveal_topk(np.ones((2, 6), np.float32), [6], [4])
    assert idx.tolist() == [0, 1, 2, 3]
    # a single finite cell among -inf comes first, then -inf cells by index
    s = np.full((2, 3), -np.inf, np.float32)
    s[1, 1] = -7.0
    idx, val = oracle.reveal_topk(s, [3], [3])
    assert idx.tolist() == [4, 0, 1] and val[0] == -7.0 and np.isneginf(val[1:]).all()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_reveal_invariants_with_heavy_ties(seed):
    C, seq = 4, [7, 1, 13, 0, 9]
    s = _reveal_case(seed, C, seq, grid=2)
    rev = [3, 4, 20, 0, 36]
    idx, val = oracle.reveal_topk(s, seq, rev)
    o = off = 0
    for T, k in zip(seq, rev):
        blk = s[:, off:off + T].reshape(-1)  # the request's [C, T] cells, row-major
        sel, sv = idx[o:o + k], val[o:o + k]
        assert len(set(sel.tolist())) == k and (sel >= 0).all() and (sel < C * T).all()
        assert np.array_equal(sv, blk[sel])
        # best first; equal scores in increasing index
        for a in range(k - 1):
            assert sv[a] > sv[a + 1] or (sv[a] == sv[a + 1] and sel[a] < sel[a + 1])
        rest = np.setdiff1d(np.arange(C * T), sel)
        if k and rest.size:
            low = sv.min()
            assert (blk[rest] <= low).all()
            # at the boundary score, every unselected cell comes after every selected one
            tied = rest[blk[rest] == low]
            assert tied.size == 0 or tied.min() > sel[sv == low].max()
        o += k
        off += T


def test_reveal_matches_torch_topk_on_distinct_scores():
    import torch

    rng = np.random.default_rng(9)
    C, seq = 8, [37, 120, 5]
    s = rng.permutation(C * sum(seq)).astype(np.float32).reshape(C, -1)
    rev = [10, 96, 40]
    idx, _ = oracle.reveal_topk(s, seq, rev)
    o = off = 0
    for T, k in zip(seq, rev):
        flat = torch.from_numpy(np.ascontiguousarray(s[:, off:off + T])).flatten()
        want = torch.topk(flat, k).indices.numpy()
        assert np.array_equal(idx[o:o + k], want)
        o += k
        off += T


def test_reveal_rejects_bad_counts_and_nan():
    s = np.zeros((2, 3), np.float32)
    with pytest.raises(ValueError):
        oracle.reveal_topk(s, [3], [7])
    s[0, 1] = np.nan
    with pytest.raises(ValueError):
        oracle.reveal_topk(s, [3], [1])


# ------------------------------------------- autoregressive mode (penalty)

def test_bf16_rounding_matches_torch_on_every_pattern_and_tie():
    import torch

    # every finite upper half with the lower halves just below, at and just above
    # the rounding tie, both signs
    hi = np.arange(0, 0x7F80, dtype=np.uint32)
    lows = np.array([0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    bits = ((hi[:, None] << 16) | lows[None, :]).reshape(-1)
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    f = bits.view(np.float32)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16(f)
    assert np.array_equal(got, want)
    # exact bf16 values and infinities map to themselves
    exact = (hi << 16).view(np.float32)
    assert np.array_equal(oracle.f32_to_bf16(exact), hi.astype(np.uint16))
    assert oracle.f32_to_bf16(np.array([np.inf, -np.inf], np.float32)).tolist() == [0x7F80, 0xFF80]


def test_repetition_penalty_identities_and_closed_forms():
    rng = np.random.default_rng(21)
    V = 1000
    x = synth.bf16_from_f32((rng.normal(size=(5, V)) * 4).astype(np.float32))
    W = (V + 31) // 32
    seen = rng.integers(0, 2**32, (5, W), dtype=np.uint64).astype(np.uint32)
    # theta = 1 and an empty mask leave the row bit for bit
    assert np.array_equal(oracle.repetition_penalty(x, seen, 1.0), x)
    assert np.array_equal(oracle.repetition_penalty(x, np.zeros_like(seen), 1.7), x)
    # theta = 2 is exact in binary32 and bf16 (a power of two): seen positive
    # logits halve, seen negative ones double, unseen ones stay
    out = oracle.repetition_penalty(x, seen, 2.0)
    xf, of = oracle.bf16_to_f32(x), oracle.bf16_to_f32(out)
    bit = ((seen[:, np.arange(V) >> 5] >> (np.arange(V) & 31)) & 1).astype(bool)
    want = np.where(bit, np.where(xf > 0, xf / 2, xf * 2), xf)
    assert np.array_equal(of, want.astype(np.float32))
    # a general theta: one binary32 rounding, then one bf16 rounding (checked with
    # exact rational arithmetic on a few values)
    th = np.float32(1.3)
    out = oracle.repetition_penalty(x[:1], seen[:1], th)
    for v in np.flatnonzero(bit[0])[:40]:
        xv = Fraction(float(xf[0, v]))
        q = xv / Fraction(float(th)) if xv > 0 else xv * Fraction(float(th))
        a = np.float32(float(q))
        cands = [np.nextafter(a, np.float32(-np.inf)), a, np.nextafter(a, np.float32(np.inf))]
        f32 = min(cands, key=lambda y: (abs(Fraction(float(y)) - q), int(np.array(y).view(np.uint32)) & 1))
        assert oracle.bf16_to_f32(out[:1, v:v + 1])[0, 0] == oracle.bf16_to_f32(oracle.f32_to_bf16(f32))[0]
    # float32 logits are penalised without a second rounding
    xf32 = (rng.normal(size=(2, 70)) * 3).astype(np.float32)
    s2 = np.full((2, 3), 0xFFFFFFFF, np.uint32)
    o2 = oracle.repetition_penalty(xf32, s2, th)
    assert np.array_equal(o2, np.where(xf32 > 0, xf32 / th, xf32 * th).astype(np.float32))


def test_repetition_penalty_rejects_bad_theta_and_shapes():
    x = np.zeros((2, 40), np.float32)
    seen = np.zeros((2, 2), np.uint32)
    for bad in (0.0, -1.0, np.inf, np.nan):
        with pytest.raises(ValueError):
            oracle.repetition_penalty(x, seen, bad)
    with pytest.raises(ValueError):
        oracle.repetition_penalty(x, np.zeros((2, 1), np.uint32), 1.5)
