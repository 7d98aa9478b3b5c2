"""The oracle's pins are strong enough to catch plausible mistakes.

Each case copies ``oracle/ds_oracle.c``, plants one mistake by a textual edit
(a dropped term, a wrong sign or index, a transposed operand, an off-by-one),
builds the copy with the same flags into a temporary directory, and asserts that
at least one of the independent checks below fails on it, while all of them pass
on the unmodified oracle.  The mistakes are planted only in these CPU copies.
"""

from __future__ import annotations

import json
import math
import os
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import scipy.stats

import near_tie_pin
import oracle
from oracle.build_oracle import SRC, build

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MUTANTS = {
    "cfg_sign": ("h = fmaf(s, c - u, c);", "h = fmaf(s, u - c, c);"),
    "cfg_drop_lc": ("g = lc + (double)s * (lc - lu);", "g = (double)s * (lc - lu);"),
    "lse_drop_max": ("return m + log(s);", "return log(s);"),
    "philox_mult": ("(uint64_t)0xD2511F53u * (uint64_t)x0", "(uint64_t)0xCD9E8D57u * (uint64_t)x0"),
    "philox_xor": ("^ x1 ^ k0;", "^ x3 ^ k0;"),
    "philox_word": ("return out[(uint32_t)v & 3u];", "return out[0];"),
    "gumbel_sign": ("return -log(-log1p(U - 1.0));", "return log(-log1p(U - 1.0));"),
    "uniform_shift": ("(x >> 9) * 2u + 1u", "(x >> 8) * 2u + 1u"),
    "tau_multiplies": ("(double)h[v] / (double)tau", "(double)h[v] * (double)tau"),
    "kth_off_by_one": ("keys[k - 1]", "keys[k]"),
    "filter_strict": ("if (dso_order_key(h[v]) < tkey) continue;",
                      "if (dso_order_key(h[v]) <= tkey) continue;"),
    "greedy_last_tie": ("if (h[v] > h[am]) am = v;", "if (h[v] >= h[am]) am = v;"),
    "merge_tie_larger": ("(a.m == b.m && a.id < b.id)", "(a.m == b.m && a.id > b.id)"),
    "chunk_floor": ("((int64_t)V + n_chunks - 1) / n_chunks", "(int64_t)V / n_chunks"),
    "bf16_shift": ("return f32_from_bits((uint32_t)b << 16);",
                   "return f32_from_bits((uint32_t)b << 15);"),
    "key_negative": ("return (b & 0x80000000u) ? ~b : (b | 0x80000000u);",
                     "return (b & 0x80000000u) ? b : (b | 0x80000000u);"),
    "sampled_lp_of_argmax": ("*logprob = (float)lp[best];", "*logprob = (float)lp[am];"),
    "no_canonical_zero": ("    return h + 0.0f;\n}", "    return h;\n}"),
    "draft_lp_dense": ("logprob[i] = (double)load_elem(row, dtype, acc.id) - acc.lse;",
                       "logprob[i] = (double)load_elem(row, dtype, acc.id);"),
    "reveal_tie_larger": ("return (a->f < b->f) ? -1 : (a->f > b->f);",
                          "return (a->f > b->f) ? -1 : (a->f < b->f);"),
    "reveal_ascending": ("if (a->s > b->s) return -1;\n    if (a->s < b->s) return 1;",
                         "if (a->s < b->s) return -1;\n    if (a->s > b->s) return 1;"),
    "reveal_flatten_transposed": ("buf[c * T + t].f = c * T + t;", "buf[c * T + t].f = t * C + c;"),
    "reveal_count_short": ("for (int32_t j = 0; j < reveal[r]; j++) {",
                           "for (int32_t j = 0; j + 1 < reveal[r]; j++) {"),
    "penalty_divides_negatives": ("return x > 0.0f ? x / theta : x * theta;", "return x / theta;"),
    "penalty_bit_index": (">> (v & 31)) & 1u", ">> (v & 15)) & 1u"),
    "penalty_word_index": ("seen[i * W + (v >> 5)]", "seen[i * W + (v >> 6)]"),
    "bf16_ties_away": ("return ((lo >> 16) & 1u) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);",
                       "return (uint16_t)(hi >> 16);"),
    "bf16_truncates": ("if (dlo < dhi) return (uint16_t)(lo >> 16);",
                       "if (dlo <= dhi + 1e300) return (uint16_t)(lo >> 16);"),
    # the near-tie classification that excuses sampled cells from token equality
    "near_tie_always": ("*near_tie = (z1 - z2) < 1e-5 * scale;", "*near_tie = 1;"),
    "near_tie_never": ("*near_tie = (z1 - z2) < 1e-5 * scale;", "*near_tie = 0;"),
    "near_tie_wide_band": ("*near_tie = (z1 - z2) < 1e-5 * scale;", "*near_tie = (z1 - z2) < 1e-1 * scale;"),
    "near_tie_absolute_band": ("double scale = fabs(z1) > 1.0 ? fabs(z1) : 1.0;", "double scale = 1.0;"),
    "z2_not_demoted": ("if (best >= 0) z2 = z1;", "if (best >= 0) z2 = z2;"),
    "z2_later_ids_ignored": ("} else if (z > z2) {", "} else if (0 && z > z2) {"),
}


# ------------------------------------------------------------- the checks

def _round_f32(q: Fraction) -> np.float32:
    a = np.float32(float(q))
    cands = [np.nextafter(a, np.float32(-np.inf)), a, np.nextafter(a, np.float32(np.inf))]
    return min(cands, key=lambda x: (abs(Fraction(float(x)) - q),
                                     int(np.array(x).view(np.uint32)) & 1))


def check_guided(lib):
    rng = np.random.default_rng(1)
    for _ in range(300):
        c, u = np.float32(rng.normal() * 8), np.float32(rng.normal() * 8)
        s = np.float32(rng.choice([2.0, 1.5, -0.7]))
        d = np.float32(c - u)
        want = _round_f32(Fraction(float(s)) * Fraction(float(d)) + Fraction(float(c))) + np.float32(0)
        got = np.float32(oracle.guided_logit(float(c), float(u), float(s), lib=lib))
        assert got.view(np.uint32) == want.view(np.uint32)
    z = np.float32(oracle.guided_logit(-0.0, 0.0, 2.0, lib=lib))
    assert z.view(np.uint32) == 0


def check_bf16(lib):
    import torch
    b = np.arange(0, 65536, 97, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f32(b, lib=lib)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok].view(np.uint32), ref[ok].view(np.uint32))


def check_logprobs(lib):
    rng = np.random.default_rng(2)
    for s in (2.0, 0.5):
        c = (rng.normal(size=12) * 2).astype(np.float32)
        u = (rng.normal(size=12) * 2).astype(np.float32)
        h64 = (1 + s) * c.astype(np.float64) - s * u.astype(np.float64)
        want = h64 - scipy.special.logsumexp(h64)
        got = oracle.row_logprobs(c, u, s, lib=lib)
        assert np.max(np.abs(got - want)) < 1e-9
    x = rng.uniform(-5, 5, 9)
    assert abs(oracle.lse(x, lib=lib) - scipy.special.logsumexp(x)) < 1e-12


def check_philox(lib):
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        for case in json.load(f)["cases"]:
            got = oracle.philox4x32_10([int(x, 16) for x in case["counter"]],
                                       [int(x, 16) for x in case["key"]], lib=lib)
            assert [int(x) for x in got] == [int(x, 16) for x in case["out"]]
    full = oracle.philox4x32_10([5, 9, (3 & 0xFFFF) | (2 << 16), 77], [11, 0], lib=lib)
    for j in range(4):
        assert oracle.noise_word(11, 77, 2, 3, 9, 20 + j, lib=lib) == int(full[j])


def check_gumbel(lib):
    rng = np.random.default_rng(3)
    for x in rng.integers(0, 2**32, 200, dtype=np.uint64):
        U = oracle.uniform(int(x), lib=lib)
        assert 0 < U < 1 and abs(U - ((int(x) >> 9) + 0.5) * 2.0**-23) < 1e-15
        assert abs(oracle.gumbel(int(x), lib=lib) - scipy.stats.gumbel_r.ppf(U)) < 1e-9


def check_threshold(lib):
    rng = np.random.default_rng(4)
    h = (rng.normal(size=500) * 3).astype(np.float32)
    for k in (1, 50, 500):
        assert oracle.kth_largest(h, k, lib=lib) == sorted(h.tolist(), reverse=True)[k - 1]


def _run(lib, c_rows, s, tau, top_k=0, u_rows=None):
    n, V = c_rows.shape
    return oracle.sample(c=c_rows.reshape(1, n, V),
                         u=None if u_rows is None else u_rows.reshape(1, n, V),
                         seq_lens=[n], request_ids=[5], iterations=[0], guidance=[s],
                         temperature=[tau], rows=1, seed=3, top_k=top_k, lib=lib)


def check_greedy(lib):
    rng = np.random.default_rng(5)
    c = (rng.integers(-4, 5, (200, 16)) * 0.5).astype(np.float32)
    res = _run(lib, c, 0.0, 0.0)
    assert np.array_equal(res.tokens, np.argmax(c, axis=1))


def check_sampling(lib):
    V, n, tau = 8, 40000, 0.7
    c = np.array([1.0, 0.5, -0.25, 0.75, 0.0, -1.0, 0.3, 0.9], np.float32)
    for k in (8, 3):
        res = _run(lib, np.broadcast_to(c, (n, V)).copy(), 0.0, tau, top_k=k)
        kept = np.argsort(-c, kind="stable")[:k]
        p = np.zeros(V)
        p[kept] = scipy.special.softmax(c[kept].astype(np.float64) / tau)
        cnt = np.bincount(res.tokens, minlength=V)
        assert cnt[p == 0].sum() == 0
        assert scipy.stats.chisquare(cnt[p > 0], n * p[p > 0]).pvalue > 1e-4
    # the returned logprob is the full-vocabulary guided logprob of the drawn token
    rng = np.random.default_rng(6)
    cr = (rng.normal(size=(30, 64)) * 2).astype(np.float32)
    ur = (rng.normal(size=(30, 64)) * 2).astype(np.float32)
    res = _run(lib, cr, 2.0, 1.0, u_rows=ur)
    for i in range(30):
        h64 = 3.0 * cr[i].astype(np.float64) - 2.0 * ur[i].astype(np.float64)
        lp = h64 - scipy.special.logsumexp(h64)
        assert abs(res.logprobs[i] - lp[res.tokens[i]]) < 1e-5


def check_draft(lib):
    rng = np.random.default_rng(7)
    x = (rng.integers(-6, 7, (40, 23)) * 0.25).astype(np.float32)
    for chunks in (1, 4, 7):
        r = oracle.greedy_lse(x, vocab_chunks=chunks, lib=lib)
        assert np.array_equal(r.token, np.argmax(x, axis=1))
        lse = scipy.special.logsumexp(x.astype(np.float64), axis=1)
        assert np.max(np.abs(r.lse - lse)) < 1e-12
        assert np.max(np.abs(r.logprob - (x[np.arange(40), r.token] - lse))) < 1e-12


def check_reveal(lib):
    # increasing scores in flattened order, then all-equal scores, on two requests
    C, seq = 3, [4, 5]
    s = np.zeros((C, 9), np.float32)
    s[:, :4] = np.arange(12, dtype=np.float32).reshape(C, 4)
    s[:, 4:] = 1.0
    idx, val = oracle.reveal_topk(s, seq, [5, 6], lib=lib)
    assert idx.tolist() == [11, 10, 9, 8, 7, 0, 1, 2, 3, 4, 5]
    assert val.tolist() == [11.0, 10.0, 9.0, 8.0, 7.0] + [1.0] * 6
    # a transposed flattening shows on a non-square block
    s2 = np.zeros((2, 3), np.float32)
    s2[0, 2] = 5.0
    assert oracle.reveal_topk(s2, [3], [1], lib=lib)[0].tolist() == [2]


def check_penalty(lib):
    import torch

    # binary32 -> bf16 against torch's conversion, on values around every kind of
    # rounding decision (below, at and above the tie, both signs)
    rng = np.random.default_rng(8)
    hi = rng.integers(0, 0x7F7F, 3000).astype(np.uint32)
    lows = np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    bits = ((hi[:, None] << 16) | lows[None, :]).reshape(-1)
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    f = bits.view(np.float32)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16(f, lib=lib), want)
    # the penalty on hand-computed values: ids 0, 1, 2, 4, 5, 6, 8, 40, 58 and 65
    # seen
    x = np.zeros((1, 70), np.float32)
    x[0, :9] = [2.0, -2.0, 0.0, 3.0, -np.inf, 1.5, -0.75, 5.0, 7.0]
    x[0, 40], x[0, 41], x[0, 58], x[0, 65] = -1.25, 9.0, 4.0, 6.0
    seen = np.zeros((1, 3), np.uint32)
    seen[0, 0] = 0b101110111
    seen[0, 1] = (1 << 8) | (1 << 26)
    seen[0, 2] = (1 << 1) | 0xFFFFFF80  # bits past id 69 are ignored
    out = oracle.repetition_penalty(x, seen, 2.0, lib=lib)
    want = x.copy()
    want[0, :9] = [1.0, -4.0, 0.0, 3.0, -np.inf, 0.75, -1.5, 5.0, 3.5]
    want[0, 40], want[0, 58], want[0, 65] = -2.5, 2.0, 3.0
    assert np.array_equal(out, want)


def check_near_tie(lib):
    near_tie_pin.check(lib=lib, noise_lib=oracle._load())


CHECKS = [check_guided, check_bf16, check_logprobs, check_philox, check_gumbel,
          check_threshold, check_greedy, check_sampling, check_draft, check_reveal, check_penalty,
          check_near_tie]


def _failures(lib):
    bad = []
    for chk in CHECKS:
        try:
            chk(lib)
        except (AssertionError, ValueError) as e:  # noqa: PERF203
            bad.append((chk.__name__, repr(e)[:80]))
    return bad


def test_checks_pass_on_the_oracle():
    assert _failures(oracle._load()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_each_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mut.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.load_variant(build(path, os.path.join(d, f"lib_{name}.so"), ["-w"]))
        assert _failures(lib), f"mutant {name} survived every check"
