"""Independent recomputation of the oracle's near-tie classification.

The sampled-token parity bar excuses a cell only when the oracle's best and
second-best perturbed scores over the kept ids differ by less than
1e-5 * max(1, |z1|).  This module recomputes that classification from pieces
pinned elsewhere: the Philox noise word (published known-answer vectors and
rocRAND's host implementation) and the Gumbel map (scipy's quantile).  The kept
set, the scores z = h / tau + G, the best z1, the runner-up z2, the gap and the
flag are all recomputed here in Python double, with none of the oracle's code.

Two kinds of cells are used:
  - random rows at small V over several temperatures and top-ratio sizes (about
    1200 cells: the flag is almost always clear there, and the gaps spread over
    several orders of magnitude);
  - constructed races: two ids whose scores differ by a chosen multiple of the
    band (0.3x to 3x, on both sides of it), with the runner-up placed before and
    after the winner, exact ties, and scores far from zero where the band is
    relative (|z1| of about 100 to 1000).
"""

from __future__ import annotations

import numpy as np

import oracle

BAND = 1e-5
SEED = 0x5EED_0001_2345


def _keys(h: np.ndarray) -> np.ndarray:
    b = h.astype(np.float32).view(np.uint32).astype(np.uint64)
    neg = (b >> np.uint64(31)) & np.uint64(1)
    return np.where(neg == 1, np.uint64(0xFFFFFFFF) - b, b | np.uint64(0x80000000))


def recompute_cell(h: np.ndarray, tau: float, top_k: int, rid: int, it: int, row: int, t: int,
                   noise_lib=None):
    """(token, z1, z2, gap, near_tie) of one sampled cell, by definition: the kept
    ids are those whose order key is at least the top_k-th largest key; each kept
    id scores h / tau + G with G = -log(-log U) of its noise word; the winner is
    the largest score, the smaller id on exact ties; z2 is the best score of the
    other kept ids (-inf when only one id is kept)."""
    V = h.size
    keys = _keys(h)
    tkey = np.sort(keys)[::-1][top_k - 1]
    kept = np.flatnonzero(keys >= tkey)
    z = np.array([float(h[v]) / float(np.float32(tau)) +
                  oracle.gumbel(oracle.noise_word(SEED, rid, it, row, t, int(v), lib=noise_lib),
                                lib=noise_lib) for v in kept])
    order = sorted(range(kept.size), key=lambda i: (-z[i], kept[i]))
    z1 = z[order[0]]
    z2 = z[order[1]] if kept.size > 1 else -np.inf
    gap = z1 - z2
    near = bool(gap < BAND * max(1.0, abs(z1)))
    assert V == h.size
    return int(kept[order[0]]), z1, z2, gap, near


def _random_cells(rng):
    """(c rows [n, V] float32, tau, top_k) for several random batches."""
    out = []
    for tau, k, V, n, sigma in ((1.0, 16, 16, 400, 2.0), (0.5, 4, 16, 300, 2.0),
                                (2.0, 3, 12, 300, 1.0), (0.05, 8, 16, 200, 0.2)):
        out.append(((rng.normal(size=(n, V)) * sigma).astype(np.float32), tau, k))
    return out


def _constructed_cells(noise_lib=None):
    """Races of two ids (a winner w and a runner-up r) at a chosen gap, every other
    id far below.  Returns (c rows, tau, intended gap / band)."""
    V = 8
    rows, ratios = [], []
    tau = 1.0
    specs = []
    for scale in (1.0, 100.0, 1000.0):  # |z1| about 1, 100 and 1000: the band is relative
        for ratio in (0.3, 0.7, 0.9, 0.97, 1.03, 1.1, 1.5, 3.0, 0.0):
            for w, r in ((0, 5), (6, 2)):  # runner-up after and before the winner
                specs.append((scale, ratio, w, r))
    for t, (scale, ratio, w, r) in enumerate(specs):
        G = [oracle.gumbel(oracle.noise_word(SEED, 1, 0, 0, t, v, lib=noise_lib), lib=noise_lib)
             for v in range(V)]
        c = np.full(V, -1e4 if scale < 1000 else -1e5, np.float32)
        c[w] = np.float32(scale)
        z1 = float(c[w]) / tau + G[w]
        band = BAND * max(1.0, abs(z1))
        # z_r = z1 - ratio * band, rounded through binary32 h
        c[r] = np.float32((z1 - ratio * band - G[r]) * tau)
        rows.append(c)
        ratios.append(ratio)
    return np.stack(rows), tau, np.array(ratios)


def check(lib=None, noise_lib=None):
    """Raise AssertionError when the oracle `lib` classifies any cell differently
    from the recomputation, or when its reported gap or token differs.  Returns
    (cells checked, near ties found, constructed cells on each side of the band)."""
    rng = np.random.default_rng(77)
    checked = near_total = 0
    batches = [(c, tau, k, False) for c, tau, k in _random_cells(rng)]
    cc, ctau, ratios = _constructed_cells(noise_lib)
    batches.append((cc, ctau, cc.shape[1], True))
    below = above = 0
    for c, tau, k, constructed in batches:
        n, V = c.shape
        res = oracle.sample(c=c.reshape(1, n, V), u=None, seq_lens=[n], request_ids=[1], iterations=[0],
                            guidance=[0.0], temperature=[tau], rows=1, seed=SEED, top_k=k, lib=lib)
        for t in range(n):
            tok, z1, z2, gap, near = recompute_cell(c[t], tau, k, 1, 0, 0, t, noise_lib)
            assert res.tokens[t] == tok, ("token", t, res.tokens[t], tok)
            assert bool(res.near_tie[t]) == near, ("near_tie", t, res.gaps[t], gap, z1)
            if np.isfinite(gap):
                assert abs(res.gaps[t] - gap) <= 1e-12 * max(1.0, abs(z1)), ("gap", t, res.gaps[t], gap)
            else:
                assert res.gaps[t] == gap
            if constructed:
                band = BAND * max(1.0, abs(z1))
                if near and gap > 0.5 * band:
                    below += 1
                if not near and gap < 2.0 * band:
                    above += 1
            near_total += near
        checked += n
    # the constructed races really straddle the band: cells just inside and just
    # outside it on every scale
    assert below >= 6 and above >= 6, (below, above)
    return checked, near_total, (below, above)
