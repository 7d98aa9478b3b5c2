"""Seeded synthetic workloads shaped like the pages' sampling steps.

The shapes come from the diffusion-sampler pages (mstar issue "Sampler support for
discrete diffusion" and PR "Add a sampler resource for discrete diffusion": logits
``[rows, positions, vocab]`` packed across requests, ragged per-request lengths around a
target length of 100, batches of 8 to 64 requests) and from the LightLLM page "perf:
avoid full-vocab all-gather for draft greedy sampling" (a 248320-entry vocabulary in
bf16, split four ways).  The value distributions (normal with a stated standard
deviation, +8 spikes, planted ties at the row maximum) are synthetic stand-ins for
real model logits; no checkpoint or dataset is involved.

Determinism: every array is a function of the workload's integer seed only.  Large
tensors are drawn in fixed blocks of rows, each from its own child of a
``numpy.random.SeedSequence``, so the result does not depend on how many threads
draw them.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Callable, Dict, Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

# elements per independently seeded block of a large tensor
_BLOCK_ELEMS = 1 << 22


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """Encode float32 values as bf16 bit patterns, rounding to nearest even.

    Inputs are finite or infinite (no NaN handling is needed for generated data).
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    # +/-inf must stay inf: 0x7F800000 + 0x7FFF does not carry into the sign.
    return (rounded >> np.uint32(16)).astype(np.uint16)


def _normal_f32(seq: np.random.SeedSequence, n: int, sigma: float) -> np.ndarray:
    """n i.i.d. N(0, sigma) float32 draws, block-seeded so threads do not matter."""
    nblocks = max(1, -(-n // _BLOCK_ELEMS))
    children = seq.spawn(nblocks)
    out = np.empty(n, dtype=np.float32)

    def fill(i: int) -> None:
        lo = i * _BLOCK_ELEMS
        hi = min(n, lo + _BLOCK_ELEMS)
        g = np.random.Generator(np.random.PCG64(children[i]))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        out[lo:hi] *= np.float32(sigma)

    workers = min(nblocks, int(os.environ.get("DS_SYNTH_THREADS", "0")) or (os.cpu_count() or 1), 16)
    if workers <= 1 or nblocks == 1:
        for i in range(nblocks):
            fill(i)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nblocks)))
    return out


def _distinct_ids(g: np.random.Generator, n_cells: int, vocab: int, count: int) -> np.ndarray:
    """Per cell, `count` (<= 3) distinct ids drawn uniformly from [0, vocab)."""
    assert 1 <= count <= 3 and vocab >= count
    a = g.integers(0, vocab, n_cells)
    ids = [a]
    if count >= 2:
        b = g.integers(0, vocab - 1, n_cells)
        b = b + (b >= a)
        ids.append(b)
    if count >= 3:
        lo = np.minimum(ids[0], ids[1])
        hi = np.maximum(ids[0], ids[1])
        c = g.integers(0, vocab - 2, n_cells)
        c = c + (c >= lo)
        c = c + (c >= hi)
        ids.append(c)
    return np.stack(ids, axis=1)


@dataclass
class DiffusionWorkload:
    """Inputs of one `ds_sample` call.

    c, u: ``[rows, positions, vocab]``; float32 values for dtype "f32", bf16 bit
    patterns (uint16) for dtype "bf16".  ``u`` is None when every request has
    guidance scale 0.  Rows of requests with guidance 0 hold NaN in ``u`` so that a
    kernel that read them would be caught.
    """

    name: str
    dtype: str
    vocab: int
    rows: int
    seq_lens: np.ndarray
    request_ids: np.ndarray
    iterations: np.ndarray
    guidance: np.ndarray
    temperature: np.ndarray
    c: np.ndarray
    u: Optional[np.ndarray]
    top_k: int
    seed: int
    vocab_chunks: int = 1
    notes: Dict[str, str] = field(default_factory=dict)

    @property
    def positions(self) -> int:
        return int(self.seq_lens.sum())

    @property
    def cells(self) -> int:
        return self.rows * self.positions

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def algorithmic_bytes(self) -> int:
        """Minimum HBM traffic of one call: c for every cell, u only where the
        request's guidance scale is non-zero, plus 8 output bytes per cell."""
        eb = self.elem_bytes
        pos_with_u = int(self.seq_lens[self.guidance != 0].sum())
        return (self.cells * self.vocab * eb
                + self.rows * pos_with_u * self.vocab * eb
                + self.cells * 8)


@dataclass
class DraftWorkload:
    """Inputs of one `ds_greedy_lse` call: logits ``[n_rows, vocab]``."""

    name: str
    dtype: str
    vocab: int
    logits: np.ndarray
    vocab_chunks: int = 1
    tie_rows: Optional[np.ndarray] = None
    notes: Dict[str, str] = field(default_factory=dict)

    @property
    def n_rows(self) -> int:
        return int(self.logits.shape[0])

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def algorithmic_bytes(self) -> int:
        """Logits once, plus token, lse and logprob (12 bytes) per row."""
        return self.n_rows * self.vocab * self.elem_bytes + self.n_rows * 12


def diffusion(name: str, *, seed: int, vocab: int, rows: int, seq_lens,
              dtype: str = "bf16", sigma: float = 3.0, guidance=2.0, temperature=0.9,
              spikes: bool = False, spike_value: float = 8.0, top_k: int = 0,
              sample_seed: int = 42, vocab_chunks: int = 1, iterations=0,
              nan_unread_u: bool = True, masked_ids=()) -> DiffusionWorkload:
    """General diffusion-step workload.

    Draw order: per-request scalars are given by the caller (or drawn by the
    named builders before calling this); then c, then u, then spikes.
    ``guidance`` / ``temperature`` / ``iterations`` are scalars or per-request arrays.
    ``masked_ids``: vocabulary ids whose c and u are set to -inf in every cell.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32).reshape(-1)
    R = seq_lens.size
    P = int(seq_lens.sum())
    guidance = np.broadcast_to(np.asarray(guidance, dtype=np.float32), (R,)).copy()
    temperature = np.broadcast_to(np.asarray(temperature, dtype=np.float32), (R,)).copy()
    iterations = np.broadcast_to(np.asarray(iterations, dtype=np.int32), (R,)).copy()
    request_ids = (1000 + np.arange(R)).astype(np.int64)

    root = np.random.SeedSequence(seed)
    s_c, s_u, s_extra = root.spawn(3)
    n = rows * P * vocab
    c = _normal_f32(s_c, n, sigma).reshape(rows, P, vocab)
    need_u = bool(np.any(guidance != 0))
    u = _normal_f32(s_u, n, sigma).reshape(rows, P, vocab) if need_u else None

    if spikes:
        g = np.random.Generator(np.random.PCG64(s_extra))
        cells = rows * P
        nspk = g.integers(1, 4, cells)
        ids = _distinct_ids(g, cells, vocab, 3)
        cf = c.reshape(cells, vocab)
        uf = u.reshape(cells, vocab) if u is not None else None
        for j in range(3):
            sel = np.nonzero(nspk > j)[0]
            cf[sel, ids[sel, j]] += np.float32(spike_value)
            if uf is not None:
                uf[sel, ids[sel, j]] += np.float32(spike_value)

    for mid in masked_ids:
        c[:, :, mid] = -np.inf
        if u is not None:
            u[:, :, mid] = -np.inf

    if dtype == "bf16":
        c = bf16_from_f32(c)
        u = bf16_from_f32(u) if u is not None else None
        nan = BF16_NAN
    elif dtype == "f32":
        nan = np.float32(np.nan)
    else:
        raise ValueError(dtype)

    if u is not None and nan_unread_u:
        offs = np.concatenate([[0], np.cumsum(seq_lens)])
        for r in range(R):
            if guidance[r] == 0:
                u[:, offs[r]:offs[r + 1], :] = nan

    if top_k == 0:
        top_k = (vocab + 9) // 10
    return DiffusionWorkload(name=name, dtype=dtype, vocab=vocab, rows=rows,
                             seq_lens=seq_lens, request_ids=request_ids,
                             iterations=iterations, guidance=guidance,
                             temperature=temperature, c=c, u=u, top_k=top_k,
                             seed=sample_seed, vocab_chunks=vocab_chunks)


def tiny(temperature: float = 0.9) -> DiffusionWorkload:
    """One request, 2 rows x 16 positions, V=1024, fp32 N(0,2) from seed 0,
    guidance 2.0; temperature 0 (greedy) or 0.9 (top-ratio + Gumbel)."""
    return diffusion(f"tiny_t{temperature:g}", seed=0, vocab=1024, rows=2, seq_lens=[16],
                     dtype="f32", sigma=2.0, guidance=2.0, temperature=temperature)


def omnivoice(n_requests: int = 8, seed: int = 1) -> DiffusionWorkload:
    """OmniVoice-shaped masked-diffusion step: 8 requests, 8 codebook rows, ragged
    lengths uniform in [80, 120] (target length about 100), V=1025 bf16, N(0,3) plus
    1-3 spikes of +8 per cell (same ids in c and u), guidance 2.0, temperature 0.9."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    seq_lens = g.integers(80, 121, n_requests)
    return diffusion("omnivoice", seed=seed, vocab=1025, rows=8, seq_lens=seq_lens,
                     dtype="bf16", sigma=3.0, guidance=2.0, temperature=0.9, spikes=True)


def mixed(n_requests: int = 64, seed: int = 2) -> DiffusionWorkload:
    """Mixed-guidance batch: 64 requests, 8 rows, lengths uniform in [50, 200],
    V=1025 bf16; a seeded half of the requests have guidance 0 (their u rows are
    NaN and must never be read), the rest 2.0; temperature per request drawn from
    {0, 0.7, 0.9, 1.2}."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    seq_lens = g.integers(50, 201, n_requests)
    perm = g.permutation(n_requests)
    guidance = np.full(n_requests, 2.0, dtype=np.float32)
    guidance[perm[: n_requests // 2]] = 0.0
    temperature = g.choice(np.array([0.0, 0.7, 0.9, 1.2], dtype=np.float32), n_requests)
    return diffusion("mixed", seed=seed, vocab=1025, rows=8, seq_lens=seq_lens,
                     dtype="bf16", sigma=3.0, guidance=guidance, temperature=temperature,
                     spikes=True)


def stress(positions: int = 2048, seed: int = 4, vocab_chunks: int = 4) -> DiffusionWorkload:
    """Large-vocabulary chunked stress: 2048 positions (one request, one row),
    V=248320 bf16 c and u N(0,4), guidance 1.5, temperature 1.0, k=24832, four
    contiguous vocabulary chunks."""
    return diffusion("stress", seed=seed, vocab=248320, rows=1, seq_lens=[positions],
                     dtype="bf16", sigma=4.0, guidance=1.5, temperature=1.0,
                     vocab_chunks=vocab_chunks)


def draft(n_rows: int = 256, vocab: int = 248320, seed: int = 3, vocab_chunks: int = 1,
          dtype: str = "bf16", sigma: float = 4.0, tie_fraction: float = 0.1) -> DraftWorkload:
    """Greedy draft path: n_rows x V bf16 logits N(0,4); ceil(0.1 n_rows) seeded rows
    get their maximum copied to 1-3 further random ids (2-4 tied maxima)."""
    root = np.random.SeedSequence(seed)
    s_x, s_tie = root.spawn(2)
    x = _normal_f32(s_x, n_rows * vocab, sigma).reshape(n_rows, vocab)
    g = np.random.Generator(np.random.PCG64(s_tie))
    n_tie = int(math.ceil(tie_fraction * n_rows))
    tie_rows = np.sort(g.choice(n_rows, n_tie, replace=False)) if n_tie else np.zeros(0, np.int64)
    for r in tie_rows:
        extra = int(g.integers(1, 4))
        ids = g.choice(vocab, extra, replace=False)
        x[r, ids] = x[r].max()
    logits = bf16_from_f32(x) if dtype == "bf16" else x
    return DraftWorkload(name="draft", dtype=dtype, vocab=vocab, logits=logits,
                         vocab_chunks=vocab_chunks, tie_rows=tie_rows)


@dataclass
class RevealWorkload:
    """Confidence scores [C, P] packed like the sampler's outputs, and how many
    cells each request reveals."""
    name: str
    scores: np.ndarray        # float32 [C, P]
    seq_lens: np.ndarray      # int32 [R]
    reveal_counts: np.ndarray  # int32 [R]

    @property
    def rows(self) -> int:
        return int(self.scores.shape[0])

    @property
    def positions(self) -> int:
        return int(self.scores.shape[1])

    def algorithmic_bytes(self) -> int:
        """Scores read once, one (index, score) pair written per revealed cell."""
        return int(self.scores.size * 4 + 8 * int(self.reveal_counts.sum()))


def reveal(n_requests: int = 8, rows: int = 8, seed: int = 5, lo: int = 80, hi: int = 120,
           committed: float = 1.0 / 3.0, ratio: float = 0.1, grid: float = 16.0,
           name: str = "reveal") -> RevealWorkload:
    """Confidence reveal after an OmniVoice-shaped step: ragged lengths uniform in
    [lo, hi], scores shaped like log-probabilities (-|N(0, 2)| rounded to 1/grid,
    so equal scores occur), a seeded fraction of cells already committed (-inf),
    and ceil(ratio * C * T_r) cells revealed per request."""
    root = np.random.SeedSequence([seed, 11])
    s_len, s_val, s_mask = root.spawn(3)
    g = np.random.Generator(np.random.PCG64(s_len))
    seq_lens = g.integers(lo, hi + 1, n_requests).astype(np.int32)
    P = int(seq_lens.sum())
    vals = -np.abs(_normal_f32(s_val, rows * P, 2.0))
    vals = (np.round(vals * grid) / grid).astype(np.float32).reshape(rows, P)
    gm = np.random.Generator(np.random.PCG64(s_mask))
    vals[gm.random((rows, P)) < committed] = -np.inf
    counts = np.ceil(ratio * rows * seq_lens).astype(np.int32)
    return RevealWorkload(name=name, scores=vals, seq_lens=seq_lens, reveal_counts=counts)


@dataclass
class ARWorkload:
    """Inputs of one autoregressive step: logits ``[R, vocab]`` (one row per
    request), seen-token masks ``[R, ceil(vocab / 32)]`` (bit v & 31 of word
    v >> 5), and per-request penalty, temperature, iteration and id."""
    name: str
    dtype: str
    vocab: int
    logits: np.ndarray
    seen: np.ndarray          # uint32 [R, W]
    penalty: np.ndarray       # float32 [R]
    temperature: np.ndarray   # float32 [R]
    iterations: np.ndarray    # int32 [R]
    request_ids: np.ndarray   # int64 [R]
    top_k: int
    seed: int

    @property
    def rows(self) -> int:
        return int(self.logits.shape[0])

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def n_seen(self) -> int:
        V = self.vocab
        ids = np.arange(V)
        bits = (self.seen[:, ids >> 5] >> (ids & 31).astype(np.uint32)) & np.uint32(1)
        return int(bits.sum())

    def algorithmic_bytes(self) -> int:
        """Masks read once, each seen logit read and written, the logits read once
        by the sampler, and token plus logprob (8 bytes) per request."""
        return int(self.seen.size * 4 + 2 * self.n_seen() * self.elem_bytes
                   + self.rows * self.vocab * self.elem_bytes + self.rows * 8)


def ar(n_requests: int = 256, vocab: int = 248320, seed: int = 6, dtype: str = "bf16",
       sigma: float = 4.0, seen_lo: int = 256, seen_hi: int = 1280, top_share: float = 0.25,
       penalty: float = 1.1, temperatures=(0.0, 0.7, 1.0), top_k: Optional[int] = None,
       name: str = "ar") -> ARWorkload:
    """Autoregressive step: R rows of N(0, sigma) logits; each request has seen
    between seen_lo and seen_hi distinct tokens (the pages' serving setting of 256
    input and up to 1024 output tokens), a top_share of them drawn from the row's
    50 largest logits (repeated tokens are likely ones) and the rest uniform;
    penalty theta for every request; temperatures cycled over the requests;
    top_k = vocab (no top-ratio filter) unless given."""
    root = np.random.SeedSequence([seed, 13])
    s_x, s_seen = root.spawn(2)
    x = _normal_f32(s_x, n_requests * vocab, sigma).reshape(n_requests, vocab)
    g = np.random.Generator(np.random.PCG64(s_seen))
    W = (vocab + 31) // 32
    seen = np.zeros((n_requests, W), dtype=np.uint32)
    for r in range(n_requests):
        n = int(g.integers(min(seen_lo, vocab), min(seen_hi, vocab) + 1))
        n_top = min(int(round(top_share * n)), 50, vocab)
        top = np.argpartition(-x[r], n_top - 1)[:n_top] if n_top > 0 else np.zeros(0, np.int64)
        picked = set(int(v) for v in g.choice(top, n_top, replace=False)) if n_top else set()
        rest = g.choice(vocab, n, replace=False)
        for v in rest:
            if len(picked) >= n:
                break
            picked.add(int(v))
        ids = np.fromiter(picked, dtype=np.int64)
        np.bitwise_or.at(seen[r], ids >> 5, (np.uint32(1) << (ids & 31).astype(np.uint32)))
    logits = bf16_from_f32(x) if dtype == "bf16" else x
    temps = np.array([temperatures[r % len(temperatures)] for r in range(n_requests)], np.float32)
    return ARWorkload(name=name, dtype=dtype, vocab=vocab, logits=logits, seen=seen,
                      penalty=np.full(n_requests, penalty, np.float32), temperature=temps,
                      iterations=np.full(n_requests, 7, np.int32),
                      request_ids=(2000 + np.arange(n_requests)).astype(np.int64),
                      top_k=vocab if top_k is None else top_k, seed=42)


WORKLOADS: Dict[str, Callable[[], object]] = {
    "tiny_greedy": lambda: tiny(0.0),
    "tiny_sampled": lambda: tiny(0.9),
    "omnivoice": omnivoice,
    "mixed": mixed,
    "draft": draft,
    "stress": stress,
    "reveal": reveal,
    "ar": ar,
}
