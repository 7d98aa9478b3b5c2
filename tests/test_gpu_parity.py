"""GPU parity: the HIP sampler (through the C ABI) against the CPU oracle.

Every case prints what it runs before launching, so a failure names its case.
Bars are stated in tests/gpu_helpers.py.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import (check_greedy, check_reveal, check_sample, log, oracle_threaded, run_greedy, run_reveal,
                         run_sample, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    torch.cuda.init()


# ------------------------------------------------------- the five workloads

@pytest.mark.parametrize("tau", [0.0, 0.9])
def test_tiny_step_all_cells(tau):
    w = synth.tiny(tau)
    got = run_sample(w)
    check_sample(w, got, oracle.sample_workload(w))


def test_omnivoice_step_all_cells():
    w = synth.omnivoice()
    ref = oracle.sample_workload(w)
    got = run_sample(w)
    check_sample(w, got, ref)
    # asking for the threshold does not change the draw
    got2 = run_sample(w, threshold=False)
    assert np.array_equal(got[0], got2[0]) and np.array_equal(got[1], got2[1])


def test_mixed_guidance_batch_all_cells():
    w = synth.mixed()
    assert np.any(w.guidance == 0) and w.u is not None
    ref = oracle.sample_workload(w)
    got = run_sample(w)
    rep = check_sample(w, got, ref)
    assert rep.greedy > 0 and rep.sampled > 0
    # the production call (no threshold output): unguided sampled cells narrow
    # the top-ratio set with a histogram and race it without the threshold
    got2 = run_sample(w, threshold=False)
    check_sample(w, got2, ref)
    assert np.array_equal(got[0], got2[0]) and np.array_equal(got[1], got2[1])


@pytest.mark.parametrize("chunks", [1, 4])
def test_draft_greedy_full_size(chunks):
    x = synth.draft().logits
    ref = oracle.greedy_lse(x, vocab_chunks=chunks)
    got = run_greedy(x, chunks)
    check_greedy(x, got, ref, f"draft chunks={chunks}")
    w = synth.draft()
    # planted ties resolve to the smallest id
    for r in w.tie_rows:
        row = oracle.bf16_to_f32(x[r])
        assert got[0][r] == int(np.flatnonzero(row == row.max())[0])


def test_stress_small_positions_dense_chunked_and_fallback():
    w = synth.stress(positions=24)
    ref = oracle.sample_workload(w)
    got4 = run_sample(w)
    check_sample(w, got4, ref)
    got1 = run_sample(w, vocab_chunks=1)
    check_sample(w, got1, ref)
    gotf = run_sample(w, force_fallback=True)
    check_sample(w, gotf, ref)
    assert np.array_equal(got1[0], got4[0]) and np.array_equal(gotf[0], got4[0])


def test_stress_full_size_sampled_cells_and_chunk_equality():
    import torch

    # the full 2048 x 248320 chunked stress step, in the production launch (4
    # chunks) with and without the threshold output, and dense
    w = synth.stress()
    c = to_dev(w.c)
    u = to_dev(w.u)
    got4t = run_sample(w, c_dev=c, u_dev=u, threshold=True)
    got4 = run_sample(w, c_dev=c, u_dev=u, threshold=False)
    got1 = run_sample(w, c_dev=c, u_dev=u, threshold=False, vocab_chunks=1)
    del c, u
    torch.cuda.empty_cache()
    # the four-chunk result equals the dense single-pass result in every cell, and
    # asking for the threshold changes no draw (its parts kernel adds the exp-sum
    # in another order, so the logprobs agree to rounding)
    assert np.array_equal(got4[0], got1[0])
    assert np.max(np.abs(got4[1] - got1[1])) <= 1e-5
    assert np.array_equal(got4t[0], got4[0])
    assert np.max(np.abs(got4t[1] - got4[1])) <= 1e-5
    # 256 evenly spaced cells against the oracle: tokens, logprobs and the
    # top-ratio threshold (k = ceil(0.1 * V) = 24832) bit for bit
    cells = np.linspace(0, w.cells - 1, 256).astype(np.int64)
    ref = oracle_threaded(w, cells)
    check_sample(w, got4t, ref, check_threshold=True)
    check_sample(w, got4, ref, check_threshold=False)


# ------------------------------------------------------------ edge cases

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 2, 3, 63, 64, 65, 127, 129, 1000, 2046])
def test_small_vocab_sizes(V, dtype):
    seq = [3, 0, 5, 2]
    for k in sorted({1, max(1, V // 3), V}):
        w = synth.diffusion(f"V{V}_k{k}", seed=V + k, vocab=V, rows=3, seq_lens=seq, dtype=dtype,
                            sigma=2.0, guidance=[2.0, 1.0, 0.0, -0.5],
                            temperature=[0.9, 0.3, 1.5, 0.0], top_k=k)
        check_sample(w, run_sample(w), oracle.sample_workload(w))


@pytest.mark.parametrize("dtype,V", [("bf16", 3000), ("bf16", 4096 + 7), ("f32", 5000)])
def test_row_kernel_mid_vocab(dtype, V):
    w = synth.diffusion(f"row_{dtype}_{V}", seed=V, vocab=V, rows=2, seq_lens=[5, 4], dtype=dtype,
                        sigma=3.0, guidance=[2.0, 0.0], temperature=[1.0, 0.0])
    ref = oracle.sample_workload(w)
    for chunks in (1, 3, 8):
        check_sample(w, run_sample(w, vocab_chunks=chunks), ref)
    check_sample(w, run_sample(w, force_fallback=True), ref)


@pytest.mark.parametrize("dtype,V,chunks", [("bf16", 3000, 1), ("bf16", 4103, 3), ("f32", 5000, 2),
                                             ("bf16", 60000, 4)])
def test_row_kernel_race_without_threshold(dtype, V, chunks):
    # the production path: the parts' Gumbel race decides the token and the
    # threshold is never located
    w = synth.diffusion(f"race_{dtype}_{V}", seed=V + 11, vocab=V, rows=2, seq_lens=[4, 3], dtype=dtype,
                        sigma=4.0, guidance=[1.5, 0.0], temperature=[1.0, 0.7], vocab_chunks=chunks)
    check_sample(w, run_sample(w, threshold=False), oracle.sample_workload(w))


def test_row_kernel_extreme_top_k_and_negative_guidance():
    # top_k = 1 (only the argmax is kept: the race can never certify) and top_k = V
    # (every id kept: the race always certifies), with a negative guidance scale
    # and masked ids, where a -inf c with a finite u also gives a NaN before the fix
    V = 6000
    for k in (1, V):
        w = synth.diffusion(f"row_k{k}", seed=40 + k, vocab=V, rows=2, seq_lens=[3, 2], sigma=3.0,
                            guidance=[-0.5, 1.5], temperature=[0.8, 1.3], top_k=k, vocab_chunks=3,
                            masked_ids=[7, 4000])
        ref = oracle.sample_workload(w)
        for thr in (False, True):
            check_sample(w, run_sample(w, threshold=thr), ref)


def test_row_kernel_flat_rows_take_the_exact_path():
    # nearly flat h at a high temperature: every id can still win, far more than
    # top_k of them, so the merge must locate the threshold itself
    w = synth.diffusion("flat", seed=21, vocab=8000, rows=1, seq_lens=[6], sigma=0.3, guidance=0.5,
                        temperature=1.5)
    ref = oracle.sample_workload(w)
    for thr in (False, True):
        check_sample(w, run_sample(w, threshold=thr), ref)


def test_row_kernel_flat_rows_kept_and_dropped_race_winners():
    # flat rows queue more than top_k ids; the race's winner (the oracle's token
    # with top_k = V, the same noise) is inside the top-ratio set at some cells
    # and outside it at others, so both ends of the merge's decision are taken
    kw = dict(seed=22, vocab=8000, rows=1, seq_lens=[40], sigma=0.6, guidance=0.5, temperature=1.2)
    w = synth.diffusion("flat_kept", **kw)
    ref = oracle.sample_workload(w)
    free = oracle.sample_workload(synth.diffusion("flat_all", top_k=8000, **kw))
    kept = ref.tokens == free.tokens
    assert kept.any() and not kept.all(), int(kept.sum())
    for thr in (False, True):
        check_sample(w, run_sample(w, threshold=thr), ref)


def test_row_kernel_small_temperature_and_masked_ids():
    # |h / tau| near 1e5 (the pruning bounds' relative margin) and masked ids
    # with guidance on, where c - u is (-inf) - (-inf)
    w = synth.diffusion("row_tau", seed=23, vocab=20000, rows=2, seq_lens=[3, 3], sigma=4.0, guidance=2.0,
                        temperature=[1e-3, 0.05], masked_ids=[0, 5, 19999], vocab_chunks=2)
    ref = oracle.sample_workload(w)
    for thr in (False, True):
        got = run_sample(w, threshold=thr)
        check_sample(w, got, ref)
        assert not np.isin(got[0], [0, 5, 19999]).any()


def test_row_kernel_threshold_bin_overflow():
    # every h lies in [0.9, 1.3): the threshold's first 11-bit key digit is shared
    # by far more ids than the select keeps in LDS, so its last two digits take
    # passes over the row; bf16 values tie heavily at the threshold
    w = synth.diffusion("bin_overflow", seed=31, vocab=30000, rows=1, seq_lens=[3], sigma=0.05, guidance=0.0,
                        temperature=1.0, top_k=3000)
    w.c = synth.bf16_from_f32(oracle.bf16_to_f32(w.c) + np.float32(1.1))
    ref = oracle.sample_workload(w)
    for thr in (False, True):
        check_sample(w, run_sample(w, threshold=thr), ref)
    check_sample(w, run_sample(w, force_fallback=True), ref)


def test_row_kernel_threshold_sample_misses_a_hidden_cluster():
    # the long-row select brackets the threshold from a sample of runs of 512
    # ids; here the largest ids sit in runs the sample skips (ids 512..2047), so
    # the bracket lies below the answer and the exact two-pass select must take
    # over; the second position, without the cluster, takes the bracket
    V = 30000
    w = synth.diffusion("hidden_cluster", seed=44, vocab=V, rows=1, seq_lens=[2], sigma=1.0, guidance=0.0,
                        temperature=1.0, top_k=1000)
    x = oracle.bf16_to_f32(w.c)
    x[0, 0, 512:2048] += np.float32(10.0)
    w.c = synth.bf16_from_f32(x)
    ref = oracle.sample_workload(w)
    for thr in (False, True):
        check_sample(w, run_sample(w, threshold=thr), ref)


def test_threshold_window_edge_rows_at_full_vocabulary():
    # V = 248320 in four chunks with the threshold output: each row's threshold
    # comes from the keys its parts collected inside a window bracketing it, or,
    # when the window misses or overflows its buffer, from the exact passes over
    # the row.  In one launch: ordinary rows, a row of heavy exact ties (the
    # window holds far more keys than its buffer), a row with all but 8320 ids
    # masked (threshold -inf), a constant row (threshold = maximum) and a row
    # whose largest ids hide in runs the window's sample skips.
    V, P = 248320, 7
    w = synth.diffusion("window_edges", seed=77, vocab=V, rows=1, seq_lens=[P], sigma=4.0, guidance=1.5,
                        temperature=1.0, top_k=24832, vocab_chunks=4)
    c = oracle.bf16_to_f32(w.c)
    u = oracle.bf16_to_f32(w.u)
    rng = np.random.default_rng(5)
    c[0, 1] = rng.integers(0, 3, V).astype(np.float32)  # values 0, 1, 2: massive ties
    u[0, 1] = c[0, 1]
    masked = rng.permutation(V)[: V - 8320]
    c[0, 2, masked] = -np.inf
    u[0, 2, masked] = -np.inf
    c[0, 3] = 1.25
    u[0, 3] = 0.5
    c[0, 5, 512:4096] += np.float32(60.0)  # ids 512..4095, skipped by a 1-in-33 run sample
    w.c = synth.bf16_from_f32(c)
    w.u = synth.bf16_from_f32(u)
    ref = oracle.sample_workload(w)
    assert np.isneginf(ref.thresholds[2]) and ref.thresholds[3] == ref.max_h[3]
    for thr in (True, False):
        check_sample(w, run_sample(w, threshold=thr), ref)
    check_sample(w, run_sample(w, force_fallback=True), ref)


def test_row_kernel_many_parts_per_row():
    # 4 positions x 4 chunks: each chunk is cut into several parts, each running
    # its own race
    w = synth.stress(positions=4)
    ref = oracle.sample_workload(w)
    for thr in (False, True):
        check_sample(w, run_sample(w, threshold=thr), ref)


def test_threshold_windows_over_several_launches():
    # 2500 cells on the streaming path with the threshold output: the handle's
    # window buffers hold 2048 rows, so the call is two launches whose window
    # kernels, parts and merges reuse the same window slots; every cell against
    # the oracle, thresholds bit for bit.  V = 65536 bf16 is long enough for the
    # window's sample (every fifth run of 512 ids), so every sampled row has one.
    w = synth.diffusion("windows_2500", seed=91, vocab=65536, rows=2, seq_lens=[700, 0, 550], sigma=3.0,
                        guidance=[1.5, 0.0, 2.0], temperature=[1.0, 0.8, 0.0], top_k=6554)
    assert w.cells == 2500
    ref = oracle_threaded(w, np.arange(w.cells, dtype=np.int64))
    check_sample(w, run_sample(w, threshold=True), ref)
    check_sample(w, run_sample(w, threshold=False), ref, check_threshold=False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunks", [1, 3])
def test_threshold_window_masked_ids(dtype, chunks):
    # rows long enough for the threshold window (V = 65536, a sample of runs
    # spread over the row), guided and not, with masked ids (c and u -inf, so the
    # guided h is NaN before it is taken as -inf) at the row's start, inside it
    # and at its end, inside sampled runs and outside them
    w = synth.diffusion(f"window_{dtype}", seed=93, vocab=65536, rows=2, seq_lens=[5, 4], dtype=dtype, sigma=3.0,
                        guidance=[1.5, 0.0], temperature=[1.0, 0.7], vocab_chunks=chunks,
                        masked_ids=[0, 11, 30000, 40961, 65535])
    ref = oracle.sample_workload(w)
    for thr in (True, False):
        check_sample(w, run_sample(w, threshold=thr), ref)
    check_sample(w, run_sample(w, force_fallback=True), ref)


def test_masked_ids_stay_masked():
    V = 1025
    w = synth.diffusion("masked", seed=5, vocab=V, rows=4, seq_lens=[30, 20], sigma=3.0,
                        guidance=[2.0, 0.0], temperature=[0.9, 1.2], masked_ids=[0, 17, 1024])
    ref = oracle.sample_workload(w)
    got = run_sample(w)
    check_sample(w, got, ref)
    assert not np.isin(got[0], [0, 17, 1024]).any()
    gotf = run_sample(w, force_fallback=True)
    check_sample(w, gotf, ref)


def test_heavy_ties_and_extreme_top_k():
    V = 1025
    for k, tau in ((1, 1.0), (103, 0.9), (1025, 2.0), (500, 50.0), (103, 1e-3)):
        w = synth.diffusion(f"ties_k{k}", seed=k, vocab=V, rows=2, seq_lens=[40], sigma=2.0,
                            guidance=0.0, temperature=tau, top_k=k)
        # snap logits to a coarse grid so thresholds and maxima tie
        f = oracle.bf16_to_f32(w.c)
        w.c = synth.bf16_from_f32(np.round(f * 2) / 2)
        ref = oracle.sample_workload(w)
        check_sample(w, run_sample(w), ref)
        check_sample(w, run_sample(w, threshold=False), ref)
        check_sample(w, run_sample(w, force_fallback=True), ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_flat_rows_histogram_narrowing(dtype):
    # Rows where far more than 256 ids can still win take the histogram
    # narrowing in the wave-per-cell kernel: guidance 0 with wide temperatures,
    # top_k from 1 to 500, a coarse grid that piles ties into the threshold's bin
    # (its top set can pass the list and fall back to the exact search), and rows
    # of one repeated value at a tiny temperature, whose range the histogram
    # cannot resolve.  Each runs with and without the threshold output.
    V = 1025
    cases = [(103, [0.7, 1.2, 5.0], 3.0, None), (1, [2.0], 3.0, None), (500, [1.5, 40.0], 3.0, None),
             (103, [3.0], 2.0, 0.5), (103, [1e-30, 1e-3], 0.0, None)]
    for k, taus, sigma, grid in cases:
        R = len(taus)
        w = synth.diffusion(f"flat_{dtype}_k{k}_s{sigma}", seed=k + R, vocab=V, rows=2, seq_lens=[24] * R,
                            dtype=dtype, sigma=max(sigma, 1.0), guidance=0.0, temperature=taus, top_k=k)
        f = oracle.bf16_to_f32(w.c) if dtype == "bf16" else w.c.copy()
        if sigma == 0.0:
            f[:] = 1.25  # every id ties with the maximum
        elif grid:
            f = np.round(f / grid) * grid
        w.c = synth.bf16_from_f32(f) if dtype == "bf16" else f.astype(np.float32)
        ref = oracle.sample_workload(w)
        # constant rows at temperatures of 1e-30 and 1e-3 score |z1| >= 1250, so
        # the relative band (>= 1.25e-2) holds every kept id's noise difference
        # at tau = 1e-30 (scores are h / tau to within 1e-29 relative) and most of
        # them at 1e-3: every sampled cell may be a near tie there
        bound = w.cells if sigma == 0.0 else None
        got = run_sample(w)
        check_sample(w, got, ref, max_near_ties=bound)
        got2 = run_sample(w, threshold=False)
        check_sample(w, got2, ref, max_near_ties=bound)
        assert np.array_equal(got[0], got2[0])


def test_many_requests_span_several_launches():
    rng = np.random.default_rng(3)
    R = 150
    seq = rng.integers(0, 6, R)
    w = synth.diffusion("many", seed=9, vocab=1025, rows=2, seq_lens=seq, sigma=3.0,
                        guidance=rng.choice([0.0, 2.0], R), temperature=rng.choice([0.0, 0.9], R),
                        iterations=rng.integers(0, 1000, R))
    check_sample(w, run_sample(w), oracle.sample_workload(w))


def test_guidance_zero_everywhere_needs_no_u():
    w = synth.diffusion("no_u", seed=4, vocab=1025, rows=2, seq_lens=[10, 7], guidance=0.0,
                        temperature=[0.9, 0.0])
    assert w.u is None
    check_sample(w, run_sample(w), oracle.sample_workload(w))


def test_unaligned_views_and_side_stream():
    import torch

    import vocab_wise_logit_amd as ds

    w = synth.diffusion("unaligned", seed=12, vocab=1025, rows=2, seq_lens=[9, 6], sigma=3.0,
                        guidance=2.0, temperature=0.9)
    n = w.c.size
    cbuf = torch.zeros(n + 1, dtype=torch.int16, device="cuda")
    ubuf = torch.zeros(n + 1, dtype=torch.int16, device="cuda")
    cbuf[1:] = torch.from_numpy(w.c.reshape(-1).view(np.int16)).cuda()
    ubuf[1:] = torch.from_numpy(w.u.reshape(-1).view(np.int16)).cuda()
    c = cbuf[1:].view(torch.bfloat16).view(w.c.shape)
    u = ubuf[1:].view(torch.bfloat16).view(w.u.shape)
    ref = oracle.sample_workload(w)
    check_sample(w, run_sample(w, c_dev=c, u_dev=u), ref)
    check_sample(w, run_sample(w, c_dev=c, u_dev=u, force_fallback=True), ref)
    side = torch.cuda.Stream()
    with ds.Sampler(w.vocab, "bf16", max_rows=2, max_positions=w.positions) as smp:
        with torch.cuda.stream(side):
            tok, lp = smp.sample(w.request_ids, c, u, w.seq_lens, w.iterations, w.guidance,
                                 w.temperature, seed=w.seed)
        side.synchronize()
    assert np.array_equal(tok.reshape(-1).cpu().numpy(), ref.tokens)


def test_repeat_calls_are_bitwise_identical():
    w = synth.omnivoice(n_requests=3)
    a = run_sample(w)
    b = run_sample(w)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


@pytest.mark.parametrize("dtype,V,chunks,rows", [("bf16", 2504, 64, 256), ("bf16", 4096, 1, 512),
                                                  ("f32", 1024, 4, 256), ("bf16", 2800, 7, 300)])
def test_greedy_one_workgroup_per_row(dtype, V, chunks, rows):
    # Rows that fill the GPU take one workgroup per row (no merge kernel); the
    # shapes put chunk edges on 16-byte pieces, with a short and an empty last
    # chunk at V=2504 / 64 chunks.  Planted ties straddle chunk edges and masked
    # ids are -inf.  The same data through the parts + merge kernels must give
    # the same ids and chunk maxima.
    rng = np.random.default_rng(V + chunks)
    x = rng.standard_normal((rows, V)).astype(np.float32) * 4
    L = -(-V // chunks)
    for r in range(0, rows, 7):
        e = min(V - 1, L * int(rng.integers(1, max(2, chunks))))
        x[r, e - 1] = x[r, e] = x[r].max() + 1.0  # tie across a chunk edge
    x[::5, 3] = -np.inf
    x[::11, :] = np.round(x[::11, :])  # rows with many equal values
    if dtype == "bf16":
        x = synth.bf16_from_f32(x)
    ref = oracle.greedy_lse(x, vocab_chunks=chunks)
    got = run_greedy(x, chunks)
    check_greedy(x, got, ref, f"rows {dtype} V={V} chunks={chunks} rows={rows}")
    fb = run_greedy(x, chunks, force_fallback=True)
    check_greedy(x, fb, ref, f"parts {dtype} V={V} chunks={chunks} rows={rows}")
    assert np.array_equal(got[0], fb[0])
    assert np.array_equal(got[3][:, :, 0], fb[3][:, :, 0])
    # id words are int32 bit patterns (an empty chunk's INT32_MAX reads as a NaN float)
    assert np.array_equal(got[3][:, :, 2].copy().view(np.int32), fb[3][:, :, 2].copy().view(np.int32))


@pytest.mark.parametrize("V,chunks", [(1, 1), (9, 4), (1025, 7), (1025, 1024), (5000, 3)])
def test_greedy_lse_shapes_and_chunks(V, chunks):
    rng = np.random.default_rng(V)
    for dtype in ("bf16", "f32"):
        x = (rng.integers(-8, 9, (37, V)) * 0.5).astype(np.float32)  # many ties
        if dtype == "bf16":
            x = synth.bf16_from_f32(x)
        ref = oracle.greedy_lse(x, vocab_chunks=chunks)
        check_greedy(x, run_greedy(x, chunks), ref, f"V={V} chunks={chunks} {dtype}")


# ------------------------------------------------------ confidence reveal

def test_reveal_omnivoice_shaped():
    w = synth.reveal()
    check_reveal(w, run_reveal(w))


def test_reveal_ties_edges_and_several_launches():
    # coarse grid (many equal scores at the boundary), empty requests, reveal 0,
    # reveal everything, a single row, and 150 requests over three launches
    rng = np.random.default_rng(12)
    R = 150
    seq = rng.integers(0, 30, R).astype(np.int32)
    seq[:3] = [0, 5, 17]
    C = 3
    scores = (np.round(rng.normal(size=(C, int(seq.sum()))) * 2) / 2).astype(np.float32)
    scores[rng.random(scores.shape) < 0.2] = -np.inf
    k = np.minimum(rng.integers(0, 40, R), C * seq).astype(np.int32)
    k[1] = 0
    k[2] = C * seq[2]
    w = synth.RevealWorkload("reveal_edges", scores, seq, k)
    check_reveal(w, run_reveal(w))
    w1 = synth.reveal(n_requests=5, rows=1, seed=13, name="reveal_one_row")
    check_reveal(w1, run_reveal(w1))


@pytest.mark.parametrize("T,counts", [(400, [1, 3200, 700]), (1500, [12000, 5, 4096]),
                                      (3000, [16384, 1, 12000])])
def test_reveal_largest_sizes(T, counts):
    # 8 x T cells per request: keys held 4 or 16 per thread in registers, or (at
    # 24000 cells) read on every pass; reveal counts up to the 16384 cap
    w = synth.reveal(n_requests=3, rows=8, seed=14 + T, lo=T, hi=T, ratio=0.5, name=f"reveal_{T}")
    w.reveal_counts = np.array(counts, np.int32)
    check_reveal(w, run_reveal(w))


def test_reveal_rejects_bad_counts():
    import torch

    import vocab_wise_logit_amd as ds

    s = torch.zeros((2, 10), dtype=torch.float32, device="cuda")
    # room for every requested slot, so that even an accepted call stays in bounds
    idx = torch.full((16400,), -7, dtype=torch.int32, device="cuda")
    with ds.Sampler(16, "f32", max_rows=2, max_positions=40000, max_requests=4) as smp:
        for seq, k, code in (([4, 6], [9, 1], ds.DS_ERR_INVALID_ARG), ([4, 6], [-1, 1], ds.DS_ERR_INVALID_ARG),
                             ([10], [21], ds.DS_ERR_INVALID_ARG)):
            with pytest.raises(ds.DSError) as e:
                ds.ds_reveal_topk(smp._h, s, 2, seq, k, idx)
            assert e.value.code == code
        big = torch.zeros((2, 20000), dtype=torch.float32, device="cuda")
        with pytest.raises(ds.DSError) as e:
            ds.ds_reveal_topk(smp._h, big, 2, [20000], [16385], idx)
        assert e.value.code == ds.DS_ERR_UNSUPPORTED
        torch.cuda.synchronize()
    assert (idx.cpu() == -7).all()


def test_calls_replay_from_a_captured_graph():
    # ds_sample (both paths) and ds_reveal_topk allocate, synchronise and clear
    # nothing, so a stream capture of them replays; every replay, with eager work
    # in between, must equal the eager result bit for bit
    import torch

    import vocab_wise_logit_amd as ds

    for w in (synth.omnivoice(n_requests=3), synth.stress(positions=6)):
        log(f"[gpu] graph capture {w.name}")
        c = to_dev(w.c)
        u = to_dev(w.u)
        with ds.Sampler(w.vocab, w.dtype, max_rows=w.rows, max_positions=w.positions,
                        max_requests=len(w.seq_lens), vocab_chunks=w.vocab_chunks) as smp:
            ref = [t.clone() for t in smp.sample(w.request_ids, c, u, w.seq_lens, w.iterations, w.guidance,
                                                 w.temperature, seed=w.seed)]
            counts = np.minimum(np.ceil(0.1 * w.rows * w.seq_lens), 16384).astype(np.int32)
            ref_rev = [t.clone() for t in smp.reveal_topk(ref[1], w.seq_lens, counts)]
            out = tuple(torch.empty_like(t) for t in ref) + (None,)
            rev = tuple(torch.empty_like(t) for t in ref_rev)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):  # warm-up on the capture stream
                smp.sample(w.request_ids, c, u, w.seq_lens, w.iterations, w.guidance, w.temperature,
                           seed=w.seed, out=out)
            torch.cuda.current_stream().wait_stream(side)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                smp.sample(w.request_ids, c, u, w.seq_lens, w.iterations, w.guidance, w.temperature,
                           seed=w.seed, out=out)
                smp.reveal_topk(out[1], w.seq_lens, counts, out=rev)
            for rep in range(3):
                for t in out[:2] + rev:
                    t.fill_(-1)
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                for a, b in zip(out[:2] + rev, ref + ref_rev):
                    assert torch.equal(a, b), f"replay {rep} differs from the eager call"
            del g


def test_invalid_calls_are_rejected_before_launch():
    import torch

    import vocab_wise_logit_amd as ds

    w = synth.tiny(0.9)
    c = to_dev(w.c)
    u = to_dev(w.u)
    with ds.Sampler(w.vocab, "f32", max_rows=2, max_positions=16, max_requests=1) as smp:
        tok = torch.full((2, 16), -7, dtype=torch.int32, device="cuda")
        lp = torch.zeros((2, 16), dtype=torch.float32, device="cuda")
        cases = [
            dict(u_logits=None),
            dict(temperature=[-1.0]),
            dict(temperature=[float("nan")]),
            dict(guidance_scale=[float("inf")]),
            dict(seq_lens=[17]),
            dict(seq_lens=[-1]),
            dict(num_rows=3),
        ]
        for bad in cases:
            args = dict(request_ids=w.request_ids, u_logits=u, seq_lens=w.seq_lens,
                        iterations=w.iterations, guidance_scale=w.guidance,
                        temperature=w.temperature, num_rows=2)
            args.update(bad)
            log(f"[gpu] invalid call {bad}")
            # straight to the C entry point (the binding refuses some of these
            # itself, by the tensors' shapes): the library must reject each one
            # before anything is enqueued
            host = [np.ascontiguousarray(args[k], dt) for k, dt in
                    (("request_ids", np.int64), ("seq_lens", np.int32), ("iterations", np.int32),
                     ("guidance_scale", np.float32), ("temperature", np.float32))]
            up = args["u_logits"].data_ptr() if args["u_logits"] is not None else None
            rc = ds.lib().ds_sample(smp._h, host[0].ctypes.data, c.data_ptr(), up, host[1].ctypes.data,
                                    host[2].ctypes.data, host[3].ctypes.data, host[4].ctypes.data,
                                    host[0].size, args["num_rows"], 1, tok.data_ptr(), lp.data_ptr(), None,
                                    torch.cuda.current_stream().cuda_stream)
            assert rc != ds.DS_OK, bad
        # the binding refuses the tensors that do not match the call's sizes
        for bad in (dict(seq_lens=[17]), dict(num_rows=3)):
            args = dict(request_ids=w.request_ids, c_logits=c, u_logits=u, seq_lens=w.seq_lens,
                        iterations=w.iterations, guidance_scale=w.guidance,
                        temperature=w.temperature, num_rows=2, seed=1, tokens_out=tok,
                        logprobs_out=lp)
            args.update(bad)
            with pytest.raises(ValueError):
                ds.ds_sample(smp._h, **args)
        torch.cuda.synchronize()
        assert int((tok == -7).sum()) == tok.numel()  # nothing was written
