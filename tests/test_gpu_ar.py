"""GPU parity of the autoregressive mode: the repetition penalty (in place,
bit-exact against the oracle) and the step that samples one token per request
from the penalised rows (to the bar of the other sampler tests)."""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import (LP_TOL, NEAR_TIE_TALLY, check_near_tie_choice, default_near_tie_bound, log,
                         to_dev)

pytestmark = pytest.mark.gpu

CASES = [
    # (name, R, V, dtype, seen range, temperatures, top_k)
    ("small_bf16", 37, 1025, "bf16", (5, 200), (0.0, 0.7, 1.0), None),
    ("small_bf16_topratio", 21, 1025, "bf16", (5, 200), (0.9,), 103),
    ("row_bf16", 9, 40961, "bf16", (100, 2000), (0.0, 0.8), None),
    ("small_f32", 13, 777, "f32", (1, 100), (0.0, 1.3), None),
    ("row_f32_ragged", 5, 3001, "f32", (10, 300), (0.6,), None),
    # more requests than one wave's table: every request is its own position
    ("many_small_bf16", 150, 1025, "bf16", (5, 100), (0.0, 0.9), None),
    ("many_row_bf16", 90, 8192, "bf16", (50, 500), (0.0, 1.0), None),
    # the large vocabulary with the top-ratio filter: the merge's top-set
    # decision runs on rows the parts penalised
    ("full_vocab_topratio", 24, 248320, "bf16", (256, 1280), (0.0, 0.7, 1.0), 24832),
]


def ar_as_diffusion(w, penalised):
    """The step's sampling half as the diffusion call it equals: one position per
    request, guidance 0, the penalised logits as c."""
    R = penalised.shape[0]
    return synth.DiffusionWorkload(name=f"{w.name}_as_cells", dtype=w.dtype, vocab=w.vocab, rows=1,
                                   seq_lens=np.ones(R, np.int32), request_ids=np.asarray(w.request_ids, np.int64),
                                   iterations=np.asarray(w.iterations, np.int32),
                                   guidance=np.zeros(R, np.float32),
                                   temperature=np.asarray(w.temperature, np.float32),
                                   c=penalised.reshape(1, R, w.vocab), u=None, top_k=w.top_k, seed=w.seed)


def _run(w, smp):
    import torch

    x = to_dev(w.logits)
    seen = torch.from_numpy(w.seen.view(np.int32)).cuda()
    pen = torch.from_numpy(w.penalty).cuda()
    tok, lp = smp.sample_ar(w.request_ids, x, seen, pen, w.iterations, w.temperature, seed=w.seed)
    torch.cuda.synchronize()
    xo = x.view(torch.int16).cpu().numpy().view(np.uint16) if w.dtype == "bf16" else x.cpu().numpy()
    return xo, tok.cpu().numpy(), lp.cpu().numpy()


def _check_against_oracle(w, name, oracle_penalty=None, **sampler_kw):
    """One step through ds_sample_ar, checked against the oracle: penalised logits
    bit for bit, greedy tokens exactly, sampled tokens except bounded near ties
    (which must still draw a kept id inside the band), logprobs to LP_TOL.  The
    oracle takes `oracle_penalty` as the thetas when given."""
    import vocab_wise_logit_amd as ds

    R, V = w.rows, w.vocab
    with ds.Sampler(V, w.dtype, max_rows=1, max_positions=R, max_requests=R, top_k=w.top_k, **sampler_kw) as smp:
        xo, tok, lp = _run(w, smp)
    pen, ref = oracle.ar_step(w if oracle_penalty is None else dataclasses.replace(w, penalty=oracle_penalty))
    assert np.array_equal(xo, pen), "penalised logits differ from the oracle"
    greedy = w.temperature == 0
    near = ref.near_tie.astype(bool) & ~greedy
    sampled = int((~greedy).sum())
    assert near.sum() <= default_near_tie_bound(sampled), f"{int(near.sum())} near ties in {sampled} sampled rows"
    assert np.array_equal(tok[greedy], ref.tokens[greedy])
    bad = np.nonzero(~greedy & ~near & (tok != ref.tokens))[0]
    assert bad.size == 0, f"sampled token mismatch at requests {bad[:10]}"
    # a near-tie row that drew another id drew a kept one within the band
    aw = ar_as_diffusion(w, pen)
    for i in np.nonzero(near & (tok != ref.tokens))[0]:
        check_near_tie_choice(aw, int(i), int(tok[i]), int(ref.tokens[i]), float(ref.thresholds[i]))
    NEAR_TIE_TALLY.append((f"ar_{name}", sampled, int(near.sum()), int((near & (tok != ref.tokens)).sum())))
    same = tok == ref.tokens
    assert np.max(np.abs(lp[same].astype(np.float64) - ref.logprobs[same])) <= LP_TOL
    log(f"[check] ar {name}: greedy={int(greedy.sum())} sampled={sampled} near_ties={int(near.sum())}")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ar_step_matches_oracle(case):
    name, R, V, dt, (lo, hi), temps, top_k = case
    w = synth.ar(n_requests=R, vocab=V, seed=31 + R, dtype=dt, seen_lo=lo, seen_hi=hi, penalty=1.0,
                 temperatures=temps, top_k=top_k, name=name)
    # varied penalties
    w.penalty[:] = np.linspace(0.6, 2.5, R).astype(np.float32)
    log(f"[gpu] ar {name}: R={R} V={V} {dt} seen={w.n_seen()} top_k={w.top_k}")
    _check_against_oracle(w, name)


PROLOGUE_CASES = [
    # (name, R, V, dtype, vocab chunks, force the streaming path)
    ("bf16_3_chunks", 5, 40961, "bf16", 3, False),
    ("f32_4_chunks", 4, 30011, "f32", 4, False),
    ("bf16_7_chunks_top_ratio", 6, 65536, "bf16", 7, False),
    ("bf16_small_row_streamed", 7, 1025, "bf16", 2, True),
]


@pytest.mark.parametrize("case", PROLOGUE_CASES, ids=[c[0] for c in PROLOGUE_CASES])
def test_ar_every_id_seen_is_penalised_once(case):
    """Every id of every row seen, the mask bits past V set too.  On the streaming
    path each part penalises its own ids in place before reading them, so an id
    penalised by two parts, or by none, at a part or chunk edge (ragged V, chunk
    lengths that are not whole 16-byte pieces or mask words) changes the
    penalised logits, which must equal the oracle's bit for bit.  One row's theta
    is not finite and leaves it unchanged."""
    name, R, V, dt, chunks, forced = case
    top_k = (V + 9) // 10 if "top_ratio" in name else None
    w = synth.ar(n_requests=R, vocab=V, seed=90 + R, dtype=dt, seen_lo=1, seen_hi=2, penalty=1.0,
                 temperatures=(0.0, 0.8, 1.1), top_k=top_k, name=name)
    w.seen[:] = np.uint32(0xFFFFFFFF)
    w.penalty[:] = np.linspace(0.55, 2.4, R).astype(np.float32)
    w.penalty[1] = np.inf
    # the oracle takes only valid thetas; theta 1 leaves every value as it is
    ora = w.penalty.copy()
    ora[1] = 1.0
    log(f"[gpu] ar all seen {name}: R={R} V={V} {dt} chunks={chunks} forced={forced}")
    _check_against_oracle(w, f"all_seen_{name}", oracle_penalty=ora, vocab_chunks=chunks, force_fallback=forced)


def test_ar_step_full_size():
    """The autoregressive step at full size, as timed: 256 requests x 248320 bf16,
    256 to 1280 seen ids each, theta 1.1, temperatures 0 / 0.7 / 1.0, no top-ratio
    filter; every row's penalised logits, token and logprob."""
    w = synth.ar()
    log(f"[gpu] ar full size: R={w.rows} V={w.vocab} seen={w.n_seen()}")
    _check_against_oracle(w, "full_size")


def test_penalty_edge_rows():
    """Invalid thetas leave their rows alone; bits past V are ignored; an empty
    call is a no-op; masked ids stay masked."""
    import torch

    import vocab_wise_logit_amd as ds

    R, V = 6, 70
    rng = np.random.default_rng(5)
    x = synth.bf16_from_f32((rng.normal(size=(R, V)) * 3).astype(np.float32))
    x[:, 3] = synth.bf16_from_f32(np.array([-np.inf], np.float32))[0]
    seen = np.full((R, 3), 0xFFFFFFFF, np.uint32)
    theta = np.array([2.0, np.nan, 0.0, -1.0, np.inf, 1.7], np.float32)
    with ds.Sampler(V, "bf16", max_rows=1, max_positions=R, max_requests=R) as smp:
        xd = to_dev(x)
        smp.repetition_penalty(xd, torch.from_numpy(seen.view(np.int32)).cuda(), torch.from_numpy(theta).cuda())
        smp.repetition_penalty(xd[:0], torch.from_numpy(seen.view(np.int32)).cuda()[:0],
                               torch.from_numpy(theta).cuda()[:0])
        torch.cuda.synchronize()
        got = xd.view(torch.int16).cpu().numpy().view(np.uint16)
    valid = np.array([True, False, False, False, False, True])
    want = x.copy()
    want[valid] = oracle.repetition_penalty(x[valid], seen[valid], theta[valid])
    assert np.array_equal(got, want)


def test_library_loaded_before_torch_uses_one_runtime():
    """A sampler created before any torch call on the GPU leaves torch working:
    the binding loads torch's HIP runtime before the library, in a fresh process."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import vocab_wise_logit_amd as ds\n"
            "s = ds.Sampler(1025, 'bf16', max_rows=1, max_positions=4, max_requests=1)\n"
            "import torch\n"
            "x = torch.ones(4, device='cuda') * 2\n"
            "torch.cuda.synchronize()\n"
            "assert float(x.sum()) == 8.0\n"
            "s.close()\n"
            "print('ok', flush=True)\n")
    log("[gpu] fresh process: sampler before torch")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=100)
    assert r.returncode == 0 and "ok" in r.stdout, r.stderr[-2000:]


def test_ar_step_without_penalty_equals_ds_sample_rows():
    """With no mask and no penalty the step is ds_sample over requests of one
    position each (the noise is keyed the same way)."""
    import torch

    import vocab_wise_logit_amd as ds

    R, V = 70, 1025
    w = synth.ar(n_requests=R, vocab=V, seed=77, seen_lo=1, seen_hi=2, temperatures=(0.0, 0.8, 1.1))
    with ds.Sampler(V, "bf16", max_rows=1, max_positions=R, max_requests=R, top_k=w.top_k) as smp:
        x = to_dev(w.logits)
        tok, lp = smp.sample_ar(w.request_ids, x, None, None, w.iterations, w.temperature, seed=w.seed)
        t2, l2 = smp.sample(w.request_ids, x.view(1, R, V), None, [1] * R, w.iterations, [0.0] * R,
                            w.temperature, seed=w.seed)
        torch.cuda.synchronize()
    assert np.array_equal(tok.cpu().numpy(), t2.view(-1).cpu().numpy())
    assert np.array_equal(lp.cpu().numpy().view(np.uint32), l2.view(-1).cpu().numpy().view(np.uint32))


def test_ar_step_replayed_from_a_graph_follows_device_parameters():
    """A captured autoregressive step reads its parameters when it runs: replays
    after the iterations and temperatures change match fresh eager calls."""
    import torch

    import vocab_wise_logit_amd as ds

    R, V = 96, 4096
    w = synth.ar(n_requests=R, vocab=V, seed=55, seen_lo=20, seen_hi=300, temperatures=(0.0, 0.8, 1.0))
    log(f"[gpu] ar graph: R={R} V={V}")
    with ds.Sampler(V, "bf16", max_rows=1, max_positions=R, max_requests=R, top_k=w.top_k) as smp:
        x0 = to_dev(w.logits)
        x = x0.clone()
        seen = torch.from_numpy(w.seen.view(np.int32)).cuda()
        pen = torch.from_numpy(w.penalty).cuda()
        rid = torch.tensor(w.request_ids, device="cuda")
        it = torch.tensor(w.iterations, device="cuda")
        tp = torch.tensor(w.temperature, device="cuda")
        out = (torch.empty(R, dtype=torch.int32, device="cuda"), torch.empty(R, dtype=torch.float32, device="cuda"))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            smp.sample_ar(rid, x, seen, pen, it, tp, seed=w.seed, out=out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        x.copy_(x0)
        with torch.cuda.graph(g):
            smp.sample_ar(rid, x, seen, pen, it, tp, seed=w.seed, out=out)
        for step in range(4):
            it.fill_(step + 3)
            tp.copy_(torch.tensor(np.roll(w.temperature, step), device="cuda"))
            x.copy_(x0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = (out[0].cpu().numpy().copy(), out[1].cpu().numpy().copy())
            xe = x0.clone()
            ref = smp.sample_ar(rid, xe, seen, pen, it, tp, seed=w.seed)
            torch.cuda.synchronize()
            assert np.array_equal(got[0], ref[0].cpu().numpy()), f"replay {step}: tokens differ"
            assert np.array_equal(got[1].view(np.uint32), ref[1].cpu().numpy().view(np.uint32))
            assert torch.equal(x, xe), f"replay {step}: penalised logits differ"


def test_sampler_left_open_at_exit_is_released_cleanly():
    """A sampler still alive when the interpreter exits is destroyed without an
    error, though the binding's module globals may already be gone."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import vocab_wise_logit_amd as ds\n"
            "s = ds.Sampler(1025, 'bf16', max_rows=1, max_positions=4, max_requests=1)\n"
            "print('ok', flush=True)\n")
    log("[gpu] fresh process: sampler alive at exit")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=100)
    assert r.returncode == 0 and "ok" in r.stdout, r.stderr[-2000:]
    assert "Exception ignored" not in r.stderr and "Traceback" not in r.stderr, r.stderr[-2000:]
