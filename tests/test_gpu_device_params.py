"""GPU parity of ds_sample_device_params: the fixed-shape call whose per-request
parameters live in device memory.  For valid values it runs the same kernel
arithmetic as ds_sample, eagerly and when replayed from a captured graph after
the parameters change: tokens and thresholds must agree bit for bit.  Logprobs
agree to fp32 rounding (LP_SAME): the order in which a lane sums its exponentials
follows the row's dword alignment, which moves with the layout's position stride.
ds_sample itself is held to the oracle by test_gpu_parity.py, and the first case
here checks the oracle again.

Every case prints what it runs before launching, so a failure names its case.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_sample, log, run_sample, to_dev

pytestmark = pytest.mark.gpu

SENTINEL_TOKEN = -7
SENTINEL_LP = 12345.0
LP_SAME = 1e-5


def _assert_same(got, want, what: str):
    """got / want: (tokens, logprobs[, thresholds]) tensors of the same cells."""
    import torch

    assert torch.equal(got[0], want[0]), f"{what}: tokens differ"
    d = (got[1] - want[1]).abs().max().item()
    assert d <= LP_SAME, f"{what}: logprobs differ by {d}"
    if len(got) > 2 and got[2] is not None:
        assert torch.equal(torch.nan_to_num(got[2], nan=-1.0), torch.nan_to_num(want[2], nan=-1.0)), \
            f"{what}: thresholds differ"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    torch.cuda.init()


def _params(rid, sl, it, gs, tp):
    import torch

    return (torch.tensor(np.asarray(rid, np.int64), device="cuda"),
            torch.tensor(np.asarray(sl, np.int32), device="cuda"),
            torch.tensor(np.asarray(it, np.int32), device="cuda"),
            torch.tensor(np.asarray(gs, np.float32), device="cuda"),
            torch.tensor(np.asarray(tp, np.float32), device="cuda"))


def _outputs(C, Pc, threshold):
    import torch

    tok = torch.full((C, Pc), SENTINEL_TOKEN, dtype=torch.int32, device="cuda")
    lp = torch.full((C, Pc), SENTINEL_LP, dtype=torch.float32, device="cuda")
    thr = torch.full((C, Pc), SENTINEL_LP, dtype=torch.float32, device="cuda") if threshold else None
    return tok, lp, thr


def _padded(a: np.ndarray, extra: int, fill) -> np.ndarray:
    """[C, P, V] -> [C, P + extra, V], the new positions set to `fill`."""
    C, P, V = a.shape
    out = np.full((C, P + extra, V), fill, dtype=a.dtype)
    out[:, :P] = a
    return out


def _check_padding_untouched(outs, P):
    for t in outs:
        if t is None:
            continue
        pad = t[:, P:]
        want = SENTINEL_TOKEN if t.dtype.is_floating_point is False else SENTINEL_LP
        assert bool((pad == want).all()), "a padding position was written"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_device_params_equal_ds_sample(dtype):
    import torch

    import vocab_wise_logit_amd as ds

    # ragged lengths with an empty request, greedy and sampled, negative and zero
    # guidance; 9 padding positions (NaN logits, never read) and one padding request
    w = synth.diffusion(f"devp_{dtype}", seed=61, vocab=1025, rows=3, seq_lens=[5, 0, 7, 4], dtype=dtype,
                        sigma=3.0, guidance=[2.0, 1.0, 0.0, -0.5], temperature=[0.9, 0.7, 0.0, 1.2],
                        iterations=[3, 1, 0, 7], spikes=True)
    eager = run_sample(w, threshold=True)
    check_sample(w, eager, oracle.sample_workload(w))
    nan = synth.workloads.BF16_NAN if dtype == "bf16" else np.float32(np.nan)
    extra = 9
    c = to_dev(_padded(w.c, extra, nan))
    u = to_dev(_padded(w.u, extra, nan))
    P, Pc = w.positions, w.positions + extra
    prm = _params(list(w.request_ids) + [99], list(w.seq_lens) + [0], list(w.iterations) + [0],
                  list(w.guidance) + [3.0], list(w.temperature) + [0.5])
    log(f"[gpu] ds_sample_device_params {w.name}: C={w.rows} P={P} positions={Pc} requests={len(w.seq_lens) + 1}")
    with ds.Sampler(w.vocab, dtype, max_rows=w.rows, max_positions=Pc, max_requests=8) as smp:
        out = _outputs(w.rows, Pc, True)
        smp.sample_device_params(*prm[:1], c, u, *prm[1:], seed=w.seed, threshold=True, out=out)
        torch.cuda.synchronize()
    _check_padding_untouched(out, P)
    got = [t[:, :P].reshape(-1).cpu() for t in out]
    _assert_same(got, [torch.from_numpy(a) for a in eager], "device params vs ds_sample")


def test_device_params_graph_replays_follow_the_parameters():
    import torch

    import vocab_wise_logit_amd as ds

    # one capture, four batches: new iterations, new lengths (filling the layout
    # up to its last position), new guidance and temperature
    C, Pc, V = 2, 24, 1025
    src = synth.diffusion("devp_graph", seed=62, vocab=V, rows=C, seq_lens=[Pc], dtype="bf16", sigma=3.0,
                          guidance=2.0, temperature=0.9, spikes=True)
    c = to_dev(src.c)
    u = to_dev(src.u)
    batches = [
        dict(sl=[6, 9, 3], it=[0, 0, 0], gs=[2.0, 0.0, 1.5], tp=[0.9, 0.0, 1.1]),
        dict(sl=[6, 9, 3], it=[1, 1, 1], gs=[2.0, 0.0, 1.5], tp=[0.9, 0.0, 1.1]),
        dict(sl=[10, 4, 8], it=[2, 5, 0], gs=[1.0, 2.0, 0.0], tp=[1.2, 0.8, 0.0]),
        dict(sl=[0, 24, 0], it=[3, 3, 3], gs=[0.5, 1.0, 2.0], tp=[0.0, 0.6, 0.9]),
    ]
    rid = [501, 502, 503]
    with ds.Sampler(V, "bf16", max_rows=C, max_positions=Pc, max_requests=3) as smp:
        prm = _params(rid, batches[0]["sl"], batches[0]["it"], batches[0]["gs"], batches[0]["tp"])
        out = _outputs(C, Pc, True)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm-up on the capture stream
            smp.sample_device_params(prm[0], c, u, *prm[1:], seed=7, threshold=True, out=out)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            smp.sample_device_params(prm[0], c, u, *prm[1:], seed=7, threshold=True, out=out)
        firsts = []
        for i, b in enumerate(batches):
            P = int(sum(b["sl"]))
            log(f"[gpu] graph replay {i}: seq_lens={b['sl']} iterations={b['it']}")
            for t, v in zip(prm[1:], (b["sl"], b["it"], b["gs"], b["tp"])):
                t.copy_(torch.tensor(np.asarray(v), dtype=t.dtype))
            out[0].fill_(SENTINEL_TOKEN)
            out[1].fill_(SENTINEL_LP)
            out[2].fill_(SENTINEL_LP)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            ref = smp.sample(rid, c[:, :P].contiguous(), u[:, :P].contiguous(), b["sl"], b["it"], b["gs"],
                             b["tp"], seed=7, threshold=True)
            torch.cuda.synchronize()
            _check_padding_untouched(out, P)
            _assert_same([t[:, :P] for t in out], ref, f"replay {i}")
            firsts.append(out[0][:, :P].clone())
        del g
    # the iteration keys the noise: the first two batches differ only there
    assert not torch.equal(firsts[0], firsts[1])


def test_device_params_take_invalid_values_as_documented():
    import torch

    import vocab_wise_logit_amd as ds

    # a negative length counts as 0, a temperature that is not a positive finite
    # number samples greedily, a guidance scale that is not finite counts as 0,
    # and without u every request is unguided
    w = synth.diffusion("devp_bad", seed=63, vocab=1025, rows=2, seq_lens=[4, 3, 5, 2, 3], dtype="bf16",
                        sigma=3.0, guidance=[2.0, 1.0, 1.0, 1.0, 1.5], temperature=[0.9, 0.9, 0.9, 0.9, 0.9],
                        spikes=True, nan_unread_u=False)
    c = to_dev(w.c)
    u = to_dev(w.u)
    raw = dict(sl=[4, -3, 5, 2, 3], gs=[2.0, float("inf"), float("nan"), 1.0, 1.5],
               tp=[0.9, 0.9, float("nan"), -1.0, float("inf")])
    clean = dict(sl=[4, 0, 5, 2, 3], gs=[2.0, 0.0, 0.0, 1.0, 1.5], tp=[0.9, 0.9, 0.0, 0.0, 0.0])
    P = int(sum(clean["sl"]))
    rid = list(w.request_ids)
    it = [0, 1, 2, 3, 4]
    with ds.Sampler(w.vocab, "bf16", max_rows=2, max_positions=w.positions, max_requests=5) as smp:
        for with_u in (True, False):
            log(f"[gpu] device params with invalid values, u {'given' if with_u else 'absent'}")
            prm = _params(rid, raw["sl"], it, raw["gs"], raw["tp"])
            out = _outputs(2, w.positions, False)
            smp.sample_device_params(prm[0], c, u if with_u else None, *prm[1:], seed=3, out=out)
            gs = clean["gs"] if with_u else [0.0] * 5
            ref = smp.sample(rid, c[:, :P].contiguous(), u[:, :P].contiguous() if with_u else None, clean["sl"],
                             it, gs, clean["tp"], seed=3)
            torch.cuda.synchronize()
            _assert_same([t[:, :P] for t in out[:2]], ref, f"invalid values, u {with_u}")
            _check_padding_untouched(out[:2], P)


@pytest.mark.parametrize("dtype,V,chunks,fallback", [("bf16", 5000, 1, False), ("bf16", 3000, 3, False),
                                                     ("f32", 4100, 2, False), ("bf16", 1025, 1, True),
                                                     ("bf16", 65536, 2, False), ("f32", 65536, 1, False)])
def test_device_params_streaming_path(dtype, V, chunks, fallback):
    import torch

    import vocab_wise_logit_amd as ds

    # vocabularies past the wave-per-cell kernel (and, with the forced fallback,
    # one inside it) go through the streaming kernels over the fixed layout; at
    # V = 65536 the threshold output takes the window path (its own window,
    # parts and merge kernels for device parameters)
    w = synth.diffusion(f"devp_row_{dtype}_{V}", seed=64 + V, vocab=V, rows=2, seq_lens=[3, 0, 4], dtype=dtype,
                        sigma=4.0, guidance=[1.5, 2.0, 0.0], temperature=[1.0, 0.5, 0.7], iterations=[2, 0, 5],
                        vocab_chunks=chunks)
    eager = run_sample(w, threshold=True, force_fallback=fallback)
    check_sample(w, eager, oracle.sample_workload(w))
    nan = synth.workloads.BF16_NAN if dtype == "bf16" else np.float32(np.nan)
    extra = 5
    c = to_dev(_padded(w.c, extra, nan))
    u = to_dev(_padded(w.u, extra, nan))
    P, Pc = w.positions, w.positions + extra
    prm = _params(w.request_ids, w.seq_lens, w.iterations, w.guidance, w.temperature)
    log(f"[gpu] ds_sample_device_params {w.name}: streaming path, positions={Pc}, chunks={chunks}, "
        f"fallback={fallback}")
    with ds.Sampler(V, dtype, max_rows=2, max_positions=Pc, max_requests=4, vocab_chunks=chunks,
                    force_fallback=fallback) as smp:
        out = _outputs(2, Pc, True)
        smp.sample_device_params(prm[0], c, u, *prm[1:], seed=w.seed, threshold=True, out=out)
        torch.cuda.synchronize()
        _check_padding_untouched(out, P)
        got = [t[:, :P].reshape(-1).cpu() for t in out]
        _assert_same(got, [torch.from_numpy(a) for a in eager], "streaming device params vs ds_sample")
        # and replayed from a graph after the iterations change
        out2 = _outputs(2, Pc, False)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            smp.sample_device_params(prm[0], c, u, *prm[1:], seed=w.seed, out=out2)
        it2 = [7, 7, 9]
        prm[2].copy_(torch.tensor(np.asarray(it2, np.int32)))
        g.replay()
        ref = smp.sample(w.request_ids, c[:, :P].contiguous(), u[:, :P].contiguous(), w.seq_lens, it2, w.guidance,
                         w.temperature, seed=w.seed)
        torch.cuda.synchronize()
        _assert_same([t[:, :P] for t in out2[:2]], ref, "streaming graph replay")
        _check_padding_untouched(out2[:2], P)
        del g


def test_device_params_rejects_what_it_cannot_run():
    import torch

    import vocab_wise_logit_amd as ds

    prm = _params([1], [4], [0], [0.0], [0.0])
    with ds.Sampler(1025, "bf16", max_rows=1, max_positions=8, max_requests=128) as smp:
        c = torch.zeros((1, 16, 1025), dtype=torch.bfloat16, device="cuda")
        log("[gpu] device params beyond max_positions, and with 65 requests")
        with pytest.raises(ds.DSError) as e:
            smp.sample_device_params(prm[0], c, None, *prm[1:])
        assert e.value.code == ds.DS_ERR_CAPACITY
        many = _params([1] * 65, [0] * 65, [0] * 65, [0.0] * 65, [0.0] * 65)
        with pytest.raises(ds.DSError) as e:
            smp.sample_device_params(many[0], c[:, :8].contiguous(), None, *many[1:])
        assert e.value.code == ds.DS_ERR_CAPACITY
        torch.cuda.synchronize()
