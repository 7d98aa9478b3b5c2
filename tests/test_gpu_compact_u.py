"""GPU parity of the compacted u layout (DS_FLAG_COMPACT_U): u holds only the
positions of requests whose guidance scale is not 0.  The kernels read the same u
values as from the full layout, so every output must equal the full-layout call
bit for bit; the full-layout call is held to the oracle by test_gpu_parity.py,
and the first case here checks the oracle again.

Every case prints what it runs before launching, so a failure names its case.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_sample, log, run_sample, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    torch.cuda.init()


def compact(w):
    """The guided requests' positions of w.u, in request order: [C, P_u, V] (None
    when no request is guided)."""
    if w.u is None:
        return None
    offs = np.concatenate([[0], np.cumsum(w.seq_lens)])
    keep = [np.arange(offs[r], offs[r + 1]) for r in range(len(w.seq_lens)) if w.guidance[r] != 0]
    idx = np.concatenate(keep) if keep else np.zeros(0, np.int64)
    return np.ascontiguousarray(w.u[:, idx])


def run_compact(w, *, threshold=True, force_fallback=False):
    import torch

    import vocab_wise_logit_amd as ds

    uc = compact(w)
    log(f"[gpu] ds_sample compact u {w.name}: C={w.rows} P={w.positions} P_u={0 if uc is None else uc.shape[1]} "
        f"V={w.vocab} "
        f"dtype={w.dtype} chunks={w.vocab_chunks} fallback={force_fallback}")
    with ds.Sampler(w.vocab, w.dtype, max_rows=w.rows, max_positions=max(1, w.positions),
                    max_requests=len(w.seq_lens), top_k=w.top_k, vocab_chunks=w.vocab_chunks,
                    force_fallback=force_fallback, compact_u=True) as smp:
        c = to_dev(w.c)
        u = to_dev(uc) if uc is not None and uc.shape[1] else None
        out = smp.sample(w.request_ids, c, u, w.seq_lens, w.iterations, w.guidance, w.temperature, seed=w.seed,
                         threshold=threshold)
        torch.cuda.synchronize()
    return [t.reshape(-1).cpu().numpy() for t in out]


def assert_equal(got, ref):
    for g, r, name in zip(got, ref, ("tokens", "logprobs", "thresholds")):
        assert np.array_equal(g, r, equal_nan=True), f"{name} differ from the full u layout"


@pytest.mark.parametrize("dtype,V", [("bf16", 1025), ("bf16", 1024), ("f32", 1025), ("bf16", 2046)])
def test_compact_u_wave_per_cell(dtype, V):
    # odd and even request lengths between guided requests put the compacted u
    # rows at both parities against their c rows (odd V in bf16)
    w = synth.diffusion(f"cu_{dtype}_{V}", seed=71 + V, vocab=V, rows=3, seq_lens=[5, 2, 0, 7, 3, 4, 1],
                        dtype=dtype, sigma=3.0, guidance=[2.0, 0.0, 1.0, -0.5, 0.0, 1.5, 2.0],
                        temperature=[0.9, 0.7, 0.5, 0.0, 1.2, 0.8, 0.9], iterations=[1, 2, 3, 4, 5, 6, 7],
                        spikes=True, masked_ids=[3])
    ref = run_sample(w)
    check_sample(w, ref, oracle.sample_workload(w))
    assert_equal(run_compact(w), ref)


@pytest.mark.parametrize("dtype,V,chunks,fallback", [("bf16", 3000, 1, False), ("bf16", 4104, 3, False),
                                                     ("f32", 4100, 2, False), ("f32", 1024, 1, True),
                                                     ("bf16", 65536, 2, False)])
def test_compact_u_streaming_path(dtype, V, chunks, fallback):
    # V * b is a multiple of 16 bytes, so every u row keeps its c row's 16-byte
    # alignment under the compaction; at V = 65536 the threshold output takes the
    # window path, whose sample reads the compacted u rows too
    w = synth.diffusion(f"cu_row_{dtype}_{V}", seed=81 + V, vocab=V, rows=2, seq_lens=[3, 2, 4, 1], dtype=dtype,
                        sigma=4.0, guidance=[1.5, 0.0, 2.0, 1.0], temperature=[1.0, 0.5, 0.0, 0.7],
                        vocab_chunks=chunks)
    ref = run_sample(w, force_fallback=fallback)
    check_sample(w, ref, oracle.sample_workload(w))
    assert_equal(run_compact(w, force_fallback=fallback), ref)


def test_compact_u_edge_layouts():
    # every request guided (P_u = P), none guided (no u at all), a single guided
    # request between unguided ones
    for name, gs in (("all", [1.0, 2.0, 0.5]), ("none", [0.0, 0.0, 0.0]), ("one", [0.0, 1.5, 0.0])):
        w = synth.diffusion(f"cu_edge_{name}", seed=91, vocab=1025, rows=2, seq_lens=[3, 5, 2], dtype="bf16",
                            sigma=3.0, guidance=gs, temperature=[0.9, 0.0, 1.1])
        assert_equal(run_compact(w), run_sample(w))


def test_compact_u_rejected_where_alignment_cannot_hold():
    import torch

    import vocab_wise_logit_amd as ds

    # the streaming kernels with V * b not a multiple of 16, and the fixed-shape
    # entry point, refuse the compacted layout before launching
    w = synth.diffusion("cu_bad", seed=93, vocab=4103, rows=1, seq_lens=[2, 2], dtype="bf16", sigma=3.0,
                        guidance=[1.0, 0.0], temperature=[0.9, 0.9])
    with ds.Sampler(4103, "bf16", max_rows=1, max_positions=4, max_requests=2, compact_u=True) as smp:
        c = to_dev(w.c)
        u = to_dev(compact(w))
        tok = torch.full((1, 4), -7, dtype=torch.int32, device="cuda")
        lp = torch.zeros((1, 4), dtype=torch.float32, device="cuda")
        log("[gpu] compact u with V * b not a multiple of 16 on the streaming path")
        with pytest.raises(ds.DSError) as e:
            smp.sample(w.request_ids, c, u, w.seq_lens, w.iterations, w.guidance, w.temperature, out=(tok, lp, None))
        assert e.value.code == ds.DS_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert bool((tok == -7).all())
    with ds.Sampler(1025, "bf16", max_rows=1, max_positions=4, max_requests=2, compact_u=True) as smp:
        c = torch.zeros((1, 4, 1025), dtype=torch.bfloat16, device="cuda")
        prm = [torch.tensor(v, dtype=dt, device="cuda") for v, dt in
               (([1, 2], torch.int64), ([2, 2], torch.int32), ([0, 0], torch.int32), ([0.0, 0.0], torch.float32),
                ([0.0, 0.0], torch.float32))]
        log("[gpu] compact u with the fixed-shape entry point")
        with pytest.raises(ds.DSError) as e:
            smp.sample_device_params(prm[0], c, None, *prm[1:])
        assert e.value.code == ds.DS_ERR_UNSUPPORTED
