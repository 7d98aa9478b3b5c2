"""ds_sample_static (the entry point that allocates nothing) against ds_sample.

Both run the same kernels; the static one keeps the streaming kernels' records
in the library's fixed device array instead of a handle's workspace.  With the
threshold output on a long row ds_sample also uses its handle's threshold
windows (a parts kernel of another workgroup size), which the static entry point
has no memory for: it takes the exact passes instead, so there the logprobs,
summed in another order, agree to rounding.  Each case calls the two entry
points through the C ABI, twice in a row with the second input smaller (so the
second static call finds the first call's records in the shared array), and
requires identical tokens and thresholds and logprobs identical or, on that
one path, within 1e-5.  The
streaming path (V = 248320 and V = 60000, which use the array) and the
wave-per-cell path (V = 1025, which does not) are both covered, as is the forced
multi-pass path.
"""

from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_helpers import log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    torch.cuda.init()


def _outputs(w, threshold):
    import torch

    shape = (w.rows, w.positions)
    return (torch.full(shape, -7, dtype=torch.int32, device="cuda"),
            torch.full(shape, 7.0, dtype=torch.float32, device="cuda"),
            torch.full(shape, 7.0, dtype=torch.float32, device="cuda") if threshold else None)


def _pair(w, *, threshold, flags):
    """(ds_sample outputs, ds_sample_static outputs) of one workload."""
    import torch

    import vocab_wise_logit_amd as ds

    dt = ds.DS_DTYPE_BF16 if w.dtype == "bf16" else ds.DS_DTYPE_F32
    c = to_dev(w.c)
    u = to_dev(w.u) if w.u is not None else None
    ref = _outputs(w, threshold)
    got = _outputs(w, threshold)
    log(f"[gpu] ds_sample vs ds_sample_static {w.name}: C={w.rows} P={w.positions} V={w.vocab} "
        f"chunks={w.vocab_chunks} flags={flags} threshold={threshold}")
    h = ds.ds_sample_create(0, w.vocab, dt, w.rows, max(1, w.positions), len(w.seq_lens), w.top_k,
                            w.vocab_chunks, flags)
    try:
        ds.ds_sample(h, w.request_ids, c, u, w.seq_lens, w.iterations, w.guidance, w.temperature, w.rows,
                     w.seed, *ref)
    finally:
        torch.cuda.synchronize()
        ds.ds_sample_destroy(h)
    ds.ds_sample_static(w.vocab, dt, w.top_k, w.vocab_chunks, flags, w.request_ids, c, u, w.seq_lens,
                        w.iterations, w.guidance, w.temperature, w.rows, w.seed, *got)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in ref if t is not None], [t.cpu().numpy() for t in got if t is not None]


def _assert_same(ref, got, what, exact_logprobs):
    for a, b, name in zip(ref, got, ("tokens", "logprobs", "thresholds")):
        if name == "logprobs" and not exact_logprobs:
            assert np.max(np.abs(a - b), initial=0.0) <= 1e-5, f"{what}: {name} differ"
        else:
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{what}: {name} differ"
    assert (got[0] >= 0).all(), f"{what}: a cell was not written"


@pytest.mark.parametrize("flags", [0, 1])
def test_static_entry_point_equals_ds_sample_twice_second_smaller(flags):
    cases = [
        # streaming path, 4 vocabulary chunks: records in the static array
        (synth.stress(positions=40, seed=14), synth.stress(positions=9, seed=15)),
        # streaming path, one chunk, guidance 0 and greedy requests mixed in
        (synth.diffusion("mid_a", seed=31, vocab=60000, rows=3, seq_lens=[7, 0, 5], sigma=4.0,
                         guidance=[1.5, 0.0, 2.0], temperature=[1.0, 0.0, 0.7]),
         synth.diffusion("mid_b", seed=32, vocab=60000, rows=2, seq_lens=[2, 3], sigma=4.0,
                         guidance=[0.0, 1.0], temperature=[0.9, 0.0])),
        # wave-per-cell path (no records), an OmniVoice-shaped batch
        (synth.omnivoice(n_requests=4), synth.omnivoice(n_requests=2, seed=9)),
    ]
    for big, small in cases:
        assert small.cells < big.cells
        for w, thr in ((big, True), (small, True), (big, False), (small, False)):
            ref, got = _pair(w, threshold=thr, flags=flags)
            # the handle's threshold windows: long rows, threshold output, not forced
            windows = thr and flags == 0 and w.vocab > 1025
            _assert_same(ref, got, f"{w.name} threshold={thr}", exact_logprobs=not windows)


def test_static_entry_point_rejects_bad_settings_before_launch():
    import torch

    import vocab_wise_logit_amd as ds

    w = synth.tiny(0.9)
    c, u = to_dev(w.c), to_dev(w.u)
    tok = torch.full((w.rows, w.positions), -7, dtype=torch.int32, device="cuda")
    lp = torch.zeros((w.rows, w.positions), dtype=torch.float32, device="cuda")
    L = ds.lib()
    host = [np.ascontiguousarray(a, dt) for a, dt in ((w.request_ids, np.int64), (w.seq_lens, np.int32),
                                                      (w.iterations, np.int32), (w.guidance, np.float32),
                                                      (w.temperature, np.float32))]
    for vocab, dtype, top_k, chunks, flags in ((0, 0, 0, 1, 0), (1024, 7, 0, 1, 0), (1024, 0, 2000, 1, 0),
                                               (1024, 0, 0, 0, 0), (1024, 0, 0, 1, 8)):
        rc = L.ds_sample_static(vocab, dtype, top_k, chunks, flags, host[0].ctypes.data, c.data_ptr(),
                                u.data_ptr(), host[1].ctypes.data, host[2].ctypes.data, host[3].ctypes.data,
                                host[4].ctypes.data, host[0].size, w.rows, 1, tok.data_ptr(), lp.data_ptr(), None,
                                None)
        assert rc == ds.DS_ERR_INVALID_ARG, (vocab, dtype, top_k, chunks, flags)
    torch.cuda.synchronize()
    assert bool((tok == -7).all())
