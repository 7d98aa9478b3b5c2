"""CPU checks of the C ABI: the library loads, exports every entry point that
include/ds_sample.h declares, and rejects invalid arguments before touching a GPU."""

from __future__ import annotations

import ctypes as C
import os
import re

import pytest

import vocab_wise_logit_amd as ds

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ds_sample.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ds_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(ds.EXPORTED)


def test_library_loads_and_exports_every_declared_symbol():
    L = ds.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
        assert getattr(L, name) is not None
    out = os.popen(f"nm -D --defined-only {ds.LIB_PATH}").read()
    exported = set(re.findall(r" T (ds_\w+)", out))
    assert set(declared_functions()) <= exported
    assert ds.ds_version() == 300


@pytest.mark.parametrize("kw,msg", [
    (dict(vocab=0), "vocab"),
    (dict(dtype=7), "dtype"),
    (dict(max_rows=0), "max_rows"),
    (dict(max_positions=0), "max_positions"),
    (dict(max_requests=0), "max_requests"),
    (dict(top_k=2000), "top_k"),
    (dict(vocab_chunks=0), "vocab_chunks"),
    (dict(vocab_chunks=1025), "vocab_chunks"),
    (dict(flags=8), "flags"),
    (dict(max_rows=1 << 20, max_positions=1 << 20), "cells"),
])
def test_create_rejects_bad_arguments_without_a_gpu(kw, msg):
    args = dict(device=0, vocab=1025, dtype=ds.DS_DTYPE_BF16, max_rows=8, max_positions=100,
                max_requests=8, top_k=0, vocab_chunks=1, flags=0)
    args.update(kw)
    with pytest.raises(ds.DSError) as e:
        ds.ds_sample_create(**args)
    assert e.value.code == ds.DS_ERR_INVALID_ARG
    assert msg in str(e.value)


def test_calls_on_a_null_handle_fail_cleanly():
    L = ds.lib()
    rc = L.ds_sample(None, None, None, None, None, None, None, None, 1, 1, 0, None, None, None, None)
    assert rc == ds.DS_ERR_INVALID_ARG
    assert "sampler is NULL" in ds.ds_last_error()
    rc = L.ds_sample_device_params(None, None, None, None, None, None, None, None, 1, 1, 1, 0, None, None, None,
                                   None)
    assert rc == ds.DS_ERR_INVALID_ARG and "sampler is NULL" in ds.ds_last_error()
    rc = L.ds_greedy_lse(None, None, 1, None, None, None, None, None)
    assert rc == ds.DS_ERR_INVALID_ARG
    rc = L.ds_reveal_topk(None, None, 1, None, None, 1, None, None, None)
    assert rc == ds.DS_ERR_INVALID_ARG and "sampler is NULL" in ds.ds_last_error()
    rc = L.ds_repetition_penalty(None, None, 1, None, None, None)
    assert rc == ds.DS_ERR_INVALID_ARG and "sampler is NULL" in ds.ds_last_error()
    rc = L.ds_sample_ar(None, None, None, None, None, None, None, 1, 0, None, None, None)
    assert rc == ds.DS_ERR_INVALID_ARG and "sampler is NULL" in ds.ds_last_error()
    h = C.c_void_p()
    assert L.ds_sample_create(None, 0, 10, 0, 1, 1, 1, 0, 1, 0) == ds.DS_ERR_INVALID_ARG
    assert L.ds_sample_create(C.byref(h), 0, -1, 0, 1, 1, 1, 0, 1, 0) == ds.DS_ERR_INVALID_ARG
    assert h.value is None
    L.ds_sample_destroy(None)  # no-op


def test_binding_refuses_to_run_without_the_library(monkeypatch, tmp_path):
    from vocab_wise_logit_amd import _binding

    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _binding.lib()


def test_request_stage_copies_values_and_refuses_what_does_not_fit():
    import numpy as np

    st = ds.RequestStage(4)
    assert st.fill([7, 8], [3, 0], [1, 2], [2.0, 0.5], [0.9, 0.0]) == 2
    assert st.rid[:2].tolist() == [7, 8] and st.sl[:2].tolist() == [3, 0]
    assert st.it[:2].tolist() == [1, 2]
    assert st.gs[:2].tolist() == [2.0, 0.5] and st.tp[:2].tolist() == [np.float32(0.9), 0.0]
    # the addresses handed to the C call are those of the staged arrays
    assert st.ptrs[0] == st.rid.ctypes.data and st.ptrs[4] == st.tp.ctypes.data
    # more requests than the capacity, unequal lengths, no requests, a 2-D array
    assert st.fill(list(range(5)), [1] * 5, [0] * 5, [1.0] * 5, [1.0] * 5) == -1
    assert st.fill([1, 2], [1], [0, 0], [1.0, 1.0], [1.0, 1.0]) == -1
    assert st.fill([], [], [], [], []) == -1
    assert st.fill([1, 2], np.ones((2, 2), np.int32), [0, 0], [1.0, 1.0], [1.0, 1.0]) == -1
    assert st.fill_reveal([5, 6, 7], [1, 2, 3]) == 3
    assert st.sl[:3].tolist() == [5, 6, 7] and st.rc[:3].tolist() == [1, 2, 3]
    assert st.fill_reveal([5], [1, 2]) == -1


# -------------------------------------------------- binding-side shape checks

class _NoCall:
    """Stands in for the library: any entry point reached fails the test."""

    def __getattr__(self, name):
        raise AssertionError(f"{name} was called despite invalid tensors")


@pytest.fixture
def fake_handle(monkeypatch):
    """A handle the binding knows (V = 1025 bf16, 4 chunks, compacted u) with the
    library replaced, so that only the binding's own checks run (CPU tensors)."""
    from vocab_wise_logit_amd import _binding

    monkeypatch.setattr(_binding, "_lib", _NoCall())
    monkeypatch.setitem(_binding._HANDLES, 0xABC0, (1025, ds.DS_DTYPE_BF16, 4, ds.DS_FLAG_COMPACT_U))
    monkeypatch.setitem(_binding._HANDLES, 0xABD0, (1025, ds.DS_DTYPE_F32, 1, 0))
    return 0xABC0


def _sample_args(torch, **over):
    a = dict(request_ids=[1, 2], c_logits=torch.zeros((2, 7, 1025), dtype=torch.bfloat16),
             u_logits=torch.zeros((2, 3, 1025), dtype=torch.bfloat16), seq_lens=[3, 4], iterations=[0, 0],
             guidance_scale=[1.5, 0.0], temperature=[0.9, 0.0], num_rows=2, seed=1,
             tokens_out=torch.zeros((2, 7), dtype=torch.int32), logprobs_out=torch.zeros((2, 7)))
    a.update(over)
    return a


@pytest.mark.parametrize("over,err", [
    (lambda t: dict(c_logits=t.zeros((2, 8, 1025), dtype=t.bfloat16)), ValueError),     # P != sum(seq_lens)
    (lambda t: dict(c_logits=t.zeros((1, 7, 1025), dtype=t.bfloat16)), ValueError),     # rows
    (lambda t: dict(c_logits=t.zeros((2, 7, 1024), dtype=t.bfloat16)), ValueError),     # V
    (lambda t: dict(c_logits=t.zeros((2, 7, 1025), dtype=t.float32)), TypeError),       # dtype
    (lambda t: dict(c_logits=t.zeros((7, 1025), dtype=t.bfloat16), num_rows=1), ValueError),  # 2-D
    (lambda t: dict(u_logits=t.zeros((2, 7, 1025), dtype=t.bfloat16)), ValueError),     # full u on a compact handle
    (lambda t: dict(tokens_out=t.zeros((2, 6), dtype=t.int32)), ValueError),            # short output
    (lambda t: dict(tokens_out=t.zeros((2, 7), dtype=t.int64)), TypeError),             # output dtype
    (lambda t: dict(logprobs_out=t.zeros(13)), ValueError),
    (lambda t: dict(threshold_out=t.zeros((2, 6))), ValueError),
])
def test_binding_refuses_mismatched_sample_tensors(fake_handle, over, err):
    import torch

    with pytest.raises(err) as e:
        ds.ds_sample(fake_handle, **_sample_args(torch, **over(torch)))
    assert "HIP device" not in str(e.value)  # refused for its shape or type, not its device


def test_binding_passes_matching_tensors_on_to_the_device_check(fake_handle):
    import torch

    # the valid CPU arguments get past the shape checks and stop at the device check
    with pytest.raises(ValueError, match="HIP device"):
        ds.ds_sample(fake_handle, **_sample_args(torch))


def test_binding_refuses_mismatched_tensors_of_the_other_calls(fake_handle, monkeypatch):
    import torch

    from vocab_wise_logit_amd import _binding

    # any tensor reaching the device check fails the test: only the size and
    # type checks may refuse these calls
    def no_device_check(*a, **k):
        raise AssertionError("the shape and type checks let an invalid tensor through")

    monkeypatch.setattr(_binding, "_dev_ptr", no_device_check)

    bf = torch.bfloat16
    i32, f32 = torch.int32, torch.float32
    h = fake_handle
    # draft greedy: V, dtype, rows, outputs, triples sized by the handle's chunks
    with pytest.raises(ValueError):
        ds.ds_greedy_lse(h, torch.zeros((4, 1024), dtype=bf), 4, torch.zeros(4, dtype=i32), torch.zeros(4),
                         torch.zeros(4))
    with pytest.raises(TypeError):
        ds.ds_greedy_lse(h, torch.zeros((4, 1025), dtype=f32), 4, torch.zeros(4, dtype=i32), torch.zeros(4),
                         torch.zeros(4))
    with pytest.raises(ValueError):
        ds.ds_greedy_lse(h, torch.zeros((3, 1025), dtype=bf), 4, torch.zeros(4, dtype=i32), torch.zeros(4),
                         torch.zeros(4))
    with pytest.raises(ValueError):
        ds.ds_greedy_lse(h, torch.zeros((4, 1025), dtype=bf), 4, torch.zeros(3, dtype=i32), torch.zeros(4),
                         torch.zeros(4))
    with pytest.raises(ValueError):
        ds.ds_greedy_lse(h, torch.zeros((4, 1025), dtype=bf), 4, torch.zeros(4, dtype=i32), torch.zeros(4),
                         torch.zeros(4), torch.zeros((1, 4, 3)))
    # penalty and autoregressive step: logits [n, V], masks of ceil(V / 32) words
    with pytest.raises(ValueError):
        ds.ds_repetition_penalty(h, torch.zeros((2, 1025), dtype=bf), 2, torch.zeros((2, 32), dtype=i32),
                                 torch.ones(2))
    with pytest.raises(ValueError):
        ds.ds_sample_ar(h, torch.zeros(2, dtype=torch.int64), torch.zeros((2, 1000), dtype=bf), None, None,
                        torch.zeros(2, dtype=i32), torch.zeros(2), 0, torch.zeros(2, dtype=i32), torch.zeros(2))
    with pytest.raises(ValueError):
        ds.ds_sample_ar(h, torch.zeros(1, dtype=torch.int64), torch.zeros((2, 1025), dtype=bf), None, None,
                        torch.zeros(2, dtype=i32), torch.zeros(2), 0, torch.zeros(2, dtype=i32), torch.zeros(2))
    with pytest.raises(ValueError):
        ds.ds_sample_ar(h, torch.zeros(2, dtype=torch.int64), torch.zeros((2, 1025), dtype=bf),
                        torch.zeros((2, 33), dtype=i32), None, torch.zeros(2, dtype=i32), torch.zeros(2), 0,
                        torch.zeros(2, dtype=i32), torch.zeros(2))
    # fixed-shape call: u like c, outputs cover [C, positions]
    prm = [torch.zeros(2, dtype=torch.int64), torch.zeros(2, dtype=i32), torch.zeros(2, dtype=i32),
           torch.zeros(2), torch.zeros(2)]
    with pytest.raises(ValueError):
        ds.ds_sample_device_params(h, prm[0], torch.zeros((1, 8, 1025), dtype=bf),
                                   torch.zeros((1, 7, 1025), dtype=bf), *prm[1:], num_rows=1, seed=0,
                                   tokens_out=torch.zeros(8, dtype=i32), logprobs_out=torch.zeros(8))
    with pytest.raises(ValueError):
        ds.ds_sample_device_params(h, prm[0], torch.zeros((1, 8, 1025), dtype=bf), None, *prm[1:], num_rows=1,
                                   seed=0, tokens_out=torch.zeros(7, dtype=i32), logprobs_out=torch.zeros(8))
    # reveal: scores [C, sum(seq_lens)] float32, outputs of sum(reveal_counts)
    with pytest.raises(ValueError):
        ds.ds_reveal_topk(0xABD0, torch.zeros((2, 9)), 2, [4, 6], [3, 1], torch.zeros(4, dtype=i32))
    with pytest.raises(ValueError):
        ds.ds_reveal_topk(0xABD0, torch.zeros((2, 10)), 2, [4, 6], [3, 1], torch.zeros(3, dtype=i32))
    with pytest.raises(TypeError):
        ds.ds_reveal_topk(0xABD0, torch.zeros((2, 10), dtype=torch.float64), 2, [4, 6], [3, 1],
                          torch.zeros(4, dtype=i32))
    # a handle the binding never created
    with pytest.raises(ValueError, match="handle"):
        ds.ds_greedy_lse(0x1234, torch.zeros((4, 1025), dtype=bf), 4, torch.zeros(4, dtype=i32),
                         torch.zeros(4), torch.zeros(4))
