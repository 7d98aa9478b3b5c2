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
