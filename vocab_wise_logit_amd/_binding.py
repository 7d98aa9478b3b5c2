"""ctypes binding of libdssample.so: argument marshalling only.

Functions carry the C entry points' names (ds_sample_create, ds_sample,
ds_sample_device_params, ds_greedy_lse, ds_reveal_topk, ds_repetition_penalty, ds_sample_ar,
ds_sample_destroy,
ds_last_error, ds_version).  Device buffers are
torch tensors on a HIP device (torch supplies memory and streams); per-request
arrays are host sequences.  Every computation happens in the HIP library; when the
library is missing the calls raise instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdssample.so")

DS_DTYPE_F32, DS_DTYPE_BF16 = 0, 1
DS_OK, DS_ERR_INVALID_ARG, DS_ERR_UNSUPPORTED, DS_ERR_CAPACITY, DS_ERR_NO_MEMORY, DS_ERR_HIP = range(6)
DS_FLAG_NONE, DS_FLAG_FORCE_FALLBACK, DS_FLAG_COMPACT_U = 0, 1, 2

EXPORTED = ("ds_sample_create", "ds_sample", "ds_sample_device_params", "ds_greedy_lse", "ds_reveal_topk",
            "ds_repetition_penalty", "ds_sample_ar", "ds_sample_destroy", "ds_last_error", "ds_version",
            "ds_read_probe", "ds_sample_static")

_lib = None

# What each live handle was created for, keyed by its address: (vocab, dtype,
# vocab_chunks, flags).  The calls below check the shapes and element types of the
# tensors they are given against it before calling into the library, which
# trusts the sizes it derives from its arguments (a short or mistyped tensor would
# otherwise be read or written past its end).
_HANDLES: dict = {}


class DSError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m vocab_wise_logit_amd.build`")
        # torch ships its own HIP runtime and loads it into the global symbol
        # scope; loaded after it, the library's HIP calls bind to that same
        # runtime, so its streams and memory are the library's.  Loaded first, the
        # library would start the system HIP runtime, and torch's own could then
        # not open the device.
        import torch  # noqa: F401
        L = C.CDLL(LIB_PATH)
        P, I32, I64, U32, U64 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32, C.c_uint64
        L.ds_sample_create.restype = C.c_int
        L.ds_sample_create.argtypes = [C.POINTER(P), C.c_int, I32, I32, I32, I64, I32, I32, I32, U32]
        L.ds_sample.restype = C.c_int
        L.ds_sample.argtypes = [P, P, P, P, P, P, P, P, I32, I32, U64, P, P, P, P]
        L.ds_sample_device_params.restype = C.c_int
        L.ds_sample_device_params.argtypes = [P, P, P, P, P, P, P, P, I32, I32, I64, U64, P, P, P, P]
        L.ds_greedy_lse.restype = C.c_int
        L.ds_greedy_lse.argtypes = [P, P, I64, P, P, P, P, P]
        L.ds_reveal_topk.restype = C.c_int
        L.ds_reveal_topk.argtypes = [P, P, I32, P, P, I32, P, P, P]
        L.ds_repetition_penalty.restype = C.c_int
        L.ds_repetition_penalty.argtypes = [P, P, I64, P, P, P]
        L.ds_sample_ar.restype = C.c_int
        L.ds_sample_ar.argtypes = [P, P, P, P, P, P, P, I32, U64, P, P, P]
        L.ds_sample_destroy.restype = None
        L.ds_sample_destroy.argtypes = [P]
        L.ds_last_error.restype = C.c_char_p
        L.ds_last_error.argtypes = []
        L.ds_version.restype = C.c_int
        L.ds_version.argtypes = []
        L.ds_sample_static.restype = C.c_int
        L.ds_sample_static.argtypes = [I32, I32, I32, I32, U32, P, P, P, P, P, P, P, I32, I32, U64, P, P, P, P]
        L.ds_read_probe.restype = C.c_int
        L.ds_read_probe.argtypes = [P, I64, I64, I32, P, P]
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != DS_OK:
        raise DSError(rc, lib().ds_last_error().decode())


_torch = None


def _t():
    global _torch
    if _torch is None:
        import torch

        _torch = torch
    return _torch


def _dev_ptr(t, what: str, dtype=None) -> Optional[int]:
    if t is None:
        return None
    torch = _t()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor on a HIP device")
    if not t.is_cuda:
        raise ValueError(f"{what} must live on a HIP device (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must have dtype {dtype} (got {t.dtype})")
    return t.data_ptr()


def _info(handle: int):
    info = _HANDLES.get(handle)
    if info is None:
        raise ValueError("unknown or destroyed sampler handle")
    return info


def _logit_dtype(code: int):
    torch = _t()
    return torch.bfloat16 if code == DS_DTYPE_BF16 else torch.float32


def _need_shape(t, what: str, shape: tuple) -> None:
    """t must be a torch tensor of exactly `shape`."""
    torch = _t()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor on a HIP device")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _need_logits(t, what: str, shape: tuple, code: int) -> None:
    _need_shape(t, what, shape)
    if t.dtype != _logit_dtype(code):
        raise TypeError(f"{what} must have dtype {_logit_dtype(code)} like the sampler (got {t.dtype})")


def _need_numel(t, what: str, n: int, dtype) -> None:
    """t (if given) must hold at least n elements of dtype."""
    if t is None:
        return
    torch = _t()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor on a HIP device")
    if t.dtype != dtype:
        raise TypeError(f"{what} must have dtype {dtype} (got {t.dtype})")
    if t.numel() < n:
        raise ValueError(f"{what} holds {t.numel()} elements; the call writes or reads {n}")


def _host(a, dtype) -> np.ndarray:
    if type(a) is np.ndarray and a.dtype == dtype and a.flags.c_contiguous:
        return a
    return np.ascontiguousarray(a, dtype=dtype)


def _stream_ptr(stream, like=None) -> Optional[int]:
    """The stream handle: the given one, else torch's current stream on the device
    of tensor `like` (read without building a Stream object)."""
    if stream is None:
        torch = _t()
        dev = like.get_device() if like is not None else torch.cuda.current_device()
        return torch._C._cuda_getCurrentRawStream(dev)
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def ds_version() -> int:
    return lib().ds_version()


def ds_last_error() -> str:
    return lib().ds_last_error().decode()


def ds_sample_create(device: int, vocab: int, dtype: int, max_rows: int, max_positions: int,
                     max_requests: int, top_k: int = 0, vocab_chunks: int = 1, flags: int = 0) -> int:
    h = C.c_void_p()
    _check(lib().ds_sample_create(C.byref(h), device, vocab, dtype, max_rows, max_positions,
                                  max_requests, top_k, vocab_chunks, flags))
    _HANDLES[h.value] = (int(vocab), int(dtype), int(vocab_chunks), int(flags))
    return h.value


def ds_sample_destroy(handle: int) -> None:
    _HANDLES.pop(handle, None)
    lib().ds_sample_destroy(handle)


class RequestStage:
    """Host arrays for the per-request arguments of ``ds_sample``, allocated once
    with room for `capacity` requests.  Reading a numpy array's address costs about
    a microsecond per array, so a sampler copies each call's values into these
    arrays, whose addresses are read once, instead.  Not for concurrent use."""

    def __init__(self, capacity: int):
        self.capacity = capacity
        self.rid = np.zeros(max(capacity, 1), np.int64)
        self.sl = np.zeros(max(capacity, 1), np.int32)
        self.it = np.zeros(max(capacity, 1), np.int32)
        self.gs = np.zeros(max(capacity, 1), np.float32)
        self.tp = np.zeros(max(capacity, 1), np.float32)
        self.rc = np.zeros(max(capacity, 1), np.int32)
        self.ptrs = tuple(a.ctypes.data for a in (self.rid, self.sl, self.it, self.gs, self.tp))
        self.reveal_ptrs = (self.sl.ctypes.data, self.rc.ctypes.data)

    def fill(self, request_ids, seq_lens, iterations, guidance_scale, temperature) -> int:
        """Copies the values in; returns the request count, or -1 when they do not
        fit (more than `capacity` requests, unequal lengths, not one-dimensional)."""
        try:
            n = len(request_ids)
            if not (0 < n <= self.capacity and len(seq_lens) == len(iterations) == len(guidance_scale)
                    == len(temperature) == n):
                return -1
            self.rid[:n] = request_ids
            self.sl[:n] = seq_lens
            self.it[:n] = iterations
            self.gs[:n] = guidance_scale
            self.tp[:n] = temperature
        except (TypeError, ValueError):
            return -1
        return n

    def fill_reveal(self, seq_lens, reveal_counts) -> int:
        """As `fill`, for the arguments of ``ds_reveal_topk``."""
        try:
            n = len(seq_lens)
            if not (0 < n <= self.capacity and len(reveal_counts) == n):
                return -1
            self.sl[:n] = seq_lens
            self.rc[:n] = reveal_counts
        except (TypeError, ValueError):
            return -1
        return n


def ds_sample(handle: int, request_ids: Sequence[int], c_logits, u_logits, seq_lens: Sequence[int],
              iterations: Sequence[int], guidance_scale: Sequence[float],
              temperature: Sequence[float], num_rows: int, seed: int, tokens_out, logprobs_out,
              threshold_out=None, stream=None, stage: Optional[RequestStage] = None) -> None:
    torch = _t()
    V, code, _, flags = _info(handle)
    n = stage.fill(request_ids, seq_lens, iterations, guidance_scale, temperature) if stage is not None else -1
    if n > 0:
        prid, psl, pit, pgs, ptp = stage.ptrs
        sl, gs = stage.sl[:n], stage.gs[:n]
    else:
        rid = _host(request_ids, np.int64)
        sl = _host(seq_lens, np.int32)
        it = _host(iterations, np.int32)
        gs = _host(guidance_scale, np.float32)
        tp = _host(temperature, np.float32)
        n = rid.size
        if not (sl.size == it.size == gs.size == tp.size == n):
            raise ValueError("per-request arrays must all have num_requests entries")
        prid, psl, pit, pgs, ptp = (a.ctypes.data for a in (rid, sl, it, gs, tp))
    P = int(sl.sum())
    _need_logits(c_logits, "c_logits", (num_rows, P, V), code)
    if u_logits is not None:
        Pu = int(sl[gs != 0].sum()) if flags & DS_FLAG_COMPACT_U else P
        _need_logits(u_logits, "u_logits", (num_rows, Pu, V), code)
    _need_numel(tokens_out, "tokens_out", num_rows * P, torch.int32)
    _need_numel(logprobs_out, "logprobs_out", num_rows * P, torch.float32)
    _need_numel(threshold_out, "threshold_out", num_rows * P, torch.float32)
    cp = _dev_ptr(c_logits, "c_logits")
    up = _dev_ptr(u_logits, "u_logits")
    _check(lib().ds_sample(handle, prid, cp, up, psl, pit, pgs, ptp, n, num_rows, seed & (2**64 - 1),
                           _dev_ptr(tokens_out, "tokens_out", torch.int32),
                           _dev_ptr(logprobs_out, "logprobs_out", torch.float32),
                           _dev_ptr(threshold_out, "threshold_out", torch.float32),
                           _stream_ptr(stream, c_logits)))


def ds_sample_static(vocab: int, dtype: int, top_k: int, vocab_chunks: int, flags: int, request_ids, c_logits,
                     u_logits, seq_lens, iterations, guidance_scale, temperature, num_rows: int, seed: int,
                     tokens_out, logprobs_out, threshold_out=None, stream=None) -> None:
    """ds_sample without a handle: the settings a handle would hold are arguments,
    and the library's static scratch replaces the handle's workspace, so the call
    allocates no device memory (the caller passes every output).  Host
    per-request sequences; device tensors as for ds_sample."""
    torch = _t()
    rid = _host(request_ids, np.int64)
    sl = _host(seq_lens, np.int32)
    it = _host(iterations, np.int32)
    gs = _host(guidance_scale, np.float32)
    tp = _host(temperature, np.float32)
    n = rid.size
    if not (sl.size == it.size == gs.size == tp.size == n):
        raise ValueError("per-request arrays must all have num_requests entries")
    P = int(sl.sum())
    _need_logits(c_logits, "c_logits", (num_rows, P, vocab), dtype)
    if u_logits is not None:
        Pu = int(sl[gs != 0].sum()) if flags & DS_FLAG_COMPACT_U else P
        _need_logits(u_logits, "u_logits", (num_rows, Pu, vocab), dtype)
    _need_numel(tokens_out, "tokens_out", num_rows * P, torch.int32)
    _need_numel(logprobs_out, "logprobs_out", num_rows * P, torch.float32)
    _need_numel(threshold_out, "threshold_out", num_rows * P, torch.float32)
    ptrs = (_dev_ptr(c_logits, "c_logits"), _dev_ptr(u_logits, "u_logits"), _dev_ptr(tokens_out, "tokens_out"),
            _dev_ptr(logprobs_out, "logprobs_out"), _dev_ptr(threshold_out, "threshold_out"))
    _check(lib().ds_sample_static(vocab, dtype, top_k, vocab_chunks, flags, rid.ctypes.data, ptrs[0], ptrs[1],
                                  sl.ctypes.data, it.ctypes.data, gs.ctypes.data, tp.ctypes.data, n, num_rows,
                                  seed & (2**64 - 1), ptrs[2], ptrs[3], ptrs[4], _stream_ptr(stream, c_logits)))


def ds_sample_device_params(handle: int, request_ids, c_logits, u_logits, seq_lens, iterations, guidance_scale,
                            temperature, num_rows: int, seed: int, tokens_out, logprobs_out,
                            threshold_out=None, stream=None) -> None:
    """Per-request parameters are device tensors of num_requests entries (int64
    ids, int32 lengths and iterations, float32 guidance and temperature); the
    packed layout's positions are c_logits.shape[1]."""
    torch = _t()
    V, code, _, _ = _info(handle)
    if not isinstance(request_ids, torch.Tensor):
        raise TypeError("request_ids must be a device tensor")
    n = int(request_ids.numel())
    for t, what in ((seq_lens, "seq_lens"), (iterations, "iterations"), (guidance_scale, "guidance_scale"),
                    (temperature, "temperature")):
        if not isinstance(t, torch.Tensor) or int(t.numel()) != n:
            raise ValueError(f"{what} must be a device tensor with as many entries as request_ids")
    if not isinstance(c_logits, torch.Tensor) or c_logits.dim() != 3:
        raise ValueError("c_logits must be a [num_rows, positions, V] tensor")
    positions = int(c_logits.shape[1])
    _need_logits(c_logits, "c_logits", (num_rows, positions, V), code)
    if u_logits is not None:
        _need_logits(u_logits, "u_logits", (num_rows, positions, V), code)
    _need_numel(tokens_out, "tokens_out", num_rows * positions, torch.int32)
    _need_numel(logprobs_out, "logprobs_out", num_rows * positions, torch.float32)
    _need_numel(threshold_out, "threshold_out", num_rows * positions, torch.float32)
    _check(lib().ds_sample_device_params(
        handle, _dev_ptr(request_ids, "request_ids", torch.int64), _dev_ptr(c_logits, "c_logits"),
        _dev_ptr(u_logits, "u_logits"), _dev_ptr(seq_lens, "seq_lens", torch.int32),
        _dev_ptr(iterations, "iterations", torch.int32), _dev_ptr(guidance_scale, "guidance_scale", torch.float32),
        _dev_ptr(temperature, "temperature", torch.float32), n, num_rows, int(c_logits.shape[1]),
        seed & (2**64 - 1), _dev_ptr(tokens_out, "tokens_out", torch.int32),
        _dev_ptr(logprobs_out, "logprobs_out", torch.float32),
        _dev_ptr(threshold_out, "threshold_out", torch.float32), _stream_ptr(stream, c_logits)))


def ds_greedy_lse(handle: int, logits, n_rows: int, token_out, lse_out, logprob_out,
                  triples_out=None, stream=None) -> None:
    torch = _t()
    V, code, chunks, _ = _info(handle)
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2 or logits.shape[0] < n_rows:
        raise ValueError(f"logits must be a [n_rows, V] tensor with at least {n_rows} rows")
    _need_logits(logits, "logits", (int(logits.shape[0]), V), code)
    _need_numel(token_out, "token_out", n_rows, torch.int32)
    _need_numel(lse_out, "lse_out", n_rows, torch.float32)
    _need_numel(logprob_out, "logprob_out", n_rows, torch.float32)
    _need_numel(triples_out, "triples_out", chunks * n_rows * 3, torch.float32)
    _check(lib().ds_greedy_lse(handle, _dev_ptr(logits, "logits"), n_rows,
                               _dev_ptr(token_out, "token_out", torch.int32),
                               _dev_ptr(lse_out, "lse_out", torch.float32),
                               _dev_ptr(logprob_out, "logprob_out", torch.float32),
                               _dev_ptr(triples_out, "triples_out", torch.float32),
                               _stream_ptr(stream, logits)))


def ds_repetition_penalty(handle: int, logits, n_rows: int, seen_mask, penalty, stream=None) -> None:
    """seen_mask: int32 tensor holding the uint32 mask words bit for bit."""
    torch = _t()
    V, code, _, _ = _info(handle)
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2 or logits.shape[0] < n_rows:
        raise ValueError(f"logits must be a [n_rows, V] tensor with at least {n_rows} rows")
    _need_logits(logits, "logits", (int(logits.shape[0]), V), code)
    _need_numel(seen_mask, "seen_mask", n_rows * ((V + 31) // 32), torch.int32)
    _need_numel(penalty, "penalty", n_rows, torch.float32)
    _check(lib().ds_repetition_penalty(handle, _dev_ptr(logits, "logits"), n_rows,
                                       _dev_ptr(seen_mask, "seen_mask", torch.int32),
                                       _dev_ptr(penalty, "penalty", torch.float32), _stream_ptr(stream, logits)))


def ds_sample_ar(handle: int, request_ids, logits, seen_mask, penalty, iterations, temperature, seed: int,
                 tokens_out, logprobs_out, stream=None) -> None:
    """Per-request arrays are device tensors (int64, int32, float32); seen_mask
    and penalty may both be None (no penalty)."""
    torch = _t()
    V, code, _, _ = _info(handle)
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise ValueError("logits must be a [num_requests, V] tensor")
    n = int(logits.shape[0])
    _need_logits(logits, "logits", (n, V), code)
    if (seen_mask is None) != (penalty is None):
        raise ValueError("seen_mask and penalty are given together or not at all")
    _need_numel(seen_mask, "seen_mask", n * ((V + 31) // 32), torch.int32)
    _need_numel(penalty, "penalty", n, torch.float32)
    _need_numel(request_ids, "request_ids", n, torch.int64)
    _need_numel(iterations, "iterations", n, torch.int32)
    _need_numel(temperature, "temperature", n, torch.float32)
    _need_numel(tokens_out, "tokens_out", n, torch.int32)
    _need_numel(logprobs_out, "logprobs_out", n, torch.float32)
    _check(lib().ds_sample_ar(handle, _dev_ptr(request_ids, "request_ids", torch.int64), _dev_ptr(logits, "logits"),
                              _dev_ptr(seen_mask, "seen_mask", torch.int32), _dev_ptr(penalty, "penalty", torch.float32),
                              _dev_ptr(iterations, "iterations", torch.int32),
                              _dev_ptr(temperature, "temperature", torch.float32), n, seed & 0xFFFFFFFFFFFFFFFF,
                              _dev_ptr(tokens_out, "tokens_out", torch.int32),
                              _dev_ptr(logprobs_out, "logprobs_out", torch.float32), _stream_ptr(stream, logits)))


def ds_reveal_topk(handle: int, scores, num_rows: int, seq_lens: Sequence[int],
                   reveal_counts: Sequence[int], index_out, score_out=None, stream=None,
                   stage: Optional[RequestStage] = None) -> None:
    torch = _t()
    _info(handle)
    n = stage.fill_reveal(seq_lens, reveal_counts) if stage is not None else -1
    if n > 0:
        psl, prc = stage.reveal_ptrs
        sl, rc = stage.sl[:n], stage.rc[:n]
    else:
        sl = _host(seq_lens, np.int32)
        rc = _host(reveal_counts, np.int32)
        if sl.size != rc.size:
            raise ValueError("seq_lens and reveal_counts must have num_requests entries")
        n, psl, prc = sl.size, sl.ctypes.data, rc.ctypes.data
    P = int(sl.sum())
    total = int(rc.sum())
    _need_shape(scores, "scores", (num_rows, P))
    if scores.dtype != torch.float32:
        raise TypeError(f"scores must have dtype torch.float32 (got {scores.dtype})")
    _need_numel(index_out, "index_out", total, torch.int32)
    _need_numel(score_out, "score_out", total, torch.float32)
    _check(lib().ds_reveal_topk(handle, _dev_ptr(scores, "scores", torch.float32), num_rows, psl, prc, n,
                                _dev_ptr(index_out, "index_out", torch.int32),
                                _dev_ptr(score_out, "score_out", torch.float32), _stream_ptr(stream, scores)))


def ds_read_probe(x, row_bytes: int, threads: int, sink, stream=None) -> None:
    """Measurement aid: read the bytes of device tensor x once as rows of
    row_bytes, one workgroup of `threads` threads per row; sink (int32, one entry
    per row) receives the xor of each row's words."""
    torch = _t()
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch tensor on a HIP device")
    nbytes = x.numel() * x.element_size()
    if row_bytes <= 0 or nbytes % row_bytes:
        raise ValueError(f"x holds {nbytes} bytes, not a whole number of {row_bytes}-byte rows")
    n_rows = nbytes // row_bytes
    _need_numel(sink, "sink", n_rows, torch.int32)
    _check(lib().ds_read_probe(_dev_ptr(x, "x"), n_rows, row_bytes, threads, _dev_ptr(sink, "sink"),
                               _stream_ptr(stream, x)))
