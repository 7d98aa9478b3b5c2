"""CPU oracle for the per-position full-vocabulary sampling reduction.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package; the product library
(``vocab_wise_logit_amd``) never does.  The arithmetic lives in ``ds_oracle.c``
(plain C, double precision, built with gcc); this module only marshals numpy arrays.

Functions with no external pin are listed as "parity unpinned" in the C header
comment and in the design doc; at present every exported function has at least one pin
in ``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .build_oracle import LIB, build

F32, BF16 = 0, 1
_lib = None


def _load(path: Optional[str] = None):
    global _lib
    if path is not None:
        return _setup(C.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = _setup(C.CDLL(LIB))
    return _lib


def load_variant(path: str):
    """Load another build of the oracle (used by the mutation tests)."""
    return _setup(C.CDLL(path))


def _setup(lib):
    P = C.c_void_p
    lib.dso_last_error.restype = C.c_char_p
    lib.dso_bf16_to_f32_array.argtypes = [P, P, C.c_int64]
    lib.dso_guided_logit.restype = C.c_float
    lib.dso_guided_logit.argtypes = [C.c_float, C.c_float, C.c_float]
    lib.dso_order_key.restype = C.c_uint32
    lib.dso_order_key.argtypes = [C.c_float]
    lib.dso_lse.restype = C.c_double
    lib.dso_lse.argtypes = [P, C.c_int64]
    lib.dso_row_logprobs.restype = C.c_int
    lib.dso_row_logprobs.argtypes = [C.c_int, P, P, C.c_float, C.c_int32, P, P]
    lib.dso_philox4x32_10.argtypes = [P, P, P]
    lib.dso_noise_word.restype = C.c_uint32
    lib.dso_noise_word.argtypes = [C.c_uint64, C.c_int64, C.c_int32, C.c_int32, C.c_int32,
                                   C.c_int32]
    lib.dso_uniform.restype = C.c_double
    lib.dso_uniform.argtypes = [C.c_uint32]
    lib.dso_gumbel.restype = C.c_double
    lib.dso_gumbel.argtypes = [C.c_uint32]
    lib.dso_kth_largest.restype = C.c_float
    lib.dso_kth_largest.argtypes = [P, C.c_int64, C.c_int64]
    lib.dso_sample.restype = C.c_int
    lib.dso_sample.argtypes = [C.c_int, C.c_int32, C.c_int32, P, P, C.c_int32, P, P, P, P, P,
                               C.c_int32, C.c_uint64, P, C.c_int64, P, P, P, P, P, P, P]
    lib.dso_merge_triples.argtypes = [P, P, P]
    lib.dso_greedy_lse.restype = C.c_int
    lib.dso_reveal_topk.restype = C.c_int
    lib.dso_reveal_topk.argtypes = [P, C.c_int32, C.c_int64, P, P, C.c_int32, P, P]
    lib.dso_greedy_lse.argtypes = [C.c_int, C.c_int32, P, P, C.c_int64, C.c_int32, P, P, P, P,
                                   P, P]
    lib.dso_f32_to_bf16.restype = C.c_uint16
    lib.dso_f32_to_bf16.argtypes = [C.c_float]
    lib.dso_philox_range.argtypes = [P, P, C.c_int64, P]
    lib.dso_noise_words.argtypes = [C.c_uint64, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                    C.c_int64, P]
    lib.dso_gumbel_array.argtypes = [P, C.c_int64, P]
    lib.dso_penalized.restype = C.c_float
    lib.dso_penalized.argtypes = [C.c_float, C.c_float]
    lib.dso_repetition_penalty.restype = C.c_int
    lib.dso_repetition_penalty.argtypes = [C.c_int, C.c_int32, P, P, P, C.c_int64]
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _err(lib) -> str:
    return lib.dso_last_error().decode()


def _dtype_code(arr: np.ndarray) -> int:
    if arr.dtype == np.uint16:
        return BF16
    if arr.dtype == np.float32:
        return F32
    raise TypeError(f"logits must be float32 or bf16 bit patterns (uint16), got {arr.dtype}")


# ----------------------------------------------------------------- pieces

def bf16_to_f32(bits: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or _load()
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    lib.dso_bf16_to_f32_array(_ptr(b), _ptr(out), b.size)
    return out


def guided_logit(c: float, u: float, s: float, lib=None) -> float:
    lib = lib or _load()
    return float(np.float32(lib.dso_guided_logit(c, u, s)))


def order_key(x: float, lib=None) -> int:
    return int((lib or _load()).dso_order_key(x))


def lse(x: np.ndarray, lib=None) -> float:
    lib = lib or _load()
    a = np.ascontiguousarray(x, dtype=np.float64)
    return float(lib.dso_lse(_ptr(a), a.size))


def row_logprobs(c_row: np.ndarray, u_row: Optional[np.ndarray], s: float, lib=None) -> np.ndarray:
    lib = lib or _load()
    c_row = np.ascontiguousarray(c_row)
    dt = _dtype_code(c_row)
    V = c_row.size
    u_row = None if u_row is None else np.ascontiguousarray(u_row, dtype=c_row.dtype)
    lp = np.empty(V, dtype=np.float64)
    work = np.empty(2 * V, dtype=np.float64)
    rc = lib.dso_row_logprobs(dt, _ptr(c_row), _ptr(u_row), s, V, _ptr(lp), _ptr(work))
    if rc:
        raise ValueError(_err(lib))
    return lp


def philox4x32_10(ctr, key, lib=None) -> np.ndarray:
    lib = lib or _load()
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.empty(4, dtype=np.uint32)
    lib.dso_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def philox_range(ctr, key, n: int, lib=None) -> np.ndarray:
    """[n, 4] Philox4x32-10 words of the counters (ctr[0] + i, ctr[1], ctr[2],
    ctr[3]), i = 0 .. n - 1 (the first word wrapping modulo 2^32)."""
    lib = lib or _load()
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.empty((n, 4), dtype=np.uint32)
    lib.dso_philox_range(_ptr(c), _ptr(k), n, _ptr(out))
    return out


def noise_words(seed: int, request_id: int, iteration: int, row: int, t: int, v0: int, n: int,
                lib=None) -> np.ndarray:
    """Noise words of ids v0 .. v0 + n - 1 of one cell."""
    lib = lib or _load()
    out = np.empty(n, dtype=np.uint32)
    lib.dso_noise_words(seed, request_id, iteration, row, t, v0, n, _ptr(out))
    return out


def gumbel_array(x: np.ndarray, lib=None) -> np.ndarray:
    """Gumbel values (double) of an array of noise words."""
    lib = lib or _load()
    xs = np.ascontiguousarray(x, dtype=np.uint32)
    out = np.empty(xs.shape, dtype=np.float64)
    lib.dso_gumbel_array(_ptr(xs), xs.size, _ptr(out))
    return out


def noise_word(seed: int, request_id: int, iteration: int, row: int, t: int, v: int,
               lib=None) -> int:
    return int((lib or _load()).dso_noise_word(seed, request_id, iteration, row, t, v))


def uniform(x: int, lib=None) -> float:
    return float((lib or _load()).dso_uniform(x))


def gumbel(x: int, lib=None) -> float:
    return float((lib or _load()).dso_gumbel(x))


def kth_largest(h: np.ndarray, k: int, lib=None) -> float:
    lib = lib or _load()
    a = np.ascontiguousarray(h, dtype=np.float32)
    return float(np.float32(lib.dso_kth_largest(_ptr(a), a.size, k)))


def merge_triples(a, b, lib=None):
    lib = lib or _load()
    x = np.asarray(a, dtype=np.float64).copy()
    y = np.asarray(b, dtype=np.float64).copy()
    out = np.empty(3, dtype=np.float64)
    lib.dso_merge_triples(_ptr(x), _ptr(y), _ptr(out))
    return out


# ------------------------------------------------------------- whole calls

@dataclass
class SampleResult:
    cells: np.ndarray
    tokens: np.ndarray
    logprobs: np.ndarray
    thresholds: np.ndarray
    gaps: np.ndarray
    near_tie: np.ndarray
    max_h: np.ndarray
    lse_h: np.ndarray


def sample(*, c: np.ndarray, u: Optional[np.ndarray], seq_lens, request_ids, iterations,
           guidance, temperature, rows: int, seed: int, top_k: int = 0,
           cells: Optional[np.ndarray] = None, lib=None) -> SampleResult:
    """Oracle of one sampler call.  c, u: [rows, P, V] float32 or bf16 bits (uint16).
    ``cells`` selects a subset of cell indices (row * P + p); default: all."""
    lib = lib or _load()
    c = np.ascontiguousarray(c)
    dt = _dtype_code(c)
    V = int(c.shape[-1])
    u = None if u is None else np.ascontiguousarray(u, dtype=c.dtype)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    request_ids = np.ascontiguousarray(request_ids, dtype=np.int64)
    iterations = np.ascontiguousarray(iterations, dtype=np.int32)
    guidance = np.ascontiguousarray(guidance, dtype=np.float32)
    temperature = np.ascontiguousarray(temperature, dtype=np.float32)
    P = int(seq_lens.sum())
    if cells is None:
        cells = np.arange(rows * P, dtype=np.int64)
    cells = np.ascontiguousarray(cells, dtype=np.int64)
    n = cells.size
    out = SampleResult(cells=cells, tokens=np.empty(n, np.int32), logprobs=np.empty(n, np.float32),
                       thresholds=np.empty(n, np.float32), gaps=np.empty(n, np.float64),
                       near_tie=np.empty(n, np.uint8), max_h=np.empty(n, np.float32),
                       lse_h=np.empty(n, np.float64))
    rc = lib.dso_sample(dt, V, top_k, _ptr(c), _ptr(u), seq_lens.size, _ptr(seq_lens),
                        _ptr(request_ids), _ptr(iterations), _ptr(guidance), _ptr(temperature),
                        rows, seed, _ptr(cells), n, _ptr(out.tokens), _ptr(out.logprobs),
                        _ptr(out.thresholds), _ptr(out.gaps), _ptr(out.near_tie),
                        _ptr(out.max_h), _ptr(out.lse_h))
    if rc:
        raise ValueError(_err(lib))
    return out


def sample_workload(w, cells: Optional[np.ndarray] = None, lib=None) -> SampleResult:
    """Oracle of a ``synth.DiffusionWorkload``."""
    return sample(c=w.c, u=w.u, seq_lens=w.seq_lens, request_ids=w.request_ids,
                  iterations=w.iterations, guidance=w.guidance, temperature=w.temperature,
                  rows=w.rows, seed=w.seed, top_k=w.top_k, cells=cells, lib=lib)


@dataclass
class GreedyResult:
    rows: np.ndarray
    token: np.ndarray
    lse: np.ndarray
    logprob: np.ndarray
    triples: Optional[np.ndarray]
    dense_token: np.ndarray
    dense_lse: np.ndarray


def greedy_lse(x: np.ndarray, vocab_chunks: int = 1, rows: Optional[np.ndarray] = None,
               want_triples: bool = True, lib=None) -> GreedyResult:
    """Oracle of the draft greedy path.  x: [n_rows, V] float32 or bf16 bits."""
    lib = lib or _load()
    x = np.ascontiguousarray(x)
    dt = _dtype_code(x)
    V = int(x.shape[-1])
    n_all = x.size // V
    rows = np.arange(n_all, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    n = rows.size
    token = np.empty(n, np.int32)
    lse_ = np.empty(n, np.float64)
    lp = np.empty(n, np.float64)
    trip = np.empty((vocab_chunks, n, 3), np.float64) if want_triples else None
    dtok = np.empty(n, np.int32)
    dlse = np.empty(n, np.float64)
    rc = lib.dso_greedy_lse(dt, V, _ptr(x), _ptr(rows), n, vocab_chunks, _ptr(token), _ptr(lse_),
                            _ptr(lp), _ptr(trip), _ptr(dtok), _ptr(dlse))
    if rc:
        raise ValueError(_err(lib))
    return GreedyResult(rows=rows, token=token, lse=lse_, logprob=lp, triples=trip,
                        dense_token=dtok, dense_lse=dlse)


def f32_to_bf16(x: np.ndarray, lib=None) -> np.ndarray:
    """binary32 values to bf16 bit patterns, round to nearest even."""
    lib = lib or _load()
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    return np.array([lib.dso_f32_to_bf16(float(v)) for v in x], dtype=np.uint16)


def penalized(x: float, theta: float, lib=None) -> float:
    lib = lib or _load()
    return float(np.float32(lib.dso_penalized(float(x), float(theta))))


def repetition_penalty(logits: np.ndarray, seen: np.ndarray, theta, lib=None) -> np.ndarray:
    """The repetition penalty over [n_rows, V] logits (float32 or bf16 bits) and
    [n_rows, ceil(V / 32)] uint32 seen masks; returns a penalised copy."""
    lib = lib or _load()
    out = np.array(logits, copy=True, order="C")
    dt = _dtype_code(out)
    V = int(out.shape[-1])
    n = out.size // V
    seen = np.ascontiguousarray(seen, dtype=np.uint32)
    th = np.ascontiguousarray(np.broadcast_to(np.asarray(theta, np.float32), (n,)))
    if seen.shape != (n, (V + 31) // 32):
        raise ValueError("seen mask must be [n_rows, ceil(V / 32)]")
    rc = lib.dso_repetition_penalty(dt, V, _ptr(out), _ptr(seen), _ptr(th), n)
    if rc:
        raise ValueError(_err(lib))
    return out


def ar_step(w, lib=None):
    """Oracle of one autoregressive step (a ``synth.ARWorkload``): the repetition
    penalty, then every row sampled as one position of its request with guidance
    0.  Returns (penalised logits, SampleResult over the R cells)."""
    pen = repetition_penalty(w.logits, w.seen, w.penalty, lib=lib)
    R = pen.shape[0]
    res = sample(c=pen.reshape(1, R, w.vocab), u=None, seq_lens=np.ones(R, np.int32),
                 request_ids=w.request_ids, iterations=w.iterations, guidance=np.zeros(R, np.float32),
                 temperature=w.temperature, rows=1, seed=w.seed, top_k=w.top_k, lib=lib)
    return pen, res


def reveal_topk(scores: np.ndarray, seq_lens, reveal_counts, lib=None):
    """Per request, the reveal_counts[r] best cells of its [C, T_r] block of the
    packed [C, P] scores: (flattened indices c * T_r + t, scores), concatenated
    over the requests in order, each request's best first."""
    lib = lib or _load()
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    Cn, P = scores.shape
    seq = np.ascontiguousarray(seq_lens, dtype=np.int32)
    rev = np.ascontiguousarray(reveal_counts, dtype=np.int32)
    total = int(rev.sum())
    idx = np.empty(max(total, 1), dtype=np.int64)
    val = np.empty(max(total, 1), dtype=np.float32)
    rc = lib.dso_reveal_topk(_ptr(scores), Cn, P, _ptr(seq), _ptr(rev), int(seq.size), _ptr(idx), _ptr(val))
    if rc != 0:
        raise ValueError(_err(lib))
    return idx[:total], val[:total]
