"""MI355X-native per-position full-vocabulary sampler.

The compute lives in ``libdssample.so`` (hand-written HIP for gfx950, C ABI in
``include/ds_sample.h``).  This package is a thin binding: the ``ds_*`` functions
mirror the C entry points one to one, and ``Sampler`` wraps a handle and allocates
output tensors with torch.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from ._binding import (  # noqa: F401
    DS_DTYPE_BF16,
    DS_DTYPE_F32,
    DS_ERR_CAPACITY,
    DS_ERR_HIP,
    DS_ERR_INVALID_ARG,
    DS_ERR_NO_MEMORY,
    DS_ERR_UNSUPPORTED,
    DS_FLAG_COMPACT_U,
    DS_FLAG_FORCE_FALLBACK,
    DS_FLAG_NONE,
    DS_OK,
    DSError,
    EXPORTED,
    LIB_PATH,
    RequestStage,
    ds_greedy_lse,
    ds_last_error,
    ds_repetition_penalty,
    ds_reveal_topk,
    ds_sample_ar,
    ds_sample,
    ds_sample_create,
    ds_sample_destroy,
    ds_read_probe,
    ds_sample_device_params,
    ds_sample_static,
    ds_version,
    lib,
)


class Sampler:
    """A sampler handle for one vocabulary size and logit dtype.

    ``sample`` follows the diffusion sampler contract
    ``sample(request_ids, c_logits, u_logits, seq_lens, iterations) -> (tokens,
    logprobs)`` with per-request guidance scale and temperature;
    ``greedy_lse`` is the draft path's (token, lse, logprob) reduction;
    ``reveal_topk`` ranks each request's cells by a confidence score and returns
    the best ones.  With ``compact_u`` the u logits of ``sample`` hold only the
    positions of requests whose guidance scale is not 0, in request order.
    """

    def __init__(self, vocab: int, dtype: str = "bf16", *, max_rows: int = 8,
                 max_positions: int = 4096, max_requests: int = 64, top_k: int = 0,
                 vocab_chunks: int = 1, device: int = 0, force_fallback: bool = False,
                 compact_u: bool = False):
        if dtype not in ("bf16", "f32"):
            raise ValueError("dtype must be 'bf16' or 'f32'")
        self.vocab = vocab
        self.dtype = dtype
        self.device = device
        self.vocab_chunks = vocab_chunks
        flags = (DS_FLAG_FORCE_FALLBACK if force_fallback else DS_FLAG_NONE) | (
            DS_FLAG_COMPACT_U if compact_u else DS_FLAG_NONE)
        self._h = ds_sample_create(device, vocab, DS_DTYPE_BF16 if dtype == "bf16" else DS_DTYPE_F32,
                                   max_rows, max_positions, max_requests, top_k, vocab_chunks, flags)
        self._stage = RequestStage(max_requests)
        # the C function itself, held by the object: at interpreter exit the
        # modules' globals (this binding's included) may be gone before a
        # sampler that is still alive is collected
        self._destroy = lib().ds_sample_destroy

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def sample(self, request_ids: Sequence[int], c_logits, u_logits, seq_lens: Sequence[int],
               iterations: Sequence[int], guidance_scale: Sequence[float],
               temperature: Sequence[float], seed: int = 0, threshold: bool = False,
               out=None, stream=None):
        """Returns (tokens int32 [C, P], logprobs float32 [C, P]) and, with
        threshold=True, the per-cell top-ratio threshold as a third tensor."""
        C_ = int(c_logits.shape[0])
        if out is None:
            import torch

            P, dev = int(c_logits.shape[1]), c_logits.device
            tokens = torch.empty((C_, P), dtype=torch.int32, device=dev)
            logprobs = torch.empty((C_, P), dtype=torch.float32, device=dev)
            thr = torch.empty((C_, P), dtype=torch.float32, device=dev) if threshold else None
        else:
            tokens, logprobs, thr = out
        ds_sample(self._h, request_ids, c_logits, u_logits, seq_lens, iterations, guidance_scale,
                  temperature, C_, seed, tokens, logprobs, thr, stream, stage=self._stage)
        return (tokens, logprobs, thr) if threshold else (tokens, logprobs)

    def sample_device_params(self, request_ids, c_logits, u_logits, seq_lens, iterations, guidance_scale,
                             temperature, seed: int = 0, threshold: bool = False, out=None, stream=None):
        """``sample`` with the per-request parameters as device tensors, read when
        the call runs (so a captured graph replays with their current values), and
        a fixed layout of c_logits.shape[1] positions: those past sum(seq_lens)
        are padding and their outputs are left as they were."""
        C_ = int(c_logits.shape[0])
        if out is None:
            import torch

            P, dev = int(c_logits.shape[1]), c_logits.device
            tokens = torch.empty((C_, P), dtype=torch.int32, device=dev)
            logprobs = torch.empty((C_, P), dtype=torch.float32, device=dev)
            thr = torch.empty((C_, P), dtype=torch.float32, device=dev) if threshold else None
        else:
            tokens, logprobs, thr = out
        ds_sample_device_params(self._h, request_ids, c_logits, u_logits, seq_lens, iterations, guidance_scale,
                                temperature, C_, seed, tokens, logprobs, thr, stream)
        return (tokens, logprobs, thr) if threshold else (tokens, logprobs)

    def greedy_lse(self, logits, triples: bool = False, out=None, stream=None):
        """logits [n_rows, V] -> (token int32, lse float32, logprob float32)
        [, triples float32 [vocab_chunks, n_rows, 3] with the id bit-cast]."""
        import torch

        n = int(logits.shape[0])
        dev = logits.device
        if out is None:
            tok = torch.empty(n, dtype=torch.int32, device=dev)
            lse = torch.empty(n, dtype=torch.float32, device=dev)
            lp = torch.empty(n, dtype=torch.float32, device=dev)
            tri = torch.empty((self.vocab_chunks, n, 3), dtype=torch.float32, device=dev) if triples else None
        else:
            tok, lse, lp, tri = out
        ds_greedy_lse(self._h, logits, n, tok, lse, lp, tri, stream)
        return (tok, lse, lp, tri) if triples else (tok, lse, lp)

    def repetition_penalty(self, logits, seen_mask, penalty, stream=None):
        """In place over logits [n_rows, V]: every id set in the row's seen_mask
        (int32 [n_rows, ceil(V / 32)] holding the uint32 words) takes x / theta
        when x > 0, else x * theta, with theta = penalty[row] (float32 device
        tensor).  Returns logits."""
        ds_repetition_penalty(self._h, logits, int(logits.shape[0]), seen_mask, penalty, stream)
        return logits

    def sample_ar(self, request_ids, logits, seen_mask, penalty, iterations, temperature, seed: int = 0,
                  out=None, stream=None):
        """Autoregressive step, one token per request, in one call: the
        repetition penalty in place on logits [R, V] (seen_mask and penalty may
        both be None), then each row sampled as the only position of its request
        (guidance 0) with the handle's top_k.  request_ids (int64), iterations
        (int32) and temperature (float32) are [R] device tensors; host sequences
        are copied to the device first.  Returns (tokens int32 [R], logprobs
        float32 [R])."""
        import torch

        R, dev = int(logits.shape[0]), logits.device

        def on_dev(x, dt):
            return x if isinstance(x, torch.Tensor) else torch.tensor(np.asarray(x), dtype=dt, device=dev)

        rid = on_dev(request_ids, torch.int64)
        it = on_dev(iterations, torch.int32)
        tp = on_dev(temperature, torch.float32)
        if out is None:
            out = (torch.empty(R, dtype=torch.int32, device=dev), torch.empty(R, dtype=torch.float32, device=dev))
        ds_sample_ar(self._h, rid, logits, seen_mask, penalty, it, tp, seed, out[0], out[1], stream)
        return out

    def reveal_topk(self, scores, seq_lens: Sequence[int], reveal_counts: Sequence[int], out=None,
                    stream=None):
        """scores float32 [C, P] -> (index int32 [sum(reveal_counts)], score float32
        [sum(reveal_counts)]): per request, the flattened indices c * T_r + t of
        its best cells, best first, and their scores."""
        if out is None:
            import torch

            total = int(sum(int(k) for k in reveal_counts))
            idx = torch.empty(max(total, 1), dtype=torch.int32, device=scores.device)[:total]
            val = torch.empty(max(total, 1), dtype=torch.float32, device=scores.device)[:total]
        else:
            idx, val = out
        ds_reveal_topk(self._h, scores, int(scores.shape[0]), seq_lens, reveal_counts, idx, val, stream,
                       stage=self._stage)
        return idx, val
