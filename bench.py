"""Benchmark of the per-position full-vocabulary sampler on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload stress] [--no-suite]

One step is one ``ds_sample`` call over one synthetic batch already resident in
HBM: CFG combine, temperature, top-ratio filter, Gumbel-max and the
full-vocabulary logprob for every (row, position) cell.  The headline workload is
the largest single-GPU configuration: 2048 positions x V=248320 bf16 conditional
and unconditional logits, guidance 1.5, temperature 1.0, top-ratio k=24832, the
vocabulary reduced in 4 contiguous chunks whose (max, lse, argmax) triples are
merged on the GPU.  Input buffers rotate through copies totalling at least 1 GiB
so that neither the L2 nor the 256 MB Infinity Cache serves a repeat.

Prints ONE JSON line: positions/s of the headline step; the roofline of its
kernels (algorithmic bytes over the average duration of the call, timed live with
HIP events on the launch stream), next to a measured read ceiling at the same
bytes and launch shape; the CPU oracle on a bounded sample of the same workload
(one thread and every thread of the host share); the oracle's parity and near-tie
counts per configuration; and the same figures for the other workloads under
"per_config".
"""

from __future__ import annotations

import argparse
import hashlib
import glob
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "sampled positions/sec + achieved HBM GB/s (% of MI355X peak) per config"
ROTATE_BYTES = 1 << 30
SUITE_BUDGET_S = 0.03  # timed work per suite entry
# Untimed work before a timed region: a sustained load after idle runs slower for
# its first 20-30 ms (the large-vocabulary parts kernel goes from 300 to 425 us
# within 3 ms, then back to 300 us by about 25 ms), so every timed region starts
# after at least this much warmup.
WARMUP_MIN_S = 0.05
# threads per workgroup of the one-workgroup-per-row draft kernel and of the
# streaming parts kernel (the launch shapes the read ceilings are measured at)
GREEDY_ROW_THREADS = 512
PARTS_THREADS = 512


# Sources each kernel is built from: a stored counter reading is valid only while
# these files are unchanged.
KERNEL_SOURCES = {
    "small": ("ds_small.hip", "ds_device.h", "ds_kernels.h"),
    "row": ("ds_row.hip", "ds_device.h", "ds_kernels.h"),
    "reveal": ("ds_reveal.hip", "ds_device.h", "ds_kernels.h"),
    "ar": ("ds_penalty.hip", "ds_row.hip", "ds_device.h", "ds_kernels.h"),
}


def kernel_family(workload: str) -> str:
    if workload in ("reveal", "ar"):
        return workload
    return "small" if workload in ("tiny", "omnivoice", "mixed") else "row"


def kernel_source_digest(family: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "vocab_wise_logit_amd", "csrc", name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE +
    WRITE_SIZE, scaled by a copy-kernel calibration), if they were taken on the
    current sources of the workload's kernels; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_digest") != kernel_source_digest(kernel_family(workload)):
        return None
    return t.get("bytes_per_launch")


def to_dev(arr: np.ndarray):
    """Copy a numpy array (float32, or bf16 bit patterns as uint16) to the GPU."""
    import torch

    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def kernel_name(w, kind: str) -> str:
    if kind == "reveal":
        return "k_reveal_topk"
    if kind == "ar":
        # the streaming parts penalise their own ids; the wave-per-cell kernel
        # takes its rows from the penalty kernel
        ks = sampler_kernels(w.vocab, w.dtype)
        dev = [k.replace("_wide", "") + "_dev" + ("_wide" if k.endswith("_wide") else "") for k in ks.split("+")]
        return "+".join(dev if ks.startswith("k_sample_parts") else ["k_repetition_penalty"] + dev)
    if kind == "draft":
        return draft_kernel(w)
    return sampler_kernels(w.vocab, w.dtype)


def sampler_kernels(vocab: int, dtype: str) -> str:
    slots = ((vocab + 2) // 2 if dtype == "bf16" else vocab + 63) // 64
    if slots > (16 if dtype == "bf16" else 32):
        return "k_sample_parts+k_sample_merge"
    return "k_sample_small" if slots <= (9 if dtype == "bf16" else 16) else "k_sample_small_wide"


def draft_kernel(w) -> str:
    """The draft path's kernels, by the library's rule: one workgroup per row when
    the rows fill every compute unit (whole rounds, or the last partial round
    costing at most a tenth) and chunk edges fall on 16-byte pieces; otherwise
    the parts + merge pair."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    epp = 8 if w.dtype == "bf16" else 4
    L = -(-w.vocab // w.vocab_chunks)
    rounds = -(-w.n_rows // cus)
    if (w.n_rows >= cus and w.n_rows * 10 >= rounds * cus * 9 and w.vocab % epp == 0 and L % epp == 0
            and w.vocab_chunks <= 64):
        return "k_greedy_rows"
    return "k_greedy_parts+k_greedy_merge"


_WORKLOADS = {}


def make_workload(name: str):
    """The named synthetic workload, generated once per process (the large ones
    take seconds to draw)."""
    import synth

    if name not in _WORKLOADS:
        _WORKLOADS[name] = synth.tiny(0.9) if name == "tiny" else synth.WORKLOADS[name]()
    return _WORKLOADS[name]


class Runner:
    """Device copies of one workload and a sampler handle; `step(i)` issues one
    call on rotating buffers (asking for the top-ratio thresholds too when
    `threshold` is set).  For sampling workloads, `mode` picks the entry point:
    "eager" calls ds_sample, "device_params" calls ds_sample_device_params with
    the per-request parameters in device memory, and "graph" replays a HIP graph
    holding that call (one captured graph per buffer set)."""

    def __init__(self, w, kind: str, threshold: bool = False, mode: str = "eager"):
        import torch

        import vocab_wise_logit_amd as ds

        self.w, self.kind, self.mode = w, kind, mode
        if kind == "ar":
            # the penalty works in place, so each buffer set is penalised again on
            # every pass over it (same seen ids, same work per step)
            x = to_dev(w.logits)
            per_set = x.numel() * x.element_size()
            self.n_sets = max(1, min(64, math.ceil(ROTATE_BYTES / per_set)))
            self.x = [x] + [x.clone() for _ in range(self.n_sets - 1)]
            self.seen = torch.from_numpy(np.ascontiguousarray(w.seen).view(np.int32)).cuda()
            self.pen = torch.from_numpy(np.ascontiguousarray(w.penalty)).cuda()
            R = w.rows
            self.smp = ds.Sampler(w.vocab, w.dtype, max_rows=1, max_positions=R, max_requests=R, top_k=w.top_k)
            self.out = (torch.empty(R, dtype=torch.int32, device="cuda"),
                        torch.empty(R, dtype=torch.float32, device="cuda"))
            self.prm = (torch.tensor(np.asarray(w.request_ids, np.int64), device="cuda"),
                        torch.tensor(np.asarray(w.iterations, np.int32), device="cuda"),
                        torch.tensor(np.asarray(w.temperature, np.float32), device="cuda"))
            self.cells = R
        elif kind == "reveal":
            x = torch.from_numpy(np.ascontiguousarray(w.scores)).cuda()
            per_set = x.numel() * x.element_size()
            self.n_sets = max(1, min(64, math.ceil(ROTATE_BYTES / per_set)))
            self.x = [x] + [x.clone() for _ in range(self.n_sets - 1)]
            self.smp = ds.Sampler(16, "f32", max_rows=w.rows, max_positions=w.positions,
                                  max_requests=len(w.seq_lens))
            total = int(w.reveal_counts.sum())
            self.out = (torch.empty(total, dtype=torch.int32, device="cuda"),
                        torch.empty(total, dtype=torch.float32, device="cuda"))
            self.cells = w.rows * w.positions
        elif kind == "draft":
            x = to_dev(w.logits)
            per_set = x.numel() * x.element_size()
            self.n_sets = max(1, min(64, math.ceil(ROTATE_BYTES / per_set)))
            self.x = [x] + [x.clone() for _ in range(self.n_sets - 1)]
            n = w.n_rows
            self.smp = ds.Sampler(w.vocab, w.dtype, max_rows=1, max_positions=n,
                                  vocab_chunks=w.vocab_chunks)
            self.out = (torch.empty(n, dtype=torch.int32, device="cuda"),
                        torch.empty(n, dtype=torch.float32, device="cuda"),
                        torch.empty(n, dtype=torch.float32, device="cuda"), None)
            self.cells = n
        else:
            c = to_dev(w.c)
            if mode == "compact_u" and w.u is not None:
                # only the guided requests' positions of u, in request order
                offs = np.concatenate([[0], np.cumsum(w.seq_lens)])
                keep = [np.arange(offs[r], offs[r + 1]) for r in range(len(w.seq_lens)) if w.guidance[r] != 0]
                u = to_dev(np.ascontiguousarray(w.u[:, np.concatenate(keep)])) if keep else None
            else:
                u = to_dev(w.u) if w.u is not None else None
            per_set = c.numel() * c.element_size() + (u.numel() * u.element_size() if u is not None else 0)
            self.n_sets = max(1, min(64, math.ceil(ROTATE_BYTES / per_set)))
            self.c = [c] + [c.clone() for _ in range(self.n_sets - 1)]
            self.u = [u] + [u.clone() for _ in range(self.n_sets - 1)] if u is not None else None
            self.smp = ds.Sampler(w.vocab, w.dtype, max_rows=w.rows, max_positions=w.positions,
                                  max_requests=len(w.seq_lens), top_k=w.top_k,
                                  vocab_chunks=w.vocab_chunks, compact_u=mode == "compact_u")
            shape = (w.rows, w.positions)
            self.out = (torch.empty(shape, dtype=torch.int32, device="cuda"),
                        torch.empty(shape, dtype=torch.float32, device="cuda"),
                        torch.empty(shape, dtype=torch.float32, device="cuda") if threshold else None)
            self.cells = w.cells
            if mode in ("device_params", "graph"):
                self.prm = (torch.tensor(np.asarray(w.request_ids, np.int64), device="cuda"),
                            torch.tensor(np.asarray(w.seq_lens, np.int32), device="cuda"),
                            torch.tensor(np.asarray(w.iterations, np.int32), device="cuda"),
                            torch.tensor(np.asarray(w.guidance, np.float32), device="cuda"),
                            torch.tensor(np.asarray(w.temperature, np.float32), device="cuda"))
            if mode == "graph":
                self.graphs = []
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    self._dev_call(0)
                torch.cuda.current_stream().wait_stream(side)
                for k in range(self.n_sets):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        self._dev_call(k)
                    self.graphs.append(g)
                torch.cuda.synchronize()

    def _dev_call(self, s: int) -> None:
        w = self.w
        self.smp.sample_device_params(self.prm[0], self.c[s], self.u[s] if self.u else None, *self.prm[1:],
                                      seed=w.seed, threshold=self.out[2] is not None, out=self.out)

    def step(self, i: int) -> None:
        s = i % self.n_sets
        w = self.w
        if self.kind == "ar":
            self.smp.sample_ar(self.prm[0], self.x[s], self.seen, self.pen, self.prm[1], self.prm[2],
                               seed=w.seed, out=self.out)
        elif self.kind == "reveal":
            self.smp.reveal_topk(self.x[s], w.seq_lens, w.reveal_counts, out=self.out)
        elif self.kind == "draft":
            self.smp.greedy_lse(self.x[s], out=self.out)
        elif self.mode == "graph":
            self.graphs[s].replay()
        elif self.mode == "device_params":
            self._dev_call(s)
        else:  # eager, or eager with the compacted u layout
            self.smp.sample(w.request_ids, self.c[s], self.u[s] if self.u else None, w.seq_lens,
                            w.iterations, w.guidance, w.temperature, seed=w.seed,
                            threshold=self.out[2] is not None, out=self.out)

    def close(self):
        self.graphs = None
        self.smp.close()


def time_runner(r: Runner, steps: int, warmup: int):
    """(ms per step over the whole timed region, then mean / median / p10 / p90 of
    per-launch times from events recorded around every launch on the same stream;
    the bracketed times include each launch's dispatch gap)."""
    import torch

    for i in range(warmup):
        r.step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        r.step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    # per-launch durations (same stream), second pass over the same buffers
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        r.step(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in evs])
    return ms_step, float(np.mean(per)), float(np.median(per)), float(np.percentile(per, 10)), float(
        np.percentile(per, 90))


def describe(w, kind: str) -> dict:
    if kind == "ar":
        return {"workload": "ar_step", "requests": w.rows, "vocab": w.vocab, "input_dtype": w.dtype,
                "top_k": w.top_k, "seen_ids": w.n_seen(), "penalty": float(w.penalty[0]),
                "temperatures": sorted(set(float(t) for t in w.temperature))}
    if kind == "reveal":
        return {"workload": "confidence_reveal", "requests": int(len(w.seq_lens)), "rows": w.rows,
                "positions": w.positions, "revealed": int(w.reveal_counts.sum())}
    if kind == "draft":
        return {"workload": "draft_greedy", "rows": w.n_rows, "vocab": w.vocab,
                "input_dtype": w.dtype, "vocab_chunks": w.vocab_chunks}
    return {"workload": {"omnivoice": "omnivoice_step", "mixed": "mixed_guidance_batch",
                         "stress": "large_vocab_chunked", "tiny": "tiny_step"}.get(w.name, w.name),
            "requests": int(len(w.seq_lens)), "rows": w.rows, "positions": w.positions,
            "cells": w.cells, "vocab": w.vocab, "input_dtype": w.dtype, "top_k": w.top_k,
            "vocab_chunks": w.vocab_chunks}


def launches_per_step(w, kind: str) -> int:
    """Kernel launches of one call: one for the wave-per-cell kernel and the
    one-workgroup-per-row draft kernel, a parts and a merge kernel for the
    streaming path (every sampling workload here fits one batch).  The
    autoregressive step samples all its requests at once: parts (which apply
    the penalty) and merge, or the penalty kernel and the wave-per-cell kernel."""
    if kind == "ar":
        return 2
    return 1 if kernel_name(w, kind).startswith(("k_sample_small", "k_reveal", "k_greedy_rows")) else 2


def auto_steps(r: "Runner", budget_s: float = SUITE_BUDGET_S) -> tuple:
    """(steps, warmup) for a suite entry: enough steps for about `budget_s` of
    timed work, so that short steps are not timed over a few microseconds."""
    import torch

    for i in range(3):
        r.step(i)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for i in range(10):
        r.step(i)
    torch.cuda.synchronize()
    est = (time.perf_counter() - t) / 10
    steps = int(min(max(budget_s / max(est, 1e-7), 10), 5000))
    return steps, max(steps // 5, math.ceil(WARMUP_MIN_S / max(est, 1e-7)), 3)


def bench_one(name: str, steps, warmup, threshold: bool = False, mode: str = "eager") -> dict:
    """Times one workload; steps=None sizes the run with auto_steps.  The result
    keeps the outputs of the last call (identical on every buffer set) under
    "outputs" for the parity check."""
    import torch

    kind = name if name in ("draft", "reveal", "ar") else "sample"
    w = make_workload(name)
    r = Runner(w, kind, threshold, mode)
    if steps is None:
        steps, warmup = auto_steps(r)
    ms_step, ms_call, med, p10, p90 = time_runner(r, steps, warmup)
    outputs = None
    if kind in ("sample", "draft") and mode == "eager":
        outputs = [t.reshape(-1).cpu().numpy() for t in r.out if t is not None]
    ceiling = None
    if kind == "draft" and draft_kernel(w) == "k_greedy_rows":
        # the same bytes at the same launch shape: one workgroup per row
        ceiling = read_ceiling([(x,) for x in r.x], w.vocab * w.elem_bytes, GREEDY_ROW_THREADS)
    elif kind == "sample" and name == "stress" and mode == "eager" and not threshold:
        # the parts kernel's shape: one 512-thread workgroup per part of a chunk,
        # over c and over u
        L = -(-w.vocab // w.vocab_chunks)
        ceiling = read_ceiling(list(zip(r.c, r.u)), L * w.elem_bytes, PARTS_THREADS)
    r.close()
    del r
    torch.cuda.empty_cache()
    alg = w.algorithmic_bytes()
    # positions: cells sampled, draft rows reduced, or cells ranked by the reveal
    cells = {"draft": lambda: w.n_rows, "reveal": lambda: w.rows * w.positions,
             "ar": lambda: w.rows}.get(kind, lambda: w.cells)()
    # one step is one call: one launch of the wave-per-cell kernel (every
    # sampling workload here has <= 64 requests, one request table), one parts +
    # merge pair, one draft kernel, or the autoregressive step's penalty kernel
    # and sampler launches (launches_per_step); its back-to-back time per step is
    # the call's average duration on its stream
    achieved = alg / (ms_step * 1e-3) / 1e9
    cfg = describe(w, kind)
    if threshold:
        cfg["workload"] += "+threshold"
        cfg["threshold_out"] = True
    kname = kernel_name(w, kind)
    launches = launches_per_step(w, kind)
    if threshold and kname == "k_sample_parts+k_sample_merge":
        # the threshold output on the streaming path: the window kernel first
        kname = "k_sample_window+" + kname
        launches += 1
    if mode in ("device_params", "graph"):
        cfg["workload"] += "+" + mode
        cfg["entry_point"] = "ds_sample_device_params" + (" in a replayed HIP graph" if mode == "graph" else "")
        kname = kname.replace("k_sample_small", "k_sample_small_dev")
    elif mode == "compact_u":
        cfg["workload"] += "+compact_u"
        cfg["u_layout"] = "compacted: guided requests' positions only"
    res = {"config": cfg, "kernel": kname, "launches_per_step": launches,
           "steps": steps, "warmup": warmup, "positions_per_s": cells / (ms_step * 1e-3),
           "ms_per_step": ms_step, "call_ms_mean": ms_step, "bracketed_ms_mean": ms_call,
           "bracketed_ms_median": med, "bracketed_ms_p10": p10, "bracketed_ms_p90": p90, "algorithmic_bytes": alg,
           "achieved_GBs": achieved, "frac_of_peak": achieved / HBM_PEAK_GBS, "workload_obj": w,
           "outputs": outputs}
    if ceiling:
        res["read_ceiling"] = ceiling
        res["frac_of_read_ceiling"] = achieved / ceiling["GBs"]
    return res


def read_ceiling(sets, row_bytes: int, threads: int, budget_s: float = 0.05) -> dict:
    """The HBM read rate of ds_read_probe over the given sets of device tensors
    (one set per step, in rotation; each tensor read as rows of row_bytes, one
    workgroup of `threads` per row): the ceiling for a kernel that reads the same
    bytes at that launch shape."""
    import torch

    import vocab_wise_logit_amd as ds

    sinks = [[torch.empty(b.numel() * b.element_size() // row_bytes, dtype=torch.int32, device="cuda")
              for b in st] for st in sets]
    nbytes = sum(b.numel() * b.element_size() for b in sets[0])

    def one(i):
        k = i % len(sets)
        for b, sk in zip(sets[k], sinks[k]):
            ds.ds_read_probe(b, row_bytes, threads, sk)

    for i in range(3):
        one(i)
    torch.cuda.synchronize()
    t = time.perf_counter()
    one(3)
    torch.cuda.synchronize()
    n = int(min(max(budget_s / max(time.perf_counter() - t, 1e-6), 10), 2000))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        one(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    rows = nbytes // row_bytes
    return {"GBs": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes, "ms": round(ms, 6), "steps": n,
            "shape": f"{rows} workgroups x {threads} threads, {row_bytes} B each",
            "kernel": "k_read_rows (ds_read_probe)"}


# ----------------------------------------------------------- the CPU oracle

def host_threads() -> int:
    """Worker threads for the oracle: the host CPUs this process may use, capped
    at 16 (the share of one GPU on a shared host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    env = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    return max(1, min(n, env or n, 16))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_cells(w, cells: np.ndarray, threads: int):
    """The oracle over the given cells, split across threads (its C entry points
    release the GIL); returns (SampleResult fields concatenated, seconds)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    parts = [p for p in np.array_split(cells, threads) if p.size]
    t = time.perf_counter()
    if len(parts) == 1:
        res = [oracle.sample_workload(w, cells=parts[0])]
    else:
        with ThreadPoolExecutor(len(parts)) as ex:
            res = list(ex.map(lambda p: oracle.sample_workload(w, cells=p), parts))
    dt = time.perf_counter() - t
    cat = {k: np.concatenate([getattr(r, k) for r in res]) for k in ("cells", "tokens", "logprobs", "near_tie")}
    return cat, dt


def parity_report(w, outputs, ref: dict) -> dict:
    """GPU tokens and logprobs against the oracle on the cells it computed: greedy
    cells and cells away from oracle near ties must draw the same token."""
    import synth  # noqa: F401

    cells = ref["cells"]
    tok = outputs[0][cells]
    lp = outputs[1][cells]
    offs = np.concatenate([[0], np.cumsum(w.seq_lens)])
    r = np.searchsorted(offs, cells % max(1, w.positions), side="right") - 1
    greedy = w.temperature[r] == 0
    near = ref["near_tie"].astype(bool) & ~greedy
    same = tok == ref["tokens"]
    err = np.abs(lp[same].astype(np.float64) - ref["logprobs"][same].astype(np.float64))
    return {"cells_checked": int(cells.size), "sampled": int((~greedy).sum()), "near_ties": int(near.sum()),
            "token_mismatch": int((~same & ~near).sum()), "near_tie_other_token": int((~same & near).sum()),
            "max_logprob_err": float(err.max()) if err.size else 0.0}


def cpu_baseline(w, outputs, single_s: float = 6.0, multi_s: float = 10.0) -> tuple:
    """The oracle as it stands (plain C, double precision) on a bounded sample of
    the workload's cells, evenly spread over the batch: about `single_s` seconds
    on one thread, then about `multi_s` seconds on every thread of the host
    share.  Returns (cpu_baseline entry, parity of the GPU outputs on the cells
    the multi-threaded run computed)."""
    import oracle

    threads = host_threads()
    probe = np.linspace(0, w.cells - 1, min(4, w.cells)).astype(np.int64)
    t = time.perf_counter()
    oracle.sample_workload(w, cells=probe)
    per_cell = (time.perf_counter() - t) / probe.size
    n1 = int(min(w.cells, max(probe.size, single_s / max(per_cell, 1e-9))))
    one, dt1 = oracle_cells(w, np.linspace(0, w.cells - 1, n1).astype(np.int64), 1)
    nm = int(min(w.cells, max(threads, multi_s * threads / max(per_cell, 1e-9))))
    cells_m = np.unique(np.linspace(0, w.cells - 1, nm).astype(np.int64))
    many, dtm = oracle_cells(w, cells_m, threads)
    entry = {"value": cells_m.size / dtm, "unit": "positions/s", "cores": threads, "kind": "oracle",
             "sample": (f"{cells_m.size} of the {w.cells} cells, evenly spaced over the batch, on {threads} threads "
                        f"in {dtm:.2f} s; single-threaded: {n1} cells in {dt1:.2f} s"),
             "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
             "single_thread": {"value": n1 / dt1, "unit": "positions/s", "cores": 1, "cells": n1,
                               "seconds": round(dt1, 3)}}
    return entry, parity_report(w, outputs, many) if outputs is not None else None


def draft_parity(w, outputs) -> dict:
    import oracle

    g = oracle.greedy_lse(w.logits, vocab_chunks=w.vocab_chunks, want_triples=False)
    tok, lse = outputs[0], outputs[1]
    return {"rows_checked": int(g.token.size), "token_mismatch": int((tok != g.token).sum()),
            "max_lse_err": float(np.max(np.abs(lse.astype(np.float64) - g.lse)))}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)  # about 65 ms of the headline step: WARMUP_MIN_S
    ap.add_argument("--workload", default="stress")
    ap.add_argument("--no-suite", action="store_true", help="skip the other workloads")
    ap.add_argument("--threshold", action="store_true",
                    help="time the headline workload with the threshold output (for profiling that path)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (10 times), to scale "
                         "the FETCH_SIZE / WRITE_SIZE counters of a profiler run")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the sampler library runs on a single GPU and "
              "has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        return 2

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 10}))
        return 0

    print(f"[bench] headline {args.workload}: {args.steps} steps after {args.warmup} warmup", file=sys.stderr,
          flush=True)
    head = bench_one(args.workload, args.steps, args.warmup, threshold=args.threshold)
    w = head.pop("workload_obj")
    head_out = head.pop("outputs")
    traffic = None if args.threshold else stored_traffic(args.workload)
    roofline = {"bound": "hbm", "achieved": round(head["achieved_GBs"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(head["frac_of_peak"], 4),
                "traffic": traffic,
                "kernel": head["kernel"],
                "algorithmic_bytes_per_launch": head["algorithmic_bytes"],
                "call_ms_mean": head["call_ms_mean"], "bracketed_ms_mean": head["bracketed_ms_mean"]}
    if "read_ceiling" in head:
        roofline["read_ceiling_GBs"] = head["read_ceiling"]["GBs"]
        roofline["frac_of_read_ceiling"] = round(head["frac_of_read_ceiling"], 4)
    per_config, parity = {}, {}
    threads = host_threads()
    if not args.no_suite:
        # every workload, then the two sampled shapes again with the threshold
        # output requested (it needs the exact k-th largest h of every row)
        runs = [(n, False) for n in ("tiny", "omnivoice", "mixed", "draft", "stress", "reveal", "ar")]
        runs += [("omnivoice", True), ("stress", True)]
        runs = [(n, thr, "eager") for n, thr in runs]
        # the fixed-shape entry point with device-resident parameters, called and replayed
        runs += [("omnivoice", False, "device_params"), ("omnivoice", False, "graph")]
        # the mixed batch with u holding only the guided requests' positions
        runs += [("mixed", False, "compact_u")]
        for name, thr, mode in runs:
            if name == args.workload and thr == args.threshold and mode == "eager":
                res = dict(head, outputs=head_out)
            else:
                print(f"[bench] {name} threshold={thr} mode={mode}", file=sys.stderr, flush=True)
                res = bench_one(name, None, None, threshold=thr, mode=mode)
                res.pop("workload_obj", None)
            outs = res.pop("outputs", None)
            if outs is not None and not thr and mode == "eager" and name != args.workload:
                if name == "draft":
                    parity[res["config"]["workload"]] = draft_parity(make_workload(name), outs)
                elif name in ("tiny", "omnivoice", "mixed"):
                    wn = make_workload(name)
                    ref, _ = oracle_cells(wn, np.arange(wn.cells, dtype=np.int64), threads)
                    parity[res["config"]["workload"]] = parity_report(wn, outs, ref)
            entry = {k: (round(v, 6) if isinstance(v, float) else v) for k, v in res.items() if k != "config"}
            if not thr and mode == "eager":
                entry["traffic"] = stored_traffic(name)
            per_config[res["config"]["workload"]] = entry
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        cpu, head_parity = cpu_baseline(w, head_out)
        if head_parity is not None:
            parity[head["config"]["workload"]] = head_parity
    line = {
        "metric": METRIC,
        "value": head["positions_per_s"],
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # every step computes in binary32 (bf16 inputs widen exactly)
        "dtype": "f32",
        "data": "synthetic",
        "config": head["config"],
        "roofline": roofline,
        "read_ceiling": head.get("read_ceiling"),
        "cpu_baseline": cpu,
        "parity": parity,
        "per_config": per_config,
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
