"""Benchmark of the per-position full-vocabulary sampler on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload omnivoice] [--no-suite]

One step is one ``ds_sample`` call over one synthetic batch already resident in
HBM: CFG combine, temperature, exact top-ratio threshold, Gumbel-max and the
full-vocabulary logprob for every (row, position) cell.  The headline workload is
the OmniVoice-shaped masked-diffusion step (8 requests x 8 codebook rows, ragged
lengths 80-120, V=1025 bf16).  Input buffers rotate through copies totalling at
least 1 GiB so that neither the L2 nor the 256 MB Infinity Cache serves a repeat.

Prints ONE JSON line: positions/s for the headline step, the roofline of its
kernel (algorithmic bytes over the kernel's average duration, timed live with HIP
events on the launch stream), the CPU oracle timed on a bounded sample, and the
same figures for the other workloads under "per_config".
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
        dev = [k.replace("_wide", "") + "_dev" + ("_wide" if k.endswith("_wide") else "")
               for k in sampler_kernels(w.vocab, w.dtype).split("+")]
        return "+".join(["k_repetition_penalty"] + dev)
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


def make_workload(name: str):
    import synth

    if name == "tiny":
        return synth.tiny(0.9)
    return synth.WORKLOADS[name]()


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
    autoregressive step is the penalty kernel and then the sampler over all its
    requests at once."""
    if kind == "ar":
        return 1 + (1 if sampler_kernels(w.vocab, w.dtype).startswith("k_sample_small") else 2)
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
    return steps, max(steps // 5, 3)


def bench_one(name: str, steps, warmup, threshold: bool = False, mode: str = "eager") -> dict:
    """Times one workload; steps=None sizes the run with auto_steps."""
    import torch

    kind = name if name in ("draft", "reveal", "ar") else "sample"
    w = make_workload(name)
    r = Runner(w, kind, threshold, mode)
    if steps is None:
        steps, warmup = auto_steps(r)
    ms_step, ms_kernel, med, p10, p90 = time_runner(r, steps, warmup)
    r.close()
    del r
    torch.cuda.empty_cache()
    alg = w.algorithmic_bytes()
    # positions: cells sampled, draft rows reduced, or cells ranked by the reveal
    cells = {"draft": lambda: w.n_rows, "reveal": lambda: w.rows * w.positions,
             "ar": lambda: w.rows}.get(kind, lambda: w.cells)()
    # one step is one launch of the wave-per-cell kernel (every sampling workload
    # here has <= 64 requests, one request table), so its back-to-back time per
    # step is that kernel's average duration on its stream; or one parts + merge
    # pair; or, for the autoregressive step, the penalty kernel and one sampler
    # launch over all its requests (launches_per_step)
    achieved = alg / (ms_step * 1e-3) / 1e9
    cfg = describe(w, kind)
    if threshold:
        cfg["workload"] += "+threshold"
        cfg["threshold_out"] = True
    kname = kernel_name(w, kind)
    if mode in ("device_params", "graph"):
        cfg["workload"] += "+" + mode
        cfg["entry_point"] = "ds_sample_device_params" + (" in a replayed HIP graph" if mode == "graph" else "")
        kname = kname.replace("k_sample_small", "k_sample_small_dev")
    elif mode == "compact_u":
        cfg["workload"] += "+compact_u"
        cfg["u_layout"] = "compacted: guided requests' positions only"
    return {"config": cfg, "kernel": kname, "launches_per_step": launches_per_step(w, kind),
            "steps": steps, "warmup": warmup, "positions_per_s": cells / (ms_step * 1e-3),
            "ms_per_step": ms_step, "kernel_ms_mean": ms_step, "bracketed_ms_mean": ms_kernel,
            "bracketed_ms_median": med, "bracketed_ms_p10": p10, "bracketed_ms_p90": p90, "algorithmic_bytes": alg,
            "achieved_GBs": achieved, "frac_of_peak": achieved / HBM_PEAK_GBS, "workload_obj": w}


def cpu_baseline(w, budget_s: float = 12.0) -> dict:
    """The oracle as it stands (single-threaded C) on a bounded sample of cells:
    enough of the batch, or whole passes over it, for about `budget_s` of work."""
    import oracle

    cells_all = np.arange(w.cells, dtype=np.int64)
    # estimate cost on a small slice, then size the sample to the time budget
    probe = cells_all[: min(256, w.cells)]
    t = time.perf_counter()
    oracle.sample_workload(w, cells=probe)
    per_cell = (time.perf_counter() - t) / probe.size
    want = int(max(probe.size, budget_s / max(per_cell, 1e-9)))
    n = min(w.cells, want)
    passes = max(1, want // w.cells) if n == w.cells else 1
    sample = cells_all[:n]
    t = time.perf_counter()
    for _ in range(passes):
        oracle.sample_workload(w, cells=sample)
    dt = time.perf_counter() - t
    what = (f"{passes} passes over the whole {w.cells}-cell batch" if n == w.cells
            else f"first {n} of {w.cells} cells of the same workload")
    return {"value": passes * n / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"{what}, {dt:.2f} s, single-threaded C oracle"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="omnivoice")
    ap.add_argument("--no-suite", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (10 times), to scale "
                         "the FETCH_SIZE / WRITE_SIZE counters of a profiler run")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this sampler has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
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

    head = bench_one(args.workload, args.steps, args.warmup)
    w = head.pop("workload_obj")
    traffic = stored_traffic(args.workload)
    roofline = {"bound": "hbm", "achieved": round(head["achieved_GBs"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(head["frac_of_peak"], 4),
                "traffic": traffic,
                "kernel": head["kernel"],
                "algorithmic_bytes_per_launch": head["algorithmic_bytes"],
                "kernel_ms_mean": head["kernel_ms_mean"], "bracketed_ms_mean": head["bracketed_ms_mean"]}
    per_config = {}
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
            if name == args.workload and not thr and mode == "eager":
                res = head
            else:
                res = bench_one(name, None, None, threshold=thr, mode=mode)
                res.pop("workload_obj", None)
            entry = {k: (round(v, 6) if isinstance(v, float) else v) for k, v in res.items() if k != "config"}
            if not thr and mode == "eager":
                entry["traffic"] = stored_traffic(name)
            per_config[res["config"]["workload"]] = entry
    cpu = None if args.no_cpu_baseline else cpu_baseline(w)
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
        "dtype": "f32",
        "data": "synthetic",
        "config": head["config"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_config": per_config,
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
