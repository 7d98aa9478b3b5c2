"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle (oracle/ds_oracle.c) is rebuilt with -fsanitize=address,undefined
and no recovery, and a child Python process (libasan preloaded, as a sanitized
shared library loaded into an unsanitized interpreter requires) runs against it:

  - every check of the planted-mistake harness (tests/test_oracle_mutants.py),
    which between them call each exported oracle function;
  - whole calls of the sampler on small workloads (a V=1024 f32 batch, an
    OmniVoice-shaped V=1025 bf16 batch, a full V=248320 row in four chunks),
    the draft reduction, the confidence reveal and the repetition penalty.

Any invalid access or undefined operation aborts the child with the
sanitizer's report.  A control run first shows that the same build flags and
preload do catch a heap overflow and a signed overflow in a small C file, so a
clean oracle run means something.
"""

from __future__ import annotations

import os
import subprocess
import sys
import textwrap

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN_FLAGS = ["-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _libasan() -> str:
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                           check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        pytest.skip("gcc not available")
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip("gcc has no AddressSanitizer runtime")
    return p


def _build(src: str, out: str) -> None:
    subprocess.run(["gcc", *SAN_FLAGS, "-o", out, src, "-lm"], check=True)


def _child(code: str, asan: str, timeout: int = 600) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    # the interpreter itself keeps memory to exit, which is not the oracle's
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["PYTHONPATH"] = os.pathsep.join([ROOT, HERE, env.get("PYTHONPATH", "")])
    return subprocess.run([sys.executable, "-c", textwrap.dedent(code)], capture_output=True, text=True,
                          env=env, timeout=timeout)


def test_sanitizers_catch_planted_errors(tmp_path):
    asan = _libasan()
    src = tmp_path / "planted.c"
    src.write_text(textwrap.dedent("""
        #include <stdlib.h>
        int heap_overflow(int n) { int* p = malloc(4 * n); int v = p[n]; free(p); return v; }
        int signed_overflow(int a) { return a + 0x7FFFFFFF; }
    """))
    lib = str(tmp_path / "libplanted.so")
    _build(str(src), lib)
    r = _child(f"import ctypes; ctypes.CDLL({lib!r}).heap_overflow(8)", asan)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]
    r = _child(f"import ctypes; ctypes.CDLL({lib!r}).signed_overflow(5)", asan)
    assert r.returncode != 0 and "runtime error" in r.stderr, r.stderr[-2000:]


def test_oracle_runs_clean_under_asan_and_ubsan(tmp_path):
    asan = _libasan()
    lib = str(tmp_path / "libdsoracle_san.so")
    _build(os.path.join(ROOT, "oracle", "ds_oracle.c"), lib)
    r = _child(f"""
        import numpy as np
        import oracle, synth
        import test_oracle_mutants as M
        lib = oracle.load_variant({lib!r})
        assert M._failures(lib) == [], M._failures(lib)
        oracle._lib = lib  # every oracle entry below goes to the sanitized build
        for w in (synth.tiny(0.9), synth.tiny(0.0), synth.omnivoice(n_requests=2),
                  synth.stress(positions=3, seed=21)):
            res = oracle.sample_workload(w)
            assert np.all(res.tokens >= 0), w.name
        d = synth.draft(n_rows=3, vocab=4096, vocab_chunks=4)
        g = oracle.greedy_lse(d.logits, vocab_chunks=4)
        assert np.all(g.token == g.dense_token)
        rv = synth.reveal(n_requests=3, rows=2)
        oracle.reveal_topk(rv.scores, rv.seq_lens, rv.reveal_counts)
        pen, res = oracle.ar_step(synth.ar(n_requests=3, vocab=5000))
        assert np.all(res.tokens >= 0)
        print("sanitized oracle: clean")
    """, asan)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "sanitized oracle: clean" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
