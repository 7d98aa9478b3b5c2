"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

libdssample.so is rebuilt with every host pass instrumented (hipcc with
`-Xarch_host -fsanitize=address` and `-Xarch_host -fsanitize=undefined`, no
recovery; device code is built as usual), and a child Python process with the
clang AddressSanitizer runtime preloaded calls every entry point on the paths
that end before any HIP call: a NULL handle, rejected settings, rejected
arguments (NULL and misaligned pointers, negative lengths, non-finite guidance,
bad temperatures, capacity limits, a missing u), and a call whose requests are
all empty, which returns DS_OK without launching.  Those paths hold all of the
host-side validation and the per-request bookkeeping that precedes it.  Any
invalid access or undefined operation aborts the child with the sanitizer's
report; the return codes are checked too.  A control run first shows that the
same flags and preload catch a heap overflow in a small HIP file's host code.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import textwrap
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "vocab_wise_logit_amd", "csrc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
       "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not available")


def _asan_runtime() -> str:
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        pytest.skip("no clang AddressSanitizer runtime")
    return found[-1]


def _flags():
    return ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", *SAN]


def _link(objs, out):
    subprocess.run([_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan", *SAN, "-o", out, *objs],
                   check=True, capture_output=True, text=True)


def _child(code: str, asan: str) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["HIP_VISIBLE_DEVICES"] = ""  # every call below ends before a device is needed
    return subprocess.run([sys.executable, "-c", textwrap.dedent(code)], capture_output=True, text=True, env=env,
                          timeout=600)


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("hsan")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src):
        obj = os.path.join(d, os.path.basename(src) + ".o")
        r = subprocess.run([_hipcc(), *_flags(), "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(min(len(srcs), os.cpu_count() or 1, 8)) as ex:
        objs = list(ex.map(compile_one, srcs))
    out = os.path.join(d, "libdssample_hsan.so")
    _link(objs, out)
    return out


def test_host_sanitizers_catch_a_planted_overflow(tmp_path):
    asan = _asan_runtime()
    src = tmp_path / "planted.hip"
    src.write_text(textwrap.dedent("""
        #include <hip/hip_runtime.h>
        #include <cstdlib>
        extern "C" int heap_overflow(int n) { int* p = (int*)malloc(4 * n); int v = p[n]; free(p); return v; }
    """))
    obj = str(tmp_path / "planted.o")
    r = subprocess.run([_hipcc(), *_flags(), "-c", str(src), "-o", obj], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    lib = str(tmp_path / "libplanted.so")
    _link([obj], lib)
    r = _child(f"import ctypes; ctypes.CDLL({lib!r}).heap_overflow(8)", asan)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]


def test_entry_points_validate_cleanly_under_asan_and_ubsan(sanitized_lib):
    asan = _asan_runtime()
    r = _child(f"""
        import ctypes as C
        import numpy as np
        L = C.CDLL({sanitized_lib!r})
        L.ds_last_error.restype = C.c_char_p
        P, I32, I64, U32, U64, F = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32, C.c_uint64, C.c_float
        OK, INVALID, UNSUPPORTED, CAPACITY = 0, 1, 2, 3
        n = 0
        def expect(rc, want, what):
            global n
            n += 1
            assert rc == want, (what, rc, want, L.ds_last_error())
            assert (rc == OK) == (L.ds_last_error() == b""), (what, L.ds_last_error())

        def arr(x, dt):
            return np.ascontiguousarray(np.asarray(x, dt))

        # a NULL handle, for every call that takes one
        for name, args in (("ds_sample", [None] * 15), ("ds_sample_device_params", [None] * 16),
                           ("ds_greedy_lse", [None] * 8), ("ds_reveal_topk", [None] * 9),
                           ("ds_repetition_penalty", [None] * 6), ("ds_sample_ar", [None] * 13)):
            f = getattr(L, name)
            f.restype = C.c_int
            expect(f(*[P(a) if a is None else a for a in args]), INVALID, name + "(NULL)")
        L.ds_sample_destroy(P(None))

        # creation refused before any device is queried
        out = P()
        for vocab, dtype, rows, pos, reqs, k, ch, fl in ((0, 0, 1, 1, 1, 0, 1, 0), (1024, 7, 1, 1, 1, 0, 1, 0),
                                                          (1024, 0, 0, 1, 1, 0, 1, 0), (1024, 0, 1, 0, 1, 0, 1, 0),
                                                          (1024, 0, 1, 1, 0, 0, 1, 0), (1024, 0, 1, 1, 1, -1, 1, 0),
                                                          (1024, 0, 1, 1, 1, 0, 0, 0), (1024, 0, 1, 1, 1, 0, 1, 64)):
            rc = L.ds_sample_create(C.byref(out), 0, I32(vocab), I32(dtype), I32(rows), I64(pos), I32(reqs),
                                    I32(k), I32(ch), U32(fl))
            assert rc != OK and out.value is None, (vocab, dtype, rows, pos, reqs, k, ch, fl, rc)
            n += 1

        # the entry point that allocates nothing: settings, then every argument check
        def static(vocab=1024, dtype=1, k=0, ch=1, fl=0, rid=None, c=64, u=64, sl=None, it=None, g=None, t=None,
                   nreq=None, rows=2, tok=64, lp=64, thr=None):
            rid = arr([5, 6, 7], np.int64) if rid is None else rid
            sl = arr([3, 0, 2], np.int32) if sl is None else sl
            it = arr([0, 1, 2], np.int32) if it is None else it
            g = arr([2.0, 0.0, 1.5], np.float32) if g is None else g
            t = arr([0.9, 0.0, 1.2], np.float32) if t is None else t
            nreq = len(sl) if nreq is None else nreq
            ptr = lambda a: a.ctypes.data_as(P) if isinstance(a, np.ndarray) else P(a)
            return L.ds_sample_static(I32(vocab), I32(dtype), I32(k), I32(ch), U32(fl), ptr(rid), P(c), P(u),
                                      ptr(sl), ptr(it), ptr(g), ptr(t), I32(nreq), I32(rows), U64(7),
                                      P(tok), P(lp), P(thr), P(None))
        L.ds_sample_static.restype = C.c_int
        expect(static(vocab=0), INVALID, "vocab 0")
        expect(static(dtype=3), INVALID, "dtype")
        expect(static(k=2000), INVALID, "top_k > V")
        expect(static(ch=0), INVALID, "no chunks")
        expect(static(fl=16), INVALID, "unknown flag")
        expect(static(rid=0), INVALID, "NULL request ids")
        expect(static(sl=0, nreq=3), INVALID, "NULL lengths")
        expect(static(c=0), INVALID, "NULL c")
        expect(static(tok=0), INVALID, "NULL tokens")
        expect(static(nreq=0), CAPACITY, "no requests")
        expect(static(rows=0), CAPACITY, "no rows")
        expect(static(c=65), INVALID, "misaligned bf16 c")
        expect(static(dtype=0, c=66), INVALID, "misaligned f32 c")
        expect(static(tok=66), INVALID, "misaligned tokens")
        expect(static(thr=70), INVALID, "misaligned thresholds")
        expect(static(sl=arr([3, -1, 2], np.int32)), INVALID, "negative length")
        expect(static(g=arr([2.0, np.inf, 1.5], np.float32)), INVALID, "infinite guidance")
        expect(static(g=arr([2.0, np.nan, 1.5], np.float32)), INVALID, "NaN guidance")
        expect(static(t=arr([0.9, -1.0, 1.2], np.float32)), INVALID, "negative temperature")
        expect(static(t=arr([0.9, np.nan, 1.2], np.float32)), INVALID, "NaN temperature")
        expect(static(t=arr([0.9, np.inf, 1.2], np.float32)), INVALID, "infinite temperature")
        expect(static(u=0), INVALID, "u missing under guidance")
        expect(static(u=66), UNSUPPORTED, "u and c apart by a non-multiple of 16 bytes")
        expect(static(vocab=3001, fl=2, sl=arr([4, 0], np.int32), g=arr([1.0, 0.0], np.float32),
                      t=arr([0.5, 0.0], np.float32), it=arr([0, 0], np.int32), rid=arr([1, 2], np.int64)),
               UNSUPPORTED, "compacted u on the streaming path with V * 2 not a multiple of 16")
        big = arr([2 ** 30, 2 ** 30], np.int32)
        expect(static(sl=big, g=arr([0.0, 0.0], np.float32), t=arr([0.0, 0.0], np.float32),
                      it=arr([0, 0], np.int32), rid=arr([1, 2], np.int64)), CAPACITY, "2^31 cells")
        # 150 requests that are all empty: validated, grouped, and nothing to launch
        m = 150
        expect(static(sl=arr(np.zeros(m), np.int32), g=arr(np.linspace(-1, 2, m), np.float32),
                      t=arr(np.linspace(0, 2, m), np.float32), it=arr(np.arange(m), np.int32),
                      rid=arr(np.arange(m), np.int64)), OK, "all requests empty")

        # the read probe's argument checks
        L.ds_read_probe.restype = C.c_int
        for x, rows, rb, thr, sink in ((0, 1, 16, 256, 64), (64, 1, 16, 256, 0), (72, 1, 16, 256, 64),
                                       (64, 1, 16, 256, 66), (64, 0, 16, 256, 64), (64, 2 ** 31, 16, 256, 64),
                                       (64, 1, 8, 256, 64), (64, 1, 24, 256, 64), (64, 1, 16, 128, 64)):
            expect(L.ds_read_probe(P(x), I64(rows), I64(rb), I32(thr), P(sink), P(None)), INVALID,
                   f"read probe {{x, rows, rb, thr, sink}}")
        print(f"sanitized library: {{n}} rejected or empty calls, clean")
    """, asan)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-5000:])
    assert "clean" in r.stdout, r.stdout[-2000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-5000:]
