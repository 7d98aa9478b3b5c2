"""GPU pins of the library's device building blocks against the CPU oracle.

The sampler's token, threshold and logprob parity all rest on a few device
functions: the Philox4x32-10 block, the per-id noise word, the Gumbel map and
bf16 widening.  Parity of whole calls only reaches them through tokens; here a
test-only HIP library (tests/gpu_pins/ds_pins.hip, compiled from the library's own
ds_device.h) runs each of them over large input ranges and every value is
compared with the oracle:

  - Philox words over 10^7 counters (four keys and counter sets, one wrapping the
    first counter word), bit-exact;
  - noise words of 2 x 10^5 ids in four cells, bit-exact (the counter layout and
    the word chosen by v & 3);
  - the Gumbel map over all 2^23 values of its uniform lattice, within 2e-6
    absolute of the oracle's double (about one fp32 unit at the largest values);
  - bf16 widening of all 65536 patterns through both dword halves, bit-exact;
  - the order key and its inverse on special values and 2 x 10^5 random patterns.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np
import pytest

import oracle
from gpu_helpers import log

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gpu_pins", "libdspins.so")
GUMBEL_ABS_TOL = 2e-6


@pytest.fixture(scope="module")
def pins():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    torch.cuda.init()
    assert os.path.exists(LIB), f"{LIB} is not built: run tests/gpu_pins/build_pins.py (or build())"
    L = C.CDLL(LIB)  # after torch, so both use torch's HIP runtime
    P, U32, I64 = C.c_void_p, C.c_uint32, C.c_int64
    L.pins_philox.argtypes = [U32, U32, U32, U32, U32, U32, I64, P]
    L.pins_noise.argtypes = [U32, U32, U32, U32, U32, U32, I64, P]
    L.pins_gumbel_lattice.argtypes = [P]
    L.pins_bf16_all.argtypes = [P, P]
    L.pins_order_key.argtypes = [P, I64, P, P]
    for f in (L.pins_philox, L.pins_noise, L.pins_gumbel_lattice, L.pins_bf16_all, L.pins_order_key):
        f.restype = C.c_int
    return L


def _u32(t):
    return t.cpu().numpy().view(np.uint32)


def test_philox_words_over_ten_million_counters(pins):
    import torch

    n = 2_500_000
    sets = [((0, 0, 0, 0), (0, 0)),
            ((0xFFFFFFFF - n // 2, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF)),
            ((12345, 17, (3 & 0xFFFF) | (250 << 16), 1000), (42, 0)),
            ((0x9E3779B9, 0xDEADBEEF, 0x0BADF00D, 0x7FFFFFFF), (0xA5A5A5A5, 0x5A5A5A5A))]
    out = torch.empty(4 * n, dtype=torch.int32, device="cuda")
    for ctr, key in sets:
        log(f"[gpu] pins_philox ctr={ctr} key={key} n={n}")
        assert pins.pins_philox(*ctr, *key, n, out.data_ptr()) == 0
        got = _u32(out).reshape(n, 4)
        want = oracle.philox_range(ctr, key, n)
        bad = np.nonzero((got != want).any(axis=1))[0]
        assert bad.size == 0, f"Philox words differ at counter offsets {bad[:5]}"


def test_noise_words_follow_the_counter_layout(pins):
    import torch

    n = 50_000
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    # (seed, request id, iteration, row, t, first id)
    for seed, rid, it, row, t, v0 in ((42, 1000, 0, 0, 0, 0), (0xFFFFFFFF12345678, 7, 65535, 65535, 2047, 248320 - n),
                                      ((1 << 63) + 5, -3, 9, 70000, 100, 123457), (1, 2**40 + 11, 3, 5, 17, 3)):
        log(f"[gpu] pins_noise seed={seed} rid={rid} it={it} row={row} t={t} v0={v0}")
        row_iter = ((row & 0xFFFF) | (it << 16)) & 0xFFFFFFFF
        assert pins.pins_noise(seed & 0xFFFFFFFF, seed >> 32, t, row_iter, rid & 0xFFFFFFFF, v0, n,
                               out.data_ptr()) == 0
        want = oracle.noise_words(seed, rid, it, row, t, v0, n)
        assert np.array_equal(_u32(out), want)


def test_gumbel_map_over_its_whole_lattice(pins):
    import torch

    n = 1 << 23
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    log("[gpu] pins_gumbel_lattice: 2^23 values")
    assert pins.pins_gumbel_lattice(out.data_ptr()) == 0
    got = out.cpu().numpy().astype(np.float64)
    j = np.arange(n, dtype=np.uint32)
    want = oracle.gumbel_array((j << np.uint32(9)) | (j & np.uint32(0x1FF)))
    err = np.abs(got - want)
    worst = int(np.argmax(err))
    log(f"[check] gumbel lattice: max |G_gpu - G| = {err[worst]:.3e} at U = {(2 * worst + 1) * 2.0**-24:.9f}")
    assert err[worst] <= GUMBEL_ABS_TOL, (worst, got[worst], want[worst])
    # the extremes the pruning bounds are built on
    assert got[-1] <= 16.75 and got[0] >= -2.82


def test_bf16_widening_of_every_pattern(pins):
    import torch

    lo = torch.empty(65536, dtype=torch.int32, device="cuda")
    hi = torch.empty(65536, dtype=torch.int32, device="cuda")
    log("[gpu] pins_bf16_all")
    assert pins.pins_bf16_all(lo.data_ptr(), hi.data_ptr()) == 0
    want = oracle.bf16_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16)).view(np.uint32)
    assert np.array_equal(_u32(lo), want)
    assert np.array_equal(_u32(hi), want)


def test_order_key_and_inverse(pins):
    import torch

    rng = np.random.default_rng(17)
    special = np.array([0x00000000, 0x80000000, 0x00000001, 0x80000001, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000,
                        0xFF800000, 0x3F800000, 0xBF800000, 0x007FFFFF, 0x807FFFFF], np.uint32)
    bits = np.concatenate([special, rng.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32)])
    b = torch.from_numpy(bits.view(np.int32)).cuda()
    key = torch.empty_like(b)
    back = torch.empty_like(b)
    log(f"[gpu] pins_order_key n={bits.size}")
    assert pins.pins_order_key(b.data_ptr(), bits.size, key.data_ptr(), back.data_ptr()) == 0
    want = np.array([oracle.order_key(float(x)) if not np.isnan(x) else None
                     for x in bits.view(np.float32)], dtype=object)
    ok = np.array([w is not None for w in want])
    assert np.array_equal(_u32(key)[ok], want[ok].astype(np.uint64).astype(np.uint32))
    assert np.array_equal(_u32(back), bits)
    # the key order is the float order (finite and infinite values)
    f = bits.view(np.float32)
    fin = ~np.isnan(f)
    order = np.argsort(_u32(key)[fin], kind="stable")
    assert np.all(np.diff(f[fin][order].astype(np.float64)) >= 0)
