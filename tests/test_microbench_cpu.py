"""The unit microbenchmark library (libflexattn_mb.so): it is built with the
attention library, exports its three entry points, and rejects bad arguments
before any HIP call (so this runs without a GPU)."""
import ctypes
import os

import pytest

from attention_tiled_attn_amd import microbench as mb


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mb.MB_PATH):
        pytest.skip("libflexattn_mb.so not built")
    return mb._lib()


def test_exports(lib):
    for name in ("flexattn_mb_units", "flexattn_mb_read", "flexattn_mb_copy"):
        assert hasattr(lib, name)


@pytest.mark.parametrize("args", [
    (-1, 1, 10, 1, 1), (8, 1, 10, 1, 1),          # unknown kind
    (0, 0, 10, 1, 1), (0, 3, 10, 1, 1),           # waves per SIMD
    (0, 1, 0, 1, 1), (3, 2, 10, 0, 1),            # iteration counts
    (0, 1, 10, 1, 0), (0, 1, 10, 1, 70000),       # workgroups
    (3, 1, 10, 10, 4), (4, 1, 10, 10, 4),         # mixed kinds need two waves per SIMD
])
def test_units_rejects(lib, args):
    kind, wps, iters, iters_vec, wgs = args
    buf = (ctypes.c_ulonglong * 8)()
    sink = (ctypes.c_float * 8)()
    assert lib.flexattn_mb_units(kind, wps, iters, iters_vec, wgs, ctypes.addressof(buf),
                                 ctypes.addressof(sink), None) == -1


def test_units_rejects_null(lib):
    assert lib.flexattn_mb_units(0, 1, 10, 1, 1, None, None, None) == -1


def test_read_copy_reject(lib):
    buf = (ctypes.c_float * 64)()
    p = ctypes.addressof(buf)
    assert lib.flexattn_mb_read(None, 16, p, 1, None) == -1
    assert lib.flexattn_mb_read(p, 15, p, 1, None) == -1          # not a multiple of 16
    assert lib.flexattn_mb_read(p, 0, p, 1, None) == -1
    assert lib.flexattn_mb_copy(p, None, 16, 1, None) == -1
    assert lib.flexattn_mb_copy(p, p, 16, 0, None) == -1
