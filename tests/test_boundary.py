"""Host-side checks of the C ABI: symbols, launch limits, argument validation.

None of these launches a kernel; the library must load and validate on a
machine without a GPU.
"""
import ctypes
import json
import os
import re

import pytest

import block_sparse_tiled_amd as bsa
from block_sparse_tiled_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "page_constants.json")

OK, INVALID, SHAPE, LIMITS, NO_DEVICE, UNSUPPORTED, HIP = range(7)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z_0-9]+)\s*\(", text)))


def _device_present():
    import torch

    return torch.cuda.device_count() > 0


@pytest.fixture(scope="module")
def lib():
    return bsa.load()


def test_library_exports_every_declared_function(lib):
    names = _declared_functions()
    assert {"bsa_fwd", "bsa_tile_layout", "bsa_within_launch_limits"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in bsa.h but not exported"


def test_abi_version(lib):
    assert lib.bsa_abi_version() == 1


def test_launch_limits_at_the_printed_boundaries(lib):
    with open(GOLDEN) as f:
        g = json.load(f)["launch_limits"]
    bh, rows, tiles = g["max_batch_heads_inclusive"], g["rows_exclusive"], g["tiles_exclusive"]
    assert (api.MAX_BATCH_HEADS, api.ROWS_LIMIT, api.TILES_LIMIT) == (bh, rows, tiles)
    assert bsa.within_launch_limits(1, bh, 1, 1)
    assert not bsa.within_launch_limits(1, bh + 1, 1, 1)
    assert bsa.within_launch_limits(3, bh // 3, 1, 1)
    assert not bsa.within_launch_limits(2, (bh + 1) // 2, 1, 1)
    assert bsa.within_launch_limits(1, 1, rows - 1, 1)
    assert not bsa.within_launch_limits(1, 1, rows, 1)
    assert bsa.within_launch_limits(1, 1, 1, tiles - 1)
    assert not bsa.within_launch_limits(1, 1, 1, tiles)
    assert not bsa.within_launch_limits(-1, 1, 1, 1)
    assert not bsa.within_launch_limits(1 << 40, 1 << 40, 1, 1)  # no overflow into "fits"


def test_python_mirror_agrees_with_the_library(lib):
    import random

    rnd = random.Random(0)
    edges = [0, 1, 2, 255, 256, 65535, 65536, (1 << 22) - 1, 1 << 22, (1 << 31) - 1, 1 << 31]
    cases = [(rnd.choice(edges), rnd.choice(edges), rnd.choice(edges), rnd.choice(edges))
             for _ in range(2000)]
    cases += [(rnd.randint(0, 300), rnd.randint(0, 300), rnd.randint(0, 1 << 32),
               rnd.randint(0, 1 << 23)) for _ in range(2000)]
    for c in cases:
        assert bsa.within_launch_limits(*c) == bsa.within_launch_limits_py(*c), c


def test_status_strings(lib):
    assert bsa.status_string(OK) == "ok"
    assert "gfx950" in bsa.status_string(UNSUPPORTED)
    assert "65535" in bsa.status_string(LIMITS)
    assert bsa.status_string(12345) == "unknown status"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first
NUL = ctypes.c_void_p(0)


def fwd_call(lib, tile=128, D=128, B=1, H=1, NT=2, MS=2, ptr=FAKE, idx=FAKE):
    return lib.bsa_fwd(ptr, ptr, ptr, idx, ptr, ptr, tile, ptr, B, H, NT, D, MS, NUL)


@pytest.mark.parametrize("tile,D", [(32, 128), (512, 128), (128, 96), (64, 256), (0, 64), (192, 64)])
def test_fwd_rejects_unsupported_shapes(lib, tile, D):
    assert fwd_call(lib, tile=tile, D=D) == SHAPE


def test_tile_256_passes_validation(lib):
    """256-row tiles pass validation (they fail only on reaching the device check, or
    run); 512 does not."""
    expected = {OK, NO_DEVICE, UNSUPPORTED}
    assert fwd_call(lib, tile=256, NT=0, ptr=NUL, idx=NUL) == OK
    assert fwd_call(lib, tile=256, D=64, B=64, H=64, NT=2048) == LIMITS  # rows = 2^31
    if not _device_present():
        assert fwd_call(lib, tile=256) in expected
    p = FAKE
    call = lambda tile: lib.bsa_bwd(p, p, p, p, p, p, p, p, p, p, p, tile, p, p, p, p, 1, 1, 2,  # noqa
                                    128, 2, 2, NUL)
    assert call(512) == SHAPE
    if not _device_present():
        assert call(256) in expected


def test_fwd_rejects_bad_sizes_and_null_pointers(lib):
    assert fwd_call(lib, B=-1) == INVALID
    assert fwd_call(lib, MS=-1) == INVALID
    assert fwd_call(lib, ptr=NUL) == INVALID
    assert fwd_call(lib, idx=NUL) == INVALID
    assert fwd_call(lib, B=1, H=65536) == LIMITS
    assert fwd_call(lib, NT=1 << 22, tile=64) == LIMITS
    assert fwd_call(lib, B=64, H=64, NT=4096, tile=128) == LIMITS  # rows = 2^31
    # empty problems are accepted and launch nothing, even with null pointers
    assert fwd_call(lib, B=0, ptr=NUL, idx=NUL) == OK
    assert fwd_call(lib, NT=0, ptr=NUL, idx=NUL) == OK


def test_layout_rejects_bad_arguments(lib):
    arr = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    call = lambda n=1, tile=64, D=64, B=1, H=1, NT=1, tok=64, m=FAKE: lib.bsa_tile_layout(  # noqa
        arr, arr, n, m, tile, B, tok, H, NT, D, NUL)
    assert call(n=0) == INVALID
    assert call(n=5) == INVALID
    assert call(tile=96) == SHAPE
    assert call(D=32) == SHAPE
    assert call(m=NUL) == INVALID
    assert call(H=70000) == LIMITS
    assert call(B=0, m=NUL) == OK


@pytest.mark.skipif("_device_present()", reason="checks the no-device path; a GPU is visible")
def test_without_a_device_launches_fail_cleanly(lib):
    assert fwd_call(lib) == NO_DEVICE
    arr = (ctypes.c_void_p * 1)(FAKE)
    assert lib.bsa_tile_layout(arr, arr, 1, FAKE, 64, 1, 64, 1, 1, 64, NUL) == NO_DEVICE
    assert lib.bsa_tile_unlayout(arr, arr, 1, FAKE, 64, 1, 64, 1, 1, 64, NUL) == NO_DEVICE
    import torch

    # a CPU tensor is refused: there is no CPU implementation to fall back on
    with pytest.raises(ValueError):
        bsa.fwd(torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16), None, None, None, None, None, 64)


def test_shape_helper():
    assert bsa.fwd_out_shape((2, 3, 256, 64)) == (2, 3, 256, 64)
