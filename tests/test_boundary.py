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
    assert lib.bsa_abi_version() == 2


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


def fake(i):
    """Distinct fake device addresses, 256 MiB apart (never dereferenced)."""
    return ctypes.c_void_p((i + 1) << 28)


def fwd_call(lib, tile=128, D=128, B=1, H=1, NT=2, MS=2, ptr=None, idx=None, out=None,
             ws=NUL, ws_bytes=0):
    q, k, v, num, bs = ((ptr if ptr is not None else fake(i)) for i in range(5))
    idx = fake(5) if idx is None else idx
    out = (ptr if ptr is not None else fake(6)) if out is None else out
    return lib.bsa_fwd(q, k, v, idx, num, bs, tile, out, B, H, NT, D, MS, ws, ws_bytes, NUL)


def bwd_call(lib, tile=128, outs=None, ins=None, B=1, H=1, NT=2):
    """bsa_bwd on a B x H x NT-tile problem with fake pointers (inputs 0..11, outputs 12..15)."""
    i = [fake(n) for n in range(12)] if ins is None else ins
    o = [fake(12 + n) for n in range(4)] if outs is None else outs
    return lib.bsa_bwd(*i, tile, o[0], o[1], o[2], o[3], B, H, NT, 128, 2, 2, NUL)


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
    assert bwd_call(lib, 512) == SHAPE
    if not _device_present():
        assert bwd_call(lib, 256) in expected


def test_outputs_that_overlap_inputs_are_refused(lib):
    """An output sharing bytes with an input or another output is INVALID_ARGUMENT
    (checked on the host before any launch); inputs may share memory."""
    expected = {OK, NO_DEVICE, UNSUPPORTED}
    assert fwd_call(lib, out=fake(0)) == INVALID  # out is q
    # out starts inside v: [1, 1, 256, 128] bf16 is 64 KiB
    assert fwd_call(lib, out=ctypes.c_void_p(fake(2).value + 65534)) == INVALID
    assert fwd_call(lib, out=ctypes.c_void_p(fake(2).value + 65536)) in expected  # just past v
    assert fwd_call(lib, idx=ctypes.c_void_p(fake(6).value + 8)) == INVALID  # out over the list
    q = fake(0)
    # q, k and v may be one tensor
    assert lib.bsa_fwd(q, q, q, fake(5), fake(3), fake(4), 128, fake(6), 1, 1, 2, 128, 2,
                       NUL, 0, NUL) in expected
    lse_on_out = ctypes.c_void_p(fake(6).value + 100)
    assert lib.bsa_fwd_lse(q, q, q, fake(5), fake(3), fake(4), 128, fake(6), fake(7), lse_on_out,
                           1, 1, 2, 128, 2, NUL, 0, NUL) == INVALID
    lo_on_q = ctypes.c_void_p(fake(0).value + 64)
    assert lib.bsa_fwd_lse(q, q, q, fake(5), fake(3), fake(4), 128, fake(6), lo_on_q, fake(8),
                           1, 1, 2, 128, 2, NUL, 0, NUL) == INVALID
    # the workspace must not overlap an input or an output
    assert fwd_call(lib, ws=fake(1), ws_bytes=4096) == INVALID
    assert fwd_call(lib, ws=ctypes.c_void_p(fake(6).value + 4096), ws_bytes=4096) == INVALID
    assert fwd_call(lib, ws=fake(9), ws_bytes=1 << 20) in expected
    # backward: dk on dq, delta on dout, dv on the transposed lists, dq on out_lo
    o = [fake(12 + n) for n in range(4)]
    assert bwd_call(lib, outs=[o[0], o[0], o[2], o[3]]) == INVALID
    assert bwd_call(lib, outs=[o[0], o[1], o[2], fake(5)]) == INVALID
    assert bwd_call(lib, outs=[o[0], o[1], fake(9), o[3]]) == INVALID
    assert bwd_call(lib, outs=[fake(4), o[1], o[2], o[3]]) == INVALID
    if not _device_present():
        assert bwd_call(lib) in expected
    # layout and its inverse: a destination on a source or on the map
    src = (ctypes.c_void_p * 2)(fake(0), fake(1))
    dst = (ctypes.c_void_p * 2)(fake(2), fake(0))
    assert lib.bsa_tile_layout(src, dst, 2, fake(4), 64, 1, 64, 1, 1, 64, NUL) == INVALID
    dst = (ctypes.c_void_p * 2)(fake(2), fake(4))
    assert lib.bsa_tile_layout(src, dst, 2, fake(4), 64, 1, 64, 1, 1, 64, NUL) == INVALID
    dst = (ctypes.c_void_p * 2)(fake(2), fake(2))
    assert lib.bsa_tile_unlayout(src, dst, 2, fake(4), 64, 1, 64, 1, 1, 64, NUL) == INVALID


def test_fwd_rejects_bad_sizes_and_null_pointers(lib):
    assert fwd_call(lib, B=-1) == INVALID
    assert fwd_call(lib, MS=-1) == INVALID
    # a workspace needs both its pointer and its size; a negative size is refused
    assert fwd_call(lib, ws=fake(9), ws_bytes=0) == INVALID
    assert fwd_call(lib, ws=NUL, ws_bytes=4096) == INVALID
    assert fwd_call(lib, ws=fake(9), ws_bytes=-1) == INVALID
    # the training forward needs both statistics outputs
    q = fake(0)
    assert lib.bsa_fwd_lse(q, q, q, fake(5), fake(3), fake(4), 128, fake(6), NUL, fake(8),
                           1, 1, 2, 128, 2, NUL, 0, NUL) == INVALID
    assert lib.bsa_fwd_lse(q, q, q, fake(5), fake(3), fake(4), 128, fake(6), fake(7), NUL,
                           1, 1, 2, 128, 2, NUL, 0, NUL) == INVALID
    ins = [fake(n) for n in range(12)]
    ins[4] = NUL  # out_lo
    assert bwd_call(lib, ins=ins) == INVALID
    assert fwd_call(lib, ptr=NUL) == INVALID
    assert fwd_call(lib, idx=NUL) == INVALID
    assert fwd_call(lib, B=1, H=65536) == LIMITS
    assert fwd_call(lib, NT=1 << 22, tile=64) == LIMITS
    assert fwd_call(lib, B=64, H=64, NT=4096, tile=128) == LIMITS  # rows = 2^31
    # empty problems are accepted and launch nothing, even with null pointers
    assert fwd_call(lib, B=0, ptr=NUL, idx=NUL) == OK
    assert fwd_call(lib, NT=0, ptr=NUL, idx=NUL) == OK


def test_layout_rejects_bad_arguments(lib):
    srcs = (ctypes.c_void_p * 4)(*[fake(n) for n in range(4)])
    dsts = (ctypes.c_void_p * 4)(*[fake(4 + n) for n in range(4)])
    call = lambda n=1, tile=64, D=64, B=1, H=1, NT=1, tok=64, m=fake(9): lib.bsa_tile_layout(  # noqa
        srcs, dsts, n, m, tile, B, tok, H, NT, D, NUL)
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
    src, dst = (ctypes.c_void_p * 1)(fake(0)), (ctypes.c_void_p * 1)(fake(1))
    assert lib.bsa_tile_layout(src, dst, 1, fake(2), 64, 1, 64, 1, 1, 64, NUL) == NO_DEVICE
    assert lib.bsa_tile_unlayout(src, dst, 1, fake(2), 64, 1, 64, 1, 1, 64, NUL) == NO_DEVICE
    import torch

    # a CPU tensor is refused: there is no CPU implementation to fall back on
    with pytest.raises(ValueError):
        bsa.fwd(torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16), None, None, None, None, None, 64)


def test_shape_helper():
    assert bsa.fwd_out_shape((2, 3, 256, 64)) == (2, 3, 256, 64)


def test_workspace_size_validation(lib):
    n = ctypes.c_int64(-5)
    assert lib.bsa_fwd_workspace_size(1, 1, 2, 128, 128, 2, None) == INVALID
    assert lib.bsa_fwd_workspace_size(-1, 1, 2, 128, 128, 2, ctypes.byref(n)) == INVALID
    assert n.value == 0  # cleared even on error
    assert lib.bsa_fwd_workspace_size(1, 1, 2, 96, 128, 2, ctypes.byref(n)) == SHAPE
    assert lib.bsa_fwd_workspace_size(1, 65536, 2, 128, 128, 2, ctypes.byref(n)) == LIMITS
    assert lib.bsa_fwd_workspace_size(0, 1, 2, 128, 128, 2, ctypes.byref(n)) == OK
    assert n.value == 0
    if not _device_present():
        assert lib.bsa_fwd_workspace_size(1, 1, 2, 128, 128, 2, ctypes.byref(n)) == NO_DEVICE


_HUGE_SIZES = """
import ctypes, sys
sys.path.insert(0, {root!r})
import block_sparse_tiled_amd as bsa
lib = bsa.load()
F = lambda i: ctypes.c_void_p((i + 1) << 28)
N = ctypes.c_void_p(0)
res = []
for B, H in (({big}, {big}), (1 << 62, 4), (4, 1 << 62), (1 << 31, 1 << 31)):
    res.append(lib.bsa_fwd(F(0), F(1), F(2), F(3), F(4), F(5), 128, F(6), B, H, 2, 128, 2,
                           N, 0, N))
    res.append(lib.bsa_fwd_lse(F(0), F(1), F(2), F(3), F(4), F(5), 128, F(6), F(7), F(8), B, H,
                               2, 128, 2, N, 0, N))
    res.append(lib.bsa_bwd(*[F(n) for n in range(12)], 128, F(12), F(13), F(14), F(15), B, H,
                           2, 128, 2, 2, N))
    src = (ctypes.c_void_p * 1)(F(0))
    dst = (ctypes.c_void_p * 1)(F(1))
    res.append(lib.bsa_tile_layout(src, dst, 1, F(2), 64, B, 64, H, 1, 64, N))
    res.append(lib.bsa_tile_unlayout(src, dst, 1, F(2), 64, B, 64, H, 1, 64, N))
    n = ctypes.c_int64(0)
    res.append(lib.bsa_fwd_workspace_size(B, H, 2, 128, 128, 2, ctypes.byref(n)))
print(res)
assert all(r == 3 for r in res), res
"""


def test_overflowing_batch_times_heads_is_refused_not_a_crash():
    """batch * heads that wraps to 0 (2^32 x 2^32) or overflows int64 must return
    BSA_ERR_LAUNCH_LIMITS from every entry point; the size checks bound batch*heads by
    division before forming any product.  Run in a child process, so that a crash
    (a division by zero) fails this test instead of ending the session."""
    import subprocess
    import sys

    code = _HUGE_SIZES.format(root=ROOT, big=1 << 32)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, f"rc {res.returncode}: {res.stdout} {res.stderr[-2000:]}"


def coarse_call(lib, topk=2, max_sel=2, NT=4, tile=64, D=64, B=1, H=1, ws=None, ws_bytes=1 << 20,
                outs=None, ins=None):
    """bsa_coarse with fake pointers: inputs q, k, v, block_sizes = 0..3, outputs
    q2k_idx, q2k_num, coarse_out = 4..6, workspace 7."""
    i = [fake(n) for n in range(4)] if ins is None else ins
    o = [fake(4 + n) for n in range(3)] if outs is None else outs
    w = fake(7) if ws is None else ws
    return lib.bsa_coarse(i[0], i[1], i[2], i[3], tile, topk, o[0], o[1], o[2], B, H, NT, D,
                          max_sel, w, ws_bytes, NUL)


def test_coarse_rejects_bad_arguments(lib):
    expected = {OK, NO_DEVICE, UNSUPPORTED}
    assert coarse_call(lib, topk=-1) == INVALID
    assert coarse_call(lib, topk=3, max_sel=2) == INVALID  # the lists cannot hold topk tiles
    assert coarse_call(lib, B=-1) == INVALID
    assert coarse_call(lib, tile=96) == SHAPE
    assert coarse_call(lib, D=32) == SHAPE
    assert coarse_call(lib, NT=4097) == SHAPE  # more tiles than the selection holds
    assert coarse_call(lib, H=65536) == LIMITS
    assert coarse_call(lib, ws=NUL) == INVALID  # the workspace is required
    need = ctypes.c_int64(0)
    assert lib.bsa_coarse_workspace_size(1, 1, 4, 64, 64, ctypes.byref(need)) == OK
    assert need.value == 4 * 1 * 4 * (3 * 64 + 4)
    assert coarse_call(lib, ws_bytes=need.value - 4) == INVALID  # too small
    assert coarse_call(lib, ws_bytes=need.value) in expected
    # outputs overlapping an input, each other or the workspace
    o = [fake(4 + n) for n in range(3)]
    assert coarse_call(lib, outs=[fake(0), o[1], o[2]]) == INVALID
    assert coarse_call(lib, outs=[o[0], o[0], o[2]]) == INVALID
    assert coarse_call(lib, ws=fake(6)) == INVALID
    # the coarse output is optional; an empty problem is accepted with null pointers
    assert coarse_call(lib, outs=[o[0], o[1], NUL]) in expected
    assert coarse_call(lib, B=0, ins=[NUL] * 4, outs=[NUL] * 3, ws=NUL, ws_bytes=0) == OK
    assert lib.bsa_coarse_workspace_size(1, 1, 4097, 64, 64, ctypes.byref(need)) == SHAPE
    assert lib.bsa_coarse_workspace_size(1, 1, 4, 64, 64, None) == INVALID


def test_coarse_combine_rejects_bad_arguments(lib):
    expected = {OK, NO_DEVICE, UNSUPPORTED}
    call = lambda out=fake(0), gate=fake(1), oc=fake(2), bs=fake(3), tile=64, D=64: (  # noqa: E731
        lib.bsa_coarse_combine(out, gate, oc, bs, tile, 1, 2, 4, D, NUL))
    assert call(tile=32) == SHAPE
    assert call(D=96) == SHAPE
    assert call(gate=NUL) == INVALID
    assert call(out=fake(1)) == INVALID  # out is the gate
    assert call(oc=ctypes.c_void_p(fake(0).value + 64)) == INVALID  # coarse output inside out
    assert call() in expected


def test_noalloc_validates_like_fwd(lib):
    expected = {OK, NO_DEVICE, UNSUPPORTED}
    q = fake(0)
    f = lambda tile=128, B=1, out=fake(6), MS=2: lib.bsa_fwd_noalloc(  # noqa: E731
        q, fake(1), fake(2), fake(5), fake(3), fake(4), tile, out, B, 1, 2, 128, MS, NUL)
    assert f(tile=96) == SHAPE
    assert f(B=-1) == INVALID
    assert f(MS=-1) == INVALID
    assert f(out=q) == INVALID
    assert f(B=0) == OK
    assert f() in expected
    assert bsa.status_string(7) != "unknown status"


def test_layout_pool_and_coarse_pooled_reject_bad_arguments(lib):
    expected = {OK, NO_DEVICE, UNSUPPORTED}
    arr = lambda *ps: (ctypes.c_void_p * len(ps))(*ps)  # noqa: E731
    src, dst = arr(fake(0), fake(1), fake(2), fake(3)), arr(fake(4), fake(5), fake(6), fake(7))

    def lp(n=3, tile=64, D=64, map_=fake(8), bs=fake(9), pooled=fake(10), B=1, H=1, NT=2, tok=100):
        return lib.bsa_tile_layout_pool(src, dst, n, map_, bs, tile, B, tok, H, NT, D, pooled, NUL)

    assert lp(n=2) == INVALID  # Q, K and V are needed
    assert lp(n=5) == INVALID
    assert lp(tile=96) == SHAPE
    assert lp(D=32) == SHAPE
    assert lp(bs=NUL) == INVALID
    assert lp(pooled=NUL) == INVALID
    assert lp(pooled=fake(0)) == INVALID  # pooled over an input
    assert lp(pooled=fake(5)) == INVALID  # pooled over an output
    assert lp(B=0, map_=NUL, bs=NUL, pooled=NUL) == OK
    assert lp() in expected
    assert lp(n=4) in expected

    def cp(topk=2, max_sel=2, NT=4, tile=64, D=64, pooled=fake(0), ws=fake(7), ws_bytes=1 << 20,
           outs=None):
        o = [fake(4 + n) for n in range(3)] if outs is None else outs
        return lib.bsa_coarse_pooled(pooled, fake(3), tile, topk, o[0], o[1], o[2], 1, 1, NT, D,
                                     max_sel, ws, ws_bytes, NUL)

    assert cp(topk=3) == INVALID
    assert cp(tile=32) == SHAPE
    assert cp(NT=4097) == SHAPE
    assert cp(pooled=NUL) == INVALID
    assert cp(ws=NUL) == INVALID
    assert cp(ws_bytes=4 * 4 * 4 - 4) == INVALID  # the logits need 4 * NT^2 bytes per head
    assert cp(ws_bytes=4 * 4 * 4) in expected
    assert cp(outs=[fake(0), fake(5), fake(6)]) == INVALID  # lists over the pooled input
    assert cp() in expected


def _declared_parameter_counts():
    """{function: number of parameters} for every function include/bsa.h declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    counts = {}
    for m in re.finditer(r"\b(bsa_[a-z_0-9]+)\s*\(([^;{]*?)\)\s*;", text):
        params = m.group(2).strip()
        counts[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return counts


def test_binding_argument_counts_match_the_header(lib):
    """Every entry point the binding declares argtypes for takes as many arguments as
    include/bsa.h declares (a drift between the two would pass wrong values silently)."""
    counts = _declared_parameter_counts()
    assert sorted(counts) == _declared_functions()
    checked = 0
    for name, n in counts.items():
        fn = getattr(lib, name)
        if fn.argtypes is None:
            continue
        assert len(fn.argtypes) == n, f"{name}: header {n} parameters, binding {len(fn.argtypes)}"
        checked += 1
    assert checked == len(counts)  # the binding declares argtypes for every entry point


def test_unlayout_combine_rejects_bad_arguments(lib):
    expected = {OK, NO_DEVICE, UNSUPPORTED}

    def uc(out=fake(0), gate=fake(1), oc=fake(2), bs=fake(3), rows=fake(4), dst=fake(5), tile=64,
           D=64, B=1, H=1, tok=100, NT=2):
        return lib.bsa_tile_unlayout_combine(out, gate, oc, bs, rows, tile, B, tok, H, NT, D, dst,
                                             NUL)

    assert uc(tile=96) == SHAPE
    assert uc(D=32) == SHAPE
    assert uc(B=-1) == INVALID
    assert uc(dst=NUL) == INVALID
    assert uc(rows=NUL) == INVALID
    assert uc(gate=NUL) == INVALID
    assert uc(dst=fake(0)) == INVALID  # dst over the fine output
    assert uc(dst=ctypes.c_void_p(fake(4).value + 8)) == INVALID  # dst over the token map
    assert uc(tok=0, rows=NUL, dst=NUL) == OK
    assert uc(NT=0, out=NUL, gate=NUL, oc=NUL, bs=NUL) in expected  # every token +0
    assert uc() in expected
