"""GPU parity of bsa_fwd against the CPU oracle, through the C ABI.

Small problems are compared element by element over every row; the full-size
configurations are compared on sampled rows (the oracle computes them one by
one) plus properties that hold at any size: padding rows and rows without keys
are +0 bit for bit, NaN appears exactly where the construction puts it.
"""
import zlib

import numpy as np
import pytest

import block_sparse_tiled_amd as bsa
from block_sparse_tiled_amd import inputs as gen
from parity import bits_from_dev, compare, run_fwd, sample_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    bsa.load()
    return torch.device("cuda")


def oracle_out(oracle_mod, w, **kw):
    return oracle_mod.fwd(w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs, w.T, **kw)


def padding_rows(w):
    """bool [B, H, S]: query rows past their tile's valid length."""
    r = np.arange(w.S) % w.T
    t = np.arange(w.S) // w.T
    return np.broadcast_to(r >= w.vbs[t], (w.B, w.H, w.S))


def empty_list_rows(w):
    """bool [B, H, S]: rows whose list holds no valid key (in-range contents)."""
    tot = np.zeros((w.B, w.H, w.NT), np.int64)
    for n in range(w.MS):
        live = w.q2k_num > n
        tot += np.where(live, w.vbs[w.q2k_idx[..., n]], 0)
    return np.repeat(tot == 0, w.T, axis=2)


def test_tiny_config(oracle_mod):
    w = gen.tiny()
    print(f"tiny: B={w.B} H={w.H} NT={w.NT} T={w.T} D={w.D}", flush=True)
    got = run_fwd(w)
    compare(got, oracle_out(oracle_mod, w), label="tiny")


def test_ragged_config_every_row(oracle_mod):
    w = gen.ragged()
    print("ragged: full oracle", flush=True)
    got = run_fwd(w)
    mx, mean = compare(got, oracle_out(oracle_mod, w), label="ragged")
    print(f"ragged max {mx:.3e} mean {mean:.3e}")


@pytest.mark.parametrize("name", ["video", "video_cube", "dense", "dense25", "stress", "dense256"])
def test_full_size_config_sampled(oracle_mod, name):
    w = gen.make(name)
    print(f"{name}: B={w.B} H={w.H} NT={w.NT} T={w.T} MS={w.MS}", flush=True)
    got = run_fwd(w)
    D = w.D
    extra = []
    if "neg_inf_row" in w.notes:
        b, h, row = w.notes["neg_inf_row"]
        extra.append((b * w.H + h) * w.S + row)
    rng = np.random.default_rng(123)
    rows = sample_rows(w, 384, rng, extra)
    ref = oracle_mod.fwd_rows(w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs, w.T, rows)
    mx, mean = compare(got.reshape(-1, D)[rows], ref, label=name)
    print(f"{name}: {rows.size} sampled rows, max {mx:.3e} mean {mean:.3e}")
    # properties over every row
    zero = padding_rows(w) | empty_list_rows(w)
    assert np.all(got[zero] == 0), "padding rows and rows without keys must be +0"
    f = gen.bf16_bits_to_f32(got)
    assert not np.isinf(f).any()
    nan_rows = np.isnan(f).any(-1)
    if "neg_inf_row" in w.notes:
        b, h, row = w.notes["neg_inf_row"]
        assert np.isnan(f[b, h, row]).all()
        nan_rows[b, h, row] = False
    assert not nan_rows.any(), f"{int(nan_rows.sum())} unexpected NaN rows"


CASES = {
    # name: (B, H, vbs builder, kwargs)
    "ragged_tail": (1, 2, lambda T: [T, T - 1, T // 2 + 3, T, 7], dict(density=0.6)),
    "odd_tiles_7": (2, 3, lambda T: [T] * 6 + [T - 5], dict(density=0.5, pad="naninf")),
    "odd_tiles_9": (1, 2, lambda T: [T] * 8 + [T // 3], dict(density=0.4, pad="nan")),
    "zeros_ones": (1, 2, lambda T: [0, 1, T, 1, 0, T - 3, 2], dict(density=0.7, pad="inf")),
    "duplicates": (1, 2, lambda T: [T, 5, T, T - 9], dict(density=0.9, duplicates=True)),
    "all_selected": (1, 2, lambda T: [T] * 5 + [T // 2], dict(counts=6)),
    "none_selected": (1, 2, lambda T: [T] * 3, dict(counts=0)),
    "many_waves": (2, 16, lambda T: [T] * 32 + [T - 11], dict(density=0.15)),
    # lists longer than one workgroup's list chunk (256 or 128 entries), with
    # repeats and entries naming an empty tile
    "long_lists": (1, 1, lambda T: [T] * 5 + [T - 3, 0], dict(counts=300, MS=300, duplicates=True)),
    # index rows far wider than the lists they hold: list segments past the
    # count are empty when the last round is split
    "wide_rows": (1, 2, lambda T: [T] * 6 + [T - 9], dict(density=0.3, MS=1000)),
    # tiles of at most T/2 rows, which share steps two by two: lengths 1, T/2 - 1
    # and T/2, and lengths whose end falls inside a 1 KiB copy block
    "short_tiles": (2, 2, lambda T: [1, T // 2, T // 2 - 1, 3, 5, T // 4 + 1, T, T // 2 + 1, 9, 2, T // 2,
                                     17, T - 2, 6], dict(density=0.7, pad="naninf")),
    # only short tiles, an odd number of them in every list (one step holds one)
    "short_only_odd": (1, 3, lambda T: [T // 2, 1, T // 2 - 3, 4, 7, T // 2, 13, 2, 11],
                       dict(counts=9, pad="nan")),
    # short tiles over several list chunks, repeated (a tile paired with itself)
    "short_long_lists": (1, 1, lambda T: [3, T // 2, T, 6, T // 2 - 1, 0, 1],
                         dict(counts=300, MS=300, duplicates=True, pad="inf")),
    # long tiles with the short ones that complete them to exactly T rows, and
    # equal lengths (ties in the order by length)
    "complementary_lengths": (2, 2, lambda T: [T - 20, 20, T - 1, 1, 3 * T // 4, T // 4, T // 2 + 5,
                                               T // 2 - 5, T, T - 20, 20, 7],
                              dict(density=0.8, pad="naninf")),
}


@pytest.mark.parametrize("T,D", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("case", sorted(CASES))
def test_random_shapes(oracle_mod, case, T, D):
    B, H, vbs_fn, kw = CASES[case]
    vbs = vbs_fn(T)
    w = gen.random_problem(zlib.crc32(f"{case}-{T}-{D}".encode()) % 10000, B=B, H=H, D=D, T=T, vbs=vbs, **kw)
    print(f"{case}: T={T} D={D} NT={w.NT} MS={w.MS}", flush=True)
    got = run_fwd(w)
    compare(got, oracle_out(oracle_mod, w), label=f"{case} T={T} D={D}")


@pytest.mark.parametrize("T,D", [(64, 128), (128, 128), (128, 64)])
def test_padding_contents_do_not_change_a_bit(T, D):
    w = gen.random_problem(41, B=1, H=3, D=D, T=T, vbs=[T, T - 7, 3, T, 0, T // 2], density=0.6)
    base = run_fwd(w)
    for pattern in ("nan", "inf", "naninf", "random"):
        q, k, v = w.q.copy(), w.k.copy(), w.v.copy()
        for x in (q, k, v):
            gen.fill_padding(x, w.vbs, T, pattern)
        print(f"padding pattern {pattern}", flush=True)
        np.testing.assert_array_equal(run_fwd(w, q=q, k=k, v=v), base)


def test_short_halves_of_256_row_tiles(oracle_mod):
    """256-row tiles run as 128-row halves: a half of at most 64 rows (the second half
    of a tile of 129..192 rows, or a tile of at most 64) shares a step with another."""
    T, D = 256, 128
    w = gen.random_problem(48, B=1, H=3, D=D, T=T, vbs=[256, 129, 192, 190, 64, 40, 1, 128, 0, 255],
                           density=0.8, pad="naninf")
    print(f"tile 256 short halves: NT={w.NT}", flush=True)
    compare(run_fwd(w), oracle_out(oracle_mod, w), label="tile 256 short halves")


def test_split_lists_of_short_tiles(oracle_mod):
    """Lists cut into segments (partials merged by a second launch) whose tiles are
    mostly short: each segment pairs its own short tiles."""
    import torch

    w = gen.random_problem(49, B=1, H=2, D=128, T=128, vbs=[40] * 20 + [90, 64, 64, 1], density=0.8,
                           pad="naninf")
    args = _launch_args(w)
    assert bsa.workspace_size(w.B, w.H, w.NT, w.T, w.D, w.MS) > 0, "this shape is meant to split its lists"
    ref = oracle_out(oracle_mod, w)
    compare(bits_from_dev(bsa.fwd(*args, w.T)), ref, label="split lists, short tiles")
    compare(bits_from_dev(bsa.fwd(*args, w.T, workspace=None)), ref, label="whole query tiles, short tiles")
    torch.cuda.synchronize()


def test_nan_filled_output_buffer_is_overwritten():
    import torch

    w = gen.random_problem(42, B=2, H=2, D=128, T=128, vbs=[128, 60, 0, 128], density=0.5)
    ref = run_fwd(w)
    out = torch.full(w.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    got = run_fwd(w, out=out)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("name", ["ragged", "stress"])
def test_repeated_runs_are_bit_identical(name):
    """Also where lists pair their tiles (stress): the pairing and the order of the
    steps are fixed by the lengths and list positions alone."""
    w = gen.make(name)
    a = run_fwd(w)
    b = run_fwd(w)
    np.testing.assert_array_equal(a, b)


def test_minus_inf_tile_before_a_finite_one(oracle_mod):
    """A listed tile whose logits are all -inf, then a finite tile: the row is finite and
    equals the run without the -inf tile (guarded online softmax)."""
    T, D = 64, 64
    w = gen.random_problem(43, B=1, H=1, D=D, T=T, vbs=[T, T, T], counts=0, MS=2)
    w.q[0, 0, 0:T, 0] = gen.to_bf16_bits(np.full(T, -1.0, np.float32))
    w.k[0, 0, T:2 * T, 0] = gen.BF16_POS_INF
    w.q2k_num[0, 0, 0] = 2
    w.q2k_idx[0, 0, 0] = [1, 2]
    ref = oracle_out(oracle_mod, w)
    assert np.isfinite(ref[0, 0, :T]).all()
    got = run_fwd(w)
    compare(got, ref, label="-inf tile first")
    w.q2k_num[0, 0, 0] = 1
    w.q2k_idx[0, 0, 0] = [2, 0]
    np.testing.assert_array_equal(got[0, 0, :T], run_fwd(w)[0, 0, :T])


def test_all_minus_inf_row_is_nan(oracle_mod):
    T, D = 128, 128
    w = gen.random_problem(44, B=1, H=1, D=D, T=T, vbs=[T, 90, T], counts=2, MS=2, pad="naninf")
    w.q[0, 0, 5] = 0
    w.q[0, 0, 5, 0] = gen.BF16_NEG_INF
    valid = gen.contiguous_map(w.vbs, T) >= 0
    w.k[0, 0, valid, 0] = gen.to_bf16_bits(np.abs(gen.bf16_bits_to_f32(w.k[0, 0, valid, 0])) + 1)
    got = run_fwd(w)
    f = gen.bf16_bits_to_f32(got)
    assert np.isnan(f[0, 0, 5]).all()
    compare(got, oracle_out(oracle_mod, w), label="-inf row")


def test_single_valid_key_is_exact():
    T, D = 128, 128
    w = gen.random_problem(45, B=1, H=2, D=D, T=T, vbs=[T, 1, T - 1], counts=1, MS=1)
    w.q2k_idx[...] = 1
    got = run_fwd(w)
    for h in range(2):
        for row in list(range(T)) + list(range(2 * T, 3 * T - 1)):
            np.testing.assert_array_equal(got[0, h, row], w.v[0, h, T])


def test_large_logits_stay_finite(oracle_mod):
    """Query scaled by 20: some logits exceed log(FLT_MAX) without the max shift."""
    w = gen.random_problem(46, B=1, H=2, D=128, T=128, vbs=[128, 100, 128, 128], density=0.8)
    w.q[...] = gen.to_bf16_bits(gen.bf16_bits_to_f32(w.q) * 20)
    ref = oracle_out(oracle_mod, w)
    compare(run_fwd(w), ref, label="large logits")


@pytest.mark.parametrize("T,D", [(64, 64), (128, 128)])
def test_rising_logit_scale(oracle_mod, T, D):
    """Key tiles scaled up along the list, so that the running max rises from
    tile to tile by amounts both below and far above the offset slack of the
    online softmax (the exponent offset moves only on large rises)."""
    NT = 12
    w = gen.random_problem(51, B=1, H=2, D=D, T=T, vbs=[T] * (NT - 1) + [T - 9], counts=NT, MS=NT)
    w.q[...] = gen.to_bf16_bits(gen.bf16_bits_to_f32(w.q) * 3)
    for j in range(NT):
        sl = slice(j * T, (j + 1) * T)
        w.k[:, :, sl] = gen.to_bf16_bits(gen.bf16_bits_to_f32(w.k[:, :, sl]) * (0.25 + 0.4 * j))
    ref = oracle_out(oracle_mod, w)
    compare(run_fwd(w), ref, label=f"rising scale T={T} D={D}")


@pytest.mark.parametrize("T,D", [(64, 64), (128, 128)])
def test_index_handling_probe(oracle_mod, T, D):
    """Q = K = 0 gives uniform weights; V rows of tile j are the one-hot e_(j mod D), so
    the output's non-zero pattern names exactly the listed tiles (bit-exact pattern)."""
    NT = 24
    vbs = [T - (3 * t) % T for t in range(NT)]
    w = gen.random_problem(47, B=1, H=2, D=D, T=T, vbs=vbs, density=0.3)
    w.q[...] = 0
    w.k[...] = 0
    w.v[...] = 0
    one = gen.to_bf16_bits(np.float32([1.0]))[0]
    for j in range(NT):
        w.v[:, :, j * T: j * T + vbs[j], j % D] = one
    ref = oracle_out(oracle_mod, w)
    got = run_fwd(w)
    f = gen.bf16_bits_to_f32(got)
    np.testing.assert_array_equal(f != 0, ref != 0)
    compare(got, ref, label="index probe")


def test_out_of_range_contents_stay_memory_safe():
    """Invalid device-resident contents are clamped or skipped (output unspecified)."""
    import torch

    w = gen.random_problem(48, B=1, H=2, D=64, T=64, vbs=[64, 30, 64], counts=2, MS=2)
    idx = w.q2k_idx.copy()
    idx[0, 0, 0] = [-5, 7]
    idx[0, 1, 1] = [3, 1 << 30]
    num = w.q2k_num.copy()
    num[0, 0, 2] = 99
    num[0, 1, 0] = -4
    vbs = w.vbs.copy()
    vbs[1] = 500
    vbs[2] = -3
    run_fwd(w, idx=idx, num=num, vbs=vbs)
    torch.cuda.synchronize()


def test_non_gfx950_architecture_fails_closed():
    import torch

    w = gen.random_problem(49, B=1, H=1, D=64, T=64, vbs=[64, 64], counts=1, MS=1)
    lib = bsa.load()
    sentinel = torch.full(w.q.shape, 7.0, dtype=torch.bfloat16, device="cuda")
    lib.bsa_test_override_arch(b"gfx942")
    try:
        with pytest.raises(bsa.BsaError) as e:
            run_fwd(w, out=sentinel)
        assert e.value.status == 5
        with pytest.raises(bsa.BsaError):
            bsa.tile_layout([to_dev(w.tok["q"])], to_dev(w.tile_src_token), 64)
    finally:
        lib.bsa_test_override_arch(None)
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all()), "nothing may be written on a refused device"
    run_fwd(w)  # the real architecture is restored


def test_runs_on_a_non_default_stream(oracle_mod):
    import torch

    w = gen.random_problem(50, B=1, H=2, D=128, T=128, vbs=[128, 77, 128], density=0.7)
    args = [to_dev(x) for x in (w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = bsa.fwd(*args, w.T)
    s.synchronize()
    compare(bits_from_dev(out), oracle_out(oracle_mod, w), label="side stream")


def _launch_args(w):
    return [to_dev(x) for x in (w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs)]


def test_split_lists_back_to_back_shapes_on_one_stream(oracle_mod):
    """Few items with long lists are cut into list segments whose partial results
    meet in the workspace and are merged by a second launch.  Two shapes alternate on
    one stream without a sync, all through ONE caller workspace (sized for the larger
    plan), so every launch overwrites slots the previous one left: the workspace
    carries nothing from call to call, and repeated calls agree bit for bit."""
    import torch

    wa = gen.random_problem(61, B=1, H=2, D=128, T=128, vbs=[128] * 20 + [90], density=0.8)
    wb = gen.random_problem(62, B=2, H=3, D=128, T=128, vbs=[128, 3] + [128] * 30, density=0.6,
                            pad="naninf")
    args_a, args_b = _launch_args(wa), _launch_args(wb)
    need = max(bsa.workspace_size(x.B, x.H, x.NT, x.T, x.D, x.MS) for x in (wa, wb))
    assert need > 0, "these shapes are meant to split their lists"
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)  # NaN bit patterns everywhere: nothing may depend on its contents
    outs = []
    for i in range(3):
        outs.append(("a", bsa.fwd(*args_a, wa.T, workspace=ws)))
        outs.append(("b", bsa.fwd(*args_b, wb.T, workspace=ws)))
    torch.cuda.synchronize()
    ref = {"a": oracle_out(oracle_mod, wa), "b": oracle_out(oracle_mod, wb)}
    first = {}
    for name, out in outs:
        bits = bits_from_dev(out)
        compare(bits, ref[name], label=f"alternating {name}")
        if name in first:  # the merge order is fixed: repeated launches agree bit for bit
            np.testing.assert_array_equal(bits, first[name])
        first.setdefault(name, bits)


def test_workspace_choices(oracle_mod):
    """A shape that splits its lists: with the library's workspace, with none (whole
    query tiles only, one launch) and with one too small (refused, nothing written).
    Both runs match the oracle; they may differ only in the last bits."""
    import torch

    w = gen.random_problem(66, B=1, H=2, D=128, T=128, vbs=[128] * 20 + [90], density=0.8)
    args = _launch_args(w)
    need = bsa.workspace_size(w.B, w.H, w.NT, w.T, w.D, w.MS)
    assert need > 0
    split = bits_from_dev(bsa.fwd(*args, w.T))
    whole = bits_from_dev(bsa.fwd(*args, w.T, workspace=None))
    ref = oracle_out(oracle_mod, w)
    compare(split, ref, label="split lists")
    compare(whole, ref, label="whole query tiles")
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    sentinel = torch.full(w.q.shape, 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bsa.BsaError) as e:
        bsa.fwd(*args, w.T, out=sentinel, workspace=small)
    assert e.value.status == 1
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all()), "a refused call writes nothing"


# Shapes with more than four rounds of query tiles for the resident workgroups of a
# 256-CU MI355X (T = D = 128: 512 resident, 2400 items; T = D = 64: 2048 resident,
# 9600 items), whose last round is at least half full (no list is cut).
PERSISTENT = {
    (128, 128): dict(H=40, vbs=[128] * 59 + [77], counts=10),
    (64, 64): dict(H=24, vbs=[64] * 399 + [41], counts=8),
}


@pytest.mark.parametrize("T,D", sorted(PERSISTENT))
def test_persistent_launch_same_bits_as_one_tile_per_workgroup(oracle_mod, T, D):
    """Four or more rounds of query tiles run as one round of workgroups taking tiles
    from per-XCD queues whose counters are the whole workspace (512 bytes): the same
    bits as the launch without a workspace (one query tile per workgroup), the same
    bits through bsa_fwd_noalloc, and the oracle's values on sampled rows."""
    import torch

    cfg = PERSISTENT[(T, D)]
    w = gen.random_problem(71 + T, B=1, H=cfg["H"], D=D, T=T, vbs=cfg["vbs"], counts=cfg["counts"],
                           pad="naninf")
    print(f"persistent T={T} D={D}: {w.B * w.H * w.NT} query tiles", flush=True)
    assert bsa.workspace_size(w.B, w.H, w.NT, w.T, w.D, w.MS) == 512
    args = _launch_args(w)
    pers = bits_from_dev(bsa.fwd(*args, w.T))
    one = bits_from_dev(bsa.fwd(*args, w.T, workspace=None))
    np.testing.assert_array_equal(pers, one)
    out = torch.empty_like(args[0])
    bsa.fwd_noalloc(*args, w.T, out)
    np.testing.assert_array_equal(bits_from_dev(out), pers)
    rows = sample_rows(w, 256, np.random.default_rng(5))
    ref = oracle_mod.fwd_rows(w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs, w.T, rows)
    compare(pers.reshape(-1, D)[rows], ref, label=f"persistent T={T} D={D}")
    assert np.all(pers[padding_rows(w)] == 0)


def test_persistent_launch_with_cut_lists_and_graph_replays(oracle_mod):
    """More than four rounds of query tiles AND a last round less than half full: the
    workspace holds the queue counters and the partials of the cut lists.  Matches
    the oracle on sampled rows; captured into a graph (the counter-clearing kernel,
    the forward and the merge), every replay gives the eager bits."""
    import torch

    w = gen.random_problem(73, B=1, H=8, D=128, T=128, vbs=[128] * 280 + [50], counts=12)
    print(f"persistent with cut lists: {w.B * w.H * w.NT} query tiles", flush=True)
    need = bsa.workspace_size(w.B, w.H, w.NT, w.T, w.D, w.MS)
    assert need > 512
    args = _launch_args(w)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(args[0])
    bsa.fwd(*args, w.T, out=out, workspace=ws)
    torch.cuda.synchronize()
    eager = bits_from_dev(out)
    rows = sample_rows(w, 256, np.random.default_rng(6))
    ref = oracle_mod.fwd_rows(w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs, w.T, rows)
    compare(eager.reshape(-1, w.D)[rows], ref, label="persistent, cut lists")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        bsa.fwd(*args, w.T, out=out, workspace=ws)
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan"))
        ws.fill_(255)  # stale counters and partials: the call clears and rewrites what it uses
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits_from_dev(out), eager, err_msg=f"replay {r}")
        bsa.fwd(*args, w.T, out=out, workspace=ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits_from_dev(out), eager, err_msg=f"eager after replay {r}")


def test_split_lists_on_two_concurrent_streams(oracle_mod):
    """Launches on different streams may overlap; each call has its own workspace."""
    import torch

    wa = gen.random_problem(63, B=1, H=1, D=128, T=64, vbs=[64] * 40, density=0.9)
    wb = gen.random_problem(64, B=1, H=3, D=64, T=128, vbs=[128] * 24 + [17], density=0.7)
    args_a, args_b = _launch_args(wa), _launch_args(wb)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for i in range(4):
        with torch.cuda.stream(s1):
            outs.append(("a", bsa.fwd(*args_a, wa.T)))
        with torch.cuda.stream(s2):
            outs.append(("b", bsa.fwd(*args_b, wb.T)))
    s1.synchronize()
    s2.synchronize()
    ref = {"a": oracle_out(oracle_mod, wa), "b": oracle_out(oracle_mod, wb)}
    for name, out in outs:
        compare(bits_from_dev(out), ref[name], label=f"two streams {name}")


def test_same_bits_on_every_stream(oracle_mod):
    """The output bits do not depend on the stream: the same split shape on twelve
    streams (used concurrently, each call with its own workspace) gives identical
    bits on all of them, streams 1 and 12 included."""
    import torch

    w = gen.random_problem(65, B=1, H=2, D=128, T=128, vbs=[128] * 20 + [90], density=0.8)
    assert bsa.workspace_size(w.B, w.H, w.NT, w.T, w.D, w.MS) > 0
    args = _launch_args(w)
    streams = [torch.cuda.Stream() for _ in range(12)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(2):
        for s in streams:
            with torch.cuda.stream(s):
                outs.append(bsa.fwd(*args, w.T))
    for s in streams:
        s.synchronize()
    first = bits_from_dev(outs[0])
    compare(first, oracle_out(oracle_mod, w), label="stream 1")
    for n, out in enumerate(outs):
        np.testing.assert_array_equal(bits_from_dev(out), first,
                                      err_msg=f"stream {n % len(streams) + 1}")


def test_graph_capture_replays_match_eager(oracle_mod):
    """The layout and the forward captured into a HIP graph on a fresh stream whose
    FIRST library call happens inside the capture (the ragged workload splits lists,
    so the capture holds the segment launch, the merge launch and a workspace from
    the graph's memory pool).  Each replay, with eager work and a sync between, gives
    the eager result bit for bit."""
    import torch

    w = gen.ragged(gate=True)
    assert bsa.workspace_size(w.B, w.H, w.NT, w.T, w.D, w.MS) > 0
    tok = [to_dev(w.tok[x]) for x in ("q", "k", "v", "gate")]
    src = to_dev(w.tile_src_token)
    idx, num, vbs = to_dev(w.q2k_idx), to_dev(w.q2k_num), to_dev(w.vbs)
    tiled = [torch.empty((w.B, w.H, w.S, w.D), dtype=torch.bfloat16, device="cuda") for _ in tok]
    out = torch.empty((w.B, w.H, w.S, w.D), dtype=torch.bfloat16, device="cuda")

    def step():
        bsa.tile_layout(tok, src, w.T, outs=tiled)
        bsa.fwd(tiled[0], tiled[1], tiled[2], idx, num, vbs, w.T, out=out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()  # the first call on this stream
    torch.cuda.synchronize()
    step()  # eager, on the default stream
    torch.cuda.synchronize()
    eager = bits_from_dev(out)
    compare(eager, oracle_out(oracle_mod, w), label="eager ragged")
    for r in range(4):
        out.fill_(float("nan"))
        for t in tiled:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits_from_dev(out), eager, err_msg=f"replay {r}")
        with torch.cuda.stream(side):
            step()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits_from_dev(out), eager, err_msg=f"eager after replay {r}")


@pytest.mark.parametrize("D", [64, 128])
def test_tile_256_random_lists(oracle_mod, D):
    """256-row tiles: lengths above and below 128 (one or two non-empty halves), an
    empty tile, long enough lists that the last round is split into segments."""
    T = 256
    vbs = [256, 200, 129, 128, 100, 0, 1, 256, 77, 250]
    w = gen.random_problem(300 + D, B=1, H=3, D=D, T=T, vbs=vbs, density=0.7, pad="naninf")
    print(f"fwd tile 256 D={D} NT={w.NT}", flush=True)
    compare(run_fwd(w), oracle_out(oracle_mod, w), label=f"tile 256 D={D}")


def test_tile_256_duplicates_and_lse(oracle_mod):
    import oracle

    T, D = 256, 128
    w = gen.random_problem(310, B=2, H=1, D=D, T=T, vbs=[256, 130, 128, 3], counts=3, MS=3,
                           duplicates=True)
    w.q2k_num[1, 0, 2] = 0
    print("fwd tile 256 duplicates + lse", flush=True)
    q, k, v = (to_dev(x) for x in (w.q, w.k, w.v))
    out, lse, _ = bsa.fwd_lse(q, k, v, to_dev(w.q2k_idx), to_dev(w.q2k_num), to_dev(w.vbs), T)
    compare(bits_from_dev(out), oracle_out(oracle_mod, w), label="tile 256 duplicates")
    _, lse64 = oracle.fwd64(w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs, T)
    got = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(got), np.isneginf(lse64))
    fin = np.isfinite(lse64)
    np.testing.assert_allclose(got[fin], lse64[fin], rtol=1e-5, atol=1e-4)
