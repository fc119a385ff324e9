"""GPU parity of the coarse stage (bsa_coarse, bsa_coarse_combine) against the oracle.

The kept tile lists and counts are compared bit for bit: the pooled means and the
logits are binary32 in the same fixed order on both sides (parity of the definition is
unpinned by the pages, which do not describe this stage; the oracle's own pins are in
test_oracle_coarse_pins.py).  The coarse output is compared within 1e-4 of its scale
(fp32 sums in another order and the GPU's exponential), and the gated layer output
out + gate * coarse with the forward's bar.
"""
import numpy as np
import pytest

import block_sparse_tiled_amd as bsa
from block_sparse_tiled_amd import inputs as gen
from parity import bits_from_dev, compare, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    bsa.load()


def run_coarse(q, k, v, vbs, T, topk, max_sel=None):
    import torch

    idx, num, oc = bsa.coarse(to_dev(q), to_dev(k), to_dev(v), to_dev(vbs), T, topk,
                              max_sel=max_sel)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), num.cpu().numpy(), oc.cpu().numpy()


def check(q, k, v, vbs, T, topk, max_sel=None, label=""):
    import oracle

    got_idx, got_num, got_oc = run_coarse(q, k, v, vbs, T, topk, max_sel)
    ref_idx, ref_num, ref_oc = oracle.coarse(q, k, v, vbs, T, topk, max_sel)
    np.testing.assert_array_equal(got_num, ref_num, err_msg=f"{label}: counts")
    np.testing.assert_array_equal(got_idx, ref_idx, err_msg=f"{label}: lists")
    assert np.array_equal(np.isnan(got_oc), np.isnan(ref_oc)), f"{label}: coarse NaN mask"
    fin = np.isfinite(ref_oc)
    scale = max(1.0, float(np.abs(ref_oc[fin]).max())) if fin.any() else 1.0
    err = float(np.abs(got_oc[fin] - ref_oc[fin]).max()) if fin.any() else 0.0
    print(f"{label}: lists equal, coarse output max |diff| {err:.2e}", flush=True)
    assert err <= 1e-4 * scale, f"{label}: coarse output max |diff| {err:.3e}"
    return ref_idx, ref_num, ref_oc


def randn(rng, shape, sigma=1.0):
    return gen.to_bf16_bits((sigma * rng.standard_normal(shape)).astype(np.float32))


@pytest.mark.parametrize("T,D,NT,topk", [(64, 64, 8, 3), (64, 128, 40, 7), (128, 128, 17, 17),
                                         (128, 64, 300, 25), (256, 128, 9, 4), (64, 128, 1100, 40),
                                         (128, 128, 5, 0)])
def test_random_problems(T, D, NT, topk):
    """NT past 256 and past 1024 reach the wider register blocks of the selection."""
    rng = np.random.default_rng(T + D + NT)
    vbs = rng.integers(0, T + 1, NT).astype(np.int32)
    vbs[rng.random(NT) < 0.15] = 0
    vbs[0] = T
    B, H = (1, 2) if NT > 200 else (2, 3)
    q, k, v = (randn(rng, (B, H, NT * T, D)) for _ in range(3))
    # padding rows hold NaN / Inf: never read
    pad = (np.arange(NT * T) % T) >= np.repeat(vbs, T)
    for x in (q, k, v):
        x[:, :, pad] = 0x7FC0
    print(f"coarse T={T} D={D} NT={NT} topk={topk}", flush=True)
    check(q, k, v, vbs, T, topk, max_sel=topk + 3, label=f"T={T} D={D} NT={NT} topk={topk}")


def test_most_tiles():
    """BSA_COARSE_MAX_TILES tiles in one head (64-row tiles, D = 64): the widest
    selection register block and eight chunks of the coarse output's staging."""
    rng = np.random.default_rng(4096)
    T, D, NT = 64, 64, bsa.COARSE_MAX_TILES
    vbs = rng.integers(1, T + 1, NT).astype(np.int32)
    vbs[rng.random(NT) < 0.05] = 0
    q, k, v = (randn(rng, (1, 1, NT * T, D)) for _ in range(3))
    print(f"coarse most tiles NT={NT}", flush=True)
    check(q, k, v, vbs, T, 40, max_sel=41, label=f"NT={NT}")


def test_ties_nan_and_every_tile():
    """Copies of one key tile give equal logits (the lower index is kept); a NaN in a
    valid key row ranks that tile as -inf; topk above the tile count keeps every
    non-empty tile."""
    rng = np.random.default_rng(5)
    T, D, NT = 64, 128, 12
    vbs = np.array([64, 64, 64, 0, 64, 64, 30, 64, 64, 64, 1, 64], np.int32)
    q, k, v = (randn(rng, (1, 2, NT * T, D)) for _ in range(3))
    for t in (4, 7, 9):  # tiles 4, 7 and 9 equal tile 1: tied logits
        k[:, :, t * T:(t + 1) * T] = k[:, :, T:2 * T]
    k[:, 1, 5 * T + 3, 7] = 0x7FC0  # a NaN in a valid row of tile 5, head 1
    for topk in (1, 2, 4, 6, 11, 20):
        check(q, k, v, vbs, T, topk, max_sel=20, label=f"ties topk={topk}")


def test_video_config_full_size():
    """The video configuration's shape (12 heads, 512 tiles of 64, the last of 56),
    32 tiles kept per query tile: every list of every head, bit for bit."""
    w = gen.video()
    print("coarse video full size", flush=True)
    check(w.q, w.k, w.v, w.vbs, w.T, 32, label="video")


def test_layer_output_coarse_then_fine_then_combine():
    """The whole layer on the ragged configuration: the coarse stage picks 16 key tiles
    per query tile, the fine forward attends to them, and the gated coarse output is
    added: out = fine + gate * coarse (the oracle chain of the same three steps)."""
    import torch

    import oracle

    w = gen.ragged(gate=True)
    (gate_bits,) = oracle.tile_layout([w.tok["gate"]], w.tile_src_token, w.T)
    q, k, v, gate = (to_dev(x) for x in (w.q, w.k, w.v, gate_bits))
    vbs = to_dev(w.vbs)
    idx, num, oc = bsa.coarse(q, k, v, vbs, w.T, 16)
    out = bsa.fwd(q, k, v, idx, num, vbs, w.T)
    bsa.coarse_combine(out, gate, oc, vbs, w.T)
    torch.cuda.synchronize()
    ref_idx, ref_num, ref_oc = oracle.coarse(w.q, w.k, w.v, w.vbs, w.T, 16)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    fine = oracle.fwd(w.q, w.k, w.v, ref_idx, ref_num, w.vbs, w.T)
    g = gen.bf16_bits_to_f32(gate_bits)
    valid = (np.arange(w.S) % w.T) < np.repeat(w.vbs, w.T)
    want = fine + np.where(valid[None, None, :, None], g * np.repeat(ref_oc, w.T, axis=2), 0.0)
    compare(bits_from_dev(out), want.astype(np.float32), label="layer output")


def test_graph_capture_of_the_coarse_stage():
    """The four coarse launches captured into a graph replay the eager lists bit for bit."""
    import torch

    rng = np.random.default_rng(11)
    T, D, NT = 128, 128, 20
    vbs = np.full(NT, T, np.int32)
    q, k, v = (to_dev(randn(rng, (1, 4, NT * T, D))) for _ in range(3))
    dvbs = to_dev(vbs)
    ws = torch.empty(bsa.coarse_workspace_size(1, 4, NT, T, D), dtype=torch.uint8, device="cuda")
    idx = torch.empty((1, 4, NT, 6), dtype=torch.int32, device="cuda")
    num = torch.empty((1, 4, NT), dtype=torch.int32, device="cuda")
    oc = torch.empty((1, 4, NT, D), dtype=torch.float32, device="cuda")
    bsa.coarse(q, k, v, dvbs, T, 6, q2k_idx=idx, q2k_num=num, coarse_out=oc, workspace=ws)
    torch.cuda.synchronize()
    eager = (idx.cpu().numpy(), num.cpu().numpy(), oc.cpu().numpy())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        bsa.coarse(q, k, v, dvbs, T, 6, q2k_idx=idx, q2k_num=num, coarse_out=oc, workspace=ws)
    for r in range(3):
        idx.fill_(-7)
        oc.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(idx.cpu().numpy(), eager[0], err_msg=f"replay {r}")
        np.testing.assert_array_equal(num.cpu().numpy(), eager[1])
        np.testing.assert_array_equal(oc.cpu().numpy(), eager[2])


def draw_coarse_problem(case):
    """A seeded random coarse-stage problem: tile 64/128/256, head size 64/128, up to 700
    tiles with empty and short ones, topk anywhere from 0 to past the tile count, and (in
    a third of the cases) inputs from a handful of values, so that equal logits are
    common and the lower-index rule decides."""
    rng = np.random.default_rng(9000 + case)
    T = int(rng.choice([64, 128, 256]))
    D = int(rng.choice([64, 128]))
    NT = int(rng.choice([1, 2, 5, 17, 64, 130, 300, 700]))
    B, H = (1, 1) if NT > 200 else (int(rng.integers(1, 3)), int(rng.integers(1, 4)))
    vbs = rng.integers(0, T + 1, NT).astype(np.int32)
    vbs[rng.random(NT) < 0.2] = 0
    vbs[rng.random(NT) < 0.3] = T
    topk = int(rng.integers(0, NT + 3))
    max_sel = topk + int(rng.integers(0, 3))
    ties = rng.random() < 0.35
    shape = (B, H, NT * T, D)
    if ties:
        vals = np.array([-1.0, -0.5, 0.0, 0.5, 1.0], np.float32)
        q, k, v = (gen.to_bf16_bits(vals[rng.integers(0, 5, shape)]) for _ in range(3))
    else:
        q, k, v = (randn(rng, shape, float(rng.choice([0.5, 1.0, 2.0]))) for _ in range(3))
    pad = (np.arange(NT * T) % T) >= np.repeat(vbs, T)
    for x in (q, k, v):
        x[:, :, pad] = rng.choice([0x7FC0, 0x7F80, 0xFF80, 0])
    return q, k, v, vbs, T, topk, max_sel, f"T={T} D={D} B={B} H={H} NT={NT} topk={topk} ties={ties}"


@pytest.mark.parametrize("case", range(40))
def test_coarse_sweep(case):
    q, k, v, vbs, T, topk, max_sel, desc = draw_coarse_problem(case)
    print(f"coarse sweep {case}: {desc}", flush=True)
    check(q, k, v, vbs, T, topk, max_sel=max_sel, label=desc)


def _layout_pool_case(name):
    """A named configuration, or a small problem whose map has padding inside the valid
    rows, tokens out of range and 256-row tiles, at D = 64."""
    if name != "odd_map":
        return gen.make(name, gate=True), name == "video"
    rng = np.random.default_rng(77)
    B, H, D, T, NT = 2, 3, 64, 256, 5
    vbs = np.array([256, 0, 200, 1, 97], np.int32)
    S_tok = 700
    tok = {x: randn(rng, (B, S_tok, H, D)) for x in ("q", "k", "v", "gate")}
    src = np.full(NT * T, -1, np.int32)
    for t in range(NT):
        src[t * T:t * T + vbs[t]] = rng.integers(0, S_tok, vbs[t])
    src[2 * T + 5] = -1                  # padding inside tile 2's valid rows
    src[4 * T + 3] = S_tok               # out of range: padding
    src[4 * T + 4] = -(2**31)
    w = gen.Workload(name="odd_map", B=B, H=H, D=D, T=T, NT=NT, q=None, k=None, v=None,
                     q2k_idx=None, q2k_num=None, vbs=vbs, tok=tok, tile_src_token=src)
    return w, False


@pytest.mark.parametrize("name", ["video", "ragged", "dense256", "odd_map"])
def test_layout_pool_then_coarse_pooled(name):
    """bsa_tile_layout_pool writes the tile buffers bsa_tile_layout writes and the pooled
    tiles the oracle forms from them (bit for bit), and bsa_coarse_pooled on those gives
    bsa_coarse's lists, counts and coarse output bit for bit."""
    import torch

    import oracle

    w, with_gate = _layout_pool_case(name)
    names = ("q", "k", "v", "gate") if with_gate else ("q", "k", "v")
    tok = [to_dev(w.tok[x]) for x in names]
    src_map, vbs = to_dev(w.tile_src_token), to_dev(w.vbs)
    print(f"layout+pool {name}: B={w.B} H={w.H} NT={w.NT} T={w.T} D={w.D} tensors={len(tok)}",
          flush=True)
    tiled, pooled = bsa.tile_layout_pool(tok, src_map, vbs, w.T)
    ref_tiled = bsa.tile_layout(tok, src_map, w.T)
    torch.cuda.synchronize()
    for x, (a, b) in enumerate(zip(tiled, ref_tiled)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name}: tensor {x}"
    got = pooled.cpu().numpy()
    for x in range(3):
        want = oracle.coarse_pool(bits_from_dev(ref_tiled[x]), w.vbs, w.T)
        np.testing.assert_array_equal(got[x].view(np.uint32), want.view(np.uint32),
                                      err_msg=f"{name}: pooled tensor {x}")
    topk = min(16, w.NT)
    a = bsa.coarse(tiled[0], tiled[1], tiled[2], vbs, w.T, topk, max_sel=topk + 2)
    b = bsa.coarse_pooled(pooled, vbs, w.T, topk, max_sel=topk + 2)
    torch.cuda.synchronize()
    for x, (ta, tb) in enumerate(zip(a, b)):
        assert torch.equal(ta.view(torch.int32), tb.view(torch.int32)), f"{name}: coarse output {x}"


@pytest.mark.parametrize("name", ["video", "ragged"])
def test_unlayout_combine_matches_the_two_calls(name):
    """bsa_tile_unlayout_combine gives the bits of bsa_coarse_combine then
    bsa_tile_unlayout (tokens mapped to padding rows and out-of-range rows included)
    and leaves the fine output unchanged."""
    import torch

    w = gen.make(name, gate=True)
    q, k, v = (to_dev(x) for x in (w.q, w.k, w.v))
    vbs = to_dev(w.vbs)
    (gate,) = bsa.tile_layout([to_dev(w.tok["gate"])], to_dev(w.tile_src_token), w.T)
    idx, num, oc = bsa.coarse(q, k, v, vbs, w.T, min(16, w.NT))
    out = bsa.fwd(q, k, v, idx, num, vbs, w.T)
    S_tok = w.tok["q"].shape[1]
    src = w.tile_src_token
    rows = np.full(S_tok, -1, np.int32)
    ok = src >= 0
    rows[src[ok]] = np.nonzero(ok)[0]
    rows[::97] = w.NT * w.T + 5   # out of range: +0
    pad = np.nonzero(~ok)[0]
    if pad.size:
        rows[1::89] = pad[0]      # a padding row of its tile: passed through unchanged
    token_row = to_dev(rows)
    print(f"unlayout+combine {name}: tokens={S_tok}", flush=True)
    before = out.clone()
    got = bsa.tile_unlayout_combine(out, gate, oc, vbs, token_row, w.T)
    combined = out.clone()
    bsa.coarse_combine(combined, gate, oc, vbs, w.T)
    (want,) = bsa.tile_unlayout([combined], token_row, w.T)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), before.view(torch.int16)), "out was modified"
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{name}: layer output"
