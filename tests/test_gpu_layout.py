"""GPU parity of bsa_tile_layout against the oracle's NumPy gather: bit-exact."""
import numpy as np
import pytest

import block_sparse_tiled_amd as bsa
from block_sparse_tiled_amd import inputs as gen
from parity import bits_from_dev, run_fwd, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    bsa.load()


def run_layout(srcs, src_map, T, outs=None):
    res = bsa.tile_layout([to_dev(x) for x in srcs], to_dev(np.asarray(src_map, np.int32)), T,
                          outs=outs)
    return [bits_from_dev(o) for o in res]


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_contiguous_map_all_tensor_counts(oracle_mod, n):
    w = gen.ragged(gate=True)
    srcs = [w.tok[k] for k in ("q", "k", "v", "gate")[:n]]
    print(f"layout ragged n={n}", flush=True)
    got = run_layout(srcs, w.tile_src_token, w.T)
    want = oracle_mod.tile_layout(srcs, w.tile_src_token, w.T)
    for g, e in zip(got, want):
        np.testing.assert_array_equal(g, e)


@pytest.mark.parametrize("T,D", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_shuffled_map_with_padding(oracle_mod, T, D):
    rng = np.random.default_rng(T + D)
    B, H, NT = 2, 3, 7
    S_tok = NT * T - 2 * T + 5
    src = np.full(NT * T, -1, np.int32)
    rows = rng.choice(NT * T, size=S_tok, replace=False)
    src[rows] = rng.permutation(S_tok)
    srcs = [rng.integers(0, 65536, size=(B, S_tok, H, D), dtype=np.uint16) for _ in range(3)]
    got = run_layout(srcs, src, T)
    want = oracle_mod.tile_layout(srcs, src, T)
    for g, e in zip(got, want):
        np.testing.assert_array_equal(g, e)


def test_out_of_range_map_entries_are_padding(oracle_mod):
    import torch

    rng = np.random.default_rng(5)
    B, H, D, T, NT, S_tok = 1, 2, 128, 64, 3, 150
    src = rng.integers(-1, S_tok, size=NT * T).astype(np.int32)
    bad = src.copy()
    bad[[0, 10, 77]] = [S_tok, -7, 1 << 30]
    x = rng.integers(0, 65536, size=(B, S_tok, H, D), dtype=np.uint16)
    outs = [torch.full((B, H, NT * T, D), float("nan"), dtype=torch.bfloat16, device="cuda")]
    (got,) = run_layout([x], bad, T, outs=outs)
    clean = np.where((bad >= 0) & (bad < S_tok), bad, -1)
    (want,) = oracle_mod.tile_layout([x], clean, T)
    np.testing.assert_array_equal(got, want)


def test_video_config_four_tensors(oracle_mod):
    w = gen.video(gate=True)
    srcs = [w.tok[k] for k in ("q", "k", "v", "gate")]
    print("layout video, 4 tensors", flush=True)
    got = run_layout(srcs, w.tile_src_token, w.T)
    want = oracle_mod.tile_layout(srcs, w.tile_src_token, w.T)
    for g, e in zip(got, want):
        np.testing.assert_array_equal(g, e)


def test_layout_then_attention_equals_attention_on_tiled_inputs():
    """The two entry points chained on device give the same bits as the tiled inputs."""
    import torch

    w = gen.ragged()
    dq, dk, dv = bsa.tile_layout([to_dev(w.tok[k]) for k in ("q", "k", "v")],
                                 to_dev(w.tile_src_token), w.T)
    out = bsa.fwd(dq, dk, dv, to_dev(w.q2k_idx), to_dev(w.q2k_num), to_dev(w.vbs), w.T)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits_from_dev(out), run_fwd(w))


def run_unlayout(tiled, token_row, T, outs=None):
    res = bsa.tile_unlayout([to_dev(x) for x in tiled], to_dev(np.asarray(token_row, np.int32)),
                            T, outs=outs)
    return [bits_from_dev(o) for o in res]


@pytest.mark.parametrize("T,D", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_unlayout_matches_the_oracle(oracle_mod, T, D):
    """Random tile buffers (any bit pattern) gathered back with a shuffled map; a few
    map entries out of range give +0 rows; the NaN-filled outputs are fully overwritten."""
    import torch

    rng = np.random.default_rng(11 * T + D)
    B, H, NT = 2, 3, 5
    S_tok = NT * T - T // 2
    row = rng.permutation(NT * T)[:S_tok].astype(np.int32)
    row[[1, 7]] = [-3, NT * T]
    tiled = [rng.integers(0, 65536, size=(B, H, NT * T, D), dtype=np.uint16) for _ in range(2)]
    print(f"unlayout T={T} D={D}", flush=True)
    outs = [torch.full((B, S_tok, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
            for _ in tiled]
    got = run_unlayout(tiled, row, T, outs=outs)
    want = oracle_mod.tile_unlayout(tiled, row)
    for g, e in zip(got, want):
        np.testing.assert_array_equal(g, e)


def test_video_latent_cube_round_trip(oracle_mod):
    """The 21 x 30 x 52 latent in 4 x 4 x 4 cubes (624 tiles, many partial): the layout
    equals the oracle's and the inverse gather restores every token bit for bit."""
    rng = np.random.default_rng(21)
    vbs, src, row = bsa.cube_tile_map((21, 30, 52), (4, 4, 4))
    H, D, T = 12, 128, 64
    toks = [rng.integers(0, 65536, size=(1, 21 * 30 * 52, H, D), dtype=np.uint16)
            for _ in range(4)]
    print("cube layout video latent, 4 tensors", flush=True)
    tiled = run_layout(toks, src, T)
    for g, e in zip(tiled, oracle_mod.tile_layout(toks, src, T)):
        np.testing.assert_array_equal(g, e)
    back = run_unlayout(tiled, row, T)
    for g, e in zip(back, toks):
        np.testing.assert_array_equal(g, e)


@pytest.mark.parametrize("T,cube", [(64, (4, 4, 4)), (128, (2, 8, 8))])
def test_cube_tiled_attention_layer_step(oracle_mod, T, cube):
    """Layout, block-sparse attention and the inverse gather on a cube-tiled latent,
    against the oracle's forward on the same tiles gathered back the same way."""
    import torch

    from parity import compare

    rng = np.random.default_rng(T)
    latent = (5, 10, 12)
    vbs, src, row = bsa.cube_tile_map(latent, cube)
    NT = vbs.size
    B, H, D, MS = 1, 2, 128, 4
    S_tok = int(np.prod(latent))
    tok = {x: gen.to_bf16_bits(rng.standard_normal((B, S_tok, H, D)).astype(np.float32))
           for x in ("q", "k", "v")}
    idx = np.zeros((B, H, NT, MS), np.int32)
    num = rng.integers(0, MS + 1, size=(B, H, NT)).astype(np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(NT):
                idx[b, h, i] = np.sort(rng.choice(NT, size=MS, replace=False))
    print(f"cube layer step T={T} NT={NT}", flush=True)
    q, k, v = bsa.tile_layout([to_dev(tok[x]) for x in ("q", "k", "v")],
                              to_dev(src.astype(np.int32)), T)
    out = bsa.fwd(q, k, v, to_dev(idx), to_dev(num), to_dev(vbs), T)
    (got,) = bsa.tile_unlayout([out], to_dev(row), T)
    torch.cuda.synchronize()
    tq, tk, tv = oracle_mod.tile_layout([tok[x] for x in ("q", "k", "v")], src, T)
    ref_tiled = oracle_mod.fwd(tq, tk, tv, idx, num, vbs, T)
    (ref,) = oracle_mod.tile_unlayout([ref_tiled], row)
    compare(bits_from_dev(got), ref, label=f"cube layer step T={T}")


def test_tile_256_layout_and_unlayout(oracle_mod):
    """256-row tiles from a 4 x 8 x 8 cube map of the video latent; both directions."""
    rng = np.random.default_rng(256)
    vbs, src, row = bsa.cube_tile_map((21, 30, 52), (4, 8, 8))
    H, D, T = 2, 128, 256
    x = rng.integers(0, 65536, size=(1, 21 * 30 * 52, H, D), dtype=np.uint16)
    print("layout tile 256", flush=True)
    (tiled,) = run_layout([x], src, T)
    (want,) = oracle_mod.tile_layout([x], src, T)
    np.testing.assert_array_equal(tiled, want)
    (back,) = run_unlayout([tiled], row, T)
    np.testing.assert_array_equal(back, x)
