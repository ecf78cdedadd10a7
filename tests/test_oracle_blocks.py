"""Pins of the block oracle (activations, sparse group norm, conv epilogue, residual block)
against things other than itself (CPU only): torch's relu / silu / group_norm / conv3d (library
routines for the textbook operations) on the active sites, closed forms and exact cases.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads
from oracle import blocks


def sites(seed, batch, grid, frac):
    rng = np.random.default_rng(seed)
    n = max(1, int(round(frac * grid[0] * grid[1] * grid[2])))
    return workloads.random_sites(rng, batch, grid, n)


def dense_conv_at_sites(coords, x, w, bias, batch, grid):
    """torch conv3d (padding 1, float64) over a zero grid holding x at the sites, read back at
    the sites: the submanifold convolution."""
    n, cin = x.shape
    cout = w.shape[2]
    dense = torch.zeros((batch, cin) + tuple(grid), dtype=torch.float64)
    c = torch.from_numpy(coords.astype(np.int64))
    dense[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]] = torch.from_numpy(np.asarray(x, np.float64))
    wt = torch.from_numpy(np.asarray(w, np.float64)).reshape(3, 3, 3, cin, cout).permute(4, 3, 0, 1, 2)
    b = torch.from_numpy(np.asarray(bias, np.float64))
    y = F.conv3d(dense, wt.contiguous(), b, padding=1)
    return y[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]]


def torch_group_norm(x, coords, batch, groups, gamma, beta, eps):
    """torch group_norm over each batch entry's rows as a [1, C, n_b] tensor."""
    x = torch.as_tensor(np.asarray(x, np.float64))
    out = torch.empty_like(x)
    b_of = torch.from_numpy(coords[:, 0].astype(np.int64))
    g = None if gamma is None else torch.from_numpy(np.asarray(gamma, np.float64))
    be = None if beta is None else torch.from_numpy(np.asarray(beta, np.float64))
    for b in range(batch):
        m = b_of == b
        if m.any():
            out[m] = F.group_norm(x[m].T.unsqueeze(0), groups, g, be, eps)[0].T
    return out


def test_activations_match_torch():
    x = np.concatenate([np.linspace(-30, 30, 601), [-1e4, -745.0, -0.0, 0.0, 1e4]])
    xt = torch.from_numpy(x)
    np.testing.assert_array_equal(blocks.activation(x, "relu"), F.relu(xt).numpy())
    np.testing.assert_allclose(blocks.activation(x, "silu"), F.silu(xt).numpy(), rtol=1e-15,
                               atol=1e-300)
    np.testing.assert_array_equal(blocks.activation(x, "none"), x)
    with pytest.raises(ValueError):
        blocks.activation(x, "gelu")


@pytest.mark.parametrize("seed,batch,c,groups", [(0, 1, 32, 32), (1, 3, 64, 32), (2, 2, 128, 8),
                                                  (3, 4, 48, 1), (4, 2, 16, 16)])
def test_group_norm_matches_torch(seed, batch, c, groups):
    coords = sites(seed, batch, (6, 5, 7), 0.3)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((len(coords), c)) * 3.0 + rng.standard_normal(c)
    gamma, beta = rng.standard_normal(c), rng.standard_normal(c)
    got = blocks.group_norm(x, coords, batch, groups, gamma, beta, 1e-5)
    want = torch_group_norm(x, coords, batch, groups, gamma, beta, 1e-5).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # with the activation applied after the affine map
    got = blocks.group_norm(x, coords, batch, groups, gamma, beta, 1e-5, "silu")
    np.testing.assert_allclose(got, F.silu(torch.from_numpy(want)).numpy(), rtol=1e-12,
                               atol=1e-12)


def test_group_stats_closed_form():
    """Two sites of one entry, one group of two channels: mean and population variance by
    hand; an entry with no sites reports zeros."""
    coords = np.array([[0, 0, 0, 0], [0, 1, 0, 0], [2, 0, 0, 0]], np.int32)
    x = np.array([[1.0, 3.0], [5.0, 7.0], [-2.0, 2.0]])
    mean, var = blocks.group_stats(x, coords, 3, 1)
    np.testing.assert_array_equal(mean, [[4.0], [0.0], [0.0]])
    np.testing.assert_array_equal(var, [[5.0], [0.0], [4.0]])
    y = blocks.group_norm(x, coords, 3, 1, eps=0.0)
    np.testing.assert_allclose(y[2], [-1.0, 1.0])
    np.testing.assert_allclose(y[:2].ravel(), (np.array([1, 3, 5, 7]) - 4.0) / np.sqrt(5.0))


@pytest.mark.parametrize("act", ["none", "relu", "silu"])
def test_conv_epilogue_matches_dense(act):
    coords = sites(5, 2, (5, 6, 4), 0.4)
    rng = np.random.default_rng(5)
    n = len(coords)
    x = rng.standard_normal((n, 8))
    w = rng.standard_normal((27, 8, 6)) * 0.2
    b = rng.standard_normal(6)
    res = rng.standard_normal((n, 6))
    nbr = oracle.build_map(coords, 2, (5, 6, 4))
    got = blocks.conv_epilogue(x, w, b, nbr, act, res)
    y = dense_conv_at_sites(coords, x, w, b, 2, (5, 6, 4))
    y = {"none": y, "relu": F.relu(y), "silu": F.silu(y)}[act]
    np.testing.assert_allclose(got, (y + torch.from_numpy(res)).numpy(), rtol=1e-12, atol=1e-12)
    lin = blocks.linear_epilogue(x, w[13], b, act, res)
    z = torch.from_numpy(x) @ torch.from_numpy(w[13]) + torch.from_numpy(b)
    z = {"none": z, "relu": F.relu(z), "silu": F.silu(z)}[act]
    np.testing.assert_allclose(lin, (z + torch.from_numpy(res)).numpy(), rtol=1e-12, atol=1e-12)


def block_params(rng, c):
    return {"w1": rng.standard_normal((27, c, c)) * 0.1, "b1": rng.standard_normal(c),
            "w2": rng.standard_normal((27, c, c)) * 0.1, "b2": rng.standard_normal(c),
            "g1": 1 + 0.1 * rng.standard_normal(c), "be1": 0.1 * rng.standard_normal(c),
            "g2": 1 + 0.1 * rng.standard_normal(c), "be2": 0.1 * rng.standard_normal(c)}


def test_res_block_matches_dense_torch():
    """The whole block with torch's group_norm on each entry's rows, silu, and conv3d on a
    grid re-zeroed off the sites before each convolution."""
    batch, grid, c, groups = 2, (5, 4, 6), 16, 4
    coords = sites(7, batch, grid, 0.35)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((len(coords), c))
    p = block_params(rng, c)
    nbr = oracle.build_map(coords, batch, grid)
    got = blocks.res_block(x, coords, batch, nbr, p, groups, 1e-5)
    h = F.silu(torch_group_norm(x, coords, batch, groups, p["g1"], p["be1"], 1e-5))
    h = dense_conv_at_sites(coords, h.numpy(), p["w1"], p["b1"], batch, grid)
    h = F.silu(torch_group_norm(h.numpy(), coords, batch, groups, p["g2"], p["be2"], 1e-5))
    h = dense_conv_at_sites(coords, h.numpy(), p["w2"], p["b2"], batch, grid)
    np.testing.assert_allclose(got, (h + torch.from_numpy(x)).numpy(), rtol=1e-11, atol=1e-11)


def test_res_block_with_zero_convolutions_is_identity():
    coords = sites(8, 1, (4, 4, 4), 0.5)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((len(coords), 8))
    p = block_params(rng, 8)
    for k in ("w1", "b1", "w2", "b2"):
        p[k] = np.zeros_like(p[k])
    nbr = oracle.build_map(coords, 1, (4, 4, 4))
    np.testing.assert_array_equal(blocks.res_block(x, coords, 1, nbr, p, 4), x)


@pytest.mark.parametrize("c,act", [(32, "none"), (128, "silu"), (7, "relu")])
def test_layer_norm_matches_torch(c, act):
    rng = np.random.default_rng(c)
    x = rng.standard_normal((50, c)) * 4.0 + 3.0
    g, b = rng.standard_normal(c), rng.standard_normal(c)
    want = F.layer_norm(torch.from_numpy(x), (c,), torch.from_numpy(g), torch.from_numpy(b), 1e-6)
    want = {"none": want, "silu": F.silu(want), "relu": F.relu(want)}[act]
    np.testing.assert_allclose(blocks.layer_norm(x, g, b, 1e-6, act), want.numpy(), rtol=1e-12,
                               atol=1e-12)


def test_layer_norm_closed_form():
    """Row (1, 3): mean 2, population variance 1 -> (-1, 1) with eps 0."""
    np.testing.assert_allclose(blocks.layer_norm(np.array([[1.0, 3.0]]), eps=0.0), [[-1.0, 1.0]])


def test_convnext_block_matches_dense_torch():
    """torch conv3d on the dense grid, layer_norm, linear, silu, linear, plus the skip."""
    grid, c = (5, 6, 4), 8
    coords = sites(11, 1, grid, 0.4)
    rng = np.random.default_rng(11)
    x = rng.standard_normal((len(coords), c))
    p = {"w": rng.standard_normal((27, c, c)) * 0.1, "b": rng.standard_normal(c),
         "ln_g": 1 + 0.1 * rng.standard_normal(c), "ln_b": 0.1 * rng.standard_normal(c),
         "w1": rng.standard_normal((c, 4 * c)) * 0.3, "b1": rng.standard_normal(4 * c),
         "w2": rng.standard_normal((4 * c, c)) * 0.2, "b2": rng.standard_normal(c)}
    got = blocks.convnext_block(x, oracle.build_map(coords, 1, grid), p)
    h = dense_conv_at_sites(coords, x, p["w"], p["b"], 1, grid)
    h = F.layer_norm(h, (c,), torch.from_numpy(p["ln_g"]), torch.from_numpy(p["ln_b"]), 1e-6)
    h = F.silu(h @ torch.from_numpy(p["w1"]) + torch.from_numpy(p["b1"]))
    h = h @ torch.from_numpy(p["w2"]) + torch.from_numpy(p["b2"])
    np.testing.assert_allclose(got, (h + torch.from_numpy(x)).numpy(), rtol=1e-11, atol=1e-11)


def test_round_bf16_matches_torch_cast():
    """The oracle's bf16 storage rounding against torch's float32 -> bfloat16 cast (round to
    nearest, ties to even) on random values, exact ties, subnormals, signed zeros, overflow."""
    import torch
    rng = np.random.default_rng(5)
    ties = np.array([1 + k * 2.0 ** -8 for k in range(1, 16, 2)])            # halfway cases
    vals = np.concatenate([rng.standard_normal(200000) * 7, rng.standard_normal(1000) * 1e-39,
                           ties, -ties, [0.0, -0.0, 3.39e38, -3.39e38, 1e-45, 65504.0]])
    got = blocks.round_bf16(vals)
    want = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))
    # ties go to the even significand: 1 + 2^-8 -> 1, 1 + 3 * 2^-8 -> 1 + 2^-6
    assert blocks.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert blocks.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6


def test_blocks_store_hook_defaults_to_float64():
    """Without a storage rounding the blocks are unchanged; with it every stored layer output
    is representable in bf16 (a fixed point of the rounding)."""
    rng = np.random.default_rng(8)
    coords = np.array([[0, x, y, z] for x in range(3) for y in range(3) for z in range(2)],
                      np.int32)
    nbr = oracle.build_map(coords, 1, (3, 3, 2))
    c = 8
    p = {k: rng.standard_normal((27, c, c)) / np.sqrt(27 * c) for k in ("w1", "w2")}
    p.update({k: 0.1 * rng.standard_normal(c) for k in ("b1", "b2", "be1", "be2")})
    p.update({k: 1 + 0.1 * rng.standard_normal(c) for k in ("g1", "g2")})
    x = rng.standard_normal((len(coords), c))
    a = blocks.res_block(x, coords, 1, nbr, p, 4, 1e-5)
    b = blocks.res_block(x, coords, 1, nbr, p, 4, 1e-5, store=None)
    assert np.array_equal(a, b)
    r = blocks.res_block(x, coords, 1, nbr, p, 4, 1e-5, store=blocks.round_bf16)
    assert np.array_equal(r, blocks.round_bf16(r))
    assert np.abs(r - a).max() <= 0.05 * np.sqrt((a ** 2).mean())
