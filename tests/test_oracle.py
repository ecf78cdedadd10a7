"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what fixes the expected value: brute force over coordinates, a dense
Conv3d from torch (a library routine for the textbook operation), closed forms, exact
special cases and invariants.  Chosen so that a dropped tap, a wrong sign or index, a
transposed weight or a batch leak in the oracle fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import torch

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
OFFSETS = [(dx, dy, dz) for dx in (-1, 0, 1) for dy in (-1, 0, 1) for dz in (-1, 0, 1)]


def rand_sites(seed, batch, grid, frac):
    rng = np.random.default_rng(seed)
    n = max(1, int(round(frac * grid[0] * grid[1] * grid[2])))
    return workloads.random_sites(rng, batch, grid, n)


def brute_force_map(coords):
    """O(N^2 * 27): for each site and offset, scan every row for an equal coordinate."""
    n = len(coords)
    out = -np.ones((n, 27), dtype=np.int64)
    for t, d in enumerate(OFFSETS):
        target = coords.astype(np.int64) + np.array([0, *d])
        eq = (target[:, None, :] == coords[None, :, :]).all(-1)   # [n, n]
        hit = eq.any(1)
        out[hit, t] = eq.argmax(1)[hit]
    return out


def dense_reference(coords, x, w, bias, batch, grid, flip=False):
    """torch conv3d (cross-correlation, padding 1, float64) on the dense grid, read back at the
    active sites.  Inactive voxels are zero."""
    n, cin = x.shape
    cout = w.shape[2]
    dense = torch.zeros((batch, cin) + tuple(grid), dtype=torch.float64)
    c = torch.from_numpy(coords.astype(np.int64))
    dense[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]] = torch.from_numpy(np.asarray(x, np.float64))
    # [27, cin, cout] -> [cout, cin, 3, 3, 3] with tap t = 9(dx+1)+3(dy+1)+(dz+1) at (dx+1,dy+1,dz+1)
    wt = torch.from_numpy(np.asarray(w, np.float64)).reshape(3, 3, 3, cin, cout).permute(4, 3, 0, 1, 2)
    if flip:
        wt = torch.flip(wt, dims=[2, 3, 4])
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float64))
    y = torch.nn.functional.conv3d(dense, wt.contiguous(), b, padding=1)
    return y[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]].numpy()


@pytest.mark.parametrize("seed,batch,grid,frac", [
    (0, 1, (5, 5, 5), 0.3), (1, 2, (3, 4, 5), 0.5), (2, 1, (6, 2, 3), 1.0), (3, 3, (4, 4, 4), 0.1),
])
def test_map_matches_brute_force(oracle_mod, seed, batch, grid, frac):
    coords = rand_sites(seed, batch, grid, frac)
    rng = np.random.default_rng(seed + 100)
    coords = coords[rng.permutation(len(coords))]
    m = oracle_mod.build_map(coords, batch, grid)
    np.testing.assert_array_equal(m, brute_force_map(coords))


def test_map_symmetry_and_centre(oracle_mod):
    coords = rand_sites(7, 2, (16, 12, 20), 0.2)
    m = oracle_mod.build_map(coords, 2, (16, 12, 20))
    n = len(coords)
    assert (m[:, 13] == np.arange(n)).all()
    for t in range(27):
        i = np.nonzero(m[:, t] >= 0)[0]
        j = m[i, t]
        assert (m[j, 26 - t] == i).all()
        # the neighbour really is at the tap's offset, in the same batch entry
        d = coords[j].astype(np.int64) - coords[i]
        assert (d == np.array([0, *OFFSETS[t]])).all()


def test_full_occupancy_tap_counts(oracle_mod):
    g = (4, 5, 6)
    occ = np.ones(g, dtype=bool)
    coords = workloads.coords_from_occupancy([occ])
    m = oracle_mod.build_map(coords, 1, g)
    for t, d in enumerate(OFFSETS):
        expect = np.prod([gi - abs(di) for gi, di in zip(g, d)])
        assert (m[:, t] >= 0).sum() == expect


def test_hit_rate_closed_form(oracle_mod):
    # For N sites drawn uniformly without replacement from G^3 voxels, the expected number of
    # valid (site, tap) pairs is N + N(N-1) * ((3G-2)^3 - G^3) / (G^3 (G^3 - 1)).
    G, N = 48, 11000
    vals = []
    for seed in range(4):
        coords = rand_sites(50 + seed, 1, (G, G, G), N / G ** 3)
        m = oracle_mod.build_map(coords, 1, (G, G, G))
        vals.append((m >= 0).sum())
    expect = N + N * (N - 1) * ((3 * G - 2) ** 3 - G ** 3) / (G ** 3 * (G ** 3 - 1))
    assert abs(np.mean(vals) - expect) / (expect - N) < 0.01


@pytest.mark.parametrize("seed,batch,grid,cin,cout,frac", [
    (0, 1, (4, 4, 4), 1, 1, 1.0), (1, 1, (6, 6, 6), 3, 8, 0.5), (2, 2, (8, 8, 8), 8, 3, 0.1),
    (3, 2, (5, 7, 6), 4, 5, 0.5), (4, 1, (8, 4, 6), 8, 8, 1.0),
])
def test_conv_matches_dense_conv3d(oracle_mod, seed, batch, grid, cin, cout, frac):
    coords = rand_sites(seed, batch, grid, frac)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((len(coords), cin))
    w = rng.standard_normal((27, cin, cout))
    b = rng.standard_normal(cout)
    m = oracle_mod.build_map(coords, batch, grid)
    y = oracle_mod.conv(x, w, b, m)
    ref = dense_reference(coords, x, w, b, batch, grid)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_flip_matches_true_convolution(oracle_mod):
    coords = rand_sites(11, 1, (6, 6, 6), 0.5)
    rng = np.random.default_rng(11)
    x = rng.standard_normal((len(coords), 3))
    w = rng.standard_normal((27, 3, 4))
    m = oracle_mod.build_map(coords, 1, (6, 6, 6))
    y = oracle_mod.conv(x, w, None, m, flip=True)
    ref = dense_reference(coords, x, w, None, 1, (6, 6, 6), flip=True)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    # and the two orientations really differ for a non-symmetric kernel
    assert np.abs(y - oracle_mod.conv(x, w, None, m)).max() > 1e-3


def test_identity_centre_tap_is_exact(oracle_mod):
    coords = rand_sites(5, 2, (10, 10, 10), 0.3)
    rng = np.random.default_rng(5)
    c = 6
    x = rng.standard_normal((len(coords), c)).astype(np.float32)
    w = np.zeros((27, c, c))
    w[13] = np.eye(c)
    m = oracle_mod.build_map(coords, 2, (10, 10, 10))
    y = oracle_mod.conv(x, w, None, m)
    assert np.array_equal(y, x.astype(np.float64))


def test_isolated_voxels(oracle_mod):
    # sites two voxels apart never see each other: Y = X W[13] + b exactly in fp64
    coords = np.array([[0, 0, 0, 0], [0, 2, 0, 0], [0, 0, 2, 2], [1, 0, 0, 0], [0, 4, 4, 4]],
                      np.int32)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 4))
    w = rng.standard_normal((27, 4, 3))
    b = rng.standard_normal(3)
    m = oracle_mod.build_map(coords, 2, (5, 5, 5))
    assert (m[:, [t for t in range(27) if t != 13]] == -1).all()
    y = oracle_mod.conv(x, w, b, m)
    np.testing.assert_allclose(y, x @ w[13] + b, rtol=1e-14, atol=1e-14)


def test_hand_worked_pair(oracle_mod):
    # Two sites at x and x+1: the site at x sees its neighbour through tap (+1,0,0) = 22, the
    # site at x+1 through tap (-1,0,0) = 4.  With scalar channels:
    #   y0 = x0*w13 + x1*w22,  y1 = x1*w13 + x0*w4.
    coords = np.array([[0, 1, 1, 1], [0, 2, 1, 1]], np.int32)
    w = np.zeros((27, 1, 1))
    w[13], w[22], w[4] = 2.0, 3.0, 5.0
    x = np.array([[7.0], [11.0]])
    m = oracle_mod.build_map(coords, 1, (4, 4, 4))
    assert m[0, 22] == 1 and m[1, 4] == 0
    y = oracle_mod.conv(x, w, None, m)
    assert y[0, 0] == 7 * 2 + 11 * 3 and y[1, 0] == 11 * 2 + 7 * 5


def test_translation_equivariance(oracle_mod):
    coords = rand_sites(9, 1, (12, 12, 12), 0.2)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((len(coords), 5))
    w = rng.standard_normal((27, 5, 6))
    m = oracle_mod.build_map(coords, 1, (20, 20, 20))
    shifted = coords + np.array([0, 3, 5, 8], np.int32)
    m2 = oracle_mod.build_map(shifted, 1, (20, 20, 20))
    np.testing.assert_array_equal(m, m2)
    assert np.array_equal(oracle_mod.conv(x, w, None, m), oracle_mod.conv(x, w, None, m2))


def test_batch_isolation(oracle_mod):
    one = rand_sites(13, 1, (8, 8, 8), 0.4)
    two = np.concatenate([one, one + np.array([1, 0, 0, 0], np.int32)])
    rng = np.random.default_rng(13)
    x = rng.standard_normal((len(two), 4))
    w = rng.standard_normal((27, 4, 4))
    m = oracle_mod.build_map(two, 2, (8, 8, 8))
    n = len(one)
    assert ((m[:n] < n) & (m[:n] >= -1)).all() and ((m[n:] >= n) | (m[n:] == -1)).all()
    y = oracle_mod.conv(x, w, None, m)
    m1 = oracle_mod.build_map(one, 1, (8, 8, 8))
    np.testing.assert_array_equal(y[:n], oracle_mod.conv(x[:n], w, None, m1))
    np.testing.assert_array_equal(y[n:], oracle_mod.conv(x[n:], w, None, m1))


def test_row_permutation_equivariance(oracle_mod):
    coords = rand_sites(17, 2, (9, 9, 9), 0.3)
    rng = np.random.default_rng(17)
    x = rng.standard_normal((len(coords), 3))
    w = rng.standard_normal((27, 3, 2))
    y = oracle_mod.conv(x, w, None, oracle_mod.build_map(coords, 2, (9, 9, 9)))
    p = rng.permutation(len(coords))
    y2 = oracle_mod.conv(x[p], w, None, oracle_mod.build_map(coords[p], 2, (9, 9, 9)))
    np.testing.assert_allclose(y2, y[p], rtol=1e-13, atol=1e-13)


def test_linearity(oracle_mod):
    coords = rand_sites(19, 1, (7, 7, 7), 0.4)
    rng = np.random.default_rng(19)
    x1, x2 = rng.standard_normal((2, len(coords), 3))
    w = rng.standard_normal((27, 3, 4))
    m = oracle_mod.build_map(coords, 1, (7, 7, 7))
    lhs = oracle_mod.conv(2.0 * x1 - 3.0 * x2, w, None, m)
    rhs = 2.0 * oracle_mod.conv(x1, w, None, m) - 3.0 * oracle_mod.conv(x2, w, None, m)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_k1_is_per_voxel_linear(oracle_mod):
    coords = rand_sites(21, 2, (6, 6, 6), 0.5)
    rng = np.random.default_rng(21)
    x = rng.standard_normal((len(coords), 5))
    w = rng.standard_normal((1, 5, 7))
    b = rng.standard_normal(7)
    m1 = oracle_mod.build_map(coords, 2, (6, 6, 6), ksize=1)
    assert (m1[:, 0] == np.arange(len(coords))).all()
    ref = x @ w[0] + b
    np.testing.assert_allclose(oracle_mod.linear(x, w, b), ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle_mod.conv(x, w, b, m1), ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("bad,status", [
    ([0, -1, 0, 0], -2), ([0, 4, 0, 0], -2), ([0, 0, 0, 5], -2), ([2, 0, 0, 0], -2),
    ([-1, 0, 0, 0], -2), ([0, 1, 1, 1], -3),
])
def test_error_paths(oracle_mod, bad, status):
    coords = np.array([[0, 1, 1, 1], [1, 2, 2, 2], bad], np.int32)
    with pytest.raises(oracle_mod.OracleError) as e:
        oracle_mod.build_map(coords, 2, (4, 5, 5))
    assert e.value.status == status


def test_empty_input(oracle_mod):
    m = oracle_mod.build_map(np.zeros((0, 4), np.int32), 1, (4, 4, 4))
    assert m.shape == (0, 27)
    y = oracle_mod.conv(np.zeros((0, 3)), np.zeros((27, 3, 2)), None, m)
    assert y.shape == (0, 2)


def test_fleet_table_metric_definition():
    # The page's Mvox/s column is voxels / conv_ms; its 209,715 voxels is floor(0.1 * 128^3).
    g = json.load(open(os.path.join(GOLDEN, "fleet_benchmark.json")))
    assert g["voxels"] == int(0.1 * g["grid"] ** 3)
    for row in g["rows"]:
        mvox = g["voxels"] / (row["conv_ms"] * 1e-3) / 1e6
        # conv_ms is printed to 0.1 ms, so the quotient agrees to within that rounding
        assert abs(mvox - row["mvox_per_s"]) / row["mvox_per_s"] < 0.004
    v = g["version_history_m3ultra_ms"]
    assert round(v["per_offset_loop"] / v["fused_gather_matmul"], 1) == 2.1
    assert round(v["per_offset_loop"] / v["cached_device_index"], 1) == 5.9
    assert g["per_offset_dispatches"] == 2 * 3 ** 3


def test_workload_recipes_realised_sizes():
    w = workloads.make("tiny")
    assert w.dtype == "f32" and w.feats.dtype == torch.float32
    assert abs(w.n - 0.1 * 32 ** 3) < 5 * np.sqrt(32 ** 3 * 0.09)
    assert (np.diff(w.coords[:, 1] * 1024 + w.coords[:, 2] * 32 + w.coords[:, 3]) > 0).all()
    b = workloads.make("batch4", with_feats=False)
    counts = np.bincount(b.coords[:, 0], minlength=4)
    for cnt, p in zip(counts, (0.05, 0.10, 0.20, 0.30)):
        assert abs(cnt - p * 64 ** 3) < 5 * np.sqrt(64 ** 3 * p * (1 - p))
    assert [l.ksize for l in b.layers] == [3, 1]
    assert tuple(b.layers[0].weight.shape) == (27, 64, 128)
    assert tuple(b.layers[1].weight.shape) == (1, 128, 128)
