"""Pins of the resample oracle (downsample / upsample / spatial2channel / subdivide) against
things other than itself (CPU only): a dense max pool from torch (the library routine for the
textbook operation), a dense space-to-depth reshape, brute force over coordinates, and exact
identities between the ops.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import resample as rs


def sites(seed, batch, grid, frac):
    rng = np.random.default_rng(seed)
    n = max(1, int(round(frac * grid[0] * grid[1] * grid[2])))
    return workloads.random_sites(rng, batch, grid, n)


def feats_for(seed, n, c):
    return np.random.default_rng(seed).standard_normal((n, c)).astype(np.float32)


@pytest.mark.parametrize("seed,batch,grid,frac", [
    (0, 1, (6, 6, 6), 0.2), (1, 2, (5, 7, 3), 0.5), (2, 1, (4, 4, 4), 1.0), (3, 3, (9, 2, 5), 0.1),
])
def test_downsample_matches_dense_max_pool(seed, batch, grid, frac):
    """torch max_pool3d(kernel 2, stride 2, ceil_mode) over a dense grid whose inactive voxels
    are -inf, read at every parent; the parents are exactly the cells with an active voxel."""
    coords = sites(seed, batch, grid, frac)
    x = feats_for(seed, len(coords), 5)
    oc, of, parent, hgrid = rs.downsample2(coords, batch, grid, x)
    dense = torch.full((batch, 5) + tuple(grid), -np.inf, dtype=torch.float64)
    c = torch.from_numpy(coords.astype(np.int64))
    dense[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]] = torch.from_numpy(x.astype(np.float64))
    pooled = torch.nn.functional.max_pool3d(dense, 2, 2, ceil_mode=True)
    assert pooled.shape[2:] == hgrid
    active = torch.isfinite(pooled[:, 0])
    want = torch.nonzero(active).numpy()                      # (b, x, y, z), ascending
    np.testing.assert_array_equal(oc, want)
    o = torch.from_numpy(oc.astype(np.int64))
    np.testing.assert_array_equal(of.astype(np.float64),
                                  pooled[o[:, 0], :, o[:, 1], o[:, 2], o[:, 3]].numpy())


@pytest.mark.parametrize("seed", [4, 5])
def test_downsample_parent_map_brute_force(seed):
    """Every site's parent row holds its coordinates halved; every parent has a site."""
    coords = sites(seed, 2, (7, 5, 6), 0.3)
    oc, _, parent, _ = rs.downsample2(coords, 2, (7, 5, 6))
    halved = coords.copy()
    halved[:, 1:] //= 2
    np.testing.assert_array_equal(oc[parent], halved)
    assert set(parent.tolist()) == set(range(len(oc)))
    # ascending, distinct
    keys = [tuple(r) for r in oc]
    assert keys == sorted(set(keys))


def test_subdivide_then_downsample_is_identity():
    """Eight identical children pool back to the site: coordinates, features and the parent
    map come back exactly (children 8i..8i+7 map to row i of the sorted input)."""
    coords = sites(6, 2, (5, 6, 4), 0.3)
    order = np.lexsort(coords.T[::-1])
    coords = coords[order]
    x = feats_for(6, len(coords), 3)
    sc, sf, sgrid = rs.subdivide2(coords, (5, 6, 4), x)
    assert sgrid == (10, 12, 8)
    assert len({tuple(r) for r in sc}) == 8 * len(coords)
    oc, of, parent, hgrid = rs.downsample2(sc, 2, sgrid, sf)
    assert hgrid == (5, 6, 4)
    np.testing.assert_array_equal(oc, coords)
    np.testing.assert_array_equal(of, x)
    np.testing.assert_array_equal(parent, np.repeat(np.arange(len(coords)), 8))


def test_subdivide_child_order_and_values():
    """Child 4dx + 2dy + dz of site (b, x, y, z) is (b, 2x+dx, 2y+dy, 2z+dz)."""
    c = np.array([[1, 3, 0, 7]], np.int32)
    sc, sf, _ = rs.subdivide2(c, (8, 8, 8), np.array([[2.5, -1.0]], np.float32))
    want = [[1, 6 + dx, 0 + dy, 14 + dz] for dx in (0, 1) for dy in (0, 1) for dz in (0, 1)]
    np.testing.assert_array_equal(sc, want)
    assert (sf == np.array([2.5, -1.0], np.float32)).all()


def test_upsample_of_downsample_dominates():
    """Each site's upsampled value is the maximum over its siblings: >= its own, and equal for
    at least one site of every parent."""
    coords = sites(7, 1, (8, 8, 8), 0.25)
    x = feats_for(7, len(coords), 4)
    oc, of, parent, _ = rs.downsample2(coords, 1, (8, 8, 8), x)
    up = rs.upsample2(of, parent)
    assert (up >= x).all()
    for p in range(len(oc)):
        rows = np.nonzero(parent == p)[0]
        assert (up[rows] == x[rows]).any(0).all()


def test_batches_never_mix():
    one = sites(8, 1, (6, 6, 6), 0.3)
    two = np.concatenate([one, one + np.array([1, 0, 0, 0], np.int32)])
    x = feats_for(8, len(one), 2)
    oc1, of1, p1, _ = rs.downsample2(one, 1, (6, 6, 6), x)
    oc2, of2, p2, _ = rs.downsample2(two, 2, (6, 6, 6), np.concatenate([x, -x]))
    m = len(oc1)
    np.testing.assert_array_equal(oc2[:m], oc1)
    np.testing.assert_array_equal(oc2[m:], oc1 + np.array([1, 0, 0, 0]))
    np.testing.assert_array_equal(of2[:m], of1)
    np.testing.assert_array_equal(p2[len(one):], p1 + m)


@pytest.mark.parametrize("seed,batch,grid,frac", [
    (10, 1, (6, 6, 6), 0.3), (11, 2, (5, 7, 3), 0.6), (12, 1, (4, 4, 4), 1.0),
])
def test_spatial2channel_matches_dense_space_to_depth(seed, batch, grid, frac):
    """A dense grid (zeros off the sites, padded to even sides) reshaped to
    [B, C, X/2, 2, Y/2, 2, Z/2, 2] and permuted to [B, X/2, Y/2, Z/2, C, 2, 2, 2]: its rows at
    the parents are the oracle's rows (channel-major: column c*8 + 4dx + 2dy + dz)."""
    coords = sites(seed, batch, grid, frac)
    x = feats_for(seed, len(coords), 3) + 10.0          # no zero among the site values
    oc, of, parent, hgrid = rs.spatial2channel2(coords, batch, grid, x)
    dc, _, dp, _ = rs.downsample2(coords, batch, grid)
    np.testing.assert_array_equal(oc, dc)
    np.testing.assert_array_equal(parent, dp)
    ex = tuple(2 * h for h in hgrid)
    dense = torch.zeros((batch, 3) + ex, dtype=torch.float64)
    c = torch.from_numpy(coords.astype(np.int64))
    dense[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]] = torch.from_numpy(x.astype(np.float64))
    d = dense.reshape(batch, 3, hgrid[0], 2, hgrid[1], 2, hgrid[2], 2)
    d = d.permute(0, 2, 4, 6, 1, 3, 5, 7).reshape(batch, *hgrid, 24)
    o = torch.from_numpy(oc.astype(np.int64))
    np.testing.assert_array_equal(of.astype(np.float64), d[o[:, 0], o[:, 1], o[:, 2], o[:, 3]].numpy())
    # the parents are exactly the cells with a nonzero value
    want = torch.nonzero((d != 0).any(-1)).numpy()
    np.testing.assert_array_equal(oc, want)


def test_spatial2channel_max_over_children_is_downsample():
    """Max over the 8 child slots of each channel, with absent slots as -inf, is the max pool."""
    coords = sites(13, 2, (7, 5, 6), 0.4)
    x = feats_for(13, len(coords), 4)
    oc, of, parent, _ = rs.spatial2channel2(coords, 2, (7, 5, 6), x)
    present = np.zeros((len(oc), 8), bool)
    k = 4 * (coords[:, 1] % 2) + 2 * (coords[:, 2] % 2) + coords[:, 3] % 2
    present[parent, k] = True
    v = np.where(present[:, None, :], of.reshape(len(oc), 4, 8), -np.inf).max(-1)
    np.testing.assert_array_equal(v, rs.downsample2(coords, 2, (7, 5, 6), x)[1])


def test_downsample_rejects_outside_sites():
    with pytest.raises(ValueError):
        rs.downsample2(np.array([[0, 8, 0, 0]], np.int32), 1, (8, 8, 8))
