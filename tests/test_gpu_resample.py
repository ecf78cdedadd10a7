"""Downsample (max) / upsample / spatial2channel / subdivide: HIP path vs the CPU oracle,
through the C ABI (needs an MI355X).  All are exact (a maximum returns one of its inputs, the
rest are copies and integer arithmetic), so every comparison is bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import resample as rs
import submanifold_sparse_convolution_coord_amd as ssc
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def as_np(t):
    """bf16 widens to float32 exactly; fp16 and float32 stay as they are."""
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def check_s2c(coords, batch, grid, x):
    gc, gf, gp, ggrid = ssc.spatial2channel2(torch.from_numpy(coords).to(DEV), batch, grid,
                                             x.to(DEV))
    oc, of, op, ogrid = rs.spatial2channel2(coords, batch, grid, as_np(x))
    assert ggrid == ogrid
    assert gf.dtype == x.dtype and gf.shape == (len(oc), 8 * x.shape[1])
    np.testing.assert_array_equal(gc.cpu().numpy(), oc)
    np.testing.assert_array_equal(gp.cpu().numpy(), op)
    np.testing.assert_array_equal(as_np(gf), of)


def check_down(coords, batch, grid, x):
    gc, gf, gp, ggrid = ssc.downsample2(torch.from_numpy(coords).to(DEV), batch, grid,
                                        None if x is None else x.to(DEV))
    oc, of, op, ogrid = rs.downsample2(coords, batch, grid, None if x is None else as_np(x))
    assert ggrid == ogrid
    np.testing.assert_array_equal(gc.cpu().numpy(), oc)
    np.testing.assert_array_equal(gp.cpu().numpy(), op)
    if x is not None:
        np.testing.assert_array_equal(as_np(gf), of)
    return gc, gf, gp


@pytest.mark.parametrize("name", ["tiny", "iid128", "batch4", "shell512"])
def test_downsample_workloads(name):
    say(f"[down] {name}")
    w = workloads.make(name)
    gc, gf, gp = check_down(w.coords, w.batch, w.grid, w.feats)
    # the new coordinate set indexes cold like any other
    hgrid = tuple((g + 1) // 2 for g in w.grid)
    nbr = ssc.build_index(gc.contiguous(), w.batch, hgrid)
    np.testing.assert_array_equal(nbr.cpu().numpy(),
                                  oracle.build_map(gc.cpu().numpy(), w.batch, hgrid))


@pytest.mark.parametrize("name", ["tiny", "batch4"])
def test_subdivide_and_upsample_workloads(name):
    say(f"[subdivide/upsample] {name}")
    w = workloads.make(name)
    c = torch.from_numpy(w.coords).to(DEV)
    sc, sf, sgrid = ssc.subdivide2(c, w.grid, w.feats.to(DEV))
    oc, of, ogrid = rs.subdivide2(w.coords, w.grid, as_np(w.feats))
    assert sgrid == ogrid
    np.testing.assert_array_equal(sc.cpu().numpy(), oc)
    np.testing.assert_array_equal(as_np(sf), of)
    # upsample through the downsample of the subdivided set: every child gets back its site
    dc, df, dp, _ = ssc.downsample2(sc, w.batch, sgrid, sf)
    up = ssc.upsample2(df, dp)
    np.testing.assert_array_equal(as_np(up), of)
    # and the upsample itself matches the oracle on a pooled set
    gc, gf, gp = check_down(w.coords, w.batch, w.grid, w.feats)
    np.testing.assert_array_equal(as_np(ssc.upsample2(gf, gp)),
                                  rs.upsample2(as_np(gf), gp.cpu().numpy()))


@pytest.mark.parametrize("dtype,c", [(torch.float32, 4), (torch.bfloat16, 8), (torch.float32, 3),
                                     (torch.bfloat16, 2)])
def test_channels_and_dtypes(dtype, c):
    say(f"[down] channels {c} {dtype}")
    rng = np.random.default_rng(c)
    coords = workloads.random_sites(rng, 2, (9, 7, 5), 120)
    x = torch.from_numpy(rng.standard_normal((len(coords), c), dtype=np.float32)).to(dtype)
    gc, gf, gp = check_down(coords, 2, (9, 7, 5), x)
    np.testing.assert_array_equal(as_np(ssc.upsample2(gf, gp)),
                                  rs.upsample2(as_np(gf), gp.cpu().numpy()))
    sc, sf, _ = ssc.subdivide2(torch.from_numpy(coords).to(DEV), (9, 7, 5), x.to(DEV))
    oc, of, _ = rs.subdivide2(coords, (9, 7, 5), as_np(x))
    np.testing.assert_array_equal(sc.cpu().numpy(), oc)
    np.testing.assert_array_equal(as_np(sf), of)


@pytest.mark.parametrize("name", ["tiny", "iid128", "batch4"])
def test_spatial2channel_workloads(name):
    say(f"[s2c] {name}")
    w = workloads.make(name)
    check_s2c(w.coords, w.batch, w.grid, w.feats)


# rows of 16 bytes multiples take the word kernel, the rest the element kernel
@pytest.mark.parametrize("dtype,c", [(torch.float32, 4), (torch.bfloat16, 8), (torch.float16, 8),
                                     (torch.float32, 12), (torch.bfloat16, 24),
                                     (torch.float32, 3), (torch.float16, 1), (torch.bfloat16, 2)])
def test_spatial2channel_channels_and_dtypes(dtype, c):
    say(f"[s2c] channels {c} {dtype}")
    rng = np.random.default_rng(20 + c)
    coords = workloads.random_sites(rng, 2, (9, 7, 5), 150)
    x = torch.from_numpy(rng.standard_normal((len(coords), c), dtype=np.float32)).to(dtype)
    check_s2c(coords, 2, (9, 7, 5), x)


def test_spatial2channel_full_cells_and_extremes():
    say("[s2c] full 2x2x2 cells, 65535^3 grid")
    full = np.array([[0, x, y, z] for x in range(4) for y in range(2) for z in range(2)], np.int32)
    check_s2c(full, 1, (4, 2, 2), torch.arange(32, dtype=torch.float32).reshape(16, 2) + 1)
    check_s2c(full, 1, (4, 2, 2), torch.arange(64, dtype=torch.float32).reshape(16, 4) + 1)
    check_s2c(full[::-1].copy(), 1, (4, 2, 2),
              (torch.arange(128, dtype=torch.float32).reshape(16, 8) + 1).bfloat16())
    G = 65535
    ext = np.array([[G - 1, G - 1, G - 1, G - 1], [G - 1, G - 2, G - 1, G - 2], [0, 0, 0, 0]],
                   np.int32)
    check_s2c(ext, G, (G, G, G), torch.arange(6, dtype=torch.bfloat16).reshape(3, 2))


def test_spatial2channel_empty_and_bad():
    say("[s2c] empty, bad coordinate")
    c = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    gc, gf, gp, _ = ssc.spatial2channel2(c, 1, (4, 4, 4), torch.zeros((0, 4), device=DEV))
    assert gc.shape == (0, 4) and gf.shape == (0, 32) and gp.shape == (0,)
    bad = torch.tensor([[0, 1, 1, 1], [0, 0, 9, 0]], dtype=torch.int32, device=DEV)
    with pytest.raises(ssc.SscError) as e:
        ssc.spatial2channel2(bad, 1, (8, 8, 8), torch.ones((2, 4), device=DEV))
    assert e.value.status == ssc.SSC_ERR_COORD_RANGE


@pytest.mark.parametrize("c", [8, 6, 5])
def test_downsample_fp16(c):
    say(f"[down] fp16 channels {c}")
    rng = np.random.default_rng(40 + c)
    coords = workloads.random_sites(rng, 2, (9, 7, 5), 150)
    x = torch.from_numpy(rng.standard_normal((len(coords), c), dtype=np.float32)).half()
    gc, gf, gp = check_down(coords, 2, (9, 7, 5), x)
    assert gf.dtype == torch.float16
    if 2 * c % 4:  # the upsample moves rows in words of 4 bytes at least
        with pytest.raises(ssc.SscError):
            ssc.upsample2(gf, gp)
        return
    np.testing.assert_array_equal(as_np(ssc.upsample2(gf, gp)),
                                  rs.upsample2(as_np(gf), gp.cpu().numpy()))


def test_coordinates_only_and_single_site():
    say("[down] coords only, single site")
    check_down(np.array([[0, 5, 6, 7]], np.int32), 1, (8, 8, 8), None)
    rng = np.random.default_rng(3)
    check_down(workloads.random_sites(rng, 3, (11, 3, 6), 60), 3, (11, 3, 6), None)


def test_extreme_coordinates():
    say("[down] 65535^3 grid, last batch entry")
    G, B = 65535, 65535
    coords = np.array([[B - 1, G - 1, G - 1, G - 1], [B - 1, G - 2, G - 1, G - 2], [0, 0, 0, 0],
                       [B - 1, 0, G - 1, 1], [0, 1, 1, 1]], np.int32)
    x = torch.from_numpy(np.arange(10, dtype=np.float32).reshape(5, 2))
    check_down(coords, B, (G, G, G), x)


def test_empty():
    say("[down] empty")
    c = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    gc, gf, gp, _ = ssc.downsample2(c, 1, (4, 4, 4), torch.zeros((0, 8), device=DEV))
    assert gc.shape == (0, 4) and gf.shape == (0, 8) and gp.shape == (0,)
    sc, sf, _ = ssc.subdivide2(c, (4, 4, 4), torch.zeros((0, 8), device=DEV))
    assert sc.shape == (0, 4) and sf.shape == (0, 8)


def test_downsample_reports_outside_sites():
    say("[down] bad coordinate")
    c = torch.tensor([[0, 1, 1, 1], [0, 8, 0, 0]], dtype=torch.int32, device=DEV)
    with pytest.raises(ssc.SscError) as e:
        ssc.downsample2(c, 1, (8, 8, 8))
    assert e.value.status == ssc.SSC_ERR_COORD_RANGE
