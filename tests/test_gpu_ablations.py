"""The pages' own convolution designs as rebuilt for comparison (dense 27-tap GEMM, per-offset
gather-GEMM-scatter, the compacted kernel without tap compaction) against the CPU oracle
(needs an MI355X).

Bars: the kernel without compaction equals the compacted kernel bit for bit (the extra
products are exact zeros); the two library-GEMM designs, whose GEMMs round their products to
bf16, within the bf16 bar of the convolution, 2e-2 * RMS.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import submanifold_sparse_convolution_coord_amd as ssc
from submanifold_sparse_convolution_coord_amd import ablations
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(y, ref):
    y = np.asarray(y, np.float64)
    return float(np.abs(y - ref).max() / np.sqrt((ref ** 2).mean()))


@pytest.mark.parametrize("cin,cout,n_sites", [(128, 128, 2500), (64, 32, 1000), (32, 64, 700)])
def test_designs_match_oracle(cin, cout, n_sites):
    say(f"[ablation] {cin}->{cout} n={n_sites}")
    rng = np.random.default_rng(cin + cout)
    grid = (16, 16, 16)
    coords = workloads.random_sites(rng, 1, grid, n_sites)
    coords = coords[rng.permutation(len(coords))]
    n = len(coords)
    x = torch.from_numpy(rng.standard_normal((n, cin), dtype=np.float32)).bfloat16()
    w = (torch.from_numpy(rng.standard_normal((27, cin, cout), dtype=np.float32)) /
         np.sqrt(27 * cin)).bfloat16()
    b = torch.from_numpy(rng.standard_normal(cout, dtype=np.float32))
    idx = ssc.SubMIndex(torch.from_numpy(coords).to(DEV), 1, grid)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    ref = oracle.conv(x.float().numpy(), w.float().numpy(), b.numpy(),
                      oracle.build_map(coords, 1, grid))
    y = ssc.subm_conv3d(xd, wd, bd, idx.plan)
    y_dense_taps = ssc.subm_conv3d(xd, wd, bd, ablations.dense_taps_plan(idx.plan))
    assert torch.equal(y.view(torch.int32), y_dense_taps.view(torch.int32))
    y_gemm = ablations.DenseGemm(idx.nbr, wd)(xd, bd)
    y_off = ablations.PerOffset(idx.nbr, wd)(xd, bd)
    for name, got in (("dense gemm", y_gemm), ("per offset", y_off)):
        err = rel_err(got.float().cpu().numpy(), ref)
        say(f"[ablation]   {name}: max|err|/rms = {err:.3e}")
        assert err <= 2e-2, name


def test_per_offset_graph_replays():
    """The per-offset loop captured in a HIP graph: every replay (with eager work between)
    equals the eager result bit for bit."""
    say("[ablation] per-offset graph replay")
    rng = np.random.default_rng(9)
    grid = (12, 12, 12)
    coords = workloads.random_sites(rng, 1, grid, 800)
    x = torch.from_numpy(rng.standard_normal((len(coords), 64), dtype=np.float32)).bfloat16().to(DEV)
    w = (torch.from_numpy(rng.standard_normal((27, 64, 64), dtype=np.float32)) / 40).bfloat16().to(DEV)
    b = torch.from_numpy(rng.standard_normal(64, dtype=np.float32)).to(DEV)
    idx = ssc.SubMIndex(torch.from_numpy(coords).to(DEV), 1, grid)
    po = ablations.PerOffset(idx.nbr, w)
    out = torch.empty((len(coords), 64), dtype=torch.float32, device=DEV)
    eager = po(x, b, out=out).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        po(x, b, out=out)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        out.fill_(1.0)
        _ = (x.float() * 2).sum().item()
