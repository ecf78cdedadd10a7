"""Fused conv epilogues (bias + activation + residual, group-norm statistics) and the sparse
group norm: HIP path vs the CPU oracle (oracle.blocks), through the C ABI (needs an MI355X).

Bars: conv outputs as for the plain convolution (the fp32-stored output max|err| <= tau *
RMS(oracle), tau 1e-4 for fp32 / fp16 inputs, 2e-2 for bf16 inputs; a 16-bit store is the
round-to-nearest-even of the fp32 one, bit for bit); group-norm statistics within fp32
summation error; normalised outputs within one rounding to the stored type per element (plus
1e-5 * RMS of fp32 arithmetic); the residual and ConvNeXt-style blocks in bf16 against an
oracle chain that rounds to bf16 wherever the library stores bf16 (after every layer):
max|err| <= 2e-2 * RMS, and per element at most one bf16 step of the value (2^-7 |v|) plus
2e-3 * RMS; in fp32 1e-4 * RMS.  Everything that runs twice must agree bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import blocks
import submanifold_sparse_convolution_coord_amd as ssc
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TAU = {torch.float32: 1e-4, torch.bfloat16: 2e-2, torch.float16: 1e-4}
# group norm outputs, per element: one rounding to the stored type (half an ulp: 2^-8 |v| for
# bf16, 2^-11 |v| for fp16) plus fp32 arithmetic on O(1) values
ROUND = {torch.float32: 0.0, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}
TAU_BLOCK = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
# bf16 chains: where the oracle and the library round the same float32-vs-float64 value to
# different neighbours, the stored values differ by one bf16 step (at most 2^-7 |v|); the
# steps of earlier layers reach the output through the convolutions as small sums.
STEP_BF16 = 2.0 ** -7
TAU_CHAIN = 2e-3


def check_chain(y, ref, dtype):
    err = rel_err(y, ref)
    assert err <= TAU_BLOCK[dtype], err
    if dtype == torch.bfloat16:
        rms = np.sqrt((ref ** 2).mean())
        bad = np.abs(y - ref) > STEP_BF16 * np.abs(ref) + TAU_CHAIN * rms
        assert not bad.any(), (int(bad.sum()), float(np.abs(y - ref)[bad].max() / rms))
    return err


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(y, ref):
    y = np.asarray(y, np.float64)
    rms = np.sqrt((ref ** 2).mean()) if ref.size else 1.0
    return float(np.abs(y - ref).max() / rms) if ref.size else 0.0


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def case(seed, batch, grid, frac, cin, cout, dtype):
    rng = np.random.default_rng(seed)
    n = max(1, int(round(frac * grid[0] * grid[1] * grid[2])))
    coords = workloads.random_sites(rng, batch, grid, n)
    coords = coords[rng.permutation(len(coords))]
    x = torch.from_numpy(rng.standard_normal((len(coords), cin), dtype=np.float32)).to(dtype)
    w = (torch.from_numpy(rng.standard_normal((27, cin, cout), dtype=np.float32)) /
         np.sqrt(27 * cin)).to(dtype)
    b = torch.from_numpy(rng.standard_normal(cout, dtype=np.float32) * 0.5)
    return coords, x, w, b, rng


def index(coords, batch, grid):
    return ssc.SubMIndex(torch.from_numpy(coords).to(DEV), batch, grid)


@pytest.mark.parametrize("cin,cout,dtype,odt,act,with_res", [
    (128, 128, torch.bfloat16, torch.float32, "silu", True),
    (128, 128, torch.bfloat16, torch.bfloat16, "relu", True),
    (64, 128, torch.bfloat16, torch.bfloat16, "silu", False),
    (32, 32, torch.bfloat16, torch.float32, "relu", True),
    (64, 16, torch.bfloat16, torch.bfloat16, "silu", True),
    (32, 64, torch.bfloat16, torch.float32, "none", True),
    (64, 64, torch.float16, torch.float16, "silu", True),
    (16, 24, torch.float32, torch.float32, "silu", True),       # vector-ALU path
    (48, 24, torch.bfloat16, torch.float32, "relu", True),      # vector-ALU path
    (256, 256, torch.bfloat16, torch.bfloat16, "silu", True),   # 2 input chunks, 2 output tiles
    (384, 128, torch.bfloat16, torch.float32, "relu", True),    # 3 input chunks
    (64, 256, torch.float16, torch.float16, "silu", True),      # 2 output tiles
])
def test_conv_epilogue(cin, cout, dtype, odt, act, with_res):
    say(f"[epi] conv {cin}->{cout} {dtype} -> {odt} act={act} res={with_res}")
    coords, x, w, b, rng = case(cin + cout, 1, (14, 13, 12), 0.5, cin, cout, dtype)
    idx = index(coords, 1, (14, 13, 12))
    res = None
    if with_res:
        res = torch.from_numpy(rng.standard_normal((len(coords), cout), dtype=np.float32)).to(odt)
    y = ssc.subm_conv3d(x.to(DEV), w.to(DEV), b.to(DEV), idx.plan, odt, act=act,
                        residual=None if res is None else res.to(DEV))
    # the fp32-stored result against the oracle; a 16-bit store is its RNE, bit for bit
    y32 = ssc.subm_conv3d(x.to(DEV), w.to(DEV), b.to(DEV), idx.plan, torch.float32, act=act,
                          residual=None if res is None else res.float().to(DEV))
    ref = blocks.conv_epilogue(f64(x), f64(w), b.numpy(), oracle.build_map(coords, 1, (14, 13, 12)),
                               act, None if res is None else f64(res))
    err = rel_err(f64(y32), ref)
    say(f"[epi]   max|err|/rms = {err:.3e}")
    assert err <= TAU[dtype]
    assert torch.equal(y.view(torch.uint8), y32.to(odt).view(torch.uint8))
    # the residual may be the output buffer itself
    if with_res:
        out = res.to(DEV).clone()
        ssc.subm_conv3d(x.to(DEV), w.to(DEV), b.to(DEV), idx.plan, odt, out=out, act=act,
                        residual=out)
        assert torch.equal(out.view(torch.uint8), y.view(torch.uint8))


@pytest.mark.parametrize("cin,cout", [(128, 128), (32, 32), (64, 16)])
def test_packed_epilogue_equals_per_call(cin, cout):
    say(f"[epi] packed {cin}->{cout}")
    coords, x, w, b, rng = case(7 + cin, 1, (12, 12, 12), 0.4, cin, cout, torch.bfloat16)
    idx = index(coords, 1, (12, 12, 12))
    res = torch.from_numpy(rng.standard_normal((len(coords), cout), dtype=np.float32)).to(DEV)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    gn1 = ssc.GroupNormPartials(len(coords), 1, 8, DEV)
    gn2 = ssc.GroupNormPartials(len(coords), 1, 8, DEV)
    y1 = ssc.subm_conv3d(xd, wd, bd, idx.plan, act="silu", residual=res, gn=gn1)
    y2 = ssc.subm_conv3d_packed(xd, ssc.pack_weights(wd), bd, idx.plan, act="silu", residual=res,
                                gn=gn2)
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    assert torch.equal(gn1.sums(), gn2.sums())


@pytest.mark.parametrize("n,cin,cout,odt,act,with_res", [
    (4097, 128, 128, torch.float32, "none", False),    # streaming kernel
    (1000, 64, 128, torch.bfloat16, "silu", True),
    (70001, 32, 32, torch.float32, "relu", True),
    (1000, 128, 512, torch.bfloat16, "silu", False),   # tiled GEMM
    (777, 512, 128, torch.float32, "none", True),
    (1, 64, 1024, torch.bfloat16, "none", False),
])
def test_packed_linear_equals_per_call(n, cin, cout, odt, act, with_res):
    say(f"[epi] packed linear n={n} {cin}->{cout} {odt} act={act} res={with_res}")
    rng = np.random.default_rng(n + 3 * cin)
    x = torch.from_numpy(rng.standard_normal((n, cin), dtype=np.float32)).to(torch.bfloat16)
    w = (torch.from_numpy(rng.standard_normal((cin, cout), dtype=np.float32))
         / np.sqrt(cin)).to(torch.bfloat16)
    b = torch.from_numpy(rng.standard_normal(cout, dtype=np.float32))
    res = (torch.from_numpy(rng.standard_normal((n, cout), dtype=np.float32)).to(odt).to(DEV)
           if with_res else None)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    gn1 = ssc.GroupNormPartials(n, 1, 8, DEV)
    gn2 = ssc.GroupNormPartials(n, 1, 8, DEV)
    y1 = ssc.linear(xd, wd, bd, odt, act=act, residual=res, gn=gn1)
    pw = ssc.pack_weights(wd)
    y2 = ssc.linear(xd, pw, bd, odt, act=act, residual=res, gn=gn2)
    assert torch.equal(y1.view(torch.uint8), y2.view(torch.uint8))
    assert torch.equal(gn1.sums(), gn2.sums())
    # the single-tap [1, Cin, Cout] form and the flip flag pack the same bytes
    assert torch.equal(pw.buf, ssc.pack_weights(wd[None]).buf)
    assert torch.equal(pw.buf, ssc.pack_weights(wd, flip=True).buf)
    y3 = ssc.linear(xd, pw, None, odt)
    ref = ssc.linear(xd, wd, None, odt)
    assert torch.equal(y3.view(torch.uint8), ref.view(torch.uint8))


@pytest.mark.parametrize("n,cin,cout,dtype,odt,act", [
    (1000, 64, 128, torch.bfloat16, torch.float32, "silu"),
    (4097, 128, 128, torch.bfloat16, torch.bfloat16, "relu"),
    (333, 32, 64, torch.float16, torch.float16, "silu"),
    (77, 16, 16, torch.float32, torch.float32, "silu"),          # vector-ALU path
    (200000, 128, 32, torch.bfloat16, torch.bfloat16, "none"),   # several tiles per workgroup
    (70001, 32, 16, torch.float16, torch.float32, "relu"),       # 128-row tiles, ragged end
    (1, 64, 64, torch.bfloat16, torch.bfloat16, "silu"),
])
def test_linear_epilogue(n, cin, cout, dtype, odt, act):
    say(f"[epi] linear n={n} {cin}->{cout} {dtype} act={act}")
    rng = np.random.default_rng(n)
    x = torch.from_numpy(rng.standard_normal((n, cin), dtype=np.float32)).to(dtype)
    w = (torch.from_numpy(rng.standard_normal((cin, cout), dtype=np.float32)) / np.sqrt(cin)).to(dtype)
    b = torch.from_numpy(rng.standard_normal(cout, dtype=np.float32))
    res = torch.from_numpy(rng.standard_normal((n, cout), dtype=np.float32)).to(odt)
    y = ssc.linear(x.to(DEV), w.to(DEV), b.to(DEV), odt, act=act, residual=res.to(DEV))
    y32 = ssc.linear(x.to(DEV), w.to(DEV), b.to(DEV), torch.float32, act=act,
                     residual=res.float().to(DEV))
    ref = blocks.linear_epilogue(f64(x), f64(w), b.numpy(), act, f64(res))
    err = rel_err(f64(y32), ref)
    say(f"[epi]   max|err|/rms = {err:.3e}")
    assert err <= TAU[dtype]
    assert torch.equal(y.view(torch.uint8), y32.to(odt).view(torch.uint8))


@pytest.mark.parametrize("dtype,batch,c,groups", [
    (torch.float32, 1, 128, 32), (torch.bfloat16, 3, 64, 32), (torch.float16, 6, 48, 16),
    (torch.bfloat16, 1, 12, 4), (torch.float32, 5, 32, 1), (torch.bfloat16, 64, 32, 32),
])
def test_group_norm(dtype, batch, c, groups):
    say(f"[gn] {dtype} batch={batch} C={c} groups={groups}")
    rng = np.random.default_rng(c + batch)
    coords = workloads.random_sites(rng, batch, (9, 8, 7), 60)
    coords = coords[rng.permutation(len(coords))]
    n = len(coords)
    x = torch.from_numpy((rng.standard_normal((n, c)) * 2.0 + 0.5).astype(np.float32)).to(dtype)
    gamma = torch.from_numpy(1 + 0.2 * rng.standard_normal(c).astype(np.float32))
    beta = torch.from_numpy(0.2 * rng.standard_normal(c).astype(np.float32))
    cd = torch.from_numpy(coords).to(DEV)
    xd = x.to(DEV)
    stats = ssc.gn_finalize(ssc.gn_partials(xd, batch, groups, cd), 1e-5)
    mean, var = blocks.group_stats(f64(x), coords, batch, groups)
    s = stats.cpu().numpy().astype(np.float64)
    assert np.abs(s[..., 0] - mean).max() <= 1e-5 * np.sqrt(var.max())
    np.testing.assert_allclose(s[..., 1], 1 / np.sqrt(var + 1e-5), rtol=1e-5)
    for act in ("none", "silu"):
        y = ssc.gn_apply(xd, stats, gamma.to(DEV), beta.to(DEV), act, cd)
        ref = blocks.group_norm(f64(x), coords, batch, groups, gamma.numpy(), beta.numpy(), 1e-5,
                                act)
        got = f64(y)
        say(f"[gn]   act={act} max|err|/rms = {rel_err(got, ref):.3e}")
        rms = np.sqrt((ref ** 2).mean())
        assert (np.abs(got - ref) <= ROUND[dtype] * np.abs(ref) + 1e-5 * rms).all()
    # in place, and bit-reproducible
    again = ssc.group_norm(xd.clone(), batch, groups, gamma.to(DEV), beta.to(DEV), 1e-5, "silu", cd)
    inplace = xd.clone()
    ssc.group_norm(inplace, batch, groups, gamma.to(DEV), beta.to(DEV), 1e-5, "silu", cd,
                   out=inplace)
    assert torch.equal(again.view(torch.uint8), inplace.view(torch.uint8))
    assert torch.equal(again.view(torch.uint8), y.view(torch.uint8))


def test_group_norm_empty_entry_and_empty_input():
    say("[gn] entry without sites, n = 0")
    coords = np.array([[0, 1, 1, 1], [0, 2, 1, 1], [2, 0, 0, 0]], np.int32)
    x = torch.tensor([[1.0, 3.0], [5.0, 7.0], [-2.0, 2.0]], device=DEV)
    st = ssc.gn_finalize(ssc.gn_partials(x, 3, 1, torch.from_numpy(coords).to(DEV)), 0.0)
    np.testing.assert_allclose(st[:, 0].cpu().numpy(), [[4.0, 1 / np.sqrt(5.0)], [0.0, np.inf],
                                                        [0.0, 0.5]], rtol=1e-6)
    e = torch.zeros((0, 8), device=DEV)
    st = ssc.gn_finalize(ssc.gn_partials(e, 1, 4), 1e-5)
    np.testing.assert_array_equal(st[0, :, 0].cpu().numpy(), 0.0)
    assert ssc.gn_apply(e, st).shape == (0, 8)


@pytest.mark.parametrize("cin,cout,odt", [(128, 128, torch.bfloat16), (32, 32, torch.float32),
                                          (64, 128, torch.float32), (32, 128, torch.bfloat16),
                                          (256, 256, torch.bfloat16)])
def test_conv_group_norm_statistics(cin, cout, odt):
    say(f"[gn] conv-fused statistics {cin}->{cout} {odt}")
    coords, x, w, b, _ = case(100 + cin + cout, 1, (16, 15, 14), 0.45, cin, cout, torch.bfloat16)
    idx = index(coords, 1, (16, 15, 14))
    n = len(coords)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    parts = [ssc.GroupNormPartials(n, 1, 32, DEV) for _ in range(2)]
    y = ssc.subm_conv3d(xd, wd, bd, idx.plan, odt, act="silu", gn=parts[0])
    ssc.subm_conv3d(xd, wd, bd, idx.plan, odt, act="silu", gn=parts[1])
    assert torch.equal(parts[0].sums(), parts[1].sums())            # bit-reproducible
    fused = ssc.gn_finalize(parts[0]).cpu().numpy().astype(np.float64)
    alone = ssc.gn_finalize(ssc.gn_partials(y, 1, 32)).cpu().numpy().astype(np.float64)
    coords_b = np.zeros((n, 4), np.int32)
    mean, var = blocks.group_stats(f64(y), coords_b, 1, 32)
    for s in (fused, alone):
        assert np.abs(s[..., 0] - mean).max() <= 1e-5 * np.sqrt(var.max())
        np.testing.assert_allclose(s[..., 1], 1 / np.sqrt(var + 1e-5), rtol=2e-5)
    # batch > 1: the statistics pass runs after the kernel and equals the standalone one
    coords2, x2, w2, b2, _ = case(200 + cin, 3, (9, 9, 9), 0.4, cin, cout, torch.bfloat16)
    c2 = torch.from_numpy(coords2).to(DEV)
    idx2 = index(coords2, 3, (9, 9, 9))
    p2 = ssc.GroupNormPartials(len(coords2), 3, 32, DEV, c2)
    y2 = ssc.subm_conv3d(x2.to(DEV), w2.to(DEV), b2.to(DEV), idx2.plan, odt, gn=p2)
    assert torch.equal(p2.sums(), ssc.gn_partials(y2, 3, 32, c2).sums())


@pytest.mark.parametrize("cin,cout,odt", [(128, 128, torch.bfloat16), (64, 64, torch.float32),
                                          (32, 32, torch.bfloat16)])
def test_conv_residual_with_group_norm_statistics(cin, cout, odt):
    """The epilogue that closes a residual block and opens the next one: the skip added and
    the next norm's statistics summed from the stored values, in one kernel."""
    say(f"[gn] residual + statistics {cin}->{cout} {odt}")
    coords, x, w, b, rng = case(300 + cin, 1, (14, 13, 15), 0.4, cin, cout, torch.bfloat16)
    n = len(coords)
    res = torch.from_numpy(rng.standard_normal((n, cout), dtype=np.float32)).to(odt)
    idx = index(coords, 1, (14, 13, 15))
    parts = ssc.GroupNormPartials(n, 1, 32, DEV)
    y = ssc.subm_conv3d(x.to(DEV), w.to(DEV), b.to(DEV), idx.plan, odt, residual=res.to(DEV),
                        gn=parts)
    y32 = ssc.subm_conv3d(x.to(DEV), w.to(DEV), b.to(DEV), idx.plan, torch.float32,
                          residual=res.float().to(DEV))
    m = oracle.build_map(coords, 1, (14, 13, 15))
    ref = blocks.conv_epilogue(f64(x), f64(w), b.numpy(), m, "none", f64(res))
    assert rel_err(f64(y32), ref) <= TAU[torch.bfloat16]
    assert torch.equal(y.view(torch.uint8), y32.to(odt).view(torch.uint8))
    fused = ssc.gn_finalize(parts).cpu().numpy().astype(np.float64)
    mean, var = blocks.group_stats(f64(y), np.zeros((n, 4), np.int32), 1, 32)
    assert np.abs(fused[..., 0] - mean).max() <= 1e-5 * np.sqrt(var.max())
    np.testing.assert_allclose(fused[..., 1], 1 / np.sqrt(var + 1e-5), rtol=2e-5)


@pytest.mark.parametrize("cin,cout,groups,n_sites,dtype", [
    (64, 128, 4, 700, torch.bfloat16),     # 32 channels a group: statistics pass after
    (128, 128, 32, 100, torch.bfloat16),   # second tile all padding
    (32, 16, 8, 300, torch.bfloat16),      # several wave rows share columns
    (64, 32, 32, 257, torch.bfloat16),     # one channel a group; ragged last tile
    (128, 64, 16, 900, torch.float16),     # fp16 stores summed in the kernel
    (32, 32, 8, 600, torch.float16),
])
def test_conv_group_norm_statistics_shapes(cin, cout, groups, n_sites, dtype):
    say(f"[gn] conv statistics {cin}->{cout} groups={groups} n={n_sites} {dtype}")
    rng = np.random.default_rng(n_sites)
    coords = workloads.random_sites(rng, 1, (12, 12, 12), n_sites)
    n = len(coords)
    x = torch.from_numpy(rng.standard_normal((n, cin), dtype=np.float32)).to(dtype).to(DEV)
    w = (torch.from_numpy(rng.standard_normal((27, cin, cout), dtype=np.float32)) /
         np.sqrt(27 * cin)).to(dtype).to(DEV)
    b = torch.from_numpy(rng.standard_normal(cout, dtype=np.float32)).to(DEV)
    idx = index(coords, 1, (12, 12, 12))
    parts = ssc.GroupNormPartials(n, 1, groups, DEV)
    y = ssc.subm_conv3d(x, w, b, idx.plan, dtype, act="relu", gn=parts)
    fused = ssc.gn_finalize(parts).cpu().numpy().astype(np.float64)
    mean, var = blocks.group_stats(f64(y), np.zeros((n, 4), np.int32), 1, groups)
    assert np.abs(fused[..., 0] - mean).max() <= 1e-5 * np.sqrt(var.max())
    np.testing.assert_allclose(fused[..., 1], 1 / np.sqrt(var + 1e-5), rtol=2e-5)
    if cout // groups > 16:  # not summed in the kernel: the standalone pass, bit for bit
        assert torch.equal(parts.sums(), ssc.gn_partials(y, 1, groups).sums())


def test_spatial_plan_epilogue_and_statistics():
    """A surface on a 256^3 grid takes the spatial site order and the per-XCD tile
    schedule; the fused epilogue (silu, residual) and the group-norm statistics summed in the
    kernel (slots indexed by tile) hold there as on the interleaved schedule."""
    say("[gn] spatial plan: epilogue and fused statistics")
    rng = np.random.default_rng(77)
    occ, _ = workloads.shell_occupancy(rng, 256, 40.0, 60.0, 1.0)
    coords = workloads.coords_from_occupancy([occ])
    n = len(coords)
    idx = index(coords, 1, (256, 256, 256))
    assert idx.plan.schedule() == 1
    x = torch.from_numpy(rng.standard_normal((n, 64), dtype=np.float32)).bfloat16()
    w = (torch.from_numpy(rng.standard_normal((27, 64, 64), dtype=np.float32)) / 40).bfloat16()
    b = torch.from_numpy(rng.standard_normal(64, dtype=np.float32) * 0.5)
    res = torch.from_numpy(rng.standard_normal((n, 64), dtype=np.float32))
    parts = ssc.GroupNormPartials(n, 1, 32, DEV)
    y = ssc.subm_conv3d(x.to(DEV), w.to(DEV), b.to(DEV), idx.plan, torch.float32, act="silu",
                        residual=res.to(DEV), gn=parts)
    m = oracle.build_map(coords, 1, (256, 256, 256))
    ref = blocks.conv_epilogue(f64(x), f64(w), b.numpy(), m, "silu", f64(res))
    err = rel_err(f64(y), ref)
    say(f"[gn]   n={n} max|err|/rms = {err:.3e}")
    assert err <= TAU[torch.bfloat16]
    fused = ssc.gn_finalize(parts).cpu().numpy().astype(np.float64)
    mean, var = blocks.group_stats(f64(y), np.zeros((n, 4), np.int32), 1, 32)
    assert np.abs(fused[..., 0] - mean).max() <= 1e-5 * np.sqrt(var.max())
    np.testing.assert_allclose(fused[..., 1], 1 / np.sqrt(var + 1e-5), rtol=2e-5)


def res_block_gpu(x, coords_d, batch, plan, p, groups, eps, packed=False):
    """The pre-norm residual block through the library: statistics + apply for the first
    norm, conv1 summing the second norm's statistics in its epilogue, apply, conv2 adding
    the skip in its epilogue."""
    n = x.shape[0]
    cd = coords_d if batch > 1 else None
    h = ssc.group_norm(x, batch, groups, p["g1"], p["be1"], eps, "silu", cd)
    parts = ssc.GroupNormPartials(n, batch, groups, x.device, cd)
    h = ssc.subm_conv3d(h, p["w1"], p["b1"], plan, x.dtype, gn=parts)
    h = ssc.gn_apply(h, ssc.gn_finalize(parts, eps), p["g2"], p["be2"], "silu", cd, out=h)
    return ssc.subm_conv3d(h, p["w2"], p["b2"], plan, x.dtype, residual=x)


@pytest.mark.parametrize("dtype,batch,c,groups", [(torch.bfloat16, 1, 128, 32),
                                                  (torch.bfloat16, 2, 64, 32),
                                                  (torch.float32, 1, 32, 8)])
def test_res_block(dtype, batch, c, groups):
    say(f"[block] {dtype} batch={batch} C={c}")
    rng = np.random.default_rng(c + batch)
    grid = (20, 18, 16)
    coords = workloads.random_sites(rng, batch, grid, 1500)
    coords = coords[rng.permutation(len(coords))]
    n = len(coords)
    x = torch.from_numpy(rng.standard_normal((n, c), dtype=np.float32)).to(dtype)
    p = {"w1": torch.from_numpy(rng.standard_normal((27, c, c), dtype=np.float32) / np.sqrt(27 * c)).to(dtype),
         "w2": torch.from_numpy(rng.standard_normal((27, c, c), dtype=np.float32) / np.sqrt(27 * c)).to(dtype),
         "b1": torch.from_numpy(0.1 * rng.standard_normal(c).astype(np.float32)),
         "b2": torch.from_numpy(0.1 * rng.standard_normal(c).astype(np.float32)),
         "g1": torch.from_numpy(1 + 0.1 * rng.standard_normal(c).astype(np.float32)),
         "be1": torch.from_numpy(0.1 * rng.standard_normal(c).astype(np.float32)),
         "g2": torch.from_numpy(1 + 0.1 * rng.standard_normal(c).astype(np.float32)),
         "be2": torch.from_numpy(0.1 * rng.standard_normal(c).astype(np.float32))}
    cd = torch.from_numpy(coords).to(DEV)
    idx = ssc.SubMIndex(cd, batch, grid)
    pd = {k: v.to(DEV) for k, v in p.items()}
    y = res_block_gpu(x.to(DEV), cd, batch, idx.plan, pd, groups, 1e-5)
    y_again = res_block_gpu(x.to(DEV), cd, batch, idx.plan, pd, groups, 1e-5)
    assert torch.equal(y.view(torch.uint8), y_again.view(torch.uint8))
    ref = blocks.res_block(f64(x), coords, batch, oracle.build_map(coords, batch, grid),
                           {k: f64(v) for k, v in p.items()}, groups, 1e-5,
                           store=blocks.round_bf16 if dtype == torch.bfloat16 else None)
    err = check_chain(f64(y), ref, dtype)
    say(f"[block]   max|err|/rms = {err:.3e}")


@pytest.mark.parametrize("n,cin,cout,dtype,odt,act", [
    (1000, 128, 512, torch.bfloat16, torch.float32, "silu"),    # 8 column tiles per row tile
    (777, 512, 128, torch.bfloat16, torch.bfloat16, "none"),
    (333, 64, 256, torch.float16, torch.float16, "relu"),
    (513, 256, 64, torch.bfloat16, torch.float32, "silu"),
    (129, 192, 192, torch.bfloat16, torch.bfloat16, "none"),
    (1, 128, 512, torch.bfloat16, torch.float32, "none"),
    (4097, 64, 1024, torch.bfloat16, torch.bfloat16, "silu"),   # 16 column tiles
    (255, 128, 192, torch.float16, torch.float32, "none"),      # 3 column tiles, 2 row tiles
])
def test_wide_linear(n, cin, cout, dtype, odt, act):
    say(f"[gemm] n={n} {cin}->{cout} {dtype} -> {odt} act={act}")
    rng = np.random.default_rng(n + cin)
    x = torch.from_numpy(rng.standard_normal((n, cin), dtype=np.float32)).to(dtype)
    w = (torch.from_numpy(rng.standard_normal((cin, cout), dtype=np.float32)) / np.sqrt(cin)).to(dtype)
    b = torch.from_numpy(rng.standard_normal(cout, dtype=np.float32))
    res = torch.from_numpy(rng.standard_normal((n, cout), dtype=np.float32)).to(odt)
    y = ssc.linear(x.to(DEV), w.to(DEV), b.to(DEV), odt, act=act, residual=res.to(DEV))
    y32 = ssc.linear(x.to(DEV), w.to(DEV), b.to(DEV), torch.float32, act=act,
                     residual=res.float().to(DEV))
    ref = blocks.linear_epilogue(f64(x), f64(w), b.numpy(), act, f64(res))
    err = rel_err(f64(y32), ref)
    say(f"[gemm]   max|err|/rms = {err:.3e}")
    assert err <= TAU[dtype]
    assert torch.equal(y.view(torch.uint8), y32.to(odt).view(torch.uint8))


@pytest.mark.parametrize("dtype,c,n", [(torch.bfloat16, 128, 3000), (torch.float32, 32, 1001),
                                       (torch.float16, 512, 257), (torch.bfloat16, 48, 300),
                                       (torch.float32, 7, 65), (torch.bfloat16, 8, 1)])
def test_layer_norm(dtype, c, n):
    say(f"[ln] {dtype} C={c} n={n}")
    rng = np.random.default_rng(c + n)
    x = torch.from_numpy((rng.standard_normal((n, c)) * 3.0 + 1.5).astype(np.float32)).to(dtype)
    g = torch.from_numpy(1 + 0.2 * rng.standard_normal(c).astype(np.float32))
    be = torch.from_numpy(0.2 * rng.standard_normal(c).astype(np.float32))
    for act in ("none", "silu"):
        y = ssc.layer_norm(x.to(DEV), g.to(DEV), be.to(DEV), 1e-6, act)
        ref = blocks.layer_norm(f64(x), g.numpy(), be.numpy(), 1e-6, act)
        got = f64(y)
        say(f"[ln]   act={act} max|err|/rms = {rel_err(got, ref):.3e}")
        rms = np.sqrt((ref ** 2).mean())
        assert (np.abs(got - ref) <= ROUND[dtype] * np.abs(ref) + 1e-5 * rms).all()
    inplace = x.to(DEV).clone()
    ssc.layer_norm(inplace, g.to(DEV), be.to(DEV), 1e-6, "silu", out=inplace)
    assert torch.equal(inplace.view(torch.uint8), y.view(torch.uint8))


@pytest.mark.parametrize("c", [128, 32, 64])
def test_convnext_block(c):
    """conv -> layer norm -> linear C->4C + silu -> linear 4C->C + skip, bf16 through the
    library (the k=1 layers on the streaming kernel or the tiled GEMM by width)."""
    say(f"[convnext] C={c}")
    rng = np.random.default_rng(c)
    grid = (20, 18, 16)
    coords = workloads.random_sites(rng, 1, grid, 1500)
    n = len(coords)
    bf = torch.bfloat16
    x = torch.from_numpy(rng.standard_normal((n, c), dtype=np.float32)).to(bf)
    p = {"w": torch.from_numpy(rng.standard_normal((27, c, c), dtype=np.float32) / np.sqrt(27 * c)).to(bf),
         "b": torch.from_numpy(0.1 * rng.standard_normal(c).astype(np.float32)),
         "ln_g": torch.from_numpy(1 + 0.1 * rng.standard_normal(c).astype(np.float32)),
         "ln_b": torch.from_numpy(0.1 * rng.standard_normal(c).astype(np.float32)),
         "w1": torch.from_numpy(rng.standard_normal((c, 4 * c), dtype=np.float32) / np.sqrt(c)).to(bf),
         "b1": torch.from_numpy(0.1 * rng.standard_normal(4 * c).astype(np.float32)),
         "w2": torch.from_numpy(rng.standard_normal((4 * c, c), dtype=np.float32) / np.sqrt(4 * c)).to(bf),
         "b2": torch.from_numpy(0.1 * rng.standard_normal(c).astype(np.float32))}
    pd = {k: v.to(DEV) for k, v in p.items()}
    idx = ssc.SubMIndex(torch.from_numpy(coords).to(DEV), 1, grid)
    xd = x.to(DEV)
    h = ssc.subm_conv3d(xd, pd["w"], pd["b"], idx.plan, bf)
    h = ssc.layer_norm(h, pd["ln_g"], pd["ln_b"], 1e-6, out=h)
    h = ssc.linear(h, pd["w1"], pd["b1"], bf, act="silu")
    y = ssc.linear(h, pd["w2"], pd["b2"], bf, residual=xd)
    ref = blocks.convnext_block(f64(x), oracle.build_map(coords, 1, grid),
                                {k: f64(v) for k, v in p.items()}, 1e-6, store=blocks.round_bf16)
    err = check_chain(f64(y), ref, bf)
    say(f"[convnext]   max|err|/rms = {err:.3e}")


@pytest.mark.parametrize("n,cin,cout,dtype", [(300, 1024, 1024, torch.bfloat16),
                                              (50, 1024, 1024, torch.float32),
                                              (130, 1024, 64, torch.float16)])
def test_maximum_channels_linear(n, cin, cout, dtype):
    """1024-channel k=1 layers: the tiled GEMM (16-bit) and the vector-ALU kernel (fp32)."""
    say(f"[max] k1 n={n} {cin}->{cout} {dtype}")
    rng = np.random.default_rng(cin + n)
    x = torch.from_numpy(rng.standard_normal((n, cin), dtype=np.float32)).to(dtype)
    w = (torch.from_numpy(rng.standard_normal((cin, cout), dtype=np.float32)) / np.sqrt(cin)).to(dtype)
    b = torch.from_numpy(rng.standard_normal(cout, dtype=np.float32))
    y = ssc.linear(x.to(DEV), w.to(DEV), b.to(DEV), torch.float32, act="relu")
    ref = blocks.linear_epilogue(f64(x), f64(w), b.numpy(), "relu")
    assert rel_err(f64(y), ref) <= TAU[dtype]


@pytest.mark.parametrize("c,dtype", [(1024, torch.bfloat16), (4096, torch.float32)])
def test_wide_layer_norm_and_group_norm(c, dtype):
    """Rows wider than 64 words take the one-thread-per-row layer norm; the group norm with
    1024 channels keeps its word kernels."""
    say(f"[max] norms C={c} {dtype}")
    rng = np.random.default_rng(c)
    n = 97
    x = torch.from_numpy((rng.standard_normal((n, c)) + 0.3).astype(np.float32)).to(dtype)
    ref = blocks.layer_norm(f64(x), eps=1e-6)
    got = f64(ssc.layer_norm(x.to(DEV), eps=1e-6))
    assert (np.abs(got - ref) <= ROUND[dtype] * np.abs(ref) + 1e-5 * np.sqrt((ref ** 2).mean())).all()
    if c <= 1024:
        coords = np.zeros((n, 4), np.int32)
        gref = blocks.group_norm(f64(x), coords, 1, 32, eps=1e-5)
        ggot = f64(ssc.group_norm(x.to(DEV), 1, 32, eps=1e-5))
        assert (np.abs(ggot - gref) <= ROUND[dtype] * np.abs(gref) + 1e-5 * np.sqrt((gref ** 2).mean())).all()
