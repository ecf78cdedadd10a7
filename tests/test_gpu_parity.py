"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Bars: neighbour maps bit-exact; conv outputs max|err| <= tau * RMS(oracle) with tau = 1e-4
for fp32 inputs and 2e-2 for bf16 inputs, taken on the fp32-stored output; the bf16-stored
output must equal the round-to-nearest-even bf16 of the fp32-stored output bit for bit.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import oracle
import submanifold_sparse_convolution_coord_amd as ssc
import workloads

pytestmark = pytest.mark.gpu

# fp16 inputs: products of two fp16 values are exact in fp32 and accumulation is fp32, as for
# fp32 inputs, so the fp32-input bound applies (the 2e-2 bf16 bound is for bf16 inputs).
TAU = {"f32": 1e-4, "bf16": 2e-2, "f16": 1e-4}
# Second bar on every fp32-stored convolution: 16-bit products are exact in fp32 and the sum
# has at most 27 * Cin terms, so an fp32 accumulator stays within ~1e-6 of RMS (measured
# 2e-7 to 8e-7); 1e-5 leaves a margin of 10x and still fails an accumulator that rounds to
# 16 bits per tap (~4e-3 of RMS).
TAU_ACC = 1e-5
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(y, ref):
    y = np.asarray(y, np.float64)
    rms = np.sqrt((ref ** 2).mean()) if ref.size else 1.0
    return float(np.abs(y - ref).max() / rms) if ref.size else 0.0


def rne_bf16(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.bfloat16)


@functools.lru_cache(maxsize=2)
def workload_case(name, shuffle=False):
    w = workloads.make(name, shuffle=shuffle)
    m = oracle.build_map(w.coords, w.batch, w.grid)
    return w, m


def run_gpu(coords, batch, grid):
    c = torch.from_numpy(coords).to(DEV)
    idx = ssc.SubMIndex(c, batch, grid)
    return idx


@pytest.mark.parametrize("name,shuffle", [
    ("tiny", False), ("tiny", True), ("iid128", False), ("iid128", True), ("shell256", False),
    ("shell256", True), ("batch4", False), ("shell512", False),
])
def test_workload_parity(name, shuffle):
    say(f"[parity] workload={name} shuffle={shuffle}")
    w, m = workload_case(name, shuffle)
    idx = run_gpu(w.coords, w.batch, w.grid)
    nbr = idx.nbr.cpu().numpy()
    assert np.array_equal(nbr, m), f"{name}: neighbour map differs from the oracle"

    layer = w.layers[0]
    x = w.feats.to(DEV)
    wt = layer.weight.to(DEV)
    b = layer.bias.to(DEV)
    y32 = idx.conv(x, wt, b, out_dtype=torch.float32)
    ybf = idx.conv(x, wt, b, out_dtype=torch.bfloat16)
    if x.dtype == torch.bfloat16:
        # the launch configuration the benchmark times: weights packed once, then the layer
        yp = ssc.subm_conv3d_packed(x, ssc.pack_weights(wt), b, idx.plan, torch.float32)
        assert torch.equal(yp, y32)
    torch.cuda.synchronize()
    ref = oracle.conv(w.feats.float().numpy(), layer.weight.float().numpy(),
                      layer.bias.numpy(), m)
    err = rel_err(y32.cpu().numpy(), ref)
    say(f"[parity] {name} n={w.n} k3 max|err|/rms = {err:.3e}")
    assert err <= TAU[w.dtype]
    assert err <= TAU_ACC
    assert torch.equal(ybf.cpu().view(torch.int16), rne_bf16(y32.cpu()).view(torch.int16))

    if len(w.layers) > 1:  # batch4: k=1 128->128 on the bf16 k=3 output
        l2 = w.layers[1]
        x2 = ybf
        y2 = ssc.linear(x2, l2.weight.to(DEV), l2.bias.to(DEV))
        torch.cuda.synchronize()
        ref2 = oracle.linear(x2.float().cpu().numpy(), l2.weight.float().numpy(), l2.bias.numpy())
        err2 = rel_err(y2.cpu().numpy(), ref2)
        say(f"[parity] {name} k1 max|err|/rms = {err2:.3e}")
        assert err2 <= TAU[w.dtype]
        # chained: the oracle rounds its own k=3 result to bf16 and applies the k=1 layer
        ref_chain = oracle.linear(rne_bf16(torch.from_numpy(ref).float()).float().numpy(),
                                  l2.weight.float().numpy(), l2.bias.numpy())
        assert rel_err(y2.cpu().numpy(), ref_chain) <= TAU[w.dtype]
        # the launch configuration the benchmark times for the two layers: one fused kernel,
        # whose bf16 intermediate is the k=3 layer's bf16 store (so ref2 is its exact input)
        w2 = l2.weight.to(DEV)
        yp2 = ssc.subm_conv3d_pair(x, ssc.pack_weights(wt), b, idx.plan,
                                   ssc.pack_weights(w2, pair=True), l2.bias.to(DEV),
                                   torch.float32)
        torch.cuda.synchronize()
        errp = rel_err(yp2.cpu().numpy(), ref2)
        say(f"[parity] {name} fused pair max|err|/rms = {errp:.3e}")
        assert errp <= TAU_ACC
        assert rel_err(yp2.cpu().numpy(), ref_chain) <= TAU[w.dtype]


def small_case(seed, batch, grid, frac, cin, cout, dtype=torch.bfloat16, bias=True):
    rng = np.random.default_rng(seed)
    n = max(1, int(round(frac * grid[0] * grid[1] * grid[2])))
    coords = workloads.random_sites(rng, batch, grid, n)
    coords = coords[rng.permutation(len(coords))]
    x = torch.from_numpy(rng.standard_normal((len(coords), cin), dtype=np.float32)).to(dtype)
    w = (torch.from_numpy(rng.standard_normal((27, cin, cout), dtype=np.float32)) /
         np.sqrt(27 * cin)).to(dtype)
    b = torch.from_numpy(rng.standard_normal(cout, dtype=np.float32)) if bias else None
    return coords, x, w, b


def check_conv(coords, batch, grid, x, w, b, tau):
    m = oracle.build_map(coords, batch, grid)
    idx = run_gpu(coords, batch, grid)
    assert np.array_equal(idx.nbr.cpu().numpy(), m)
    y = idx.conv(x.to(DEV), w.to(DEV), None if b is None else b.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.conv(x.float().numpy(), w.float().numpy(), None if b is None else b.numpy(), m)
    err = rel_err(y.cpu().numpy(), ref)
    assert err <= tau, err
    assert err <= TAU_ACC, err
    return idx, y


@pytest.mark.parametrize("cin,cout,dtype", [
    (256, 128, torch.bfloat16), (256, 256, torch.bfloat16), (512, 64, torch.bfloat16),
    (128, 256, torch.bfloat16), (64, 384, torch.float16), (384, 32, torch.float16),
    (1024, 16, torch.bfloat16), (32, 1024, torch.bfloat16)])
def test_wide_layers(cin, cout, dtype):
    """Layers wider than the 128-channel matrix-core kernel: cin in chunks of 128 summed in the
    stage loop, cout in tiles of 128 as separate workgroups.  fp32 store against the oracle
    (both bars); the 16-bit store is its RNE bit for bit; packed weights (bf16) give the same
    bits as the per-call path, and the flipped packing matches the oracle's other
    orientation."""
    say(f"[parity] wide {cin}->{cout} {dtype}")
    tau = TAU["bf16" if dtype == torch.bfloat16 else "f16"]
    coords, x, w, b = small_case(cin + 7 * cout, 1, (13, 12, 11), 0.35, cin, cout, dtype)
    idx, y = check_conv(coords, 1, (13, 12, 11), x, w, b, tau)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    y16 = idx.conv(xd, wd, bd, out_dtype=dtype)
    assert torch.equal(y16.cpu().view(torch.int16), y.cpu().to(dtype).view(torch.int16))
    if dtype == torch.bfloat16:
        yp = ssc.subm_conv3d_packed(xd, ssc.pack_weights(wd), bd, idx.plan, torch.float32)
        assert torch.equal(yp.view(torch.int32), y.view(torch.int32))
        yf = ssc.subm_conv3d_packed(xd, ssc.pack_weights(wd, flip=True), bd, idx.plan,
                                    torch.float32)
        m = oracle.build_map(coords, 1, (13, 12, 11))
        ref = oracle.conv(x.float().numpy(), w.float().numpy(), b.numpy(), m, flip=True)
        assert rel_err(yf.cpu().numpy(), ref) <= TAU_ACC


@pytest.mark.parametrize("cin,cmid,cout,odt,frac", [
    (64, 128, 128, torch.float32, 0.3), (64, 128, 128, torch.bfloat16, 0.3),
    (128, 128, 64, torch.float32, 0.5), (128, 128, 128, torch.bfloat16, 0.05),
    (32, 64, 64, torch.float32, 0.3), (64, 64, 64, torch.bfloat16, 0.3),
    (128, 64, 64, torch.float32, 0.001)])
def test_pair_equals_two_layers(cin, cmid, cout, odt, frac):
    """The fused k=3 -> k=1 kernel against the two calls it replaces (the conv stored as bf16,
    then the k=1 layer) and against the oracle's k=1 layer applied to that bf16 intermediate
    (16-bit products are exact in fp32, so the fp32 result is within TAU_ACC); a bf16 output
    is the RNE of the fp32 one, bit for bit."""
    say(f"[parity] pair {cin}->{cmid}->{cout} {odt} occupancy {frac}")
    grid = (15, 14, 13)
    coords, x, w, b = small_case(cin + 3 * cmid + cout, 1, grid, frac, cin, cmid)
    rng = np.random.default_rng(cout + 11)
    w2 = (torch.from_numpy(rng.standard_normal((cmid, cout), dtype=np.float32))
          / np.sqrt(cmid)).to(torch.bfloat16)
    b2 = torch.from_numpy(rng.standard_normal(cout, dtype=np.float32))
    idx = run_gpu(coords, 1, grid)
    xd, wd, bd, w2d, b2d = x.to(DEV), w.to(DEV), b.to(DEV), w2.to(DEV), b2.to(DEV)
    pk1, pk2 = ssc.pack_weights(wd), ssc.pack_weights(w2d, pair=True)
    mid = ssc.subm_conv3d_packed(xd, pk1, bd, idx.plan, torch.bfloat16)
    two = ssc.linear(mid, w2d, b2d, torch.float32)
    f32 = ssc.subm_conv3d_pair(xd, pk1, bd, idx.plan, pk2, b2d, torch.float32)
    ref = oracle.linear(mid.float().cpu().numpy(), w2.float().numpy(), b2.numpy())
    err = rel_err(f32.cpu().numpy(), ref)
    diff = rel_err(f32.cpu().numpy(), two.cpu().numpy().astype(np.float64))
    say(f"[parity]   vs oracle k=1 {err:.3e}, vs the two calls {diff:.3e}, bit-identical "
        f"{bool(torch.equal(f32.view(torch.int32), two.view(torch.int32)))}")
    assert err <= TAU_ACC and diff <= TAU_ACC
    if odt != torch.float32:
        y = ssc.subm_conv3d_pair(xd, pk1, bd, idx.plan, pk2, b2d, odt)
        assert torch.equal(y.cpu().view(torch.int16), f32.cpu().to(odt).view(torch.int16))
    # no biases
    f0 = ssc.subm_conv3d_pair(xd, pk1, None, idx.plan, pk2, None, torch.float32)
    mid0 = ssc.subm_conv3d_packed(xd, pk1, None, idx.plan, torch.bfloat16)
    ref0 = oracle.linear(mid0.float().cpu().numpy(), w2.float().numpy(), None)
    assert rel_err(f0.cpu().numpy(), ref0) <= TAU_ACC


@pytest.mark.parametrize("cin,cout", [(c, o) for c in (32, 64, 128) for o in (16, 32, 64, 128)])
def test_mfma_shapes_ragged(cin, cout):
    # ~1500 sites: several 128-row tiles and a ragged last tile
    say(f"[shapes] cin={cin} cout={cout}")
    coords, x, w, b = small_case(cin * 7 + cout, 2, (20, 20, 20), 0.09, cin, cout)
    check_conv(coords, 2, (20, 20, 20), x, w, b, TAU["bf16"])


@pytest.mark.parametrize("cin,cout,dtype", [
    (16, 16, torch.float32), (5, 7, torch.float32), (16, 16, torch.bfloat16),
    (48, 24, torch.bfloat16), (3, 130, torch.bfloat16),
])
def test_valu_paths(cin, cout, dtype):
    say(f"[valu] cin={cin} cout={cout} {dtype}")
    coords, x, w, b = small_case(cin + cout, 1, (12, 12, 12), 0.3, cin, cout, dtype)
    check_conv(coords, 1, (12, 12, 12), x, w, b,
               TAU["f32"] if dtype == torch.float32 else TAU["bf16"])


@pytest.mark.parametrize("n_sites", [1, 2, 15, 16, 17, 255, 256, 257])
def test_ragged_site_counts(n_sites):
    say(f"[ragged] n={n_sites}")
    rng = np.random.default_rng(n_sites)
    grid = (8, 8, 8)
    coords = workloads.random_sites(rng, 1, grid, n_sites)
    x = torch.from_numpy(rng.standard_normal((n_sites, 32), dtype=np.float32)).to(torch.bfloat16)
    w = (torch.from_numpy(rng.standard_normal((27, 32, 32), dtype=np.float32)) / 30).to(torch.bfloat16)
    b = torch.from_numpy(rng.standard_normal(32, dtype=np.float32))
    check_conv(coords, 1, grid, x, w, b, TAU["bf16"])


def test_full_occupancy_and_boundaries():
    say("[full] 10x9x8 fully occupied")
    grid = (10, 9, 8)
    coords = workloads.coords_from_occupancy([np.ones(grid, bool)])
    rng = np.random.default_rng(3)
    x = torch.from_numpy(rng.standard_normal((len(coords), 64), dtype=np.float32)).to(torch.bfloat16)
    w = (torch.from_numpy(rng.standard_normal((27, 64, 64), dtype=np.float32)) / 40).to(torch.bfloat16)
    idx, _ = check_conv(coords, 1, grid, x, w, None, TAU["bf16"])
    nbr = idx.nbr.cpu().numpy()
    assert (nbr >= 0).sum() == np.prod([3 * g - 2 for g in grid])


def test_extreme_coordinates():
    """Largest supported grid and batch: clusters at both ends of every axis, in the first and
    last batch entries (keys use all 16 bits of every field)."""
    say("[extreme] grid 65535^3, batch 65535")
    G, B = 65535, 65535
    blk = np.array([(x, y, z) for x in range(4) for y in range(4) for z in range(3)], np.int32)
    parts = []
    for b, off in ((0, (0, 0, 0)), (0, (G - 4, G - 4, G - 3)), (B - 1, (0, G - 4, 0)),
                   (B - 1, (G - 4, 0, G - 3)), (B - 1, (0, 0, 0))):
        parts.append(np.concatenate([np.full((len(blk), 1), b, np.int32), blk + np.array(off)], 1))
    coords = np.concatenate(parts).astype(np.int32)
    rng = np.random.default_rng(12)
    x = torch.from_numpy(rng.standard_normal((len(coords), 32), dtype=np.float32)).to(torch.bfloat16)
    w = (torch.from_numpy(rng.standard_normal((27, 32, 32), dtype=np.float32)) / 30).to(torch.bfloat16)
    idx, _ = check_conv(coords, B, (G, G, G), x, w, None, TAU["bf16"])
    # clusters never see each other: every cluster is the same 4x4x3 block
    nbr = idx.nbr.cpu().numpy()
    per = (nbr >= 0).sum(1).reshape(len(parts), -1)
    assert (per == per[0]).all()


def test_isolated_sites_only_centre():
    say("[isolated]")
    g = 16
    pts = np.array([(x, y, z) for x in range(0, g, 2) for y in range(0, g, 2) for z in range(0, g, 2)])
    coords = np.concatenate([np.zeros((len(pts), 1), np.int32), pts.astype(np.int32)], 1)
    rng = np.random.default_rng(4)
    x = torch.from_numpy(rng.standard_normal((len(coords), 64), dtype=np.float32)).to(torch.bfloat16)
    w = (torch.from_numpy(rng.standard_normal((27, 64, 32), dtype=np.float32)) / 40).to(torch.bfloat16)
    idx, y = check_conv(coords, 1, (g, g, g), x, w, None, TAU["bf16"])
    assert (idx.nbr.cpu().numpy() >= 0).sum() == len(coords)


def test_identity_centre_tap_exact():
    say("[identity]")
    coords, x, _, _ = small_case(5, 2, (16, 16, 16), 0.1, 64, 64)
    w = torch.zeros((27, 64, 64))
    w[13] = torch.eye(64)
    idx = run_gpu(coords, 2, (16, 16, 16))
    y = idx.conv(x.to(DEV), w.to(torch.bfloat16).to(DEV), None)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), x.float())


def test_translation_and_determinism():
    say("[translation]")
    coords, x, w, b = small_case(6, 1, (24, 24, 24), 0.1, 128, 128)
    idx = run_gpu(coords, 1, (40, 40, 40))
    idx2 = run_gpu(coords + np.array([0, 5, 9, 13], np.int32), 1, (40, 40, 40))
    assert torch.equal(idx.nbr, idx2.nbr)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    y1 = idx.conv(xd, wd, bd)
    y2 = idx2.conv(xd, wd, bd)
    y3 = idx.conv(xd, wd, bd)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y3)


def test_row_order_does_not_change_results():
    # each output row is computed the same way whatever block it lands in
    say("[order]")
    coords, x, w, b = small_case(8, 1, (24, 24, 24), 0.1, 64, 128)
    p = np.random.default_rng(8).permutation(len(coords))
    idx = run_gpu(coords, 1, (24, 24, 24))
    idxp = run_gpu(np.ascontiguousarray(coords[p]), 1, (24, 24, 24))
    y = idx.conv(x.to(DEV), w.to(DEV), b.to(DEV))
    yp = idxp.conv(x[p].contiguous().to(DEV), w.to(DEV), b.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(y.cpu()[torch.from_numpy(p)], yp.cpu())


def test_batch_isolation():
    say("[batch]")
    one, x, w, b = small_case(9, 1, (12, 12, 12), 0.2, 32, 32)
    two = np.concatenate([one, one + np.array([1, 0, 0, 0], np.int32)])
    x2 = torch.cat([x, -x])
    idx = run_gpu(two, 2, (12, 12, 12))
    y = idx.conv(x2.to(DEV), w.to(DEV), b.to(DEV)).cpu()
    idx1 = run_gpu(one, 1, (12, 12, 12))
    y1 = idx1.conv(x.to(DEV), w.to(DEV), b.to(DEV)).cpu()
    ym = idx1.conv((-x).contiguous().to(DEV), w.to(DEV), b.to(DEV)).cpu()
    n = len(one)
    assert torch.equal(y[:n], y1) and torch.equal(y[n:], ym)


@pytest.mark.parametrize("bad,status", [([0, 12, 0, 0], ssc.SSC_ERR_COORD_RANGE),
                                        ([1, 0, 0, 0], ssc.SSC_ERR_COORD_RANGE),
                                        ([0, 0, -1, 0], ssc.SSC_ERR_COORD_RANGE),
                                        (None, ssc.SSC_ERR_DUPLICATE)])
def test_bad_coordinates_are_reported(bad, status):
    say(f"[errors] {bad}")
    coords, _, _, _ = small_case(10, 1, (12, 12, 12), 0.1, 32, 32)
    row = coords[3] if bad is None else np.array(bad, np.int32)
    c = np.concatenate([coords, row[None]]).astype(np.int32)
    with pytest.raises(ssc.SscError) as e:
        ssc.build_index(torch.from_numpy(c).to(DEV), 1, (12, 12, 12))
    assert e.value.status == status


def test_empty_input():
    say("[empty]")
    c = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    idx = ssc.SubMIndex(c, 1, (4, 4, 4))
    y = idx.conv(torch.zeros((0, 32), dtype=torch.bfloat16, device=DEV),
                 torch.zeros((27, 32, 16), dtype=torch.bfloat16, device=DEV), None)
    assert y.shape == (0, 16)


@pytest.mark.parametrize("n,cin,cout", [(1, 64, 64), (1000, 64, 128), (4097, 128, 128),
                                        (300, 32, 16), (77, 16, 16)])
def test_linear(n, cin, cout):
    say(f"[linear] n={n} {cin}->{cout}")
    rng = np.random.default_rng(n)
    x = torch.from_numpy(rng.standard_normal((n, cin), dtype=np.float32)).to(torch.bfloat16)
    w = (torch.from_numpy(rng.standard_normal((cin, cout), dtype=np.float32)) / np.sqrt(cin)).to(torch.bfloat16)
    b = torch.from_numpy(rng.standard_normal(cout, dtype=np.float32))
    y = ssc.linear(x.to(DEV), w.to(DEV), b.to(DEV))
    ybf = ssc.linear(x.to(DEV), w.to(DEV), b.to(DEV), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.linear(x.float().numpy(), w.float().numpy(), b.numpy())
    assert rel_err(y.cpu().numpy(), ref) <= TAU["bf16"]
    assert torch.equal(ybf.cpu().view(torch.int16), rne_bf16(y.cpu()).view(torch.int16))


@pytest.mark.parametrize("cin,cout", [(128, 128), (64, 32), (32, 64)])
def test_packed_matches_per_call_packing(cin, cout):
    say(f"[packed] cin={cin} cout={cout}")
    coords, x, w, b = small_case(cin + 3 * cout, 1, (20, 20, 20), 0.1, cin, cout)
    idx = run_gpu(coords, 1, (20, 20, 20))
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    y = idx.conv(xd, wd, bd)
    pw = ssc.pack_weights(wd)
    yp = ssc.subm_conv3d_packed(xd, pw, bd, idx.plan)
    ypb = ssc.subm_conv3d_packed(xd, pw, bd, idx.plan, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y, yp)
    assert torch.equal(ypb.cpu().view(torch.int16), rne_bf16(y.cpu()).view(torch.int16))


def test_flip_orientation_matches_oracle():
    say("[flip]")
    coords, x, w, b = small_case(31, 2, (14, 14, 14), 0.2, 64, 64)
    m = oracle.build_map(coords, 2, (14, 14, 14))
    idx = run_gpu(coords, 2, (14, 14, 14))
    pw = ssc.pack_weights(w.to(DEV), flip=True)
    y = ssc.subm_conv3d_packed(x.to(DEV), pw, b.to(DEV), idx.plan)
    torch.cuda.synchronize()
    ref = oracle.conv(x.float().numpy(), w.float().numpy(), b.numpy(), m, flip=True)
    assert rel_err(y.cpu().numpy(), ref) <= TAU["bf16"]
    ref_cc = oracle.conv(x.float().numpy(), w.float().numpy(), b.numpy(), m)
    assert rel_err(y.cpu().numpy(), ref_cc) > 0.1  # really the other orientation


def gray_rank_keys(nbr: np.ndarray) -> np.ndarray:
    """Sort key of the plan, computed here from its definition: the 26-bit mask of valid
    non-centre taps (tap t < 13 at bit t, t > 13 at bit t - 1), read as a reflected Gray code
    and converted to its rank (bit i = XOR of mask bits i..25)."""
    valid = np.delete(nbr >= 0, 13, axis=1).astype(np.int64)
    rank = np.zeros(len(valid), np.int64)
    for i in range(26):
        rank |= np.bitwise_xor.reduce(valid[:, i:], axis=1) << i
    return rank


def morton3(bx, by, bz, bits):
    key = np.zeros(len(bx), np.int64)
    for k in range(bits):
        key |= ((bx >> k) & 1) << (3 * k + 2)
        key |= ((by >> k) & 1) << (3 * k + 1)
        key |= ((bz >> k) & 1) << (3 * k)
    return key


def block_tap_pairs(nbr_sorted: np.ndarray) -> int:
    """(16-row block, non-centre tap present) pairs of a site order."""
    valid = np.delete(nbr_sorted >= 0, 13, axis=1)
    pad = (-len(valid)) % 16
    valid = np.concatenate([valid, np.zeros((pad, 26), bool)]).reshape(-1, 16, 26)
    return int(valid.any(axis=1).sum())


TILE_ROWS, STAGE_COST, ORDER_TILES = 128, 11, 32768


def tile_costs(m_sorted: np.ndarray) -> np.ndarray:
    """Cost of each full 128-row tile of a site order: STAGE_COST per tap present anywhere in
    the tile plus one per (16-row block, tap present) pair, the centre tap included."""
    f = len(m_sorted) // TILE_ROWS
    blk = (m_sorted[:f * TILE_ROWS] >= 0).reshape(f, TILE_ROWS // 16, 16, 27).any(axis=2)
    return STAGE_COST * blk.any(axis=1).sum(axis=1) + blk.sum(axis=(1, 2))


def tile_cost_order(order: np.ndarray, m: np.ndarray) -> np.ndarray:
    """The mask order with its full tiles stably re-sorted by ascending cost (the tiles that
    hold padding stay last); unchanged for one tile or more than ORDER_TILES."""
    f = len(order) // TILE_ROWS
    if f < 2 or f > ORDER_TILES:
        return order
    t = np.argsort(tile_costs(m[order]), kind="stable")
    full = order[:f * TILE_ROWS].reshape(f, TILE_ROWS)[t].reshape(-1)
    return np.concatenate([full, order[f * TILE_ROWS:]])


def expected_site_order(coords, batch, grid, m):
    """The plan's site order from its definition: the mask order (stable sort by Gray rank,
    then its full 128-row tiles stably sorted by ascending cost);
    when the grid holds >= 8 bricks of 128^3 (batch entries apart), also the brick order (the
    mask order stably re-sorted by (entry, Morton code of the brick)), kept when its
    (block, tap) pairs are at most 21/20 of the mask order's.  Returns (order, spatial)."""
    mask_order = np.argsort(gray_rank_keys(m), kind="stable")
    per_axis = [(g - 1) // 128 + 1 for g in grid]
    if batch * np.prod(per_axis) < 8:
        return tile_cost_order(mask_order, m), False
    bits = max(int(np.ceil(np.log2(p))) if p > 1 else 0 for p in per_axis)
    c = coords.astype(np.int64)[mask_order]
    key = (c[:, 0] << (3 * bits)) | morton3(c[:, 1] >> 7, c[:, 2] >> 7, c[:, 3] >> 7, bits)
    brick_order = mask_order[np.argsort(key, kind="stable")]
    spatial = block_tap_pairs(m[brick_order]) * 20 <= block_tap_pairs(m[mask_order]) * 21
    return (brick_order if spatial else tile_cost_order(mask_order, m)), spatial


def check_plan(idx, coords, batch, grid, m):
    perm, bmask, gidx = (t.cpu().numpy() for t in idx.plan.parts())
    n, npad = len(m), perm.shape[0]
    assert npad % 256 == 0 and npad >= n
    assert np.array_equal(np.sort(perm[:n]), np.arange(n)) and (perm[n:] == -1).all()
    assert np.array_equal(gidx[:, :n], m[perm[:n]].T) and (gidx[:, n:] == -1).all()
    bits = ((gidx >= 0).astype(np.int64) << np.arange(27)[:, None]).reshape(27, -1, 16)
    want = np.bitwise_or.reduce(np.bitwise_or.reduce(bits, axis=2), axis=0)
    assert np.array_equal(bmask.astype(np.uint32).astype(np.int64), want)
    order, spatial = expected_site_order(coords, batch, grid, m)
    assert np.array_equal(perm[:n], order)
    assert idx.plan.schedule() == (1 if spatial else 0)
    return spatial


@pytest.mark.parametrize("name,shuffle,spatial", [
    ("tiny", False, False), ("batch4", False, False), ("iid128", False, False),
    ("shell256", False, True), ("shell256", True, True), ("shell512", False, True)])
def test_plan_structure(name, shuffle, spatial):
    """The plan's site order is the stable sort by Gray rank of the tap mask, or (surfaces on
    grids of 8 or more 128^3 bricks) that order re-sorted by brick, with every part (row ids,
    block masks, tap-major neighbour rows, tile schedule) consistent with the map."""
    say(f"[plan] {name} shuffle={shuffle}")
    w, m = workload_case(name, shuffle)
    idx = run_gpu(w.coords, w.batch, w.grid)
    np.testing.assert_array_equal(idx.nbr.cpu().numpy(), m)
    assert check_plan(idx, w.coords, w.batch, w.grid, m) == spatial
    if not spatial:
        # whole tiles of the mask order, in ascending cost
        perm = idx.plan.parts()[0][:w.n].cpu().numpy()
        f = w.n // TILE_ROWS
        keys = gray_rank_keys(m)[perm]
        assert (np.diff(keys[:f * TILE_ROWS].reshape(f, TILE_ROWS), axis=1) >= 0).all()
        assert (np.diff(keys[f * TILE_ROWS:]) >= 0).all()
        assert (np.diff(tile_costs(m[perm])) >= 0).all()


def test_plan_spatial_candidate_rejected_and_batched():
    """Sparse i.i.d. sites on a grid of 8 bricks: the brick order costs far more than 5% extra
    (block, tap) pairs, so the mask order stays; a batch of 8 small surfaces counts 8 bricks
    and takes the spatial order.  Both plans convolve to the oracle's result."""
    rng = np.random.default_rng(41)
    coords = workloads.random_sites(rng, 1, (256, 256, 256), 200000)
    m = oracle.build_map(coords, 1, (256, 256, 256))
    idx = run_gpu(coords, 1, (256, 256, 256))
    assert not check_plan(idx, coords, 1, (256, 256, 256), m)
    occ = np.zeros((8, 48, 48, 48), bool)
    g = np.indices((48, 48, 48)) - 23.5
    for b in range(8):
        r = np.sqrt(((g / (np.array([15, 17, 19]) + b % 3)[:, None, None, None]) ** 2).sum(0))
        occ[b] = np.abs(r - 1.0) < 0.12
    coords = np.ascontiguousarray(np.argwhere(occ), dtype=np.int32)
    m = oracle.build_map(coords, 8, (48, 48, 48))
    idx = run_gpu(coords, 8, (48, 48, 48))
    assert check_plan(idx, coords, 8, (48, 48, 48), m)
    x = torch.from_numpy(rng.standard_normal((len(coords), 64), dtype=np.float32)).bfloat16()
    wt = (torch.from_numpy(rng.standard_normal((27, 64, 64), dtype=np.float32)) / 40).bfloat16()
    y = idx.conv(x.to(DEV), wt.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.conv(x.float().numpy(), wt.float().numpy(), None, m)
    assert rel_err(y.cpu().numpy(), ref) <= TAU["bf16"]


@pytest.mark.parametrize("cin,cout", [(32, 16), (64, 64), (128, 128), (64, 128), (128, 32)])
def test_fp16_inputs_matrix_cores(cin, cout):
    """fp16 features and weights (the checkpoints' source precision): fp32 store within the
    fp32-input bound; the fp16 store is the round-to-nearest-even fp16 of the fp32 store."""
    say(f"[fp16] k3 cin={cin} cout={cout}")
    coords, x, w, b = small_case(cin * 3 + cout, 2, (20, 20, 20), 0.09, cin, cout, torch.float16)
    idx, y32 = check_conv(coords, 2, (20, 20, 20), x, w, b, TAU["f16"])
    y16 = idx.conv(x.to(DEV), w.to(DEV), b.to(DEV), torch.float16)
    torch.cuda.synchronize()
    assert y16.dtype == torch.float16
    assert torch.equal(y16.cpu(), y32.cpu().to(torch.float16))


@pytest.mark.parametrize("cin,cout,odt", [(16, 16, torch.float32), (48, 24, torch.float16),
                                          (3, 130, torch.float32)])
def test_fp16_inputs_valu(cin, cout, odt):
    say(f"[fp16] valu cin={cin} cout={cout} {odt}")
    coords, x, w, b = small_case(cin + cout + 1, 1, (12, 12, 12), 0.3, cin, cout, torch.float16)
    m = oracle.build_map(coords, 1, (12, 12, 12))
    idx = run_gpu(coords, 1, (12, 12, 12))
    y = idx.conv(x.to(DEV), w.to(DEV), b.to(DEV), odt)
    torch.cuda.synchronize()
    ref = oracle.conv(x.float().numpy(), w.float().numpy(), b.numpy(), m)
    if odt == torch.float32:
        assert rel_err(y.cpu().numpy(), ref) <= TAU["f16"]
    else:
        y32 = idx.conv(x.to(DEV), w.to(DEV), b.to(DEV), torch.float32)
        assert torch.equal(y.cpu(), y32.cpu().to(torch.float16))


@pytest.mark.parametrize("n,cin,cout", [(1000, 64, 128), (4097, 128, 128), (77, 16, 16)])
def test_fp16_linear(n, cin, cout):
    say(f"[fp16] linear n={n} {cin}->{cout}")
    rng = np.random.default_rng(n + 7)
    x = torch.from_numpy(rng.standard_normal((n, cin), dtype=np.float32)).to(torch.float16)
    w = (torch.from_numpy(rng.standard_normal((cin, cout), dtype=np.float32)) / np.sqrt(cin)).to(torch.float16)
    b = torch.from_numpy(rng.standard_normal(cout, dtype=np.float32))
    y = ssc.linear(x.to(DEV), w.to(DEV), b.to(DEV))
    y16 = ssc.linear(x.to(DEV), w.to(DEV), b.to(DEV), torch.float16)
    torch.cuda.synchronize()
    ref = oracle.linear(x.float().numpy(), w.float().numpy(), b.numpy())
    assert rel_err(y.cpu().numpy(), ref) <= TAU["f16"]
    assert torch.equal(y16.cpu(), y.cpu().to(torch.float16))


@pytest.mark.parametrize("cin,cout,dtype", [(1024, 8, torch.bfloat16), (4, 1024, torch.float32)])
def test_maximum_channels_conv(cin, cout, dtype):
    """The largest channel counts the entry points accept (1024), on the vector-ALU path."""
    say(f"[max] k3 cin={cin} cout={cout} {dtype}")
    coords, x, w, b = small_case(cin * 3 + cout, 1, (6, 5, 4), 0.5, cin, cout, dtype)
    check_conv(coords, 1, (6, 5, 4), x, w, b,
               TAU["f32"] if dtype == torch.float32 else TAU["bf16"])


def test_map_entry_matches_plan_and_oracle():
    """ssc_subm_conv3d takes the neighbour map itself (it plans the map on every call): on the
    128^3 benchmark workload it equals the warm plan path bit for bit and the oracle within
    the bars."""
    say("[map entry] iid128")
    w, m = workload_case("iid128")
    layer = w.layers[0]
    c = torch.from_numpy(w.coords).to(DEV)
    nbr = ssc.build_index(c, w.batch, w.grid)
    x, wt, b = w.feats.to(DEV), layer.weight.to(DEV), layer.bias.to(DEV)
    y_map = ssc.subm_conv3d(x, wt, b, nbr)
    y_map16 = ssc.subm_conv3d(x, wt, b, nbr, out_dtype=torch.bfloat16)
    plan = ssc.build_plan(nbr)  # the map entry's own plan: mask order, no coordinates
    y_plan = ssc.subm_conv3d(x, wt, b, plan)
    torch.cuda.synchronize()
    assert torch.equal(y_map, y_plan)
    assert torch.equal(y_map16.cpu().view(torch.int16), rne_bf16(y_map.cpu()).view(torch.int16))
    ref = oracle.conv(w.feats.float().numpy(), layer.weight.float().numpy(), layer.bias.numpy(), m)
    err = rel_err(y_map.cpu().numpy(), ref)
    say(f"[map entry] max|err|/rms = {err:.3e}")
    assert err <= TAU["bf16"] and err <= TAU_ACC


def test_map_entry_small_and_fp32():
    say("[map entry] ragged bf16 and fp32")
    for dtype, tau in ((torch.bfloat16, TAU["bf16"]), (torch.float32, TAU["f32"])):
        coords, x, w, b = small_case(77, 2, (14, 14, 14), 0.12, 32, 64, dtype)
        m = oracle.build_map(coords, 2, (14, 14, 14))
        nbr = ssc.build_index(torch.from_numpy(coords).to(DEV), 2, (14, 14, 14))
        y = ssc.subm_conv3d(x.to(DEV), w.to(DEV), b.to(DEV), nbr)
        torch.cuda.synchronize()
        ref = oracle.conv(x.float().numpy(), w.float().numpy(), b.numpy(), m)
        err = rel_err(y.cpu().numpy(), ref)
        assert err <= tau and err <= TAU_ACC, (dtype, err)


def test_cached_index_reuse_and_invalidation():
    """cached_index returns the cached SubMIndex while the coordinate tensor is the same object
    with the same version, and rebuilds after an in-place edit, for a new tensor with equal
    contents, and for another grid or batch; freed tensors' entries are dropped."""
    say("[cache]")
    rng = np.random.default_rng(31)
    grid = (16, 16, 16)
    coords = workloads.random_sites(rng, 2, grid, 700)
    c = torch.from_numpy(coords).to(DEV)
    i1 = ssc.cached_index(c, 2, grid)
    assert ssc.cached_index(c, 2, grid) is i1                      # hit
    assert np.array_equal(i1.nbr.cpu().numpy(), oracle.build_map(coords, 2, grid))
    # in-place edit: move every site one voxel in x inside the grid (bumps the version)
    keep = coords[:, 1] < grid[0] - 1
    c = torch.from_numpy(coords[keep]).to(DEV)
    i2 = ssc.cached_index(c, 2, grid)
    c[:, 1] += 1
    i3 = ssc.cached_index(c, 2, grid)
    assert i3 is not i2
    moved = coords[keep].copy()
    moved[:, 1] += 1
    assert np.array_equal(i3.nbr.cpu().numpy(), oracle.build_map(moved, 2, grid))
    assert ssc.cached_index(c, 2, grid) is i3                      # hit again after rebuild
    c2 = c.clone()                                                 # equal contents, new tensor
    i4 = ssc.cached_index(c2, 2, grid)
    assert i4 is not i3 and torch.equal(i4.nbr, i3.nbr)
    i5 = ssc.cached_index(c2, 2, (17, 16, 16))                     # another grid
    assert i5 is not i4 and torch.equal(i5.nbr, i4.nbr)
    i6 = ssc.cached_index(c2, 3, grid)                             # another batch
    assert i6 is not i4 and i6 is not i5
    # entries of freed tensors do not pile up beyond the cache's bound
    for k in range(ssc._CACHE_MAX + 4):
        t = torch.from_numpy(workloads.random_sites(rng, 1, (8, 8, 8), 50 + k)).to(DEV)
        ssc.cached_index(t, 1, (8, 8, 8))
        del t
    assert len(ssc._CACHE) <= ssc._CACHE_MAX
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["tiny", "iid128", "shell256", "batch4", "shell512"])
def test_index_methods_bit_exact(name):
    """Both index structures (the hash and the dense rank index) build the oracle's map bit for
    bit on every workload, and the automatic choice is the dense one at these sizes."""
    say(f"[index] {name} hash and dense")
    w, m = workload_case(name)
    c = torch.from_numpy(w.coords).to(DEV)
    for method in ("hash", "dense"):
        nbr = ssc.build_index(c, w.batch, w.grid, method=method)
        torch.cuda.synchronize()
        assert np.array_equal(nbr.cpu().numpy(), m), f"{name}: {method} map differs"
    g = (__import__("ctypes").c_int32 * 3)(*w.grid)
    assert ssc.load_library().ssc_index_method(w.n, w.batch, g) == 2


def test_dense_index_errors_and_edges():
    """Dense index: out-of-range rows and duplicates are reported like the hash's; grids at the
    edge of their axes; sites only in the last batch entry; one site."""
    say("[index] dense errors and edges")
    grid = (9, 1, 70)
    rng = np.random.default_rng(44)
    coords = workloads.random_sites(rng, 3, grid, 40)
    coords = coords[coords[:, 0] == 2]                               # last batch entry only
    coords = np.concatenate([coords, np.array([[2, 8, 0, 69], [2, 0, 0, 0]], np.int32)])
    coords = np.unique(coords, axis=0)[rng.permutation(len(np.unique(coords, axis=0)))]
    c = torch.from_numpy(np.ascontiguousarray(coords)).to(DEV)
    for method in ("hash", "dense"):
        nbr = ssc.build_index(c, 3, grid, method=method)
        assert np.array_equal(nbr.cpu().numpy(), oracle.build_map(coords, 3, grid))
        one = torch.from_numpy(coords[:1].copy()).to(DEV)
        assert np.array_equal(ssc.build_index(one, 3, grid, method=method).cpu().numpy(),
                              oracle.build_map(coords[:1], 3, grid))
        bad = coords.copy()
        bad[0, 3] = grid[2]                                          # z outside the grid
        with pytest.raises(ssc.SscError) as e:
            ssc.build_index(torch.from_numpy(bad).to(DEV), 3, grid, method=method)
        assert e.value.status == ssc.SSC_ERR_COORD_RANGE
        dup = np.concatenate([coords, coords[3:4]])
        with pytest.raises(ssc.SscError) as e:
            ssc.build_index(torch.from_numpy(dup).to(DEV), 3, grid, method=method)
        assert e.value.status == ssc.SSC_ERR_DUPLICATE
