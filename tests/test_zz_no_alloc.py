"""The allocation-free entry point ssc_subm_conv3d_plan_static (needs an MI355X): called
through the C ABI twice in a row, the second time on a smaller input, it equals
ssc_subm_conv3d_plan (the workspace-taking entry with the same kernels) bit for bit and the
oracle within the conv bars; a layer whose re-laid-out weights exceed the static array is
refused before anything runs."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import submanifold_sparse_convolution_coord_amd as ssc
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def case(seed, grid, n, cin, cout, dtype):
    rng = np.random.default_rng(seed)
    coords = workloads.random_sites(rng, 1, grid, n)
    x = torch.from_numpy(rng.standard_normal((n, cin), dtype=np.float32)).to(dtype)
    w = (torch.from_numpy(rng.standard_normal((27, cin, cout), dtype=np.float32)) /
         np.sqrt(27 * cin)).to(dtype)
    b = torch.from_numpy(rng.standard_normal(cout, dtype=np.float32))
    return coords, x, w, b


def run_static(lib, x, w, b, plan, cout, odt):
    n, cin = x.shape
    y = torch.empty((n, cout), dtype=odt, device=DEV)
    dt = {torch.bfloat16: ssc.SSC_BF16, torch.float16: ssc.SSC_F16, torch.float32: ssc.SSC_F32}
    st = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    r = lib.ssc_subm_conv3d_plan_static(ctypes.c_void_p(x.data_ptr()), dt[x.dtype],
                                        ctypes.c_void_p(w.data_ptr()),
                                        ctypes.c_void_p(b.data_ptr()),
                                        ctypes.c_void_p(plan.buf.data_ptr()), n, cin, cout,
                                        ctypes.c_void_p(y.data_ptr()), dt[odt], st)
    return r, y


def test_static_entry_two_calls_match_workspace_entry():
    lib = ssc.load_library()
    # first call: 128 -> 128 (884,736 bytes of re-laid-out weights), several hundred tiles;
    # second call: a smaller input, 64 -> 32, which must not see the first call's leftovers
    for seed, grid, n, cin, cout in ((1, (40, 40, 40), 6400, 128, 128),
                                     (2, (16, 16, 16), 700, 64, 32)):
        say(f"[static] n={n} {cin}->{cout}")
        coords, x, w, b = case(seed, grid, n, cin, cout, torch.bfloat16)
        idx = ssc.SubMIndex(torch.from_numpy(coords).to(DEV), 1, grid)
        xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
        for odt in (torch.float32, torch.bfloat16):
            r, y = run_static(lib, xd, wd, bd, idx.plan, cout, odt)
            assert r == ssc.SSC_OK, r
            ref = ssc.subm_conv3d(xd, wd, bd, idx.plan, odt)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.uint8), ref.view(torch.uint8))
        m = oracle.build_map(coords, 1, grid)
        want = oracle.conv(x.float().numpy(), w.float().numpy(), b.numpy(), m)
        r, y = run_static(lib, xd, wd, bd, idx.plan, cout, torch.float32)
        torch.cuda.synchronize()
        err = float(np.abs(y.cpu().numpy() - want).max() / np.sqrt((want ** 2).mean()))
        say(f"[static]   max|err|/rms = {err:.3e}")
        assert err <= 1e-5


def test_static_entry_rejects_layers_beyond_its_array():
    lib = ssc.load_library()
    fake = ctypes.c_void_p(1 << 20)
    # 256 -> 256 bf16 needs 27 * 256 * 256 * 2 bytes of re-laid-out weights (> 1 MiB)
    r = lib.ssc_subm_conv3d_plan_static(fake, ssc.SSC_BF16, fake, None, fake, 10, 256, 256, fake,
                                        ssc.SSC_F32, None)
    assert r == ssc.SSC_ERR_WORKSPACE
    assert lib.ssc_conv_workspace_bytes(128, 128, ssc.SSC_BF16) <= 1 << 20
