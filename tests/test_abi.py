"""libssc.so loads and exports every entry point include/ssc.h declares; host-side argument
checks return their status before anything is launched (CPU only, no GPU needed)."""
import ctypes
import os
import re

import pytest

import submanifold_sparse_convolution_coord_amd as ssc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssc.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssc_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssc.library_path()):
        from submanifold_sparse_convolution_coord_amd import build
        build.build()
    return ssc.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    assert lib.ssc_version() >= 100
    for st in range(-6, 1):
        assert lib.ssc_status_string(st)
    assert b"unknown" in lib.ssc_status_string(42)


def test_workspace_sizes(lib):
    assert lib.ssc_index_workspace_bytes(0) > 0
    a, b = lib.ssc_index_workspace_bytes(1000), lib.ssc_index_workspace_bytes(100000)
    assert b > a and b >= 100000 * 2 * 12
    assert lib.ssc_index_workspace_bytes(-1) == 0
    p = lib.ssc_plan_bytes(1000)
    assert p >= 1024 * 28 * 4 and p % 256 == 0
    assert lib.ssc_plan_workspace_bytes(1000) >= 1000 * 16
    assert lib.ssc_conv_workspace_bytes(128, 128, ssc.SSC_BF16) >= 27 * 128 * 128 * 2
    assert lib.ssc_conv_workspace_bytes(16, 16, ssc.SSC_F32) == 0
    # the map-taking conv: plan + plan scratch + re-laid-out weights
    for n in (1, 1000, 209473):
        m = lib.ssc_subm_conv3d_workspace_bytes(n, 128, 128, ssc.SSC_BF16)
        assert m >= (lib.ssc_plan_bytes(n) + lib.ssc_plan_workspace_bytes(n)
                     + lib.ssc_conv_workspace_bytes(128, 128, ssc.SSC_BF16))
    assert lib.ssc_subm_conv3d_workspace_bytes(-1, 128, 128, ssc.SSC_BF16) == 0
    assert lib.ssc_subm_conv3d_workspace_bytes(10, 0, 128, ssc.SSC_BF16) == 0


FAKE = ctypes.c_void_p(1 << 20)       # aligned, never dereferenced: every call below returns
GRID = (ctypes.c_int32 * 3)(8, 8, 8)  # before launching anything


def test_build_index_argument_errors(lib):
    f = lib.ssc_build_index
    assert f(FAKE, -1, 1, GRID, FAKE, FAKE, 1 << 30, 0, None) == ssc.SSC_ERR_ARG
    assert f(FAKE, 10, 1, None, FAKE, FAKE, 1 << 30, 0, None) == ssc.SSC_ERR_ARG
    assert f(None, 10, 1, GRID, FAKE, FAKE, 1 << 30, 0, None) == ssc.SSC_ERR_ARG
    assert f(FAKE, 10, 0, GRID, FAKE, FAKE, 1 << 30, 0, None) == ssc.SSC_ERR_UNSUPPORTED
    assert f(FAKE, 10, 70000, GRID, FAKE, FAKE, 1 << 30, 0, None) == ssc.SSC_ERR_UNSUPPORTED
    bad = (ctypes.c_int32 * 3)(8, 0, 8)
    assert f(FAKE, 10, 1, bad, FAKE, FAKE, 1 << 30, 0, None) == ssc.SSC_ERR_UNSUPPORTED
    big = (ctypes.c_int32 * 3)(8, 65536, 8)
    assert f(FAKE, 10, 1, big, FAKE, FAKE, 1 << 30, 0, None) == ssc.SSC_ERR_UNSUPPORTED
    assert f(FAKE, 10, 1, GRID, FAKE, FAKE, 16, 0, None) == ssc.SSC_ERR_WORKSPACE
    assert f(ctypes.c_void_p((1 << 20) + 4), 10, 1, GRID, FAKE, FAKE, 1 << 30, 0,
             None) == ssc.SSC_ERR_ARG
    assert f(None, 0, 1, GRID, None, None, 0, 1, None) == ssc.SSC_OK  # empty: nothing to do


def test_build_index_method_choice_and_errors(lib):
    f = lib.ssc_build_index_ex
    big = 1 << 30
    assert f(FAKE, 10, 1, GRID, FAKE, FAKE, big, 0, 3, None) == ssc.SSC_ERR_ARG   # method
    assert f(FAKE, 10, 1, GRID, FAKE, FAKE, big, 0, -1, None) == ssc.SSC_ERR_ARG
    huge = (ctypes.c_int32 * 3)(65535, 65535, 65535)
    # forced dense over 2^48 * batch voxels: beyond 62 bits -> unsupported; else short space
    assert f(FAKE, 10, 65535, huge, FAKE, FAKE, big, 0, 2, None) == ssc.SSC_ERR_UNSUPPORTED
    assert f(FAKE, 10, 1, huge, FAKE, FAKE, big, 0, 2, None) == ssc.SSC_ERR_WORKSPACE
    # automatic choice: dense while its arrays fit the hash's workspace
    m = lib.ssc_index_method
    assert m(209473, 1, (ctypes.c_int32 * 3)(128, 128, 128)) == 2
    assert m(1223408, 1, (ctypes.c_int32 * 3)(512, 512, 512)) == 2
    assert m(10, 1, huge) == 1
    assert m(1000, 1, (ctypes.c_int32 * 3)(512, 512, 512)) == 1      # too sparse for a bitmap
    assert m(-1, 1, GRID) == 1
    wb = lib.ssc_index_workspace_bytes_ex
    assert wb(1000, 1, GRID, 0) == wb(1000, 1, GRID, 1) == lib.ssc_index_workspace_bytes(1000)
    assert wb(1, 1, (ctypes.c_int32 * 3)(64, 64, 64), 2) >= 64 ** 3 // 8
    assert wb(10, 65535, huge, 2) == 0 and wb(10, 1, GRID, 7) == 0 and wb(-1, 1, GRID, 0) == 0


def test_build_plan_argument_errors(lib):
    f = lib.ssc_build_plan
    big = 1 << 30

    def call(nbr=FAKE, coords=None, n=10, batch=1, grid=GRID, plan=FAKE, pb=big, ws=FAKE,
             wsb=big):
        return f(nbr, coords, n, batch, grid, plan, pb, ws, wsb, None)

    assert call(n=-1) == ssc.SSC_ERR_ARG
    assert call(nbr=None) == ssc.SSC_ERR_ARG
    assert call(plan=None) == ssc.SSC_ERR_ARG
    assert call(pb=64) == ssc.SSC_ERR_WORKSPACE
    assert call(wsb=8) == ssc.SSC_ERR_WORKSPACE
    assert call(plan=ctypes.c_void_p((1 << 20) + 16)) == ssc.SSC_ERR_ARG
    # with coordinates: grid required, coords 16-byte aligned, batch and grid in range
    assert call(coords=FAKE, grid=None) == ssc.SSC_ERR_ARG
    assert call(coords=ctypes.c_void_p((1 << 20) + 4)) == ssc.SSC_ERR_ARG
    assert call(coords=FAKE, batch=0) == ssc.SSC_ERR_UNSUPPORTED
    assert call(coords=FAKE, batch=70000) == ssc.SSC_ERR_UNSUPPORTED
    assert call(coords=FAKE, grid=(ctypes.c_int32 * 3)(8, 0, 8)) == ssc.SSC_ERR_UNSUPPORTED
    assert call(coords=FAKE, grid=(ctypes.c_int32 * 3)(8, 65536, 8)) == ssc.SSC_ERR_UNSUPPORTED
    assert call(coords=FAKE, wsb=8) == ssc.SSC_ERR_WORKSPACE
    # without coordinates, batch and grid are not looked at
    assert call(batch=0, grid=None, wsb=8) == ssc.SSC_ERR_WORKSPACE


def test_conv_argument_errors(lib):
    f = lib.ssc_subm_conv3d_plan
    big = 1 << 30
    ok = dict(x=FAKE, din=ssc.SSC_BF16, w=FAKE, b=None, plan=FAKE, n=0, cin=64, cout=64, y=FAKE,
              dout=ssc.SSC_F32, ws=FAKE, wsb=big)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["din"], a["w"], a["b"], a["plan"], a["n"], a["cin"], a["cout"], a["y"],
                 a["dout"], a["ws"], a["wsb"], None)

    assert call() == ssc.SSC_OK                        # n = 0 launches nothing
    assert call(din=7) == ssc.SSC_ERR_ARG
    assert call(dout=-1) == ssc.SSC_ERR_ARG
    assert call(n=-5) == ssc.SSC_ERR_ARG
    assert call(cin=0) == ssc.SSC_ERR_UNSUPPORTED
    assert call(cout=4096) == ssc.SSC_ERR_UNSUPPORTED
    assert call(w=None) == ssc.SSC_ERR_ARG
    assert call(plan=None) == ssc.SSC_ERR_ARG
    assert call(n=10, x=None) == ssc.SSC_ERR_ARG
    assert call(n=10, x=ctypes.c_void_p((1 << 20) + 2)) == ssc.SSC_ERR_ARG
    assert call(n=10, wsb=100) == ssc.SSC_ERR_WORKSPACE
    assert call(n=10, ws=None) == ssc.SSC_ERR_WORKSPACE
    lf = lib.ssc_linear
    assert lf(FAKE, ssc.SSC_BF16, FAKE, None, 0, 64, 64, FAKE, ssc.SSC_F32, FAKE, big,
              None) == ssc.SSC_OK
    assert lf(FAKE, 3, FAKE, None, 10, 64, 64, FAKE, ssc.SSC_F32, FAKE, big,
              None) == ssc.SSC_ERR_ARG


def test_map_conv_argument_errors(lib):
    # ssc_subm_conv3d(feats, in_dtype, weight, bias, nbr, n, cin, cout, out, out_dtype,
    #                 workspace, workspace_bytes, stream): every error before any launch
    f = lib.ssc_subm_conv3d
    big = 1 << 30
    ok = dict(x=FAKE, din=ssc.SSC_BF16, w=FAKE, b=None, nbr=FAKE, n=10, cin=128, cout=128,
              y=FAKE, dout=ssc.SSC_F32, ws=FAKE, wsb=big)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["din"], a["w"], a["b"], a["nbr"], a["n"], a["cin"], a["cout"], a["y"],
                 a["dout"], a["ws"], a["wsb"], None)

    assert call(n=0, nbr=None, ws=None, wsb=0) == ssc.SSC_OK      # n = 0 launches nothing
    assert call(n=-1) == ssc.SSC_ERR_ARG
    assert call(din=9) == ssc.SSC_ERR_ARG
    assert call(dout=9) == ssc.SSC_ERR_ARG
    assert call(cin=0) == ssc.SSC_ERR_UNSUPPORTED
    assert call(cout=2048) == ssc.SSC_ERR_UNSUPPORTED
    assert call(nbr=None) == ssc.SSC_ERR_ARG
    assert call(w=None) == ssc.SSC_ERR_ARG
    assert call(x=None) == ssc.SSC_ERR_ARG
    assert call(y=None) == ssc.SSC_ERR_ARG
    assert call(ws=None) == ssc.SSC_ERR_ARG
    assert call(x=ctypes.c_void_p((1 << 20) + 2)) == ssc.SSC_ERR_ARG
    assert call(nbr=ctypes.c_void_p((1 << 20) + 2)) == ssc.SSC_ERR_ARG
    assert call(ws=ctypes.c_void_p((1 << 20) + 64)) == ssc.SSC_ERR_ARG
    assert call(b=ctypes.c_void_p((1 << 20) + 2)) == ssc.SSC_ERR_ARG
    need = lib.ssc_subm_conv3d_workspace_bytes(10, 128, 128, ssc.SSC_BF16)
    assert call(wsb=need - 1) == ssc.SSC_ERR_WORKSPACE


def test_library_digest_matches_sources(lib):
    from submanifold_sparse_convolution_coord_amd import build
    assert lib.ssc_source_digest().decode() == build.source_digest()


def test_stale_library_is_refused(monkeypatch):
    # A library built from other sources than those on disk is never loaded.
    from submanifold_sparse_convolution_coord_amd import build
    monkeypatch.setattr(build, "source_digest", lambda: "0000000000000000")
    monkeypatch.setattr(ssc, "_lib", None)
    with pytest.raises(RuntimeError, match="other sources"):
        ssc.load_library()


def test_pack_weights_argument_errors(lib):
    f = lib.ssc_pack_weights_ex
    big = 1 << 30
    assert f(FAKE, 27, 128, 128, 0, None, big, None) == ssc.SSC_ERR_ARG
    assert f(None, 27, 128, 128, 0, FAKE, big, None) == ssc.SSC_ERR_ARG
    assert f(FAKE, 27, 128, 128, 4, FAKE, big, None) == ssc.SSC_ERR_ARG        # unknown flag
    assert f(FAKE, 2, 128, 128, 0, FAKE, big, None) == ssc.SSC_ERR_UNSUPPORTED  # 27 or 1 taps
    assert f(FAKE, 1, 48, 48, 0, FAKE, big, None) == ssc.SSC_ERR_UNSUPPORTED    # no k=1 kernel
    assert f(FAKE, 1, 128, 128, 0, FAKE, 100, None) == ssc.SSC_ERR_WORKSPACE
    assert f(FAKE, 1, 128, 512, 0, ctypes.c_void_p((1 << 20) + 16), big,
             None) == ssc.SSC_ERR_ARG                                               # misaligned
    assert f(FAKE, 27, 48, 128, 0, FAKE, big, None) == ssc.SSC_ERR_UNSUPPORTED  # no MFMA shape
    assert f(FAKE, 27, 128, 128, 1, FAKE, 100, None) == ssc.SSC_ERR_WORKSPACE
    assert lib.ssc_packed_weight_bytes(27, 128, 128) >= 27 * 128 * 128 * 2
    # SSC_PACK_PAIR: single-tap only, not with FLIP, pair shapes only
    assert f(FAKE, 27, 128, 128, ssc.SSC_PACK_PAIR, FAKE, big, None) == ssc.SSC_ERR_ARG
    assert f(FAKE, 1, 128, 128, ssc.SSC_PACK_PAIR | ssc.SSC_PACK_FLIP, FAKE, big,
             None) == ssc.SSC_ERR_ARG
    assert f(FAKE, 1, 128, 32, ssc.SSC_PACK_PAIR, FAKE, big, None) == ssc.SSC_ERR_UNSUPPORTED
    assert f(FAKE, 1, 32, 32, ssc.SSC_PACK_PAIR, FAKE, big, None) == ssc.SSC_ERR_UNSUPPORTED
    assert f(FAKE, 1, 128, 128, ssc.SSC_PACK_PAIR, FAKE, 100, None) == ssc.SSC_ERR_WORKSPACE
    pp = lib.ssc_subm_conv3d_pair_packed
    # (feats, packed1, bias1, plan, n, cin, cmid, packed2, bias2, cout, out, out_dtype, stream)
    assert pp(FAKE, FAKE, None, FAKE, 0, 64, 128, FAKE, None, 128, FAKE, ssc.SSC_F32,
              None) == ssc.SSC_OK
    assert pp(FAKE, FAKE, None, FAKE, 10, 32, 128, FAKE, None, 128, FAKE, ssc.SSC_F32,
              None) == ssc.SSC_ERR_UNSUPPORTED                          # intermediate too wide
    assert pp(FAKE, FAKE, None, FAKE, 10, 64, 128, FAKE, None, 32, FAKE, ssc.SSC_F32,
              None) == ssc.SSC_ERR_UNSUPPORTED
    assert pp(FAKE, FAKE, None, FAKE, 10, 64, 128, FAKE, None, 128, FAKE, ssc.SSC_F16,
              None) == ssc.SSC_ERR_UNSUPPORTED
    assert pp(FAKE, None, None, FAKE, 10, 64, 128, FAKE, None, 128, FAKE, ssc.SSC_F32,
              None) == ssc.SSC_ERR_ARG
    assert pp(None, FAKE, None, FAKE, 10, 64, 128, FAKE, None, 128, FAKE, ssc.SSC_F32,
              None) == ssc.SSC_ERR_ARG
    assert pp(FAKE, FAKE, None, FAKE, 10, 64, 128, FAKE, ctypes.c_void_p((1 << 20) + 2), 128,
              FAKE, ssc.SSC_F32, None) == ssc.SSC_ERR_ARG                # misaligned bias2
    h = lib.ssc_linear_packed
    assert h(FAKE, FAKE, None, 0, 128, 128, FAKE, ssc.SSC_F32, None) == ssc.SSC_OK
    assert h(FAKE, FAKE, None, 10, 48, 48, FAKE, ssc.SSC_F32, None) == ssc.SSC_ERR_UNSUPPORTED
    assert h(FAKE, FAKE, None, 10, 128, 128, FAKE, ssc.SSC_F16, None) == ssc.SSC_ERR_UNSUPPORTED
    assert h(FAKE, None, None, 10, 128, 128, FAKE, ssc.SSC_F32, None) == ssc.SSC_ERR_ARG
    assert h(None, FAKE, None, 10, 128, 128, FAKE, ssc.SSC_F32, None) == ssc.SSC_ERR_ARG
    assert h(FAKE, FAKE, None, -1, 128, 128, FAKE, ssc.SSC_F32, None) == ssc.SSC_ERR_ARG
    assert h(FAKE, FAKE, None, 10, 128, 128, ctypes.c_void_p((1 << 20) + 4), ssc.SSC_F32,
             None) == ssc.SSC_ERR_ARG
    g = lib.ssc_subm_conv3d_packed
    assert g(FAKE, FAKE, None, FAKE, 0, 128, 128, FAKE, ssc.SSC_F32, None) == ssc.SSC_OK
    assert g(FAKE, FAKE, None, FAKE, 10, 48, 128, FAKE, ssc.SSC_F32, None) == ssc.SSC_ERR_UNSUPPORTED
    assert g(FAKE, None, None, FAKE, 10, 128, 128, FAKE, ssc.SSC_F32, None) == ssc.SSC_ERR_ARG


def test_python_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        ssc.build_index(torch.zeros((4, 4), dtype=torch.int32), 1, (4, 4, 4))


def test_product_path_does_not_import_oracle():
    # The package and its binding never reach the CPU oracle.
    pkg = os.path.dirname(ssc.__file__)
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in text and "liboracle" not in text, fn


def test_plan_layout(lib):
    lay = (ctypes.c_int64 * 5)()
    assert lib.ssc_plan_layout(-1, lay) == ssc.SSC_ERR_ARG
    assert lib.ssc_plan_layout(10, None) == ssc.SSC_ERR_ARG
    for n in (0, 1, 255, 256, 257, 100000):
        assert lib.ssc_plan_layout(n, lay) == ssc.SSC_OK
        npad, o_perm, o_bm, o_g, o_zero = lay
        assert npad % 256 == 0 and npad >= max(n, 1) and npad - max(n, 1) < 256
        assert o_zero + 2048 <= o_perm and o_perm + 4 * npad <= o_bm
        assert o_bm + 4 * (npad // 16) <= o_g
        assert o_g + 4 * 27 * npad <= lib.ssc_plan_bytes(n)
        assert all(o % 256 == 0 for o in (o_perm, o_bm, o_g, o_zero))


def test_resample_argument_errors(lib):
    big = 1 << 30
    f = lib.ssc_downsample2
    # coords, n, batch, grid, feats, dtype, channels, out_coords, out_feats, parent, result, ws, wsb, stream
    assert f(FAKE, -1, 1, GRID, None, 0, 0, FAKE, None, FAKE, FAKE, FAKE, big, None) == ssc.SSC_ERR_ARG
    assert f(FAKE, 10, 1, None, None, 0, 0, FAKE, None, FAKE, FAKE, FAKE, big, None) == ssc.SSC_ERR_ARG
    assert f(FAKE, 10, 1, GRID, None, 0, 0, FAKE, None, FAKE, None, FAKE, big, None) == ssc.SSC_ERR_ARG
    assert f(FAKE, 10, 1, GRID, None, 5, 0, FAKE, None, FAKE, FAKE, FAKE, big, None) == ssc.SSC_ERR_ARG
    assert f(FAKE, 10, 0, GRID, None, 0, 0, FAKE, None, FAKE, FAKE, FAKE, big, None) == ssc.SSC_ERR_UNSUPPORTED
    assert f(FAKE, 10, 1, GRID, None, 0, 4, FAKE, None, FAKE, FAKE, FAKE, big, None) == ssc.SSC_ERR_ARG
    assert f(FAKE, 10, 1, GRID, None, 0, 0, None, None, FAKE, FAKE, FAKE, big, None) == ssc.SSC_ERR_ARG
    assert f(FAKE, 10, 1, GRID, None, 0, 0, FAKE, None, FAKE, FAKE, FAKE, 64, None) == ssc.SSC_ERR_WORKSPACE
    assert lib.ssc_downsample_workspace_bytes(1000) > 1000 * 16
    assert lib.ssc_downsample_workspace_bytes(-1) == 0
    s2c = lib.ssc_spatial2channel2                                   # same arguments
    assert s2c(FAKE, 10, 1, GRID, FAKE, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == ssc.SSC_ERR_ARG
    assert s2c(FAKE, 10, 1, GRID, FAKE, 5, 4, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == ssc.SSC_ERR_ARG
    assert s2c(FAKE, 10, 1, None, FAKE, 0, 4, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == ssc.SSC_ERR_ARG
    assert s2c(FAKE, 10, 1, GRID, None, 0, 4, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == ssc.SSC_ERR_ARG
    assert s2c(FAKE, 10, 1, GRID, FAKE, 2, 4, FAKE, FAKE, FAKE, FAKE, FAKE, 64, None) == ssc.SSC_ERR_WORKSPACE
    u = lib.ssc_upsample2
    assert u(FAKE, 0, 0, FAKE, 10, 5, FAKE, None) == ssc.SSC_ERR_ARG          # channels 0
    assert u(FAKE, 3, 4, FAKE, 10, 5, FAKE, None) == ssc.SSC_ERR_ARG          # dtype
    assert u(FAKE, ssc.SSC_BF16, 3, FAKE, 10, 5, FAKE, None) == ssc.SSC_ERR_ARG  # 6-byte rows
    assert u(FAKE, 0, 4, FAKE, 0, 5, FAKE, None) == ssc.SSC_OK                # nothing to do
    s = lib.ssc_subdivide2
    big_grid = (ctypes.c_int32 * 3)(8, 40000, 8)
    assert s(FAKE, 10, big_grid, None, 0, 0, FAKE, None, None) == ssc.SSC_ERR_UNSUPPORTED
    assert s(FAKE, 10, None, None, 0, 0, FAKE, None, None) == ssc.SSC_ERR_ARG
    assert s(FAKE, 10, GRID, None, 0, 4, FAKE, None, None) == ssc.SSC_ERR_ARG
    assert s(FAKE, 0, GRID, None, 0, 0, FAKE, None, None) == ssc.SSC_OK


def test_epilogue_and_group_norm_argument_errors(lib):
    big = 1 << 30
    E = ssc._Epilogue

    def conv(epi, n=10, cout=64):
        return lib.ssc_subm_conv3d_plan_ex(FAKE, ssc.SSC_BF16, FAKE, None, FAKE, n, 64, cout, FAKE,
                                      ssc.SSC_F32, ctypes.byref(epi), FAKE, big, None)

    assert conv(E(act=3)) == ssc.SSC_ERR_ARG                               # unknown activation
    assert conv(E(act=-1)) == ssc.SSC_ERR_ARG
    assert conv(E(reserved=1)) == ssc.SSC_ERR_ARG
    assert conv(E(residual=(1 << 20) + 8)) == ssc.SSC_ERR_ARG             # misaligned residual
    gn = dict(gn_partials=1 << 20, gn_partials_bytes=big, batch=1)
    assert conv(E(gn_groups=0, **gn)) == ssc.SSC_ERR_ARG
    assert conv(E(gn_groups=24, **gn)) == ssc.SSC_ERR_ARG                 # 64 % 24 != 0
    assert conv(E(gn_groups=512, **gn)) == ssc.SSC_ERR_ARG
    assert conv(E(gn_groups=32, gn_partials=1 << 20, gn_partials_bytes=big, batch=0)) == ssc.SSC_ERR_ARG
    assert conv(E(gn_groups=32, gn_partials=1 << 20, gn_partials_bytes=big, batch=65)) == ssc.SSC_ERR_ARG
    assert conv(E(gn_groups=32, gn_partials=1 << 20, gn_partials_bytes=big, batch=2)) == ssc.SSC_ERR_ARG  # no coords
    assert conv(E(gn_groups=32, gn_partials=1 << 20, gn_partials_bytes=64, batch=1)) == ssc.SSC_ERR_WORKSPACE
    lin = lib.ssc_linear_ex(FAKE, ssc.SSC_BF16, FAKE, None, 10, 64, 64, FAKE, ssc.SSC_F32,
                            ctypes.byref(E(act=9)), FAKE, big, None)
    assert lin == ssc.SSC_ERR_ARG
    pk = lib.ssc_subm_conv3d_packed_ex(FAKE, FAKE, None, FAKE, 10, 128, 128, FAKE, ssc.SSC_F32,
                                       ctypes.byref(E(act=9)), None)
    assert pk == ssc.SSC_ERR_ARG
    lp = lib.ssc_linear_packed_ex(FAKE, FAKE, None, 10, 128, 128, FAKE, ssc.SSC_F32,
                                  ctypes.byref(E(act=9)), None)
    assert lp == ssc.SSC_ERR_ARG
    # partial-sum buffer sizes: one float4 per (128-row slot, batch entry, group)
    assert lib.ssc_gn_partials_bytes(1000, 1, 32) == 8 * 32 * 16
    assert lib.ssc_gn_partials_bytes(0, 2, 4) >= 2 * 2 * 4 * 16
    assert lib.ssc_gn_partials_bytes(10, 65, 32) == 0 and lib.ssc_gn_partials_bytes(-1, 1, 1) == 0
    p = lib.ssc_gn_partials
    assert p(FAKE, 0, 10, 64, None, 1, 0, FAKE, big, None) == ssc.SSC_ERR_ARG       # groups 0
    assert p(FAKE, 0, 10, 64, None, 1, 24, FAKE, big, None) == ssc.SSC_ERR_ARG      # 64 % 24
    assert p(FAKE, 7, 10, 64, None, 1, 32, FAKE, big, None) == ssc.SSC_ERR_ARG      # dtype
    assert p(FAKE, 0, 10, 64, None, 2, 32, FAKE, big, None) == ssc.SSC_ERR_ARG      # coords
    assert p(FAKE, 0, 10, 64, None, 1, 32, FAKE, 16, None) == ssc.SSC_ERR_WORKSPACE
    f = lib.ssc_gn_finalize
    assert f(FAKE, 10, 0, 32, 1e-5, FAKE, None) == ssc.SSC_ERR_ARG
    assert f(FAKE, 10, 1, 32, float("nan"), FAKE, None) == ssc.SSC_ERR_ARG
    assert f(None, 10, 1, 32, 1e-5, FAKE, None) == ssc.SSC_ERR_ARG
    a = lib.ssc_gn_apply
    assert a(FAKE, 0, 10, 64, None, 1, 32, FAKE, None, None, 7, FAKE, None) == ssc.SSC_ERR_ARG
    assert a(FAKE, 0, 10, 64, None, 1, 32, None, None, None, 0, FAKE, None) == ssc.SSC_ERR_ARG
    assert a(FAKE, 0, 0, 64, None, 1, 32, FAKE, None, None, 0, None, None) == ssc.SSC_OK


def test_layer_norm_argument_errors(lib):
    f = lib.ssc_layer_norm
    assert f(FAKE, 0, -1, 32, None, None, 1e-6, 0, FAKE, None) == ssc.SSC_ERR_ARG
    assert f(FAKE, 0, 10, 0, None, None, 1e-6, 0, FAKE, None) == ssc.SSC_ERR_ARG
    assert f(FAKE, 9, 10, 32, None, None, 1e-6, 0, FAKE, None) == ssc.SSC_ERR_ARG
    assert f(FAKE, 0, 10, 32, None, None, -1.0, 0, FAKE, None) == ssc.SSC_ERR_ARG
    assert f(FAKE, 0, 10, 32, None, None, 1e-6, 5, FAKE, None) == ssc.SSC_ERR_ARG
    assert f(None, 0, 10, 32, None, None, 1e-6, 0, FAKE, None) == ssc.SSC_ERR_ARG
    assert f(None, 0, 0, 32, None, None, 1e-6, 0, None, None) == ssc.SSC_OK
