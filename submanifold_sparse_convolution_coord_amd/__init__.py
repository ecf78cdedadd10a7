"""Submanifold sparse 3x3x3 convolution (SubMConv3d) for AMD MI355X.

Thin Python binding over libssc.so (include/ssc.h).  Every step of the computation runs
in the library's HIP kernels; this module only checks and marshals arguments, allocates
outputs and workspaces with torch, and passes torch's current HIP stream.  There is no
fallback: if libssc.so has not been built, importing works but every call raises.

    nbr  = build_index(coords, batch, grid)          # [N, 27] int32, -1 = no neighbour
    y    = subm_conv3d(x, w, b, nbr)                 # k=3 on the map (plans it every call)
    plan = build_plan(nbr, coords, batch, grid)      # warm payload, reused by every layer
    y    = subm_conv3d(x, w, b, plan)                # k=3, w [27, Cin, Cout], warm path
    y2   = linear(y.to(torch.bfloat16), w1, b1)      # k=1

``SubMIndex`` bundles the map and the plan of one coordinate set, and ``cached_index``
reuses it while the coordinate tensor is unchanged (the pages' spatial cache).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import weakref
from typing import Optional, Sequence

import torch

__all__ = ["SscError", "build_index", "build_plan", "subm_conv3d", "linear", "Plan",
           "PackedWeight", "pack_weights", "subm_conv3d_packed",
           "GroupNormPartials", "gn_partials", "gn_finalize", "gn_apply", "group_norm",
           "layer_norm",
           "downsample2", "upsample2", "spatial2channel2", "subdivide2",
           "SubMIndex", "cached_index", "library_path", "load_library", "TAPS", "CENTRE_TAP"]

TAPS = 27
CENTRE_TAP = 13

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libssc.so")

SSC_OK, SSC_ERR_ARG, SSC_ERR_COORD_RANGE, SSC_ERR_DUPLICATE = 0, -1, -2, -3
SSC_ERR_UNSUPPORTED, SSC_ERR_WORKSPACE, SSC_ERR_HIP = -4, -5, -6
SSC_F32, SSC_BF16, SSC_F16 = 0, 1, 2
SSC_PACK_FLIP, SSC_PACK_PAIR = 1, 2
ACTS = {"none": 0, "relu": 1, "silu": 2}
GN_MAX_BATCH = 64


class _Epilogue(ctypes.Structure):
    """ssc_epilogue (include/ssc.h)."""
    _fields_ = [("act", ctypes.c_int32), ("gn_groups", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("residual", ctypes.c_void_p), ("coords", ctypes.c_void_p),
                ("gn_partials", ctypes.c_void_p), ("gn_partials_bytes", ctypes.c_size_t)]


class SscError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({_status_string(status)})")
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libssc.so and declare its signatures; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "submanifold_sparse_convolution_coord_amd.build.build()")
    lib = ctypes.CDLL(_LIB_PATH)
    # Refuse a library built from other sources than the ones on disk (a failed or skipped
    # rebuild would otherwise run stale kernels).
    from . import build as _build
    lib.ssc_source_digest.argtypes = []
    lib.ssc_source_digest.restype = ctypes.c_char_p
    built, current = lib.ssc_source_digest().decode(), _build.source_digest()
    if built != current:
        raise RuntimeError(f"{_LIB_PATH} was built from other sources (digest {built}, sources "
                           f"{current}): rebuild it with "
                           "submanifold_sparse_convolution_coord_amd.build.build()")
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "ssc_version": ([], ctypes.c_int),
        "ssc_source_digest": ([], ctypes.c_char_p),
        "ssc_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "ssc_index_workspace_bytes": ([i64], sz),
        "ssc_build_index": ([p, i64, i32, p, p, p, sz, i32, p], ctypes.c_int),
        "ssc_build_index_ex": ([p, i64, i32, p, p, p, sz, i32, i32, p], ctypes.c_int),
        "ssc_index_method": ([i64, i32, p], ctypes.c_int32),
        "ssc_index_workspace_bytes_ex": ([i64, i32, p, i32], sz),
        "ssc_plan_bytes": ([i64], sz),
        "ssc_plan_workspace_bytes": ([i64], sz),
        "ssc_build_plan": ([p, p, i64, i32, p, p, sz, p, sz, p], ctypes.c_int),
        "ssc_plan_layout": ([i64, p], ctypes.c_int),
        "ssc_conv_workspace_bytes": ([i32, i32, i32], sz),
        "ssc_subm_conv3d_workspace_bytes": ([i64, i32, i32, i32], sz),
        "ssc_subm_conv3d": ([p, i32, p, p, p, i64, i32, i32, p, i32, p, sz, p], ctypes.c_int),
        "ssc_subm_conv3d_plan": ([p, i32, p, p, p, i64, i32, i32, p, i32, p, sz, p],
                                 ctypes.c_int),
        "ssc_subm_conv3d_plan_static": ([p, i32, p, p, p, i64, i32, i32, p, i32, p],
                                        ctypes.c_int),
        "ssc_linear": ([p, i32, p, p, i64, i32, i32, p, i32, p, sz, p], ctypes.c_int),
        "ssc_packed_weight_bytes": ([i32, i32, i32], sz),
        "ssc_pack_weights": ([p, i32, i32, i32, p, sz, p], ctypes.c_int),
        "ssc_pack_weights_ex": ([p, i32, i32, i32, i32, p, sz, p], ctypes.c_int),
        "ssc_subm_conv3d_packed": ([p, p, p, p, i64, i32, i32, p, i32, p], ctypes.c_int),
        "ssc_downsample_workspace_bytes": ([i64], sz),
        "ssc_downsample2": ([p, i64, i32, p, p, i32, i32, p, p, p, p, p, sz, p], ctypes.c_int),
        "ssc_upsample2": ([p, i32, i32, p, i64, i64, p, p], ctypes.c_int),
        "ssc_spatial2channel2": ([p, i64, i32, p, p, i32, i32, p, p, p, p, p, sz, p],
                                 ctypes.c_int),
        "ssc_subdivide2": ([p, i64, p, p, i32, i32, p, p, p], ctypes.c_int),
        "ssc_subm_conv3d_plan_ex": ([p, i32, p, p, p, i64, i32, i32, p, i32, p, p, sz, p],
                                    ctypes.c_int),
        "ssc_subm_conv3d_packed_ex": ([p, p, p, p, i64, i32, i32, p, i32, p, p], ctypes.c_int),
        "ssc_linear_ex": ([p, i32, p, p, i64, i32, i32, p, i32, p, p, sz, p], ctypes.c_int),
        "ssc_linear_packed": ([p, p, p, i64, i32, i32, p, i32, p], ctypes.c_int),
        "ssc_subm_conv3d_pair_packed": ([p, p, p, p, i64, i32, i32, p, p, i32, p, i32, p],
                                        ctypes.c_int),
        "ssc_linear_packed_ex": ([p, p, p, i64, i32, i32, p, i32, p, p], ctypes.c_int),
        "ssc_gn_partials_bytes": ([i64, i32, i32], sz),
        "ssc_gn_partials": ([p, i32, i64, i32, p, i32, i32, p, sz, p], ctypes.c_int),
        "ssc_gn_finalize": ([p, i64, i32, i32, ctypes.c_float, p, p], ctypes.c_int),
        "ssc_gn_apply": ([p, i32, i64, i32, p, i32, i32, p, p, p, i32, p, p], ctypes.c_int),
        "ssc_layer_norm": ([p, i32, i64, i32, p, p, ctypes.c_float, i32, p, p], ctypes.c_int),
        "ssc_gather_taps": ([p, i32, i64, i32, p, p, p], ctypes.c_int),
        "ssc_scatter_add_rows": ([p, i32, p, i64, i32, p, i64, p], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _status_string(status: int) -> str:
    try:
        return load_library().ssc_status_string(status).decode()
    except Exception:  # library missing while formatting an error
        return "?"


def _check(status: int, what: str):
    if status != SSC_OK:
        raise SscError(status, what)


# torch's raw current-stream lookup (one C call) when this torch has it; the Stream object
# route costs about 2 us per call, which small layers pay on every launch.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(dev: torch.device) -> ctypes.c_void_p:
    if _raw_stream is not None:
        idx = dev.index if dev.index is not None else torch.cuda.current_device()
        return ctypes.c_void_p(_raw_stream(idx))
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _on(dev: torch.device):
    """torch.cuda.device(dev), or nothing when dev is already the current device."""
    if dev.index is None or dev.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(dev)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_cuda(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(nbytes: int, dev: torch.device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=dev)


def _dtype_code(dt: torch.dtype, name: str) -> int:
    if dt == torch.float32:
        return SSC_F32
    if dt == torch.bfloat16:
        return SSC_BF16
    if dt == torch.float16:
        return SSC_F16
    raise ValueError(f"{name}: dtype {dt} not supported (float32, bfloat16 or float16)")


INDEX_METHODS = {"auto": 0, "hash": 1, "dense": 2}


def build_index(coords: torch.Tensor, batch: int, grid: Sequence[int],
                check: bool = True, method: str = "auto") -> torch.Tensor:
    """[N, 27] int32 neighbour map of the sites ``coords`` ([N, 4] int32 (b, x, y, z)).
    ``method``: "auto", "hash" or "dense" (the index structure; the map is the same)."""
    if method not in INDEX_METHODS:
        raise ValueError(f"method must be one of {sorted(INDEX_METHODS)}")
    _need_cuda(coords, "coords")
    if coords.dtype != torch.int32 or coords.dim() != 2 or coords.shape[1] != 4:
        raise ValueError("coords must be int32 [N, 4]")
    lib = load_library()
    dev = coords.device
    n = coords.shape[0]
    nbr = torch.empty((n, TAPS), dtype=torch.int32, device=dev)
    g = (ctypes.c_int32 * 3)(*[int(v) for v in grid])
    ws = _workspace(lib.ssc_index_workspace_bytes_ex(n, int(batch), g, INDEX_METHODS[method]),
                    dev)
    with _on(dev):
        st = lib.ssc_build_index_ex(_ptr(coords), n, int(batch), g, _ptr(nbr), _ptr(ws),
                                    ws.numel(), 1 if check else 0, INDEX_METHODS[method],
                                    _stream(dev))
    _check(st, "ssc_build_index")
    return nbr


class Plan:
    """Warm plan of one coordinate set (sites sorted by tap mask, or by 128^3 brick and then
    tap mask; tap-major neighbour rows)."""

    def __init__(self, buf: torch.Tensor, n: int):
        self.buf = buf
        self.n = n

    @property
    def device(self):
        return self.buf.device

    def parts(self):
        """Device views of the plan: (perm int32 [npad], block masks int32 [npad/16],
        neighbour rows int32 [27, npad]) as laid out by ssc_plan_layout."""
        lay = (ctypes.c_int64 * 5)()
        _check(load_library().ssc_plan_layout(self.n, lay), "ssc_plan_layout")
        npad, o_perm, o_bm, o_g = lay[0], lay[1], lay[2], lay[3]

        def view(off, count):
            return self.buf[off:off + 4 * count].view(torch.int32)

        return (view(o_perm, npad), view(o_bm, npad // 16),
                view(o_g, TAPS * npad).view(TAPS, npad))

    def schedule(self) -> int:
        """The tile schedule recorded with the site order: 0 interleaved (mask order), 1 one
        contiguous share of the tiles per XCD (spatial order).  Reads the device header."""
        return int(self.buf[:64].view(torch.int64)[4].item())


def build_plan(nbr: torch.Tensor, coords: Optional[torch.Tensor] = None, batch: int = 1,
               grid: Optional[Sequence[int]] = None) -> Plan:
    """Warm plan from the neighbour map; with the coordinates (and their batch and grid) the
    spatial site order is tried too."""
    _need_cuda(nbr, "nbr")
    if nbr.dtype != torch.int32 or nbr.dim() != 2 or nbr.shape[1] != TAPS:
        raise ValueError("nbr must be int32 [N, 27]")
    lib = load_library()
    dev = nbr.device
    n = nbr.shape[0]
    g = None
    if coords is not None:
        _need_cuda(coords, "coords")
        if coords.dtype != torch.int32 or coords.shape != (n, 4) or not coords.is_contiguous():
            raise ValueError("coords must be contiguous int32 [N, 4] matching nbr")
        if grid is None:
            raise ValueError("grid is required with coords")
        g = (ctypes.c_int32 * 3)(*[int(v) for v in grid])
    buf = _workspace(lib.ssc_plan_bytes(n), dev)
    ws = _workspace(lib.ssc_plan_workspace_bytes(n), dev)
    with _on(dev):
        st = lib.ssc_build_plan(_ptr(nbr), None if coords is None else _ptr(coords), n,
                                int(batch), g, _ptr(buf), buf.numel(), _ptr(ws), ws.numel(),
                                _stream(dev))
    _check(st, "ssc_build_plan")
    return Plan(buf, n)


def _conv_args(x, weight, bias, taps, out_dtype):
    _need_cuda(x, "x")
    _need_cuda(weight, "weight")
    if x.dim() != 2:
        raise ValueError("x must be [N, Cin]")
    n, cin = x.shape
    wshape = (1, *weight.shape) if weight.dim() == 2 else tuple(weight.shape)
    if len(wshape) != 3 or wshape[0] != taps or wshape[1] != cin:
        raise ValueError(f"weight must be [{taps}, {cin}, Cout], got {tuple(weight.shape)}")
    if weight.dtype != x.dtype:
        raise ValueError("weight and x must have the same dtype")
    cout = wshape[2]
    if bias is not None:
        _need_cuda(bias, "bias")
        if bias.dtype != torch.float32 or bias.numel() != cout:
            raise ValueError("bias must be float32 [Cout]")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    return n, cin, cout, _dtype_code(x.dtype, "x"), _dtype_code(out_dtype, "out_dtype"), out_dtype


class GroupNormPartials:
    """Group-norm partial sums of n sites (ssc_gn_partials_bytes): filled by gn_partials or
    by a convolution's epilogue, read by gn_finalize."""

    def __init__(self, n: int, batch: int, groups: int, device, coords=None):
        if not 1 <= batch <= GN_MAX_BATCH:
            raise ValueError(f"batch must be in [1, {GN_MAX_BATCH}]")
        if batch > 1 and coords is None:
            raise ValueError("coords (batch ids) are needed when batch > 1")
        nbytes = load_library().ssc_gn_partials_bytes(n, batch, groups)
        if nbytes == 0:
            raise ValueError("bad group-norm shape")
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.n, self.batch, self.groups, self.coords = int(n), int(batch), int(groups), coords
        # one slot per 128 rows of n rounded up to a multiple of 256 (the header's layout)
        self.slots = (max(self.n, 1) + 255) // 256 * 2

    def sums(self) -> torch.Tensor:
        """The partial sums as float32 [slots, batch, groups, 4] = (count, sum, sum of
        squares, 0); the buffer's tail past them is alignment padding."""
        used = self.slots * self.batch * self.groups * 16
        return self.buf[:used].view(torch.float32).view(self.slots, self.batch, self.groups, 4)


def _epilogue(n, cout, out_dtype, act, residual, gn):
    """The ssc_epilogue struct for the _ex entry points (None when it would be the plain
    convolution)."""
    if act == "none" and residual is None and gn is None:
        return None
    if act not in ACTS:
        raise ValueError(f"act must be one of {sorted(ACTS)}")
    e = _Epilogue()
    e.act = ACTS[act]
    if residual is not None:
        _need_cuda(residual, "residual")
        if residual.shape != (n, cout) or residual.dtype != out_dtype:
            raise ValueError(f"residual must be [{n}, {cout}] {out_dtype}")
        e.residual = residual.data_ptr()
    if gn is not None:
        if not isinstance(gn, GroupNormPartials) or gn.n != n:
            raise ValueError(f"gn must be GroupNormPartials for {n} sites")
        e.gn_groups, e.batch = gn.groups, gn.batch
        e.coords = None if gn.coords is None else gn.coords.data_ptr()
        e.gn_partials, e.gn_partials_bytes = gn.buf.data_ptr(), gn.buf.numel()
    return e


def subm_conv3d(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor], index,
                out_dtype: Optional[torch.dtype] = None,
                out: Optional[torch.Tensor] = None, act: str = "none",
                residual: Optional[torch.Tensor] = None,
                gn: Optional[GroupNormPartials] = None) -> torch.Tensor:
    """k=3 SubMConv3d: out[i] = bias + sum_t x[nbr[i][t]] @ weight[t] (cross-correlation).
    ``weight`` is [27, Cin, Cout] with the dtype of ``x``; output fp32 unless ``out_dtype``.
    ``index`` is the neighbour map (int32 [N, 27] from build_index: ssc_subm_conv3d, which builds
    the warm plan of the map on every call), or a Plan / SubMIndex of it (ssc_subm_conv3d_plan:
    the warm path).  Epilogue (plan path): out = act(conv + bias) + residual, and with ``gn``
    the group-norm partial sums of the stored output."""
    n, cin, cout, din, dout, odt = _conv_args(x, weight, bias, TAPS, out_dtype)
    lib = load_library()
    dev = x.device
    if isinstance(index, SubMIndex):
        index = index.plan
    if isinstance(index, torch.Tensor):
        nbr = index
        _need_cuda(nbr, "nbr")
        if nbr.dtype != torch.int32 or tuple(nbr.shape) != (n, TAPS):
            raise ValueError(f"nbr must be int32 [{n}, {TAPS}]")
        if act != "none" or residual is not None or gn is not None:
            raise ValueError("epilogues take a Plan (build_plan) or a SubMIndex")
        if out is None:
            out = torch.empty((n, cout), dtype=odt, device=dev)
        ws = _workspace(lib.ssc_subm_conv3d_workspace_bytes(n, cin, cout, din), dev)
        with _on(dev):
            st = lib.ssc_subm_conv3d(_ptr(x), din, _ptr(weight), _ptr(bias), _ptr(nbr), n, cin,
                                     cout, _ptr(out), dout, _ptr(ws), ws.numel(), _stream(dev))
        _check(st, "ssc_subm_conv3d")
        return out
    plan = index
    if not isinstance(plan, Plan):
        raise TypeError("index must be an int32 [N, 27] map, a Plan or a SubMIndex")
    if plan.n != n:
        raise ValueError(f"plan is for {plan.n} sites, x has {n}")
    if out is None:
        out = torch.empty((n, cout), dtype=odt, device=dev)
    epi = _epilogue(n, cout, odt, act, residual, gn)
    need = lib.ssc_conv_workspace_bytes(cin, cout, din)
    ws = _workspace(need, dev) if need > 0 else None  # none when nothing is re-laid out
    wsn = ws.numel() if ws is not None else 0
    with _on(dev):
        if epi is None:
            st = lib.ssc_subm_conv3d_plan(_ptr(x), din, _ptr(weight), _ptr(bias), _ptr(plan.buf),
                                          n, cin, cout, _ptr(out), dout, _ptr(ws), wsn,
                                          _stream(dev))
        else:
            st = lib.ssc_subm_conv3d_plan_ex(_ptr(x), din, _ptr(weight), _ptr(bias),
                                             _ptr(plan.buf), n, cin, cout, _ptr(out), dout,
                                             ctypes.byref(epi), _ptr(ws), wsn,
                                             _stream(dev))
    _check(st, "ssc_subm_conv3d_plan")
    return out


def linear(x: torch.Tensor, weight, bias: Optional[torch.Tensor],
           out_dtype: Optional[torch.dtype] = None,
           out: Optional[torch.Tensor] = None, act: str = "none",
           residual: Optional[torch.Tensor] = None,
           gn: Optional[GroupNormPartials] = None) -> torch.Tensor:
    """k=1 SubMConv3d = per-voxel linear map x @ weight + bias (weight [Cin, Cout] or
    [1, Cin, Cout], or a single-tap PackedWeight from pack_weights); the same epilogue as
    subm_conv3d."""
    if isinstance(weight, PackedWeight):
        return _linear_packed(x, weight, bias, out_dtype, out, act, residual, gn)
    n, cin, cout, din, dout, odt = _conv_args(x, weight, bias, 1, out_dtype)
    lib = load_library()
    dev = x.device
    if out is None:
        out = torch.empty((n, cout), dtype=odt, device=dev)
    epi = _epilogue(n, cout, odt, act, residual, gn)
    ws = _workspace(lib.ssc_conv_workspace_bytes(cin, cout, din), dev)
    with _on(dev):
        if epi is None:
            st = lib.ssc_linear(_ptr(x), din, _ptr(weight), _ptr(bias), n, cin, cout, _ptr(out),
                                dout, _ptr(ws), ws.numel(), _stream(dev))
        else:
            st = lib.ssc_linear_ex(_ptr(x), din, _ptr(weight), _ptr(bias), n, cin, cout,
                                   _ptr(out), dout, ctypes.byref(epi), _ptr(ws), ws.numel(),
                                   _stream(dev))
    _check(st, "ssc_linear")
    return out


def _gn_coords(coords, batch, n):
    if batch == 1:
        return None
    _need_cuda(coords, "coords")
    if coords.dtype != torch.int32 or coords.shape != (n, 4):
        raise ValueError(f"coords must be int32 [{n}, 4]")
    return coords


def gn_partials(x: torch.Tensor, batch: int = 1, groups: int = 32,
                coords: Optional[torch.Tensor] = None) -> GroupNormPartials:
    """Group-norm partial sums of x [N, C] (the statistics pass of SparseGroupNorm32)."""
    _need_cuda(x, "x")
    n, c = x.shape
    coords = _gn_coords(coords, batch, n)
    parts = GroupNormPartials(n, batch, groups, x.device, coords)
    lib = load_library()
    with torch.cuda.device(x.device):
        st = lib.ssc_gn_partials(_ptr(x), _dtype_code(x.dtype, "x"), n, c, _ptr(coords), batch,
                                 groups, _ptr(parts.buf), parts.buf.numel(), _stream(x.device))
    _check(st, "ssc_gn_partials")
    return parts


def gn_finalize(parts: GroupNormPartials, eps: float = 1e-5) -> torch.Tensor:
    """[batch, groups, 2] float32 (mean, 1 / sqrt(var + eps)) from the partial sums."""
    dev = parts.buf.device
    stats = torch.empty((parts.batch, parts.groups, 2), dtype=torch.float32, device=dev)
    lib = load_library()
    with _on(dev):
        st = lib.ssc_gn_finalize(_ptr(parts.buf), parts.n, parts.batch, parts.groups,
                                 float(eps), _ptr(stats), _stream(dev))
    _check(st, "ssc_gn_finalize")
    return stats


def gn_apply(x: torch.Tensor, stats: torch.Tensor, gamma: Optional[torch.Tensor] = None,
             beta: Optional[torch.Tensor] = None, act: str = "none",
             coords: Optional[torch.Tensor] = None,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """act((x - mean) * rstd * gamma + beta) with stats from gn_finalize; ``out`` may be x."""
    _need_cuda(x, "x")
    _need_cuda(stats, "stats")
    n, c = x.shape
    batch, groups = stats.shape[0], stats.shape[1]
    coords = _gn_coords(coords, batch, n)
    for t, name in ((gamma, "gamma"), (beta, "beta")):
        if t is not None:
            _need_cuda(t, name)
            if t.dtype != torch.float32 or t.numel() != c:
                raise ValueError(f"{name} must be float32 [{c}]")
    if act not in ACTS:
        raise ValueError(f"act must be one of {sorted(ACTS)}")
    if out is None:
        out = torch.empty_like(x)
    lib = load_library()
    with torch.cuda.device(x.device):
        st = lib.ssc_gn_apply(_ptr(x), _dtype_code(x.dtype, "x"), n, c, _ptr(coords), batch,
                              groups, _ptr(stats), _ptr(gamma), _ptr(beta), ACTS[act], _ptr(out),
                              _stream(x.device))
    _check(st, "ssc_gn_apply")
    return out


def layer_norm(x: torch.Tensor, gamma: Optional[torch.Tensor] = None,
               beta: Optional[torch.Tensor] = None, eps: float = 1e-6, act: str = "none",
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """LayerNorm32 over each site's channels (+ activation); ``out`` may be x."""
    _need_cuda(x, "x")
    n, c = x.shape
    for t, name in ((gamma, "gamma"), (beta, "beta")):
        if t is not None:
            _need_cuda(t, name)
            if t.dtype != torch.float32 or t.numel() != c:
                raise ValueError(f"{name} must be float32 [{c}]")
    if act not in ACTS:
        raise ValueError(f"act must be one of {sorted(ACTS)}")
    if out is None:
        out = torch.empty_like(x)
    lib = load_library()
    with torch.cuda.device(x.device):
        st = lib.ssc_layer_norm(_ptr(x), _dtype_code(x.dtype, "x"), n, c, _ptr(gamma),
                                _ptr(beta), float(eps), ACTS[act], _ptr(out), _stream(x.device))
    _check(st, "ssc_layer_norm")
    return out


def group_norm(x: torch.Tensor, batch: int = 1, groups: int = 32,
               gamma: Optional[torch.Tensor] = None, beta: Optional[torch.Tensor] = None,
               eps: float = 1e-5, act: str = "none", coords: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """SparseGroupNorm32 (+ activation): statistics, finalize and apply, three launches."""
    stats = gn_finalize(gn_partials(x, batch, groups, coords), eps)
    return gn_apply(x, stats, gamma, beta, act, coords, out)


def _feat_args(feats: Optional[torch.Tensor], n: int):
    if feats is None:
        return None, SSC_F32, 0
    _need_cuda(feats, "feats")
    if feats.dim() != 2 or feats.shape[0] != n:
        raise ValueError(f"feats must be [{n}, C]")
    return feats, _dtype_code(feats.dtype, "feats"), feats.shape[1]


def downsample2(coords: torch.Tensor, batch: int, grid: Sequence[int],
                feats: Optional[torch.Tensor] = None):
    """SparseDownsample(2), max reduction.  Returns (parent coords [m, 4] int32 in ascending
    (b, x, y, z) order, parent features [m, C] (None without feats), parent [n] int32 = the
    output row of each input site's parent, the parent grid)."""
    _need_cuda(coords, "coords")
    if coords.dtype != torch.int32 or coords.dim() != 2 or coords.shape[1] != 4:
        raise ValueError("coords must be int32 [N, 4]")
    n = coords.shape[0]
    feats, dt, ch = _feat_args(feats, n)
    lib = load_library()
    dev = coords.device
    g = (ctypes.c_int32 * 3)(*[int(v) for v in grid])
    out_c = torch.empty((max(n, 1), 4), dtype=torch.int32, device=dev)
    out_f = torch.empty((max(n, 1), ch), dtype=feats.dtype, device=dev) if ch else None
    parent = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    result = torch.zeros(2, dtype=torch.int64, device=dev)
    ws = _workspace(lib.ssc_downsample_workspace_bytes(n), dev)
    with _on(dev):
        st = lib.ssc_downsample2(_ptr(coords), n, int(batch), g, _ptr(feats), dt, ch, _ptr(out_c),
                                 _ptr(out_f), _ptr(parent), _ptr(result), _ptr(ws), ws.numel(),
                                 _stream(dev))
    _check(st, "ssc_downsample2")
    m, bad = (int(v) for v in result.cpu())
    if bad:
        raise SscError(SSC_ERR_COORD_RANGE, "ssc_downsample2")
    hgrid = tuple((int(v) + 1) // 2 for v in grid)
    return out_c[:m], (out_f[:m] if ch else None), parent[:n], hgrid


def spatial2channel2(coords: torch.Tensor, batch: int, grid: Sequence[int],
                     feats: torch.Tensor):
    """SparseSpatial2Channel(2): returns (parent coords [m, 4], features [m, 8C] with channel c
    of child k = 4(x&1) + 2(y&1) + (z&1) at column c*8 + k (zeros for absent children),
    parent [n], the parent grid)."""
    _need_cuda(coords, "coords")
    if coords.dtype != torch.int32 or coords.dim() != 2 or coords.shape[1] != 4:
        raise ValueError("coords must be int32 [N, 4]")
    n = coords.shape[0]
    feats, dt, ch = _feat_args(feats, n)
    if ch < 1:
        raise ValueError("spatial2channel2 needs features")
    lib = load_library()
    dev = coords.device
    g = (ctypes.c_int32 * 3)(*[int(v) for v in grid])
    out_c = torch.empty((max(n, 1), 4), dtype=torch.int32, device=dev)
    out_f = torch.empty((max(n, 1), 8 * ch), dtype=feats.dtype, device=dev)
    parent = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    result = torch.zeros(2, dtype=torch.int64, device=dev)
    ws = _workspace(lib.ssc_downsample_workspace_bytes(n), dev)
    with _on(dev):
        st = lib.ssc_spatial2channel2(_ptr(coords), n, int(batch), g, _ptr(feats), dt, ch,
                                      _ptr(out_c), _ptr(out_f), _ptr(parent), _ptr(result),
                                      _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "ssc_spatial2channel2")
    m, bad = (int(v) for v in result.cpu())
    if bad:
        raise SscError(SSC_ERR_COORD_RANGE, "ssc_spatial2channel2")
    return out_c[:m], out_f[:m], parent[:n], tuple((int(v) + 1) // 2 for v in grid)


def upsample2(parent_feats: torch.Tensor, parent: torch.Tensor) -> torch.Tensor:
    """SparseUpsample(2) through a downsample's parent map: out[i] = parent_feats[parent[i]]."""
    _need_cuda(parent_feats, "parent_feats")
    _need_cuda(parent, "parent")
    if parent.dtype != torch.int32 or parent.dim() != 1 or parent_feats.dim() != 2:
        raise ValueError("parent must be int32 [N], parent_feats [M, C]")
    m, ch = parent_feats.shape
    n = parent.shape[0]
    dt = _dtype_code(parent_feats.dtype, "parent_feats")
    out = torch.empty((n, ch), dtype=parent_feats.dtype, device=parent.device)
    lib = load_library()
    with torch.cuda.device(parent.device):
        st = lib.ssc_upsample2(_ptr(parent_feats), dt, ch, _ptr(parent), n, m, _ptr(out),
                               _stream(parent.device))
    _check(st, "ssc_upsample2")
    return out


def subdivide2(coords: torch.Tensor, grid: Sequence[int], feats: Optional[torch.Tensor] = None):
    """SparseSubdivide: each site -> 8 children 8i + 4dx + 2dy + dz at (b, 2x+dx, 2y+dy, 2z+dz)
    carrying its features.  Returns (coords [8N, 4], feats [8N, C] or None, the doubled grid)."""
    _need_cuda(coords, "coords")
    if coords.dtype != torch.int32 or coords.dim() != 2 or coords.shape[1] != 4:
        raise ValueError("coords must be int32 [N, 4]")
    n = coords.shape[0]
    feats, dt, ch = _feat_args(feats, n)
    dev = coords.device
    g = (ctypes.c_int32 * 3)(*[int(v) for v in grid])
    out_c = torch.empty((8 * n, 4), dtype=torch.int32, device=dev)
    out_f = torch.empty((8 * n, ch), dtype=feats.dtype, device=dev) if ch else None
    lib = load_library()
    with _on(dev):
        st = lib.ssc_subdivide2(_ptr(coords), n, g, _ptr(feats), dt, ch, _ptr(out_c), _ptr(out_f),
                                _stream(dev))
    _check(st, "ssc_subdivide2")
    return out_c, out_f, tuple(2 * int(v) for v in grid)


class PackedWeight:
    """A layer's [taps, Cin, Cout] bf16 weights re-laid out once for the matrix cores (pair:
    packed as the k=1 layer of subm_conv3d_pair)."""

    def __init__(self, buf: torch.Tensor, taps: int, cin: int, cout: int, pair: bool = False):
        self.buf, self.taps, self.cin, self.cout, self.pair = buf, taps, cin, cout, pair


def pack_weights(weight: torch.Tensor, flip: bool = False, pair: bool = False) -> PackedWeight:
    """Re-lay out bf16 weights once: [27, Cin, Cout] for subm_conv3d_packed, [Cin, Cout] or
    [1, Cin, Cout] for linear.  flip=True packs the other kernel orientation (tap at offset d
    reads site c - d; nothing changes for a single tap).  pair=True packs a single-tap weight
    as the k=1 layer of subm_conv3d_pair."""
    _need_cuda(weight, "weight")
    if weight.dtype != torch.bfloat16:
        raise ValueError("pack_weights takes bfloat16 weights")
    wshape = (1, *weight.shape) if weight.dim() == 2 else tuple(weight.shape)
    taps, cin, cout = wshape
    lib = load_library()
    dev = weight.device
    buf = _workspace(lib.ssc_packed_weight_bytes(taps, cin, cout), dev)
    with _on(dev):
        st = lib.ssc_pack_weights_ex(_ptr(weight), taps, cin, cout,
                                     (SSC_PACK_FLIP if flip else 0) | (SSC_PACK_PAIR if pair else 0),
                                     _ptr(buf), buf.numel(), _stream(dev))
    _check(st, "ssc_pack_weights")
    return PackedWeight(buf, taps, cin, cout, pair)


def subm_conv3d_pair(x: torch.Tensor, packed1: PackedWeight, bias1: Optional[torch.Tensor],
                     plan: Plan, packed2: PackedWeight, bias2: Optional[torch.Tensor],
                     out_dtype: Optional[torch.dtype] = None,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """A k=3 layer and the k=1 layer after it in one kernel: the result of subm_conv3d_packed
    with a bf16 output followed by linear, the intermediate never written (packed2 from
    pack_weights(w2, pair=True))."""
    _need_cuda(x, "x")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != packed1.cin:
        raise ValueError("x must be bfloat16 [N, Cin] matching packed1")
    if packed1.taps != TAPS or packed2.taps != 1 or not packed2.pair:
        raise ValueError("packed1 must be a 27-tap weight, packed2 a pair=True single-tap one")
    if packed2.cin != packed1.cout:
        raise ValueError("packed2's inputs must be packed1's outputs")
    n = x.shape[0]
    if plan.n != n:
        raise ValueError(f"plan is for {plan.n} sites, x has {n}")
    for b, c, name in ((bias1, packed1.cout, "bias1"), (bias2, packed2.cout, "bias2")):
        if b is not None:
            _need_cuda(b, name)
            if b.dtype != torch.float32 or b.numel() != c:
                raise ValueError(f"{name} must be float32 [{c}]")
    odt = torch.float32 if out_dtype is None else out_dtype
    dout = _dtype_code(odt, "out_dtype")
    lib = load_library()
    dev = x.device
    if out is None:
        out = torch.empty((n, packed2.cout), dtype=odt, device=dev)
    with _on(dev):
        st = lib.ssc_subm_conv3d_pair_packed(_ptr(x), _ptr(packed1.buf), _ptr(bias1),
                                             _ptr(plan.buf), n, packed1.cin, packed1.cout,
                                             _ptr(packed2.buf), _ptr(bias2), packed2.cout,
                                             _ptr(out), dout, _stream(dev))
    _check(st, "ssc_subm_conv3d_pair_packed")
    return out


def subm_conv3d_packed(x: torch.Tensor, packed: PackedWeight, bias: Optional[torch.Tensor],
                       plan: Plan, out_dtype: Optional[torch.dtype] = None,
                       out: Optional[torch.Tensor] = None, act: str = "none",
                       residual: Optional[torch.Tensor] = None,
                       gn: Optional[GroupNormPartials] = None) -> torch.Tensor:
    """subm_conv3d with weights from pack_weights: a single kernel launch (plus one
    statistics pass when ``gn`` has batch > 1)."""
    _need_cuda(x, "x")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != packed.cin or packed.taps != TAPS:
        raise ValueError("x must be bfloat16 [N, Cin] matching a 27-tap packed weight")
    n = x.shape[0]
    if plan.n != n:
        raise ValueError(f"plan is for {plan.n} sites, x has {n}")
    if bias is not None:
        _need_cuda(bias, "bias")
        if bias.dtype != torch.float32 or bias.numel() != packed.cout:
            raise ValueError("bias must be float32 [Cout]")
    odt = torch.float32 if out_dtype is None else out_dtype
    dout = _dtype_code(odt, "out_dtype")
    lib = load_library()
    dev = x.device
    if out is None:
        out = torch.empty((n, packed.cout), dtype=odt, device=dev)
    epi = _epilogue(n, packed.cout, odt, act, residual, gn)
    with _on(dev):
        if epi is None:
            st = lib.ssc_subm_conv3d_packed(_ptr(x), _ptr(packed.buf), _ptr(bias), _ptr(plan.buf),
                                            n, packed.cin, packed.cout, _ptr(out), dout,
                                            _stream(dev))
        else:
            st = lib.ssc_subm_conv3d_packed_ex(_ptr(x), _ptr(packed.buf), _ptr(bias),
                                               _ptr(plan.buf), n, packed.cin, packed.cout,
                                               _ptr(out), dout, ctypes.byref(epi), _stream(dev))
    _check(st, "ssc_subm_conv3d_packed")
    return out


def _linear_packed(x, packed, bias, out_dtype, out, act, residual, gn):
    _need_cuda(x, "x")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != packed.cin or packed.taps != 1:
        raise ValueError("x must be bfloat16 [N, Cin] matching a single-tap packed weight")
    n = x.shape[0]
    if bias is not None:
        _need_cuda(bias, "bias")
        if bias.dtype != torch.float32 or bias.numel() != packed.cout:
            raise ValueError("bias must be float32 [Cout]")
    odt = torch.float32 if out_dtype is None else out_dtype
    dout = _dtype_code(odt, "out_dtype")
    lib = load_library()
    dev = x.device
    if out is None:
        out = torch.empty((n, packed.cout), dtype=odt, device=dev)
    epi = _epilogue(n, packed.cout, odt, act, residual, gn)
    with _on(dev):
        if epi is None:
            st = lib.ssc_linear_packed(_ptr(x), _ptr(packed.buf), _ptr(bias), n, packed.cin,
                                       packed.cout, _ptr(out), dout, _stream(dev))
        else:
            st = lib.ssc_linear_packed_ex(_ptr(x), _ptr(packed.buf), _ptr(bias), n, packed.cin,
                                          packed.cout, _ptr(out), dout, ctypes.byref(epi),
                                          _stream(dev))
    _check(st, "ssc_linear_packed")
    return out


class SubMIndex:
    """Neighbour map + warm plan of one coordinate set, built once and shared by every
    SubMConv3d layer on that set."""

    def __init__(self, coords: torch.Tensor, batch: int, grid: Sequence[int], check: bool = True):
        self.batch = int(batch)
        self.grid = tuple(int(g) for g in grid)
        self.nbr = build_index(coords, batch, grid, check=check)
        self.plan = build_plan(self.nbr, coords, batch, grid)
        self.n = int(coords.shape[0])

    def conv(self, x, weight, bias=None, out_dtype=None):
        return subm_conv3d(x, weight, bias, self.plan, out_dtype)


_CACHE: dict = {}
_CACHE_MAX = 16


def cached_index(coords: torch.Tensor, batch: int, grid: Sequence[int]) -> SubMIndex:
    """SubMIndex of ``coords``, rebuilt only when the tensor object, its storage, shape or
    in-place version counter, or the batch or grid, changes (the per-tensor cache of the
    trellis-mac article's flowchart; the LATO.2 page rebuilds the map whenever coordinates
    change).  Entries whose tensor has been freed are dropped before the oldest live entry is
    evicted, so at most _CACHE_MAX indices stay alive."""
    key = (coords.data_ptr(), tuple(coords.shape), coords.device, int(batch),
           tuple(int(g) for g in grid))
    hit = _CACHE.get(key)
    if hit is not None:
        ref, version, idx = hit
        if ref() is coords and version == coords._version:
            return idx
        del _CACHE[key]
    idx = SubMIndex(coords, batch, grid)
    for k in [k for k, (r, _, _) in _CACHE.items() if r() is None]:
        del _CACHE[k]
    while len(_CACHE) >= _CACHE_MAX:
        _CACHE.pop(next(iter(_CACHE)))
    _CACHE[key] = (weakref.ref(coords), coords._version, idx)
    return idx
