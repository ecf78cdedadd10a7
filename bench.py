"""Benchmark: warm-map SubMConv3d on one MI355X.

Workload (the pages' benchmark shape, LATO.2 MLX port page, "Fleet benchmark"): batch 1,
128^3 grid, i.i.d. occupancy 10 %, Cin = Cout = 128, k=3, bf16 features and weights, fp32
accumulation, neighbour map and plan built once before the timed region (warm).  A step is one
SubMConv3d layer call on resident inputs with the layer's weights re-laid out once at load time
(the per-call entries are reported beside it); the two-layer workload adds its k=1 layer.

Timing: after the warm-up steps, windows of --steps back-to-back steps are timed with HIP
events on the kernels' stream (one before the window, one after it, nothing between the
steps) until there are at least 25 windows and about 0.25 s of GPU work; ms_per_step is the
median window / steps.  The k=3 kernel's time is the step itself for one layer (the same
windows); for two layers it comes from further windows of the k=3 layer alone.

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload iid128]
                    [--out-dtype f32|bf16] [--no-cpu-baseline] [--extras]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PAGES_MVOX_PER_S = 15.25   # M3 Ultra, 128^3, 128 ch, ~10 % occupancy, warm (context only)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 matrix (256 CU x 2.4 GHz x 4096 FLOP/clk)
METRIC = "SubMConv3d Mvox/s + % bf16 MFMA peak, 128^3 C=128 10% occ, warm map"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def mvox_per_s(n_sites: int, seconds: float) -> float:
    """The pages' throughput unit: active sites per second, in millions."""
    return n_sites / seconds / 1e6


def source_digest() -> str:
    """Digest of the sources the convolution kernels are compiled from (their file and the
    device helpers they include); counter figures taken on other sources do not apply."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "submanifold_sparse_convolution_coord_amd", "csrc")
    for path in (os.path.join(csrc, "conv.hip"), os.path.join(csrc, "common.h")):
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def counters_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"conv_{workload}_counters.json")


def counted_traffic(kernel: str, digest: str, workload: str, out_dtype: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources for this kernel, workload and output type; else None."""
    path = counters_path(workload)
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if (d.get("source_digest") != digest or d.get("kernel") != kernel
            or d.get("workload") != workload or d.get("out_dtype", "f32") != out_dtype):
        return None
    return d.get("hbm_bytes_per_launch")


def _counter_rows(d: str, kernel_substr: str, counter: str):
    """Per-dispatch values of `counter` for kernels whose name contains `kernel_substr`, read
    from a rocprofv3 --pmc csv directory."""
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if kernel_substr in row.get("Kernel_Name", "") and row.get("Counter_Name") == counter:
                vals.append(float(row["Counter_Value"]))
    return vals


def conv_kernel_name(cin: int, cout: int, out16: bool, c2: int = 0) -> str:
    """The k=3 kernel instantiation a workload's timed step runs (bf16 inputs): the plain one,
    or with c2 > 0 the pair kernel that applies the k=1 layer of c2 outputs after it."""
    wc = 4 if cout >= 64 else cout // 16
    return (f"k_subm_lds<{cin}, {cout}, 8, {4 // wc}, {wc}, {'true' if out16 else 'false'}, 0, "
            f"false, false, {c2}>")


PAIR_SHAPES = {(32, 64, 64), (64, 64, 64), (128, 64, 64), (64, 128, 64), (64, 128, 128),
               (128, 128, 64), (128, 128, 128)}  # (cin, cmid, cout) of the fused k=3 -> k=1 kernel


def step_kernel(layers) -> tuple:
    """(kernel instance, label, output dtype name) of the dominant kernel of a workload's step:
    the pair kernel when its two layers fit one, else the k=3 kernel."""
    l1 = layers[0]
    if len(layers) > 1 and (l1.cin, l1.cout, layers[1].cout) in PAIR_SHAPES:
        c2 = layers[1].cout
        return (conv_kernel_name(l1.cin, l1.cout, True, c2),
                f"k_subm_lds<{l1.cin},{l1.cout}> + k=1 {l1.cout}->{c2} (pair)", "f32")
    out16 = len(layers) > 1
    return conv_kernel_name(l1.cin, l1.cout, out16), f"k_subm_lds<{l1.cin},{l1.cout}>", None


def summarize_counters(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, cal_mb, out_path,
                       workload="iid128", out_dtype="f32"):
    """HBM traffic of one kernel per launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch,
    the median over the dispatches) scaled by what the same counters read for a plain device
    copy of cal_mb MiB.  The kernel filter names the plain variant the workload's timed layer
    runs (its output type as stored between layers: bf16 for the two-layer workload)."""
    import workloads
    layers = workloads.make(workload).layers
    kernel, label, pair_out = step_kernel(layers)
    if pair_out is None and out_dtype == "bf16":
        kernel = conv_kernel_name(layers[0].cin, layers[0].cout, True)
    out16 = (pair_out is None and len(layers) > 1) or out_dtype == "bf16"
    copy = "copy"  # torch's elementwise copy kernel
    f = _counter_rows(fetch_dir, kernel, "FETCH_SIZE")
    w = _counter_rows(write_dir, kernel, "WRITE_SIZE")
    cf = _counter_rows(cal_fetch_dir, copy, "FETCH_SIZE")
    cw = _counter_rows(cal_write_dir, copy, "WRITE_SIZE")
    if not (f and w and cf and cw):
        raise SystemExit("missing counter rows")
    known = cal_mb * 1024.0  # KiB read and written by the copy
    fetch_scale = known / float(np.median(cf))
    write_scale = known / float(np.median(cw))
    fetch_b = float(np.median(f)) * 1024.0 * fetch_scale
    write_b = float(np.median(w)) * 1024.0 * write_scale
    d = {"kernel": label, "kernel_instance": kernel, "workload": workload,
         "out_dtype": "bf16" if out16 else "f32", "source_digest": source_digest(),
         "fetch_kib_per_dispatch": float(np.median(f)), "write_kib_per_dispatch": float(np.median(w)),
         "dispatches": [len(f), len(w)],
         "copy_calibration_mib": cal_mb, "copy_fetch_kib": float(np.median(cf)),
         "copy_write_kib": float(np.median(cw)), "fetch_scale": fetch_scale,
         "write_scale": write_scale, "hbm_bytes_per_launch": fetch_b + write_b,
         "hbm_read_bytes_per_launch": fetch_b, "hbm_write_bytes_per_launch": write_b}
    json.dump(d, open(out_path, "w"), indent=1)
    print(json.dumps(d))


def counter_table(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, cal_mb) -> str:
    """Markdown table of every kernel's HBM bytes per dispatch (median FETCH_SIZE and
    WRITE_SIZE, scaled by the copy calibration), from rocprofv3 --pmc csv directories."""
    import csv
    import glob
    import re

    def rows(d, counter):
        per = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r.get("Counter_Name") == counter:
                    name = r["Kernel_Name"].replace("void ", "").replace(
                        "ssc::(anonymous namespace)::", "")
                    m = re.match(r"([A-Za-z_0-9:]+(<[^()]*>)?)", name)
                    per.setdefault(m.group(1) if m else name[:60], []).append(
                        float(r["Counter_Value"]))
        return per

    cf = rows(cal_fetch_dir, "FETCH_SIZE")
    cw = rows(cal_write_dir, "WRITE_SIZE")
    copy_f = [v for k, vs in cf.items() if "copy" in k for v in vs]
    copy_w = [v for k, vs in cw.items() if "copy" in k for v in vs]
    known = cal_mb * 1024.0
    fs, ws = known / float(np.median(copy_f)), known / float(np.median(copy_w))
    f, w = rows(fetch_dir, "FETCH_SIZE"), rows(write_dir, "WRITE_SIZE")
    out = [f"FETCH_SIZE scale {fs:.3f}, WRITE_SIZE scale {ws:.3f} (plain {cal_mb} MiB copy)", "",
           "| kernel | dispatches | read MB | write MB | total MB |", "|---|---|---|---|---|"]
    for k in sorted(f, key=lambda k: -float(np.median(f[k]))):
        if k not in w:
            continue
        rd = float(np.median(f[k])) * 1024 * fs / 1e6
        wr = float(np.median(w[k])) * 1024 * ws / 1e6
        out.append(f"| {k[:90]} | {len(f[k])} | {rd:.1f} | {wr:.1f} | {rd + wr:.1f} |")
    return "\n".join(out)


def time_resample(ssc, torch, coords, x, w, dev, reps: int = 20) -> dict:
    """Device time of the downsample (max), its upsample, the spatial-to-channel shuffle and the
    subdivide on the workload's sites and features, called through the C ABI on preallocated
    buffers (the binding's downsample reads the parent count back, which would put a host
    round trip in the timing).  GB/s from the algorithmic bytes of each op."""
    import ctypes
    lib = ssc.load_library()
    n, ch = x.shape
    esz = x.element_size()
    dt = ssc.SSC_BF16 if x.dtype == torch.bfloat16 else ssc.SSC_F32
    g = (ctypes.c_int32 * 3)(*w.grid)
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    oc = torch.empty((n, 4), dtype=torch.int32, device=dev)
    of = torch.empty((n, ch), dtype=x.dtype, device=dev)
    par = torch.empty(n, dtype=torch.int32, device=dev)
    res = torch.zeros(2, dtype=torch.int64, device=dev)
    ws = torch.empty(lib.ssc_downsample_workspace_bytes(n), dtype=torch.uint8, device=dev)
    sc = torch.empty((8 * n, 4), dtype=torch.int32, device=dev)
    sf = torch.empty((8 * n, ch), dtype=x.dtype, device=dev)
    up = torch.empty((n, ch), dtype=x.dtype, device=dev)
    s2c = torch.empty((n, 8 * ch), dtype=x.dtype, device=dev)

    def down():
        return lib.ssc_downsample2(p(coords), n, w.batch, g, p(x), dt, ch, p(oc), p(of), p(par),
                                   p(res), p(ws), ws.numel(), st)

    assert down() == 0
    torch.cuda.synchronize()
    m = int(res[0].item())

    def ups():
        return lib.ssc_upsample2(p(of), dt, ch, p(par), n, m, p(up), st)

    def sub():
        return lib.ssc_subdivide2(p(coords), n, g, p(x), dt, ch, p(sc), p(sf), st)

    def front():  # the parent numbering alone (sort, scan, parent map, parent coordinates)
        return lib.ssc_downsample2(p(coords), n, w.batch, g, None, dt, 0, p(oc), None, p(par),
                                   p(res), p(ws), ws.numel(), st)

    def s2ch():
        return lib.ssc_spatial2channel2(p(coords), n, w.batch, g, p(x), dt, ch, p(oc), p(s2c),
                                        p(par), p(res), p(ws), ws.numel(), st)

    def t(fn):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    row = ch * esz
    d_us, u_us, s_us, c_us, f_us = t(down), t(ups), t(sub), t(s2ch), t(front)
    d_bytes = n * (16 + row + 4) + m * (16 + row)
    c_bytes = n * (16 + row + 4) + m * (16 + 8 * row)
    u_bytes = n * (4 + row) + m * row
    s_bytes = n * (16 + row) + 8 * n * (16 + row)
    return {"n": n, "parents": m, "channels": ch, "parent_numbering_us": round(f_us, 2),
            "downsample_us": round(d_us, 2), "downsample_gbs": round(d_bytes / d_us / 1e3, 1),
            "upsample_us": round(u_us, 2), "upsample_gbs": round(u_bytes / u_us / 1e3, 1),
            "subdivide_us": round(s_us, 2), "subdivide_gbs": round(s_bytes / s_us / 1e3, 1),
            "spatial2channel_us": round(c_us, 2),
            "spatial2channel_gbs": round(c_bytes / c_us / 1e3, 1)}


def time_block(ssc, torch, coords, x, plan, batch, dev, reps: int = 50) -> dict:
    """A pre-norm residual block on the workload's sites, C = the input channels (bf16, C in
    {32, 64, 128}): h = conv1(silu(gn1(x))); y = conv2(silu(gn2(h))) + x with 32-group norms.
    Launches (C ABI, preallocated buffers): gn1 statistics + finalize + apply; conv1 summing
    gn2's statistics in its epilogue (batch 1; else a pass after it); gn2 finalize + apply in
    place; conv2 adding x in its epilogue.  Random weights (seeded), device time per stage."""
    import ctypes
    import math
    lib = ssc.load_library()
    n, c = x.shape
    groups, eps = 32, 1e-5
    gen = torch.Generator().manual_seed(1234)

    def rnd(*shape, scale=1.0):
        return (torch.randn(*shape, generator=gen) * scale)

    w1 = rnd(27, c, c, scale=1 / math.sqrt(27 * c)).to(torch.bfloat16).to(dev)
    w2 = rnd(27, c, c, scale=1 / math.sqrt(27 * c)).to(torch.bfloat16).to(dev)
    pw1, pw2 = ssc.pack_weights(w1), ssc.pack_weights(w2)
    b1, b2 = rnd(c, scale=0.1).to(dev), rnd(c, scale=0.1).to(dev)
    g1, g2 = (1 + rnd(c, scale=0.1)).to(dev), (1 + rnd(c, scale=0.1)).to(dev)
    be1, be2 = rnd(c, scale=0.1).to(dev), rnd(c, scale=0.1).to(dev)
    cd = coords if batch > 1 else None
    parts0 = ssc.GroupNormPartials(n, batch, groups, dev, cd)
    parts1 = ssc.GroupNormPartials(n, batch, groups, dev, cd)
    stats0 = torch.empty((batch, groups, 2), dtype=torch.float32, device=dev)
    stats1 = torch.empty_like(stats0)
    h, h1, y = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    BF, SILU = ssc.SSC_BF16, ssc.ACTS["silu"]
    nb = parts0.buf.numel()
    epi1 = ssc._Epilogue(gn_groups=groups, batch=batch, coords=None if cd is None else cd.data_ptr(),
                         gn_partials=parts1.buf.data_ptr(), gn_partials_bytes=nb)
    epi2 = ssc._Epilogue(residual=x.data_ptr())
    # In a chain of blocks, conv2 also sums the next block's first-norm statistics, so that
    # norm1 of every block but the first is finalize + apply only.
    epi2_chain = ssc._Epilogue(residual=x.data_ptr(), gn_groups=groups, batch=batch,
                               coords=None if cd is None else cd.data_ptr(),
                               gn_partials=parts0.buf.data_ptr(), gn_partials_bytes=nb)

    def norm1():
        lib.ssc_gn_partials(p(x), BF, n, c, p(cd), batch, groups, p(parts0.buf), nb, st)
        lib.ssc_gn_finalize(p(parts0.buf), n, batch, groups, eps, p(stats0), st)
        lib.ssc_gn_apply(p(x), BF, n, c, p(cd), batch, groups, p(stats0), p(g1), p(be1), SILU,
                         p(h), st)

    def conv1():
        lib.ssc_subm_conv3d_packed_ex(p(h), p(pw1.buf), p(b1), p(plan.buf), n, c, c, p(h1), BF,
                                      ctypes.byref(epi1), st)

    def norm2():
        lib.ssc_gn_finalize(p(parts1.buf), n, batch, groups, eps, p(stats1), st)
        lib.ssc_gn_apply(p(h1), BF, n, c, p(cd), batch, groups, p(stats1), p(g2), p(be2), SILU,
                         p(h1), st)

    def conv2():
        lib.ssc_subm_conv3d_packed_ex(p(h1), p(pw2.buf), p(b2), p(plan.buf), n, c, c, p(y), BF,
                                      ctypes.byref(epi2), st)

    def plain_conv():
        lib.ssc_subm_conv3d_packed(p(h), p(pw1.buf), p(b1), p(plan.buf), n, c, c, p(h1), BF, st)

    def norm1_chained():
        lib.ssc_gn_finalize(p(parts0.buf), n, batch, groups, eps, p(stats0), st)
        lib.ssc_gn_apply(p(x), BF, n, c, p(cd), batch, groups, p(stats0), p(g1), p(be1), SILU,
                         p(h), st)

    def conv2_chained():
        lib.ssc_subm_conv3d_packed_ex(p(h1), p(pw2.buf), p(b2), p(plan.buf), n, c, c, p(y), BF,
                                      ctypes.byref(epi2_chain), st)

    def block():
        norm1()
        conv1()
        norm2()
        conv2()

    def block_chained():
        norm1_chained()
        conv1()
        norm2()
        conv2_chained()

    def t(fn):
        for _ in range(5):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    norm1()  # the chained block's first finalize reads statistics that exist
    us = {k: t(f) for k, f in (("block", block), ("block_chained", block_chained),
                               ("norm1", norm1), ("conv1_gn_stats", conv1),
                               ("norm2", norm2), ("conv2_residual", conv2),
                               ("conv2_residual_gn_stats", conv2_chained),
                               ("conv_plain", plain_conv))}
    row = c * 2
    # algorithmic bytes of the two norms: read x twice (statistics, apply) and write h; read
    # and write h1 (its statistics come from conv1's epilogue)
    norm_bytes = n * row * 3 + n * row * 2
    return {"channels": c, "groups": groups, "batch": batch,
            "block_us": round(us["block"], 2), "block_mvox_s": round(n / us["block"], 1),
            # a block inside a chain: its first norm's statistics come from the previous
            # block's last conv
            "block_chained_us": round(us["block_chained"], 2),
            "stages_us": {k: round(v, 2) for k, v in us.items()
                          if k not in ("block", "block_chained")},
            "norm_gbs": round(norm_bytes / (us["norm1"] + us["norm2"]) / 1e3, 1),
            "epilogue_overhead_us": {
                "gn_stats": round(us["conv1_gn_stats"] - us["conv_plain"], 2),
                "residual": round(us["conv2_residual"] - us["conv_plain"], 2)}}


def time_convnext(ssc, torch, x, plan, dev, reps: int = 50) -> dict:
    """A ConvNeXt-style block on the workload's sites, C = the input channels (bf16):
    h = layer_norm(conv(x)); y = linear2(silu(linear1(h))) + x with linear1 C -> 4C and
    linear2 4C -> C (k=1 layers on the streaming kernel or the tiled GEMM by width).  Launches
    through the C ABI on preallocated buffers; random weights (seeded); device time per stage
    and the k=1 layers' algorithmic GB/s (rows in and out, weights)."""
    import ctypes
    import math
    lib = ssc.load_library()
    n, c = x.shape
    gen = torch.Generator().manual_seed(4321)
    bf = torch.bfloat16

    def rnd(*shape, scale=1.0):
        return torch.randn(*shape, generator=gen) * scale

    w = rnd(27, c, c, scale=1 / math.sqrt(27 * c)).to(bf).to(dev)
    pw = ssc.pack_weights(w)
    b = rnd(c, scale=0.1).to(dev)
    g, be = (1 + rnd(c, scale=0.1)).to(dev), rnd(c, scale=0.1).to(dev)
    w1 = rnd(c, 4 * c, scale=1 / math.sqrt(c)).to(bf).to(dev)
    w2 = rnd(4 * c, c, scale=1 / math.sqrt(4 * c)).to(bf).to(dev)
    b1, b2 = rnd(4 * c, scale=0.1).to(dev), rnd(c, scale=0.1).to(dev)
    h = torch.empty_like(x)
    m = torch.empty((n, 4 * c), dtype=bf, device=dev)
    y = torch.empty_like(x)
    # k=1 weights re-laid out once, like the k=3 ones
    pw1, pw2 = ssc.pack_weights(w1), ssc.pack_weights(w2)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    BF = ssc.SSC_BF16
    e1 = ssc._Epilogue(act=ssc.ACTS["silu"])
    e2 = ssc._Epilogue(residual=x.data_ptr())

    def conv():
        lib.ssc_subm_conv3d_packed(p(x), p(pw.buf), p(b), p(plan.buf), n, c, c, p(h), BF, st)

    def norm():
        lib.ssc_layer_norm(p(h), BF, n, c, p(g), p(be), 1e-6, 0, p(h), st)

    def lin1():
        lib.ssc_linear_packed_ex(p(h), p(pw1.buf), p(b1), n, c, 4 * c, p(m), BF,
                                 ctypes.byref(e1), st)

    def lin2():
        lib.ssc_linear_packed_ex(p(m), p(pw2.buf), p(b2), n, 4 * c, c, p(y), BF,
                                 ctypes.byref(e2), st)

    def block():
        conv()
        norm()
        lin1()
        lin2()

    def t(fn):
        for _ in range(5):
            fn()
        e0, e1_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1_.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1_) / reps * 1e3

    us = {k: t(f) for k, f in (("block", block), ("conv", conv), ("layer_norm", norm),
                               ("linear_c_4c_silu", lin1), ("linear_4c_c_residual", lin2))}
    row = c * 2
    l1_bytes = n * row + n * 4 * row + c * 4 * c * 2
    l2_bytes = n * 4 * row + 2 * n * row + c * 4 * c * 2
    return {"channels": c, "block_us": round(us["block"], 2),
            "block_mvox_s": round(n / us["block"], 1),
            "stages_us": {k: round(v, 2) for k, v in us.items() if k != "block"},
            "linear_gbs": {"c_4c": round(l1_bytes / us["linear_c_4c_silu"] / 1e3, 1),
                           "4c_c": round(l2_bytes / us["linear_4c_c_residual"] / 1e3, 1)},
            "layer_norm_gbs": round(2 * n * row / us["layer_norm"] / 1e3, 1)}


def time_ablations(ssc, torch, x, wt, bias, plan, nbr, dev, reps: int = 20) -> dict:
    """The pages' own designs on the same layer (comparison only): the compacted kernel with
    tap compaction off (every block walks all 27 taps), the dense 27-tap GEMM (gather of the
    [N, 27*Cin] operand + a library GEMM, bf16 out) and the per-offset gather -> GEMM ->
    scatter-add (81 launches, replayed from a HIP graph; every replay is checked against the
    eager result).  Device time per layer."""
    from submanifold_sparse_convolution_coord_amd import ablations
    n, cin = x.shape
    cout = wt.shape[2]

    def t(fn, k=reps):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(k):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k * 1e3

    packed = ssc.pack_weights(wt)
    y32 = torch.empty((n, cout), dtype=torch.float32, device=dev)
    compact_us = t(lambda: ssc.subm_conv3d_packed(x, packed, bias, plan, out=y32))
    ref = y32.clone()
    dplan = ablations.dense_taps_plan(plan)
    dense_taps_us = t(lambda: ssc.subm_conv3d_packed(x, packed, bias, dplan, out=y32))
    same = bool(torch.equal(ref.view(torch.int32), y32.view(torch.int32)))
    res = {"compacted_us": round(compact_us, 2),
           "no_compaction_us": round(dense_taps_us, 2), "no_compaction_identical": same}
    operand = n * 27 * cin * x.element_size()
    if operand <= (8 << 30):
        dg = ablations.DenseGemm(nbr, wt)
        ybf = torch.empty((n, cout), dtype=wt.dtype, device=dev)
        g_us = t(lambda: dg.gather(x))
        m_us = t(lambda: dg.gemm(out=ybf))
        res["dense_gemm"] = {"gather_us": round(g_us, 2), "gemm_us": round(m_us, 2),
                             "total_us": round(g_us + m_us, 2),
                             "operand_gb": round(operand / 1e9, 3),
                             "gather_gbs": round(operand / g_us / 1e3, 1)}
    po = ablations.PerOffset(nbr, wt)
    out = torch.empty((n, cout), dtype=torch.float32, device=dev)
    eager = po(x, bias, out=out).clone()
    torch.cuda.synchronize()
    launches = 3 * sum(1 for r in po.rows_out if r.numel() > 0)
    try:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            po(x, bias, out=out)
        replays_ok = True
        for _ in range(3):
            graph.replay()
            torch.cuda.synchronize()
            replays_ok &= bool(torch.equal(out, eager))
            out.fill_(0.0)   # eager work between replays
            torch.cuda.synchronize()
        po_us = t(graph.replay)
        res["per_offset"] = {"us": round(po_us, 2), "launches": launches,
                             "graph_replays_match_eager": replays_ok}
    except RuntimeError as e:  # capture refused: time the eager loop (host enqueue included)
        torch.cuda.synchronize()
        po_us = t(lambda: po(x, bias, out=out))
        res["per_offset"] = {"us_eager": round(po_us, 2), "launches": launches,
                             "graph": f"not captured: {e}"[:200]}
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w) -> dict:
    """The CPU oracle as it stands (fp64 dictionary + per-voxel loop) on the same workload,
    timed on this host's cores: cold (dictionary + 27-tap map) and warm (the convolution over
    every site, map prebuilt), with all threads and with one.  Each phase repeats until it has
    at least 3 runs and about 3 s of work (one-thread warm: 3 runs); the median run is kept.
    ``value`` is the warm all-thread throughput, the counterpart of the GPU's warm-map metric.
    About 10-30 s in all on a many-core host."""
    import oracle
    x = w.feats.float().numpy()
    wt = w.layers[0].weight.float().numpy()
    b = w.layers[0].bias.numpy()
    all_threads = oracle.num_threads()

    def phase(fn, min_runs, min_s, max_s):
        ts = []
        while len(ts) < min_runs or (sum(ts) < min_s and sum(ts) < max_s):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts)), len(ts)

    m = oracle.build_map(w.coords, w.batch, w.grid)
    out = {}
    for threads in (all_threads, 1):
        oracle.set_num_threads(threads)
        tag = "all" if threads == all_threads else "1"
        t, k = phase(lambda: oracle.build_map(w.coords, w.batch, w.grid), 3, 2.0, 6.0)
        out[f"cold_{tag}"] = {"threads": threads, "median_s": round(t, 4), "runs": k,
                              "mvox_s": round(mvox_per_s(w.n, t), 3)}
        t, k = phase(lambda: oracle.conv(x, wt, b, m), 3, 3.0 if threads > 1 else 0.0, 12.0)
        out[f"warm_{tag}"] = {"threads": threads, "median_s": round(t, 4), "runs": k,
                              "mvox_s": round(mvox_per_s(w.n, t), 3)}
        log(f"[bench] oracle {threads} thread(s): cold {out[f'cold_{tag}']['median_s']} s, "
            f"warm {out[f'warm_{tag}']['median_s']} s")
    oracle.set_num_threads(all_threads)
    return {"value": out["warm_all"]["mvox_s"], "unit": "Mvox/s", "cores": all_threads,
            "kind": "oracle", "cpu": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": (f"full workload, all {w.n} sites, fp64; value = warm conv (map prebuilt) "
                       f"on {all_threads} threads, median of {out['warm_all']['runs']} runs; "
                       f"phases: cold = dictionary + 27-tap map, warm = conv only, "
                       f"each on all threads and on 1"),
            "phases": out}


class Windows:
    """Device time of ``k`` back-to-back steps per window, over many windows: one event on the
    stream the kernels run on (torch's current stream) before the first step and one after the
    last, so nothing is enqueued between the steps.  Windows repeat until there are at least
    ``min_windows`` and about ``min_s`` seconds of timed GPU work (at most ``max_windows``);
    each window is synchronised before the next starts."""

    def __init__(self, torch, step, k, min_windows=25, min_s=0.25, max_windows=400):
        self.step_ms, self.windows = [], 0
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        total = 0.0
        while self.windows < min_windows or (total < min_s * 1e3 and
                                             self.windows < max_windows):
            e0.record()
            for _ in range(k):
                step()
            e1.record()
            torch.cuda.synchronize()
            win = e0.elapsed_time(e1)
            total += win
            self.step_ms.append(win / k)
            self.windows += 1
        self.k = k

    def summary(self, values):
        v = np.asarray(values)
        return {"median": float(np.median(v)), "p10": float(np.percentile(v, 10)),
                "p90": float(np.percentile(v, 90)), "first": float(v[0])}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="iid128")
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extras", action="store_true",
                    help="also time single warm and cache-flushed calls and the pages' designs "
                         "(ablations); these launch the headline kernel under other conditions")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (for counter calibration)")
    ap.add_argument("--summarize-counters", nargs=5, metavar=("FETCH_DIR", "WRITE_DIR",
                    "CAL_FETCH_DIR", "CAL_WRITE_DIR", "CAL_MIB"),
                    help="write the conv counter summary of --workload from rocprofv3 --pmc "
                         "output")
    ap.add_argument("--counter-table", nargs=5, metavar=("FETCH_DIR", "WRITE_DIR",
                    "CAL_FETCH_DIR", "CAL_WRITE_DIR", "CAL_MIB"),
                    help="print every kernel's HBM bytes per dispatch from rocprofv3 --pmc output")
    args = ap.parse_args()
    if args.counter_table:
        a = args.counter_table
        print(counter_table(a[0], a[1], a[2], a[3], int(a[4])))
        return
    if args.summarize_counters:
        a = args.summarize_counters
        summarize_counters(a[0], a[1], a[2], a[3], int(a[4]), counters_path(args.workload),
                           workload=args.workload, out_dtype=args.out_dtype)
        return
    if args.copy_calibration:
        import torch
        src = torch.ones(args.copy_calibration * 262144, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_calibration} MiB x3")
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path is a single-GPU "
              "kernel library with no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch
    import submanifold_sparse_convolution_coord_amd as ssc
    import workloads

    dev = torch.device("cuda:0")
    log(f"[bench] generating workload {args.workload}")
    w = workloads.make(args.workload)
    layer = w.layers[0]
    cin, cout = layer.cin, layer.cout
    odt = torch.float32 if args.out_dtype == "f32" else torch.bfloat16
    coords = torch.from_numpy(w.coords).to(dev)
    x = w.feats.to(dev)
    wt = layer.weight.to(dev)
    bias = layer.bias.to(dev)
    torch.cuda.synchronize()

    # Cold path, timed on its own: neighbour map + plan (once per coordinate set).
    cold, cold_index, cold_plan = [], [], []
    for _ in range(7):
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record()
        nbr = ssc.build_index(coords, w.batch, w.grid, check=False)
        e1.record()
        plan = ssc.build_plan(nbr, coords, w.batch, w.grid)
        e2.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e2))
        cold_index.append(e0.elapsed_time(e1))
        cold_plan.append(e1.elapsed_time(e2))
    cold, cold_index, cold_plan = cold[2:], cold_index[2:], cold_plan[2:]
    pairs = int((nbr >= 0).sum().item())
    log(f"[bench] n={w.n} valid_pairs={pairs} cold index+plan median {np.median(cold):.3f} ms "
        f"(index {np.median(cold_index):.3f}, plan {np.median(cold_plan):.3f})")

    # Layer weights are re-laid out once, at load time, as the pages' ports convert their
    # checkpoints once (Pixal3D README / LATO.2 page, weight converters); a step is then the
    # layer calls on resident inputs: the k=3 SubMConv3d, and for the two-layer workload the
    # k=1 layer on its bf16 output.
    mfma_shapes = (16, 32, 64, 128)
    use_packed = (wt.dtype == torch.bfloat16 and cin in (32, 64, 128) and cout in mfma_shapes)
    packed = ssc.pack_weights(wt) if use_packed else None
    two = len(w.layers) > 1
    mid_dt = torch.bfloat16 if two else odt
    y1 = torch.empty((w.n, cout), dtype=mid_dt, device=dev)
    pair = None
    if two:
        l2 = w.layers[1]
        w2, b2 = l2.weight.to(dev), l2.bias.to(dev)
        if w2.dtype == torch.bfloat16:
            # the k=1 layer's weights, re-laid out once as well: for the pair kernel when the
            # two layers fit one (the bf16 intermediate then never leaves the chip), and for
            # the k=1 kernel of the two-launch step reported beside it
            if use_packed and (cin, cout, l2.cout) in PAIR_SHAPES:
                pair = ssc.pack_weights(w2, pair=True)
            w2 = ssc.pack_weights(w2)
        y2 = torch.empty((w.n, l2.cout), dtype=odt, device=dev)

    def conv():
        # fp32 features and channel counts without an MFMA shape run the VALU kernel, which
        # reads the [27, Cin, Cout] weights as they are (nothing to pack).
        if use_packed:
            ssc.subm_conv3d_packed(x, packed, bias, plan, mid_dt, out=y1)
        else:
            ssc.subm_conv3d(x, wt, bias, plan, mid_dt, out=y1)

    def two_launches():
        conv()
        ssc.linear(y1, w2, b2, odt, out=y2)

    def step():
        if pair is not None:
            ssc.subm_conv3d_pair(x, packed, bias, plan, pair, b2, odt, out=y2)
        elif two:
            two_launches()
        else:
            conv()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    win = Windows(torch, step, args.steps)
    t_wall = time.perf_counter() - t_wall
    st = win.summary(win.step_ms)
    # The dominant kernel's time: the step itself for one layer or the pair kernel (same
    # windows); for two launches, windows of the k=3 layer alone on the same inputs (events
    # between the layers would lengthen what they bracket).
    kwin = Windows(torch, conv, args.steps) if two and pair is None else win
    kt = kwin.summary(kwin.step_ms)
    ms_step, ms_kernel = st["median"], kt["median"]
    two_launch = None
    if pair is not None:
        # The same two layers as two launches (k=3 with a bf16 store, then k=1), and the k=3
        # layer alone, for comparison.
        w2l = Windows(torch, two_launches, args.steps, min_windows=10, min_s=0.05)
        w3 = Windows(torch, conv, args.steps, min_windows=10, min_s=0.05)
        two_launch = {"step_us": round(float(np.median(w2l.step_ms)) * 1e3, 2),
                      "k3_us": round(float(np.median(w3.step_ms)) * 1e3, 2)}
        log(f"[bench] pair kernel {ms_step * 1e3:.2f} us; as two launches "
            f"{two_launch['step_us']} us (k=3 alone {two_launch['k3_us']} us)")
    log(f"[bench] {win.windows} windows of {args.steps} steps ({t_wall:.2f} s wall): step "
        f"median {ms_step * 1e3:.2f} us (p10 {st['p10'] * 1e3:.2f}, p90 {st['p90'] * 1e3:.2f}, "
        f"first window {st['first'] * 1e3:.2f}); k=3 kernel {ms_kernel * 1e3:.2f} us")
    # Host cost of enqueueing one step through the binding (no wait): the step is GPU-bound
    # while this stays below ms_per_step.
    t_host = time.perf_counter()
    for _ in range(args.steps):
        step()
    t_host = (time.perf_counter() - t_host) / args.steps
    torch.cuda.synchronize()

    # The same layer through the per-call entries: the weights re-laid out on every call
    # (ssc_subm_conv3d_plan: two launches), and on the neighbour map alone (ssc_subm_conv3d:
    # the plan of the map is built on every call too).  A few warm-up calls, then the median
    # of windows as for the step.
    def windowed(fn):
        for _ in range(3):
            fn()
        wn = Windows(torch, fn, args.steps, min_windows=10, min_s=0.05)
        return float(np.median(wn.step_ms))

    ms_percall = windowed(lambda: ssc.subm_conv3d(x, wt, bias, plan, mid_dt, out=y1))
    ms_map = windowed(lambda: ssc.subm_conv3d(x, wt, bias, nbr, mid_dt, out=y1))
    log(f"[bench] layer with per-call weight re-layout {ms_percall * 1e3:.1f} us; "
        f"on the map alone {ms_map * 1e3:.1f} us")

    extras = {}
    if args.extras:
        # Single launches, each between its own pair of events (warm caches), and with the
        # caches flushed (a 512 MiB fill between calls, outside the events).
        warm = []
        for _ in range(200):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            conv()
            e1.record()
            torch.cuda.synchronize()
            warm.append(e0.elapsed_time(e1) * 1e3)
        flush = torch.empty(512 * 262144, dtype=torch.float32, device=dev)
        single = []
        for _ in range(100):
            flush.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            conv()
            e1.record()
            torch.cuda.synchronize()
            single.append(e0.elapsed_time(e1) * 1e3)
        del flush
        q = lambda v: {"median_us": round(float(np.median(v)), 2),
                       "p10_us": round(float(np.percentile(v, 10)), 2),
                       "p90_us": round(float(np.percentile(v, 90)), 2), "calls": len(v)}
        extras["conv_single_warm"], extras["conv_flushed"] = q(warm), q(single)
        log(f"[bench] single warm calls {extras['conv_single_warm']}, flushed "
            f"{extras['conv_flushed']}")
        if x.dtype == torch.bfloat16 and use_packed:
            extras["ablations"] = time_ablations(ssc, torch, x, wt, bias, plan, nbr, dev)
            log(f"[bench] ablations {extras['ablations']}")

    resample = time_resample(ssc, torch, coords, x, w, dev)
    block = convnext = None
    if x.dtype == torch.bfloat16 and cin in (32, 64, 128):
        block = time_block(ssc, torch, coords, x, plan, w.batch, dev)
        log(f"[bench] residual block {block['block_us']} us (chained {block['block_chained_us']} us) "
            f"{block['stages_us']}")
        convnext = time_convnext(ssc, torch, x, plan, dev)
        log(f"[bench] convnext block {convnext['block_us']} us {convnext['stages_us']}")

    out_bytes = 4 if mid_dt == torch.float32 else 2
    in_bytes = x.element_size()
    # Algorithmic bytes and FLOP of the dominant kernel: X, W and 4 B per valid pair in, Y out
    # (for the pair kernel: W2 in as well, its output out, the intermediate on chip; FLOP of
    # both layers).
    if pair is not None:
        c2 = w.layers[1].cout
        out_bytes = 4 if odt == torch.float32 else 2
        bytes_alg = (w.n * cin * in_bytes + 27 * cin * cout * in_bytes + cout * c2 * in_bytes
                     + w.n * c2 * out_bytes + 4 * pairs)
        flops = 2.0 * pairs * cin * cout + 2.0 * w.n * cout * c2
    else:
        bytes_alg = (w.n * cin * in_bytes + w.n * cout * out_bytes + 27 * cin * cout * in_bytes
                     + 4 * pairs)
        flops = 2.0 * pairs * cin * cout
    achieved_gbs = bytes_alg / (ms_kernel * 1e-3) / 1e9
    tflops_kernel = flops / (ms_kernel * 1e-3) / 1e12
    # The ceiling that binds at the algorithmic level: the matrix cores when the layer's FLOP
    # take longer at the bf16 dense peak than its bytes at the HBM peak (arithmetic intensity
    # above the ridge, 314.6 FLOP/B), else HBM.
    mfma_bound = use_packed and flops / PEAK_BF16_TFLOPS > bytes_alg / PEAK_HBM_GBS * 1e3
    if mfma_bound:
        roofline = {"bound": "mfma", "achieved": round(tflops_kernel, 1),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops_kernel / PEAK_BF16_TFLOPS, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved_gbs / PEAK_HBM_GBS, 4)}
    flops_step = flops + (2.0 * w.n * w.layers[1].cin * w.layers[1].cout
                          if two and pair is None else 0.0)
    tflops_step = flops_step / (ms_step * 1e-3) / 1e12
    value = mvox_per_s(w.n, ms_step * 1e-3)
    kname = (step_kernel(w.layers)[1] if pair is not None
             else f"k_subm_lds<{cin},{cout}>" if use_packed else "k_conv_valu")
    digest = source_digest()
    traffic = counted_traffic(kname, digest, args.workload, "f32" if out_bytes == 4 else "bf16")
    roofline.update({"traffic": traffic, "kernel": kname, "bytes_alg_per_launch": bytes_alg,
                     "flops_alg_per_launch": flops, "kernel_us": round(ms_kernel * 1e3, 2)})
    rnd = lambda d, k=1e3, nd=2: {a: round(v * k, nd) for a, v in d.items()}

    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "Mvox/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        # the pages' figure for this workload (M3 Ultra, LATO.2 page): context, other hardware
        "vs_baseline": round(value / PAGES_MVOX_PER_S, 2) if args.workload == "iid128" else None,
        "dtype": "bf16" if in_bytes == 2 else "f32",
        "data": "synthetic (seeded i.i.d. occupancy, N(0,1) features, fan-in-scaled weights)",
        "config": {"workload": f"{args.workload}: {w.description}", "n_sites": w.n,
                   "valid_pairs": pairs, "cin": cin, "cout": cout,
                   "out_dtype": args.out_dtype, "map": "warm (built once, outside the timing)",
                   "weights": ("re-laid out once at load time (packed)" if use_packed
                               else "read as given ([27, Cin, Cout])"),
                   "parallelism": "single GPU"},
        "timing": {"windows": win.windows, "steps_per_window": args.steps,
                   "step_us": rnd(st), "kernel_us": rnd(kt),
                   "note": "median over windows of back-to-back steps with events only at "
                           "the window ends; kernel_us: the step's dominant kernel, i.e. the "
                           "step itself for one layer or the fused two-layer kernel (same "
                           "windows), else windows of the k=3 layer alone"},
        "two_launch": two_launch,
        "roofline": roofline,
        "mfma": {"effective_tflops_kernel": round(tflops_kernel, 2),
                 "frac_bf16_peak_kernel": round(tflops_kernel / PEAK_BF16_TFLOPS, 5),
                 "effective_tflops_step": round(tflops_step, 2),
                 "frac_bf16_peak_step": round(tflops_step / PEAK_BF16_TFLOPS, 5),
                 "peak_tflops": PEAK_BF16_TFLOPS, "flops_alg": flops},
        "pages_context": {"mvox_s": PAGES_MVOX_PER_S, "hardware": "Apple M3 Ultra (80 GPU cores)",
                          "source": "LATO.2 MLX port page, Fleet benchmark table"},
        "layer_us_per_call_weight_relayout": round(ms_percall * 1e3, 2),
        "layer_us_on_map_alone": round(ms_map * 1e3, 2),
        "cold_index_plan_ms": round(float(np.median(cold)), 4),
        # Algorithmic bytes of the cold path: the index reads the coordinates (16 B per site)
        # and writes the map (27 x 4 B); the plan reads the map and writes the row ids, block
        # masks and tap-major rows (4 + 27 x 4 + 0.25 B).
        "cold_index": {
            "index_ms": round(float(np.median(cold_index)), 4),
            "index_gbs": round(w.n * (16 + 108) / (float(np.median(cold_index)) * 1e-3) / 1e9, 1),
            "plan_ms": round(float(np.median(cold_plan)), 4),
            "plan_gbs": round(w.n * (108 + 4 + 108 + 0.25) / (float(np.median(cold_plan)) * 1e-3)
                              / 1e9, 1),
            # which site order the plan kept: mask order (interleaved tiles) or spatial order
            # (one contiguous share of the tiles per XCD)
            "site_order": "spatial" if plan.schedule() == 1 else "mask"},
        "resample": resample,
        "res_block": block,
        "convnext_block": convnext,
        "host_enqueue_us_per_step": round(t_host * 1e6, 2),
        "source_digest": digest,
    }
    res.update(extras)
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline (cold: dictionary + map; warm: conv)")
        res["cpu_baseline"] = cpu_baseline(w)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
