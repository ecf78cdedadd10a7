"""CPU oracle for what sits around the convolution in the sparse blocks: the activations, the
sparse group norm, the convolution with its epilogue (bias, activation, residual), and a
residual block built from them.

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the product path.  Plain numpy in
float64; the convolution itself is the oracle's own (oracle.conv / oracle.linear).  It shares
nothing with the HIP library.

Definitions followed.  The pages name the modules and say what "32" means for the norms:
LayerNorm32 accumulates in fp32 (LATO.2 MLX port page, repository layout), and the remaining
sparse ops listed on that page's "Status" are SparseLinear, LayerNorm32, SparseGroupNorm32,
activations and SparseResBlock.  They give no formulas, so the readings here are the plain
ones (each is also listed among the readings of the design notes):
  activation   "none", "relu" (max(x, 0)) or "silu" (x * sigmoid(x)).
  group norm   per batch entry b and channel group g (groups of C / G consecutive channels):
               mean and population variance over every active site of entry b and every
               channel of g; y = (x - mean) / sqrt(var + eps) * gamma[c] + beta[c].  A sparse
               norm sees the active sites only (the inactive ones are not zeros).
  epilogue     out = act(conv(x) + bias) + residual.
  res block    pre-norm, identity skip (cin = cout):
               h = conv1(silu(gn1(x))); out = conv2(silu(gn2(h))) + x.
  layer norm   per site over its C channels: mean and population variance;
               y = (x - mean) / sqrt(var + eps) * gamma[c] + beta[c].
  ConvNeXt     h = ln(conv(x)); out = linear2(silu(linear1(h))) + x, linear1 C -> 4C,
  block        linear2 4C -> C (the inverted-bottleneck MLP after a 3x3x3 SubM conv).
"""
from __future__ import annotations

import numpy as np

import oracle

ACTS = ("none", "relu", "silu")


def activation(x, kind: str):
    """The activation in float64."""
    x = np.asarray(x, dtype=np.float64)
    if kind == "none":
        return x
    if kind == "relu":
        return np.where(x > 0.0, x, 0.0)
    if kind == "silu":
        # x * sigmoid(x) = x / (1 + exp(-x)); exp overflow at very negative x gives -0.
        with np.errstate(over="ignore"):
            return x / (1.0 + np.exp(-x))
    raise ValueError(kind)


def group_stats(x, coords, batch: int, groups: int):
    """(mean [batch, groups], var [batch, groups]) in float64 over the active sites of each
    batch entry and the channels of each group; entries without sites give mean 0, var 0."""
    x = np.asarray(x, dtype=np.float64)
    n, c = x.shape
    if c % groups:
        raise ValueError("channels must be a multiple of groups")
    gs = c // groups
    b_of = np.asarray(coords, dtype=np.int64).reshape(-1, 4)[:, 0]
    mean = np.zeros((batch, groups))
    var = np.zeros((batch, groups))
    for b in range(batch):
        rows = x[b_of == b]
        if len(rows) == 0:
            continue
        for g in range(groups):
            vals = rows[:, g * gs:(g + 1) * gs].ravel()
            m = vals.sum() / len(vals)
            mean[b, g] = m
            var[b, g] = ((vals - m) ** 2).sum() / len(vals)
    return mean, var


def group_norm(x, coords, batch: int, groups: int = 32, gamma=None, beta=None,
               eps: float = 1e-5, act: str = "none"):
    """act(group norm of x) in float64; gamma / beta default to 1 / 0."""
    x = np.asarray(x, dtype=np.float64)
    n, c = x.shape
    gs = c // groups
    mean, var = group_stats(x, coords, batch, groups)
    b_of = np.asarray(coords, dtype=np.int64).reshape(-1, 4)[:, 0]
    g_of = np.arange(c) // gs
    m = mean[b_of][:, g_of]
    v = var[b_of][:, g_of]
    y = (x - m) / np.sqrt(v + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    if beta is not None:
        y = y + np.asarray(beta, dtype=np.float64)
    return activation(y, act)


def conv_epilogue(x, w, bias, nbr, act: str = "none", residual=None, flip: bool = False):
    """act(SubMConv3d(x) + bias) + residual, float64."""
    y = activation(oracle.conv(x, w, bias, nbr, flip=flip), act)
    if residual is not None:
        y = y + np.asarray(residual, dtype=np.float64)
    return y


def linear_epilogue(x, w, bias, act: str = "none", residual=None):
    """act(x @ w + bias) + residual, float64 (the k=1 layer)."""
    y = activation(oracle.linear(x, w, bias), act)
    if residual is not None:
        y = y + np.asarray(residual, dtype=np.float64)
    return y


def round_bf16(x):
    """Each value rounded to bfloat16 (round to nearest, ties to even) and returned as float64:
    first to float32 (numpy's round to nearest even), then to the 8-bit significand of bf16 on
    the float32 bits.  This is where a layer that stores bf16 rounds its float32 result."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(f)
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    out[nan] = np.nan
    return out


def _keep(x):
    return x


def res_block(x, coords, batch: int, nbr, p: dict, groups: int = 32, eps: float = 1e-5,
              store=None):
    """The pre-norm residual block: p holds w1, b1, w2, b2 ([27, C, C] / [C]) and the norms'
    g1, be1, g2, be2 ([C]).  ``store`` rounds a layer's result where a chain keeps it in a
    narrower type (round_bf16 for bf16 storage: after each norm, after each convolution);
    None keeps float64 throughout."""
    st = store or _keep
    h = st(group_norm(x, coords, batch, groups, p["g1"], p["be1"], eps, "silu"))
    h = st(oracle.conv(h, p["w1"], p["b1"], nbr))
    h = st(group_norm(h, coords, batch, groups, p["g2"], p["be2"], eps, "silu"))
    return st(conv_epilogue(h, p["w2"], p["b2"], nbr, "none", x))


def layer_norm(x, gamma=None, beta=None, eps: float = 1e-6, act: str = "none"):
    """act(layer norm over each row's channels) in float64; gamma / beta default to 1 / 0."""
    x = np.asarray(x, dtype=np.float64)
    m = x.mean(axis=1, keepdims=True)
    v = ((x - m) ** 2).mean(axis=1, keepdims=True)
    y = (x - m) / np.sqrt(v + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    if beta is not None:
        y = y + np.asarray(beta, dtype=np.float64)
    return activation(y, act)


def convnext_block(x, nbr, p: dict, eps: float = 1e-6, store=None):
    """p holds w ([27, C, C]), b, ln_g, ln_b ([C]), w1 ([C, 4C]), b1, w2 ([4C, C]), b2.
    ``store`` as for res_block: applied after the convolution, the norm and each linear."""
    st = store or _keep
    h = st(oracle.conv(x, p["w"], p["b"], nbr))
    h = st(layer_norm(h, p["ln_g"], p["ln_b"], eps))
    h = st(linear_epilogue(h, p["w1"], p["b1"], "silu"))
    return st(linear_epilogue(h, p["w2"], p["b2"], "none", x))
