"""CPU oracle for the coordinate-changing neighbours of the convolution: the factor-2 sparse
downsample with the max reduction, its paired upsample, and the x8 subdivide.

TEST INFRASTRUCTURE ONLY: imported by the tests and the benchmark's checks, never by the
product path.  Plain Python dictionaries and loops over numpy rows; it shares nothing with
the HIP library.

Definitions followed (LATO.2 MLX port page, "Status" and its module table; Pixal3D README,
module table):
  downsample  each site (b, x, y, z) belongs to the parent (b, x//2, y//2, z//2); the output
              sites are the distinct parents, in ascending (b, x, y, z) order (the ordering is
              this build's reading: the pages fix none); a parent's feature is the channel-wise
              maximum over the sites that belong to it ("max pool, not average").
  upsample    a site of the finer set takes the feature of its parent (the downsample's
              cached mapping, run backwards).
  spatial2channel  the downsample's parents, each holding its 8 children's features side by
              side (a sparse pixel unshuffle); absent children contribute zeros.
  subdivide   a site becomes its 8 children (b, 2x+dx, 2y+dy, 2z+dz), dx, dy, dz in {0, 1},
              listed as child 4dx + 2dy + dz of the site, each with the site's feature.
"""
from __future__ import annotations

import numpy as np


def downsample2(coords, batch: int, grid, feats=None):
    """Returns (parent coords [m, 4] int32, parent feats [m, C] or None, parent [n] int32,
    parent grid).  Raises ValueError on a site outside [0, batch) x grid."""
    c = np.asarray(coords, dtype=np.int64).reshape(-1, 4)
    n = len(c)
    children = {}
    for i in range(n):
        b, x, y, z = (int(v) for v in c[i])
        if not (0 <= b < batch and 0 <= x < grid[0] and 0 <= y < grid[1] and 0 <= z < grid[2]):
            raise ValueError(f"site {i} outside the grid")
        children.setdefault((b, x // 2, y // 2, z // 2), []).append(i)
    keys = sorted(children)
    parent = np.empty(n, dtype=np.int32)
    out_c = np.array(keys, dtype=np.int32).reshape(-1, 4)
    out_f = None
    if feats is not None:
        f = np.asarray(feats)
        out_f = np.empty((len(keys), f.shape[1]), dtype=f.dtype)
    for p, k in enumerate(keys):
        rows = children[k]
        parent[rows] = p
        if out_f is not None:
            out_f[p] = f[rows].max(axis=0)
    hgrid = tuple((int(g) + 1) // 2 for g in grid)
    return out_c, out_f, parent, hgrid


def spatial2channel2(coords, batch: int, grid, feats):
    """Parents as in downsample2; parent p's row has, for channel c of its child k (child
    (b, x, y, z) is k = 4(x%2) + 2(y%2) + z%2), the value at column c*8 + k, and zeros where
    a child is absent (the channel-major order torch's pixel_unshuffle uses; the pages fix
    no order)."""
    c = np.asarray(coords, dtype=np.int64).reshape(-1, 4)
    f = np.asarray(feats)
    out_c, _, parent, hgrid = downsample2(c, batch, grid)
    ch = f.shape[1]
    out_f = np.zeros((len(out_c), ch * 8), dtype=f.dtype)
    for i in range(len(c)):
        _, x, y, z = (int(v) for v in c[i])
        k = 4 * (x % 2) + 2 * (y % 2) + z % 2
        out_f[parent[i], k::8] = f[i]
    return out_c, out_f, parent, hgrid


def upsample2(parent_feats, parent):
    """out[i] = parent_feats[parent[i]]."""
    pf = np.asarray(parent_feats)
    return np.stack([pf[int(p)] for p in np.asarray(parent)]) if len(parent) else pf[:0]


def subdivide2(coords, grid, feats=None):
    """Returns (coords [8n, 4] int32, feats [8n, C] or None, doubled grid)."""
    c = np.asarray(coords, dtype=np.int64).reshape(-1, 4)
    n = len(c)
    out_c = np.empty((8 * n, 4), dtype=np.int32)
    f = None if feats is None else np.asarray(feats)
    out_f = None if f is None else np.empty((8 * n, f.shape[1]), dtype=f.dtype)
    for i in range(n):
        b, x, y, z = (int(v) for v in c[i])
        for dx in (0, 1):
            for dy in (0, 1):
                for dz in (0, 1):
                    k = 8 * i + 4 * dx + 2 * dy + dz
                    out_c[k] = (b, 2 * x + dx, 2 * y + dy, 2 * z + dz)
                    if out_f is not None:
                        out_f[k] = f[i]
    return out_c, out_f, tuple(2 * int(g) for g in grid)
