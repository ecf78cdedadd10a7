"""Seeded synthetic inputs for the submanifold 3x3x3 convolution workloads.

This module only draws inputs: active voxel coordinates, feature rows, weights
and biases.  It holds none of the method's arithmetic (no neighbour search, no
convolution); both the CPU oracle and the HIP path consume what it returns.

Workloads (the LATO.2 MLX port page, "Fleet benchmark", times the 128^3,
128-channel, ~10%-occupancy case; the other shapes exercise surfaces, batches
and large site counts):

  tiny       batch 1, 32^3, i.i.d. occupancy 0.10, C 16->16, fp32
  iid128     batch 1, 128^3, i.i.d. occupancy 0.10, C 128->128, bf16
  shell256   batch 1, 256^3, sites within 1 voxel of a random centred
             ellipsoid (semi-axes U[80,120]), C 64->64, bf16
  batch4     4 scenes on 64^3 with i.i.d. occupancy 5/10/20/30 %, k=3 64->128
             then k=1 128->128, bf16
  shell512   batch 1, 512^3, two-voxel-thick shell of a random centred
             ellipsoid (semi-axes U[180,240]), C 32->32, bf16

Recipe (stated once, used everywhere):
  * RNG: numpy default_rng(SeedSequence([2026, k])) for workload number k,
    spawned into five children in this fixed order: occupancy/axes, row
    shuffle, features, layer-1 weights, layer-2 weights.
  * i.i.d. occupancy: voxel active iff U[0,1) < p, drawn as one (G,G,G) array
    per scene.  Realised site counts vary with the seed and are reported.
  * Shell: F(p) = sum_i ((p_i - c)/a_i)^2 with c = (G-1)/2 on every axis; the
    first-order signed distance is d = (F - 1) / |grad F|; a voxel is active
    iff |d| <= 1 (a band two voxels thick).
  * Coordinates are int32 rows (b, x, y, z) in lexicographic order (as
    numpy.argwhere emits them); ``shuffle=True`` applies a seeded permutation.
  * Features: fp32 N(0,1); for bf16 workloads rounded to bf16 with
    round-to-nearest-even (torch's float->bfloat16 cast).
  * Weights: layout [K^3, Cin, Cout]; N(0, variance 1/(K^3*Cin)) in fp32, then
    bf16 for bf16 workloads.  Bias: fp32 zeros of length Cout.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np
import torch

__all__ = ["Layer", "Workload", "WORKLOADS", "make", "iid_occupancy", "shell_occupancy",
           "coords_from_occupancy", "random_features", "random_weight"]

SEED_ROOT = 2026


@dataclasses.dataclass
class Layer:
    ksize: int                    # 3 (SubMConv3d) or 1 (per-voxel linear)
    weight: torch.Tensor          # [ksize^3, cin, cout], fp32 or bf16, CPU
    bias: torch.Tensor            # [cout] fp32, CPU

    @property
    def cin(self) -> int:
        return int(self.weight.shape[1])

    @property
    def cout(self) -> int:
        return int(self.weight.shape[2])


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    grid: Tuple[int, int, int]
    coords: np.ndarray            # int32 [N, 4] (b, x, y, z)
    feats: torch.Tensor           # [N, Cin] fp32 or bf16, CPU
    layers: List[Layer]
    dtype: str                    # "f32" or "bf16"
    description: str

    @property
    def n(self) -> int:
        return int(self.coords.shape[0])


# name -> (index k used in the seed, description)
WORKLOADS = {
    "tiny": (1, "batch 1, 32^3 grid, i.i.d. occupancy 0.10, Cin=Cout=16, k=3, fp32"),
    "iid128": (2, "batch 1, 128^3 grid, i.i.d. occupancy 0.10, Cin=Cout=128, k=3, bf16"),
    "shell256": (3, "batch 1, 256^3 grid, |d|<=1 band around a centred ellipsoid, "
                    "semi-axes U[80,120], Cin=Cout=64, k=3, bf16"),
    "batch4": (4, "4 scenes on 64^3, i.i.d. occupancy 5/10/20/30%, k=3 64->128 "
                  "then k=1 128->128, bf16"),
    "shell512": (5, "batch 1, 512^3 grid, |d|<=1 band (two voxels thick) around a "
                    "centred ellipsoid, semi-axes U[180,240], Cin=Cout=32, k=3, bf16"),
}


def _rngs(k: int):
    ss = np.random.SeedSequence([SEED_ROOT, k])
    return [np.random.default_rng(c) for c in ss.spawn(5)]


def iid_occupancy(rng: np.random.Generator, grid, p: float) -> np.ndarray:
    """Boolean (Gx,Gy,Gz) array, each voxel active independently with probability p."""
    return rng.random(tuple(grid)) < p


def shell_occupancy(rng: np.random.Generator, g: int, axis_lo: float, axis_hi: float,
                    half_width: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """Boolean (g,g,g) band |d| <= half_width around an axis-aligned ellipsoid centred
    at (g-1)/2 with semi-axes drawn U[axis_lo, axis_hi].  Evaluated one x-slab at a time
    so that 512^3 fits in memory.  Returns (occupancy, semi_axes)."""
    a = rng.uniform(axis_lo, axis_hi, size=3)
    c = (g - 1) / 2.0
    ax = np.arange(g, dtype=np.float64)
    v = ((ax - c) / a[1])[:, None]
    w = ((ax - c) / a[2])[None, :]
    occ = np.zeros((g, g, g), dtype=bool)
    for x in range(g):
        u = (x - c) / a[0]
        F = u * u + v * v + w * w
        grad = 2.0 * np.sqrt((u / a[0]) ** 2 + (v / a[1]) ** 2 + (w / a[2]) ** 2)
        with np.errstate(divide="ignore", invalid="ignore"):
            d = (F - 1.0) / grad
        occ[x] = np.abs(d) <= half_width
    return occ, a


def coords_from_occupancy(occs: List[np.ndarray]) -> np.ndarray:
    """Stack per-scene occupancy arrays into int32 rows (b, x, y, z), lexicographic order."""
    rows = []
    for b, occ in enumerate(occs):
        pts = np.argwhere(occ).astype(np.int32)
        rows.append(np.concatenate([np.full((len(pts), 1), b, np.int32), pts], axis=1))
    if not rows:
        return np.zeros((0, 4), np.int32)
    return np.ascontiguousarray(np.concatenate(rows, axis=0))


def random_features(rng: np.random.Generator, n: int, c: int, dtype: str) -> torch.Tensor:
    x = torch.from_numpy(rng.standard_normal((n, c), dtype=np.float32))
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def random_weight(rng: np.random.Generator, ksize: int, cin: int, cout: int,
                  dtype: str) -> torch.Tensor:
    taps = ksize ** 3
    std = 1.0 / np.sqrt(taps * cin)
    w = torch.from_numpy((rng.standard_normal((taps, cin, cout)) * std).astype(np.float32))
    return w.to(torch.bfloat16) if dtype == "bf16" else w


def make(name: str, shuffle: bool = False, seed_offset: int = 0,
         with_feats: bool = True) -> Workload:
    """Build one named workload.  ``seed_offset`` draws another instance of the same
    recipe (used for several seeds in tests)."""
    k, desc = WORKLOADS[name]
    r_occ, r_perm, r_x, r_w1, r_w2 = _rngs(k + 1000 * seed_offset)
    if name == "tiny":
        grid, batch, dtype = (32, 32, 32), 1, "f32"
        occs = [iid_occupancy(r_occ, grid, 0.10)]
        specs = [(3, 16, 16)]
    elif name == "iid128":
        grid, batch, dtype = (128, 128, 128), 1, "bf16"
        occs = [iid_occupancy(r_occ, grid, 0.10)]
        specs = [(3, 128, 128)]
    elif name == "shell256":
        grid, batch, dtype = (256, 256, 256), 1, "bf16"
        occ, _ = shell_occupancy(r_occ, 256, 80.0, 120.0, 1.0)
        occs = [occ]
        specs = [(3, 64, 64)]
    elif name == "batch4":
        grid, batch, dtype = (64, 64, 64), 4, "bf16"
        occs = [iid_occupancy(r_occ, grid, p) for p in (0.05, 0.10, 0.20, 0.30)]
        specs = [(3, 64, 128), (1, 128, 128)]
    elif name == "shell512":
        grid, batch, dtype = (512, 512, 512), 1, "bf16"
        occ, _ = shell_occupancy(r_occ, 512, 180.0, 240.0, 1.0)
        occs = [occ]
        specs = [(3, 32, 32)]
    else:  # pragma: no cover
        raise KeyError(name)
    coords = coords_from_occupancy(occs)
    del occs
    if shuffle:
        coords = np.ascontiguousarray(coords[r_perm.permutation(len(coords))])
    n = len(coords)
    feats = random_features(r_x, n, specs[0][1], dtype) if with_feats else torch.empty(0)
    layers = []
    for (ks, ci, co), rw in zip(specs, (r_w1, r_w2)):
        layers.append(Layer(ks, random_weight(rw, ks, ci, co, dtype),
                            torch.zeros(co, dtype=torch.float32)))
    return Workload(name, batch, grid, coords, feats, layers, dtype, desc)


def random_sites(rng: np.random.Generator, batch: int, grid, n_per_scene: int) -> np.ndarray:
    """``n_per_scene`` distinct uniformly drawn voxels in each scene, lexicographic rows
    (b, x, y, z).  Used for small tests."""
    gx, gy, gz = grid
    rows = []
    for b in range(batch):
        flat = rng.choice(gx * gy * gz, size=n_per_scene, replace=False)
        flat.sort()
        x, rem = np.divmod(flat, gy * gz)
        y, z = np.divmod(rem, gz)
        rows.append(np.stack([np.full_like(x, b), x, y, z], axis=1))
    return np.ascontiguousarray(np.concatenate(rows).astype(np.int32))
