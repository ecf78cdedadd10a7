"""The pages' own designs for the submanifold convolution, rebuilt on this GPU so that the
compacted kernel (``subm_conv3d``) can be measured against them.  Comparison only: nothing in
the package's product path calls this module.

* ``dense_taps_plan`` -- the compacted kernel with its tap compaction switched off: every
  16-row block walks all 27 taps (missing neighbours read the zero row).  Same results bit for
  bit (the extra products are exact zeros); it isolates what skipping (block, tap) pairs
  without neighbours buys.
* ``DenseGemm`` -- one dense matmul over the 27 neighbour rows of every site side by side
  (LATO.2 MLX port page, "Fleet benchmark" version history): ``ssc_gather_taps`` builds the
  [N, 27 * Cin] operand, a library GEMM (torch -> hipBLASLt) multiplies it by the
  [27 * Cin, Cout] weights.
* ``PerOffset`` -- per tap: gather the rows that have that neighbour (``ssc_upsample2``), a
  library GEMM by W[t], scatter-add into fp32 outputs (``ssc_scatter_add_rows``): 27 x 3
  launches (trellis-mac article, gather-scatter flowchart; the LATO.2 page's per-offset loop).

The per-tap row lists of ``PerOffset`` are built once per coordinate set from the map (torch
``nonzero``, like the map itself outside the timed work).
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import (SSC_BF16, SSC_F32, TAPS, Plan, _check, _dtype_code, _need_cuda, _ptr, _stream,
               load_library)


def dense_taps_plan(plan: Plan) -> Plan:
    """A copy of ``plan`` whose block tap masks hold all 27 taps."""
    buf = plan.buf.clone()
    dense = Plan(buf, plan.n)
    _, bmask, _ = dense.parts()
    bmask.fill_((1 << TAPS) - 1)
    return dense


class DenseGemm:
    """The one-matmul design: Y = gather_taps(X) @ W.reshape(27 * Cin, Cout) (+ bias)."""

    def __init__(self, nbr: torch.Tensor, weight: torch.Tensor):
        _need_cuda(nbr, "nbr")
        self.nbr = nbr
        self.n = nbr.shape[0]
        self.cin, self.cout = weight.shape[1], weight.shape[2]
        self.w2 = weight.reshape(TAPS * self.cin, self.cout).contiguous()
        self.a = torch.empty((self.n, TAPS * self.cin), dtype=weight.dtype, device=nbr.device)

    def gather(self, x: torch.Tensor):
        lib = load_library()
        with torch.cuda.device(x.device):
            st = lib.ssc_gather_taps(_ptr(x), _dtype_code(x.dtype, "x"), self.n, self.cin,
                                     _ptr(self.nbr), _ptr(self.a), _stream(x.device))
        _check(st, "ssc_gather_taps")

    def gemm(self, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        return torch.matmul(self.a, self.w2, out=out)

    def __call__(self, x: torch.Tensor, bias: Optional[torch.Tensor] = None) -> torch.Tensor:
        """fp32 result: the GEMM's output (rounded once, to the GEMM's dtype) plus the bias."""
        self.gather(x)
        y = self.gemm().float()
        return y if bias is None else y + bias


class PerOffset:
    """The per-offset design: for each tap, gather -> GEMM -> scatter-add (fp32 outputs)."""

    def __init__(self, nbr: torch.Tensor, weight: torch.Tensor):
        _need_cuda(nbr, "nbr")
        self.n = nbr.shape[0]
        self.cin, self.cout = weight.shape[1], weight.shape[2]
        self.w = weight
        self.rows_out, self.rows_in = [], []
        for t in range(TAPS):
            i = torch.nonzero(nbr[:, t] >= 0).flatten()
            self.rows_out.append(i.to(torch.int32).contiguous())
            self.rows_in.append(nbr[i, t].to(torch.int32).contiguous())
        most = max(int(r.numel()) for r in self.rows_out)
        self.g = torch.empty((max(most, 1), self.cin), dtype=weight.dtype, device=nbr.device)
        self.part = torch.empty((max(most, 1), self.cout), dtype=weight.dtype,
                                device=nbr.device)

    def __call__(self, x: torch.Tensor, bias: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
        lib = load_library()
        dev = x.device
        dt = _dtype_code(x.dtype, "x")
        pdt = SSC_BF16 if self.part.dtype == torch.bfloat16 else SSC_F32
        if out is None:
            out = torch.empty((self.n, self.cout), dtype=torch.float32, device=dev)
        if bias is None:
            out.zero_()
        else:
            out.copy_(bias.expand(self.n, self.cout))
        st = _stream(dev)
        with torch.cuda.device(dev):
            for t in range(TAPS):
                p = int(self.rows_out[t].numel())
                if p == 0:
                    continue
                g, part = self.g[:p], self.part[:p]
                _check(lib.ssc_upsample2(_ptr(x), dt, self.cin, _ptr(self.rows_in[t]), p,
                                         self.n, _ptr(g), st), "ssc_upsample2")
                torch.matmul(g, self.w[t], out=part)
                _check(lib.ssc_scatter_add_rows(_ptr(part), pdt, _ptr(self.rows_out[t]), p,
                                                self.cout, _ptr(out), self.n, st),
                       "ssc_scatter_add_rows")
        return out
