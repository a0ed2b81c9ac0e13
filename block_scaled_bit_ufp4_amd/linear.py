"""A linear layer whose three GEMMs run on 4-bit block-scaled operands.

Y = X W^T (fwd_y), dX = dY W (bwd_dx) and dW = dY^T X (bwd_dw), each GEMM on
operands quantized along its own contraction axis:

  fwd_y   X along K (rows of X), W along K (rows of W);
  bwd_dx  dY along N (rows of dY), W along N (columns of W);
  bwd_dw  dY along T (columns of dY), X along T (columns of X).

The recipes are those of the UFP4 page ("当你的 GPU 学不会算账", section
"UFP4：换一把尺子", recipe table): UFP4 quantizes every operand to E1M2 with an
FP32 scale per 1x16 block, applies the 16-wide RHT to all of them, and rounds
dY stochastically (its two quantizations on separate Philox streams). The E2M1
baseline uses E2M1 with the same blocks and scale, with the RHT only on the
bwd_dw operands. Every operand of one GEMM shares the RHT seed, so the rotation
cancels in the product. The GEMMs dequantize to bf16 and multiply on the bf16
MFMA, accumulating in fp32 (the software route for formats with no native
MFMA: "FP4 训练 vs FP4 推理", UFP4 section).

Every step runs in libufp4. torch provides device memory, and the conversion
of fp32 results to the caller's dtype for autograd.
"""
from dataclasses import dataclass
from typing import Optional

import torch

from . import Cfg, QTensor, ufp4_qgemm, ufp4_quantize


@dataclass(frozen=True)
class Recipe:
    """Format, scale, RHT coverage and SR of the three GEMMs' operands."""
    fmt: str = "e1m2"
    scale: str = "fp32"
    rht_fwd: bool = True      # X, W in fwd_y
    rht_dx: bool = True       # dY, W in bwd_dx
    rht_dw: bool = True       # dY, X in bwd_dw
    sr_dy: bool = True        # stochastic rounding of dY
    rht_seed: int = 0
    sr_seed: int = 0

    def cfg(self, rht: bool, axis: str, sr: bool = False, stream: int = 0) -> Cfg:
        return Cfg(self.fmt, self.scale, 16, rht="random" if rht else "none", rht_seed=self.rht_seed,
                   rounding="sr" if sr else "rtne", axis=axis, sr_seed=self.sr_seed, sr_stream=stream)


UFP4 = Recipe()
E2M1_BASELINE = Recipe(fmt="e2m1", rht_fwd=False, rht_dx=False, rht_dw=True)


def _gemm(a: QTensor, b: QTensor, out: Optional[torch.Tensor] = None,
          ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    return ufp4_qgemm(a, b, "bf16", c=out, ws=ws)


def operands_fwd(x: torch.Tensor, w: torch.Tensor, r: Recipe):
    """Quantized operands of fwd_y: X and W along K."""
    return (ufp4_quantize(x, r.cfg(r.rht_fwd, "row")), ufp4_quantize(w, r.cfg(r.rht_fwd, "row")))


def operands_dx(dy: torch.Tensor, w: torch.Tensor, r: Recipe):
    """Quantized operands of bwd_dx: dY along N (row view), W along N (column view)."""
    return (ufp4_quantize(dy, r.cfg(r.rht_dx, "row", r.sr_dy, 0)), ufp4_quantize(w, r.cfg(r.rht_dx, "col")))


def operands_dw(dy: torch.Tensor, x: torch.Tensor, r: Recipe):
    """Quantized operands of bwd_dw: dY along T and X along T (column views)."""
    return (ufp4_quantize(dy, r.cfg(r.rht_dw, "col", r.sr_dy, 1)), ufp4_quantize(x, r.cfg(r.rht_dw, "col")))


def linear_fwd(x: torch.Tensor, w: torch.Tensor, r: Recipe = UFP4) -> torch.Tensor:
    """Y = X W^T in fp32 from 4-bit operands; x [T][K], w [N][K] (bf16)."""
    return _gemm(*operands_fwd(x, w, r))


def linear_bwd(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, r: Recipe = UFP4):
    """dX = dY W and dW = dY^T X in fp32 from 4-bit operands."""
    return _gemm(*operands_dx(dy, w, r)), _gemm(*operands_dw(dy, x, r))


class UFP4LinearFunction(torch.autograd.Function):
    """Autograd function: forward and both backward GEMMs quantized per recipe."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, w: torch.Tensor, recipe: Recipe = UFP4):
        ctx.save_for_backward(x, w)
        ctx.recipe = recipe
        return linear_fwd(x, w, recipe).to(x.dtype)

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x, w = ctx.saved_tensors
        dx, dw = linear_bwd(dy.contiguous(), x, w, ctx.recipe)
        return dx.to(x.dtype), dw.to(w.dtype), None


def ufp4_linear(x: torch.Tensor, w: torch.Tensor, recipe: Recipe = UFP4) -> torch.Tensor:
    """Y = X W^T with the recipe's 4-bit GEMMs in forward and backward."""
    return UFP4LinearFunction.apply(x, w, recipe)
