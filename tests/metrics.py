"""Error measures and tolerance checks used by the parity tests (pure numpy).

Tolerances (fp32 accumulate, bf16 storage):
* y (fp32 output), da, dgamma: max|x - ref| / rms(ref) <= 1e-2;
* r: max_i |r_i / r_ref,i - 1| <= 1e-3;   s: max_i |s_i - s_ref,i| / rms(s_ref) <= 1e-3;
* bf16 outputs: bitwise equal to the round-to-nearest-even of the fp32 output of
  the same kernel, and |x - ref| <= 1e-2 rms(ref) + half a bf16 ulp of max(|x|, |ref|);
* h, g (bf16): |x - ref| <= one bf16 ulp of |ref| + 1e-6 rms(ref);
* dW1: the weight-gradient GEMM contracts over rows with r on the contraction
  index, so its bf16 operand r*g is rounded once before the MFMA. The bound is
  |x - ref| <= 1e-2 rms(ref) + sum_i ulp(r_i g_ij)/2 |dY_in| (the exact
  first-order effect of that one rounding); at M = 1 (a rank-1 product) nothing
  averages it and it alone exceeds 1e-2 rms.
"""
from __future__ import annotations

import numpy as np
import torch

Y_TOL = 1e-2
R_TOL = 1e-3
S_TOL = 1e-3


def f64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").to(torch.float64).numpy()


def rms(a) -> float:
    a = f64(a)
    return float(np.sqrt(np.mean(a * a)))


def normwise(x, ref) -> float:
    """max |x - ref| / rms(ref)."""
    x, ref = f64(x), f64(ref)
    return float(np.max(np.abs(x - ref)) / max(rms(ref), 1e-300))


def max_rel(x, ref) -> float:
    x, ref = f64(x), f64(ref)
    return float(np.max(np.abs(x / ref - 1.0)))


def bf16_ulp(a) -> np.ndarray:
    """Spacing of bf16 numbers at |a| (8 significant bits)."""
    a = np.abs(f64(a))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def bf16_within(x, ref, tol=Y_TOL) -> float:
    """Largest |x - ref| / (tol rms(ref) + ulp/2 of max(|x|,|ref|)); <= 1 passes."""
    x, ref = f64(x), f64(ref)
    bound = tol * rms(ref) + 0.5 * bf16_ulp(np.maximum(np.abs(x), np.abs(ref)))
    return float(np.max(np.abs(x - ref) / bound))


def bf16_one_ulp(x, ref) -> float:
    """Largest |x - ref| / (ulp(ref) + 1e-6 rms(ref)); <= 1 passes."""
    x, ref = f64(x), f64(ref)
    return float(np.max(np.abs(x - ref) / (bf16_ulp(ref) + 1e-6 * rms(ref))))


def operand_rounding_allowance(g, r, dY, cols=None) -> np.ndarray:
    """[D, C] bound sum_i ulp(r_i g_ij)/2 |dY_in| for the sampled columns n."""
    a = 0.5 * bf16_ulp(f64(g) * f64(r)[:, None])
    d = np.abs(f64(dY if cols is None else dY.index_select(1, torch.as_tensor(cols))))
    return a.T @ d


def within_allowance(x, ref, allow, tol=Y_TOL) -> float:
    """Largest |x - ref| / (tol rms(ref) + allow); <= 1 passes."""
    x, ref = f64(x), f64(ref)
    return float(np.max(np.abs(x - ref) / (tol * rms(ref) + allow)))


def rne_bf16(t: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16 with torch's round-to-nearest-even."""
    return t.to(torch.bfloat16)
