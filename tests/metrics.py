"""Error measures and tolerance checks used by the parity tests (pure numpy).

Tolerances (fp32 accumulate, bf16 storage):
* y (fp32 output), da, dgamma: max|x - ref| / rms(ref) <= 1e-2;
* r: max_i |r_i / r_ref,i - 1| <= 1e-3;   s: max_i |s_i - s_ref,i| / rms(s_ref) <= 1e-3;
* bf16 outputs: bitwise equal to the round-to-nearest-even of the fp32 output of
  the same kernel, and |x - ref| <= 1e-2 rms(ref) + half a bf16 ulp of max(|x|, |ref|);
* h, g (bf16): |x - ref| <= one bf16 ulp of |ref| + 1e-6 rms(ref);
* dW1: the weight-gradient GEMM contracts over rows with r on the contraction
  index, so its bf16 operand r*g is rounded once before the MFMA (the reading of
  the weight gradient). Two checks: against the oracle's dW1 on the same rounded
  operand, within 1e-4 rms (the GEMM itself: fp32 accumulation only); and against
  the exact definition, within 1e-4 rms + SIGMA_K sigma of that rounding (below).
  Where dY is itself produced in fp32 and rounded to bf16 before the product (the
  SwiGLU backward), sigma also carries dY's rounding.
* SwiGLU o = silu(gate) up, computed from the fp32 y: with |y - y_ref| <= d =
  1e-2 rms(y_ref) elementwise, |silu'| <= 1.1 and |silu''| <= 0.5 (Taylor with
  remainder), |o - o_ref| <= d (1.1 |up| + |silu(gate)|) + d^2 (1.1 + 0.25 |up|)
  + 0.25 d^3, plus 1e-5 |o_ref| for the fp32 evaluation itself.
* dY of the SwiGLU backward and dW2 (plain products of bf16 operands with fp32
  accumulation, rounded once): within 1e-4 rms plus half a bf16 ulp.
* cross-entropy: lse and loss (fp32 logits of exact bf16 products, never rounded)
  within 1e-4 rms; dlogits (bf16) faithfully rounded: within one bf16 ulp of the
  exact value (+1e-4 rms), because the softmax makes a few elements much larger
  than the rms and their fp32 error, though far below an ulp, can tip the
  rounding; dh and dW within 1e-4 rms + SIGMA_K sigma of that rounding of
  dlogits before the two products.
* da and dgamma of the SwiGLU backward: dY is produced in fp32 and rounded to
  bf16 before G = dY @ W1^T: within 1e-4 rms + SIGMA_K sigma of that rounding.
"""
from __future__ import annotations

import numpy as np
import torch

Y_TOL = 1e-2
R_TOL = 1e-3
S_TOL = 1e-3


def f64(t) -> np.ndarray:
    if isinstance(t, (np.ndarray, np.generic, float, int)):
        return np.asarray(t, dtype=np.float64)
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


def bf16_faithful(x, ref, tol) -> float:
    """Largest |x - ref| / (ulp of max(|x|,|ref|) + tol rms(ref)); <= 1 passes: x is one of the two
    bf16 neighbours of ref (up to tol rms)."""
    x, ref = f64(x), f64(ref)
    bound = tol * rms(ref) + bf16_ulp(np.maximum(np.abs(x), np.abs(ref)))
    return float(np.max(np.abs(x - ref) / bound))


def bf16_one_ulp(x, ref) -> float:
    """Largest |x - ref| / (ulp(ref) + 1e-6 rms(ref)); <= 1 passes."""
    x, ref = f64(x), f64(ref)
    return float(np.max(np.abs(x - ref) / (bf16_ulp(ref) + 1e-6 * rms(ref))))


# Statistical bounds for a contraction whose operand was rounded to bf16 once, element by element
# (the weight gradient's bf16(r g); a gradient produced in fp32 and stored in bf16 before the next
# product). Each element's rounding error is uniform on [-u, u], u = half a bf16 ulp, independent of the
# others, so the error of C = A @ B has variance sum_k u_ik^2 / 3 B_kj^2 (central limit: Gaussian once a
# few terms add). The gates allow SIGMA_K = 6.5 of those sigmas: P(|Z| > 6.5) = 8e-11 per element, so
# a check over up to ~1e8 elements fails by chance with probability below 1 %, while a real error of the
# GEMM (a dropped term, a wrong row or column, a lost scale) lands tens to thousands of sigmas away. A
# single rounded term is at most sqrt(3) sigma, so the bound also covers a one-term contraction.
SIGMA_K = 6.5


def half_ulp_sq_over_3(a) -> np.ndarray:
    """u^2 / 3 (float32) for u = half a bf16 ulp of |a|: the variance of rounding a to bf16."""
    u = 0.5 * bf16_ulp(a)
    return (u * u / 3.0).astype(np.float32)


def rounding_sigma(var_a, B) -> np.ndarray:
    """sqrt(var_a @ B^2): the sigma of (A_rounded - A) @ B for per-element rounding variances var_a
    [R, K] and B [K, C] (float32 arithmetic: two significant digits are all a bound needs)."""
    Bs = np.asarray(f64(B), dtype=np.float32)
    return np.sqrt(np.asarray(var_a, dtype=np.float32) @ (Bs * Bs)).astype(np.float64)


def operand_rounding_sigma(g, r, dY, cols=None, dY_var=None, chunk=8192) -> np.ndarray:
    """[D, C] sigma of dW1 = bf16(r g)^T dY against the exact (r g)^T dY (columns `cols` of dW1), from
    the one rounding of r_i g_ij; with dY_var ([M, N] rounding variances of a dY that was itself rounded
    to bf16 from an exact value) also sum_i (r_i g_ij)^2 var(dY_in). Accumulated over blocks of rows."""
    idx = None if cols is None else np.asarray(cols)
    if idx is not None:   # the sampled columns first (dY may be a large torch tensor)
        dY = dY[:, idx] if isinstance(dY, np.ndarray) else dY[:, torch.as_tensor(idx)]
        if dY_var is not None:
            dY_var = dY_var[:, idx]
    var = None
    for i0 in range(0, g.shape[0], chunk):
        rg = f64(g[i0:i0 + chunk]) * f64(r[i0:i0 + chunk])[:, None]
        d = f64(dY[i0:i0 + chunk])
        v = half_ulp_sq_over_3(rg).T @ (d * d).astype(np.float32)
        if dY_var is not None:
            v += (rg * rg).astype(np.float32).T @ dY_var[i0:i0 + chunk]
        var = v if var is None else var + v
    return np.sqrt(var.astype(np.float64))


def dgrad_rounding_sigma(dY_var, W1, r, gamma, h, rows=None, cols=None) -> tuple:
    """(da [R, D], dgamma [C]) sigmas of rounding dY (variances dY_var [M, N]) before G = dY @ W1^T:
    sigma_G = sqrt(var_dY @ W1^T^2), da = r gamma G, dgamma_j = sum_i G_ij r_i h_ij (rows independent)."""
    W1t = f64(W1).T
    rd, ga = f64(r), np.abs(f64(gamma))
    ridx = np.arange(dY_var.shape[0]) if rows is None else np.asarray(rows)
    s_da = rd[ridx, None] * ga[None, :] * rounding_sigma(dY_var[ridx], W1t)
    jc = np.arange(W1t.shape[1]) if cols is None else np.asarray(cols)
    sG = rounding_sigma(dY_var, W1t[:, jc])
    s_dg = np.sqrt(((sG * rd[:, None] * f64(h)[:, jc]) ** 2).sum(axis=0))
    return s_da, s_dg


def within_sigma(x, ref, sigma, tol=1e-4, k=SIGMA_K) -> float:
    """Largest |x - ref| / (tol rms(ref) + k sigma); <= 1 passes. tol covers the fp32 accumulation."""
    x, ref = f64(x), f64(ref)
    return float(np.max(np.abs(x - ref) / (tol * rms(ref) + k * np.asarray(sigma))))


def within_allowance(x, ref, allow, tol=Y_TOL) -> float:
    """Largest |x - ref| / (tol rms(ref) + allow); <= 1 passes."""
    x, ref = f64(x), f64(ref)
    return float(np.max(np.abs(x - ref) / (tol * rms(ref) + allow)))


def swiglu_o_bound(y_ref, silu_gate, tol=Y_TOL) -> np.ndarray:
    """Per-element bound on o's error given y's elementwise error tol rms(y_ref)."""
    y = f64(y_ref)
    d = tol * rms(y)
    up, sg = np.abs(y[:, 1::2]), np.abs(f64(silu_gate))
    return d * (1.1 * up + sg) + d * d * (1.1 + 0.25 * up) + 0.25 * d ** 3 + 1e-5 * sg * up


def rne_bf16(t: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16 with torch's round-to-nearest-even."""
    return t.to(torch.bfloat16)
