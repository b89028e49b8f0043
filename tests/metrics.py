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
  averages it and it alone exceeds 1e-2 rms. Where dY is itself produced in fp32
  and rounded to bf16 before the product (the SwiGLU backward), the bound adds
  sum_i |r_i g_ij| ulp(dY_in)/2.
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
  rounding; dh and dW within 1e-4 rms plus sum ulp(dlogits) |W| (resp. |h|), the
  first-order effect of that rounding.
* da and dgamma of the SwiGLU backward: dY is produced in fp32 and rounded to
  bf16 before G = dY @ W1^T, so |dG_ij| <= A_ij = sum_n ulp(dY_in)/2 |W1_jn| and
  the bounds add r_i |gamma_j| A_ij (da) and sum_i r_i |h_ij| A_ij (dgamma).
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


def operand_rounding_allowance(g, r, dY, cols=None, dY_rounded=False, chunk=65536) -> np.ndarray:
    """[D, C] bound sum_i ulp(r_i g_ij)/2 |dY_in| for the sampled columns n; with
    dY_rounded (dY itself rounded to bf16 before the product, from an exact value)
    also sum_i |r_i g_ij| ulp(dY_in)/2. Accumulated over blocks of rows."""
    if cols is None:
        dYc = dY
    else:
        idx = np.asarray(cols)
        dYc = dY[:, idx] if isinstance(dY, np.ndarray) else dY[:, torch.as_tensor(idx)]
    allow = None
    for i0 in range(0, g.shape[0], chunk):
        rg = f64(g[i0:i0 + chunk]) * f64(r[i0:i0 + chunk])[:, None]
        d = f64(dYc[i0:i0 + chunk])
        a = (0.5 * bf16_ulp(rg)).T @ np.abs(d)
        if dY_rounded:
            a += np.abs(rg).T @ (0.5 * bf16_ulp(d))
        allow = a if allow is None else allow + a
    return allow


def dgrad_rounding_allowance(dY, W1, r, gamma, h, rows=None, cols=None) -> tuple:
    """(da [R, D], dgamma [C]) first-order bounds of the bf16 rounding of dY in G = dY @ W1^T."""
    u = 0.5 * bf16_ulp(dY)
    aw = np.abs(f64(W1))
    rd = f64(r)
    ridx = np.arange(u.shape[0]) if rows is None else np.asarray(rows)
    da = rd[ridx, None] * np.abs(f64(gamma))[None, :] * (u[ridx] @ aw.T)
    jc = np.arange(aw.shape[0]) if cols is None else np.asarray(cols)
    hd = f64(h)[:, jc]
    dg = ((u @ aw[jc].T) * rd[:, None] * np.abs(hd)).sum(axis=0)
    return da, dg


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
