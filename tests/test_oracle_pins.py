"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test fixes the oracle against mathematics the pages determine: exact
rational / 50-digit arithmetic on tiny inputs, a different library's RMSNorm and
autograd, finite differences, closed forms, invariants of the backward, the
reparameterisation identity (hotdry blog, section "GEMM-Residual-RMSNorm-GEMM
重参数化": r is a row scalar and commutes with the second GEMM), and
hand-worked examples under tests/golden/.
"""
import json
import os
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

from oracle import coda_oracle as orc
from transformer_gemm_epilogue_res_amd import inputs

mpmath.mp.dps = 50
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _rng_int(shape, lo, hi, seed):
    return np.random.default_rng(seed).integers(lo, hi + 1, size=shape).astype(np.float64)


def _relerr(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- brute force

def _exact_forward(x, W0, z, gamma, W1, eps):
    """Forward with Fractions for the rational steps and 50-digit mpmath for the root."""
    M, K0 = x.shape
    D, N = W1.shape
    F = lambda v: Fraction(v).limit_denominator(10**12)  # noqa: E731  inputs are small dyadics
    h = [[sum(F(x[i, k]) * F(W0[k, j]) for k in range(K0)) + F(z[i, j]) for j in range(D)] for i in range(M)]
    out_r, out_y = [], []
    for i in range(M):
        ms = sum(v * v for v in h[i]) / D
        r = 1 / mpmath.sqrt(mpmath.mpf(ms.numerator) / ms.denominator + mpmath.mpf(eps))
        n = [r * mpmath.mpf(F(h[i][j]).numerator) / F(h[i][j]).denominator * mpmath.mpf(gamma[j]) for j in range(D)]
        y = [mpmath.fsum(n[j] * mpmath.mpf(W1[j, c]) for j in range(D)) for c in range(N)]
        out_r.append(r)
        out_y.append(y)
    hf = np.array([[float(v) for v in row] for row in h])
    return hf, np.array([float(v) for v in out_r]), np.array([[float(v) for v in row] for row in out_y])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_forward_brute_force_exact(seed):
    M, K0, D, N = 2, 4, 4, 3
    x = _rng_int((M, K0), -3, 3, seed)
    W0 = _rng_int((K0, D), -2, 2, seed + 10) / 2
    z = _rng_int((M, D), -3, 3, seed + 20)
    gamma = 1 + _rng_int((D,), -2, 2, seed + 30) / 8
    W1 = _rng_int((D, N), -3, 3, seed + 40) / 4
    eps = 1e-5
    h, r, y = _exact_forward(x, W0, z, gamma, W1, eps)
    o = orc.forward(x, W0, z, gamma, W1, eps)
    assert _relerr(o["h"], h) == 0.0          # small dyadic rationals: exact in fp64
    assert _relerr(o["r"], r) < 1e-15
    assert _relerr(o["y"], y) < 1e-14


def _exact_backward_by_derivative(x, W0, z, gamma, W1, dY, eps):
    """dL/dh, dL/dgamma, dL/dW1 for L = <dY, y> by 50-digit numerical differentiation.

    This uses no backward formula: L is re-evaluated from the forward definition
    and differentiated by mpmath.diff (Richardson-extrapolated differences).
    """
    M, D = z.shape
    N = W1.shape[1]
    h0 = [[mpmath.mpf(float(v)) for v in row] for row in (x @ W0 + z)]
    g0 = [mpmath.mpf(float(v)) for v in gamma]
    w0 = [[mpmath.mpf(float(v)) for v in row] for row in W1]
    dy = [[mpmath.mpf(float(v)) for v in row] for row in dY]

    def L(h, g, w):
        tot = mpmath.mpf(0)
        for i in range(M):
            ms = mpmath.fsum(v * v for v in h[i]) / D
            r = 1 / mpmath.sqrt(ms + eps)
            n = [r * h[i][j] * g[j] for j in range(D)]
            for c in range(N):
                tot += dy[i][c] * mpmath.fsum(n[j] * w[j][c] for j in range(D))
        return tot

    def dh(i, j):
        def f(t):
            h = [row[:] for row in h0]
            h[i][j] = t
            return L(h, g0, w0)
        return mpmath.diff(f, h0[i][j])

    def dg(j):
        def f(t):
            g = g0[:]
            g[j] = t
            return L(h0, g, w0)
        return mpmath.diff(f, g0[j])

    def dw(j, c):
        def f(t):
            w = [row[:] for row in w0]
            w[j][c] = t
            return L(h0, g0, w)
        return mpmath.diff(f, w0[j][c])

    da = np.array([[float(dh(i, j)) for j in range(D)] for i in range(M)])
    dgam = np.array([float(dg(j)) for j in range(D)])
    dW1 = np.array([[float(dw(j, c)) for c in range(N)] for j in range(D)])
    return da, dgam, dW1


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_brute_force_derivative(seed):
    M, K0, D, N = 2, 3, 4, 3
    x = _rng_int((M, K0), -3, 3, seed)
    W0 = _rng_int((K0, D), -2, 2, seed + 10) / 2
    z = _rng_int((M, D), -3, 3, seed + 20)
    gamma = 1 + _rng_int((D,), -2, 2, seed + 30) / 8
    W1 = _rng_int((D, N), -3, 3, seed + 40) / 4
    dY = _rng_int((M, N), -3, 3, seed + 50)
    eps = 1e-5
    f = orc.forward(x, W0, z, gamma, W1, eps)
    b = orc.backward(dY, f["y"], f["h"], f["h"] * gamma[None, :], f["r"], gamma, W1)
    da, dgam, dW1 = _exact_backward_by_derivative(x, W0, z, gamma, W1, dY, eps)
    assert _relerr(b["da"], da) < 1e-12
    assert _relerr(b["dgamma"], dgam) < 1e-12
    assert _relerr(b["dW1"], dW1) < 1e-12
    # G and s from their definitions in exact arithmetic
    assert _relerr(b["G"], dY @ W1.T) == 0.0


# ------------------------------------------------------------- plain product

def _bf16_dyadics(shape, seed):
    """bf16 tensor of m * 2^e with |m| < 256 (8 significant bits, exact in bf16), e in [-4, 4]."""
    g = np.random.default_rng(seed)
    m = g.integers(-255, 256, size=shape).astype(np.float64)
    e = g.integers(-4, 5, size=shape).astype(np.float64)
    t = torch.from_numpy(m * 2.0 ** e).to(torch.bfloat16)
    assert torch.equal(t.double(), torch.from_numpy(m * 2.0 ** e))   # exactly representable
    return t


def _fraction_product(A, B):
    a = [[Fraction(float(v)) for v in row] for row in A.double().tolist()]
    b = [[Fraction(float(v)) for v in row] for row in B.double().tolist()]
    return np.array([[float(sum(a[i][k] * b[k][j] for k in range(len(b)))) for j in range(len(b[0]))]
                     for i in range(len(a))])


@pytest.mark.parametrize("a_col", [False, True], ids=["A_row", "A_col"])
@pytest.mark.parametrize("b_col", [False, True], ids=["B_row", "B_col"])
@pytest.mark.parametrize("shape", [(3, 5, 2), (7, 4, 6)])
def test_gemm_exact_in_every_storage_layout(a_col, b_col, shape):
    """oracle.gemm (the checker of the plain-mainloop GPU test) is the exact product A @ B of the
    logical operands, whichever way they are stored: a row-major tensor, or the transposed view of a
    column-major one. The sizes differ pairwise, so a transposed operand or a wrong contraction axis
    fails on shape or value; the operands carry 8 significant bits at exponents -4..4, so a widening
    that drops mantissa bits or sign changes the exact rational result (every partial sum is exact in
    fp64, so the comparison is equality)."""
    M, K, N = shape
    A = _bf16_dyadics((M, K), 100 + M)
    B = _bf16_dyadics((K, N), 200 + N)
    A_view = A.t().contiguous().t() if a_col else A          # stored [K, M], read as its transpose
    B_view = B.t().contiguous().t() if b_col else B          # stored [N, K], read as its transpose
    assert A_view.is_contiguous() == (not a_col) and B_view.is_contiguous() == (not b_col)
    want = _fraction_product(A, B)
    got = orc.gemm(A_view, B_view)
    assert got.shape == (M, N)
    assert np.array_equal(got, want)
    assert np.array_equal(orc.gemm(A.double().numpy(), B.double().numpy()), want)   # ndarray inputs
    with pytest.raises(ValueError):
        orc.gemm(A_view, B_view.t())                           # a transposed B cannot multiply


# ----------------------------------------------------------- bf16 rounding

def test_bf16_round_matches_torch_conversion():
    """bf16_round against torch's float32 -> bfloat16 conversion (a separate implementation) on random
    values over the whole exponent range, exact ties with an even and an odd kept bit, subnormals,
    +-0, +-inf, NaN and the largest floats (which round to inf); float64 inputs go through float32
    first, as a kernel's fp32 value does."""
    g = np.random.default_rng(0)
    bits = g.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    ties = (g.integers(0, 2 ** 16, size=4000, dtype=np.uint64).astype(np.uint32) << 16) | np.uint32(0x8000)
    special = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000,
                        0x00000001, 0x00008000, 0x00018000, 0x007FFFFF, 0x3F808000, 0x3F818000], dtype=np.uint32)
    x32 = np.concatenate([bits, ties, special]).view(np.float32)
    want = torch.from_numpy(x32.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = orc.bf16_round(x32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    x64 = g.standard_normal(100000) * 10.0 ** g.integers(-30, 30, size=100000)
    want64 = torch.from_numpy(x64).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.bf16_round(x64), want64)


def test_backward_rounded_operand_and_given_s():
    """The backward's two options: round_rg (dW1 from bf16(r g)) equals the exact dW1 when r g is a bf16
    value already (r a power of two), and otherwise differs from it by exactly (bf16(r g) - r g)^T dY,
    with the rounding computed by torch (within the first-order bound sum_i ulp(r g)/2 |dY|); a given s
    equal to sum dY y changes nothing, and da is affine in s with slope -r^2 h / D."""
    M, D, N = 40, 16, 24
    gen = torch.Generator().manual_seed(3)
    bf = torch.bfloat16
    dY, y = torch.randn(M, N, generator=gen).to(bf), torch.randn(M, N, generator=gen).to(bf)
    h = torch.randn(M, D, generator=gen).to(bf)
    gamma = (1 + 0.1 * torch.randn(D, generator=gen)).to(bf)
    g = (h.double() * gamma.double()).to(bf)
    W1 = (torch.randn(D, N, generator=gen) / 4).to(bf)
    r2 = torch.full((M,), 0.5, dtype=torch.float32)
    a = orc.backward(dY, y, h, g, r2, gamma, W1)
    b = orc.backward(dY, y, h, g, r2, gamma, W1, round_rg=True)
    assert np.array_equal(a["dW1"], b["dW1"])
    r = (0.5 + torch.rand(M, generator=gen)).to(torch.float32)
    a = orc.backward(dY, y, h, g, r, gamma, W1)
    b = orc.backward(dY, y, h, g, r, gamma, W1, round_rg=True)
    rg32 = r[:, None] * g.float()                       # torch's fp32 product
    delta = (rg32.to(bf).double() - r.double()[:, None] * g.double()).numpy()
    assert np.allclose(b["dW1"] - a["dW1"], delta.T @ dY.double().numpy(), rtol=0, atol=1e-12)
    rg = (r.double()[:, None] * g.double()).abs().numpy()
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(rg, 2.0 ** -126))) - 7)
    assert np.all(np.abs(b["dW1"] - a["dW1"]) <= (0.5 * ulp).T @ np.abs(dY.double().numpy()) + 1e-12)
    assert np.abs(b["dW1"] - a["dW1"]).max() > 0
    c = orc.backward(dY, y, h, g, r, gamma, W1, s=a["s"])
    for k in ("s", "G", "da", "dgamma", "dW1"):
        assert np.array_equal(c[k], a[k]), k
    s2 = a["s"] + np.arange(M)
    d = orc.backward(dY, y, h, g, r, gamma, W1, s=s2)
    assert np.allclose(d["da"] - a["da"], -(np.arange(M) * r.double().numpy() ** 2)[:, None] * h.double().numpy() / D,
                       rtol=0, atol=1e-12)
    assert np.array_equal(d["dgamma"], a["dgamma"]) and np.array_equal(d["dW1"], a["dW1"])


# --------------------------------------------------------- library special case

def _rand_problem(M, K0, D, N, seed, eps=1e-5):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, K0, generator=g, dtype=torch.float64)
    W0 = torch.randn(K0, D, generator=g, dtype=torch.float64) / K0 ** 0.5
    z = torch.randn(M, D, generator=g, dtype=torch.float64)
    gamma = 1 + 0.1 * torch.randn(D, generator=g, dtype=torch.float64)
    W1 = torch.randn(D, N, generator=g, dtype=torch.float64) / D ** 0.5
    dY = torch.randn(M, N, generator=g, dtype=torch.float64)
    return x, W0, z, gamma, W1, dY, eps


def test_forward_matches_torch_rms_norm():
    x, W0, z, gamma, W1, _, eps = _rand_problem(16, 32, 48, 40, 0)
    h = x @ W0 + z
    y_ref = torch.nn.functional.rms_norm(h, (h.shape[1],), gamma, eps) @ W1
    o = orc.forward(x, W0, z, gamma, W1, eps)
    assert _relerr(o["y"], y_ref.numpy()) < 1e-12
    assert _relerr(o["h"], h.numpy()) < 1e-14


def test_backward_matches_torch_autograd():
    x, W0, z, gamma, W1, dY, eps = _rand_problem(12, 24, 32, 40, 1)
    h = (x @ W0 + z).requires_grad_(True)
    gam = gamma.clone().requires_grad_(True)
    W = W1.clone().requires_grad_(True)
    y = torch.nn.functional.rms_norm(h, (h.shape[1],), gam, eps) @ W
    (y * dY).sum().backward()
    f = orc.forward(x, W0, z, gamma, W1, eps)
    b = orc.backward(dY, f["y"], f["h"], f["h"] * gamma.numpy()[None, :], f["r"], gamma, W1)
    assert _relerr(b["da"], h.grad.numpy()) < 1e-10
    assert _relerr(b["dgamma"], gam.grad.numpy()) < 1e-10
    assert _relerr(b["dW1"], W.grad.numpy()) < 1e-10


def test_backward_through_gemm0_matches_torch_autograd():
    # the whole chain in float64 autograd: x, W0, z are leaves; the oracle composes
    # backward (da) with backward_gemm0 (dx, dW0, dz = da)
    x, W0, z, gamma, W1, dY, eps = _rand_problem(12, 24, 32, 40, 9)
    xl, wl, zl = (t.clone().requires_grad_(True) for t in (x, W0, z))
    h = xl @ wl + zl
    y = torch.nn.functional.rms_norm(h, (h.shape[1],), gamma, eps) @ W1
    (y * dY).sum().backward()
    f = orc.forward(x, W0, z, gamma, W1, eps)
    b = orc.backward(dY, f["y"], f["h"], f["h"] * gamma.numpy()[None, :], f["r"], gamma, W1)
    b0 = orc.backward_gemm0(b["da"], x, W0)
    assert _relerr(b0["dx"], xl.grad.numpy()) < 1e-10
    assert _relerr(b0["dW0"], wl.grad.numpy()) < 1e-10
    assert _relerr(b0["dz"], zl.grad.numpy()) < 1e-10


def test_backward_through_gemm0_finite_differences_and_subsets():
    M, K0, D, N = 6, 8, 16, 12
    x, W0, z, gamma, W1, dY, eps = (t.numpy() if isinstance(t, torch.Tensor) else t
                                     for t in _rand_problem(M, K0, D, N, 10))
    f = orc.forward(x, W0, z, gamma, W1, eps)
    b = orc.backward(dY, f["y"], f["h"], f["h"] * gamma[None, :], f["r"], gamma, W1)
    b0 = orc.backward_gemm0(b["da"], x, W0)

    def L(xx, ww):
        return float((orc.forward(xx, ww, z, gamma, W1, eps)["y"] * dY).sum())

    step = 1e-6
    rng = np.random.default_rng(1)
    for _ in range(20):
        i, k = rng.integers(M), rng.integers(K0)
        xp, xm = x.copy(), x.copy()
        xp[i, k] += step
        xm[i, k] -= step
        fd = (L(xp, W0) - L(xm, W0)) / (2 * step)
        assert abs(fd - b0["dx"][i, k]) <= 1e-7 * max(1.0, abs(fd))
        k, j = rng.integers(K0), rng.integers(D)
        wp, wm = W0.copy(), W0.copy()
        wp[k, j] += step
        wm[k, j] -= step
        fd = (L(x, wp) - L(x, wm)) / (2 * step)
        assert abs(fd - b0["dW0"][k, j]) <= 1e-7 * max(1.0, abs(fd))
    part = orc.backward_gemm0(b["da"], x, W0, rows=[1, 4], dw0_cols=[0, 9, 15])
    assert np.allclose(part["dx"], b0["dx"][[1, 4]], rtol=0, atol=1e-13)
    assert np.allclose(part["dW0"], b0["dW0"][:, [0, 9, 15]], rtol=0, atol=1e-13)


# --------------------------------------------------------------------- SwiGLU

def test_silu_closed_forms_and_torch():
    # silu(0) = 0, silu(1) = e / (1 + e), silu(v) -> v and silu(-v) -> 0 for large v; torch's silu in fp64
    assert orc.silu(0.0) == 0.0
    e = float(mpmath.e)
    assert abs(orc.silu(1.0) - e / (1 + e)) < 1e-15
    assert abs(orc.silu(40.0) - 40.0) < 1e-12 and abs(orc.silu(-40.0)) < 1e-15
    v = torch.linspace(-12, 12, 2001, dtype=torch.float64)
    assert _relerr(orc.silu(v.numpy()), torch.nn.functional.silu(v).numpy()) < 1e-15


def test_swiglu_pairs_interleaved_columns():
    # column 2f is the gate and 2f+1 the up value of feature f
    y = np.array([[1.0, 2.0, 0.0, 5.0, -3.0, 0.5]])
    e = float(mpmath.e)
    want = [e / (1 + e) * 2.0, 0.0, orc.silu(-3.0) * 0.5]
    assert np.allclose(orc.swiglu(y)[0], want, rtol=0, atol=1e-15)
    # hand-derived backward of one pair (gate 1, up 2) for dO = 1: d/dgate = up silu'(1), d/dup = silu(1),
    # silu'(1) = sig(1) (1 + 1 - sig(1)) with sig(1) = e / (1 + e)
    sg = e / (1 + e)
    W2 = np.array([[1.0]])
    b = orc.swiglu_backward(np.array([[1.0]]), W2, y[:, :2], orc.swiglu(y[:, :2]))
    assert abs(b["dY"][0, 0] - 2.0 * sg * (2.0 - sg)) < 1e-15
    assert abs(b["dY"][0, 1] - sg) < 1e-15


def test_swiglu_block_backward_matches_torch_autograd():
    # the whole block in float64 autograd: h -> rms_norm -> @W1 -> swiglu -> @W2, L = <dOut, out>;
    # the oracle composes swiglu_backward (dY, s, dW2) with the chain's backward (da, dgamma, dW1)
    x, W0, z, gamma, W1, _, eps = _rand_problem(12, 24, 32, 40, 11)
    g = torch.Generator().manual_seed(11)
    W2 = torch.randn(20, 28, generator=g, dtype=torch.float64) / np.sqrt(20)
    dOut = torch.randn(12, 28, generator=g, dtype=torch.float64)
    h = (x @ W0 + z).requires_grad_(True)
    gam, w1, w2 = (t.clone().requires_grad_(True) for t in (gamma, W1, W2))
    y = torch.nn.functional.rms_norm(h, (h.shape[1],), gam, eps) @ w1
    y.retain_grad()
    o = torch.nn.functional.silu(y[:, 0::2]) * y[:, 1::2]
    ((o @ w2) * dOut).sum().backward()
    f = orc.forward(x, W0, z, gamma, W1, eps)
    of = orc.swiglu(f["y"])
    assert _relerr(of, o.detach().numpy()) < 1e-13
    sb = orc.swiglu_backward(dOut, W2, f["y"], of)
    assert _relerr(sb["dY"], y.grad.numpy()) < 1e-10
    assert _relerr(sb["dW2"], w2.grad.numpy()) < 1e-10
    b = orc.backward(sb["dY"], f["y"], f["h"], f["h"] * gamma.numpy()[None, :], f["r"], gamma, W1)
    assert _relerr(b["s"], sb["s"]) < 1e-13
    assert _relerr(b["da"], h.grad.numpy()) < 1e-10
    assert _relerr(b["dgamma"], gam.grad.numpy()) < 1e-10
    assert _relerr(b["dW1"], w1.grad.numpy()) < 1e-10


def test_swiglu_backward_finite_differences_and_subsets():
    rng = np.random.default_rng(3)
    M, F, E = 5, 6, 7
    y = rng.standard_normal((M, 2 * F)) * 2
    W2 = rng.standard_normal((F, E))
    dOut = rng.standard_normal((M, E))
    b = orc.swiglu_backward(dOut, W2, y, orc.swiglu(y))

    def L(yy):
        return float(((orc.swiglu(yy) @ W2) * dOut).sum())

    step = 1e-6
    for _ in range(30):
        i, n = rng.integers(M), rng.integers(2 * F)
        yp, ym = y.copy(), y.copy()
        yp[i, n] += step
        ym[i, n] -= step
        fd = (L(yp) - L(ym)) / (2 * step)
        assert abs(fd - b["dY"][i, n]) <= 1e-7 * max(1.0, abs(fd))
    part = orc.swiglu_backward(dOut, W2, y, orc.swiglu(y), rows=[0, 3], dw2_cols=[1, 6])
    for k in ("dO", "dY", "s"):
        assert np.allclose(part[k], b[k][[0, 3]], rtol=0, atol=1e-13)
    assert np.allclose(part["dW2"], b["dW2"][:, [1, 6]], rtol=0, atol=1e-13)


# ------------------------------------------------------------ finite differences

# ------------------------------------------------------- cross-entropy (LM head)

def _ce_problem(M, D, V, seed, scale=2.0):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(M, D, generator=g).to(torch.bfloat16)
    W = (torch.randn(V, D, generator=g) * (scale / D ** 0.5)).to(torch.bfloat16)
    t = torch.randint(0, V, (M,), generator=g)
    return h, W, t


def test_cross_entropy_matches_torch():
    h, W, t = _ce_problem(24, 64, 300, 1)
    t[3] = -100                                    # torch's ignore index
    ref = orc.lm_head_cross_entropy(h, W, t)
    L = h.double() @ W.double().T
    want = torch.nn.functional.cross_entropy(L, t, reduction="none", ignore_index=-100)
    assert _relerr(ref["loss"], want.numpy()) < 1e-14
    assert _relerr(ref["lse"], torch.logsumexp(L, dim=1).numpy()) < 1e-14
    assert ref["loss"][3] == 0.0 and not ref["valid"][3]
    # any target outside [0, V) is an ignored row
    t2 = t.clone()
    t2[5] = 300
    assert orc.lm_head_cross_entropy(h, W, t2)["loss"][5] == 0.0


def test_cross_entropy_brute_force_and_closed_forms():
    # 50-digit log-sum-exp on small integer logits
    rng = np.random.default_rng(3)
    L = rng.integers(-30, 31, size=(4, 9)).astype(np.float64)
    t = np.array([0, 8, 4, 2])
    r = orc.cross_entropy_logits(L, t)
    for i in range(4):
        lse = mpmath.log(mpmath.fsum(mpmath.e ** mpmath.mpf(v) for v in L[i]))
        assert abs(float(lse) - r["lse"][i]) <= 1e-14 * abs(float(lse))
        assert abs(float(lse - mpmath.mpf(L[i, t[i]])) - r["loss"][i]) <= 1e-13
    # uniform logits: loss = lse = log V
    V = 1000
    r = orc.cross_entropy_logits(np.full((2, V), 3.25), [7, 999])
    assert np.allclose(r["loss"], np.log(V), rtol=0, atol=1e-13)
    assert np.allclose(r["lse"], 3.25 + np.log(V), rtol=0, atol=1e-13)
    # one dominant target logit: loss = log(1 + (V - 1) e^-s), to the rounding of lse (~ulp(s))
    Ld = np.zeros((1, V))
    for sh in (5.0, 50.0):
        Ld[0, 17] = sh
        got = orc.cross_entropy_logits(Ld, [17])["loss"][0]
        assert abs(got - np.log1p((V - 1) * np.exp(-sh))) <= 4 * np.spacing(sh)
    # shift invariance per row, no overflow at large logits
    L = rng.standard_normal((3, 50)) * 4
    a = orc.cross_entropy_logits(L, [1, 2, 3])
    b = orc.cross_entropy_logits(L + np.array([[1000.0], [-1000.0], [0.5]]), [1, 2, 3])
    assert np.all(np.isfinite(b["loss"])) and np.allclose(a["loss"], b["loss"], rtol=0, atol=1e-10)


def test_cross_entropy_backward_matches_torch_autograd():
    h, W, t = _ce_problem(20, 64, 260, 2)
    t[0] = -100
    dloss = torch.randn(20, generator=torch.Generator().manual_seed(5), dtype=torch.float64)
    hd, Wd = h.double().requires_grad_(), W.double().requires_grad_()
    loss = torch.nn.functional.cross_entropy(hd @ Wd.T, t, reduction="none", ignore_index=-100)
    (loss * dloss).sum().backward()
    f = orc.lm_head_cross_entropy(h, W, t)
    b = orc.lm_head_cross_entropy_backward(h, W, t, f["lse"], dloss)
    assert _relerr(b["dh"], hd.grad.numpy()) < 1e-12
    assert _relerr(b["dW"], Wd.grad.numpy()) < 1e-12
    # gradient rows of valid targets sum to zero; ignored rows are zero; dloss = 0 gives zero gradients
    assert np.max(np.abs(b["dlogits"][1:].sum(axis=1))) < 1e-14
    assert np.all(b["dlogits"][0] == 0)
    z = orc.lm_head_cross_entropy_backward(h, W, t, f["lse"], np.zeros(20))
    assert not np.any(z["dh"]) and not np.any(z["dW"])


def test_cross_entropy_backward_finite_differences_and_subsets():
    h, W, t = _ce_problem(6, 16, 40, 4)
    dloss = np.random.default_rng(6).standard_normal(6)
    hd, Wd = orc.f64(h), orc.f64(W)

    def total(hh, WW):
        return float((orc.cross_entropy_logits(hh @ WW.T, t.numpy())["loss"] * dloss).sum())

    f = orc.lm_head_cross_entropy(h, W, t)
    b = orc.lm_head_cross_entropy_backward(h, W, t, f["lse"], dloss)
    e = 1e-6
    for (i, j) in ((0, 0), (3, 7), (5, 15)):
        hp, hm = hd.copy(), hd.copy()
        hp[i, j] += e
        hm[i, j] -= e
        assert abs((total(hp, Wd) - total(hm, Wd)) / (2 * e) - b["dh"][i, j]) < 1e-7
    for (v, j) in ((0, 0), (int(t[2]), 3), (39, 15)):
        Wp, Wm = Wd.copy(), Wd.copy()
        Wp[v, j] += e
        Wm[v, j] -= e
        assert abs((total(hd, Wp) - total(hd, Wm)) / (2 * e) - b["dW"][v, j]) < 1e-7
    # row and vocabulary-row subsets equal the full computation
    rows, vr = [1, 4], [0, 17, 39]
    fs = orc.lm_head_cross_entropy(h, W, t, rows=rows)
    assert np.array_equal(fs["loss"], f["loss"][rows]) and np.array_equal(fs["lse"], f["lse"][rows])
    bs = orc.lm_head_cross_entropy_backward(h, W, t, f["lse"], dloss, rows=rows, dw_rows=vr)
    assert np.allclose(bs["dh"], b["dh"][rows], rtol=0, atol=1e-15)
    assert np.allclose(bs["dlogits"], b["dlogits"][rows], rtol=0, atol=1e-15)
    assert np.allclose(bs["dW"], b["dW"][vr], rtol=0, atol=1e-14)
    # dlogits on a (row, vocabulary-column) block equals that block of the full backward's dlogits,
    # whose dh and dW pass the finite differences above
    blk = orc.lm_head_dlogits(h, W, t, f["lse"], dloss, rows=rows, vcols=vr)
    assert np.allclose(blk, b["dlogits"][np.ix_(rows, vr)], rtol=0, atol=1e-15)


def test_backward_finite_differences():
    M, K0, D, N = 6, 8, 16, 12
    x, W0, z, gamma, W1, dY, eps = (t.numpy() if isinstance(t, torch.Tensor) else t
                                     for t in _rand_problem(M, K0, D, N, 2))
    f = orc.forward(x, W0, z, gamma, W1, eps)
    b = orc.backward(dY, f["y"], f["h"], f["h"] * gamma[None, :], f["r"], gamma, W1)
    h = f["h"]

    def L(hh, gg, ww):
        ms = (hh * hh).mean(axis=1)
        n = hh / np.sqrt(ms + eps)[:, None] * gg[None, :]
        return float(((n @ ww) * dY).sum())

    step = 1e-6
    rng = np.random.default_rng(0)
    for _ in range(20):
        i, j = rng.integers(M), rng.integers(D)
        hp, hm = h.copy(), h.copy()
        hp[i, j] += step
        hm[i, j] -= step
        fd = (L(hp, gamma, W1) - L(hm, gamma, W1)) / (2 * step)
        assert abs(fd - b["da"][i, j]) <= 1e-7 * max(1.0, abs(fd))
        j = rng.integers(D)
        gp, gm = gamma.copy(), gamma.copy()
        gp[j] += step
        gm[j] -= step
        fd = (L(h, gp, W1) - L(h, gm, W1)) / (2 * step)
        assert abs(fd - b["dgamma"][j]) <= 1e-7 * max(1.0, abs(fd))
        j, c = rng.integers(D), rng.integers(N)
        wp, wm = W1.copy(), W1.copy()
        wp[j, c] += step
        wm[j, c] -= step
        fd = (L(h, gamma, wp) - L(h, gamma, wm)) / (2 * step)
        assert abs(fd - b["dW1"][j, c]) <= 1e-7 * max(1.0, abs(fd))


# ----------------------------------------------------------------- identities

def test_reparameterised_order_equals_definition():
    x, W0, z, gamma, W1, _, eps = (t.numpy() if isinstance(t, torch.Tensor) else t
                                   for t in _rand_problem(32, 64, 96, 80, 3))
    o = orc.forward(x, W0, z, gamma, W1, eps)
    h = x @ W0 + z
    r = 1 / np.sqrt((h * h).mean(axis=1) + eps)
    y_reparam = r[:, None] * ((h * gamma[None, :]) @ W1)
    assert _relerr(o["y"], y_reparam) < 1e-13


def test_constant_and_zero_rows():
    M, K0, D, N = 4, 8, 16, 8
    x, W0, z, gamma, W1, _, eps = (t.numpy() if isinstance(t, torch.Tensor) else t
                                   for t in _rand_problem(M, K0, D, N, 4))
    x[1] = 0.0
    z[1] = 1.5            # constant row: h = c
    x[2] = 0.0
    z[2] = 0.0            # zero row
    o = orc.forward(x, W0, z, gamma, W1, eps)
    c = 1.5
    assert abs(o["r"][1] - 1 / np.sqrt(c * c + eps)) < 1e-15
    assert _relerr(o["y"][1], o["r"][1] * c * (gamma @ W1)) < 1e-13
    assert abs(o["r"][2] - eps ** -0.5) < 1e-10
    assert np.all(o["y"][2] == 0.0)


def test_unit_rms_and_scale_invariance_without_eps():
    x, W0, z, _, W1, _, _ = (t.numpy() if isinstance(t, torch.Tensor) else t
                             for t in _rand_problem(8, 16, 32, 24, 5))
    ones = np.ones(32)
    o = orc.forward(x, W0, z, ones, W1, 0.0)
    assert np.max(np.abs((o["n"] ** 2).mean(axis=1) - 1)) < 1e-13
    o2 = orc.forward(3.0 * x, W0, 3.0 * z, ones, W1, 0.0)
    assert _relerr(o2["y"], o["y"]) < 1e-13


def test_row_isolation_nan():
    x, W0, z, gamma, W1, _, eps = (t.numpy() if isinstance(t, torch.Tensor) else t
                                   for t in _rand_problem(6, 8, 16, 8, 6))
    x = x.copy()
    x[3, 2] = np.nan
    o = orc.forward(x, W0, z, gamma, W1, eps)
    bad = ~np.isfinite(o["y"]).all(axis=1)
    assert bad.tolist() == [False, False, False, True, False, False]
    assert np.isnan(o["r"][3]) and np.isfinite(np.delete(o["r"], 3)).all()


def test_backward_invariants_and_zero_grad():
    x, W0, z, gamma, W1, dY, eps = (t.numpy() if isinstance(t, torch.Tensor) else t
                                    for t in _rand_problem(10, 16, 24, 20, 7, eps=1e-3))
    f = orc.forward(x, W0, z, gamma, W1, eps)
    g = f["h"] * gamma[None, :]
    b = orc.backward(dY, f["y"], f["h"], g, f["r"], gamma, W1)
    s = b["s"]
    lhs = (b["da"] * f["h"]).sum(axis=1)
    assert np.max(np.abs(lhs - s * eps * f["r"] ** 2)) < 1e-12 * np.max(np.abs(s))
    assert abs((gamma * b["dgamma"]).sum() - s.sum()) < 1e-11 * np.abs(s).sum()
    assert abs((b["dW1"] * W1).sum() - s.sum()) < 1e-11 * np.abs(s).sum()
    z0 = orc.backward(np.zeros_like(dY), f["y"], f["h"], g, f["r"], gamma, W1)
    for k in ("s", "da", "dgamma", "dW1"):
        assert np.all(z0[k] == 0.0)


def test_subsets_match_full_computation():
    x, W0, z, gamma, W1, dY, eps = (t.numpy() if isinstance(t, torch.Tensor) else t
                                    for t in _rand_problem(40, 16, 24, 36, 8))
    full = orc.forward(x, W0, z, gamma, W1, eps)
    rows = [0, 5, 17, 39]
    part = orc.forward(x, W0, z, gamma, W1, eps, rows=rows, chunk=3)
    for k in ("h", "r", "n", "y"):   # BLAS blocking may differ with the batch: compare to fp64 rounding
        assert _relerr(part[k], full[k][rows]) < 1e-14
    g = full["h"] * gamma[None, :]
    bf = orc.backward(dY, full["y"], full["h"], g, full["r"], gamma, W1)
    bp = orc.backward(dY, full["y"], full["h"], g, full["r"], gamma, W1,
                      rows=rows, dgamma_cols=[1, 7, 23], dw1_cols=[0, 35])
    assert np.allclose(bp["da"], bf["da"][rows], rtol=0, atol=1e-13)
    assert np.allclose(bp["dgamma"], bf["dgamma"][[1, 7, 23]], rtol=0, atol=1e-12)
    assert np.allclose(bp["dW1"], bf["dW1"][:, [0, 35]], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- hand-worked

def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_hand_worked(case):
    a = {k: np.array(v, dtype=np.float64) for k, v in case.items() if isinstance(v, list)}
    o = orc.forward(a["x"], a["W0"], a["z"], a["gamma"], a["W1"], case["eps"])
    assert np.allclose(o["h"], a["h"], rtol=0, atol=1e-15)
    assert np.allclose(o["r"], a["r"], rtol=1e-15, atol=0)
    assert np.allclose(o["y"], a["y"], rtol=1e-15, atol=1e-15)
    if "dY" in a:
        g = o["h"] * a["gamma"][None, :]
        b = orc.backward(a["dY"], o["y"], o["h"], g, o["r"], a["gamma"], a["W1"])
        for k in ("s", "da", "dgamma", "dW1"):
            assert np.allclose(b[k], a[k], rtol=1e-14, atol=1e-14), k


# ------------------------------------------------------------------- inputs

def test_inputs_are_seeded_and_distributed_as_stated():
    a = inputs.forward_inputs(64, 256, 256, 512, seed=0)
    b = inputs.forward_inputs(64, 256, 256, 512, seed=0)
    c = inputs.forward_inputs(64, 256, 256, 512, seed=1)
    for k in a:
        assert a[k].dtype == torch.bfloat16
        assert torch.equal(a[k], b[k])
        assert not torch.equal(a[k], c[k])
    assert a["x"].shape == (64, 256) and a["W0"].shape == (256, 256)
    assert a["W1"].shape == (256, 512) and a["gamma"].shape == (256,)
    assert abs(a["x"].float().std().item() - 1) < 0.05
    assert abs(a["W1"].float().std().item() * 16 - 1) < 0.05          # 1/sqrt(D), D = 256
    assert abs(a["gamma"].float().mean().item() - 1) < 0.02
    assert abs(a["gamma"].float().std().item() - 0.1) < 0.02
    rows = inputs.sample(8192, 256, 0, "rows")
    assert rows.tolist() == sorted(set(rows.tolist())) and len(rows) == 256
    assert inputs.sample(64, 256, 0, "rows").tolist() == list(range(64))
    lm = inputs.lm_head_inputs(4096, 256, 512, seed=0)
    assert torch.equal(lm["targets"], inputs.lm_head_inputs(4096, 256, 512, seed=0)["targets"])
    assert lm["W"].shape == (512, 256) and abs(lm["W"].float().std().item() * 8 - 1) < 0.05   # 2/sqrt(D)
    ign = (lm["targets"] == -100).float().mean().item()
    assert 0.02 < ign < 0.04 and int(lm["targets"].max()) < 512
    assert len(set(inputs.IDS.values())) == len(inputs.IDS)
