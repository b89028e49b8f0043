"""fp64 CPU oracle for the GEMM -> residual -> RMSNorm -> GEMM chain and its backward.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The HIP library
never calls it and shares no code with it.

Source of every formula: "CODA: Rewriting Transformer Blocks as GEMM-Epilogue
Programs" as described on the hotdry blog page (section "GEMM-Residual-RMSNorm-
GEMM reparameterisation": the chain's definition and its reparameterised form;
section "backward GEMM-epilogue structure": the row statistic s) and on the
kucoin page (section "CODA: treasure hidden in the coda": r is a row-shared
scalar that commutes with the second GEMM).

What it computes is the plain, *unfused* definition of the chain, in float64,
from the exact values of its (bf16) inputs, with no intermediate rounding:

    h   = x @ W0 + z                      (GEMM, residual add)
    ms  = mean over the D columns of h^2  (RMSNorm statistic)
    r   = 1 / sqrt(ms + eps)              (row-wise inverse RMS factor)
    n   = r * h * gamma                   (normalised activation)
    y   = n @ W1                          (second GEMM)

RMSNorm form (the pages only say "row-wise inverse RMS factor r"): mean over the
D columns, eps inside the root, no bias, no mean subtraction, gamma multiplies
elementwise.

Backward of L = <dY, y> for the saved set (h, g, y, r) of a forward, with
g = h * gamma:

    G      = dY @ W1^T                    (data-gradient GEMM)
    s_i    = sum_n dY_in * y_in           (the pages' row statistic, moved to the
                                           GEMM boundary: sum_cols(dY . y))
    da_ij  = r_i gamma_j G_ij - s_i r_i^2 h_ij / D
    dgam_j = sum_i G_ij r_i h_ij
    dW1    = (r . g)^T @ dY               i.e. dW1_jn = sum_i g_ij r_i dY_in

The da formula is the exact gradient of the definition above (d r_i / d h_ij =
-r_i^3 h_ij / D, and sum_k G_ik gamma_k h_ik = s_i / r_i because
sum_k G_ik n_ik = sum_n dY_in y_in); the pages print only s. It is pinned
against torch autograd and finite differences in the tests.

Backward through the first GEMM and the residual (the rest of the chain's
backward, h = x @ W0 + z), for an upstream gradient dh of h (da above, plus any
gradient the residual stream brings, which this chain does not model):

    dz  = dh
    dx  = dh @ W0^T
    dW0 = x^T @ dh

SwiGLU on the second GEMM's output (blog, section "成对激活的寄存器级融合":
paired features sit in adjacent output columns, so the gated activation is
applied where the pair is produced; the backward of such a pairwise epilogue is
a dimension-expanding one). Column 2f of y is gate f and column 2f+1 is up f:

    o_if   = silu(y_i,2f) * y_i,2f+1,      silu(v) = v / (1 + exp(-v))

and for an output projection out = o @ W2 (W2 [F, E]) with L = <dOut, out>:

    dO       = dOut @ W2^T                 (the down projection's data gradient)
    dY_i,2f  = dO_if * y_i,2f+1 * silu'(y_i,2f),   silu'(v) = sig(v) (1 + v (1 - sig(v)))
    dY_i,2f+1 = dO_if * silu(y_i,2f)
    s_i      = sum_n dY_in * y_in          (the same row statistic, now taken where
                                            dY is produced)
    dW2      = o^T @ dOut

after which the chain's backward above continues with this dY.

Cross-entropy on an LM-head GEMM (blog, section "五类 Epilogue 原语", the
stateful-transform primitive: tile-level online log-sum-exp and cross-entropy
statistics; kucoin, section "五つの「ブロック」": block log-sum-exp and the
running max / sum-exp statistics, and section "CODAの機能": cross-entropy loss
and its gradient are in scope). For hidden states h [M, D], an output weight
W [V, D] (one row per vocabulary entry) and targets t [M]:

    logits_iv = sum_d h_id W_vd                     (logits = h @ W^T)
    lse_i     = m_i + log sum_v exp(logits_iv - m_i),  m_i = max_v logits_iv
    loss_i    = lse_i - logits_i,t_i                (0 for a row whose target lies
                                                     outside [0, V): an ignored row)

and for L = sum_i dloss_i loss_i:

    dlogits_iv = dloss_i (exp(logits_iv - lse_i) - [v = t_i])   (0 on ignored rows)
    dh         = dlogits @ W
    dW         = dlogits^T @ h

The max shift is the textbook way to write log-sum-exp (exact in real
arithmetic); the oracle takes it over the whole row, with no tiling.

Rounded operands. Where a kernel must round an operand to bf16 before a contraction (the weight
gradient's r_i g_ij, which carries r on its contraction index; a gradient produced in fp32 and stored
in bf16 before the next product), ``bf16_round`` gives that operand (fp32, then bf16 round-to-nearest-
even) and ``backward(round_rg=True, s=...)`` the backward on it, so a test can check the contraction
itself on the very operand the kernel uses, beside the exact definition above.

Matrix products use numpy's float64 matmul as a library primitive. Row subsets
(``rows``) and column subsets are supported because rows of the forward are
independent and the large configurations are checked on seeded samples.
"""
from __future__ import annotations

import numpy as np


def f64(t) -> np.ndarray:
    """Exact widening of a torch tensor (bf16/fp32/fp64) or array to a float64 ndarray."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64, copy=False)
    import torch  # local: the oracle itself is numpy-only
    return t.detach().to("cpu").to(torch.float64).numpy()


def _take(t, rows=None, cols=None) -> np.ndarray:
    """float64 copy of t[rows][:, cols] (None = all); t is a torch tensor or ndarray."""
    if not isinstance(t, np.ndarray):
        import torch
        if rows is not None:
            t = t.index_select(0, torch.as_tensor(np.asarray(rows, dtype=np.int64)))
        if cols is not None:
            t = t.index_select(1, torch.as_tensor(np.asarray(cols, dtype=np.int64)))
        return f64(t)
    a = t if rows is None else t[np.asarray(rows, dtype=np.int64)]
    a = a if cols is None else a[:, np.asarray(cols, dtype=np.int64)]
    return f64(a)


def bf16_round(x) -> np.ndarray:
    """The bf16 value a kernel stores for x when it computes x in fp32: x rounded to fp32, then to the
    nearest bf16 with ties to even (the top 16 bits of the fp32 word after adding 0x7fff plus the
    lowest kept bit); NaN stays NaN and +-inf stays +-inf. Returned widened to float64."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    nan = np.isnan(x32)
    u = np.where(nan, np.uint64(0x7FC00000), x32.view(np.uint32).astype(np.uint64))
    r = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32)
    return np.where(nan, np.nan, r.view(np.float32).astype(np.float64))


def gemm(A, B) -> np.ndarray:
    """Plain product C = A @ B in float64."""
    return f64(A) @ f64(B)


def forward(x, W0, z, gamma, W1, eps: float, rows=None, chunk: int = 1024) -> dict:
    """Unfused forward of y = RMSNorm(x @ W0 + z, gamma) @ W1 for the given rows.

    Returns float64 arrays h [R,D], r [R], n [R,D], y [R,N] for R = len(rows)
    (all rows when ``rows`` is None).
    """
    W0d, W1d, gd = f64(W0), f64(W1), f64(gamma)
    M = x.shape[0]
    idx = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    D = W0d.shape[1]
    out = {"h": [], "r": [], "n": [], "y": []}
    for c0 in range(0, len(idx), chunk):
        sel = idx[c0:c0 + chunk]
        xs, zs = _take(x, sel), _take(z, sel)
        h = xs @ W0d + zs                       # GEMM, then residual add
        ms = (h * h).sum(axis=1) / D            # mean of squares over D columns
        r = 1.0 / np.sqrt(ms + eps)             # row-wise inverse RMS
        n = (r[:, None] * h) * gd[None, :]      # RMSNorm output
        y = n @ W1d                             # second GEMM
        for k, v in (("h", h), ("r", r), ("n", n), ("y", y)):
            out[k].append(v)
    return {k: np.concatenate(v, axis=0) for k, v in out.items()}


def backward(dY, y, h, g, r, gamma, W1, rows=None, dgamma_cols=None, dw1_cols=None, s=None,
             round_rg=False) -> dict:
    """Backward of the chain for the saved set (h, g, y, r).

    * ``rows``: rows i for which s_i, G_i and da_i are returned (all when None).
    * ``dgamma_cols``: columns j of dgamma (sums over *all* M rows; all when None).
    * ``dw1_cols``: columns n of dW1 (all D rows of each; all when None).
    * ``s``: the row statistic [M] to use instead of sum_n dY_in y_in (for a dY that is itself a
      rounded copy of the gradient s was taken from, as when dY is produced in fp32 and stored in bf16).
    * ``round_rg``: dW1 from the operand r_i g_ij rounded once to bf16 (``bf16_round`` of the fp32
      product), the form the weight gradient takes when r lies on its contraction index; otherwise
      the exact r_i g_ij.
    """
    W1d, gd, rd = f64(W1), f64(gamma), f64(r)
    M, N = dY.shape
    D = W1d.shape[0]
    ridx = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    out = {}

    # rows: s, G, da
    dYr, yr, hr = _take(dY, ridx), _take(y, ridx), _take(h, ridx)
    s = (dYr * yr).sum(axis=1) if s is None else f64(s)[ridx]
    G = dYr @ W1d.T
    rr = rd[ridx]
    da = (rr[:, None] * gd[None, :]) * G - ((s * rr * rr) / D)[:, None] * hr
    out.update(s=s, G=G, da=da)
    del dYr, yr

    # dgamma columns: G[:, cols] for every row
    jc = np.arange(D) if dgamma_cols is None else np.asarray(dgamma_cols, dtype=np.int64)
    dgam = np.zeros(len(jc))
    for c0 in range(0, M, 2048):
        blk = np.arange(c0, min(M, c0 + 2048))
        Gc = _take(dY, blk) @ W1d[jc, :].T
        dgam += (Gc * rd[blk, None] * _take(h, blk, jc)).sum(axis=0)
    out["dgamma"] = dgam

    # dW1 columns: (r . g)^T @ dY[:, cols]
    nc = np.arange(N) if dw1_cols is None else np.asarray(dw1_cols, dtype=np.int64)
    dW1 = np.zeros((D, len(nc)))
    for c0 in range(0, M, 2048):
        blk = np.arange(c0, min(M, c0 + 2048))
        if round_rg:   # the fp32 product of the fp32 r and the bf16 g, rounded to bf16
            gr = bf16_round(rd[blk, None].astype(np.float32) * _take(g, blk).astype(np.float32))
        else:
            gr = _take(g, blk) * rd[blk, None]
        dW1 += gr.T @ _take(dY, blk, nc)
    out["dW1"] = dW1
    return out


def backward_gemm0(dh, x, W0, rows=None, dw0_cols=None) -> dict:
    """Backward through h = x @ W0 + z for the upstream gradient dh [M, D].

    * ``rows``: rows i of dx (and dz) returned (all when None);
    * ``dw0_cols``: columns j of dW0 (sums over *all* M rows; all when None).
    """
    W0d = f64(W0)
    M, D = dh.shape
    K0 = W0d.shape[0]
    ridx = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    dhr = _take(dh, ridx)
    out = {"dz": dhr, "dx": dhr @ W0d.T}
    jc = np.arange(D) if dw0_cols is None else np.asarray(dw0_cols, dtype=np.int64)
    dW0 = np.zeros((K0, len(jc)))
    for c0 in range(0, M, 2048):
        blk = np.arange(c0, min(M, c0 + 2048))
        dW0 += _take(x, blk).T @ _take(dh, blk, jc)
    out["dW0"] = dW0
    return out


def _sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v))


def silu(v) -> np.ndarray:
    """silu(v) = v * sigmoid(v)."""
    v = np.asarray(v, dtype=np.float64)
    return v * _sigmoid(v)


def swiglu(y) -> np.ndarray:
    """o[:, f] = silu(y[:, 2f]) * y[:, 2f+1] (gate/up interleaved along the columns)."""
    yd = f64(y)
    return silu(yd[:, 0::2]) * yd[:, 1::2]


def swiglu_backward(dOut, W2, y, o, rows=None, dw2_cols=None) -> dict:
    """Backward of o = swiglu(y), out = o @ W2 for L = <dOut, out>, for the saved y (and o).

    * ``rows``: rows i of dO, dY and s returned (all when None);
    * ``dw2_cols``: columns e of dW2 = o^T @ dOut (sums over all M rows; all when None).
    """
    W2d = f64(W2)
    M = dOut.shape[0]
    ridx = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    dO = _take(dOut, ridx) @ W2d.T
    yr = _take(y, ridx)
    gate, up = yr[:, 0::2], yr[:, 1::2]
    sg = _sigmoid(gate)
    dY = np.empty_like(yr)
    dY[:, 0::2] = dO * up * (sg * (1.0 + gate * (1.0 - sg)))
    dY[:, 1::2] = dO * gate * sg
    out = {"dO": dO, "dY": dY, "s": (dY * yr).sum(axis=1)}
    ec = np.arange(W2d.shape[1]) if dw2_cols is None else np.asarray(dw2_cols, dtype=np.int64)
    dW2 = np.zeros((W2d.shape[0], len(ec)))
    for c0 in range(0, M, 2048):
        blk = np.arange(c0, min(M, c0 + 2048))
        dW2 += _take(o, blk).T @ _take(dOut, blk, ec)
    out["dW2"] = dW2
    return out


def log_sum_exp(L) -> np.ndarray:
    """lse_i = m_i + log sum_v exp(L_iv - m_i) with m_i the row maximum (float64)."""
    L = np.asarray(L, dtype=np.float64)
    m = L.max(axis=1)
    return m + np.log(np.exp(L - m[:, None]).sum(axis=1))


def cross_entropy_logits(L, targets) -> dict:
    """Per-row cross-entropy of logits L [R, V] against targets [R]: dict(lse, loss, valid);
    rows with a target outside [0, V) are ignored (loss 0)."""
    L = np.asarray(L, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64)
    V = L.shape[1]
    valid = (t >= 0) & (t < V)
    lse = log_sum_exp(L)
    picked = np.where(valid, L[np.arange(L.shape[0]), np.where(valid, t, 0)], 0.0)
    return {"lse": lse, "loss": np.where(valid, lse - picked, 0.0), "valid": valid}


def lm_head_cross_entropy(h, W, targets, rows=None, chunk: int = 512) -> dict:
    """Forward of loss_i = lse_i(h @ W^T) - (h @ W^T)_i,t_i for the given rows (all when None).
    Returns float64 lse [R], loss [R], and the boolean valid [R]."""
    Wd = f64(W)
    t = np.asarray(targets, dtype=np.int64) if not hasattr(targets, "numpy") else targets.numpy().astype(np.int64)
    M = len(t)
    idx = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    out = {"lse": [], "loss": [], "valid": []}
    for c0 in range(0, len(idx), chunk):
        sel = idx[c0:c0 + chunk]
        r = cross_entropy_logits(_take(h, sel) @ Wd.T, t[sel])
        for k in out:
            out[k].append(r[k])
    return {k: np.concatenate(v) for k, v in out.items()}


def lm_head_dlogits(h, W, targets, lse, dloss, rows=None, vcols=None) -> np.ndarray:
    """dlogits_iv = dloss_i (exp(logits_iv - lse_i) - [v = t_i]) for the given rows i and vocabulary
    columns v (all when None), 0 on ignored rows, from the logits h @ W^T recomputed in float64 and the
    saved lse."""
    Wd = f64(W)
    t = np.asarray(targets, dtype=np.int64) if not hasattr(targets, "numpy") else targets.numpy().astype(np.int64)
    lse_d, dl = f64(lse), f64(dloss)
    V = Wd.shape[0]
    sel = np.arange(len(t)) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(V) if vcols is None else np.asarray(vcols, dtype=np.int64)
    L = _take(h, sel) @ Wd[cols].T
    P = np.exp(L - lse_d[sel, None])
    tv = t[sel]
    valid = (tv >= 0) & (tv < V)
    onehot = (cols[None, :] == tv[:, None]).astype(np.float64)
    return np.where(valid[:, None], dl[sel, None] * (P - onehot), 0.0)


def lm_head_cross_entropy_backward(h, W, targets, lse, dloss, rows=None, dw_rows=None, chunk: int = 512) -> dict:
    """Backward of L = sum_i dloss_i loss_i for the saved lse [M]:

    * ``rows``: rows i of dlogits [R, V] and dh [R, D] returned (all when None);
    * ``dw_rows``: vocabulary rows v of dW [*, D] (sums over *all* M rows; all when None).
    """
    Wd = f64(W)
    M, V = len(targets), Wd.shape[0]
    idx = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    dL = np.concatenate([lm_head_dlogits(h, Wd, targets, lse, dloss, rows=idx[c0:c0 + chunk])
                         for c0 in range(0, len(idx), chunk)])
    out = {"dlogits": dL, "dh": dL @ Wd}
    vc = np.arange(V) if dw_rows is None else np.asarray(dw_rows, dtype=np.int64)
    dW = np.zeros((len(vc), Wd.shape[1]))
    for c0 in range(0, M, chunk):
        blk = np.arange(c0, min(M, c0 + chunk))
        dW += lm_head_dlogits(h, Wd, targets, lse, dloss, rows=blk, vcols=vc).T @ _take(h, blk)
    out["dW"] = dW
    return out
