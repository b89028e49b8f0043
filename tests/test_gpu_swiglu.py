"""Parity of the SwiGLU forward and backward (coda_fwd_swiglu, coda_bwd_swiglu)
with the fp64 oracle on one MI355X.

Forward: y is checked as for the chain, o = silu(gate) up against the oracle's
SwiGLU of its fp64 y within the bound that y's own tolerance implies. Backward:
the saved set (h, g, y, r, o) comes from the oracle forward rounded to its
storage types; dY and dW2 are checked at fp32-level agreement, s, da, dgamma
and dW1 against the oracle's chain backward on the oracle's (exact) dY, within
1e-4 rms plus a statistical bound (metrics.SIGMA_K sigma) of the kernels'
rounding of dY to bf16 before the two products that consume it.
"""
import numpy as np
import pytest
import torch

import metrics as mt
from oracle import coda_oracle as orc
from transformer_gemm_epilogue_res_amd import _lib as L
from transformer_gemm_epilogue_res_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EPS = inputs.EPS

SMALL = {
    "tiny": dict(M=64, K0=256, D=256, N=512, E=256),
    "ragged": dict(M=300, K0=256, D=512, N=1024, E=768),
    "one_row": dict(M=1, K0=256, D=256, N=512, E=256),
    "dims64": dict(M=300, K0=192, D=320, N=640, E=192),   # sizes in multiples of 64 (N of 128)
}


def announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


def to_dev(d):
    return {k: v.to(DEV) for k, v in d.items()}


def rsel(t, rows):
    return t.cpu() if rows is None else t.index_select(0, torch.as_tensor(rows, device=t.device)).cpu()


def csel(t, cols):
    return t.cpu() if cols is None else t.index_select(-1, torch.as_tensor(cols, device=t.device)).cpu()


# ------------------------------------------------------------------ forward

def run_fwd(d):
    args = (d["x"], d["W0"], d["z"], d["gamma"], d["W1"], EPS)
    o32 = L.fwd_swiglu(*args, o_dtype=torch.float32)
    o16 = L.fwd_swiglu(*args, o_dtype=torch.bfloat16)
    y32 = L.fwd(*args, y_dtype=torch.float32)["y"]  # the chain's fp32 y, same kernels
    torch.cuda.synchronize()
    return o32, o16, y32


def check_fwd(o32, o16, y32, ref, rows=None):
    y, y32 = rsel(o32["y"], rows), rsel(y32, rows)
    o, o_b = rsel(o32["o"], rows), rsel(o16["o"], rows)
    o_ref = orc.swiglu(ref["y"])
    e_y = mt.normwise(y32, ref["y"])
    bound = mt.swiglu_o_bound(ref["y"], orc.silu(ref["y"][:, 0::2]))
    e_o = float(np.max(np.abs(mt.f64(o) - o_ref) / bound))
    print(f"  y(fp32) max|d|/rms={e_y:.3e}  o max|d|/rms={mt.normwise(o, o_ref):.3e}  o |d|/bound max={e_o:.3f}")
    # y is stored in bf16: the round-to-nearest-even of the chain's fp32 y
    assert torch.equal(mt.rne_bf16(y32).view(torch.int16), y.view(torch.int16))
    assert torch.equal(mt.rne_bf16(o).view(torch.int16), o_b.view(torch.int16))
    for k in ("h", "g", "r"):
        assert torch.equal(rsel(o32[k], rows), rsel(o16[k], rows)), k
    assert e_y <= mt.Y_TOL
    assert e_o <= 1.0
    assert mt.max_rel(rsel(o32["r"], rows), ref["r"]) <= mt.R_TOL


@pytest.mark.parametrize("name", list(SMALL))
def test_fwd_swiglu_small_full(name):
    c = SMALL[name]
    announce(f"coda_fwd_swiglu {name} {c} seed=0")
    inp = inputs.forward_inputs(c["M"], c["K0"], c["D"], c["N"], seed=0)
    o32, o16, y32 = run_fwd(to_dev(inp))
    ref = orc.forward(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], EPS)
    check_fwd(o32, o16, y32, ref)


# ------------------------------------------------------------------ backward

def saved_set(inp, eps=EPS):
    """The forward's saved tensors (o included), from the oracle forward rounded to their storage types."""
    f = orc.forward(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], eps)
    gam = orc.f64(inp["gamma"])
    return {"h": torch.from_numpy(f["h"]).to(torch.bfloat16),
            "g": torch.from_numpy(f["h"] * gam[None, :]).to(torch.bfloat16),
            "y": torch.from_numpy(f["y"]).to(torch.bfloat16),
            "r": torch.from_numpy(f["r"]).to(torch.float32),
            "o": torch.from_numpy(orc.swiglu(f["y"])).to(torch.bfloat16)}


def host_case(c, seed=0):
    inp = inputs.forward_inputs(c["M"], c["K0"], c["D"], c["N"], seed=seed)
    host = dict(saved_set(inp), gamma=inp["gamma"], W1=inp["W1"], **inputs.swiglu_inputs(c["M"], c["N"], c["E"], seed))
    return host


def run_bwd(d):
    args = (d["dOut"], d["W2"], d["o"], d["y"], d["h"], d["g"], d["r"], d["gamma"], d["W1"])
    o32 = L.bwd_swiglu(*args, da_dtype=torch.float32, dW1_dtype=torch.float32, dW2_dtype=torch.float32)
    o16 = L.bwd_swiglu(*args)
    torch.cuda.synchronize()
    return o32, o16


def check_bwd(o32, o16, host, rows=None, jcols=None, ncols=None, ecols=None):
    sw_all = orc.swiglu_backward(host["dOut"], host["W2"], host["y"], host["o"], dw2_cols=ecols)
    ref = orc.backward(sw_all["dY"], host["y"], host["h"], host["g"], host["r"], host["gamma"], host["W1"],
                       rows=rows, dgamma_cols=jcols, dw1_cols=ncols)
    ridx = slice(None) if rows is None else np.asarray(rows)
    dY_ref = sw_all["dY"][ridx]
    dY = rsel(o32["dY"], rows)
    assert torch.equal(dY, rsel(o16["dY"], rows))      # same kernel, same bf16 dY
    s, da = rsel(o32["s"], rows), rsel(o32["da"], rows)
    dg, dW1, dW2 = csel(o32["dgamma"], jcols), csel(o32["dW1"], ncols), csel(o32["dW2"], ecols)
    # dY is rounded to bf16 (from its fp32 value) before G = dY @ W1^T and dW1 = bf16(r g)^T dY: the
    # statistical bound of those roundings (metrics, SIGMA_K sigma) on top of 1e-4 rms of fp32 error
    dY_var = mt.half_ulp_sq_over_3(sw_all["dY"])
    s_da, s_dg = mt.dgrad_rounding_sigma(dY_var, host["W1"], host["r"], host["gamma"], host["h"], rows, jcols)
    s_w1 = mt.operand_rounding_sigma(host["g"], host["r"], sw_all["dY"], ncols, dY_var=dY_var)
    e = {"dY": mt.bf16_within(dY, dY_ref, 1e-4), "dW2": mt.normwise(dW2, sw_all["dW2"]),
         "s": mt.normwise(s, ref["s"]), "da": mt.within_sigma(da, ref["da"], s_da),
         "dgamma": mt.within_sigma(dg, ref["dgamma"], s_dg), "dW1": mt.within_sigma(dW1, ref["dW1"], s_w1)}
    print("  " + "  ".join(f"{k}={v:.3e}" for k, v in e.items()) +
          f"  (dW2, s: max|d|/rms; dY |d|/(1e-4 rms + ulp/2); da, dgamma, dW1 |d|/(1e-4 rms + {mt.SIGMA_K} sigma))")
    print(f"  da max|d|/rms={mt.normwise(da, ref['da']):.3e}  dgamma max|d|/rms={mt.normwise(dg, ref['dgamma']):.3e}"
          f"  dW1 max|d|/rms={mt.normwise(dW1, ref['dW1']):.3e}")
    assert torch.equal(mt.rne_bf16(da).view(torch.int16), rsel(o16["da"], rows).view(torch.int16))
    assert torch.equal(mt.rne_bf16(dW1).view(torch.int16), csel(o16["dW1"], ncols).view(torch.int16))
    assert torch.equal(mt.rne_bf16(dW2).view(torch.int16), csel(o16["dW2"], ecols).view(torch.int16))
    assert torch.equal(rsel(o16["s"], rows), s) and torch.equal(csel(o16["dgamma"], jcols), dg)
    assert e["dY"] <= 1.0
    assert e["dW2"] <= 1e-4
    assert e["s"] <= mt.S_TOL
    assert e["da"] <= 1.0 and e["dgamma"] <= 1.0 and e["dW1"] <= 1.0


@pytest.mark.parametrize("name", list(SMALL))
def test_bwd_swiglu_small_full(name):
    c = SMALL[name]
    announce(f"coda_bwd_swiglu {name} {c} seed=0")
    host = host_case(c)
    o32, o16 = run_bwd(to_dev(host))
    check_bwd(o32, o16, host)


def test_swiglu_forward_then_backward_on_device():
    """The backward fed by the GPU forward's own saved tensors (the training-step
    composition), against the oracle's composition from the same inputs."""
    c = SMALL["ragged"]
    announce(f"coda_fwd_swiglu -> coda_bwd_swiglu {c} seed=1")
    inp = inputs.forward_inputs(c["M"], c["K0"], c["D"], c["N"], seed=1)
    sw = inputs.swiglu_inputs(c["M"], c["N"], c["E"], seed=1)
    d = to_dev(dict(inp, **sw))
    f = L.fwd_swiglu(d["x"], d["W0"], d["z"], d["gamma"], d["W1"], EPS)
    b = L.bwd_swiglu(d["dOut"], d["W2"], f["o"], f["y"], f["h"], f["g"], f["r"], d["gamma"], d["W1"],
                     da_dtype=torch.float32, dW2_dtype=torch.float32)
    torch.cuda.synchronize()
    fr = orc.forward(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], EPS)
    o_ex = orc.swiglu(fr["y"])
    g_ex = fr["h"] * orc.f64(inp["gamma"])[None, :]
    sw_ref = orc.swiglu_backward(sw["dOut"], sw["W2"], fr["y"], o_ex)
    ref = orc.backward(sw_ref["dY"], fr["y"], fr["h"], g_ex, fr["r"], inp["gamma"], inp["W1"])
    # dW2 = o^T dOut: the device's bf16 o is within the forward's o bound plus half an ulp of o_ex
    ob = mt.swiglu_o_bound(fr["y"], orc.silu(fr["y"][:, 0::2]))
    allow = (ob + 0.5 * mt.bf16_ulp(np.abs(o_ex) + ob)).T @ np.abs(mt.f64(sw["dOut"]))
    e = {"s": mt.normwise(b["s"], ref["s"]), "da": mt.normwise(b["da"], ref["da"]),
         "dW2": mt.normwise(b["dW2"], sw_ref["dW2"]), "dW2/bound": mt.within_allowance(b["dW2"], sw_ref["dW2"], allow)}
    print("  " + "  ".join(f"{k}={v:.3e}" for k, v in e.items()))
    assert e["dW2/bound"] <= 1.0
    # s and da see the saved y's forward error (1e-2 rms, then bf16) through smooth functions of y
    assert e["da"] <= 3 * mt.Y_TOL and e["s"] <= 3 * mt.Y_TOL


@pytest.mark.parametrize("name", ["tiny", "ragged"])
def test_swiglu_unfused_baseline(name):
    """coda_unfused_ref's SwiGLU: o from the stored bf16 y, dY from a stored bf16 dO. Its roundings
    (y and dO to bf16 before the activation and its backward) make it a looser match to the oracle."""
    c = SMALL[name]
    announce(f"coda_unfused_ref fwd/bwd SwiGLU {name} {c} seed=0")
    inp = inputs.forward_inputs(c["M"], c["K0"], c["D"], c["N"], seed=0)
    d = to_dev(inp)
    args = (d["x"], d["W0"], d["z"], d["gamma"], d["W1"], EPS)
    fu = L.fwd_swiglu(*args, o_dtype=torch.float32, unfused=True)
    ff = L.fwd_swiglu(*args, o_dtype=torch.float32)
    torch.cuda.synchronize()
    for k in ("h", "g", "r", "y"):            # the chain part is the same fused forward
        assert torch.equal(fu[k], ff[k]), k
    ref = orc.forward(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], EPS)
    # o from the bf16 y: y's elementwise error is at most 1e-2 rms + half an ulp of the largest |y|
    yr = ref["y"]
    tol = mt.Y_TOL + 0.5 * float(mt.bf16_ulp(np.max(np.abs(yr)) * (1 + mt.Y_TOL))) / mt.rms(yr)
    bound = mt.swiglu_o_bound(yr, orc.silu(yr[:, 0::2]), tol)
    e_o = float(np.max(np.abs(mt.f64(fu["o"]) - orc.swiglu(yr)) / bound))
    print(f"  unfused o |d|/bound max={e_o:.3f}")
    assert e_o <= 1.0
    host = host_case(c)
    dv = to_dev(host)
    bargs = (dv["dOut"], dv["W2"], dv["o"], dv["y"], dv["h"], dv["g"], dv["r"], dv["gamma"], dv["W1"])
    bu = L.bwd_swiglu(*bargs, da_dtype=torch.float32, dW1_dtype=torch.float32, dW2_dtype=torch.float32, unfused=True)
    bf = L.bwd_swiglu(*bargs, da_dtype=torch.float32, dW1_dtype=torch.float32, dW2_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(bu["dW2"], bf["dW2"])   # the same product of the same operands
    sw = orc.swiglu_backward(host["dOut"], host["W2"], host["y"], host["o"])
    rb = orc.backward(sw["dY"], host["y"], host["h"], host["g"], host["r"], host["gamma"], host["W1"])
    # dO is rounded to bf16 before the SwiGLU backward: a relative error of up to 2^-9 of dY (up to
    # half an ulp of dY, uniform, shared by the two elements of a pair) on top of dY's own half-ulp
    # rounding -- up to 1.5 ulp elementwise, and at most three times the rounding variance in any
    # contraction (the pair's shared part counts twice); the bounds take twice the fused path's sigma
    dYu, dYr = mt.f64(bu["dY"]), sw["dY"]
    dY_var = 4.0 * mt.half_ulp_sq_over_3(dYr)
    s_da, s_dg = mt.dgrad_rounding_sigma(dY_var, host["W1"], host["r"], host["gamma"], host["h"])
    s_w1 = mt.operand_rounding_sigma(host["g"], host["r"], dYr, None, dY_var=dY_var)
    b_dY = 1.5 * mt.bf16_ulp(np.maximum(np.abs(dYu), np.abs(dYr))) + 1e-4 * mt.rms(dYr)
    e = {"dY": float(np.max(np.abs(dYu - dYr) / b_dY)), "s": mt.normwise(bu["s"], rb["s"]),
         "da": mt.within_sigma(bu["da"], rb["da"], s_da), "dgamma": mt.within_sigma(bu["dgamma"], rb["dgamma"], s_dg),
         "dW1": mt.within_sigma(bu["dW1"], rb["dW1"], s_w1)}
    print("  unfused " + "  ".join(f"{k}={v:.3e}" for k, v in e.items()) + "  (s: max|d|/rms; others |d| / bound)")
    assert e["s"] <= 1e-2
    assert e["dY"] <= 1.0 and e["da"] <= 1.0 and e["dgamma"] <= 1.0 and e["dW1"] <= 1.0


@pytest.mark.slow
def test_swiglu_llama3_8b_sampled():
    c = dict(inputs.CONFIGS["llama3_8b"], E=inputs.CONFIGS["llama3_8b"]["D"])
    announce(f"coda_fwd_swiglu/coda_bwd_swiglu llama3_8b {c} seed=0, sampled")
    host = host_case(c)
    rows = inputs.sample(c["M"], 256, 0, "rows").numpy()
    f_in = inputs.forward_inputs(c["M"], c["K0"], c["D"], c["N"], seed=0)
    o32, o16, y32 = run_fwd(to_dev(f_in))
    ref_f = orc.forward(f_in["x"], f_in["W0"], f_in["z"], f_in["gamma"], f_in["W1"], EPS, rows=rows)
    check_fwd(o32, o16, y32, ref_f, rows=rows)
    del o32, o16, y32, f_in
    torch.cuda.empty_cache()
    jcols = inputs.sample(c["D"], 256, 0, "dgamma_cols").numpy()
    ncols = inputs.sample(c["N"], 256, 0, "dw1_cols").numpy()
    ecols = inputs.sample(c["E"], 256, 0, "dw2_cols").numpy()
    o32, o16 = run_bwd(to_dev(host))
    check_bwd(o32, o16, host, rows=rows, jcols=jcols, ncols=ncols, ecols=ecols)


def test_swiglu_graph_capture():
    """The SwiGLU block's forward and backward captured into one HIP graph: every replay
    reproduces the eager results bit for bit (the library allocates and clears nothing)."""
    from graph_util import assert_replays_match_eager
    c = SMALL["ragged"]
    M, K0, D, N, E = c["M"], c["K0"], c["D"], c["N"], c["E"]
    announce(f"graph capture coda_fwd_swiglu + coda_bwd_swiglu {c}")
    inp = to_dev(inputs.forward_inputs(M, K0, D, N, seed=6))
    sw = to_dev(inputs.swiglu_inputs(M, N, E, seed=6))
    bf = torch.bfloat16
    fo = {"h": torch.empty(M, D, dtype=bf, device=DEV), "g": torch.empty(M, D, dtype=bf, device=DEV),
          "r": torch.empty(M, dtype=torch.float32, device=DEV), "y": torch.empty(M, N, dtype=bf, device=DEV),
          "o": torch.empty(M, N // 2, dtype=bf, device=DEV)}
    bo = {"dY": torch.empty(M, N, dtype=bf, device=DEV), "da": torch.empty(M, D, dtype=bf, device=DEV),
          "dgamma": torch.empty(D, dtype=torch.float32, device=DEV), "dW1": torch.empty(D, N, dtype=bf, device=DEV),
          "dW2": torch.empty(N // 2, E, dtype=bf, device=DEV), "s": torch.empty(M, dtype=torch.float32, device=DEV)}
    fws = L.workspace(L.CODA_OP_FWD_SWIGLU, M, D, N, DEV)
    bws = L.workspace(L.CODA_OP_BWD_SWIGLU, M, D, N, DEV)

    def step():
        L.fwd_swiglu(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], EPS, ws=fws, out=fo)
        L.bwd_swiglu(sw["dOut"], sw["W2"], fo["o"], fo["y"], fo["h"], fo["g"], fo["r"], inp["gamma"], inp["W1"],
                     ws=bws, out=bo)

    assert_replays_match_eager(step, list(fo.values()) + list(bo.values()))
