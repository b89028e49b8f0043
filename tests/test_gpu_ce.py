"""Parity of the cross-entropy LM head (coda_ce_fwd, coda_ce_bwd) with the fp64
oracle on one MI355X.

Forward: lse and loss at fp32-level agreement (the logits are fp32 accumulations
of exact bf16 products and never rounded); ignored rows have loss exactly 0.
Backward, fed the oracle's lse: dlogits faithfully rounded to bf16 (within one
ulp, +1e-4 rms); dh and dW within 1e-4 rms plus a statistical bound
(metrics.SIGMA_K sigma) of that rounding of dlogits before the two products.

The unfused baseline (coda_unfused_ref: fp32 logits stored, then row kernels) is
held to the same bounds; its logits come from the same mainloop, so its backward
matches the fused one bit for bit. So does the backward from the forward's stored
logits (coda_ce_fwd with a logits output, coda_ce_bwd reading them).
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
TOL = 1e-4

SMALL = {
    "tiny": dict(M=64, D=256, V=512),
    "ragged": dict(M=300, D=512, V=1280),
    "one_row": dict(M=1, D=256, V=256),
    "llama_vocab": dict(M=64, D=256, V=inputs.LM_VOCAB),
    "dims64": dict(M=300, D=320, V=576),                  # sizes in multiples of 64
}


def announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


def case_inputs(c, seed=0):
    d = inputs.lm_head_inputs(c["M"], c["D"], c["V"], seed=seed)
    t = d["targets"]
    if c["M"] > 2:  # a target in the first and in the last column, and an ignored row
        t[0], t[c["M"] - 1], t[1] = 0, c["V"] - 1, -100
    return d


def rsel(t, rows):
    return t.cpu() if rows is None else t.index_select(0, torch.as_tensor(rows, device=t.device)).cpu()


def check_fwd(out, ref, targets, rows=None):
    lse, loss = rsel(out["lse"], rows), rsel(out["loss"], rows)
    e = {"lse": mt.normwise(lse, ref["lse"]), "loss": mt.normwise(loss, ref["loss"])}
    print("  " + "  ".join(f"{k} max|d|/rms={v:.3e}" for k, v in e.items()))
    ign = ~ref["valid"]
    assert torch.all(loss[torch.as_tensor(ign)] == 0)
    assert e["lse"] <= TOL and e["loss"] <= TOL


def check_bwd(out, host, lse_ref, rows=None, vrows=None):
    h, W, t, dloss = host["h"], host["W"], host["targets"], host["dloss"]
    ref = orc.lm_head_cross_entropy_backward(h, W, t, lse_ref, dloss, rows=rows, dw_rows=vrows)
    dL = rsel(out["dlogits"], rows)
    dh = rsel(out["dh"], rows)
    dW = out["dW"].cpu() if vrows is None else out["dW"].index_select(0, torch.as_tensor(vrows, device=DEV)).cpu()
    # statistical bounds (metrics.SIGMA_K sigma) of rounding dlogits to bf16 before the products; dW's
    # rows v need dlogits[:, v] over all M rows
    s_dh = mt.rounding_sigma(mt.half_ulp_sq_over_3(ref["dlogits"]), W)
    vcols = np.arange(W.shape[0]) if vrows is None else np.asarray(vrows)
    dLv = np.concatenate([orc.lm_head_dlogits(h, W, t, lse_ref, dloss, rows=np.arange(c0, min(h.shape[0], c0 + 512)), vcols=vcols)
                          for c0 in range(0, h.shape[0], 512)])
    s_dW = mt.rounding_sigma(mt.half_ulp_sq_over_3(dLv).T, h)
    e = {"dlogits": mt.bf16_faithful(dL, ref["dlogits"], TOL),
         "dh": mt.within_sigma(dh, ref["dh"], s_dh, TOL), "dW": mt.within_sigma(dW, ref["dW"], s_dW, TOL)}
    print("  " + "  ".join(f"{k} |d|/bound={v:.3e}" for k, v in e.items()) +
          f"  (dh max|d|/rms={mt.normwise(dh, ref['dh']):.3e}, dW max|d|/rms={mt.normwise(dW, ref['dW']):.3e})")
    ign = torch.as_tensor(~((rsel(t, rows) >= 0) & (rsel(t, rows) < W.shape[0])))
    assert torch.all(dL[ign] == 0)
    assert e["dlogits"] <= 1.0 and e["dh"] <= 1.0 and e["dW"] <= 1.0


@pytest.mark.parametrize("name", list(SMALL))
def test_ce_small_full(name):
    c = SMALL[name]
    announce(f"coda_ce_fwd / coda_ce_bwd {name} {c} seed=0")
    host = case_inputs(c)
    d = {k: v.to(DEV) for k, v in host.items()}
    f = L.ce_fwd(d["h"], d["W"], d["targets"])
    torch.cuda.synchronize()
    ref = orc.lm_head_cross_entropy(host["h"], host["W"], host["targets"])
    check_fwd(f, ref, host["targets"])
    # the backward on the oracle's lse (no oracle input comes from the device), fp32 and bf16 outputs
    lse_ref = torch.from_numpy(ref["lse"]).to(torch.float32)
    b32 = L.ce_bwd(d["h"], d["W"], d["targets"], lse_ref.to(DEV), d["dloss"], dh_dtype=torch.float32,
                   dW_dtype=torch.float32)
    b16 = L.ce_bwd(d["h"], d["W"], d["targets"], lse_ref.to(DEV), d["dloss"])
    torch.cuda.synchronize()
    assert torch.equal(b32["dlogits"], b16["dlogits"])
    assert torch.equal(mt.rne_bf16(b32["dh"]).view(torch.int16), b16["dh"].view(torch.int16))
    assert torch.equal(mt.rne_bf16(b32["dW"]).view(torch.int16), b16["dW"].view(torch.int16))
    check_bwd(b32, host, lse_ref)
    # the unfused baseline
    fu = L.ce_fwd(d["h"], d["W"], d["targets"], unfused=True)
    bu = L.ce_bwd(d["h"], d["W"], d["targets"], lse_ref.to(DEV), d["dloss"], dh_dtype=torch.float32,
                  dW_dtype=torch.float32, unfused=True)
    torch.cuda.synchronize()
    check_fwd(fu, ref, host["targets"])
    for k in ("dlogits", "dh", "dW"):
        assert torch.equal(bu[k], b32[k]), k
    # the forward storing its fp32 logits, and the backward reading them
    fs = L.ce_fwd(d["h"], d["W"], d["targets"], store_logits=True)
    bs = L.ce_bwd(d["h"], d["W"], d["targets"], lse_ref.to(DEV), d["dloss"], dh_dtype=torch.float32,
                  dW_dtype=torch.float32, logits=fs["logits"])
    torch.cuda.synchronize()
    assert torch.equal(fs["lse"], f["lse"]) and torch.equal(fs["loss"], f["loss"])
    e_logits = mt.normwise(fs["logits"], mt.f64(host["h"]) @ mt.f64(host["W"]).T)
    print(f"  stored logits max|d|/rms={e_logits:.3e}")
    assert e_logits <= 1e-5
    for k in ("dlogits", "dh", "dW"):
        assert torch.equal(bs[k], b32[k]), k


def test_ce_forward_then_backward_on_device():
    """The backward fed the device forward's lse: the same bounds hold (lse agrees to ~1e-6)."""
    c = SMALL["ragged"]
    announce(f"coda_ce_fwd -> coda_ce_bwd {c} seed=1")
    host = case_inputs(c, seed=1)
    d = {k: v.to(DEV) for k, v in host.items()}
    f = L.ce_fwd(d["h"], d["W"], d["targets"])
    b = L.ce_bwd(d["h"], d["W"], d["targets"], f["lse"], d["dloss"], dh_dtype=torch.float32, dW_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = orc.lm_head_cross_entropy(host["h"], host["W"], host["targets"])
    check_bwd(b, host, torch.from_numpy(ref["lse"]).to(torch.float32))


@pytest.mark.parametrize("mode", ["fused", "unfused", "stored"])
def test_ce_extreme_logits(mode):
    """Logits of size ~60 (a peaked softmax) and an all-equal row: the tile statistics keep exp in range.
    The ignored row 1 has logits above 88 (exp overflows fp32 there): its gradient is still exactly 0."""
    c = dict(M=32, D=256, V=768)
    announce(f"coda_ce_fwd / coda_ce_bwd extreme logits {c} mode={mode}")
    unfused = mode == "unfused"
    host = case_inputs(c, seed=2)
    host["W"] = (host["W"].float() * 30).to(torch.bfloat16)   # logits std ~60
    host["h"][5] = 0                                          # all logits 0: lse = log V, loss = log V
    assert host["targets"][1] == -100
    assert (mt.f64(host["h"][1]) @ mt.f64(host["W"]).T).max() > 89.0
    d = {k: v.to(DEV) for k, v in host.items()}
    f = L.ce_fwd(d["h"], d["W"], d["targets"], unfused=unfused, store_logits=mode == "stored")
    torch.cuda.synchronize()
    ref = orc.lm_head_cross_entropy(host["h"], host["W"], host["targets"])
    assert torch.all(torch.isfinite(f["lse"])) and torch.all(torch.isfinite(f["loss"]))
    assert abs(f["lse"][5].item() - np.log(768)) < 1e-5
    check_fwd(f, ref, host["targets"])
    lse_ref = torch.from_numpy(ref["lse"]).to(torch.float32)
    b = L.ce_bwd(d["h"], d["W"], d["targets"], lse_ref.to(DEV), d["dloss"], dh_dtype=torch.float32,
                 dW_dtype=torch.float32, unfused=unfused, logits=f.get("logits"))
    torch.cuda.synchronize()
    for k in ("dlogits", "dh", "dW"):
        assert torch.all(torch.isfinite(b[k].float())), k
    assert torch.all(b["dlogits"][1] == 0)
    check_bwd(b, host, lse_ref)


def test_ce_all_rows_ignored():
    """Every target outside [0, V) (negative and >= V): loss 0, lse still the row's log-sum-exp,
    and every gradient exactly 0."""
    c = dict(M=70, D=256, V=512)
    announce(f"coda_ce_fwd / coda_ce_bwd all rows ignored {c}")
    host = inputs.lm_head_inputs(c["M"], c["D"], c["V"], seed=5)
    host["targets"][:] = -100
    host["targets"][::3] = c["V"]           # past the vocabulary: also ignored
    d = {k: v.to(DEV) for k, v in host.items()}
    ref = orc.lm_head_cross_entropy(host["h"], host["W"], host["targets"])
    assert not ref["valid"].any()
    for unfused in (False, True):
        f = L.ce_fwd(d["h"], d["W"], d["targets"], unfused=unfused)
        b = L.ce_bwd(d["h"], d["W"], d["targets"], f["lse"], d["dloss"], dh_dtype=torch.float32,
                     dW_dtype=torch.float32, unfused=unfused)
        torch.cuda.synchronize()
        assert torch.all(f["loss"] == 0)
        assert mt.normwise(f["lse"], ref["lse"]) <= TOL
        for k in ("dlogits", "dh", "dW"):
            assert torch.all(b[k] == 0), (k, unfused)


@pytest.mark.slow
def test_ce_llama3_8b_lm_head_sampled():
    c = dict(M=8192, D=4096, V=inputs.LM_VOCAB)
    announce(f"coda_ce_fwd / coda_ce_bwd llama3_8b LM head {c} seed=0, sampled")
    host = case_inputs(c)
    rows = inputs.sample(c["M"], 256, 0, "rows").numpy()
    vrows = inputs.sample(c["V"], 256, 0, "dw_lm_rows").numpy()
    d = {k: v.to(DEV) for k, v in host.items()}
    f = L.ce_fwd(d["h"], d["W"], d["targets"])
    torch.cuda.synchronize()
    ref_all = orc.lm_head_cross_entropy(host["h"], host["W"], host["targets"])   # every row: dW needs them
    check_fwd(f, {k: v[rows] for k, v in ref_all.items()}, host["targets"], rows=rows)
    del f
    lse_ref = torch.from_numpy(ref_all["lse"]).to(torch.float32)
    b = L.ce_bwd(d["h"], d["W"], d["targets"], lse_ref.to(DEV), d["dloss"], dh_dtype=torch.float32,
                 dW_dtype=torch.float32)
    torch.cuda.synchronize()
    check_bwd(b, host, lse_ref, rows=rows, vrows=vrows)
    # from the forward's stored logits: the same gradients, bit for bit
    fs = L.ce_fwd(d["h"], d["W"], d["targets"], store_logits=True)
    bs = L.ce_bwd(d["h"], d["W"], d["targets"], lse_ref.to(DEV), d["dloss"], dh_dtype=torch.float32,
                  dW_dtype=torch.float32, logits=fs["logits"])
    torch.cuda.synchronize()
    for k in ("dlogits", "dh", "dW"):
        assert torch.equal(bs[k], b[k]), k


@pytest.mark.parametrize("stored", [False, True], ids=["recompute", "stored_logits"])
def test_ce_graph_capture(stored):
    """The LM head's forward and backward captured into one HIP graph (the backward on the
    forward's lse, with or without the stored logits): every replay reproduces the eager
    results bit for bit."""
    from graph_util import assert_replays_match_eager
    c = SMALL["ragged"]
    M, D, V = c["M"], c["D"], c["V"]
    announce(f"graph capture coda_ce_fwd + coda_ce_bwd {c} stored={stored}")
    d = {k: v.to(DEV) for k, v in case_inputs(c, seed=7).items()}
    fo = {"lse": torch.empty(M, dtype=torch.float32, device=DEV), "loss": torch.empty(M, dtype=torch.float32, device=DEV)}
    if stored:
        fo["logits"] = torch.empty(M, V, dtype=torch.float32, device=DEV)
    bo = {"dlogits": torch.empty(M, V, dtype=torch.bfloat16, device=DEV),
          "dh": torch.empty(M, D, dtype=torch.bfloat16, device=DEV),
          "dW": torch.empty(V, D, dtype=torch.bfloat16, device=DEV)}
    ws = L.workspace(L.CODA_OP_CE_FWD, M, D, V, DEV)

    def step():
        L.ce_fwd(d["h"], d["W"], d["targets"], ws=ws, out=fo)
        L.ce_bwd(d["h"], d["W"], d["targets"], fo["lse"], d["dloss"], out=bo, logits=fo.get("logits"))

    assert_replays_match_eager(step, list(fo.values()) + list(bo.values()))
