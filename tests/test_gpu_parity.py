"""Parity of the HIP path (through the C ABI) with the fp64 oracle on one MI355X.

Inputs are the seeded synthetic tensors of transformer_gemm_epilogue_res_amd.inputs;
expected values come only from oracle/. Small shapes are compared in full
(several 256-tiles, a ragged last row tile, a single row); the Llama-3 shapes run
in the same launch configuration the benchmark times and are compared on a
seeded 256-row sample (rows are independent) and, for the backward's column
sums, on seeded 256-column samples.
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


def announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


def to_dev(d):
    return {k: v.to(DEV) for k, v in d.items()}


# ------------------------------------------------------------------ mainloop

@pytest.mark.parametrize("a_layout", [L.CODA_ROW, L.CODA_COL], ids=["A_row", "A_col"])
@pytest.mark.parametrize("b_layout", [L.CODA_ROW, L.CODA_COL], ids=["B_row", "B_col"])
@pytest.mark.parametrize("M,N,K", [(320, 512, 768), (1, 512, 768), (320, 576, 448)])
def test_gemm_mainloop_layouts(a_layout, b_layout, M, N, K):
    announce(f"coda_gemm M={M} N={N} K={K} a_layout={a_layout} b_layout={b_layout}")
    g = torch.Generator().manual_seed(11)
    Am = torch.randn(M, K, generator=g).to(torch.bfloat16)     # logical A [M, K]
    Bm = torch.randn(K, N, generator=g).to(torch.bfloat16)     # logical B [K, N]
    if a_layout == L.CODA_ROW:
        A = Am
    else:  # [K, lda] with lda padded to a multiple of 8
        A = torch.zeros(K, (M + 7) // 8 * 8, dtype=torch.bfloat16)
        A[:, :M] = Am.t()
    B = Bm if b_layout == L.CODA_ROW else Bm.t().contiguous()
    Ad, Bd = A.to(DEV), B.to(DEV)
    C32 = L.gemm(Ad, Bd, a_layout, b_layout, torch.float32, M=M, N=N, K=K)
    C16 = L.gemm(Ad, Bd, a_layout, b_layout, torch.bfloat16, M=M, N=N, K=K)
    torch.cuda.synchronize()
    ref = orc.gemm(Am, Bm)
    assert mt.normwise(C32, ref) <= 1e-4
    assert torch.equal(mt.rne_bf16(C32).cpu().view(torch.int16), C16.cpu().view(torch.int16))


# ------------------------------------------------------------------ forward

FWD_SMALL = {
    "tiny": dict(M=64, K0=256, D=256, N=512),
    "ragged": dict(M=300, K0=256, D=512, N=768),
    "one_row": dict(M=1, K0=256, D=256, N=256),
    "k0_ne_d": dict(M=130, K0=768, D=256, N=512),
    "deep_k0": dict(M=64, K0=1024, D=256, N=512),     # GEMM0 split over K0 into 4 slices
    # sizes in multiples of 64: a last column tile of 64 (D) or 64 (N) live columns, K0 of 3 K steps
    "dims64": dict(M=300, K0=192, D=320, N=576),
    "dims64_split": dict(M=64, K0=1088, D=320, N=576),      # GEMM0 in 4 slices, the last one 2 K steps
    "dims64_rows": dict(M=24576, K0=192, D=320, N=576),     # 192 GEMM0 tiles: the fused epilogue, unsplit
    # GEMM1 combines r itself while its 128-row blocks of partials fit 16 KB (ceil(D / 256) <= 32) and it has
    # at most 512 tiles (every case above); else a separate kernel does: the two edges of that rule
    "folded_widest": dict(M=64, K0=256, D=8192, N=256),     # 32 partials per row: the whole staging area
    "unfolded_wide": dict(M=64, K0=256, D=8256, N=256),     # 33 partials per row
    "unfolded_tiles": dict(M=2048, K0=128, D=128, N=16640),  # 8 x 65 = 520 GEMM1 tiles
}


def run_fwd_both(dev_in, unfused=False):
    o32 = L.fwd(dev_in["x"], dev_in["W0"], dev_in["z"], dev_in["gamma"], dev_in["W1"], EPS, torch.float32,
                unfused=unfused)
    o16 = L.fwd(dev_in["x"], dev_in["W0"], dev_in["z"], dev_in["gamma"], dev_in["W1"], EPS, torch.bfloat16,
                unfused=unfused)
    torch.cuda.synchronize()
    return o32, o16


def check_fwd(o32, o16, ref, gamma, rows=None, unfused=False):
    def sel(t):
        return t.cpu() if rows is None else t.index_select(0, torch.as_tensor(rows, device=t.device)).cpu()
    y32, y16, r, h = sel(o32["y"]), sel(o16["y"]), sel(o32["r"]), sel(o32["h"])
    e_y = mt.normwise(y32, ref["y"])
    e_r = mt.max_rel(r, ref["r"])
    print(f"  y(fp32) max|d|/rms={e_y:.3e}  r max rel={e_r:.3e}")
    # the bf16 output is the round-to-nearest-even of the fp32 output of the same kernel
    assert torch.equal(mt.rne_bf16(y32).view(torch.int16), y16.view(torch.int16))
    assert torch.equal(sel(o16["r"]), r) and torch.equal(sel(o16["h"]), h)
    if unfused:
        assert e_y <= 3 * mt.Y_TOL
        assert mt.bf16_within(y16, ref["y"], 3 * mt.Y_TOL) <= 1.0
        # h = bf16(bf16(x@W0) + z): the rounding of t can exceed ulps of h where z cancels t
        assert mt.bf16_within(h, ref["h"], 3 * mt.Y_TOL) <= 1.0
    else:
        assert e_y <= mt.Y_TOL
        assert mt.bf16_within(y16, ref["y"]) <= 1.0
        assert mt.bf16_one_ulp(h, ref["h"]) <= 1.0
        g = sel(o32["g"])
        assert torch.equal(sel(o16["g"]), g)
        assert mt.bf16_one_ulp(g, ref["h"] * mt.f64(gamma)[None, :]) <= 1.0
    assert e_r <= mt.R_TOL


@pytest.mark.parametrize("name", list(FWD_SMALL))
@pytest.mark.parametrize("unfused", [False, True], ids=["fused", "unfused"])
def test_fwd_small_full(name, unfused):
    c = FWD_SMALL[name]
    announce(f"{'coda_unfused_ref' if unfused else 'coda_fwd'} {name} {c} seed=0")
    inp = inputs.forward_inputs(**c, seed=0)
    o32, o16 = run_fwd_both(to_dev(inp), unfused)
    ref = orc.forward(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], EPS)
    check_fwd(o32, o16, ref, inp["gamma"], unfused=unfused)


def test_fwd_special_rows():
    """Zero rows, constant rows and a NaN row (row isolation) through the fused kernels."""
    c = FWD_SMALL["ragged"]
    announce(f"coda_fwd special rows {c}")
    inp = inputs.forward_inputs(**c, seed=3)
    inp["x"][5] = 0
    inp["z"][5] = 0                                       # h row = 0 -> r = eps^-1/2, y row = 0
    inp["x"][7] = 0
    inp["z"][7] = 1.5                                     # constant row
    inp["x"][299, 3] = float("nan")                       # last (ragged) row
    o32, _ = run_fwd_both(to_dev(inp))
    y, r = o32["y"].cpu(), o32["r"].cpu()
    assert abs(r[5].item() / EPS ** -0.5 - 1) < 1e-6 and torch.all(y[5] == 0)
    assert abs(r[7].item() * (1.5 ** 2 + EPS) ** 0.5 - 1) < 1e-6
    bad = ~torch.isfinite(y).all(dim=1)
    assert bad.nonzero().flatten().tolist() == [299]
    keep = [i for i in range(c["M"]) if i != 299]
    ref = orc.forward(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], EPS, rows=keep)
    assert mt.normwise(y[keep], ref["y"]) <= mt.Y_TOL


FWD_LARGE = ["llama3_1b", "llama3_8b", "llama3_70b", "llama3_8b_dp8"]


@pytest.mark.slow
@pytest.mark.parametrize("name", FWD_LARGE)
def test_fwd_llama_shapes_sampled(name):
    c = inputs.CONFIGS[name]
    announce(f"coda_fwd {name} {c} seed=0, 256 sampled rows")
    inp = inputs.forward_inputs(**c, seed=0)
    rows = inputs.sample(c["M"], 256, 0, "rows").numpy()
    o32, o16 = run_fwd_both(to_dev(inp))
    ref = orc.forward(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], EPS, rows=rows)
    check_fwd(o32, o16, ref, inp["gamma"], rows=rows)


# ------------------------------------------------------------------ backward

def saved_set(inp, eps=EPS):
    """The forward's saved tensors, from the oracle forward rounded to their storage types."""
    f = orc.forward(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], eps)
    gam = orc.f64(inp["gamma"])
    return {"h": torch.from_numpy(f["h"]).to(torch.bfloat16),
            "g": torch.from_numpy(f["h"] * gam[None, :]).to(torch.bfloat16),
            "y": torch.from_numpy(f["y"]).to(torch.bfloat16),
            "r": torch.from_numpy(f["r"]).to(torch.float32)}


def run_bwd_both(dev, unfused=False):
    args = (dev["dY"], dev["y"], dev["h"], dev["g"], dev["r"], dev["gamma"], dev["W1"])
    o32 = L.bwd(*args, da_dtype=torch.float32, dW1_dtype=torch.float32, unfused=unfused)
    o16 = L.bwd(*args, da_dtype=torch.bfloat16, dW1_dtype=torch.bfloat16, unfused=unfused)
    torch.cuda.synchronize()
    return o32, o16


def check_bwd(o32, o16, host, rows=None, jcols=None, ncols=None, unfused=False, ref=None, sig=None, ref_rg=None):
    """ref: the oracle's exact backward; ref_rg: its dW1 on the one-rounding operand bf16(r g) that the
    weight-gradient GEMM contracts; sig: the sigma of that rounding (metrics.operand_rounding_sigma)."""
    args = (host["dY"], host["y"], host["h"], host["g"], host["r"], host["gamma"], host["W1"])
    if ref is None:
        ref = orc.backward(*args, rows=rows, dgamma_cols=jcols, dw1_cols=ncols)
    if ref_rg is None:   # only dW1 is wanted: one row and one dgamma column keep the rest cheap
        ref_rg = orc.backward(*args, rows=[0], dgamma_cols=[0], dw1_cols=ncols, round_rg=True)["dW1"]
    if sig is None:
        sig = mt.operand_rounding_sigma(host["g"], host["r"], host["dY"], ncols)

    def rsel(t):
        return t.cpu() if rows is None else t.index_select(0, torch.as_tensor(rows, device=t.device)).cpu()

    def csel(t, cols):
        return t.cpu() if cols is None else t.index_select(-1, torch.as_tensor(cols, device=t.device)).cpu()

    s, da = rsel(o32["s"]), rsel(o32["da"])
    dg, dW1 = csel(o32["dgamma"], jcols), csel(o32["dW1"], ncols)
    e = {"s": mt.normwise(s, ref["s"]), "da": mt.normwise(da, ref["da"]),
         "dgamma": mt.normwise(dg, ref["dgamma"]), "dW1": mt.normwise(dW1, ref["dW1"])}
    print("  " + "  ".join(f"{k} max|d|/rms={v:.3e}" for k, v in e.items()))
    assert torch.equal(mt.rne_bf16(da).view(torch.int16), rsel(o16["da"]).view(torch.int16))
    assert torch.equal(mt.rne_bf16(dW1).view(torch.int16), csel(o16["dW1"], ncols).view(torch.int16))
    assert torch.equal(rsel(o16["s"]), s) and torch.equal(csel(o16["dgamma"], jcols), dg)
    e_w = mt.within_sigma(dW1, ref["dW1"], sig)
    e_rg = mt.normwise(dW1, ref_rg)
    print(f"  dW1 vs the same rounded operand max|d|/rms={e_rg:.3e};  vs exact |d| / (1e-4 rms + "
          f"{mt.SIGMA_K} sigma of the operand rounding) max = {e_w:.3f}")
    assert e["s"] <= mt.S_TOL
    assert e_rg <= 1e-4
    assert e_w <= 1.0
    tol = 3 * mt.Y_TOL if unfused else mt.Y_TOL
    assert e["da"] <= tol and e["dgamma"] <= tol


BWD_SMALL = {
    "tiny": dict(M=64, K0=256, D=256, N=512),       # dW1 contracts over one K step
    "ragged": dict(M=300, K0=256, D=512, N=768),
    "one_row": dict(M=1, K0=256, D=256, N=256),
    "two_k_steps": dict(M=100, K0=256, D=256, N=512),  # dW1 contracts over two K steps (rows padded to 128)
    "dims64": dict(M=300, K0=192, D=320, N=576),          # the data gradient split in 2 slices
    "dims64_rows": dict(M=24576, K0=192, D=320, N=576),   # unsplit: the last column tile has one live wave
    # s from the dW1 GEMM's side work (at least 16 row tiles, D > 3840): its K steps are 64 rows of M
    "rowdot": dict(M=300, K0=256, D=4096, N=576),         # 5 K steps, a ragged last one; 64 live columns in the last tile
    "rowdot_k1": dict(M=40, K0=256, D=3904, N=320),       # one K step; 61 x 64 = 16 row tiles, the last one ragged
    "rowdot_k2": dict(M=100, K0=256, D=4096, N=256),      # two K steps
    "rowdot_k3": dict(M=150, K0=256, D=4096, N=512),      # three: the first, the one without a next DMA, the last
    "rowdot_wide": dict(M=130, K0=256, D=8192, N=320),    # 32 row tiles: one row per block and K step
    "rowdot_flush": dict(M=4100, K0=256, D=4096, N=320),  # 65 K steps: a flush after 64 and a tail of one
}


@pytest.mark.parametrize("name", list(BWD_SMALL))
@pytest.mark.parametrize("unfused", [False, True], ids=["fused", "unfused"])
def test_bwd_small_full(name, unfused):
    c = BWD_SMALL[name]
    announce(f"{'coda_unfused_ref' if unfused else 'coda_bwd'} {name} {c} seed=0")
    inp = inputs.forward_inputs(**c, seed=0)
    host = dict(saved_set(inp), dY=inputs.output_grad(c["M"], c["N"], seed=0), gamma=inp["gamma"], W1=inp["W1"])
    o32, o16 = run_bwd_both(to_dev(host), unfused)
    check_bwd(o32, o16, host, unfused=unfused)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["llama3_8b", "llama3_1b", "llama3_70b", "llama3_8b_dp8"])
def test_bwd_llama_shapes_sampled(name):
    c = inputs.CONFIGS[name]
    announce(f"coda_bwd {name} {c} seed=0 (saved set from the oracle forward), sampled")
    inp = inputs.forward_inputs(**c, seed=0)
    host = dict(saved_set(inp), dY=inputs.output_grad(c["M"], c["N"], seed=0), gamma=inp["gamma"], W1=inp["W1"])
    del inp
    rows = inputs.sample(c["M"], 256, 0, "rows").numpy()
    jcols = inputs.sample(c["D"], 256, 0, "dgamma_cols").numpy()
    ncols = inputs.sample(c["N"], 256, 0, "dw1_cols").numpy()
    o32, o16 = run_bwd_both(to_dev(host))
    check_bwd(o32, o16, host, rows=rows, jcols=jcols, ncols=ncols)


# ---------------------------------------------------------- the largest row count

MAX_ROWS = 1 << 22  # the entry points reject more rows (host validation)


def test_max_rows_forward_and_backward():
    """M = 2^22 rows, the largest the entry points accept, at the smallest widths: every launch
    at its largest grid (one block per row, 65536 row blocks of the transposed operand, 16384
    tile rows, the unfused kernels' 131072 row groups) and byte offsets past 2^31; forward and
    backward, fused and unfused. The inputs (2 GB each) are drawn on the device; the forward is
    checked on 256 sampled rows, the backward (on a saved set drawn directly, since its formulas
    hold for any saved tensors) on every row where dY is not zero and on every column."""
    M, K0, D, N = MAX_ROWS, 256, 256, 256
    announce(f"coda_fwd / coda_bwd M={M} K0={K0} D={D} N={N} seed=0, fused and unfused, sampled")
    dev = {"x": inputs.device_randn_bf16((M, K0), 0, "x", DEV),
           "z": inputs.device_randn_bf16((M, D), 0, "z", DEV),
           "W0": inputs.device_randn_bf16((K0, D), 0, "W0", DEV, scale=K0 ** -0.5),
           "gamma": inputs.device_randn_bf16((D,), 0, "gamma", DEV, scale=0.1, shift=1.0),
           "W1": inputs.device_randn_bf16((D, N), 0, "W1", DEV, scale=D ** -0.5)}
    rows = inputs.sample(M, 256, 0, "rows").numpy()
    ridx = torch.as_tensor(rows, device=DEV)
    gamma, W1 = dev["gamma"].cpu(), dev["W1"].cpu()
    ref = orc.forward(dev["x"].index_select(0, ridx).cpu(), dev["W0"].cpu(), dev["z"].index_select(0, ridx).cpu(),
                      gamma, W1, EPS)
    for unfused in (False, True):
        o32, o16 = run_fwd_both(dev, unfused=unfused)
        check_fwd(o32, o16, ref, gamma, rows=rows, unfused=unfused)
        del o32, o16
    del dev["x"], dev["z"]
    torch.cuda.empty_cache()
    # dY is zero outside a seeded set of rows spread over the whole range (and the last 64), so
    # dgamma and dW1, sums over all rows, are exactly the sums over those rows; the kernels still
    # run over all 2^22 rows, and on the zero rows s and da must come out exactly 0.
    R = np.union1d(inputs.sample(M, 4096, 0, "rows").numpy(), np.arange(M - 64, M))
    Ridx = torch.as_tensor(R, device=DEV)
    dY = torch.zeros(M, N, dtype=torch.bfloat16, device=DEV)
    dY.index_copy_(0, Ridx, inputs.device_randn_bf16((len(R), N), 0, "dY", DEV))
    dev.update(dY=dY,
               y=inputs.device_randn_bf16((M, N), 0, "y_s", DEV),
               h=inputs.device_randn_bf16((M, D), 0, "h_s", DEV, scale=2 ** 0.5),
               g=inputs.device_randn_bf16((M, D), 0, "g_s", DEV, scale=2 ** 0.5),
               r=inputs.device_uniform_f32((M,), 0, "r_s", DEV, 0.5, 1.0))
    sub = {k: dev[k].index_select(0, Ridx).cpu() for k in ("dY", "y", "h", "g", "r")}
    sub.update(gamma=gamma, W1=W1)
    ref_b = orc.backward(sub["dY"], sub["y"], sub["h"], sub["g"], sub["r"], gamma, W1)
    sig = mt.operand_rounding_sigma(sub["g"], sub["r"], sub["dY"])
    ref_rg = orc.backward(sub["dY"], sub["y"], sub["h"], sub["g"], sub["r"], gamma, W1, rows=[0], dgamma_cols=[0],
                          round_rg=True)["dW1"]
    zero_rows = torch.as_tensor(np.setdiff1d(inputs.sample(M, 256, 1, "rows").numpy(), R), device=DEV)
    assert zero_rows.numel() > 200
    for unfused in (False, True):
        o32, o16 = run_bwd_both(dev, unfused=unfused)
        check_bwd(o32, o16, sub, rows=R, unfused=unfused, ref=ref_b, sig=sig, ref_rg=ref_rg)
        for o in (o32, o16):
            assert not o["s"].index_select(0, zero_rows).any()
            assert not o["da"].index_select(0, zero_rows).any()
        del o32, o16


MAX_DIM = 1 << 20  # the entry points reject wider K0, D or N (host validation)
MAX_WIDTH = {"N": dict(M=256, K0=256, D=256, N=MAX_DIM), "D": dict(M=256, K0=256, D=MAX_DIM, N=256)}


@pytest.mark.parametrize("name", list(MAX_WIDTH))
def test_max_width_forward_and_backward(name):
    """The widest D or N the entry points accept (2^20): the longest row loops (the row statistics
    over 2^20 columns, the sums of squares over 16384 partials per row), contractions of 16384 K
    steps and 4096 tile columns; forward on 16 sampled rows, backward (on a saved set drawn directly)
    on 16 rows, 8 dgamma columns and 8 dW1 columns."""
    c = MAX_WIDTH[name]
    M, K0, D, N = c["M"], c["K0"], c["D"], c["N"]
    announce(f"coda_fwd / coda_bwd max {name}: M={M} K0={K0} D={D} N={N} seed=0, sampled")
    inp = inputs.forward_inputs(M, K0, D, N, seed=0)
    rows = inputs.sample(M, 16, 0, "rows").numpy()
    dev = to_dev(inp)
    ref = orc.forward(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], EPS, rows=rows)
    o32, o16 = run_fwd_both(dev)
    check_fwd(o32, o16, ref, inp["gamma"], rows=rows)
    del o32, o16, ref
    host = {"dY": inputs.output_grad(M, N, seed=0),
            "y": inputs.device_randn_bf16((M, N), 0, "y_s", DEV).cpu(),
            "h": inputs.device_randn_bf16((M, D), 0, "h_s", DEV, scale=2 ** 0.5).cpu(),
            "g": inputs.device_randn_bf16((M, D), 0, "g_s", DEV, scale=2 ** 0.5).cpu(),
            "r": inputs.device_uniform_f32((M,), 0, "r_s", DEV, 0.5, 1.0).cpu(),
            "gamma": inp["gamma"], "W1": inp["W1"]}
    jcols = inputs.sample(D, 8, 0, "dgamma_cols").numpy()
    ncols = inputs.sample(N, 8, 0, "dw1_cols").numpy()
    o32, o16 = run_bwd_both(to_dev(host))
    check_bwd(o32, o16, host, rows=rows, jcols=jcols, ncols=ncols)


# --------------------------------------------- backward through the first GEMM

BWD0_SMALL = {
    "tiny": dict(M=64, K0=256, D=256),
    "ragged": dict(M=300, K0=512, D=256),
    "one_row": dict(M=1, K0=256, D=512),
    "dims64": dict(M=300, K0=192, D=320),
}


def check_bwd_gemm0(o32, o16, ref, rows=None, cols=None):
    def rsel(t):
        return t.cpu() if rows is None else t.index_select(0, torch.as_tensor(rows, device=t.device)).cpu()

    def csel(t):
        return t.cpu() if cols is None else t.index_select(1, torch.as_tensor(cols, device=t.device)).cpu()

    dx, dW0 = rsel(o32["dx"]), csel(o32["dW0"])
    e = {"dx": mt.normwise(dx, ref["dx"]), "dW0": mt.normwise(dW0, ref["dW0"])}
    print("  " + "  ".join(f"{k} max|d|/rms={v:.3e}" for k, v in e.items()))
    assert torch.equal(mt.rne_bf16(dx).view(torch.int16), rsel(o16["dx"]).view(torch.int16))
    assert torch.equal(mt.rne_bf16(dW0).view(torch.int16), csel(o16["dW0"]).view(torch.int16))
    return e


@pytest.mark.parametrize("name", list(BWD0_SMALL))
def test_bwd_gemm0_small_full(name):
    # a plain pair of products of bf16 operands with fp32 accumulation: fp32-level agreement
    c = BWD0_SMALL[name]
    announce(f"coda_bwd_gemm0 {name} {c} seed=0 (dh random)")
    inp = inputs.forward_inputs(M=c["M"], K0=c["K0"], D=c["D"], N=256, seed=0)
    dh = inputs.upstream_grad(c["M"], c["D"], seed=0)
    d = to_dev({"dh": dh, "x": inp["x"], "W0": inp["W0"]})
    o32 = L.bwd_gemm0(d["dh"], d["x"], d["W0"], dx_dtype=torch.float32, dW0_dtype=torch.float32)
    o16 = L.bwd_gemm0(d["dh"], d["x"], d["W0"])
    torch.cuda.synchronize()
    e = check_bwd_gemm0(o32, o16, orc.backward_gemm0(dh, inp["x"], inp["W0"]))
    assert e["dx"] <= 1e-4 and e["dW0"] <= 1e-4


@pytest.mark.parametrize("name", ["tiny", "ragged"])
def test_bwd_gemm0_after_chain_backward(name):
    # the whole chain's backward on the GPU (da stored as bf16 and fed on) against
    # the oracle's composition: the error is the bf16 rounding of da
    c = BWD_SMALL[name]
    announce(f"coda_bwd -> coda_bwd_gemm0 {name} {c} seed=0")
    inp = inputs.forward_inputs(**c, seed=0)
    host = dict(saved_set(inp), dY=inputs.output_grad(c["M"], c["N"], seed=0), gamma=inp["gamma"], W1=inp["W1"])
    dev = to_dev(dict(host, x=inp["x"], W0=inp["W0"]))
    b = L.bwd(dev["dY"], dev["y"], dev["h"], dev["g"], dev["r"], dev["gamma"], dev["W1"])
    o32 = L.bwd_gemm0(b["da"], dev["x"], dev["W0"], dx_dtype=torch.float32, dW0_dtype=torch.float32)
    o16 = L.bwd_gemm0(b["da"], dev["x"], dev["W0"])
    torch.cuda.synchronize()
    ref_b = orc.backward(host["dY"], host["y"], host["h"], host["g"], host["r"], host["gamma"], host["W1"])
    e = check_bwd_gemm0(o32, o16, orc.backward_gemm0(ref_b["da"], inp["x"], inp["W0"]))
    assert e["dx"] <= mt.Y_TOL and e["dW0"] <= mt.Y_TOL


@pytest.mark.slow
def test_bwd_gemm0_llama3_8b_sampled():
    c = inputs.CONFIGS["llama3_8b"]
    announce(f"coda_bwd_gemm0 llama3_8b M={c['M']} K0={c['K0']} D={c['D']} seed=0 (dh random), sampled")
    inp = inputs.forward_inputs(**c, seed=0)
    dh = inputs.upstream_grad(c["M"], c["D"], seed=0)
    rows = inputs.sample(c["M"], 256, 0, "rows").numpy()
    cols = inputs.sample(c["D"], 256, 0, "dw0_cols").numpy()
    d = to_dev({"dh": dh, "x": inp["x"], "W0": inp["W0"]})
    o32 = L.bwd_gemm0(d["dh"], d["x"], d["W0"], dx_dtype=torch.float32, dW0_dtype=torch.float32)
    o16 = L.bwd_gemm0(d["dh"], d["x"], d["W0"])
    torch.cuda.synchronize()
    e = check_bwd_gemm0(o32, o16, orc.backward_gemm0(dh, inp["x"], inp["W0"], rows=rows, dw0_cols=cols),
                        rows=rows, cols=cols)
    assert e["dx"] <= 1e-4 and e["dW0"] <= 1e-4


# ------------------------------------------------------ determinism, canaries

def shape(name):
    return FWD_SMALL[name] if name in FWD_SMALL else BWD_SMALL[name]


@pytest.mark.parametrize("name", ["ragged", "rowdot", "rowdot_flush"])
def test_run_to_run_bitwise_determinism(name):
    c = shape(name)
    announce(f"determinism coda_fwd/coda_bwd {name} {c}")
    inp = to_dev(inputs.forward_inputs(**c, seed=1))
    a = L.fwd(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], EPS)
    b = L.fwd(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], EPS)
    torch.cuda.synchronize()
    for k in ("h", "g", "r", "y"):
        assert torch.equal(a[k], b[k]), k
    dY = inputs.output_grad(c["M"], c["N"], seed=1).to(DEV)
    args = (dY, a["y"], a["h"], a["g"], a["r"], inp["gamma"], inp["W1"])
    p, q = L.bwd(*args), L.bwd(*args)
    torch.cuda.synchronize()
    for k in ("da", "dgamma", "dW1", "s"):
        assert torch.equal(p[k], q[k]), k


@pytest.mark.parametrize("name", ["ragged", "unfolded_wide", "rowdot", "rowdot_flush"])
def test_stages_match_whole_call(name):
    """coda_fwd_stage / coda_bwd_stage 0..n-1 in order give the whole call's results bit for bit, whether
    GEMM1 combines r itself (ragged: stage 1 launches nothing) or a separate kernel does (unfolded_wide),
    whether s comes from a row kernel or from the dW1 GEMM's side work (rowdot), and whether the data
    gradient is split over its contraction (rowdot) or not (rowdot_flush, 17 row tiles)."""
    c = shape(name)
    announce(f"stages vs whole call {name} {c}")
    M, D, N = c["M"], c["D"], c["N"]
    inp = to_dev(inputs.forward_inputs(**c, seed=5))
    dY = inputs.output_grad(M, N, seed=5).to(DEV)
    sp = L.current_stream(DEV)

    def fwd_out():
        return {"h": torch.empty(M, D, dtype=torch.bfloat16, device=DEV),
                "g": torch.empty(M, D, dtype=torch.bfloat16, device=DEV),
                "r": torch.empty(M, dtype=torch.float32, device=DEV),
                "y": torch.empty(M, N, dtype=torch.bfloat16, device=DEV)}

    def bwd_out():
        return {"da": torch.empty(M, D, dtype=torch.bfloat16, device=DEV),
                "dgamma": torch.empty(D, dtype=torch.float32, device=DEV),
                "dW1": torch.empty(D, N, dtype=torch.bfloat16, device=DEV),
                "s": torch.empty(M, dtype=torch.float32, device=DEV)}

    res = []
    for staged in (False, True):
        fo, bo = fwd_out(), bwd_out()
        for t in list(fo.values()) + list(bo.values()):
            t.fill_(float("nan"))
        F = L.bind_fwd(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], EPS, fo,
                       L.workspace(L.CODA_OP_FWD, M, D, N, DEV))
        B = L.bind_bwd(dY, fo["y"], fo["h"], fo["g"], fo["r"], inp["gamma"], inp["W1"], bo,
                       L.workspace(L.CODA_OP_BWD, M, D, N, DEV))
        for obj in (F, B):
            if staged:
                for i in range(obj.nstages):
                    obj.stage(i, sp)
            else:
                obj.run(sp)
        torch.cuda.synchronize()
        res.append(dict(fo, **bo))
    for k in res[0]:
        assert torch.equal(res[0][k], res[1][k]), k
    assert torch.isfinite(res[1]["r"]).all() and torch.isfinite(res[1]["y"].float()).all()


GUARD = 4096  # elements of guard band on each side of every output


def guarded(shape, dtype):
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * GUARD,), 0, dtype=dtype, device=DEV)
    buf.view(torch.uint8).fill_(0x5A)
    return buf, buf[GUARD:GUARD + n].view(*shape)


def guards_intact(buf):
    n = buf.numel()
    g = torch.cat([buf[:GUARD], buf[n - GUARD:]]).view(torch.uint8)
    return bool(torch.all(g == 0x5A).item())


@pytest.mark.parametrize("name,M", [("ragged", 300), ("ragged", 1), ("dims64", 300), ("dims64_rows", 24576),
                                    ("unfolded_wide", 64), ("rowdot", 300), ("rowdot_k1", 1), ("rowdot_wide", 130)])
def test_no_writes_outside_outputs(name, M):
    c = dict(shape(name), M=M)
    announce(f"canaries coda_fwd/coda_bwd {c}")
    inp = to_dev(inputs.forward_inputs(**c, seed=2))
    D, N = c["D"], c["N"]
    bufs, out = {}, {}
    for k, shp, dt in (("h", (M, D), torch.bfloat16), ("g", (M, D), torch.bfloat16), ("r", (M,), torch.float32),
                       ("y", (M, N), torch.bfloat16)):
        bufs[k], out[k] = guarded(shp, dt)
    wsb = L.workspace_bytes(L.CODA_OP_FWD, M, D, N)
    bufs["ws"], ws = guarded((wsb,), torch.uint8)
    L.fwd(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], EPS, ws=ws, out=out)
    dY = inputs.output_grad(M, N, seed=2).to(DEV)
    bo = {}
    for k, shp, dt in (("da", (M, D), torch.float32), ("dgamma", (D,), torch.float32),
                       ("dW1", (D, N), torch.bfloat16), ("s", (M,), torch.float32)):
        bufs["b" + k], bo[k] = guarded(shp, dt)
    wsb = L.workspace_bytes(L.CODA_OP_BWD, M, D, N)
    bufs["bws"], bws = guarded((wsb,), torch.uint8)
    L.bwd(dY, out["y"], out["h"], out["g"], out["r"], inp["gamma"], inp["W1"], ws=bws, out=bo)
    torch.cuda.synchronize()
    for k, b in bufs.items():
        assert guards_intact(b), k
    assert torch.isfinite(out["y"].float()).all() and torch.isfinite(bo["da"]).all()


@pytest.mark.parametrize("name", ["ragged", "rowdot", "rowdot_flush"])
def test_graph_capture_replays_match_eager(name):
    """The step (coda_fwd + coda_bwd) captured into a HIP graph: the library allocates, frees and
    clears nothing, so every replay reproduces the eager results bit for bit."""
    c = shape(name)
    announce(f"graph capture coda_fwd + coda_bwd {name} {c}")
    M, D, N = c["M"], c["D"], c["N"]
    inp = to_dev(inputs.forward_inputs(**c, seed=4))
    dY = inputs.output_grad(M, N, seed=4).to(DEV)
    fo = {"h": torch.empty(M, D, dtype=torch.bfloat16, device=DEV), "g": torch.empty(M, D, dtype=torch.bfloat16, device=DEV),
          "r": torch.empty(M, dtype=torch.float32, device=DEV), "y": torch.empty(M, N, dtype=torch.bfloat16, device=DEV)}
    bo = {"da": torch.empty(M, D, dtype=torch.bfloat16, device=DEV), "dgamma": torch.empty(D, dtype=torch.float32, device=DEV),
          "dW1": torch.empty(D, N, dtype=torch.bfloat16, device=DEV), "s": torch.empty(M, dtype=torch.float32, device=DEV)}
    fws = L.workspace(L.CODA_OP_FWD, M, D, N, DEV)
    bws = L.workspace(L.CODA_OP_BWD, M, D, N, DEV)

    def step():
        L.fwd(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], EPS, ws=fws, out=fo)
        L.bwd(dY, fo["y"], fo["h"], fo["g"], fo["r"], inp["gamma"], inp["W1"], ws=bws, out=bo)

    step()
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in list(fo.items()) + list(bo.items())}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in list(fo.values()) + list(bo.values()):
            t.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in list(fo.items()) + list(bo.items()):
            assert torch.equal(v, want[k]), (rep, k)


def test_binding_reports_errors_without_launch():
    inp = to_dev(inputs.forward_inputs(**FWD_SMALL["tiny"], seed=0))
    with pytest.raises(L.CodaError) as e:
        L.fwd(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], 0.0)
    assert e.value.status == L.CODA_ERR_ARG


def test_binding_checks_outputs_and_workspace_bytes():
    """Outputs of the wrong shape or on the host are refused before any launch; a workspace is measured
    in bytes whatever its dtype (a float32 workspace of exactly the needed bytes works; one byte short of
    it is rejected by the library's own check)."""
    c = FWD_SMALL["ragged"]
    M, D, N = c["M"], c["D"], c["N"]
    announce(f"binding misuse checks {c}")
    inp = to_dev(inputs.forward_inputs(**c, seed=0))
    args = (inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], EPS)

    def outs(**over):
        o = {"h": torch.empty(M, D, dtype=torch.bfloat16, device=DEV), "g": torch.empty(M, D, dtype=torch.bfloat16, device=DEV),
             "r": torch.empty(M, dtype=torch.float32, device=DEV), "y": torch.empty(M, N, dtype=torch.float32, device=DEV)}
        o.update(over)
        return o
    with pytest.raises(ValueError):
        L.fwd(*args, out=outs(y=torch.empty(M, N - 256, dtype=torch.float32, device=DEV)))
    with pytest.raises(ValueError):
        L.fwd(*args, out=outs(h=torch.empty(M, D, dtype=torch.bfloat16)))
    with pytest.raises(TypeError):
        L.fwd(*args, out=outs(r=torch.empty(M, dtype=torch.bfloat16, device=DEV)))
    need = L.workspace_bytes(L.CODA_OP_FWD, M, D, N)
    assert need % 4 == 0
    ref = L.fwd(*args, torch.float32)
    got = L.fwd(*args, ws=torch.empty(need // 4, dtype=torch.float32, device=DEV), out=outs())
    torch.cuda.synchronize()
    assert torch.equal(ref["y"], got["y"]) and torch.equal(ref["r"], got["r"])
    with pytest.raises(L.CodaError) as e:
        L.fwd(*args, ws=torch.empty(need - 1, dtype=torch.uint8, device=DEV), out=outs())
    assert e.value.status == L.CODA_ERR_WORKSPACE
