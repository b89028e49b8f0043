"""coda_fwd_noalloc (the forward whose partials live in the library's own device scratch) against
coda_fwd, through the C ABI, on two calls in a row with the second on a smaller input, then the first
input again (the scratch keeps the previous call's contents, which no call may depend on)."""
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

# first call: 256 GEMM0 tiles, where coda_fwd does not split GEMM0 either (the same kernels: bitwise
# equal results); second call: smaller in every dimension, where coda_fwd splits GEMM0 over K0 and the
# no-allocation forward does not (equal up to fp32 summation order)
BIG = dict(M=4000, K0=256, D=4096, N=512)
SMALL = dict(M=64, K0=512, D=256, N=256)


def run_pair(c, seed):
    inp = inputs.forward_inputs(**c, seed=seed)
    d = {k: v.to(DEV) for k, v in inp.items()}
    args = (d["x"], d["W0"], d["z"], d["gamma"], d["W1"], EPS, torch.float32)
    print(f"\n[gpu-case] coda_fwd_noalloc vs coda_fwd {c} seed={seed}", flush=True)
    got = L.fwd_noalloc(*args)
    want = L.fwd(*args)
    torch.cuda.synchronize()
    return inp, got, want


def test_no_alloc_forward_matches_coda_fwd_on_consecutive_calls():
    inp, got, want = run_pair(BIG, 0)
    for k in ("h", "g", "r", "y"):
        assert torch.equal(got[k], want[k]), k
    first = {k: v.clone() for k, v in got.items()}

    inp, got, want = run_pair(SMALL, 1)
    assert mt.normwise(got["y"], want["y"].cpu()) <= 1e-4
    assert mt.max_rel(got["r"], want["r"].cpu()) <= 1e-5
    for k in ("h", "g"):
        assert mt.bf16_one_ulp(got[k], want[k].cpu()) <= 1.0, k
    ref = orc.forward(inp["x"], inp["W0"], inp["z"], inp["gamma"], inp["W1"], EPS)
    assert mt.normwise(got["y"], ref["y"]) <= mt.Y_TOL
    assert mt.max_rel(got["r"], ref["r"]) <= mt.R_TOL
    assert mt.bf16_one_ulp(got["h"], ref["h"]) <= 1.0

    _, got, _ = run_pair(BIG, 0)
    for k in ("h", "g", "r", "y"):
        assert torch.equal(got[k], first[k]), k


def test_no_alloc_forward_rejects_sizes_beyond_its_scratch():
    M, D = (16 << 20) // ((4096 // 256) * 4) + 1, 4096   # partials M * ceil(D / 256) * 4 bytes: one row past 16 MiB
    x = torch.empty(M, 256, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(L.CodaError) as e:
        L.fwd_noalloc(x, torch.empty(256, D, dtype=torch.bfloat16, device=DEV),
                      torch.empty(M, D, dtype=torch.bfloat16, device=DEV),
                      torch.empty(D, dtype=torch.bfloat16, device=DEV),
                      torch.empty(D, 256, dtype=torch.bfloat16, device=DEV), EPS)
    assert e.value.status == L.CODA_ERR_WORKSPACE
