"""The hand-scheduled mainloop's assembly obeys its wait and hazard rules (CPU only).

The LDS fragment reads and the MFMAs are inline asm, so the compiler neither
waits for those loads nor pads MFMA result reads; the check compiles the
kernels to gfx950 assembly and verifies both by static analysis."""
import pytest

import check_lds_waits as chk


@pytest.fixture(scope="module")
def asm():
    return chk.device_asm()


def test_every_kernel_waits_for_its_lds_loads_and_mfma_results(asm):
    funcs = chk.split_functions(asm)
    assert sum("gemm_kernel" in n for n in funcs) >= 13
    report = chk.check(asm)
    assert report == {}, {k[:60]: v[:3] for k, v in report.items()}


def test_checker_catches_a_missing_wait(asm):
    funcs = chk.split_functions(asm)
    name = next(n for n in funcs if "gemm_kernel" in n)
    body = funcs[name]
    cut = "s_waitcnt lgkmcnt(0)"
    i = body.index(cut, body.index("v_mfma"))  # a wait inside the mainloop
    assert chk.check_function(name, body[:i] + "s_nop 0" + body[i + len(cut):])


def test_checker_catches_an_early_accumulator_read(asm):
    funcs = chk.split_functions(asm)
    name = next(n for n in funcs if "gemm_kernel" in n)
    body = funcs[name]
    i = body.rindex("v_mfma_f32_16x16x32_bf16")
    j = body.index("\n", i)
    dst = body[i:j].split()[1].rstrip(",").replace("[", "").split(":")[0]
    assert chk.check_function(name, body[:j] + f"\n\tv_accvgpr_read_b32 v0, {dst}" + body[j:])
