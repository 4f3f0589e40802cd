"""Static checks of the built library's gfx950 code (no GPU needed).

The kernels that issue MFMAs from inline asm rely on their own placement of
wait states; the register allocator may still put a copy or a spill next to
an MFMA.  These tests read the AMD assembly of the library as built
(tests/isa_check.py) and check, on every control-flow path, that no
instruction touches an MFMA's result before the wait the compiler itself
would insert for that MFMA shape, and that no MFMA reads a register a VALU
instruction has just written.  They also check that the head and GEMM
kernels keep every value in registers (no scratch), and that the checker
itself catches both kinds of mistake when one is planted into a kernel's
instruction list.
"""
import os

import pytest

import invariant_logprobs_amd as tim
import isa_check as ic

pytestmark = pytest.mark.skipif(not ic.tools_available() or not os.path.exists(tim.LIB_PATH),
                                reason="needs the ROCm LLVM tools and the built library")

MFMA_KERNELS = ("lmhead8w_kernel", "lmhead_narrow_kernel", "lmhead_partials_kernel",
                "gemm8w_kernel")
# kernels whose every value must stay in registers (the statistics stream
# keeps its row ring in registers: a scratch spill would put memory
# operations between a row's loads and the waits that count them)
NO_SCRATCH = ("lmhead8w_kernelILb0E", "lmhead_narrow_kernel", "gemm8w_kernelILi1E",
              "gemm8w_kernelILi2E", "stats_stream_kernel")


@pytest.fixture(scope="module")
def kernels():
    return ic.kernels(tim.LIB_PATH)


def test_required_waits_come_from_the_compiler():
    w = ic.required_waits()
    assert set(w) == {"v_mfma_f32_16x16x32_bf16", "v_mfma_f32_32x32x16_bf16",
                      "v_mfma_f32_32x32x2_f32"}
    # more passes need more wait states; none exceeds the largest table entry
    assert 0 < w["v_mfma_f32_16x16x32_bf16"] < w["v_mfma_f32_32x32x16_bf16"] \
        < w["v_mfma_f32_32x32x2_f32"] <= ic.MFMA_WAIT


def test_every_mfma_kernel_is_found(kernels):
    with_mfma = [k for k, code in kernels.items() if any(i.is_mfma for i in code)]
    for name in MFMA_KERNELS:
        assert any(name in k for k in with_mfma), name


@pytest.mark.parametrize("name", MFMA_KERNELS)
def test_no_mfma_hazard(kernels, name):
    found = 0
    for k, code in kernels.items():
        if name not in k:
            continue
        found += 1
        bad = ic.check_kernel(code)
        assert not bad, f"{k}:\n" + "\n".join(bad[:10])
    assert found


@pytest.mark.parametrize("name", MFMA_KERNELS)
def test_no_lds_read_destination_is_read_before_its_wait(kernels, name):
    found = 0
    for k, code in kernels.items():
        if name not in k:
            continue
        found += 1
        bad = ic.check_lds_reads(code)
        assert not bad, f"{k}:\n" + "\n".join(bad[:10])
    assert found


def test_checker_catches_a_copy_planted_between_a_read_and_its_wait(kernels):
    code = next(c for k, c in kernels.items() if "gemm8w_kernelILi3ELb1E" in k)
    assert not ic.check_lds_reads(code)
    k = next(i for i, ins in enumerate(code) if ins.op == "ds_read_b64_tr_b16")
    r = sorted(r for f, r in code[k].dst if f == "v")[-1]
    plant = ic.Insn(code[k].addr + 1, "v_mov_b32_e32", f"v0, v{r}", None)
    bad = ic.check_lds_reads(code[:k + 1] + [plant] + code[k + 1:])
    assert any(f"v_mov_b32_e32 v0, v{r}" in b for b in bad)


def test_head_gemm_and_stats_stream_kernels_use_no_scratch():
    sizes = ic.private_segment_sizes(tim.LIB_PATH)
    checked = 0
    for k, size in sizes.items():
        if any(n in k for n in NO_SCRATCH):
            checked += 1
            assert size == 0, f"{k}: {size} bytes of scratch per lane"
    assert checked >= 11


def _head_kernel(kernels):
    return next(code for k, code in kernels.items() if "lmhead8w_kernelILb0E" in k)


def test_checker_catches_a_read_planted_after_an_mfma(kernels):
    code = list(_head_kernel(kernels))
    assert not ic.check_kernel(code)
    k = max(i for i, ins in enumerate(code) if ins.is_mfma)
    a = sorted(r for f, r in code[k].dst if f == "a")[0]
    plant = ic.Insn(code[k].addr + 1, "v_accvgpr_read_b32", f"v0, a{a}", None)
    mutated = code[:k + 1] + [plant] + code[k + 1:]
    bad = ic.check_kernel(mutated)
    assert any("v_accvgpr_read_b32 v0" in b for b in bad)


def test_checker_catches_a_write_planted_before_an_mfma(kernels):
    code = list(_head_kernel(kernels))
    k = max(i for i, ins in enumerate(code) if ins.is_mfma)
    src = sorted(r for f, r in code[k].regs - code[k].dst if f == "v")[0]
    plant = ic.Insn(code[k].addr - 1, "v_mov_b32_e32", f"v{src}, 0", None)
    mutated = code[:k] + [plant] + code[k:]
    bad = ic.check_kernel(mutated)
    assert any(f"0 wait states after v_mov_b32_e32 v{src}" in b for b in bad)


def test_register_ranges_are_parsed():
    assert ic.regs("a[0:3], v[98:101], v7, s[4:7]") == \
        {("a", 0), ("a", 1), ("a", 2), ("a", 3), ("v", 98), ("v", 99), ("v", 100),
         ("v", 101), ("v", 7)}
