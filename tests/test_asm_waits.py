"""The inline-asm LDS reads of the bf16 forward and the backward kernels are
waited for before their registers are used, and their inline-asm matrix
products are spaced from the instructions around them (tests/asm_waits.py),
checked in the gfx950 assembly the build flags produce; a weakened wait, a
wait that no longer holds back a builtin product and a missing drain in
copies of the sources are caught, and the walks are checked on short
sequences (branches and loops included)."""
import os
import shutil
import subprocess

import pytest

from sequence_transformer_attention_amd import build
from tests import asm_waits

CSRC = build.CSRC
HIPCC = build.hipcc()
pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")

KERNELS = {
    "ra_kernels.hip": ["_ZN12_GLOBAL__N_120attn_bf16_w64_kernelILi128EEEv10RaAttnArgs",
                       "_ZN12_GLOBAL__N_120attn_bf16_w64_kernelILi64EEEv10RaAttnArgs"],
    "ra_bwd.hip": ["_ZN12_GLOBAL__N_113bwd_dq_kernelILi128EEEv9RaBwdArgs",
                   "_ZN12_GLOBAL__N_113bwd_dq_kernelILi64EEEv9RaBwdArgs",
                   "_ZN12_GLOBAL__N_115bwd_dkdv_kernelILi128EEEv9RaBwdArgs",
                   "_ZN12_GLOBAL__N_115bwd_dkdv_kernelILi64EEEv9RaBwdArgs"],
}


def device_asm(src: str, out: str) -> str:
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [HIPCC] + flags + ["-I", CSRC, "-x", "hip", "--cuda-device-only", "-S", src, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out) as f:
        return f.read()


@pytest.mark.parametrize("source", sorted(KERNELS))
def test_every_lds_read_is_waited_for(source, tmp_path):
    asm = device_asm(os.path.join(CSRC, source), str(tmp_path / "k.s"))
    for sym in KERNELS[source]:
        nreads, nwaits, bad = asm_waits.check(asm_waits.kernel_lines(asm, sym))
        assert nreads > 0 and nwaits > 0, sym
        assert not bad, (sym, bad[:5])


def test_a_weakened_wait_is_caught(tmp_path):
    # the dQ kernel's wait for a unit's K rows, dropped in a copy of the source
    with open(os.path.join(CSRC, "ra_bwd.hip")) as f:
        src = f.read()
    tag = ('asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fk[0]), "+v"(fk[1]), "+v"(fk[2]), "+v"(fk[3]), "+v"(fk[4]),\n'
           '                     "+v"(fk[5]), "+v"(fk[6]), "+v"(fk[7]));')
    assert src.count(tag) == 1
    mutant = tmp_path / "ra_bwd.hip"
    mutant.write_text(src.replace(tag, 'asm volatile("" : "+v"(fk[0]), "+v"(fk[1]), "+v"(fk[2]), "+v"(fk[3]), '
                                       '"+v"(fk[4]), "+v"(fk[5]), "+v"(fk[6]), "+v"(fk[7]));'))
    for h in ("ra_bwd.h", "ra_plan.h", "ra_launch.h"):
        shutil.copy(os.path.join(CSRC, h), tmp_path / h)
    asm = device_asm(str(mutant), str(tmp_path / "m.s"))
    _, _, bad = asm_waits.check(asm_waits.kernel_lines(asm, KERNELS["ra_bwd.hip"][0]))
    assert bad


@pytest.mark.parametrize("source", sorted(KERNELS))
def test_matrix_products_are_spaced(source, tmp_path):
    asm = device_asm(os.path.join(CSRC, source), str(tmp_path / "k.s"))
    for sym in KERNELS[source]:
        lines = asm_waits.kernel_lines(asm, sym)
        assert "v_mfma" in "\n".join(lines), sym
        bad = asm_waits.check_mfma_results(lines)
        assert not bad, (sym, bad[:5])
        bad = asm_waits.check_mfma_operands(lines)
        assert not bad, (sym, bad[:5])


def mutant_asm(tmp_path, source: str, tag: str, repl: str) -> str:
    with open(os.path.join(CSRC, source)) as f:
        src = f.read()
    assert src.count(tag) == 1
    (tmp_path / source).write_text(src.replace(tag, repl))
    for h in ("ra_bwd.h", "ra_plan.h", "ra_launch.h"):
        if os.path.exists(os.path.join(CSRC, h)):
            shutil.copy(os.path.join(CSRC, h), tmp_path / h)
    return device_asm(str(tmp_path / source), str(tmp_path / "m.s"))


def test_a_missing_drain_is_caught(tmp_path):
    # the backward's drain between the S and dP chains and the vector code
    # that reads their results, emptied in a copy of the source
    asm = mutant_asm(tmp_path, "ra_bwd.hip",
                     'void qk_drain(f32x16& c) { asm volatile("s_nop 7\\n\\ts_nop 3" : "+v"(c)); }',
                     'void qk_drain(f32x16& c) { asm volatile("" : "+v"(c)); }')
    assert any(asm_waits.check_mfma_results(asm_waits.kernel_lines(asm, sym)) for sym in KERNELS["ra_bwd.hip"])


def test_the_spacing_walks_on_short_sequences():
    # a vector write right before an MFMA that reads it, then spaced; an MFMA
    # result read 5 and 12 wait states later; an accumulating MFMA right after
    # (allowed).  (The compiler itself puts an s_nop 0 in front of an asm
    # MFMA after a vector write, so no source change of the kernels shows
    # the first case.)
    close = ["v_cvt_pk_bf16_f32 v26, v26, v46", "s_waitcnt lgkmcnt(8)",
             "v_mfma_f32_32x32x16_bf16 a[64:79], v[34:37], v[24:27], a[64:79]"]
    assert asm_waits.check_mfma_operands(close)
    assert not asm_waits.check_mfma_operands(close[:2] + ["s_nop 0"] + close[2:])
    prod = ["v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0"]
    read = ["v_add_f32_e32 v30, v3, v31"]
    assert asm_waits.check_mfma_results(prod + ["s_nop 3"] + read)
    assert not asm_waits.check_mfma_results(prod + ["s_nop 7", "s_nop 3"] + read)
    assert not asm_waits.check_mfma_results(prod + ["v_mfma_f32_32x32x16_bf16 v[0:15], v[24:27], v[20:23], v[0:15]"])
    assert asm_waits.check_mfma_results(prod + ["v_mfma_f32_32x32x16_bf16 v[32:47], v[0:3], v[20:23], 0"])


def test_the_walks_follow_branches():
    # a read waited for on the fall-through path only, used where the paths
    # join; waited for on both paths (clean)
    rd = ["ds_read_b128 v[0:3], v10", "s_cbranch_scc1 .LBB0_2", "s_waitcnt lgkmcnt(0)", ".LBB0_2:",
          "v_mov_b32_e32 v20, v0"]
    assert asm_waits.check(rd)[2]
    assert not asm_waits.check(rd[:1] + ["s_waitcnt lgkmcnt(0)"] + rd[1:])[2]
    # a read issued at the end of a loop body and used at its head before a
    # wait: seen on the pass that takes the backward branch's state
    loop = [".LBB0_1:", "v_add_f32_e32 v20, v0, v1", "ds_read_b128 v[0:3], v10", "s_cbranch_scc1 .LBB0_1",
            "s_waitcnt lgkmcnt(0)"]
    assert asm_waits.check(loop)[2]
    assert not asm_waits.check(loop[:1] + ["s_waitcnt lgkmcnt(0)"] + loop[1:])[2]
    # an MFMA result drained on the fall-through only; an unconditional
    # branch over a block leaves that block's state out of the join
    prod = ["v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]", "s_cbranch_scc1 .LBB0_2",
            "s_nop 7", "s_nop 7", ".LBB0_2:", "v_mov_b32_e32 v30, v0"]
    assert asm_waits.check_mfma_results(prod)
    assert not asm_waits.check_mfma_results(prod[:1] + ["s_nop 7", "s_nop 7"] + prod[1:])
    skip = ["s_branch .LBB0_3", "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]", ".LBB0_3:",
            "s_nop 7", "s_nop 3", "v_mov_b32_e32 v30, v0"]
    assert not asm_waits.check_mfma_results(skip)
    assert asm_waits.check_mfma_results(skip[:2] + skip[3:4] + ["v_mov_b32_e32 v30, v0"])


def test_a_wait_that_does_not_hold_back_a_builtin_product_is_caught(tmp_path):
    # the dQ kernel's products are builtins: a wait that takes their V row
    # fragment only as an input lets the compiler move the product above it,
    # onto a register its LDS read has yet to write
    asm = mutant_asm(tmp_path, "ra_bwd.hip",
                     'asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(fv[c]) : "n"(n));',
                     'asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(n), "v"(fv[c]));')
    _, _, bad = asm_waits.check(asm_waits.kernel_lines(asm, KERNELS["ra_bwd.hip"][0]))
    assert any(why == "uses a pending read" and t.startswith("v_mfma") for _, why, t in bad)
