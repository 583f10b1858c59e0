"""The inline-asm LDS reads of the bf16 forward and the backward kernels are
waited for before their registers are used (tests/asm_waits.py), checked
in the gfx950 assembly the build flags produce; a weakened wait in a copy
of the backward source is caught."""
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
