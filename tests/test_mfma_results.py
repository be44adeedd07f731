"""No instruction writes an MFMA's result registers before the result is first read.

The compiler checks MFMA hazards for the instructions it generates, but not for
inline asm: with some of a result's registers unused, it may hand one of them to
an inline-asm output while the MFMA is still writing it, and the MFMA's late
write then replaces that output (wrong results, no fault). This test compiles
every source with matrix-core kernels to gfx950 assembly, with the library's
own flags, and checks each MFMA: between it and the first instruction that
reads any of its result registers (or the next branch), nothing may write one of
those registers. CPU only: it needs hipcc, not a GPU."""
import os
import re
import shutil
import subprocess

import pytest

from routed_expert_quantized_amd import build

SOURCES = ["k_gemm.hip", "k_lora.hip", "k_route.hip"]

_REG = re.compile(r"^([va])(?:\[(\d+):(\d+)\]|(\d+))$")


def _regs(tok):
    m = _REG.match(tok)
    if not m:
        return set()
    kind = m.group(1)
    if m.group(4) is not None:
        return {(kind, int(m.group(4)))}
    return {(kind, r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}


def _operands(line):
    return [t.strip(",") for t in line.split()]


def mfma_result_writes(asm: str):
    """(function, mfma line, offending line) for every write into an MFMA result
    ahead of the result's first read, and the number of MFMAs checked."""
    bad, checked = [], 0
    for chunk in asm.split(".Lfunc_end"):
        names = re.findall(r"^([A-Za-z_][\w.$]*):", chunk, re.M)
        name = names[0] if names else "?"
        lines = [l.strip() for l in chunk.splitlines()]
        # instructions only: no directives, comments or labels (which may carry a comment)
        ins = [l for l in lines if l and not l.startswith((".", ";")) and not re.match(r"^[\w.$]+:", l)]
        for n, line in enumerate(ins):
            if not line.startswith("v_mfma"):
                continue
            checked += 1
            dst = _regs(_operands(line)[1])
            for nxt in ins[n + 1:]:
                ops = _operands(nxt)
                if ops[0].startswith(("s_cbranch", "s_branch", "s_setpc", "s_endpgm")):
                    break
                if ops[0].startswith("s_"):
                    continue
                written = _regs(ops[1]) if len(ops) > 1 else set()
                read = set()
                for o in ops[2:]:
                    read |= _regs(o)
                if ops[0].startswith(("global_store", "buffer_store", "scratch_store", "ds_write", "ds_store")):
                    read |= written
                    written = set()
                if read & dst:
                    break  # the first use waits for the MFMA: its registers are complete from here
                if written & dst:
                    bad.append((name, line, nxt))
                    break
    return bad, checked


@pytest.mark.skipif(shutil.which(build.HIPCC) is None and not os.path.exists(build.HIPCC), reason="hipcc missing")
@pytest.mark.parametrize("src", SOURCES)
def test_no_write_into_a_pending_mfma_result(src, tmp_path):
    out = tmp_path / (src + ".s")
    flags = [f for f in build.CFLAGS if f != "-fPIC"]
    r = subprocess.run([build.HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", str(out)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    bad, checked = mfma_result_writes(out.read_text())
    assert checked > 0, f"no MFMA found in {src}"
    assert not bad, "\n".join(f"{f}: {m}  ->  {w}" for f, m, w in bad[:10])


def test_the_check_sees_a_write_into_a_pending_result():
    asm = "\n".join([
        "k_bad:",
        "  v_mfma_f32_16x16x32_f16 v[32:35], v[40:43], v[36:39], 0",
        "  ;;#ASMSTART",
        "  v_bitop3_b32 v35, v45, v165, v164 bitop3:0xea",
        "  ;;#ASMEND",
        "  v_fmac_f32_e32 v0, s1, v32",
        ".Lfunc_end0:",
        "k_good:",
        "  v_mfma_f32_16x16x32_f16 v[32:35], v[40:43], v[36:39], 0",
        "  v_fmac_f32_e32 v0, s1, v32",
        "  v_bitop3_b32 v35, v45, v165, v164 bitop3:0xea",
        ".Lfunc_end1:",
    ])
    bad, checked = mfma_result_writes(asm)
    assert checked == 2
    assert [b[0] for b in bad] == ["k_bad"]
