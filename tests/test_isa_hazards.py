"""CPU check of the gfx950 code the kernels compile to: every opaque LDS read (inline
asm, which the compiler's hazard recognizer does not see) keeps clear of MFMAs issued
just before it that still read the registers it overwrites.

An MFMA reads its A, B and C operands during its first passes; a VALU or LDS write
of one of those registers within the next few wait states is a write-after-read
hazard. The compiler pads its own LDS loads with s_nop there (7 wait states after a
16x16x32 MFMA); it cannot do so for inline asm. The kernels either place their
opaque reads where no such MFMA precedes them or lead the asm block with an s_nop.
This test compiles each kernel source to assembly with the library's flags and scans
every opaque LDS read against the MFMAs within 8 wait states before it.
"""
import os
import re
import shutil
import subprocess

import pytest

from linear_attention_attn_amd import _build

WAIT_STATES = 8  # covers the 7 a 16x16x32 bf16 MFMA needs (the compiler pads its own LDS
# loads after a 32x32x16 that reads the overwritten register as A or B by fewer)


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _instructions(asm_text):
    out, in_asm = [], False
    for raw in asm_text.splitlines():
        line = raw.strip()
        if line.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if line.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not line or line.startswith((";", ".")) or line.endswith(":"):
            continue
        op = line.split()[0]
        args = [a.strip() for a in line[len(op):].split(";")[0].split(",")]
        out.append((op, args, in_asm, line))
    return out


def unguarded_reads(asm_text, wait_states=WAIT_STATES):
    """Opaque LDS reads whose destination overlaps an operand of an MFMA issued
    fewer than `wait_states` wait states earlier (s_nop n counts n + 1)."""
    ins = _instructions(asm_text)
    found = []
    for i, (op, args, opaque, line) in enumerate(ins):
        if not (opaque and op.startswith("ds_read")):
            continue
        dst = _regs(args[0])
        waits = 0
        for j in range(i - 1, -1, -1):
            op2, args2, _, line2 = ins[j]
            waits += int(args2[0]) + 1 if op2 == "s_nop" else 1
            if waits > wait_states:
                break
            if op2.startswith("v_mfma") and dst & set().union(*(_regs(a) for a in args2[1:])):
                found.append(f"{line}  ({waits} wait states after: {line2})")
    return found


def test_scanner_flags_a_planted_hazard():
    asm = "\n".join([
        "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]",
        ";;#ASMSTART", "ds_read_b64_tr_b16 v[4:5], v20", ";;#ASMEND",
        "v_mfma_f32_16x16x32_bf16 v[12:15], v[4:7], v[8:11], 0",
        ";;#ASMSTART", "s_nop 7", "ds_read_b64_tr_b16 v[8:9], v21", ";;#ASMEND",
    ])
    got = unguarded_reads(asm)
    assert len(got) == 1 and "v[4:5]" in got[0]


@pytest.mark.parametrize("source", ["k_linear.hip", "k_paged.hip", "k_prefill.hip"])
def test_opaque_lds_reads_are_clear_of_mfma_operands(source, tmp_path):
    try:
        cc = _build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    src = os.path.join(_build.CSRC, source)
    out = tmp_path / (source + ".s")
    cmd = [cc, *_build.COMMON, *_build.PER_FILE.get(source, []), "--cuda-device-only", "-S",
           "-x", "hip", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = out.read_text()
    opaque = sum(1 for op, _, o, _ in _instructions(text) if o and op.startswith("ds_read"))
    assert opaque > 0, "no opaque LDS reads found: the scan would pass vacuously"
    bad = unguarded_reads(text)
    assert not bad, "\n".join(bad[:10])
