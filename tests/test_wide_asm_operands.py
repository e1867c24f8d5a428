"""Placement of the compiler-assigned operands of the wide kernel's scheduled assembly.

The sweep's assembly blocks pin most registers by name (scores, accumulators, Q/K/V^T
operands, weights) and leave a few operands to the compiler (the exponent reference, the row
sum, read addresses, copy offsets).  The compiler may place such an operand in a pinned
register whose value is dead or undefined at that point -- the block would then overwrite its
own operand.  Every block starts with a comment naming its pinned range and its free
operands; this test compiles the kernel for gfx950 and checks, in every block of every
instantiation, that no free operand landed in a pinned vector register or (in the sweep loops,
which pin the copy pointers) a pinned scalar register.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "hybrid_softmax_linear_chunked_amd", "csrc", "attn_wide.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _regs(tok):
    # VCC's halves are scalar registers outside the numbered range (the blocks write no VCC)
    if tok in ("vcc_lo", "vcc_hi", "vcc"):
        return "s", []
    m = re.fullmatch(r"([vs])\[(\d+):(\d+)\]", tok)
    if m:
        return m.group(1), list(range(int(m.group(2)), int(m.group(3)) + 1))
    m = re.fullmatch(r"([vs])(\d+)", tok)
    if m:
        return m.group(1), [int(m.group(2))]
    return None, []


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "attn_wide.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S", "-o", str(out), SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def test_free_operands_avoid_pinned_registers(kernel_asm):
    blocks = re.findall(r"; pinned v0-v(\d+)(?: s(\d+)-s(\d+))?; free ([^\n]*)", kernel_asm)
    assert len(blocks) > 20
    # the sweep loops pin the scalar copy pointers too
    assert sum(1 for b in blocks if b[1]) >= 6
    for vend, s0, s1, free in blocks:
        vend = int(vend)
        s0, s1 = (int(s0), int(s1)) if s0 else (0, -1)
        for item in free.split():
            name, tok = item.split("=")
            kind, regs = _regs(tok)
            assert kind is not None, item
            if kind == "v":
                assert min(regs) > vend, f"operand {name} in pinned {tok} (pinned v0-v{vend})"
            else:
                assert not any(s0 <= r <= s1 for r in regs), f"operand {name} in pinned scalar {tok}"


def test_blocks_leave_vcc_alone():
    """A free scalar operand may sit in VCC, so no sweep block may write it: none of the
    instructions that set VCC implicitly (compares, carry adds, divide scaling) appears."""
    inc = open(os.path.join(ROOT, "hybrid_softmax_linear_chunked_amd", "csrc", "wide_substep.inc")).read()
    assert not re.search(r"\b(v_cmp\w*|v_cmpx\w*|v_add_co\w*|v_sub_co\w*|v_subrev_co\w*|v_addc\w*|v_subb\w*|"
                         r"v_div_scale\w*|v_cndmask\w*)\b|\bvcc", inc)
