"""CPU check of the decode library's generated gfx950 code: no MFMA reads a
register sooner than two wait states after a VALU instruction wrote it.

The compiler pads this hazard around the instructions it generates, but not
around inline asm, and an MFMA that reads a register one wait state after a
v_fma_mixhi_f16 wrote its high half can read the old half (it did: the BF16
decode then gave wrong rows whenever the register had held an accumulator).
The check compiles uq_decode.hip to assembly (no GPU needed) and, for every
kernel, follows each VALU write in program order to the first MFMA that reads
the register as an operand, counting wait states (one per instruction, N + 1
per s_nop N) until the register is written again."""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "bit_kv_cache_wht_amd", "csrc", "uq_decode.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form=1", "--cuda-device-only", "-S"]


def _regs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"^([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {tok} if re.match(r"^[va]\d+$", tok) else set()


def valu_to_mfma_distances(body):
    """(least wait states, example) over VALU writes later read by an MFMA."""
    ins = []
    for line in body.splitlines():
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        parts = t.split(None, 1)
        ins.append((parts[0], re.split(r",\s*", parts[1]) if len(parts) > 1 else [], t))
    least, example = 10 ** 9, None
    for k, (op, ops, t) in enumerate(ins):
        if not op.startswith("v_") or op.startswith(("v_mfma", "v_accvgpr_read", "v_readlane", "v_readfirstlane",
                                                     "v_cmp")) or not ops:
            continue
        dst = _regs(ops[0])
        if not dst:
            continue
        ws = 0
        for op2, ops2, t2 in ins[k + 1:k + 40]:
            if op2 == "s_nop":
                ws += int(ops2[0], 0) + 1 if ops2 else 1
                continue
            if op2.startswith("v_mfma") and len(ops2) >= 4 and any(_regs(o) & dst for o in ops2[1:4]):
                if ws < least:
                    least, example = ws, f"{t} -> {t2}"
            if ops2 and _regs(ops2[0]) & dst and not op2.startswith(("global_store", "ds_write")):
                break
            ws += 1
    return least, example


@pytest.fixture(scope="module")
def asm_text():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "uq_decode.s")
        res = subprocess.run([HIPCC, *FLAGS, SRC, "-o", out], capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        return open(out).read()


def test_no_mfma_reads_a_valu_result_within_two_wait_states(asm_text):
    names = re.findall(r"\n(_ZN\w*(?:decode|prefill)_kernel\w*):", asm_text)
    assert len(names) >= 20
    worst = []
    for name in names:
        i = asm_text.index("\n" + name + ":")
        body = asm_text[i:asm_text.index(".Lfunc_end", i)]
        least, example = valu_to_mfma_distances(body)
        if least < 2:
            worst.append((name, least, example))
    assert not worst, worst[:3]


def test_checker_sees_an_unpadded_write():
    # the analysis itself: a VALU write one instruction before the MFMA that
    # reads it is found; with s_nop 1 in between it is not
    bad = """
        v_fma_mixhi_f16 v141, v149, -1.0, v200 op_sel:[1,0,0] op_sel_hi:[1,0,0]
        v_cvt_pk_f16_f32 v165, v198, v199
        v_mfma_f32_16x16x32_f16 a[0:3], v[26:29], v[138:141], a[0:3]
    """
    assert valu_to_mfma_distances(bad)[0] == 1
    good = bad.replace("v_cvt_pk_f16_f32 v165, v198, v199", "s_nop 1\n v_cvt_pk_f16_f32 v165, v198, v199")
    assert valu_to_mfma_distances(good)[0] == 3
