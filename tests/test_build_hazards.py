"""Build check of the attention kernels' machine code (no GPU): every matrix instruction that
reads a VGPR written by a vector ALU instruction must have at least two wait states between
them without counting s_waitcnt instructions.

Why: the compiler counts an s_waitcnt as a wait state when it pads the VALU-write -> MFMA-read
distance.  Where restored K operands reached the score products through a branch join (register
copies, the uncompressed branch's s_waitcnt, one s_nop), compressed and uncompressed tiles of
equal values gave different scores on the GPU: the product read a stale operand.  The kernel
source now puts an explicit two-wait-state nop between restored operands and the products; this
test keeps the padding pattern out of every attention kernel the library builds.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "decode_attention_kvz_amd", "csrc", "attention.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
NEED = 2   # wait states between a VALU write of a VGPR and an MFMA read of it


def _regs(operand: str) -> set:
    out = set()
    for m in re.finditer(r"v\[(\d+):(\d+)\]", operand):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\bv(\d+)\b", re.sub(r"v\[\d+:\d+\]", "", operand)):
        out.add(int(m.group(1)))
    return out


def _kernels(asm: str):
    lines = asm.split("\n")
    cur, body = None, []
    for line in lines:
        m = re.match(r"^(_Z\w*attn_split_kernel\w*):", line)
        if m:
            cur, body = m.group(1), []
            continue
        if cur is None:
            continue
        if "s_endpgm" in line:
            yield cur, body
            cur = None
            continue
        t = line.split(";")[0].strip()
        if t and not t.startswith("."):
            body.append(t)


def waitcnt_padded_mfma_reads(asm: str):
    """(kernel, writer, mfma) for MFMAs whose VALU-written source is fewer than NEED real wait
    states back, with an s_waitcnt in between (in straight-line order)."""
    hits = []
    for kernel, body in _kernels(asm):
        for i, ins in enumerate(body):
            if not ins.startswith("v_mfma"):
                continue
            fields = [f.strip() for f in ins.split(None, 1)[1].split(",")]
            srcs = set().union(*[_regs(f) for f in fields[1:4]])
            real = waits = 0
            for j in range(i - 1, max(i - 24, -1), -1):
                prev = body[j]
                if prev.endswith(":"):
                    continue
                if prev.startswith("s_waitcnt"):
                    waits += 1
                    continue
                if prev.startswith("s_nop"):
                    real += int(prev.split()[1]) + 1
                    continue
                if not prev.startswith("v_") or prev.startswith("v_mfma"):
                    real += 1
                    if real >= NEED:
                        break
                    continue
                pf = [f.strip() for f in prev.split(None, 1)[1].split(",")] if " " in prev else []
                written = _regs(pf[0]) if pf else set()
                if prev.startswith("v_permlane") and len(pf) > 1:
                    written |= _regs(pf[1])
                if written & srcs:
                    if real < NEED and waits:
                        hits.append((kernel, prev, ins))
                    break
                real += 1
                if real >= NEED:
                    break
    return hits


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_no_mfma_operand_distance_relies_on_waitcnt(tmp_path):
    out = tmp_path / "attention.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-S", "--cuda-device-only", "-o", str(out), SRC]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr[-2000:]
    asm = out.read_text()
    kernels = [k for k, _ in _kernels(asm)]
    assert len(kernels) >= 15, "expected the attention kernel instances in the listing"
    hits = waitcnt_padded_mfma_reads(asm)
    assert not hits, "\n".join(f"{k}: {w} -> {m}" for k, w, m in hits[:10])


def test_checker_finds_the_pattern():
    """The checker flags the listing pattern that went wrong, and not the fixed one."""
    bad = """_ZN3kvz1_attn_split_kernelX:
\tv_perm_b32 v164, v111, v108, s80
.LBB4_127:
\tv_mov_b32_e32 v121, v159
\tv_mov_b32_e32 v120, v158
.LBB4_128:
\ts_waitcnt vmcnt(14)
\ts_nop 0
\tv_mfma_f32_16x16x32_bf16 v[156:159], v[120:123], v[96:99], 0
\ts_endpgm
"""
    good = bad.replace("\ts_waitcnt vmcnt(14)\n\ts_nop 0\n", "\ts_waitcnt vmcnt(14)\n\ts_nop 1\n")
    assert len(waitcnt_padded_mfma_reads(bad)) == 1
    assert waitcnt_padded_mfma_reads(good) == []
