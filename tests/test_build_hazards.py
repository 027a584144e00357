"""Build checks of the attention kernels' machine code (no GPU), for two distances the
compiler was seen to get wrong:

* VALU write -> MFMA read of the same VGPR: at least two wait states, without counting
  s_waitcnt instructions.  The compiler counts an s_waitcnt as a wait state when it pads this
  distance.  Where restored K operands reached the score products through a branch join
  (register copies, the uncompressed branch's s_waitcnt, one s_nop), compressed and
  uncompressed tiles of equal values gave different scores on the GPU: the product read a stale
  operand.
* MFMA write -> read of its result by any other instruction: at least as many wait states as
  the compiler itself pads in straight-line code (8 after a 16x16x32 product, 12 after a
  32x32x16 one), along every control-flow path and again without counting s_waitcnt.  Where an
  uncompressed V block skipped the V restore, the score products were followed by a branch to
  the block that compares the scores, with nothing in between: the compare read a score before
  the last product had written it, on some runs.

The kernel source puts explicit nops at both places; these tests keep the patterns out of every
attention kernel the library builds.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "decode_attention_kvz_amd", "csrc", "attention.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
NEED = 2   # wait states between a VALU write of a VGPR and an MFMA read of it
# wait states between an MFMA and a read of its result (what the compiler pads straight-line)
RESULT_NEED = {"v_mfma_f32_16x16x32_bf16": 8, "v_mfma_f32_32x32x16_bf16": 12}


def _regs(operand: str) -> set:
    out = set()
    for m in re.finditer(r"v\[(\d+):(\d+)\]", operand):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\bv(\d+)\b", re.sub(r"v\[\d+:\d+\]", "", operand)):
        out.add(int(m.group(1)))
    return out


def _kernels(asm: str, labels: bool = False):
    """(name, instructions) of each attention kernel, up to its first s_endpgm; with labels,
    the whole function, block labels included."""
    lines = asm.split("\n")
    cur, body = None, []
    for line in lines:
        m = re.match(r"^(_Z\w*attn_split_kernel\w*):", line)
        if m:
            cur, body = m.group(1), []
            continue
        if cur is None:
            continue
        if (line.startswith(".Lfunc_end") if labels else "s_endpgm" in line):
            yield cur, body
            cur = None
            continue
        t = line.split(";")[0].strip()
        if t and (not t.startswith(".") or (labels and re.match(r"^\.LBB\w+:$", t))):
            body.append(t)


def _fields(ins: str):
    parts = ins.split(None, 1)
    return parts[0], ([f.strip() for f in parts[1].split(",")] if len(parts) > 1 else [])


def mfma_results_read_too_soon(asm: str):
    """(kernel, mfma, reader, wait states) for reads of an MFMA's result, by a non-MFMA
    instruction, fewer than RESULT_NEED wait states after it on some control-flow path."""
    hits = []
    for kernel, body in _kernels(asm, labels=True):
        where = {t[:-1]: i for i, t in enumerate(body) if t.endswith(":")}
        for i, ins in enumerate(body):
            op, f = _fields(ins)
            if op not in RESULT_NEED:
                continue
            dst = _regs(f[0])
            todo, seen = [(i + 1, 0)], set()
            while todo:
                j, ws = todo.pop()
                while j < len(body) and ws < RESULT_NEED[op] and (j, ws) not in seen:
                    seen.add((j, ws))
                    t = body[j]
                    if t.endswith(":"):
                        j += 1
                        continue
                    o, g = _fields(t)
                    if o == "s_endpgm":
                        break
                    if o == "s_branch":
                        j, ws = where[g[0]], ws + 1
                        continue
                    if o.startswith("s_cbranch"):
                        todo.append((where[g[0]], ws + 1))
                    elif not o.startswith("v_mfma") and g:
                        reads = g if o.startswith(("buffer_store", "global_store", "ds_write")) else g[1:]
                        if set().union(*[_regs(x) for x in reads]) & dst:
                            hits.append((kernel, ins, t, ws))
                            break
                        if not o.startswith("s_") and _regs(g[0]) >= dst:
                            break   # overwritten first
                    if o == "s_nop":
                        ws += int(g[0]) + 1
                    elif not o.startswith("s_waitcnt"):
                        ws += 1
                    j += 1
    return hits


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


@pytest.fixture(scope="module")
def listing(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "attention.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-S", "--cuda-device-only", "-o", str(out), SRC]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr[-2000:]
    asm = out.read_text()
    assert len([k for k, _ in _kernels(asm)]) >= 15, "expected the attention kernel instances in the listing"
    return asm


def test_no_mfma_operand_distance_relies_on_waitcnt(listing):
    hits = waitcnt_padded_mfma_reads(listing)
    assert not hits, "\n".join(f"{k}: {w} -> {m}" for k, w, m in hits[:10])


def test_no_mfma_result_read_too_soon(listing):
    hits = mfma_results_read_too_soon(listing)
    assert not hits, "\n".join(f"{k}: {m} -> {r} after {w} wait states" for k, m, r, w in hits[:10])


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


def test_result_checker_finds_the_pattern():
    """The result checker follows branches: the listing pattern that went wrong (products, a
    branch, a compare of the scores) is flagged, the padded one is not."""
    bad = """_ZN3kvz1_attn_split_kernelX:
\tv_mfma_f32_16x16x32_bf16 v[154:157], v[106:109], v[82:85], v[154:157]
\ts_cbranch_scc1 .LBB5_155
\tv_lshrrev_b32_e32 v74, v220, v80
\ts_nop 7
\ts_nop 7
.LBB5_155:
\tv_sub_f32_e32 v66, v213, v212
\ts_waitcnt vmcnt(3)
\tv_cmp_ge_f32_e64 s[2:3], |v154|, v211
\ts_endpgm
.Lfunc_end5:
"""
    hits = mfma_results_read_too_soon(bad)
    assert len(hits) == 1 and hits[0][3] == 2
    good = bad.replace("\ts_cbranch_scc1 .LBB5_155\n", "\ts_nop 7\n\ts_cbranch_scc1 .LBB5_155\n")
    assert mfma_results_read_too_soon(good) == []
