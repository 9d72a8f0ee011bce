"""Wait states around the inline-asm MFMAs of the kernels that issue some.

The large-K statistics kernels that run one wave per SIMD issue their score
and s0 MFMAs from inline asm, and the D <= 128 full-covariance kernels their
whitening MFMAs (accumulators in VGPRs; in the full-covariance kernels half
of the A operands come from AGPRs).  The compiler does not see an MFMA
inside an asm statement, so it inserts none of the wait states the
matrix-core dependency rules ask for; the kernels write them out.  This test
compiles the kernel sources for gfx950 and checks the emitted code:

* before each such MFMA no vector-ALU instruction writes one of its A / B
  source registers within the 8 preceding instructions (a VALU write of an
  MFMA operand needs wait states the compiler would not add);
* after each such MFMA at least 20 wait states (one per instruction, N + 1 per
  ``s_nop N``) pass before any instruction other than a later MFMA of the
  same accumulation chain reads or writes its result (a 32x32x16 result needs
  11 before a VALU reads it; 20 leaves a margin).

It needs hipcc (no GPU) and takes about a minute.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "soft_clustering_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _split(ins):
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    return parts[0], [t.strip() for t in re.split(r",(?![^\[]*\])", parts[1])]


def _kernels(asm_text, key):
    """{kernel symbol: [(instruction, from inline asm)]} of the kernels whose
    symbol contains `key`."""
    out, cur, in_asm = {}, None, False
    for raw in asm_text.split("\n"):
        if ";;#ASMSTART" in raw:
            in_asm = True
            continue
        if ";;#ASMEND" in raw:
            in_asm = False
            continue
        line = raw.split(";")[0].strip()
        m = re.match(r"^(_ZN3gmm\S*" + key + r"\S*):$", line)
        if m:
            cur = m.group(1)
            out[cur] = []
            continue
        if cur is None or not line or line.endswith(":") or line.startswith("."):
            continue
        out[cur].append((line, in_asm))
        if line.startswith("s_endpgm"):
            cur = None
    return out


def _check(code):
    """(number of inline-asm MFMAs, list of findings) for one kernel."""
    ins = [c for c, _ in code]
    n, bad = 0, []
    for i, (line, from_asm) in enumerate(code):
        op, args = _split(line)
        if not op.startswith("v_mfma") or not from_asm:
            continue
        n += 1
        src = set().union(*[_regs(a) for a in args[1:3]])
        dst = _regs(args[0])
        for j in range(max(0, i - 8), i):
            o2, a2 = _split(ins[j])
            if o2.startswith("v_") and not o2.startswith("v_mfma") and a2 and _regs(a2[0]) & src:
                bad.append(f"VALU write of an operand before: {ins[j]} | {line}")
        ws = 0
        for j in range(i + 1, min(len(ins), i + 400)):
            o2, a2 = _split(ins[j])
            if o2.startswith("s_nop"):
                ws += int(a2[0]) + 1 if a2 else 1
                continue
            used = set().union(*[_regs(a) for a in a2]) if a2 else set()
            if o2.startswith("v_mfma"):
                if used & dst and _regs(a2[0]) != dst:
                    bad.append(f"result used as an MFMA operand: {ins[j]} | {line}")
                ws += 1
                continue
            if used & dst:
                if ws < 20:
                    bad.append(f"{ws} wait states before {ins[j]} | {line}")
                break
            if o2.startswith(("s_cbranch", "s_branch", "s_setpc", "s_endpgm")):
                break
            ws += 1
    return n, bad


CASES = [
    # source, kernel symbol key, {asm MFMAs per kernel: kernels with that many}
    # large K: the diagonal statistics kernels at D = 128 (sweep 2 and fused
    # E+M, x 2 storage types x 2 load paths): 34 score MFMAs (17 steps x 2
    # blocks) and 4 s0 MFMAs per tile
    ("largek.hip", "k_lk", {38: 8}),
    # full covariance, D <= 128: 40 whitening MFMAs per 32-point block (20
    # lower-triangle blocks, hi and lo); the statistics kernels (2 load paths)
    # unroll the tile's 8 blocks, the E-step kernels (k_full_wide_e, 2 load
    # paths) hold one copy of the block loop for each half of the blocks
    ("full_fused.hip", "k_full_wide", {40: 2, 320: 2}),
]


@pytest.mark.parametrize("src,key,expect", CASES, ids=[c[1] for c in CASES])
def test_inline_asm_mfma_wait_states(tmp_path, src, key, expect):
    from soft_clustering_amd import build as b
    out = tmp_path / (src + ".s")
    cmd = [b.HIPCC, *b.FLAGS, *b.NO_IEEE.get(src, []), "-w", "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    kernels = _kernels(out.read_text(), key)
    assert kernels, f"no {key} kernels found in the device code"
    counts = {}
    findings = []
    for name, ins in kernels.items():
        n, bad = _check(ins)
        if n:
            counts[n] = counts.get(n, 0) + 1
        findings += [f"{name}: {x}" for x in bad]
    assert counts == expect, counts
    assert not findings, "\n".join(findings[:20])


def test_checker_flags_short_waits():
    """The checker itself, on hand-written code: too few wait states before a
    VALU read of the result, and a VALU write of an operand just before the
    MFMA, are both reported; the settled form is not."""
    mfma = ("v_mfma_f32_32x32x16_f16 v[10:25], v[2:5], v[6:9], v[10:25]", True)
    read = ("v_add_f32_e32 v30, v10, v31", False)
    n, bad = _check([mfma, ("s_nop 3", True), read])
    assert n == 1 and len(bad) == 1 and "wait states" in bad[0]
    n, bad = _check([("v_mov_b32_e32 v6, 0", False), mfma, ("s_nop 7", True), ("s_nop 7", True),
                     ("s_nop 7", True), read])
    assert n == 1 and len(bad) == 1 and "operand" in bad[0]
    n, bad = _check([mfma, ("s_nop 7", True), ("s_nop 7", True), ("s_nop 7", True), read])
    assert n == 1 and not bad
