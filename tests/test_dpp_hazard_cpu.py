"""Host-side check of the score kernels' inline-asm DPP FMAs (no GPU needed).

The centroid scores take each query value from its owner lane with
`v_fmac_f64_dpp ... row_newbcast:N`, written as inline asm.  On gfx950 a DPP
read of a VGPR written by a VALU instruction needs two wait states, and the
compiler does not look inside inline asm for that hazard.  The kernels keep the
broadcast registers loaded from LDS (not written by VALU) and open every float4
step with `s_nop 1`; this test compiles score.hip for gfx950 and checks, in every
instantiation, that no VALU instruction among the two before a DPP FMA writes
that FMA's broadcast source pair.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_long_context_centroid_amd", "csrc")


def _regs(tok: str) -> set:
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _hazards(lines):
    """(count of DPP FMAs, list of offending instruction pairs) for one kernel body."""
    ins = [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]
    n, bad = 0, []
    for i, l in enumerate(ins):
        if not l.startswith("v_fmac_f64_dpp"):
            continue
        n += 1
        src0 = _regs(l.split(None, 1)[1].split(",")[1].strip().split()[0])
        for prev in ins[max(0, i - 2):i]:
            if prev.startswith("v_") and " " in prev:
                dst = _regs(prev.split(None, 1)[1].split(",")[0].strip())
                if dst & src0:
                    bad.append((prev, l))
    return n, bad


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_score_dpp_broadcast_reads_have_no_valu_hazard(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    out = tmp_path / "score.s"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", f"-I{ROOT}/include", f"-I{CSRC}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "--cuda-device-only",
           "-S", os.path.join(CSRC, "score.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    text = [l.split(";")[0].strip() for l in out.read_text().splitlines()]
    kernels, cur = {}, None
    for l in text:
        m = re.match(r"^(_ZN3ckv\S*score_kernel\S*):$", l)
        if m:
            cur = m.group(1)
            kernels[cur] = []
            continue
        if cur is not None:
            kernels[cur].append(l)
            if l.startswith("s_endpgm"):
                cur = None
    assert len(kernels) >= 16, sorted(kernels)  # score and layer-score instantiations
    total = 0
    for name, body in kernels.items():
        n, bad = _hazards(body)
        assert n > 0, f"{name}: no DPP FMAs found"
        assert not bad, f"{name}: VALU write of a DPP source right before its read: {bad[:3]}"
        total += n
    print(f"{len(kernels)} kernels, {total} DPP FMAs, no read hazard")


def test_hazard_scan_flags_a_valu_write_before_the_dpp_read():
    """The scanner itself: a VALU write of the DPP source one or two instructions
    before the read is flagged; a write three instructions before, or a write of
    another register, is not."""
    dpp = "v_fmac_f64_dpp v[2:3], v[6:7], v[4:5] row_newbcast:5 row_mask:0xf bank_mask:0xf"
    n, bad = _hazards(["v_add_f64 v[6:7], v[6:7], v[8:9]", dpp])
    assert n == 1 and len(bad) == 1
    n, bad = _hazards(["v_mov_b32_e32 v7, 0", "s_nop 0", dpp])
    assert n == 1 and len(bad) == 1
    n, bad = _hazards(["v_add_f64 v[6:7], v[6:7], v[8:9]", "s_nop 0", "s_nop 0", dpp])
    assert n == 1 and not bad
    n, bad = _hazards(["v_add_f64 v[10:11], v[6:7], v[8:9]", dpp])
    assert n == 1 and not bad
    n, bad = _hazards(["ds_read_b64 v[6:7], v1", dpp])
    assert n == 1 and not bad
