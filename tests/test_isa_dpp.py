"""The indexer's multiply-adds take their query operand by DPP inside inline
assembly (v_fmac_f32_dpp ... row_newbcast), which the compiler does not look
into: it inserts no wait states for it.  On gfx950 a DPP instruction must not
read a VGPR that a VALU instruction wrote in the two instructions before it,
and must not follow a write of EXEC closely.  This compiles the indexer for
gfx950 with the library's own flags and checks every such instruction in the
generated code (no GPU needed)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "compressed_kv_cache_decode_amd", "csrc", "csa2_index.hip")


def vgprs(op):
    m = re.match(r"v\[(\d+):(\d+)\]$", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", op)
    return {int(m.group(1))} if m else set()


def dpp_violations(asm):
    """(kernel, instruction, reason) for every v_fmac_f32_dpp whose DPP source
    was written by one of the two instructions before it (VALU), or that
    follows an EXEC write or a branch target within six instructions."""
    bad, counts = [], {}
    fn, prev = None, []
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            fn, prev = m.group(1), []
            continue
        t = line.split(";")[0].strip()
        if fn is None or not t:
            continue
        if t.endswith(":"):  # a label: control may arrive from elsewhere
            prev.append("<label>")
            continue
        if t.startswith("."):  # an assembler directive
            continue
        if t.startswith("v_fmac_f32_dpp"):
            counts[fn] = counts.get(fn, 0) + 1
            src0 = vgprs(t.split(None, 1)[1].split(",")[1].strip())
            for p in prev[-2:]:
                if p.startswith("v_") and " " in p and vgprs(p.split(None, 1)[1].split(",")[0].strip()) & src0:
                    bad.append((fn, t, "VALU write of the DPP source: " + p))
            for p in prev[-6:]:
                if p == "<label>" or "exec" in p or p.startswith("v_cmpx"):
                    bad.append((fn, t, "EXEC write or branch target nearby: " + p))
        prev.append(t)
    return bad, counts


def test_dpp_multiply_adds_have_their_wait_states(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    from compressed_kv_cache_decode_amd import build
    out = tmp_path / "index.s"
    cmd = [hipcc, *build.CFLAGS, "-x", "hip", "--cuda-device-only", "-S", SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    bad, counts = dpp_violations(out.read_text())
    # the FP8 and FP4 scans and pool rescoring: 256 multiply-adds each
    assert sum(counts.values()) >= 4 * 256, counts
    assert not bad, bad[:5]


def test_the_check_finds_a_planted_hazard():
    asm = "\n".join([
        "_Zk:",
        "\tv_mov_b32_e32 v2, v9",
        "\tv_fmac_f32_dpp v7, v2, v1 row_newbcast:0 row_mask:0xf bank_mask:0xf",
        "\tv_add_f32_e32 v3, v4, v5",
        "\tv_nop",
        "\tv_nop",
        "\tv_fmac_f32_dpp v7, v2, v1 row_newbcast:1 row_mask:0xf bank_mask:0xf",
        ".LBB0_1:",
        "\tv_fmac_f32_dpp v7, v3, v1 row_newbcast:1 row_mask:0xf bank_mask:0xf",
    ])
    bad, counts = dpp_violations(asm)
    assert counts == {"_Zk": 3}
    reasons = [b[2] for b in bad]
    assert any(r.startswith("VALU write") and "v_mov_b32_e32 v2" in r for r in reasons)
    assert any(r.startswith("EXEC write or branch target") for r in reasons)
    assert len([b for b in bad if "row_newbcast:1" in b[1] and b[2].startswith("VALU")]) == 0
