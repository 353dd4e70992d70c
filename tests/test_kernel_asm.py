"""Static checks of the gfx950 assembly of the FFN and router kernels (CPU only: hipcc
cross-compiles, nothing runs on a GPU).

1. No instruction reads, copies, spills or overwrites the destination
   registers of an LDS read before an ``s_waitcnt`` has retired it (the fat
   kernels' operand reads are inline assembly, which the compiler takes as
   complete at once; a register copy placed before the wait would hold stale
   data and give wrong results only on some paths).
2. The fat kernels' K-loops (the innermost loops) spill nothing to scratch.
3. The streaming kernel's chunk loop never waits for all of its loads
   (``s_waitcnt vmcnt(0)``): the next chunk's weights stay in flight while
   the current one is multiplied, across items too.
4. The 3-bit down kernels of decode batches (activation rows in LDS, four
   blocks per CU under a 128-register bound) spill nothing anywhere: a
   spilled register is a memory round trip in every item.

The checker itself is pinned on hand-written snippets with and without such
a hazard.
"""
import hashlib
import os
import re
import shutil
import subprocess

import pytest

from tests.asm_check import kernel_bodies, stale_lds_uses
from routed_expert_ffn_03_amd.build import BUILD, CSRC, HIPCC_FLAGS

# sources compiled to assembly, and every file their hash covers
UNITS = ["ffn.hip", "fat8.hip", "stream.hip", "route.hip"]
SOURCES = UNITS + ["common.h", "kernels.h", "lds_dma.h", "ffn_shared.h"]


def _hipcc():
    return shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)


@pytest.fixture(scope="module")
def ffn_asm():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    h = hashlib.sha256(" ".join(HIPCC_FLAGS).encode())
    for s in SOURCES:
        with open(os.path.join(CSRC, s), "rb") as f:
            h.update(f.read())
    text = []
    for unit in UNITS:
        out = os.path.join(BUILD, f"{unit.split('.')[0]}_device_{h.hexdigest()[:12]}.s")
        if not os.path.exists(out):
            os.makedirs(BUILD, exist_ok=True)
            cmd = [hipcc, *HIPCC_FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, unit), "-o", out + ".tmp"]
            res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
            assert res.returncode == 0, res.stderr[-2000:]
            os.replace(out + ".tmp", out)
        with open(out) as f:
            text.append(f.read())
    return "\n".join(text)


def test_checker_flags_a_copy_before_the_wait():
    bad = """
    ds_read_b128 v[4:7], v1 offset:64
    v_mov_b64_e32 v[10:11], v[4:5]
    s_waitcnt lgkmcnt(0)
    v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[20:23], a[0:15]
    """.split("\n")
    r = stale_lds_uses(bad)
    assert len(r) == 1 and "v_mov_b64" in r[0][1]


def test_checker_follows_branches_and_partial_waits():
    # the read is in flight on the path through .LBB0_1 only
    lines = """
    s_cbranch_scc1 .LBB0_2
.LBB0_1:
    ds_read_b128 v[4:7], v1
    ds_read_b128 v[8:11], v1 offset:16
    s_waitcnt lgkmcnt(1)
    v_mov_b32_e32 v30, v4
.LBB0_2:
    scratch_store_dwordx4 off, v[8:11], off offset:16
    s_waitcnt lgkmcnt(0)
    v_mov_b32_e32 v31, v8
    s_endpgm
    """.split("\n")
    r = stale_lds_uses(lines)
    assert [x[1].split()[0] for x in r] == ["scratch_store_dwordx4"]


def test_checker_accepts_clean_code():
    lines = """
    ds_read_b128 v[4:7], v1
    s_waitcnt lgkmcnt(0)
    v_mov_b64_e32 v[10:11], v[4:5]
    s_load_dword s4, s[0:1], 0x0
    ds_read_b128 v[8:11], v1
    s_waitcnt lgkmcnt(0)
    v_add_u32_e32 v12, v8, v9
    s_endpgm
    """.split("\n")
    assert stale_lds_uses(lines) == []


def test_no_lds_result_used_before_its_wait(ffn_asm):
    kernels = {k: v for k, v in kernel_bodies(ffn_asm).items() if "ffn_" in k or "router_" in k}
    assert any("ffn_fat_kernel" in k for k in kernels) and any("router_topk_kernel" in k for k in kernels)
    assert any("ffn_fat8_kernel" in k for k in kernels)
    assert any("ffn_stream_kernel" in k for k in kernels)
    assert any("router_logits_split_kernel" in k for k in kernels)
    bad = {}
    for name, lines in kernels.items():
        r = stale_lds_uses(lines)
        if r:
            bad[name] = r[:3]
    assert not bad, bad


def _loops(lines):
    """(label, body lines) of every loop: from the first block of the loop to
    the last branch back to its header."""
    out = []
    for i, l in enumerate(lines):
        if "Inner Loop Header" in l and i > 0:
            # the header label sits on the comment's line or on the one before
            own = l.split(":")[0].strip()
            lab = own if own.startswith(".LBB") else lines[i - 1].split(":")[0].strip()
            if not lab.startswith(".LBB"):
                continue
            tag = "Header=" + lab[2:] + " "
            ends = [j for j, x in enumerate(lines) if re.search(r"s_c?branch\w*\s+" + re.escape(lab) + r"\s*$", x)]
            starts = [j for j, x in enumerate(lines) if tag in x]
            if ends:
                out.append((lab, lines[min(starts + [i - 1]):max(ends) + 1]))
    return out


def test_fat_k_loops_do_not_spill(ffn_asm):
    kernels = {k: v for k, v in kernel_bodies(ffn_asm).items() if "ffn_fat_kernel" in k or "ffn_fat8_kernel" in k}
    assert any("ffn_fat8_kernel" in k for k in kernels)
    checked = 0
    for name, lines in kernels.items():
        for lab, body in _loops(lines):
            if sum("v_mfma" in x for x in body) < 8:
                continue
            checked += 1
            spills = [x.strip() for x in body if "scratch_" in x]
            assert not spills, (name, lab, spills[:3])
    assert checked > 0


def test_decode_down_kernels_do_not_spill(ffn_asm):
    kernels = {k: v for k, v in kernel_bodies(ffn_asm).items()
               if re.search(r"ffn_thin_q3_kernelILi2ELi(4|8|16)E", k)}
    assert len(kernels) == 3, sorted(kernels)
    for name, lines in kernels.items():
        spills = [x.strip() for x in lines if "scratch_" in x]
        assert not spills, (name, spills[:3])


def _loop_blocks(lines):
    """(label, lines) of every loop as the union of its basic blocks: the
    header and every block tagged as inside it (the back edge may fall
    through, so the loop need not end in a branch to its header)."""
    starts = [i for i, x in enumerate(lines) if re.match(r"^(\.LBB\w+:|; %bb\.\d+:)", x.strip())]
    blocks = [(i, (starts[n + 1] if n + 1 < len(starts) else len(lines))) for n, i in enumerate(starts)]
    out = []
    for i, _ in blocks:
        if "Inner Loop Header" not in lines[i]:
            continue
        lab = lines[i].split(":")[0].strip()
        tag = "Header=" + lab[2:] + " "
        body = []
        for b0, b1 in blocks:
            if b0 == i or tag in lines[b0]:
                body += lines[b0:b1]
        out.append((lab, body))
    return out


def test_stream_loop_keeps_loads_in_flight(ffn_asm):
    kernels = {k: v for k, v in kernel_bodies(ffn_asm).items() if "ffn_stream_kernel" in k}
    assert len(kernels) == 2
    for name, lines in kernels.items():
        loops = [(lab, body) for lab, body in _loop_blocks(lines) if any("v_mfma" in x for x in body)]
        assert len(loops) == 1, (name, [lab for lab, _ in loops])
        body = loops[0][1]
        assert sum(" lds" in x and "buffer_load_dwordx4" in x for x in body) >= 4
        drains = [x.strip() for x in body if re.search(r"s_waitcnt\s+vmcnt\(0\)", x)]
        assert not drains, (name, drains)
        assert not [x for x in body if "scratch_" in x], name


def test_loop_blocks_follow_fall_through_back_edges():
    lines = """
.LBB0_1:                                ;   in Loop: Header=BB0_2 Depth=1
    s_mov_b32 s1, s2
    s_waitcnt vmcnt(0)
    s_cbranch_vccnz .LBB0_9
.LBB0_2:                                ; =>This Inner Loop Header: Depth=1
    buffer_load_dwordx4 v1, s[4:7], s8 offen nt lds
    v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]
    s_cbranch_scc1 .LBB0_1
.LBB0_9:
    s_endpgm
""".split("\n")
    loops = _loop_blocks(lines)
    assert [lab for lab, _ in loops] == [".LBB0_2"]
    body = loops[0][1]
    assert any("vmcnt(0)" in x for x in body) and not any("s_endpgm" in x for x in body)
