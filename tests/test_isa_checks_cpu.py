"""Static checks of the built device code (CPU only), on every source that
uses block barriers or DPP operands, compiled exactly as the library is:

* every s_barrier is preceded, in its own basic block, by a wait for the
  wavefront's LDS operations (s_waitcnt lgkmcnt(0)) with no LDS instruction
  in between.  Without it an LDS store issued just before a loop's back edge
  can still be in flight when other wavefronts pass the barrier at the loop
  head and read the tile (observed as stale y tiles in the single-pass scan
  with feedthrough and gate);
* every instruction that reads a VGPR through DPP has two wait states (an
  instruction each, s_nop k gives k + 1) after the last VALU write of that
  VGPR.  The compiler inserts them for its own code but not around inline
  asm, which the scan kernels use for bank-masked DPP adds and v_fmac_f32
  with a broadcast operand.  A DPP read closer than two instructions to a
  block label is flagged too (its predecessors are not looked at)."""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from selective_state_space_54_amd import build as hipbuild

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _sources_to_check():
    """Sources whose own text or included headers (other than the one that
    defines block_sync) use block barriers or DPP."""
    marks = ("block_sync()", "_dpp", "update_dpp")
    out = []
    for src in hipbuild.sources():
        text = open(src).read()
        heads = re.findall(r'#include "(\w+\.h)"', text)
        texts = [text] + [open(os.path.join(hipbuild.CSRC, h)).read()
                          for h in heads if h != "scan_device.h"]
        if any(m in t for m in marks for t in texts):
            out.append(src)
    return out


def _device_asm(src, outdir):
    dst = os.path.join(outdir, os.path.basename(src) + ".s")
    cmd = [HIPCC, *hipbuild.HIPCC_FLAGS, "-I", hipbuild.INCLUDE, "-I", hipbuild.CSRC,
           "--cuda-device-only", "-S", src, "-o", dst]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return dst


def barriers_without_lds_wait(asm_text):
    """(line, kernel) of each s_barrier not preceded in its basic block by
    s_waitcnt lgkmcnt(0) (or s_waitcnt 0) with no ds_* instruction between."""
    lines = asm_text.split("\n")
    kernel, bad = None, []
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            kernel = m.group(1)
        if not re.match(r"\s*s_barrier\b", line):
            continue
        ok = False
        for j in range(i - 1, -1, -1):
            t = lines[j]
            if re.match(r"\s*s_waitcnt\b.*lgkmcnt\(0\)", t) or re.match(r"\s*s_waitcnt\s+0\s*$", t):
                ok = True
                break
            if re.match(r"\s*ds_", t) or re.match(r"^\.LBB|^\S+:", t):
                break
        if not ok:
            bad.append((i + 1, kernel))
    return bad


def _vgprs(tok):
    m = re.match(r"v(\d+)$", tok)
    if m:
        return {int(m.group(1))}
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def dpp_read_hazards(asm_text):
    """(line, kernel, reason) of each DPP instruction whose DPP source (its
    first source operand) was written by a VALU instruction less than two wait
    states earlier, or that is less than two wait states after a label."""
    lines = asm_text.split("\n")
    kernel, bad = None, []
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            kernel = m.group(1)
        t = line.strip()
        if not re.match(r"v_\w+_dpp\b", t):
            continue
        ops = t.split(None, 1)[1].split(",")
        src = _vgprs(ops[1].split()[0]) if len(ops) > 1 else set()
        waits = 0
        for j in range(i - 1, -1, -1):
            u = lines[j].strip()
            if re.match(r"^\S+:", lines[j]):
                bad.append((i + 1, kernel, "label"))
                break
            if not u or u.startswith(";") or u.startswith("."):
                continue
            mnem = u.split()[0]
            if mnem == "s_nop":
                waits += int(u.split()[1], 0) + 1
            else:
                if mnem.startswith("v_") and not mnem.startswith(("v_cmp", "v_readfirstlane")):
                    dst = _vgprs(u.split(None, 1)[1].split(",")[0].strip()) if " " in u else set()
                    if dst & src:
                        bad.append((i + 1, kernel, u))
                        break
                waits += 1
            if waits >= 2:
                break
    return bad


def test_dpp_checker_flags_close_writes():
    asm = "\n".join(["_Zk:", "\tv_mul_f32_e32 v5, v1, v2",
                      "\tv_add_f32_dpp v6, v5, v5 row_ror:8 row_mask:0xf bank_mask:0x3",
                      "\tv_mul_f32_e32 v7, v1, v2", "\ts_nop 1",
                      "\tv_add_f32_dpp v6, v7, v7 row_ror:8 row_mask:0xf bank_mask:0x3",
                      "\tv_mul_f32_e32 v8, v1, v2", "\tv_mul_f32_e32 v9, v1, v2",
                      "\tv_mov_b32_dpp v6, v9 row_newbcast:1 row_mask:0xf bank_mask:0xf",
                      "\tv_mul_f32_e32 v10, v1, v2", "\tv_mul_f32_e32 v11, v1, v2",
                      "\tv_mul_f32_e32 v12, v1, v2",
                      "\tv_mov_b32_dpp v6, v10 row_newbcast:1 row_mask:0xf bank_mask:0xf",
                      ".LBB0_1:", "\tv_mov_b32_dpp v6, v3 row_newbcast:1 row_mask:0xf bank_mask:0xf"])
    # line 3: no wait state; 9: one (v9 two instructions back); 13: two, fine;
    # 15: right after a label
    assert [b[0] for b in dpp_read_hazards(asm)] == [3, 9, 15]


def test_checker_flags_a_barrier_after_an_lds_store():
    asm = "\n".join(["_Zk:", "\tds_write_b32 v1, v2", "\ts_barrier",
                     ".LBB0_1:", "\ts_barrier",
                     "\tds_read_b32 v3, v1", "\ts_waitcnt lgkmcnt(0)", "\ts_barrier"])
    assert [b[0] for b in barriers_without_lds_wait(asm)] == [3, 5]


def test_barriers_wait_for_lds_and_dpp_reads_have_their_wait_states():
    srcs = _sources_to_check()
    assert any(s.endswith("chain_bwd.hip") for s in srcs)
    assert any(s.endswith("chain_euler_plain.hip") for s in srcs)
    os.makedirs(hipbuild.OBJ_DIR, exist_ok=True)
    outdir = tempfile.mkdtemp(prefix="asm_", dir=hipbuild.OBJ_DIR)
    try:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
            files = list(pool.map(lambda s: _device_asm(s, outdir), srcs))
        barrier_problems, dpp_problems, barriers, dpps = [], [], 0, 0
        for f in files:
            text = open(f).read()
            barriers += len(re.findall(r"^\s*s_barrier\b", text, flags=re.M))
            dpps += len(re.findall(r"^\s*v_\w+_dpp\b", text, flags=re.M))
            name = os.path.basename(f)
            barrier_problems += [(name, *b) for b in barriers_without_lds_wait(text)]
            dpp_problems += [(name, *b) for b in dpp_read_hazards(text)]
        assert barriers > 0 and dpps > 0
        assert not barrier_problems, barrier_problems[:10]
        assert not dpp_problems, dpp_problems[:10]
    finally:
        shutil.rmtree(outdir, ignore_errors=True)
