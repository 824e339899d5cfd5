"""Static check of the built kernels (CPU only): every s_barrier in the device
code of the sources that use block barriers is preceded, in its own basic
block, by a wait for the wavefront's LDS operations (s_waitcnt lgkmcnt(0))
with no LDS instruction in between.  Without it an LDS store issued just
before a loop's back edge can still be in flight when other wavefronts pass
the barrier at the loop head and read the tile (observed as stale y tiles in
the single-pass scan with feedthrough and gate)."""
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


def _sources_with_barriers():
    out = []
    for src in hipbuild.sources():
        text = open(src).read()
        heads = re.findall(r'#include "(\w+\.h)"', text)
        if "block_sync()" in text or any(
                "block_sync()" in open(os.path.join(hipbuild.CSRC, h)).read()
                for h in heads if h != "scan_device.h"):
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


def test_checker_flags_a_barrier_after_an_lds_store():
    asm = "\n".join(["_Zk:", "\tds_write_b32 v1, v2", "\ts_barrier",
                     ".LBB0_1:", "\ts_barrier",
                     "\tds_read_b32 v3, v1", "\ts_waitcnt lgkmcnt(0)", "\ts_barrier"])
    assert [b[0] for b in barriers_without_lds_wait(asm)] == [3, 5]


def test_every_barrier_waits_for_lds():
    srcs = _sources_with_barriers()
    assert any(s.endswith("chain_bwd.hip") for s in srcs)
    os.makedirs(hipbuild.OBJ_DIR, exist_ok=True)
    outdir = tempfile.mkdtemp(prefix="asm_", dir=hipbuild.OBJ_DIR)
    try:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
            files = list(pool.map(lambda s: _device_asm(s, outdir), srcs))
        problems, count = [], 0
        for f in files:
            text = open(f).read()
            count += len(re.findall(r"^\s*s_barrier\b", text, flags=re.M))
            problems += [(os.path.basename(f), *b) for b in barriers_without_lds_wait(text)]
        assert count > 0
        assert not problems, problems[:10]
    finally:
        shutil.rmtree(outdir, ignore_errors=True)
