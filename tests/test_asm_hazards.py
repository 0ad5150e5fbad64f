"""Compiled-code check for a gfx950 hazard the compiler does not always space out.

A DPP lane move that reads a register written by `v_dot2c_f32_bf16` fewer than three wait
states earlier returned that register's older value on the GPU (a decode row sum came out
missing its last dot-product term), and the compiler had spaced such a pair by two
instructions.  The kernels pass such sums through `settle_dot` before a DPP reduction.  This
test compiles every kernel source to gfx950 assembly with the library's own flags and traces
each DPP source register back to its last writer in program order; a dot-product writer
closer than three wait states fails.  CPU only: hipcc cross-compiles without a GPU.
"""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from grouped_expert_ffn_amd import build as B

MIN_WAIT_STATES = 3


def _hipcc():
    try:
        return B.hipcc()
    except RuntimeError:
        return None


def _compile(src: str, out_dir: str) -> str:
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    cmd = [_hipcc(), *flags, "--cuda-device-only", "-S", "-I", os.path.join(B.ROOT, "include"), src,
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


def dot_to_dpp_distances(asm_lines):
    """(wait states, writer, function, line) for every DPP source traced back to a VALU
    writer within eight wait states; s_nop N counts N + 1, any other instruction one."""
    out = []
    fn = None
    for i, line in enumerate(asm_lines):
        if re.match(r"^_Z\S+:", line):
            fn = line.split(":")[0]
        m = re.match(r"\s+(v_\w+_dpp)\s+(v\d+),\s*(v\d+)", line)
        if not m:
            continue
        src = m.group(3)
        ws, j = 0, i - 1
        while j >= 0 and ws < 8:
            t = asm_lines[j].strip()
            if not t or t.startswith(";") or t.endswith(":") or t.startswith("."):
                j -= 1
                continue
            nop = re.match(r"s_nop\s+(\d+)", t)
            if nop:
                ws += int(nop.group(1)) + 1
                j -= 1
                continue
            w = re.match(r"(\S+)\s+(\S+?),", t)
            if w and w.group(2) == src and w.group(1).startswith("v_"):
                out.append((ws, w.group(1), fn, i + 1))
                break
            ws += 1
            j -= 1
    return out


@pytest.fixture(scope="module")
def kernel_asm():
    if _hipcc() is None:
        pytest.skip("hipcc not found")
    d = tempfile.mkdtemp(prefix="moe_asm_")
    try:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            paths = list(ex.map(lambda s: _compile(s, d), B.sources()))
        yield {os.path.basename(p): open(p).read().splitlines() for p in paths}
    finally:
        shutil.rmtree(d, ignore_errors=True)


def test_no_dpp_read_too_close_after_a_dot_product(kernel_asm):
    bad = []
    checked = 0
    for name, lines in kernel_asm.items():
        for ws, writer, fn, ln in dot_to_dpp_distances(lines):
            if "dot" in writer:
                checked += 1
                if ws < MIN_WAIT_STATES:
                    bad.append((name, ln, writer, ws, (fn or "")[:80]))
    assert not bad, bad


def test_the_scan_sees_dot_products_feeding_dpp(kernel_asm):
    """Not vacuous: the decode GEMV's sums do reach DPP reductions (now through settle_dot,
    which ends the trace at its s_nop), and the scan finds DPP reads of other VALU results."""
    lines = kernel_asm["k_gemv.hip.s"]
    assert any("v_dot2c_f32_bf16" in l for l in lines)
    found = dot_to_dpp_distances(lines)
    assert found, "no DPP source traced back to a VALU writer"
    planted = ["\tv_dot2c_f32_bf16_e32 v3, v23, v36", "\ts_nop 0", "\tv_add_f32_dpp v3, v3, v3 quad_perm:[1,0,3,2]"]
    assert dot_to_dpp_distances(planted) == [(1, "v_dot2c_f32_bf16_e32", None, 3)]
