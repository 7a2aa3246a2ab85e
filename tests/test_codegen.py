"""Checks on the gfx950 code hipcc generates from this repository's kernels
(device assembly of our own sources, no GPU needed):

  * m0 is written only by the buffer-to-LDS staging asm, which lists it as
    clobbered; the compiler treats m0 as reserved and would not preserve a
    value of its own across that asm, so it must hold none;
  * v_permlane16/32_swap appear only inside the asm helpers (the compiler's
    builtins for them returned the first register as both results);
  * no scalar-memory store or atomic anywhere (every store goes through the
    vector memory path).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_int2_amd", "csrc")
HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SOURCES = ("decode_attn.hip", "quant_write.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    out = {}
    d = tmp_path_factory.mktemp("asm")
    for src in SOURCES:
        s = str(d / (src + ".s"))
        cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
               os.path.join(CSRC, src), "-o", s]
        subprocess.run(cmd, check=True, capture_output=True, timeout=600)
        out[src] = open(s).read().split("\n")
    return out


def _instructions(lines):
    """(function, in_asm, text) of every instruction line."""
    func, in_asm = None, False
    for line in lines:
        m = re.match(r"^(\S+):\s*;\s*@", line)
        if m:
            func = m.group(1)
        if "ASMSTART" in line:
            in_asm = True
            continue
        if "ASMEND" in line:
            in_asm = False
            continue
        s = line.strip()
        if not s or s.startswith((";", ".")) or s.endswith(":"):
            continue
        yield func, in_asm, s


@pytest.mark.parametrize("src", SOURCES)
def test_m0_only_in_staging_asm(asm, src):
    bad = [(f, s) for f, a, s in _instructions(asm[src]) if not a and re.search(r"\bm0\b", s)]
    assert not bad, bad[:5]


@pytest.mark.parametrize("src", SOURCES)
def test_permlane_swaps_only_in_asm(asm, src):
    swaps = [(a, s) for _, a, s in _instructions(asm[src]) if "v_permlane" in s and "swap" in s]
    assert swaps, "the row swaps are expected in these kernels"
    assert all(a for a, _ in swaps), [s for a, s in swaps if not a][:5]


@pytest.mark.parametrize("src", SOURCES)
def test_no_scalar_memory_writes(asm, src):
    bad = [s for _, _, s in _instructions(asm[src])
           if re.match(r"s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb|dcache_discard)", s)]
    assert not bad, bad[:5]
