"""The debug build (MOE_DEBUG_BOUNDS) compiles for gfx950, its bounds checks
are in the device code, and the normal build has none (CPU only: the
kernels are compiled to assembly and read, never run)."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from mixture_experts_layer_permute_amd import build

# sources whose kernels carry checks on data-driven indexes
CHECKED = {"permute.hip": "perm_scatter_kernel", "ggemm.hip": "ggemm_bf16_dma_kernel"}


def device_asm(src, debug, out_dir):
    out = os.path.join(out_dir, src.replace(".hip", "_debug.s" if debug else ".s"))
    cmd = [build.hipcc()] + build.FLAGS + build.EXTRA.get(src, []) + \
        (build.DEBUG_FLAGS if debug else []) + \
        ["--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return open(out).read()


def traps_in(asm, kernel):
    """s_trap instructions in the functions whose names contain `kernel`."""
    n = 0
    for m in re.finditer(r"^(_Z\w+):", asm, re.M):
        if kernel not in m.group(1):
            continue
        end = asm.find(".Lfunc_end", m.end())
        n += len(re.findall(r"^\s+s_trap\b", asm[m.end():end], re.M))
    return n


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(build.hipcc()):
        pytest.skip("no hipcc")
    d = str(tmp_path_factory.mktemp("dbg"))
    jobs = [(s, True) for s in build.SOURCES] + [(s, False) for s in CHECKED]
    with ThreadPoolExecutor(len(jobs)) as ex:
        res = list(ex.map(lambda j: device_asm(j[0], j[1], d), jobs))
    return {j: r for j, r in zip(jobs, res)}


def test_debug_build_compiles_every_source(asm):
    for s in build.SOURCES:
        assert ".amdhsa_kernel" in asm[(s, True)], s


def test_checks_only_in_the_debug_build(asm):
    for src, kernel in CHECKED.items():
        assert traps_in(asm[(src, True)], kernel) > 0, src
        assert traps_in(asm[(src, False)], kernel) == 0, src
