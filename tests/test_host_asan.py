"""The host side of the C-ABI library under AddressSanitizer (CPU only).

The library is built a second time with AddressSanitizer on its host code
only (every kernel is compiled as usual, the sanitizer never touches device
code), loaded into a child Python with the sanitizer's runtime preloaded,
and the CPU ABI tests (argument validation, workspace queries, empty
inputs, error strings, the binding's checks) run against it.  Any invalid
access, use after free or overflow in the host paths aborts the child with
a sanitizer report.  No kernel is launched: there is no GPU here, and every
call returns before a launch.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from mixture_experts_layer_permute_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "llvm", "bin")
CLANG = os.path.join(LLVM, "clang++")
# the sanitizer applies to the host compilation only
HOST_ASAN = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def asan_runtime():
    if not os.path.exists(CLANG):
        return None
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    p = r.stdout.strip()
    return p if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p) else None


def build_host_asan(out_dir):
    flags = [f for f in build.FLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_ASAN

    def comp(src):
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        cmd = [build.hipcc()] + flags + build.EXTRA.get(src, []) + \
            ["-c", os.path.join(build.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(len(build.SOURCES)) as ex:
        objs = list(ex.map(comp, build.SOURCES))
    so = os.path.join(out_dir, "libmoe_host_asan.so")
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    link = [CLANG, "-shared", "-fsanitize=address", "-shared-libsan", "-o", so] + objs + \
        ["-L" + rocm_lib, "-lamdhip64", "-Wl,-rpath," + rocm_lib]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return so


CHILD = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
from mixture_experts_layer_permute_amd import _lib
_lib.load({so!r})          # every later load returns this library
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {abi!r}]))
"""


def test_cpu_abi_tests_pass_under_host_asan(tmp_path):
    rt = asan_runtime()
    if rt is None or shutil.which(build.hipcc()) is None and not os.path.exists(build.hipcc()):
        pytest.skip("no hipcc or AddressSanitizer runtime in this toolchain")
    so = build_host_asan(str(tmp_path))
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    # the interpreter itself is not instrumented and keeps objects until exit
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), so=so,
                        abi=os.path.join(ROOT, "tests", "test_abi_cpu.py"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       env=env, cwd=str(tmp_path), timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]


PLANTED = r"""
extern "C" int planted(int n) {
    int* a = new int[n];
    for (int i = 0; i < n; ++i) a[i] = i;
    const int v = a[n];          // one past the end
    delete[] a;
    return v;
}
"""


def test_the_harness_reports_a_planted_host_overflow(tmp_path):
    """The same build flags, preload and options catch a one-past-the-end
    read in a test-only host function, so a clean run above means something."""
    rt = asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    src = tmp_path / "planted.cpp"
    src.write_text(PLANTED)
    so = str(tmp_path / "libplanted.so")
    r = subprocess.run([CLANG, "-shared", "-fPIC", "-O1", "-g", "-fsanitize=address",
                        "-shared-libsan", "-o", so, str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    code = "import ctypes; print(ctypes.CDLL(%r).planted(4))" % so
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
