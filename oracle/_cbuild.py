"""Builds and loads the oracle's one C helper (fixed-order fp32 gate logits).

Test infrastructure only: imported by the oracle, the tests, the smoke check
and the benchmark's CPU-baseline leg, never by the product path.
"""
import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gate_logits.c")
LIB = os.path.join(HERE, "_oracle_gate.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile gate_logits.c with gcc (no FMA contraction, no fast-math)."""
    if force or not os.path.exists(LIB) or \
            os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", SRC, "-o", tmp]
        subprocess.check_call(cmd)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(LIB)
        fp = ctypes.POINTER(ctypes.c_float)
        L.oracle_gate_logits_f32.argtypes = [fp, fp, fp, ctypes.c_long,
                                             ctypes.c_long, ctypes.c_long, fp]
        L.oracle_gate_logits_f32.restype = None
        _lib = L
    return _lib
