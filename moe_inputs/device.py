"""Workload tensors generated directly in GPU memory, bit-identical to the
host generator in rng.py (same counter-based definition, see csrc/fill.hip).

Test and benchmark infrastructure: builds inputs, computes nothing of the
layer.
"""
import ctypes
import os

import numpy as np
import torch

from . import rng
from .configs import MoEConfig

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_inputs.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe_inputs.so not built (moe_inputs/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_inputs_fill_normal.restype = ctypes.c_int
        L.moe_inputs_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_int,
                                             ctypes.c_uint64, ctypes.c_uint64,
                                             ctypes.c_uint64, ctypes.c_float,
                                             ctypes.c_void_p]
        _lib = L
    return _lib


def torch_dtype(cfg: MoEConfig):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def fill(out: torch.Tensor, key: int, scale: float, start: int = 0):
    assert out.is_cuda and out.is_contiguous()
    s = torch.cuda.current_stream(out.device).cuda_stream
    r = _load().moe_inputs_fill_normal(out.data_ptr(),
                                       1 if out.dtype == torch.bfloat16 else 0,
                                       key, start, out.numel(),
                                       float(np.float32(scale)), s)
    if r != 0:
        raise RuntimeError("moe_inputs_fill_normal failed (%d)" % r)
    return out


def gen(cfg: MoEConfig, name: str, device="cuda") -> torch.Tensor:
    """One named layer input on the device: x, Wg, dy [2-D]; W1/W3/W2 stacked
    over experts [E, ...]."""
    tid, shape, std = rng.tensor_spec(cfg, name)
    dt = torch_dtype(cfg)
    if name in ("W1", "W3", "W2"):
        out = torch.empty((cfg.E,) + shape, dtype=dt, device=device)
        for e in range(cfg.E):
            fill(out[e], rng.stream_key(cfg.seed, tid, e), std)
        return out
    out = torch.empty(shape, dtype=dt, device=device)
    return fill(out, rng.stream_key(cfg.seed, tid, 0), std)


def gen_all(cfg: MoEConfig, device="cuda"):
    """Every input of one layer step: dict of device tensors (bias f32 or None)."""
    t = {n: gen(cfg, n, device) for n in ("x", "Wg", "W1", "W2", "dy")}
    t["W3"] = gen(cfg, "W3", device) if cfg.swiglu else None
    b = rng.logit_bias(cfg)
    t["bias"] = None if b is None else torch.from_numpy(b).to(device)
    return t
