"""Helpers shared by the GPU tests: uploads, tolerance checks, case banners."""
import sys

import numpy as np
import pytest
import torch

TOL = {"bf16": 2e-2, "f32": 1e-5}   # max|err| <= TOL * max|ref|, per tensor
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(),
                               reason="needs an MI355X")


def banner(*what):
    """Print (and flush) what the next GPU step is, so a crash names it."""
    print("[gpu case]", *what, flush=True)
    sys.stdout.flush()


def dev(a, dt="f32"):
    """fp32 values (exactly representable in dt) -> device tensor of dt."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return t.to(TDT[dt]).contiguous()


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def host_i(t):
    return t.detach().cpu().numpy()


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    if scale == 0.0:
        return err
    return err / scale


def assert_close(got, ref, dt, name):
    if isinstance(got, torch.Tensor):
        got = host(got)
    e = rel_err(got, ref)
    assert e <= TOL[dt], "%s: max|err|/max|ref| = %.3g > %.1g" % (name, e, TOL[dt])
    return e


def assert_equal_i(got, ref, name):
    if isinstance(got, torch.Tensor):
        got = host_i(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    bad = np.flatnonzero(got.reshape(-1) != ref.reshape(-1))
    assert bad.size == 0, "%s: %d mismatches, first at %d" % (name, bad.size, bad[0])


def saved_state(act, H, H3=None):
    """What the FFN forward saves for its backward, from the oracle's
    pre-activations: GeLU'(H), or [H3 * SiLU'(H1) | SiLU(H1)] for SwiGLU."""
    import oracle
    if act == "gelu":
        return oracle.gelu_grad(H)
    return np.concatenate([np.asarray(H3, np.float64) * oracle.silu_grad(H),
                           oracle.silu(H)], axis=1)
