"""Timing of the expert FFN's grouped GEMMs on equal segments.

    python -m mixture_experts_layer_permute_amd.gemm_bench E ROWS D F ACT [--reps N]
        [--operands random|zero|const] [--vendor]

E experts of ROWS rows each (uniform routing), model width D, hidden width F,
ACT gelu or swiglu, bf16.  Runs moe_expert_ffn_fwd and moe_expert_ffn_bwd
REPS times with the library's per-launch event timing and prints, per
product, the median time and its rate in TFLOP/s (2 * rows * D * F per
product, twice that for the SwiGLU up and dX products), plus a hash of the
outputs (equal hashes: equal bits).

--operands zero / const fill every input with zeros / one constant instead
of random values: the matrix cores' sustained rate depends on the data, and
this shows by how much.  --vendor also times torch.matmul on the flattened
shapes (a reference only; nothing in the library calls it).
"""
import argparse
import hashlib

import torch

from . import _lib
from .ops import moe_expert_ffn_bwd, moe_expert_ffn_fwd, moe_init


def _products(E, n, d, f, act):
    g1 = 2.0 * E * n * d * f
    return {"gemm_up_gelu": g1, "gemm_up_swiglu": 2 * g1, "gemm_down": g1,
            "gemm_dA_gelu": g1, "gemm_dA_swiglu": g1, "gemm_dW2": g1, "gemm_dW1": g1,
            "gemm_dW3": g1, "gemm_dX": 2 * g1 if act == "swiglu" else g1}


def run(E, n, d, f, act="gelu", reps=3, operands="random", vendor=False):
    L = _lib.load()
    torch.cuda.set_device(0)
    moe_init(0)
    R = E * n
    bf = torch.bfloat16
    g = torch.Generator(device="cuda").manual_seed(0)

    def make(*shape, scale=1.0):
        if operands == "zero":
            return torch.zeros(*shape, device="cuda", dtype=bf)
        if operands == "const":
            return torch.full(shape, 0.25, device="cuda", dtype=bf)
        return (torch.randn(*shape, device="cuda", generator=g) * scale).to(bf)

    xp = make(R, d)
    W1 = make(E, d, f, scale=d ** -0.5)
    W2 = make(E, f, d, scale=f ** -0.5)
    W3 = make(E, d, f, scale=d ** -0.5) if act == "swiglu" else None
    dO = make(R, d)
    off = torch.arange(0, R + 1, n, dtype=torch.int32, device="cuda")
    h, a, o = moe_expert_ffn_fwd(xp, off, W1, W2, W3, act)
    outs = moe_expert_ffn_bwd(dO, xp, h, a, off, W1, W2, W3, act)
    torch.cuda.synchronize()
    # with event timing on, the library runs every launch on the caller's
    # stream, one at a time, so each time is the launch's own
    _lib.check(L.moe_profile_enable(64 * reps), "moe_profile_enable")
    for _ in range(reps):
        moe_expert_ffn_fwd(xp, off, W1, W2, W3, act, out=(h, a, o))
        moe_expert_ffn_bwd(dO, xp, h, a, off, W1, W2, W3, act, out=outs)
    torch.cuda.synchronize()
    recs = _lib.profile_records()
    L.moe_profile_disable()
    per = {}
    for name, ms in recs:
        per.setdefault(name, []).append(ms)
    work = _products(E, n, d, f, act)
    res = {}
    for name, v in per.items():
        if name in work:
            ms = sorted(v)[len(v) // 2]
            res[name] = (ms, work[name] / (ms * 1e-3) / 1e12)
    hh = hashlib.sha256()
    for t in (h, a, o) + tuple(x for x in outs if x is not None):
        hh.update(t.view(torch.int16).cpu().numpy().tobytes())
    ref = {}
    if vendor:
        def timed(fn, flops):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return flops / (e0.elapsed_time(e1) / reps * 1e-3) / 1e12
        g1 = 2.0 * R * d * f
        W1f, W2f = W1[0].contiguous(), W2[0].contiguous()
        ref["matmul [R,d]x[d,f]"] = timed(lambda: xp @ W1f, g1)
        ref["matmul [R,f]x[f,d]"] = timed(lambda: a[:, :f] @ W2f, g1)
    return res, hh.hexdigest()[:12], ref


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("E", type=int)
    ap.add_argument("rows", type=int)
    ap.add_argument("d", type=int)
    ap.add_argument("f", type=int)
    ap.add_argument("act", choices=["gelu", "swiglu"])
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--operands", choices=["random", "zero", "const"], default="random")
    ap.add_argument("--vendor", action="store_true")
    a = ap.parse_args()
    res, h, ref = run(a.E, a.rows, a.d, a.f, a.act, a.reps, a.operands, a.vendor)
    tot_ms = sum(ms for ms, _ in res.values())
    tot_f = sum(_products(a.E, a.rows, a.d, a.f, a.act)[k] for k in res)
    print("E%d rows%d d%d f%d %s %s | total %.0f TFLOP/s | %s | hash %s" % (
        a.E, a.rows, a.d, a.f, a.act, a.operands, tot_f / (tot_ms * 1e-3) / 1e12,
        " ".join("%s=%.3fms/%.0fTF" % (k[5:], ms, tf) for k, (ms, tf) in res.items()), h))
    for k, tf in ref.items():
        print("  vendor %s: %.0f TFLOP/s" % (k, tf))


if __name__ == "__main__":
    main()
