"""Rates of the LDS paths of the grouped GEMM's main loop, per compute unit.

    python -m mixture_experts_layer_permute_amd.lds_probe [--iters N] [--reps N]
        [--src-kb KB]

Runs moe_lds_probe on two 4-wave workgroups per compute unit: each kind
alone, then the direct-to-LDS loads beside each kind of read, with as many
read bytes as loaded bytes and with three times as many (the ratio of
fragment reads to ring loads of a 256 x 256 tile).  Prints bytes per ns per
compute unit for every kind in the run, and for the side-by-side runs the
time against the longer of the two kinds' times alone for the same bytes
(1.00: they overlap fully; their sum over that: they serialise).

    ds_read_b128          plain 16-byte fragment reads (K-contiguous operands)
    ds_read_b64_tr_b16    transposing 8-byte reads (M/N-contiguous operands)
    buffer_load ... lds   the ring's direct-to-LDS loads, from a source of
                          --src-kb KB (a power of two from 8 to 1048576) that
                          stays in the L2 at the default size
"""
import argparse

import torch

from . import _lib
from .ops import moe_init

KINDS = {1: "ds_read_b128", 2: "ds_read_b64_tr_b16", 4: "buffer_load ... lds"}
MODES = (1, 2, 4, 5, 6, 13, 14)
ROUND = 32 * 1024                 # bytes per workgroup, round and kind (reads x3 with bit 8)


def kind_bytes(mode, kind_bit):
    return ROUND * (3 if (mode & 8) and kind_bit != 4 else 1)


def run(iters=2000, reps=5, src_kb=1024):
    """{mode: ({kind: bytes per ns per compute unit}, time / longer time alone
    or None)}, medians over reps."""
    L = _lib.load()
    torch.cuda.set_device(0)
    moe_init(0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 2 * cus
    src = torch.zeros(src_kb * 1024 // 2, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(blocks * 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def launch(mode, n):
        _lib.check(L.moe_lds_probe(mode, blocks, n, src.data_ptr(), src.numel() * 2,
                                   out.data_ptr(), out.numel(), stream.cuda_stream),
                   "moe_lds_probe")

    res = {}
    for mode in MODES:
        launch(mode, 10)
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch(mode, iters)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e6)          # ns
        ns = sorted(times)[len(times) // 2]
        rates = {KINDS[b]: blocks * iters * kind_bytes(mode, b) / ns / cus
                 for b in (1, 2, 4) if mode & b}
        ratio = None
        if len(rates) > 1:
            alone = [blocks * iters * kind_bytes(mode, b) / cus / res[b][0][KINDS[b]]
                     for b in (1, 2, 4) if mode & b]
            ratio = ns / max(alone)
        res[mode] = (rates, ratio)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--iters", type=int, default=2000)
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--src-kb", type=int, default=1024)
    a = ap.parse_args()
    for mode, (rates, ratio) in run(a.iters, a.reps, a.src_kb).items():
        line = " + ".join(rates) + (" (reads x3)" if mode & 8 else "") + ": " + \
            ", ".join("%s %.0f B/ns per CU" % (k, v) for k, v in rates.items())
        if ratio is not None:
            line += "; time / longer kind alone %.2f" % ratio
        print(line)


if __name__ == "__main__":
    main()
