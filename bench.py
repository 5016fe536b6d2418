#!/usr/bin/env python3
"""One MoE layer forward + backward step on one MI355X, timed.

A step is the whole path: moe_gate_topk -> moe_permute -> moe_expert_ffn_fwd
-> moe_combine -> moe_combine_bwd -> moe_expert_ffn_bwd -> moe_unpermute_grad
-> moe_gate_topk_bwd, on inputs already resident in HBM.  Default workload:
the long-context chunk (T=65536 tokens, d=4096, f=14336, 128 SwiGLU
experts, top-8, Zipf 0.8 routing skew, bf16 storage with fp32
accumulation), the largest workload, seeded synthetic inputs.

Prints ONE JSON line.  Besides tokens/s it reports the grouped-GEMM TFLOP/s,
a per-kernel table from HIP events recorded around every kernel launch in a
second timed pass, the roofline of the dominant kernel, and the CPU oracle
timed on a bounded sample of the same workload (--no-cpu-baseline to skip).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoE layer fwd+bwd tokens/s and grouped-GEMM TFLOP/s "
          "(% of bf16 MFMA peak)")
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA, 256 CU x 2.4 GHz
PEAK_F32_TFLOPS = 157.3       # fp32 vector
PEAK_HBM_GBS = 8000.0

# HBM bytes per call (fetch + write; a GEMM stage's main and partial-tile
# launches together) per workload, from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE runs scaled by the readings of a plain 4 GiB device copy with a
# cold source in the same run (the summaries under profiles/ give commands
# and factors).  Valid only for the kernel sources whose code (comments and
# blank lines aside, see source_hash) has the SHA-256 prefix TRAFFIC_SRC;
# null once it changes.
TRAFFIC_SRC = "0a2b78b8595eaa05"
TRAFFIC_SOURCES = ("ggemm.hip", "common.h", "permute.hip", "combine.hip")
TRAFFIC = {
    # profiles/hbm_traffic_long_ctx_swiglu.md
    "long_ctx_swiglu": {
        "perm_copy": 9672133384,
        "gemm_up_swiglu": 680165917984,
        "gemm_down": 236757132844,
        "combine": 9680331290,
        "combine_bwd": 18275052402,
        "gemm_dA_swiglu": 433597753192,
        "gemm_dW2": 280430147842,
        "gemm_dW1": 280430147842,
        "gemm_dW3": 280430147842,
        "gemm_dX": 483202696840,
        "unpermute_grad": 10745676047,
    },
    # profiles/hbm_traffic_moe_s_like.md
    "moe_s_like": {
        "perm_copy": 101251013,
        "gemm_up_gelu": 1186682603,
        "gemm_down": 788540932,
        "combine": 101796089,
        "combine_bwd": 169050614,
        "gemm_dA_gelu": 1187828439,
        "gemm_dW2": 1141079018,
        "gemm_dW1": 1141079018,
        "gemm_dX": 784848258,
        "unpermute_grad": 134848008,
    },
    # profiles/hbm_traffic_skewed_zipf1.2.md
    "skewed_zipf1.2": {
        "perm_copy": 403755542,
        "gemm_up_gelu": 6901379050,
        "gemm_down": 5470188000,
        "combine": 404828755,
        "combine_bwd": 673548440,
        "gemm_dA_gelu": 6838157630,
        "gemm_dW2": 4295753454,
        "gemm_dW1": 4295753454,
        "gemm_dX": 5521059388,
        "unpermute_grad": 538016106,
    },
    # profiles/hbm_traffic_many_expert_zipf1.0.md
    "many_expert_zipf1.0": {
        "perm_copy": 404818532,
        "gemm_up_gelu": 4728292717,
        "gemm_down": 3071496410,
        "combine": 406925514,
        "combine_bwd": 675905913,
        "gemm_dA_gelu": 4751986138,
        "gemm_dW2": 5437037659,
        "gemm_dW1": 5437037659,
        "gemm_dX": 3071414822,
        "unpermute_grad": 539064293,
    },
}


def source_hash():
    """SHA-256 prefix of the kernel sources' code: // comments and blank
    lines are left out, so that a comment edit keeps the measured traffic."""
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_layer_permute_amd", "csrc", f),
                  encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def traffic_for(kernel, workload):
    """Measured HBM bytes per launch, or None if stale or not measured."""
    t = TRAFFIC.get(workload, {})
    if kernel not in t:
        return None
    return t[kernel] if source_hash() == TRAFFIC_SRC else None


def kernel_work(cfg):
    """Algorithmic work of one launch of each kernel: (amount, unit)."""
    R, T, d, f, E, k = cfg.R, cfg.T, cfg.d, cfg.f, cfg.E, cfg.k
    b = 2 if cfg.dtype == "bf16" else 4
    g = 2.0 * R * d * f
    w = {
        "gemm_up_gelu": (g, "flop"), "gemm_up_swiglu": (2 * g, "flop"),
        "gemm_down": (g, "flop"), "gemm_dA_gelu": (g, "flop"),
        "gemm_dA_swiglu": (g, "flop"), "gemm_dW2": (g, "flop"),
        "gemm_dW1": (g, "flop"), "gemm_dW3": (g, "flop"),
        "gemm_dX": ((2 * g if cfg.swiglu else g), "flop"),
        # bytes every memory-bound kernel must move at least once
        "perm_copy": (T * d * b + R * d * b + 4 * R, "byte"),
        "combine": (R * d * b + T * d * b + 8 * R, "byte"),
        "combine_bwd": (T * d * b + 2 * R * d * b + 12 * R, "byte"),
        # the layer calls it in accumulate mode: dx is read and written
        "unpermute_grad": (R * d * b + 2 * T * d * b + 4 * R, "byte"),
    }
    return w


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_ctx_swiglu",
                    help="workload name (moe_inputs.configs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--serial", action="store_true",
                    help="run every kernel on one stream (moe_set_overlap(0), the gate "
                         "backward on the step's stream) in the headline too; the "
                         "per-kernel pass is always serial")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU work for the oracle baseline")
    ap.add_argument("--cpu-tokens", type=int, default=32768,
                    help="sampled oracle baseline of a large workload: tokens "
                         "routed and carried through the row steps")
    ap.add_argument("--cpu-rows", type=int, default=800,
                    help="sampled oracle baseline: rows of each of the four "
                         "seeded experts carried through the FFN")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB before the "
                         "steps (a known-size reference for HBM byte counters)")
    ap.add_argument("--fuse-gather", action="store_true",
                    help="headline layer reads x through src inside the expert "
                         "GEMMs (no x_perm, no row-copy kernel); by default that "
                         "variant is timed after the headline as fused_gather")
    ap.add_argument("--chunk-tokens", type=int, default=0,
                    help="run the step over chunks of this many tokens with one "
                         "chunk's activation buffers (ChunkedMoELayer)")
    ap.add_argument("--no-graph-pass", action="store_true",
                    help="skip the timing of the step replayed from a HIP graph")
    ap.add_argument("--no-fused-pass", action="store_true",
                    help="skip the fused_gather timing (profiler runs: one kernel "
                         "variant per name)")
    ap.add_argument("--offload-experts", type=int, default=0,
                    help="after the headline, time the step with the expert weights "
                         "in pinned host memory, uploaded this many experts at a time "
                         "beside the GEMMs (OffloadedMoELayer); reported as "
                         "'offloaded', never as the value (it includes PCIe)")
    ap.add_argument("--pin-frac", type=float, default=0.0,
                    help="with --offload-experts: keep this fraction of the experts, "
                         "the most routed in the headline step, on the GPU (expert "
                         "pinning); their weights are not moved each step")
    ap.add_argument("--flush-mall", action="store_true",
                    help="add a per-kernel pass that reads a 512 MiB buffer before "
                         "every entry point, so memory kernels read from HBM")
    return ap.parse_args()


def mfma_loop_tflops(torch, L, s, stream, iters=50000, reps=3, random=False):
    """Attainable bf16 matrix-instruction rate: moe_mfma_loop on two
    workgroups of 4 waves per compute unit (two waves per SIMD), register
    operands only, timed with events on the step's stream.  random: the
    operands change with every instruction (moe_mfma_loop_random), the
    ceiling for GEMMs on random data (the rate depends on the data)."""
    from mixture_experts_layer_permute_amd import _lib
    blocks = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(blocks * 4, dtype=torch.float32, device="cuda")
    fn = L.moe_mfma_loop_random if random else L.moe_mfma_loop
    run = lambda: _lib.check(fn(blocks, iters, out.data_ptr(), out.numel(), s),
                             "moe_mfma_loop")
    run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return blocks * 4 * 4 * iters * 2.0 * 32 * 32 * 16 / (ms * 1e-3) / 1e12


def stream_copy_gbs(torch, mib=1024, reps=5):
    """Measured device copy bandwidth (read + write bytes / time), the
    reference for the memory kernels' GB/s."""
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * (mib << 20) / (ms * 1e-3) / 1e9


def parity(cfg, layer, fw, gr):
    """max|gpu - oracle| / max|oracle| per output of the step, against the
    oracle run of the CPU baseline (same inputs), with the test tolerance."""
    import numpy as np
    tol = 2e-2 if cfg.dtype == "bf16" else 1e-5
    pairs = {"y": (layer.y, fw["y"]), "dx": (layer.dx, gr["dx"]),
             "dW1": (layer.dW1, gr["dW1"]), "dW2": (layer.dW2, gr["dW2"]),
             "dWg": (layer.dWg, gr["dWg"])}
    out, ok = {}, True
    for n, (g, r) in pairs.items():
        g = g.float().cpu().numpy().astype(np.float64).reshape(np.shape(r))
        r = np.asarray(r, dtype=np.float64)
        den = float(np.abs(r).max())
        e = float(np.abs(g - r).max()) / den if den > 0 else float(np.abs(g).max())
        out[n] = round(e, 6)
        ok = ok and e <= tol
    idx_ok = bool(np.array_equal(layer.topk_idx.cpu().numpy(), fw["idx"]))
    out["topk_idx_exact"] = idx_ok
    out["tolerance"] = tol
    out["pass"] = bool(ok and idx_ok)
    return out


# Largest workload (grouped-GEMM FLOPs of a step) the full-layer oracle is
# timed on; beyond it a bounded sample of the same workload is timed.
ORACLE_FULL_FLOPS = 2e12


def oracle_threads():
    from threadpoolctl import threadpool_info
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return min(threads, len(os.sched_getaffinity(0)))


def cpu_baseline(cfg, budget_s):
    """The oracle, as it stands, on the host cores: full layer fwd+bwd."""
    import numpy as np
    import oracle
    from moe_inputs import rng

    # bounded sample: the first Ts tokens of the workload (all of it when it
    # fits the budget); weights are the workload's own
    Ts = cfg.T
    x = rng.gen(cfg, "x")[:Ts]
    dy = rng.gen(cfg, "dy")[:Ts]
    Wg = rng.gen(cfg, "Wg")
    W1 = rng.gen_experts(cfg, "W1")
    W2 = rng.gen_experts(cfg, "W2")
    W3 = rng.gen_experts(cfg, "W3") if cfg.swiglu else None
    bias = rng.logit_bias(cfg)
    reps, t_tot = 0, 0.0
    while True:
        t0 = time.perf_counter()
        fw = oracle.layer_forward(x, Wg, W1, W2, W3, k=cfg.k, act=cfg.act,
                                  bias=bias, renorm=cfg.renorm)
        gr = oracle.layer_backward(fw, dy, x, Wg, W1, W2, W3, act=cfg.act,
                                   renorm=cfg.renorm)
        t_tot += time.perf_counter() - t0
        reps += 1
        if t_tot >= budget_s or reps >= 5:
            break
    return {"value": reps * Ts / t_tot, "unit": "tokens/s", "cores": oracle_threads(),
            "kind": "oracle",
            "sample": "NumPy float64 oracle, full layer fwd+bwd of all %d tokens "
                      "(%d rep%s, %.1f s)" % (Ts, reps, "s" if reps > 1 else "", t_tot)}, fw, gr


def cpu_baseline_sampled(cfg, layer, args):
    """The oracle, as it stands, on a bounded sample of a workload whose full
    host pass would not fit: the routing of the first Ts tokens (fixed-order
    logits, top-k, weights, counting sort), the FFN forward and backward of
    sampled rows of the four seeded experts (weight gradients over those
    rows), and the row steps of the Ts tokens (combine, its backward, the
    unpermute, the gate backward) fed the GPU's own out_perm / dx_perm rows.
    Each part is timed; the per-token cost is (routing + row steps) / Ts +
    k * FFN / rows, reported as tokens/s.  Parity on the same sample: logits
    bits and top-k of the Ts tokens; y, d_out_perm, d_topk_w and dx rows of
    the Ts tokens; out_perm and dx_perm rows of the seeded experts."""
    import numpy as np
    import torch
    import oracle
    from moe_inputs import rng

    T, k, d, E, f = cfg.T, cfg.k, cfg.d, cfg.E, cfg.f
    Ts = max(1, min(T, args.cpu_tokens))
    toks = np.arange(Ts)
    tol = 2e-2 if cfg.dtype == "bf16" else 1e-5

    def rows(t, r):
        i = torch.as_tensor(np.asarray(r, np.int64), device=t.device)
        return t.index_select(0, i).float().cpu().numpy().astype(np.float64)

    def rel(g, r):
        den = float(np.abs(r).max())
        e = float(np.abs(g - r).max())
        return e / den if den > 0 else e

    x = rng.gen_rows(cfg, "x", toks)
    dy = rng.gen_rows(cfg, "dy", toks)
    Wg = rng.gen(cfg, "Wg")
    bias = rng.logit_bias(cfg)
    g_dest = layer.dest[:Ts].cpu().numpy()
    g_out = rows(layer.out_perm, g_dest.reshape(-1))
    g_dxp = rows(layer.dx_perm, g_dest.reshape(-1))
    dest_local = np.arange(Ts * k).reshape(Ts, k)

    t0 = time.perf_counter()
    logits = oracle.gate_logits(x, Wg, bias)
    idx = oracle.topk_select(logits, k)
    w = oracle.gate_weights(logits, idx, cfg.renorm)
    oracle.permute(idx, E)
    t_route = time.perf_counter() - t0

    t0 = time.perf_counter()
    y = oracle.combine(g_out, dest_local, w)
    d_out, dw = oracle.combine_bwd(dy, g_out, dest_local, w)
    dx = oracle.unpermute_grad(g_dxp, dest_local)
    _, _, dx_gate = oracle.gate_bwd(x, Wg, logits, idx, w, dw, cfg.renorm)
    dx = dx + dx_gate
    t_rows = time.perf_counter() - t0

    par = {"sample_tokens": Ts}
    par["logits_bit_exact"] = bool(np.array_equal(
        layer.logits[:Ts].cpu().numpy().view(np.uint32), logits.view(np.uint32)))
    par["topk_idx_exact"] = bool(np.array_equal(layer.topk_idx[:Ts].cpu().numpy(), idx))
    par["y"] = rel(rows(layer.y, toks), y)
    par["d_out_perm"] = rel(rows(layer.d_out_perm, g_dest.reshape(-1)),
                            d_out.reshape(Ts * k, d))
    par["d_topk_w"] = rel(layer.d_topk_w[:Ts].cpu().numpy().astype(np.float64), dw)
    par["dx"] = rel(rows(layer.dx, toks), dx)

    # FFN: sampled rows of the seeded experts (rows and tokens from the GPU's
    # routing; each token's gate weight from the oracle's own routing of it)
    offsets = layer.offsets.cpu().numpy()
    src = layer.src.cpu().numpy()
    g = np.random.default_rng(cfg.seed + 5)
    t_ffn, n_rows, e_out, e_dxp = 0.0, 0, 0.0, 0.0
    for e in rng.seeded_experts(cfg):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        r = np.sort(g.choice(np.arange(a, b), size=min(args.cpu_rows, b - a),
                             replace=False))
        tok = src[r]
        W1e = rng.gen(cfg, "W1", int(e))
        W2e = rng.gen(cfg, "W2", int(e))
        W3e = rng.gen(cfg, "W3", int(e)) if cfg.swiglu else None
        xr = rng.gen_rows(cfg, "x", tok)
        dyr = rng.gen_rows(cfg, "dy", tok)
        t0 = time.perf_counter()
        lr = oracle.gate_logits(xr, Wg, bias)
        ir = oracle.topk_select(lr, k)
        wr = oracle.gate_weights(lr, ir, cfg.renorm)
        slot = np.argmax(ir == e, axis=1)
        assert np.all(ir[np.arange(len(r)), slot] == e), "routing of a sampled row"
        dO = wr[np.arange(len(r)), slot][:, None] * dyr
        _, _, _, O = oracle.ffn_fwd_segment(xr, W1e, W2e, W3e, cfg.act)
        dX = oracle.ffn_bwd_segment(dO, xr, W1e, W2e, W3e, cfg.act)[0]
        t_ffn += time.perf_counter() - t0
        n_rows += len(r)
        e_out = max(e_out, rel(rows(layer.out_perm, r), O))
        e_dxp = max(e_dxp, rel(rows(layer.dx_perm, r), dX))
        del W1e, W2e, W3e
    par["out_perm_seeded_rows"] = e_out
    par["dx_perm_seeded_rows"] = e_dxp
    par["seeded_rows"] = n_rows
    par["tolerance"] = tol
    par["pass"] = bool(par["logits_bit_exact"] and par["topk_idx_exact"] and
                       max(par[n] for n in ("y", "d_out_perm", "d_topk_w", "dx",
                                            "out_perm_seeded_rows",
                                            "dx_perm_seeded_rows")) <= tol)
    for n in ("y", "d_out_perm", "d_topk_w", "dx", "out_perm_seeded_rows",
              "dx_perm_seeded_rows"):
        par[n] = round(par[n], 6)
    per_tok = (t_route + t_rows) / Ts + (k * t_ffn / n_rows if n_rows else 0.0)
    return {"value": round(1.0 / per_tok, 2), "unit": "tokens/s", "cores": oracle_threads(),
            "kind": "oracle",
            "sample": "NumPy float64 oracle on a bounded sample: routing of %d tokens "
                      "(%.2f s), row steps of those tokens (%.2f s), FFN forward and "
                      "backward of %d rows of the 4 seeded experts (%.2f s); tokens/s = "
                      "1 / ((routing + row steps) / %d + k * FFN / %d)"
                      % (Ts, t_route, t_rows, n_rows, t_ffn, Ts, n_rows),
            "parity": par}


def load_stats(counts, cfg):
    """Per-expert row counts of the routing the step ran on."""
    if counts.dim() == 2:             # per chunk
        counts = counts.sum(0)
    c = sorted(int(v) for v in counts.cpu().tolist())
    return {"max_over_mean": round(c[-1] * cfg.E / cfg.R, 3),
            "empty_experts": sum(1 for v in c if v == 0),
            "rows_min": c[0], "rows_median": c[len(c) // 2], "rows_max": c[-1],
            "zipf_s": cfg.zipf_s}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(no collectives, no sharding); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import mixture_experts_layer_permute_amd as M
    from mixture_experts_layer_permute_amd import _lib
    from moe_inputs import CONFIGS, device

    cfg = CONFIGS[args.workload]
    torch.cuda.set_device(0)
    M.moe_init(0)
    M.moe_set_overlap(not args.serial)
    t = device.gen_all(cfg)
    inputs_bytes = sum(v.numel() * v.element_size() for v in t.values() if v is not None)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    if args.chunk_tokens:
        layer = M.ChunkedMoELayer(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act,
                                  device.torch_dtype(cfg), cfg.renorm,
                                  chunk_tokens=args.chunk_tokens)
    else:
        layer = M.MoELayer(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act,
                           device.torch_dtype(cfg), cfg.renorm, fuse_gather=args.fuse_gather,
                           overlap_gate=not args.serial)
    layer.bind(t["x"], t["Wg"], t["W1"], t["W2"], t["W3"], t["bias"], t["dy"])
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    if args.calib_copy_mb:
        # plain elementwise copy (ordinary loads and stores) of a known size:
        # reads and writes calib_copy_mb MiB each.  The source is evicted from
        # the 256 MB MALL first (a 1 GiB read of other data), and the copy
        # should be many times the MALL, so that few of its writes are still
        # waiting there when it ends: otherwise the counters see less than
        # the copy moves
        n = (args.calib_copy_mb << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        junk = torch.ones(256 << 20, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        junk.sum()
        torch.cuda.synchronize()
        torch.add(src, 0.0, out=dst)
        torch.cuda.synchronize()
        del src, dst, junk

    for _ in range(args.warmup):
        layer.step(s)
    torch.cuda.synchronize()

    # ---- headline: K steps, nothing else in the stream
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        layer.step(s)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1) / args.steps
    hbm_peak = torch.cuda.max_memory_allocated()

    # ---- step-time distribution: an event pair around every step
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        layer.step(s)
        b.record(stream)
    torch.cuda.synchronize()
    step_ms = sorted(a.elapsed_time(b) for a, b in evs)

    def pct(q):
        return step_ms[min(len(step_ms) - 1, int(q * (len(step_ms) - 1) + 0.5))]

    # ---- the same step captured once in a HIP graph (side-stream fork and
    # join inside it) and replayed K times; bit-identity: tests/test_gpu_graph.py
    graph = None
    if not args.chunk_tokens and not args.no_graph_pass:
        y0 = layer.y.clone()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            layer.step()
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.step()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                g.replay()
            ev0.record(stream)
            for _ in range(args.steps):
                g.replay()
            ev1.record(stream)
        torch.cuda.synchronize()
        gms = ev0.elapsed_time(ev1) / args.steps
        graph = {"ms_per_step": round(gms, 5), "value": round(cfg.T / (gms * 1e-3), 1),
                 "y_bit_identical": bool(torch.equal(y0, layer.y))}
        del g

    # ---- per-kernel pass: HIP events around every launch, same K steps
    L = _lib.load()
    # every kernel alone: the library keeps its side stream off while events
    # are on, and the layer's gate backward stays on the step's stream
    og = getattr(layer, "overlap_gate", None)
    if og is not None:
        layer.overlap_gate = False
    # room for every launch of the step (a chunked step launches per chunk);
    # the library drops records past its capacity, so a full buffer is an error
    per_step = 64 * (getattr(layer, "nch", 0) + 1)
    cap = args.steps * per_step
    _lib.check(L.moe_profile_enable(cap), "moe_profile_enable")
    for _ in range(args.steps):
        layer.step(s)
    torch.cuda.synchronize()
    if og is not None:
        layer.overlap_gate = og
    recs = _lib.profile_records()
    if len(recs) >= cap:
        raise RuntimeError("per-kernel pass: %d launch records filled the buffer" % len(recs))
    L.moe_profile_disable()
    per = {}
    for name, kms in recs:
        per.setdefault(name, []).append(kms)

    # ---- optional pass with the MALL flushed before every entry point
    flushed = {}
    if args.flush_mall and hasattr(layer, "stage_calls"):
        # reading 512 MiB evicts the 256 MB MALL with clean lines (a write
        # would leave dirty lines to be written back during the next kernel)
        junk = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
        calls = layer.stage_calls()
        nsteps = max(1, min(args.steps, 10))
        _lib.check(L.moe_profile_enable(nsteps * per_step), "moe_profile_enable")
        for _ in range(nsteps):
            for _, call in calls:
                junk.sum()
                call()
        torch.cuda.synchronize()
        frecs = _lib.profile_records()
        if len(frecs) >= nsteps * per_step:
            raise RuntimeError("flushed pass: launch records filled the buffer")
        for name, kms in frecs:
            flushed.setdefault(name, []).append(kms)
        L.moe_profile_disable()
        del junk
        torch.cuda.empty_cache()
    copy_gbs = stream_copy_gbs(torch)
    mfma_tf = mfma_loop_tflops(torch, L, s, stream)
    mfma_rand_tf = mfma_loop_tflops(torch, L, s, stream, iters=20000, random=True)
    work = kernel_work(cfg)
    kernels = {}
    for name, v in per.items():
        kernels[name] = {"avg_ms": round(sum(v) / len(v), 5),
                         "launches_per_step": len(v) / args.steps,
                         "ms_per_step": round(sum(v) / args.steps, 5)}
    # A grouped GEMM whose last round of workgroups would be nearly empty is
    # launched as a main kernel plus a narrow-tile "<name>_tail" kernel; its
    # work and rates belong to the pair (one launch of each per call).
    parts = {}
    for name in kernels:
        base = name[:-5] if name.endswith("_tail") else name
        parts.setdefault(base, []).append(name)
    gemm_ms = 0.0
    stage_ms = {}          # per call of the stage (main + tail)
    for base, names in parts.items():
        if base not in work:
            continue
        calls = kernels[base]["launches_per_step"] if base in kernels else 1.0
        if args.chunk_tokens:
            # one launch per chunk (plus GEMM1's recomputation): rates are the
            # step's algorithmic work over the stage's time per step
            calls = 1.0
        per_call = sum(kernels[n]["ms_per_step"] for n in names) / calls
        stage_ms[base] = per_call
        amt, unit = work[base]
        ent = kernels[base] if base in kernels else kernels[names[0]]
        if len(names) > 1:
            ent["with_tail_avg_ms"] = round(per_call, 5)
            for n in names:
                if n != base:
                    kernels[n]["part_of"] = base
        if unit == "flop":
            ent["tflops"] = round(amt / (per_call * 1e-3) / 1e12, 2)
            ent["frac_of_peak"] = round(ent["tflops"] / PEAK_BF16_TFLOPS, 4)
            if cfg.dtype == "bf16":
                ent["frac_of_mfma_loop"] = round(ent["tflops"] / mfma_tf, 4)
                ent["frac_of_mfma_random"] = round(ent["tflops"] / mfma_rand_tf, 4)
            gemm_ms += per_call * calls
        else:
            ent["gbs"] = round(amt / (per_call * 1e-3) / 1e9, 1)
            ent["frac_of_peak"] = round(ent["gbs"] / PEAK_HBM_GBS, 4)
            ent["frac_of_copy"] = round(ent["gbs"] / copy_gbs, 4)
            # working set under the 256 MB MALL: the rate is cache-assisted
            ent["cache_resident"] = amt < 256e6
            if base in flushed:
                fms = sum(flushed[base]) / len(flushed[base])
                ent["gbs_mall_flushed"] = round(amt / (fms * 1e-3) / 1e9, 1)
    gemm_flops = cfg.gemm_flops_fwd_bwd()
    dom = max(stage_ms, key=lambda n: stage_ms[n] * kernels.get(n, {}).get(
        "launches_per_step", 1.0))
    amt, unit = work[dom]
    launches = sorted(parts[dom])
    if unit == "flop":
        peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
        ach = amt / (stage_ms[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                "traffic": traffic_for(dom, cfg.name),
                "kernel": dom, "launches": launches, "work_per_launch": amt}
    else:
        ach = amt / (stage_ms[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": traffic_for(dom, cfg.name), "kernel": dom,
                "launches": launches, "work_per_launch": amt}

    out = {
        "metric": METRIC,
        "value": round(cfg.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded counter-based generator, inputs resident in HBM)",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "f": cfg.f,
                   "E": cfg.E, "k": cfg.k, "act": cfg.act, "renorm": cfg.renorm,
                   "routing_skew_zipf_s": cfg.zipf_s, "stream_overlap": not args.serial,
                   "fused_gather": args.fuse_gather,
                   "chunk_tokens": args.chunk_tokens or None},
        "hbm_peak_bytes": hbm_peak,
        "hbm_inputs_bytes": inputs_bytes,
        "gemm_tflops_layer": round(gemm_flops / (ms * 1e-3) / 1e12, 2),
        "gemm_tflops_kernels": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 2)
        if gemm_ms else None,
        "gemm_frac_of_bf16_peak": round(gemm_flops / (gemm_ms * 1e-3) / 1e12
                                        / PEAK_BF16_TFLOPS, 4) if gemm_ms else None,
        "wall_s_timed_region": round(wall, 4),
        "step_ms": {"p10": round(pct(0.1), 5), "p50": round(pct(0.5), 5),
                    "p90": round(pct(0.9), 5)},
        "value_at_median_step": round(cfg.T / (pct(0.5) * 1e-3), 1),
        "stream_copy_gbs": round(copy_gbs, 1),
        "mfma_loop_tflops": round(mfma_tf, 1),
        "mfma_loop_random_tflops": round(mfma_rand_tf, 1),
        "gemm_frac_of_mfma_loop": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / mfma_tf, 4)
        if gemm_ms and cfg.dtype == "bf16" else None,
        "gemm_frac_of_mfma_random": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / mfma_rand_tf, 4)
        if gemm_ms and cfg.dtype == "bf16" else None,
        "roofline": roof,
        "graph_replay": graph,
        "kernels": kernels,
        "load": load_stats(layer.counts, cfg),
    }
    full_oracle = cfg.gemm_flops_fwd_bwd() <= ORACLE_FULL_FLOPS
    if not args.no_cpu_baseline and not full_oracle:
        # the sample reads the step's whole-batch buffers (not a chunked step's)
        if isinstance(layer, M.MoELayer):
            out["cpu_baseline"] = cpu_baseline_sampled(cfg, layer, args)
    elif not args.no_cpu_baseline:
        base, fw, gr = cpu_baseline(cfg, args.cpu_seconds)
        base["parity"] = parity(cfg, layer, fw, gr)
        out["cpu_baseline"] = base
    if not args.fuse_gather and not args.no_fused_pass and not args.chunk_tokens:
        # the same step with the row copy fused into the expert GEMMs (its
        # results are bit-identical: tests/test_gpu_gather.py); timed after
        # the headline layer is freed, so that both never share HBM
        y0 = layer.y.clone()
        del layer
        torch.cuda.empty_cache()
        fl = M.MoELayer(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act,
                        device.torch_dtype(cfg), cfg.renorm, fuse_gather=True,
                        overlap_gate=not args.serial)
        fl.bind(t["x"], t["Wg"], t["W1"], t["W2"], t["W3"], t["bias"], t["dy"])
        for _ in range(args.warmup):
            fl.step(s)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            fl.step(s)
        ev1.record(stream)
        torch.cuda.synchronize()
        fms = ev0.elapsed_time(ev1) / args.steps
        out["fused_gather"] = {"ms_per_step": round(fms, 5),
                               "value": round(cfg.T / (fms * 1e-3), 1),
                               "y_bit_identical": bool(torch.equal(y0, fl.y)),
                               "x_perm_bytes_not_allocated": cfg.T * cfg.k * cfg.d
                               * (2 if cfg.dtype == "bf16" else 4)}
        del fl
        layer = None
    if args.offload_experts and not args.chunk_tokens:
        counts = None
        if layer is not None:             # the headline layer's buffers out of HBM
            y0 = layer.y.clone()
            counts = layer.counts.cpu()
            del layer
        out["offloaded"] = offloaded_pass(args, cfg, t, y0, s, stream, counts)
    print(json.dumps(out), flush=True)


def offloaded_pass(args, cfg, t, y0, s, stream, counts=None):
    """The same step with the expert weights in pinned host memory
    (OffloadedMoELayer): the weights of G experts at a time are uploaded
    beside the GEMMs, the weight gradients downloaded.  The device copies of
    the weights are freed first, so the HBM peak is the offloaded one."""
    import torch
    import mixture_experts_layer_permute_amd as M
    from moe_inputs import device

    def pinned(name):
        if t[name] is None:
            return None
        h = torch.empty(t[name].shape, dtype=t[name].dtype, pin_memory=True)
        h.copy_(t[name])
        t[name] = None                      # drop the device copy
        return h
    W1, W2, W3 = pinned("W1"), pinned("W2"), pinned("W3")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    G = args.offload_experts
    pinned = (M.OffloadedMoELayer.most_routed(counts, args.pin_frac)
              if args.pin_frac > 0 and counts is not None else [])
    lay = M.OffloadedMoELayer(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act,
                              device.torch_dtype(cfg), cfg.renorm, group_experts=G,
                              pinned=pinned)
    lay.bind(t["x"], t["Wg"], W1, W2, W3, t["bias"], t["dy"])
    for _ in range(args.warmup):
        lay.step(s)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        lay.step(s)
    stream.wait_event(lay.grads_ready)     # the last step's gradients are on the host
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    b = 2 if cfg.dtype == "bf16" else 4
    per_expert = cfg.d * cfg.f * (3 if cfg.swiglu else 2) * b
    n = len(lay.groups)
    off_experts = cfg.E - len(pinned)
    # uploads: every offloaded group in the forward, all but the last two
    # again in the backward; downloads: every offloaded expert's weight
    # gradients (pinned experts' weights and gradients stay on the GPU)
    up = (off_experts + sum(ne for _, ne in lay.groups[:max(0, n - 2)])) * per_expert
    down = off_experts * per_expert
    return {"experts_per_group": lay.G, "pinned_experts": len(pinned),
            "ms_per_step": round(ms, 5),
            "value": round(cfg.T / (ms * 1e-3), 1), "unit": "tokens/s",
            "pcie_bytes_per_step": up + down,
            "pcie_gbs": round((up + down) / (ms * 1e-3) / 1e9, 1),
            "hbm_peak_bytes": torch.cuda.max_memory_allocated(),
            "expert_weight_bytes_on_host": cfg.E * per_expert,
            "pinned_weight_bytes_on_gpu": len(pinned) * per_expert,
            "y_bit_identical": bool(torch.equal(y0, lay.y))}


if __name__ == "__main__":
    main()
