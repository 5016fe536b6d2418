"""ChunkedMoELayer: the layer step over chunks of tokens with one chunk's
dispatch and activation buffers.  Routing, y, dx and dWg must be bit-identical
to MoELayer's (the same per-row arithmetic and the same gate backward); dW1,
dW2, dW3 are the same sums taken chunk by chunk, so they are compared within
the dtype's tolerance, with MoELayer and with the oracle."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_permute_amd as M
import oracle
from moe_inputs import device, rng, small_variant

from _gpu import assert_close, banner, host, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]

CASES = [  # workload, overrides, chunk_tokens
    ("moe_s_like", dict(T=1000, d=256, f=512, E=8, k=2), 256),      # ragged last chunk
    ("moe_s_like", dict(T=1000, d=256, f=512, E=8, k=2), 1000),     # one chunk
    ("long_ctx_swiglu", dict(T=777, d=128, f=256, E=16, k=4), 300),
    ("many_expert_zipf1.0", dict(T=1200, d=128, f=256, E=32, k=2), 400),
    ("tiny_fp32", {}, 64),
    ("tiny_fp32", dict(T=100), 1),                                   # one token per chunk
]

SAME = ["logits", "topk_idx", "topk_w", "y", "d_topk_w", "dx", "dWg"]


def run(layer, t):
    layer.bind(t["x"], t["Wg"], t["W1"], t["W2"], t["W3"], t["bias"], t["dy"])
    layer.step()
    torch.cuda.synchronize()
    return layer


@pytest.mark.parametrize("case", CASES)
def test_chunked_matches_whole_layer(case):
    name, kw, C = case
    cfg = small_variant(name, **kw)
    banner("chunked", cfg.short(), C)
    t = device.gen_all(cfg)
    args = (cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act, device.torch_dtype(cfg), cfg.renorm)
    whole = run(M.MoELayer(*args), t)
    ch = run(M.ChunkedMoELayer(*args, chunk_tokens=C), t)
    for n in SAME:
        assert torch.equal(getattr(whole, n), getattr(ch, n)), n
    dt = cfg.dtype
    wnames = ["dW1", "dW2"] + (["dW3"] if cfg.swiglu else [])
    for n in wnames:
        assert_close(getattr(ch, n), host(getattr(whole, n)), dt, n + " vs whole layer")
    # and against the oracle on the host copy of the inputs
    x, Wg, dy = (rng.gen(cfg, n) for n in ("x", "Wg", "dy"))
    W1, W2 = rng.gen_experts(cfg, "W1"), rng.gen_experts(cfg, "W2")
    W3 = rng.gen_experts(cfg, "W3") if cfg.swiglu else None
    fw = oracle.layer_forward(x, Wg, W1, W2, W3, k=cfg.k, act=cfg.act,
                              bias=rng.logit_bias(cfg), renorm=cfg.renorm)
    gr = oracle.layer_backward(fw, dy, x, Wg, W1, W2, W3, act=cfg.act, renorm=cfg.renorm)
    for n in wnames:
        assert_close(getattr(ch, n), gr[n], dt, n + " vs oracle")
    # a zero-load expert keeps an exact zero gradient through the accumulation
    counts = host(whole.counts)
    for e in np.nonzero(counts == 0)[0]:
        assert float(ch.dW1[e].abs().max()) == 0.0 and float(ch.dW2[e].abs().max()) == 0.0


def test_backward_twice_recomputes_every_chunk():
    cfg = small_variant("moe_s_like", T=900, d=128, f=256, E=8, k=2)
    banner("chunked backward twice", cfg.short())
    t = device.gen_all(cfg)
    ch = M.ChunkedMoELayer(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act,
                           device.torch_dtype(cfg), cfg.renorm, chunk_tokens=256)
    run(ch, t)
    first = {n: getattr(ch, n).clone() for n in ("dx", "dW1", "dW2", "dWg")}
    ch.backward()                      # the buffers now hold chunk 0, not the last one
    torch.cuda.synchronize()
    for n, v in first.items():
        assert torch.equal(v, getattr(ch, n)), n


def test_chunking_bounds_the_activation_memory():
    cfg = small_variant("moe_s_like", T=8192, d=1024, f=4096, E=8, k=2)
    banner("chunked memory", cfg.short())
    t = device.gen_all(cfg)
    args = (cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act, device.torch_dtype(cfg), cfg.renorm)
    peaks = []
    for make in (lambda: M.MoELayer(*args), lambda: M.ChunkedMoELayer(*args, chunk_tokens=1024)):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        layer = run(make(), t)
        peaks.append(torch.cuda.max_memory_allocated() - base)
        del layer
    # per-row activations: x_perm, h_save, a_save, d_out_perm, dx_perm and dH
    # for T*k rows against one 1024-token chunk (out_perm stays whole)
    assert peaks[1] < 0.5 * peaks[0], peaks


@pytest.mark.parametrize("counts", [[300, 0, 17, 513, 64], [9000, 0, 20000, 64]])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_accumulate_entry_point_and_gemm1_only(act, dt, counts):
    """moe_expert_ffn_bwd_accumulate adds to what dW holds (old + new in fp32,
    one rounding; a segment split over its rows adds its chunks after the old
    value); R = 0 leaves dW untouched; moe_expert_ffn_fwd with out_perm =
    NULL writes the same saved state as the full call."""
    from moe_inputs import stage
    from _gpu import dev, dev_i32
    banner("accumulate", act, dt, counts)
    E, d, f = len(counts), 128, 192
    offsets = stage.counts_to_offsets(counts)
    R = int(offsets[-1])
    xp = stage.normal(51, (R, d), 1.0, dt)
    W1 = stage.normal(52, (E, d, f), 1 / np.sqrt(d), dt)
    W2 = stage.normal(53, (E, f, d), 1 / np.sqrt(f), dt)
    W3 = stage.normal(54, (E, d, f), 1 / np.sqrt(d), dt) if act == "swiglu" else None
    dO = stage.normal(55, (R, d), 1.0, dt)
    base1 = stage.normal(56, (E, d, f), 0.1, dt)
    base2 = stage.normal(57, (E, f, d), 0.1, dt)
    g = dict(xp=dev(xp, dt), off=dev_i32(offsets), W1=dev(W1, dt), W2=dev(W2, dt),
             W3=dev(W3, dt) if W3 is not None else None, dO=dev(dO, dt))
    h, a, o = M.moe_expert_ffn_fwd(g["xp"], g["off"], g["W1"], g["W2"], g["W3"], act)
    h1, a1 = torch.empty_like(h), torch.empty_like(a)
    L = M.load()
    from mixture_experts_layer_permute_amd import _lib
    ws = torch.empty(max(L.moe_ffn_workspace_bytes(R, E, d, f, 1 if act == "swiglu" else 0,
                                                   1 if dt == "bf16" else 0, 0), 1),
                     dtype=torch.uint8, device="cuda")
    p = lambda t: None if t is None else t.data_ptr()
    _lib.check(L.moe_expert_ffn_fwd(p(g["xp"]), p(g["off"]), R, E, d, f,
                                    1 if act == "swiglu" else 0, 1 if dt == "bf16" else 0,
                                    p(g["W1"]), p(g["W3"]), None, p(h1), p(a1), None, p(ws),
                                    ws.numel(), torch.cuda.current_stream().cuda_stream),
               "moe_expert_ffn_fwd (GEMM1 only)")
    torch.cuda.synchronize()
    assert torch.equal(h, h1) and torch.equal(a, a1)
    # accumulate onto base values
    dW1 = dev(base1, dt)
    dW2 = dev(base2, dt)
    dW3 = dev(base1, dt) if act == "swiglu" else None
    bw = M.moe_expert_ffn_bwd(g["dO"], g["xp"], h, a, g["off"], g["W1"], g["W2"], g["W3"], act)
    ws_b = torch.empty(max(L.moe_ffn_workspace_bytes(R, E, d, f, 1 if act == "swiglu" else 0,
                                                     1 if dt == "bf16" else 0, 1), 1),
                       dtype=torch.uint8, device="cuda")
    dxp = torch.empty_like(g["dO"])
    _lib.check(L.moe_expert_ffn_bwd_accumulate(
        p(g["dO"]), p(g["xp"]), p(h), p(a), p(g["off"]), R, E, d, f,
        1 if act == "swiglu" else 0, 1 if dt == "bf16" else 0, p(g["W1"]), p(g["W3"]),
        p(g["W2"]), p(dxp), p(dW1), p(dW3), p(dW2), p(ws_b), ws_b.numel(),
        torch.cuda.current_stream().cuda_stream), "moe_expert_ffn_bwd_accumulate")
    torch.cuda.synchronize()
    assert torch.equal(dxp, bw[0]), "dx_perm"
    want1 = base1.astype(np.float64) + host(bw[1])
    want2 = base2.astype(np.float64) + host(bw[3])
    assert_close(dW1, want1, dt, "dW1 += ")
    assert_close(dW2, want2, dt, "dW2 += ")
    if act == "swiglu":
        assert_close(dW3, base1.astype(np.float64) + host(bw[2]), dt, "dW3 += ")
    # an empty expert adds nothing: its rows of dW keep the old bits exactly
    assert torch.equal(dW1[1], dev(base1, dt)[1]) and torch.equal(dW2[1], dev(base2, dt)[1])
    # R = 0: dW unchanged
    before = dW1.clone()
    zero_off = dev_i32(np.zeros(E + 1, np.int32))
    _lib.check(L.moe_expert_ffn_bwd_accumulate(
        None, None, None, None, p(zero_off), 0, E, d, f, 1 if act == "swiglu" else 0,
        1 if dt == "bf16" else 0, p(g["W1"]), p(g["W3"]), p(g["W2"]), None, p(dW1), p(dW3),
        p(dW2), p(ws_b), ws_b.numel(), torch.cuda.current_stream().cuda_stream),
        "moe_expert_ffn_bwd_accumulate R=0")
    torch.cuda.synchronize()
    assert torch.equal(before, dW1)


def test_chunked_back_to_back_steps():
    """Six steps issued with no host synchronisation, re-bound each time to
    one of two input sets (x and dy negated/halved: other routing, other
    gradients): the last step equals one step of a fresh layer on the same
    inputs, bit for bit (dW accumulation across chunks restarts every step,
    and a re-bind drops the resident chunk)."""
    cfg = small_variant("moe_s_like", T=1000, d=256, f=512, E=8, k=2)
    banner("chunked back-to-back", cfg.short())
    t = device.gen_all(cfg)
    tb = dict(t)
    tb["x"] = (-t["x"]).contiguous()
    tb["dy"] = (t["dy"] * -0.5).contiguous()
    args = (cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act, device.torch_dtype(cfg), cfg.renorm)
    ref = run(M.ChunkedMoELayer(*args, chunk_tokens=256), tb)
    ch = M.ChunkedMoELayer(*args, chunk_tokens=256)
    for i in range(6):
        u = tb if i % 2 else t
        ch.bind(u["x"], u["Wg"], u["W1"], u["W2"], u["W3"], u["bias"], u["dy"])
        ch.step()
    torch.cuda.synchronize()
    for n in SAME + ["dW1", "dW2"]:
        assert torch.equal(getattr(ch, n), getattr(ref, n)), n


def test_chunked_many_chunks_at_full_width():
    """Sixteen chunks of the skewed workload at its full sizes (T 16384,
    d 2048, f 8192, 16 experts): every chunk adds one bf16 rounding of the
    running weight gradient.  The four seeded experts and the heaviest one
    are compared with the oracle on every entry of dW1 and dW2; y, dx and dWg
    must equal the whole layer's bit for bit."""
    cfg = small_variant("skewed_zipf1.2")
    C = 1024
    banner("chunked 16 chunks", cfg.short(), C)
    t = device.gen_all(cfg)
    args = (cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act, device.torch_dtype(cfg), cfg.renorm)
    ch = run(M.ChunkedMoELayer(*args, chunk_tokens=C), t)
    whole = run(M.MoELayer(*args), t)
    for n in SAME:
        assert torch.equal(getattr(whole, n), getattr(ch, n)), n
    counts = whole.counts.cpu().numpy()
    offsets = whole.offsets.cpu().numpy()
    src = whole.src.cpu().numpy()
    dest = whole.dest.cpu().numpy()
    w = whole.topk_w.cpu().numpy().astype(np.float64)
    del whole
    torch.cuda.empty_cache()
    x, dy = rng.gen(cfg, "x"), rng.gen(cfg, "dy")
    wrow = np.empty(cfg.R)
    wrow[dest.reshape(-1)] = w.reshape(-1)
    checked = [int(e) for e in rng.seeded_experts(cfg)]
    heavy = int(np.argmax(counts))
    checked += [heavy] if heavy not in checked else []
    for e in checked:
        a, b = int(offsets[e]), int(offsets[e + 1])
        banner("expert", e, "rows", b - a)
        if b == a:
            assert float(ch.dW1[e].abs().max()) == 0.0
            continue
        W1e, W2e = rng.gen(cfg, "W1", e), rng.gen(cfg, "W2", e)
        xs = x[src[a:b]]
        dO = wrow[a:b, None] * dy[src[a:b]]
        _, dW1, _, dW2 = oracle.ffn_bwd_segment(dO, xs, W1e, W2e, None, cfg.act)
        assert_close(host(ch.dW1[e]), dW1, cfg.dtype, "dW1[e=%d]" % e)
        assert_close(host(ch.dW2[e]), dW2, cfg.dtype, "dW2[e=%d]" % e)
