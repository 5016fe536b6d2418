"""Edge cases of the whole layer, bit-for-bit determinism, and randomized
gate/permute cases, all against the oracle on the host copy of the inputs.

* E = 1: the layer reduces to one MLP applied to every token.
* Every token routed to one expert (a large logit bias on it).
* k = E: every token visits every expert.
* T = 1 and a token count that is no multiple of any tile.
* About a thousand experts of a few rows each, some of them empty.
* Two runs of the same step give identical bits (no float atomics, fixed
  reduction orders), with side-stream overlap on.
* Randomized (T, d, E, k, skew) for the gate and the permute, bit-exact
  routing (a fixed number of seeded draws).
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_permute_amd as M
import oracle
from moe_inputs import CONFIGS, device, rng, small_variant, stage

from _gpu import (assert_close, assert_equal_i, banner, dev, dev_i32, host, host_i,
                  needs_gpu, saved_state)

pytestmark = [pytest.mark.gpu, needs_gpu]


def layer_case(cfg, bias=None):
    """Run the layer on the workload's seeded inputs (bias overrides the
    workload's own) and the oracle on their host copy; compare everything."""
    t = device.gen_all(cfg)
    if bias is not None:
        t["bias"] = torch.from_numpy(bias).cuda()
    layer = M.MoELayer(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act,
                       device.torch_dtype(cfg), cfg.renorm)
    layer.bind(t["x"], t["Wg"], t["W1"], t["W2"], t["W3"], t["bias"], t["dy"])
    layer.step()
    torch.cuda.synchronize()
    x, Wg, dy = (rng.gen(cfg, n) for n in ("x", "Wg", "dy"))
    W1, W2 = rng.gen_experts(cfg, "W1"), rng.gen_experts(cfg, "W2")
    W3 = rng.gen_experts(cfg, "W3") if cfg.swiglu else None
    b = bias if bias is not None else rng.logit_bias(cfg)
    fw = oracle.layer_forward(x, Wg, W1, W2, W3, k=cfg.k, act=cfg.act, bias=b,
                              renorm=cfg.renorm)
    gr = oracle.layer_backward(fw, dy, x, Wg, W1, W2, W3, act=cfg.act, renorm=cfg.renorm)
    dt = cfg.dtype
    assert_equal_i(layer.logits.cpu().numpy().view(np.uint32),
                   fw["logits"].view(np.uint32), "logits")
    assert_equal_i(layer.topk_idx, fw["idx"], "topk_idx")
    for n in ("counts", "offsets", "dest", "src"):
        assert_equal_i(getattr(layer, n), fw[n], n)
    assert_close(layer.topk_w, fw["w"], "f32", "topk_w")
    assert_close(layer.h_save, saved_state(cfg.act, fw["H"], fw.get("H3")), dt, "saved")
    assert_close(layer.a_save, fw["A"], dt, "A")
    assert_close(layer.y, fw["y"], dt, "y")
    assert_close(layer.dx_perm, gr["dx_perm"], dt, "dx_perm")
    assert_close(layer.dW1, gr["dW1"], dt, "dW1")
    assert_close(layer.dW2, gr["dW2"], dt, "dW2")
    if cfg.swiglu:
        assert_close(layer.dW3, gr["dW3"], dt, "dW3")
    assert_close(layer.dx, gr["dx"], dt, "dx")
    if np.abs(gr["dWg"]).max() > 0:
        assert_close(layer.dWg, gr["dWg"], dt, "dWg")
    else:       # top-1 with renormalised weights: the gate gets no gradient
        assert float(layer.dWg.abs().max()) == 0.0
    return layer, fw


def small(name="moe_s_like", **kw):
    base = dict(T=300, d=128, f=256, E=8, k=2, zipf_s=None, alpha=0.0)
    base.update(kw)
    return small_variant(name, **base)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_one_expert_is_an_mlp(dt):
    cfg = small(E=1, k=1, dtype=dt)
    banner("edge E=1", dt)
    layer, fw = layer_case(cfg)
    assert int(layer.counts[0]) == cfg.T
    # with one expert the layer is y = GeLU(x W1) W2 for every token
    x = rng.gen(cfg, "x")
    W1, W2 = rng.gen(cfg, "W1", 0), rng.gen(cfg, "W2", 0)
    mlp = oracle.gelu(x.astype(np.float64) @ W1) @ W2
    assert_close(layer.y, mlp, dt, "y = MLP(x)")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_all_tokens_to_one_expert(dt):
    cfg = small(E=8, k=1, T=517, dtype=dt)
    bias = np.zeros(cfg.E, np.float32)
    bias[5] = 1000.0                    # every token's top-1 is expert 5
    banner("edge all to one", dt)
    layer, _ = layer_case(cfg, bias)
    counts = layer.counts.cpu().numpy()
    assert counts[5] == cfg.T and counts.sum() == cfg.T
    for e in range(cfg.E):              # the other experts get exact zero gradients
        if e != 5:
            assert float(layer.dW1[e].abs().max()) == 0.0
            assert float(layer.dW2[e].abs().max()) == 0.0


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_k_equals_e(act):
    cfg = small("long_ctx_swiglu" if act == "swiglu" else "moe_s_like", E=4, k=4, T=203,
                act=act, dtype="bf16")
    banner("edge k=E", act)
    layer, _ = layer_case(cfg)
    assert np.all(layer.counts.cpu().numpy() == cfg.T)


@pytest.mark.parametrize("dt,zipf", [("bf16", 1.0), ("f32", None)])
def test_many_small_experts(dt, zipf):
    """About a thousand experts of a few rows each, some empty: the tile plan's
    block scans over its 1024 threads, a partial tile for almost every
    expert, and exact zero weight gradients for the empty ones."""
    cfg = small(E=1000, k=4, T=1500, d=64, f=128, dtype=dt, zipf_s=zipf)
    banner("edge many small experts", dt, zipf)
    layer, _ = layer_case(cfg)
    counts = layer.counts.cpu().numpy()
    assert counts.sum() == cfg.T * cfg.k and (counts == 0).any()
    for e in np.flatnonzero(counts == 0)[:50]:
        assert float(layer.dW1[e].abs().max()) == 0.0
        assert float(layer.dW2[e].abs().max()) == 0.0


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_empty_input_through_every_entry_point(dt):
    """T = 0 (so R = 0) through the layer's eight calls: every call succeeds,
    counts and offsets are zeros, and the weight gradients that the calls
    still write (dW1, dW2 and dWg) are exact zeros, over buffers that held
    other values."""
    E, k, d, f = 8, 2, 64, 128
    banner("edge T=0", dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    x = torch.empty(0, d, dtype=tdt, device="cuda")
    Wg = torch.randn(d, E, device="cuda").to(tdt)
    logits, idx, w = M.moe_gate_topk(x, Wg, k)
    counts, offsets, dest, src, xp = M.moe_permute(idx, x, E)
    W1 = torch.randn(E, d, f, device="cuda").to(tdt)
    W2 = torch.randn(E, f, d, device="cuda").to(tdt)
    h, a, o = M.moe_expert_ffn_fwd(xp, offsets, W1, W2, None, "gelu")
    y = M.moe_combine(o, dest, w)
    dy = torch.empty(0, d, dtype=tdt, device="cuda")
    d_out, dw = M.moe_combine_bwd(dy, o, dest, w)
    dW1, dW2 = torch.ones_like(W1), torch.ones_like(W2)
    dxp = torch.empty(0, d, dtype=tdt, device="cuda")
    M.moe_expert_ffn_bwd(d_out, xp, h, a, offsets, W1, W2, None, "gelu",
                         out=(dxp, dW1, None, dW2))
    dx = M.moe_unpermute_grad(dxp, dest)
    dWg = M.moe_gate_topk_bwd(x, Wg, logits, idx, w, dw, dx, dWg=torch.ones_like(Wg))
    torch.cuda.synchronize()
    assert y.shape == (0, d) and dx.shape == (0, d)
    assert int(counts.abs().sum()) == 0 and int(offsets.abs().sum()) == 0
    for n, g in (("dW1", dW1), ("dW2", dW2), ("dWg", dWg)):
        assert float(g.float().abs().max()) == 0.0, n


@pytest.mark.parametrize("T", [1, 17, 1031])
def test_token_counts(T):
    cfg = small(T=T, E=6, k=2, dtype="bf16")
    banner("edge T", T)
    layer_case(cfg)


def test_step_is_deterministic():
    """Two runs of the same step, side-stream overlap on, give identical bits."""
    cfg = CONFIGS["many_expert_zipf1.0"]
    cfg = small_variant(cfg.name, T=4096)
    banner("determinism", cfg.short())
    t = device.gen_all(cfg)
    outs = []
    for _ in range(2):
        layer = M.MoELayer(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act,
                           device.torch_dtype(cfg), cfg.renorm)
        layer.bind(t["x"], t["Wg"], t["W1"], t["W2"], t["W3"], t["bias"], t["dy"])
        layer.step()
        layer.step()
        torch.cuda.synchronize()
        outs.append({n: getattr(layer, n).clone() for n in
                     ("logits", "topk_w", "x_perm", "h_save", "a_save", "out_perm", "y",
                      "d_out_perm", "d_topk_w", "dx_perm", "dW1", "dW2", "dx", "dWg")})
        del layer
    for n in outs[0]:
        assert torch.equal(outs[0][n], outs[1][n]), n


# ------------------------------------------------------- randomized cases

def _draws(n, seed):
    g = np.random.default_rng(seed)
    for _ in range(n):
        E = int(g.integers(1, 80))
        k = int(g.integers(1, min(E, 8) + 1))
        T = int(g.integers(1, 400))
        d = int(g.choice([8, 16, 64, 136]))
        skew = float(g.choice([0.0, 0.5, 0.95]))
        yield T, d, E, k, skew, int(g.integers(0, 2**31))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_random_gate_and_permute(dt):
    for T, d, E, k, skew, seed in _draws(24, 4242 if dt == "bf16" else 4343):
        banner("random", T, d, E, k, skew, dt)
        x = stage.normal(seed, (T, d), 1.0, dt)
        Wg = stage.normal(seed + 1, (d, E), 1.0 / np.sqrt(d), dt)
        bias = np.zeros(E, np.float32)
        if skew > 0:                       # one hot expert takes most first choices
            bias[seed % E] = 4.0 * skew
        lg, idx, w = M.moe_gate_topk(dev(x, dt), dev(Wg, dt), k, dev(bias), 1)
        ref_l = oracle.gate_logits(x, Wg, bias)
        ref_i = oracle.topk_select(ref_l, k)
        assert_equal_i(lg.cpu().numpy().view(np.uint32), ref_l.view(np.uint32), "logits")
        assert_equal_i(idx, ref_i, "topk_idx")
        assert_close(w, oracle.gate_weights(ref_l, ref_i, 1), "f32", "topk_w")
        counts, offsets, dest, src, xp = M.moe_permute(idx, dev(x, dt), E)
        torch.cuda.synchronize()
        rc, ro, rd, rs = oracle.permute(ref_i, E)
        assert_equal_i(counts, rc, "counts")
        assert_equal_i(offsets, ro, "offsets")
        assert_equal_i(dest, rd, "dest")
        assert_equal_i(src, rs, "src")
        got = host(xp)
        assert np.array_equal(got, oracle.dispatch_rows(x, rs)), "x_perm"


def test_permute_skips_invalid_expert_ids():
    """Pairs whose expert id lies outside [0,E) are left out of counts and
    offsets and get dest = -1; the valid pairs keep their stable order."""
    g = np.random.default_rng(99)
    T, k, E, d = 300, 3, 7, 64
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    bad = g.choice(T * k, size=11, replace=False)
    flat = idx.reshape(-1)
    flat[bad[:6]] = E                      # one past the last expert
    flat[bad[6:]] = -1
    x = stage.normal(5, (T, d), 1.0, "bf16")
    banner("permute with invalid ids", T, k, E)
    counts, offsets, dest, src, xp = M.moe_permute(dev_i32(idx), dev(x, "bf16"), E)
    torch.cuda.synchronize()
    valid = (flat >= 0) & (flat < E)
    nv = int(valid.sum())
    order = np.argsort(np.where(valid, flat, E), kind="stable")
    want_dest = np.full(T * k, -1, np.int64)
    want_dest[order[:nv]] = np.arange(nv)
    want_counts = np.bincount(flat[valid], minlength=E)
    assert_equal_i(counts, want_counts, "counts")
    assert_equal_i(offsets, np.concatenate([[0], np.cumsum(want_counts)]), "offsets")
    assert_equal_i(dest, want_dest.reshape(T, k), "dest")
    assert_equal_i(host_i(src)[:nv], order[:nv] // k, "src")
    assert np.array_equal(host(xp[:nv]), x.astype(np.float64)[order[:nv] // k]), "x_perm"


@pytest.mark.parametrize("k", [3, 8, 11])
def test_row_kernels_skip_invalid_slots(k):
    """dest = -1 (a pair whose expert id was invalid) contributes nothing: the
    combine sums the other slots, its backward writes no row and a zero gate
    gradient for the slot, the unpermute adds nothing.  The oracle sees the
    same slots pointed at an extra all-zero row with weight 0."""
    g = np.random.default_rng(7 + k)
    T, d, E = 211, 128, 16
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, _, dest, _ = oracle.permute(idx, E)
    bad = g.choice(T * k, size=T // 3, replace=False)
    R = T * k
    gdest = dest.reshape(-1).copy()
    gdest[bad] = -1
    odest = dest.reshape(-1).copy()
    odest[bad] = R                               # the extra zero row
    gdest, odest = gdest.reshape(T, k), odest.reshape(T, k)
    out = stage.normal(71, (R, d), 1.0, "bf16")
    dxp = stage.normal(72, (R, d), 1.0, "bf16")
    dy = stage.normal(73, (T, d), 1.0, "bf16")
    w = np.abs(stage.normal(74, (T, k), 1.0, "f32"))
    ow = w.copy()
    ow.reshape(-1)[bad] = 0.0
    out1 = np.concatenate([out, np.zeros((1, d), out.dtype)])
    dxp1 = np.concatenate([dxp, np.zeros((1, d), dxp.dtype)])
    banner("row kernels with dest = -1", T, k)
    g_out, g_dest, g_w = dev(out, "bf16"), dev_i32(gdest), dev(w)
    y = M.moe_combine(g_out, g_dest, g_w)
    # rows no slot maps to are not written: start them at zero
    d_out = torch.zeros_like(g_out)
    dw = torch.empty(T, k, dtype=torch.float32, device=g_out.device)
    d_out, dw = M.moe_combine_bwd(dev(dy, "bf16"), g_out, g_dest, g_w, out=(d_out, dw))
    dx = M.moe_unpermute_grad(dev(dxp, "bf16"), g_dest)
    torch.cuda.synchronize()
    assert_close(y, oracle.combine(out1, odest, ow), "bf16", "y")
    rd_out, rdw = oracle.combine_bwd(dy, out1, odest, ow)
    assert_close(d_out, rd_out[:R], "bf16", "d_out_perm")
    dwh = dw.cpu().numpy()
    assert np.all(dwh.reshape(-1)[bad] == 0.0), "d_topk_w of skipped slots"
    assert_close(dw, rdw, "bf16", "d_topk_w")
    assert_close(dx, oracle.unpermute_grad(dxp1, odest), "bf16", "dx")

