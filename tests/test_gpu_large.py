"""Parity at the full sizes of the three large workloads (16-expert skewed,
64-expert skewed, 128-expert SwiGLU long-context chunk), in the launch
configuration the benchmark uses.

* The whole layer runs on the GPU once.  Routing is compared in full and bit
  for bit (logits, top-k, counts, offsets, dest, src); the gate weights to
  fp32 precision.
* Four seeded experts plus the heaviest one (the ragged segments the skewed
  workloads exist for) against the oracle on the host copy of the inputs.
  On the 16- and 64-expert workloads every row of H, A, out_perm,
  d_out_perm and dx_perm and the whole dW1 / dW2 of those experts are
  compared.  On the long-context chunk (57 K rows in its heaviest expert)
  48 sampled rows per expert, and one hidden unit in every 256-wide column
  tile of dW1 / dW3 (all d rows) and row tile of dW2 (all d columns).  An
  expert with no rows must have dW exactly 0.
* The row kernels (combine, combine backward, unpermute, gate backward) are
  fed independent seeded tensors of the full sizes, and their outputs are
  compared on sampled tokens (dWg in full).
"""
import time

import numpy as np
import pytest
import torch

import mixture_experts_layer_permute_amd as M
import oracle
from moe_inputs import CONFIGS, device, rng

from _gpu import (assert_close, assert_equal_i, banner, dev, dev_i32, host,
                  needs_gpu, saved_state)

pytestmark = [pytest.mark.gpu, needs_gpu]

LARGE = ["skewed_zipf1.2", "many_expert_zipf1.0", "long_ctx_swiglu"]
# workloads whose checked experts are compared on every row and every dW entry
FULL = {"skewed_zipf1.2", "many_expert_zipf1.0"}
TILE = 256          # column tile of the dW products


def checked_experts(cfg, counts):
    """The four seeded experts, then the heaviest (lowest index on a tie)."""
    out = [int(e) for e in rng.seeded_experts(cfg)]
    heavy = int(np.argmax(counts))
    return out + ([heavy] if heavy not in out else [])


def tile_units(g, f):
    """One hidden unit in every TILE-wide block of [0, f)."""
    return np.array([lo + int(g.integers(min(TILE, f - lo))) for lo in range(0, f, TILE)])


def take_rows(t, rows):
    idx = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=t.device)
    return host(t.index_select(0, idx))


def sample(g, lo, hi, n):
    """Up to n distinct sorted indices in [lo, hi), always with both ends."""
    if hi - lo <= n:
        return np.arange(lo, hi)
    mid = g.choice(np.arange(lo + 1, hi - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[lo, hi - 1], mid]))


def host_routing(cfg):
    x = rng.gen(cfg, "x")
    Wg = rng.gen(cfg, "Wg")
    bias = rng.logit_bias(cfg)
    logits = oracle.gate_logits(x, Wg, bias)
    idx = oracle.topk_select(logits, cfg.k)
    w = oracle.gate_weights(logits, idx, cfg.renorm)
    counts, offsets, dest, src = oracle.permute(idx, cfg.E)
    return dict(x=x, Wg=Wg, bias=bias, logits=logits, idx=idx, w=w,
                counts=counts, offsets=offsets, dest=dest, src=src)


@pytest.mark.parametrize("name", LARGE)
def test_large_layer(name):
    cfg = CONFIGS[name]
    dt = cfg.dtype
    banner("large layer", name, cfg.short())
    t0 = time.time()
    t = device.gen_all(cfg)
    layer = M.MoELayer(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act,
                       device.torch_dtype(cfg), cfg.renorm)
    layer.bind(t["x"], t["Wg"], t["W1"], t["W2"], t["W3"], t["bias"], t["dy"])
    layer.step()
    torch.cuda.synchronize()
    banner("gpu step done %.1fs" % (time.time() - t0))

    h = host_routing(cfg)
    banner("host routing done %.1fs" % (time.time() - t0))
    assert_equal_i(layer.logits.cpu().numpy().view(np.uint32),
                   h["logits"].view(np.uint32), "logits")
    assert_equal_i(layer.topk_idx, h["idx"], "topk_idx")
    assert_close(layer.topk_w, h["w"], "f32", "topk_w")
    for n in ("counts", "offsets", "dest", "src"):
        assert_equal_i(getattr(layer, n), h[n], n)
    g = np.random.default_rng(cfg.seed + 7)
    rows = np.sort(g.choice(cfg.R, size=1024, replace=False))
    assert np.array_equal(take_rows(layer.x_perm, rows), h["x"][h["src"][rows]])

    # every expert that received no token has exactly zero weight gradients
    for e in np.flatnonzero(h["counts"] == 0):
        assert float(layer.dW1[e].abs().max()) == 0.0, "dW1 of empty expert %d" % e
        assert float(layer.dW2[e].abs().max()) == 0.0, "dW2 of empty expert %d" % e
    dy = rng.gen(cfg, "dy")
    wrow = np.empty(cfg.R)
    wrow[h["dest"].reshape(-1)] = h["w"].reshape(-1)      # gate weight of each row
    f = cfg.f
    full = name in FULL
    for e in checked_experts(cfg, h["counts"]):
        a, b = int(h["offsets"][e]), int(h["offsets"][e + 1])
        banner("expert", int(e), "rows", b - a, "full" if full else "sampled",
               "%.1fs" % (time.time() - t0))
        if b == a:
            assert float(layer.dW1[e].abs().max()) == 0.0
            assert float(layer.dW2[e].abs().max()) == 0.0
            if cfg.swiglu:
                assert float(layer.dW3[e].abs().max()) == 0.0
            continue
        W1e = rng.gen(cfg, "W1", int(e))
        W2e = rng.gen(cfg, "W2", int(e))
        W3e = rng.gen(cfg, "W3", int(e)) if cfg.swiglu else None
        r = np.arange(a, b) if full else sample(g, a, b, 48)
        xr = h["x"][h["src"][r]]
        H, H3, A, O = oracle.ffn_fwd_segment(xr, W1e, W2e, W3e, cfg.act)
        hs = take_rows(layer.h_save, r)
        want = saved_state(cfg.act, H, H3)
        if cfg.swiglu:
            assert_close(hs[:, :f], want[:, :f], dt, "H3 SiLU'(H1)[e=%d]" % e)
            assert_close(hs[:, f:], want[:, f:], dt, "SiLU(H1)[e=%d]" % e)
        else:
            assert_close(hs, want, dt, "GeLU'(H)[e=%d]" % e)
        del hs, want
        assert_close(take_rows(layer.a_save, r), A, dt, "A[e=%d]" % e)
        assert_close(take_rows(layer.out_perm, r), O, dt, "out_perm[e=%d]" % e)
        # backward: dO of every row of the segment, from the gate and dy
        dO_seg = wrow[a:b, None] * dy[h["src"][a:b]]
        assert_close(take_rows(layer.d_out_perm, r), dO_seg[r - a], dt,
                     "d_out_perm[e=%d]" % e)
        saved = (H, H3, A)
        del O
        if full:
            # every row of dx_perm and every entry of dW1 / dW2
            dX, dW1, _, dW2 = oracle.ffn_bwd_segment(dO_seg, xr, W1e, W2e, W3e,
                                                     cfg.act, saved=saved)
            assert_close(take_rows(layer.dx_perm, r), dX, dt, "dx_perm[e=%d]" % e)
            assert_close(host(layer.dW1[e]), dW1, dt, "dW1[e=%d]" % e)
            assert_close(host(layer.dW2[e]), dW2, dt, "dW2[e=%d]" % e)
            del dX, dW1, dW2, saved, H, H3, A
            continue
        dXr = oracle.ffn_bwd_segment(dO_seg[r - a], xr, W1e, W2e, W3e, cfg.act,
                                     saved=saved)[0]
        assert_close(take_rows(layer.dx_perm, r), dXr, dt, "dx_perm[e=%d]" % e)
        # one hidden unit per column tile of dW1 / dW3 and row tile of dW2
        cols = tile_units(g, f)
        c1, c3, c2 = oracle.ffn_bwd_columns(dO_seg, h["x"][h["src"][a:b]], W1e, W2e,
                                           W3e, cfg.act, cols)
        ci = torch.as_tensor(cols, device="cuda")
        assert_close(host(layer.dW1[e].index_select(1, ci)), c1, dt, "dW1[e=%d]" % e)
        assert_close(host(layer.dW2[e].index_select(0, ci)), c2, dt, "dW2[e=%d]" % e)
        if cfg.swiglu:
            assert_close(host(layer.dW3[e].index_select(1, ci)), c3, dt,
                         "dW3[e=%d]" % e)
    banner("done %.1fs" % (time.time() - t0))
    del layer, t
    torch.cuda.empty_cache()


def gen_rows_key(key, rows, ncol, dtype):
    out = np.empty((len(rows), ncol), dtype=np.float32)
    for i, r in enumerate(rows):
        out[i] = rng.normal_f32(key, int(r) * ncol, ncol, 1.0)
    return rng.round_to_dtype(out, dtype)


@pytest.mark.parametrize("name", LARGE)
def test_large_row_kernels(name):
    cfg = CONFIGS[name]
    dt = cfg.dtype
    tdt = device.torch_dtype(cfg)
    banner("large row kernels", name)
    t0 = time.time()
    h = host_routing(cfg)
    T, k, d, R, E = cfg.T, cfg.k, cfg.d, cfg.R, cfg.E
    g_dest = dev_i32(h["dest"])
    g_w = dev(h["w"].astype(np.float32))
    keys = {n: rng.stream_key(cfg.seed + 1000, i) for i, n in
            enumerate(("out", "dxp", "dw", "dx0"))}
    out_perm = device.fill(torch.empty(R, d, dtype=tdt, device="cuda"), keys["out"], 1.0)
    dy_g = device.gen(cfg, "dy")
    y = M.moe_combine(out_perm, g_dest, g_w)
    d_out, dw = M.moe_combine_bwd(dy_g, out_perm, g_dest, g_w)
    dxp = device.fill(torch.empty(R, d, dtype=tdt, device="cuda"), keys["dxp"], 1.0)
    dx = M.moe_unpermute_grad(dxp, g_dest)
    dwr = device.fill(torch.empty(T, k, dtype=torch.float32, device="cuda"),
                      keys["dw"], 1.0)
    dx0 = device.fill(torch.empty(T, d, dtype=tdt, device="cuda"), keys["dx0"], 1.0)
    dWg = M.moe_gate_topk_bwd(device.gen(cfg, "x"), device.gen(cfg, "Wg"),
                              dev(h["logits"]), g_dest.new_tensor(h["idx"]), g_w,
                              dwr, dx0, cfg.renorm)
    torch.cuda.synchronize()
    banner("gpu done %.1fs" % (time.time() - t0))

    g = np.random.default_rng(cfg.seed + 11)
    toks = np.sort(g.choice(T, size=256, replace=False))
    dest_t = h["dest"][toks]                               # [n, k]
    rows = dest_t.reshape(-1)
    o_rows = gen_rows_key(keys["out"], rows, d, dt).reshape(len(toks), k, d)
    wt = h["w"][toks]
    assert_close(take_rows(y, toks), (wt[:, :, None] * o_rows).sum(1), dt, "y")
    dy = rng.gen_rows(cfg, "dy", toks)
    assert_close(take_rows(d_out, rows).reshape(len(toks), k, d),
                 wt[:, :, None] * dy[:, None, :], dt, "d_out_perm")
    assert_close(host(dw)[toks], np.einsum("nkd,nd->nk", o_rows, dy), dt, "d_topk_w")
    x_rows = gen_rows_key(keys["dxp"], rows, d, dt).reshape(len(toks), k, d)
    assert_close(take_rows(dx, toks), x_rows.sum(1), dt, "dx (unpermute)")
    # gate backward: dWg in full, dx rows sampled
    dw_h = rng.normal_f32(keys["dw"], 0, T * k, 1.0).reshape(T, k)
    dl = oracle.gate_logits_grad(h["logits"], h["idx"], h["w"], dw_h, cfg.renorm)
    dWg_ref = np.zeros((d, E))
    for lo in range(0, T, 8192):
        dWg_ref += h["x"][lo:lo + 8192].astype(np.float64).T @ dl[lo:lo + 8192]
    if k > 1 or cfg.renorm == 0:
        assert_close(dWg, dWg_ref, dt, "dWg")
    dx0_rows = gen_rows_key(keys["dx0"], toks, d, dt)
    ref_dx = dx0_rows + dl[toks] @ h["Wg"].astype(np.float64).T
    assert_close(take_rows(dx0, toks), ref_dx, dt, "dx += dl Wg^T")
    banner("done %.1fs" % (time.time() - t0))
