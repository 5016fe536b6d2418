"""Each C entry point against the oracle on small seeded inputs that span
several tiles and a ragged tail.  Integers bit-exact; floats within
max|err| <= 2e-2 max|ref| (bf16) or 1e-5 max|ref| (fp32)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_permute_amd as M
import oracle
from moe_inputs import stage

from _gpu import (TDT, assert_close, assert_equal_i, banner, dev, dev_i32, host,
                  needs_gpu, saved_state)

pytestmark = [pytest.mark.gpu, needs_gpu]


# ----------------------------------------------------------------- gate

GATE_CASES = [  # T, d, E, k, bias, renorm
    (1000, 128, 16, 2, True, 1), (517, 96, 8, 2, False, 1),
    (300, 64, 4, 1, False, 1), (200, 64, 100, 3, True, 1),
    (64, 128, 128, 8, True, 0), (33, 64, 5, 5, False, 1),
    (40, 64, 1, 1, False, 1), (1, 64, 64, 4, True, 1), (16, 72, 1024, 3, False, 1),
    # grids of at least two blocks per compute unit take the logits kernel's
    # 2-token x 8-expert form: ragged tokens and experts, a partial feature
    # chunk (136 = 2 x 64 + 8), and the threshold itself (512 blocks)
    (20000, 136, 100, 3, True, 1), (32768, 64, 64, 2, False, 1),
    # and with 9-16 experts the 2-expert form
    (16384, 64, 12, 2, True, 1), (20001, 264, 16, 3, False, 1),
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", GATE_CASES)
def test_gate_topk(case, dt):
    T, d, E, k, use_bias, renorm = case
    banner("gate_topk", case, dt)
    x = stage.normal(1, (T, d), 1.0, dt)
    Wg = stage.normal(2, (d, E), 1.0 / np.sqrt(d), dt)
    bias = stage.normal(3, (E,), 1.0, "f32") if use_bias else None
    lg, idx, w = M.moe_gate_topk(dev(x, dt), dev(Wg, dt), k,
                                 dev(bias) if use_bias else None, renorm)
    torch.cuda.synchronize()
    ref_l = oracle.gate_logits(x, Wg, bias)
    ref_i = oracle.topk_select(ref_l, k)
    assert_equal_i(lg.cpu().numpy().view(np.uint32), ref_l.view(np.uint32), "logits")
    assert_equal_i(idx, ref_i, "topk_idx")
    assert_close(w, oracle.gate_weights(ref_l, ref_i, renorm), "f32", "topk_w")


def test_gate_ties_lower_index_first():
    banner("gate ties")
    T, d, E, k = 8, 64, 6, 3
    x = np.zeros((T, d), np.float32)
    Wg = np.zeros((d, E), np.float32)          # every logit 0: all tie
    bias = np.array([0, 1, 0, 1, 0, 1], np.float32)
    _, idx, w = M.moe_gate_topk(dev(x), dev(Wg), k, dev(bias))
    assert_equal_i(idx, np.tile([1, 3, 5], (T, 1)), "ties")
    assert np.allclose(w.cpu().numpy(), 1 / 3, rtol=1e-6)


# -------------------------------------------------------------- permute

PERM_CASES = [  # T, E, k, hot, hot_frac, dead
    (1000, 8, 2, None, 0.0, ()), (2500, 16, 2, 3, 0.9, (7, 8, 15)),
    (777, 64, 8, 0, 0.5, tuple(range(40, 64))), (5, 4, 4, None, 0.0, ()),
    (1, 3, 1, None, 0.0, ()), (3000, 1, 1, None, 0.0, ()),
    (1500, 1024, 3, 5, 0.7, ()), (4097, 128, 8, 127, 0.95, (0, 1, 2)),
    # 64 blocks (the scatter sums the block counts itself), 65 blocks and
    # 157 blocks (through the separate scan)
    (32768, 16, 2, 4, 0.5, ()), (32769, 16, 2, 4, 0.5, (9,)),
    (20000, 64, 8, 3, 0.6, (60, 61)),
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", PERM_CASES)
def test_permute(case, dt):
    T, E, k, hot, frac, dead = case
    d = 64
    banner("permute", case, dt)
    idx = stage.routing(10 + T, T, E, k, hot, frac, dead)
    x = stage.normal(11, (T, d), 1.0, dt)
    counts, offsets, dest, src, xp = M.moe_permute(dev_i32(idx), dev(x, dt), E)
    torch.cuda.synchronize()
    rc, ro, rd, rs = oracle.permute(idx, E)
    assert_equal_i(counts, rc, "counts")
    assert_equal_i(offsets, ro, "offsets")
    assert_equal_i(dest, rd, "dest")
    assert_equal_i(src, rs, "src")
    got = xp.cpu()
    want = torch.from_numpy(oracle.dispatch_rows(x, rs)).to(TDT[dt])
    assert torch.equal(got.view(torch.int16) if dt == "bf16" else got.view(torch.int32),
                       want.view(torch.int16) if dt == "bf16" else want.view(torch.int32))


# ----------------------------------------------------------- expert FFN

FFN_CASES = [  # counts per expert, d, f
    ([300, 0, 17, 513, 1], 128, 192),
    ([600, 0, 300, 1000, 45], 512, 768),
    ([256, 256], 64, 64),
    ([0, 0, 70], 256, 320),
    ([1], 64, 128),
    # partial last tiles of every size class for the 64-row slices of the
    # split launch (64, 63, 65, 192, 1, 255, 64, ...), more partial experts
    # than one row-tile group, and one expert with 8 full tiles + 130 rows
    ([64, 63, 65, 192, 257, 511, 320, 0, 1, 700, 130, 5], 128, 256),
    ([2178], 64, 128),
    # dW split over rows: two experts above 8192 rows with one dW tile each
    # (chunks of 4096 rows, fp32 partials summed in order), beside short ones
    # (segments of 5861 rows on average: the dW products' 64-deep ring)
    ([9000, 5, 20000, 0, 300], 128, 256),
    # a split segment with 1538 rows on average (the 32-deep ring)
    ([9000, 5, 3000, 0, 300, 0, 0, 0], 128, 256),
    # 4398 rows on average, ragged ends and a partial column tile (64-deep ring)
    ([4096, 4100, 4999], 128, 192),
]


def _ffn_inputs(counts, d, f, dt, act, seed=20):
    E = len(counts)
    offsets = stage.counts_to_offsets(counts)
    R = int(offsets[-1])
    xp = stage.normal(seed, (R, d), 1.0, dt)
    W1 = stage.normal(seed + 1, (E, d, f), 1 / np.sqrt(d), dt)
    W2 = stage.normal(seed + 2, (E, f, d), 1 / np.sqrt(f), dt)
    W3 = stage.normal(seed + 3, (E, d, f), 1 / np.sqrt(d), dt) if act == "swiglu" else None
    return offsets, xp, W1, W2, W3


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("case", FFN_CASES)
def test_expert_ffn_fwd(case, act, dt):
    counts, d, f = case
    banner("ffn_fwd", case, act, dt)
    offsets, xp, W1, W2, W3 = _ffn_inputs(counts, d, f, dt, act)
    h, a, o = M.moe_expert_ffn_fwd(dev(xp, dt), dev_i32(offsets), dev(W1, dt),
                                   dev(W2, dt), dev(W3, dt) if W3 is not None else None,
                                   act)
    torch.cuda.synchronize()
    ref = oracle.expert_ffn_fwd(xp, offsets, W1, W2, W3, act)
    f_ = W1.shape[2]
    want = saved_state(act, ref["H"], ref.get("H3"))
    if act == "gelu":
        assert_close(h, want, dt, "GeLU'(H)")
    else:
        hh = host(h)
        assert_close(hh[:, :f_], want[:, :f_], dt, "H3 SiLU'(H1)")
        assert_close(hh[:, f_:], want[:, f_:], dt, "SiLU(H1)")
    assert_close(a, ref["A"], dt, "A")
    assert_close(o, ref["out"], dt, "out_perm")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("case", FFN_CASES)
def test_expert_ffn_bwd(case, act, dt):
    counts, d, f = case
    banner("ffn_bwd", case, act, dt)
    offsets, xp, W1, W2, W3 = _ffn_inputs(counts, d, f, dt, act, seed=30)
    R = int(offsets[-1])
    dO = stage.normal(35, (R, d), 1.0, dt)
    dW3_ = dev(W3, dt) if W3 is not None else None
    g_xp, g_off = dev(xp, dt), dev_i32(offsets)
    g_W1, g_W2 = dev(W1, dt), dev(W2, dt)
    h, a, _ = M.moe_expert_ffn_fwd(g_xp, g_off, g_W1, g_W2, dW3_, act)
    dxp, dW1, dW3, dW2 = M.moe_expert_ffn_bwd(dev(dO, dt), g_xp, h, a, g_off, g_W1,
                                              g_W2, dW3_, act)
    torch.cuda.synchronize()
    ref = oracle.expert_ffn_bwd(dO, xp, offsets, W1, W2, W3, act)
    E = len(counts)
    if R:
        assert_close(dxp, ref["dx_perm"], dt, "dx_perm")
    hW1, hW2 = host(dW1), host(dW2)
    for e in range(E):
        if counts[e] == 0:
            assert np.all(hW1[e] == 0) and np.all(hW2[e] == 0), "zero-load dW"
    assert_close(hW1, np.stack([ref["dW1"][e] for e in range(E)]), dt, "dW1")
    assert_close(hW2, np.stack([ref["dW2"][e] for e in range(E)]), dt, "dW2")
    if act == "swiglu":
        assert_close(dW3, np.stack([ref["dW3"][e] for e in range(E)]), dt, "dW3")


# ------------------------------------------------- combine / unpermute

ROW_CASES = [(1000, 8, 2, 128), (333, 16, 4, 64), (64, 128, 8, 512), (1, 4, 1, 64),
             (2049, 64, 2, 1024),
             # slot groups of 4 and 8 with padded slots (k = 3, 6), two and
             # three groups of 8 (k = 12, 20)
             (257, 16, 3, 192), (130, 32, 6, 320), (77, 64, 12, 256), (50, 40, 20, 128)]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", ROW_CASES)
def test_combine_and_backward(case, dt):
    T, E, k, d = case
    banner("combine", case, dt)
    idx = stage.routing(40 + T, T, E, k)
    _, _, dest, _ = oracle.permute(idx, E)
    R = T * k
    out = stage.normal(41, (R, d), 1.0, dt)
    w = np.abs(stage.normal(42, (T, k), 1.0, "f32"))
    dy = stage.normal(43, (T, d), 1.0, dt)
    g_out, g_dest, g_w = dev(out, dt), dev_i32(dest), dev(w)
    y = M.moe_combine(g_out, g_dest, g_w)
    d_out, dw = M.moe_combine_bwd(dev(dy, dt), g_out, g_dest, g_w)
    torch.cuda.synchronize()
    assert_close(y, oracle.combine(out, dest, w), dt, "y")
    rd_out, rdw = oracle.combine_bwd(dy, out, dest, w)
    assert_close(d_out, rd_out, dt, "d_out_perm")
    assert_close(dw, rdw, dt, "d_topk_w")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", ROW_CASES)
def test_unpermute_grad(case, dt):
    T, E, k, d = case
    banner("unpermute", case, dt)
    idx = stage.routing(50 + T, T, E, k)
    _, _, dest, _ = oracle.permute(idx, E)
    dxp = stage.normal(51, (T * k, d), 1.0, dt)
    base = stage.normal(52, (T, d), 1.0, dt)
    g = M.moe_unpermute_grad(dev(dxp, dt), dev_i32(dest))
    acc = dev(base, dt)
    M.moe_unpermute_grad(dev(dxp, dt), dev_i32(dest), acc, accumulate=1)
    torch.cuda.synchronize()
    ref = oracle.unpermute_grad(dxp, dest)
    assert_close(g, ref, dt, "dx")
    assert_close(acc, ref + base, dt, "dx accumulated")


# -------------------------------------------------------------- gate bwd

GB_CASES = [(1000, 128, 16, 2, 1), (3000, 64, 8, 2, 1), (517, 128, 64, 8, 1),
            (300, 64, 4, 1, 1), (200, 128, 32, 4, 0), (1, 64, 4, 2, 0),
            (2500, 256, 128, 8, 0), (97, 64, 1024, 4, 1), (61, 64, 1024, 3, 0)]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", GB_CASES)
def test_gate_topk_bwd(case, dt):
    T, d, E, k, renorm = case
    banner("gate_bwd", case, dt)
    x = stage.normal(60, (T, d), 1.0, dt)
    Wg = stage.normal(61, (d, E), 1 / np.sqrt(d), dt)
    l = oracle.gate_logits(x, Wg)
    idx = oracle.topk_select(l, k)
    w = oracle.gate_weights(l, idx, renorm).astype(np.float32)
    dw = stage.normal(62, (T, k), 1.0, "f32")
    dx0 = stage.normal(63, (T, d), 1.0, dt)
    g_dx = dev(dx0, dt)
    dWg = M.moe_gate_topk_bwd(dev(x, dt), dev(Wg, dt), dev(l), dev_i32(idx), dev(w),
                              dev(dw), g_dx, renorm)
    torch.cuda.synchronize()
    _, rdWg, rdx = oracle.gate_bwd(x, Wg, l, idx, w, dw, renorm)
    if k > 1 or renorm == 0:
        assert_close(dWg, rdWg, dt, "dWg")
    else:
        assert np.all(host(dWg) == 0)
    assert_close(g_dx, dx0 + rdx, dt, "dx += dl Wg^T")
    # overwrite mode: the old dx is not read (NaN garbage stays out)
    g_dx.fill_(float("nan"))
    dWg2 = M.moe_gate_topk_bwd(dev(x, dt), dev(Wg, dt), dev(l), dev_i32(idx), dev(w),
                               dev(dw), g_dx, renorm, accumulate=False)
    torch.cuda.synchronize()
    assert torch.equal(dWg2, dWg)
    assert bool(torch.isfinite(g_dx).all())
    assert_close(g_dx, rdx, dt, "dx = dl Wg^T")
