"""The permute's row copy fused into the expert GEMMs: moe_permute without
x_perm (routing only) and moe_expert_ffn_fwd_gather / _bwd_gather, which read
permuted row r as x[src[r]].  Their results must be bit-identical to the copy
followed by the plain entry points (same arithmetic, other addresses), and
within tolerance of the oracle.  Cases cover ragged segments, empty experts,
T = 1, and an expert with more rows than the reduction-row map holds at once
(the dW gather reloads it between stages)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_permute_amd as M
import oracle
from moe_inputs import device, small_variant, stage

from _gpu import assert_close, assert_equal_i, banner, dev, dev_i32, host, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]

CASES = [  # T, E, k, d, f, hot expert (every token's first choice) or None
    (300, 5, 2, 128, 192, None),
    (1031, 12, 3, 128, 256, None),
    (257, 4, 1, 64, 128, None),
    (1, 3, 2, 64, 64, None),
    (9000, 6, 2, 64, 128, 4),      # expert 4 gets 9000 rows: three map chunks
    (12500, 3, 2, 64, 128, 1),     # 8333 rows per expert: the dW products' 64-deep ring
]


def routing(T, E, k, hot, seed):
    g = np.random.default_rng(seed)
    idx = np.empty((T, k), np.int32)
    for t in range(T):
        if hot is None:
            idx[t] = g.permutation(E)[:k]
        else:
            rest = [e for e in g.permutation(E) if e != hot]
            idx[t] = [hot] + rest[:k - 1]
    return idx


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("case", CASES)
def test_gather_matches_copy_and_oracle(case, act, dt):
    T, E, k, d, f, hot = case
    banner("gather", case, act, dt)
    seed = 7 * T + E
    idx = routing(T, E, k, hot, seed)
    x = stage.normal(seed + 1, (T, d), 1.0, dt)
    W1 = stage.normal(seed + 2, (E, d, f), 1 / np.sqrt(d), dt)
    W2 = stage.normal(seed + 3, (E, f, d), 1 / np.sqrt(f), dt)
    W3 = stage.normal(seed + 4, (E, d, f), 1 / np.sqrt(d), dt) if act == "swiglu" else None
    R = T * k
    dO = stage.normal(seed + 5, (R, d), 1.0, dt)
    gx, gi = dev(x, dt), dev_i32(idx)
    gW1, gW2 = dev(W1, dt), dev(W2, dt)
    gW3 = dev(W3, dt) if W3 is not None else None
    gdO = dev(dO, dt)

    counts, offsets, dest, src, xp = M.moe_permute(gi, gx, E)
    c2, o2, d2, s2, none = M.moe_permute(gi, gx, E, copy=False)
    assert none is None
    for a, b, n in ((counts, c2, "counts"), (offsets, o2, "offsets"), (dest, d2, "dest"),
                    (src, s2, "src")):
        assert torch.equal(a, b), n

    h, a, o = M.moe_expert_ffn_fwd(xp, offsets, gW1, gW2, gW3, act)
    hg, ag, og = M.moe_expert_ffn_fwd_gather(gx, src, offsets, gW1, gW2, gW3, act)
    bw = M.moe_expert_ffn_bwd(gdO, xp, h, a, offsets, gW1, gW2, gW3, act)
    bg = M.moe_expert_ffn_bwd_gather(gdO, gx, src, hg, ag, offsets, gW1, gW2, gW3, act)
    torch.cuda.synchronize()
    for n, u, v in (("h_save", h, hg), ("a_save", a, ag), ("out_perm", o, og),
                    ("dx_perm", bw[0], bg[0]), ("dW1", bw[1], bg[1]), ("dW2", bw[3], bg[3])):
        assert torch.equal(u, v), n + " differs from the copy path"
    if act == "swiglu":
        assert torch.equal(bw[2], bg[2]), "dW3 differs from the copy path"

    # the oracle on the host copy of the same inputs
    rc, ro, rd, rs = oracle.permute(idx, E)
    assert_equal_i(src, rs, "src")
    if R > 4096:       # the bit-identity above carries the oracle checks of smaller cases
        return
    xph = oracle.dispatch_rows(x, rs)
    ref = oracle.expert_ffn_fwd(xph, ro, W1, W2, W3, act)
    assert_close(ag, ref["A"], dt, "A")
    assert_close(og, ref["out"], dt, "out_perm")
    rb = oracle.expert_ffn_bwd(dO, xph, ro, W1, W2, W3, act)
    assert_close(bg[0], rb["dx_perm"], dt, "dx_perm")
    assert_close(host(bg[1]), np.stack(list(rb["dW1"][e] for e in range(E))), dt, "dW1")
    assert_close(host(bg[3]), np.stack(list(rb["dW2"][e] for e in range(E))), dt, "dW2")
    if act == "swiglu":
        assert_close(host(bg[2]), np.stack(list(rb["dW3"][e] for e in range(E))), dt, "dW3")


@pytest.mark.parametrize("name", ["moe_s_like", "long_ctx_swiglu", "tiny_fp32"])
def test_layer_fused_gather_is_bit_identical(name):
    """MoELayer(fuse_gather=True) keeps no x_perm and gives the same bits."""
    kw = {} if name == "tiny_fp32" else dict(T=1000, d=256, f=512, E=8, k=2)
    cfg = small_variant(name, **kw)
    banner("layer fuse_gather", cfg.short())
    t = device.gen_all(cfg)
    outs = []
    for fuse in (False, True):
        layer = M.MoELayer(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act,
                           device.torch_dtype(cfg), cfg.renorm, fuse_gather=fuse)
        assert (layer.x_perm is None) == fuse
        layer.bind(t["x"], t["Wg"], t["W1"], t["W2"], t["W3"], t["bias"], t["dy"])
        layer.step()
        torch.cuda.synchronize()
        names = ["y", "h_save", "a_save", "out_perm", "dx_perm", "dW1", "dW2", "dx", "dWg"]
        if cfg.swiglu:
            names.append("dW3")
        outs.append({n: getattr(layer, n).clone() for n in names})
        del layer
    for n in outs[0]:
        assert torch.equal(outs[0][n], outs[1][n]), n
