"""OffloadedMoELayer: the layer step with the expert weights in pinned host
memory, uploaded group by group beside the GEMMs, and the weight gradients
downloaded the same way.  Every output must be bit-identical to MoELayer's
(the group calls compute the same tiles in the same order), for ragged last
groups, one expert per group, one group, SwiGLU and fp32, and over steps
issued back to back with other inputs."""
import pytest
import torch

import mixture_experts_layer_permute_amd as M
from moe_inputs import device, small_variant

from _gpu import banner, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]

CASES = [  # workload, overrides, experts per group
    ("moe_s_like", dict(T=1000, d=256, f=512, E=8, k=2), 3),       # groups 3, 3, 2
    ("moe_s_like", dict(T=1000, d=256, f=512, E=8, k=2), 1),
    ("moe_s_like", dict(T=1000, d=256, f=512, E=8, k=2), 8),       # one group
    ("long_ctx_swiglu", dict(T=777, d=128, f=256, E=16, k=4), 5),
    ("many_expert_zipf1.0", dict(T=1200, d=128, f=256, E=32, k=2), 6),   # empty experts
    ("tiny_fp32", {}, 3),
]
OUT = ["logits", "topk_idx", "topk_w", "y", "d_topk_w", "dx_perm", "dx", "dWg"]


def host_pinned(t):
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


def whole_step(cfg, t, x=None, dy=None):
    L = M.MoELayer(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act, device.torch_dtype(cfg),
                   cfg.renorm)
    L.bind(t["x"] if x is None else x, t["Wg"], t["W1"], t["W2"], t["W3"], t["bias"],
           t["dy"] if dy is None else dy)
    L.step()
    torch.cuda.synchronize()
    return L


def offloaded(cfg, t, G, pinned=()):
    L = M.OffloadedMoELayer(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act,
                            device.torch_dtype(cfg), cfg.renorm, group_experts=G,
                            pinned=pinned)
    W3 = host_pinned(t["W3"]) if t["W3"] is not None else None
    L.bind(t["x"], t["Wg"], host_pinned(t["W1"]), host_pinned(t["W2"]), W3, t["bias"],
           t["dy"])
    return L


def same(off, ref, swiglu):
    for n in OUT:
        assert torch.equal(getattr(off, n), getattr(ref, n)), n
    for n in ["dW1", "dW2"] + (["dW3"] if swiglu else []):
        assert torch.equal(getattr(off, n), getattr(ref, n).cpu()), n


@pytest.mark.parametrize("case", CASES)
def test_offloaded_matches_resident_layer(case):
    name, kw, G = case
    cfg = small_variant(name, **kw)
    banner("offload", cfg.short(), G)
    t = device.gen_all(cfg)
    ref = whole_step(cfg, t)
    off = offloaded(cfg, t, G)
    off.step()
    torch.cuda.synchronize()
    same(off, ref, cfg.swiglu)


def test_offloaded_back_to_back_steps():
    """Five steps issued with no host synchronisation, x and dy switched
    between two sets (other routing, other gradients) each step: the last
    step equals one resident step on the same inputs."""
    cfg = small_variant("moe_s_like", T=1000, d=256, f=512, E=8, k=2)
    banner("offload back-to-back", cfg.short())
    t = device.gen_all(cfg)
    xB, dyB = (-t["x"]).contiguous(), (t["dy"] * -0.5).contiguous()
    ref = whole_step(cfg, t, xB, dyB)
    off = offloaded(cfg, t, 3)
    for i in range(5):
        off.x, off.dy = (xB, dyB) if i % 2 == 0 else (t["x"], t["dy"])
        off.step()
    torch.cuda.synchronize()
    same(off, ref, cfg.swiglu)


def test_grads_ready_covers_the_downloads():
    """Waiting on grads_ready alone (no device synchronisation) is enough
    for the host weight gradients: they equal the resident layer's."""
    cfg = small_variant("moe_s_like", T=1000, d=256, f=512, E=8, k=2)
    banner("offload grads_ready", cfg.short())
    t = device.gen_all(cfg)
    ref = whole_step(cfg, t)
    for G in (2, 4):                  # four groups (downloads as slots recycle), two groups
        off = offloaded(cfg, t, G)
        off.dW1.zero_()
        off.dW2.zero_()
        off.step()
        off.grads_ready.synchronize()
        assert torch.equal(off.dW1, ref.dW1.cpu()), G
        assert torch.equal(off.dW2, ref.dW2.cpu()), G
        torch.cuda.synchronize()


def test_offloaded_against_oracle():
    """The offloaded step against the oracle itself (not only against the
    resident layer): routing bit-exact, y, dx, dWg and every expert's weight
    gradients within the dtype's tolerance (SwiGLU, ragged last group)."""
    import numpy as np
    import oracle
    from moe_inputs import rng
    from _gpu import assert_close, assert_equal_i, host
    cfg = small_variant("long_ctx_swiglu", T=777, d=128, f=256, E=16, k=4)
    banner("offload vs oracle", cfg.short())
    t = device.gen_all(cfg)
    off = offloaded(cfg, t, 5)
    off.step()
    off.grads_ready.synchronize()
    torch.cuda.synchronize()
    x, Wg, dy = (rng.gen(cfg, n) for n in ("x", "Wg", "dy"))
    W1, W2, W3 = (rng.gen_experts(cfg, n) for n in ("W1", "W2", "W3"))
    fw = oracle.layer_forward(x, Wg, W1, W2, W3, k=cfg.k, act=cfg.act,
                              bias=rng.logit_bias(cfg), renorm=cfg.renorm)
    gr = oracle.layer_backward(fw, dy, x, Wg, W1, W2, W3, act=cfg.act, renorm=cfg.renorm)
    assert_equal_i(off.logits.cpu().numpy().view(np.uint32), fw["logits"].view(np.uint32),
                   "logits")
    assert_equal_i(off.topk_idx, fw["idx"], "topk_idx")
    dt = cfg.dtype
    assert_close(off.y, fw["y"], dt, "y")
    assert_close(off.dx, gr["dx"], dt, "dx")
    assert_close(off.dWg, gr["dWg"], dt, "dWg")
    for n in ("dW1", "dW2", "dW3"):
        assert_close(host(getattr(off, n)), gr[n], dt, n)


PIN_CASES = [  # workload, overrides, experts per group, pinned (None: the most-routed quarter)
    ("many_expert_zipf1.0", dict(T=1200, d=128, f=256, E=32, k=2), 6, None),
    ("moe_s_like", dict(T=1000, d=256, f=512, E=10, k=2), 3, [0, 3, 4, 9]),
    ("moe_s_like", dict(T=1000, d=256, f=512, E=10, k=2), 2, [2, 3, 4, 5, 6]),  # run > G
    ("long_ctx_swiglu", dict(T=777, d=128, f=256, E=16, k=4), 5, None),
    ("moe_s_like", dict(T=1000, d=256, f=512, E=8, k=2), 3, list(range(8))),    # all pinned
    ("tiny_fp32", {}, 2, [1]),
]


@pytest.mark.parametrize("case", PIN_CASES)
def test_pinned_experts_match_resident_layer(case):
    """Pinned experts (weights copied to the GPU once, gradients kept there)
    beside offloaded groups: every output bit-identical to MoELayer's, the
    pinned experts' gradients in dW1p/dW2p/dW3p, the others' on the host."""
    name, kw, G, pinned = case
    cfg = small_variant(name, **kw)
    t = device.gen_all(cfg)
    ref = whole_step(cfg, t)
    if pinned is None:
        pinned = M.OffloadedMoELayer.most_routed(ref.counts, 0.25)
    banner("offload pinned", cfg.short(), G, pinned)
    off = offloaded(cfg, t, G, pinned)
    for _ in range(2):                   # the second step reuses the pinned copies
        off.step()
    off.grads_ready.synchronize()
    torch.cuda.synchronize()
    for n in OUT:
        assert torch.equal(getattr(off, n), getattr(ref, n)), n
    rest = [e for e in range(cfg.E) if e not in pinned]
    for n in ["dW1", "dW2"] + (["dW3"] if cfg.swiglu else []):
        want = getattr(ref, n)
        if rest:
            assert torch.equal(getattr(off, n)[rest], want.cpu()[rest]), n
        if pinned:
            assert torch.equal(getattr(off, n + "p"), want[pinned]), n + "p"
