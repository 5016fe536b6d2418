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


def offloaded(cfg, t, G):
    L = M.OffloadedMoELayer(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act,
                            device.torch_dtype(cfg), cfg.renorm, group_experts=G)
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
