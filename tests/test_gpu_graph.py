"""The layer step captured in one HIP graph (with the side-stream fork and
join inside it) and replayed: every replay must give the eager step's bits.
Replays are interleaved with eager steps on other inputs and synchronizations,
so that state left by one replay cannot hide in the next."""
import pytest
import torch

import mixture_experts_layer_permute_amd as M
from moe_inputs import device, small_variant

from _gpu import banner, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]

OUTS = ["logits", "topk_idx", "topk_w", "h_save", "a_save", "out_perm", "y", "d_out_perm",
        "d_topk_w", "dx_perm", "dW1", "dW2", "dx", "dWg"]


@pytest.mark.parametrize("name,kw", [
    ("moe_s_like", dict(T=2000, d=256, f=512, E=8, k=2)),
    ("long_ctx_swiglu", dict(T=1500, d=256, f=512, E=16, k=4)),
    ("many_expert_zipf1.0", dict(T=3000, d=128, f=256, E=64, k=2)),
])
def test_graph_replay_is_bit_identical(name, kw):
    cfg = small_variant(name, **kw)
    banner("graph", cfg.short())
    M.moe_set_overlap(True)
    t = device.gen_all(cfg)
    args = (cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act, device.torch_dtype(cfg), cfg.renorm)
    ref = M.MoELayer(*args).bind(t["x"], t["Wg"], t["W1"], t["W2"], t["W3"], t["bias"],
                                 t["dy"])
    ref.step()
    torch.cuda.synchronize()
    want = {n: getattr(ref, n).clone() for n in OUTS + (["dW3"] if cfg.swiglu else [])}
    layer = M.MoELayer(*args).bind(t["x"], t["Wg"], t["W1"], t["W2"], t["W3"], t["bias"],
                                   t["dy"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up off the default stream
        layer.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.step()
    torch.cuda.synchronize()
    other = device.gen_all(small_variant(name, **dict(kw, seed=cfg.seed + 1)))
    for rep in range(3):
        for n in want:                       # poison the outputs
            getattr(layer, n).fill_(7)
        g.replay()
        torch.cuda.synchronize()
        for n, v in want.items():
            assert torch.equal(getattr(layer, n), v), (rep, n)
        ref.bind(other["x"], other["Wg"], other["W1"], other["W2"], other["W3"],
                 other["bias"], other["dy"])
        ref.step()                           # eager work between replays
        torch.cuda.synchronize()
