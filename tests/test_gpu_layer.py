"""Whole-layer parity: the eight entry points chained exactly as the
benchmark chains them, on the workloads' own shapes and seeded inputs,
against the oracle run on the host copy of the same inputs."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_permute_amd as M
import oracle
from moe_inputs import CONFIGS, device, rng

from _gpu import assert_close, assert_equal_i, banner, host, needs_gpu, saved_state

pytestmark = [pytest.mark.gpu, needs_gpu]


def run_layer(cfg, overlap_gate=True):
    t = device.gen_all(cfg)
    layer = M.MoELayer(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act,
                       device.torch_dtype(cfg), cfg.renorm, overlap_gate=overlap_gate)
    layer.bind(t["x"], t["Wg"], t["W1"], t["W2"], t["W3"], t["bias"], t["dy"])
    layer.step()
    torch.cuda.synchronize()
    return layer, t


@pytest.mark.parametrize("name", ["tiny_fp32", "moe_s_like"])
def test_layer_full(name):
    cfg = CONFIGS[name]
    banner("layer full", name)
    layer, t = run_layer(cfg)
    x, Wg, dy = (rng.gen(cfg, n) for n in ("x", "Wg", "dy"))
    W1, W2 = rng.gen_experts(cfg, "W1"), rng.gen_experts(cfg, "W2")
    # the device generator reproduces the host inputs bit for bit
    assert torch.equal(t["x"].cpu().float(), torch.from_numpy(x))
    assert torch.equal(t["W2"].cpu().float(), torch.from_numpy(W2))
    bias = rng.logit_bias(cfg)
    fw = oracle.layer_forward(x, Wg, W1, W2, None, k=cfg.k, act=cfg.act, bias=bias,
                              renorm=cfg.renorm)
    gr = oracle.layer_backward(fw, dy, x, Wg, W1, W2, None, act=cfg.act,
                               renorm=cfg.renorm)
    dt = cfg.dtype
    assert_equal_i(layer.logits.cpu().numpy().view(np.uint32),
                   fw["logits"].view(np.uint32), "logits")
    for n in ("idx", "counts", "offsets", "dest", "src"):
        got = {"idx": layer.topk_idx}.get(n, getattr(layer, n, None))
        assert_equal_i(got, fw[n], n)
    assert_close(layer.topk_w, fw["w"], "f32", "topk_w")
    assert_close(layer.x_perm, fw["x_perm"], dt, "x_perm")
    assert_close(layer.h_save, saved_state(cfg.act, fw["H"], fw.get("H3")), dt,
                 "saved GeLU'(H)")
    assert_close(layer.a_save, fw["A"], dt, "A")
    assert_close(layer.out_perm, fw["out_perm"], dt, "out_perm")
    assert_close(layer.y, fw["y"], dt, "y")
    assert_close(layer.d_out_perm, gr["d_out_perm"], dt, "d_out_perm")
    assert_close(layer.d_topk_w, gr["dw"], dt, "d_topk_w")
    assert_close(layer.dx_perm, gr["dx_perm"], dt, "dx_perm")
    assert_close(layer.dW1, gr["dW1"], dt, "dW1")
    assert_close(layer.dW2, gr["dW2"], dt, "dW2")
    assert_close(layer.dx, gr["dx"], dt, "dx")
    if cfg.k > 1:
        assert_close(layer.dWg, gr["dWg"], dt, "dWg")
    else:
        assert np.all(host(layer.dWg) == 0)


OVERLAP_CASES = {
    "moe_s_like": None,                       # every RAGGED_M product split
    "small_swiglu": ("long_ctx_swiglu", dict(T=1500, d=256, f=512, E=8)),
    # up and dA (N = f = 8192) run whole, down and dX (N = d = 512) split
    "mixed_split": ("moe_s_like", dict(d=512, f=8192)),
}


@pytest.mark.parametrize("name", list(OVERLAP_CASES))
def test_stream_overlap_bit_identical(name):
    """The side-stream schedule (partial tiles and dW2 beside the main
    launches, the gate's backward beside the expert GEMMs' backward) gives
    exactly the bits of the single-stream schedule."""
    from moe_inputs import small_variant
    spec = OVERLAP_CASES[name]
    cfg = CONFIGS[name] if spec is None else small_variant(spec[0], **spec[1])
    banner("overlap", name, cfg.short())
    outs = []
    try:
        for on in (False, True):
            M.moe_set_overlap(on)
            # the gate's backward on its own stream only with the side stream
            layer, _ = run_layer(cfg, overlap_gate=on)
            outs.append({n: getattr(layer, n).clone() for n in
                         ("h_save", "a_save", "out_perm", "y", "dx_perm", "dW1", "dW2",
                          "dW3", "dx", "dWg") if getattr(layer, n) is not None})
            del layer
    finally:
        M.moe_set_overlap(True)
    for n in outs[0]:
        assert torch.equal(outs[0][n], outs[1][n]), n


@pytest.mark.parametrize("stream_kind", ["default", "created"])
def test_back_to_back_steps(stream_kind):
    """Steps issued back to back with no host synchronisation, alternating
    two input sets (x and dy negated/halved: other routing, other
    gradients), under every schedule: the library's side stream on/off and
    the gate backward on its own stream or not, on torch's default stream
    (raw handle 0) and on a created stream.  The last step's outputs must
    equal one serial step on the same inputs, bit for bit: a missing wait
    between streams shows up as a stale read or a raced read-modify-write of
    dx."""
    cfg = CONFIGS["moe_s_like"]
    banner("back-to-back steps", stream_kind)
    t = device.gen_all(cfg)
    xB = (-t["x"]).contiguous()
    dyB = (t["dy"] * -0.5).contiguous()
    names = ("logits", "topk_idx", "y", "out_perm", "d_out_perm", "d_topk_w",
             "dx_perm", "dx", "dWg", "dW1", "dW2")

    def make(og):
        return M.MoELayer(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act,
                          device.torch_dtype(cfg), cfg.renorm, overlap_gate=og)

    def bind(layer, x, dy):
        layer.bind(x, t["Wg"], t["W1"], t["W2"], t["W3"], t["bias"], dy)

    other = torch.cuda.Stream()
    handle = 0 if stream_kind == "default" else other.cuda_stream
    try:
        M.moe_set_overlap(False)
        ref = make(False)
        bind(ref, xB, dyB)
        ref.step()
        torch.cuda.synchronize()
        want = {n: getattr(ref, n).clone() for n in names}
        del ref
        torch.cuda.synchronize()
        for lib_overlap in (True, False):
            M.moe_set_overlap(lib_overlap)
            for og in (False, True):
                layer = make(og)
                for i in range(8):
                    if i % 2:
                        bind(layer, xB, dyB)
                    else:
                        bind(layer, t["x"], t["dy"])
                    layer.step(handle)
                torch.cuda.synchronize()
                bad = [n for n in names if not torch.equal(getattr(layer, n), want[n])]
                assert not bad, (lib_overlap, og, bad)
                del layer
    finally:
        M.moe_set_overlap(True)
