"""Plant plausible mistakes in the oracle (on the CPU) and show that the
pins catch each one.  A pin that passes a wrong oracle proves nothing."""
import numpy as np
import pytest

import oracle
from oracle import moe_oracle as M

import _pins as P


def _run_pins():
    """Worst result over a battery of pins; a crash counts as caught."""
    L2 = P.rand_layer(50, 6, 4, 5, 4, 2, "gelu", True)
    Ls = P.rand_layer(51, 6, 3, 4, 5, 2, "swiglu", True)
    g = np.random.default_rng(52)
    tied = g.integers(-2, 3, size=(30, 6)).astype(np.float32)
    idx = np.stack([g.permutation(5)[:2] for _ in range(20)]).astype(np.int32)
    checks = [
        lambda: P.check_dense_equivalence(L2) > 1e-12,
        lambda: P.check_dense_equivalence(Ls) > 1e-12,
        lambda: P.check_finite_differences(L2, 1, ncoord=6) > 1e-6,
        lambda: P.check_finite_differences(Ls, 1, ncoord=6) > 1e-6,
        lambda: P.check_torch_autograd(L2) > 1e-11,
        lambda: P.check_permute_brute(idx, 5) > 0,
        lambda: P.check_topk_brute(tied, 3) > 0,
        lambda: P.check_golden_hand_example() > 1e-12,
    ]
    caught = []
    for c in checks:
        try:
            caught.append(bool(c()))
        except Exception:
            caught.append(True)
    return caught


def test_unmutated_oracle_passes_every_pin():
    assert not any(_run_pins())


def _gelu_grad_no_pdf_term(z):
    z = np.asarray(z, np.float64)
    return 0.5 * (1.0 + M._erf(z / np.sqrt(2.0)))


def _silu_grad_wrong(z):
    s = M._sigmoid(np.asarray(z, np.float64))
    return s * (1.0 + z * s)


def _combine_swapped_slots(out_perm, dest, w):
    return M.__dict__["_orig_combine"](out_perm, dest, np.asarray(w)[:, ::-1])


def _permute_dest_src_confused(idx, E):
    counts, offsets, dest, src = M.__dict__["_orig_permute"](idx, E)
    order = np.argsort(np.asarray(idx).reshape(-1), kind="stable")
    return counts, offsets, order.reshape(dest.shape).astype(np.int32), src


def _topk_ties_to_higher_index(logits, k):
    order = np.argsort(np.asarray(logits), axis=1, kind="stable")[:, ::-1]
    return order[:, :k].astype(np.int32)


def _gate_grad_sign_flipped(logits, idx, w, dw, renorm=1):
    return -M.__dict__["_orig_gate_logits_grad"](logits, idx, w, dw, renorm)


def _weights_not_renormalised(logits, idx, renorm=1):
    return M.__dict__["_orig_gate_weights"](logits, idx, 0)


def _ffn_bwd_preact_for_dw2(dO, xs, W1e, W2e, W3e=None, act="gelu", saved=None):
    H, H3, A, _ = M.ffn_fwd_segment(xs, W1e, W2e, W3e, act)
    dX, dW1, dW3, dW2 = M.__dict__["_orig_ffn_bwd_segment"](
        dO, xs, W1e, W2e, W3e, act, (H, H3, A))
    return dX, dW1, dW3, np.asarray(H).T @ np.asarray(dO, np.float64)


def _combine_bwd_extra_weight(dy, out_perm, dest, w):
    d_out, dw = M.__dict__["_orig_combine_bwd"](dy, out_perm, dest, w)
    return d_out, dw * np.asarray(w)


def _unpermute_drops_last_slot(dx_perm, dest):
    return M.__dict__["_orig_unpermute_grad"](dx_perm, np.asarray(dest)[:, :-1])


def _ffn_fwd_off_by_one(x_perm, offsets, W1, W2, W3=None, act="gelu",
                        experts=None):
    off = np.asarray(offsets).copy()
    off[1:-1] = np.maximum(off[1:-1] - 1, 0)
    return M.__dict__["_orig_expert_ffn_fwd"](x_perm, off, W1, W2, W3, act,
                                              experts)


MUTATIONS = {
    "gelu_grad": ("gelu_grad", _gelu_grad_no_pdf_term),
    "silu_grad": ("silu_grad", _silu_grad_wrong),
    "combine": ("combine", _combine_swapped_slots),
    "permute": ("permute", _permute_dest_src_confused),
    "topk": ("topk_select", _topk_ties_to_higher_index),
    "gate_grad": ("gate_logits_grad", _gate_grad_sign_flipped),
    "weights": ("gate_weights", _weights_not_renormalised),
    "dW2": ("ffn_bwd_segment", _ffn_bwd_preact_for_dw2),
    "combine_bwd": ("combine_bwd", _combine_bwd_extra_weight),
    "unpermute": ("unpermute_grad", _unpermute_drops_last_slot),
    "segments": ("expert_ffn_fwd", _ffn_fwd_off_by_one),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setitem(M.__dict__, "_orig_" + attr, getattr(M, attr))
    monkeypatch.setattr(M, attr, bad)
    monkeypatch.setattr(oracle, attr, bad, raising=False)
    assert any(_run_pins()), f"no pin caught the planted mistake in {attr}"
