"""The oracle against what the pages and mathematics fix (CPU only).

No page prints a worked numeric example, so the oracle is pinned by: the
dense masked formulation (exactness of reordering, long-context MoE paper,
abstract), brute-force counting sort and top-k, the recursive-summation
error bound, closed-form hand-worked values, central finite differences and
torch autograd.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from moe_inputs import CONFIGS, rng

import _pins as P


# ------------------------------------------------------------------ gate

def test_gate_c_equals_numpy_definition_bitwise():
    g = np.random.default_rng(1)
    x = g.standard_normal((37, 129)).astype(np.float32)
    Wg = g.standard_normal((129, 11)).astype(np.float32)
    b = g.standard_normal(11).astype(np.float32)
    for bias in (None, b):
        a = oracle.gate_logits(x, Wg, bias)
        n = oracle.gate_logits_numpy(x, Wg, bias)
        assert a.dtype == np.float32 and np.array_equal(a, n)


def test_gate_within_recursive_summation_bound():
    # Higham, Accuracy and Stability of Numerical Algorithms, (3.5):
    # |fl(x.y) - x.y| <= gamma_n |x|.|y|, gamma_n = n u / (1 - n u).
    g = np.random.default_rng(2)
    d = 512
    x = g.standard_normal((64, d)).astype(np.float32)
    Wg = g.standard_normal((d, 8)).astype(np.float32)
    b = g.standard_normal(8).astype(np.float32)
    l32 = oracle.gate_logits(x, Wg, b).astype(np.float64)
    exact = x.astype(np.float64) @ Wg.astype(np.float64) + b
    u = 2.0 ** -24
    n = d + 1
    gamma = n * u / (1 - n * u)
    bound = gamma * (np.abs(x).astype(np.float64) @ np.abs(Wg).astype(np.float64)
                     + np.abs(b))
    assert np.all(np.abs(l32 - exact) <= bound)
    # and the order matters: the same sum taken from i = d-1 down differs
    # somewhere (fp32 addition is not associative), so the pin fixes order
    rev = oracle.gate_logits_numpy(x[:, ::-1], Wg[::-1, :])
    assert not np.array_equal(rev, oracle.gate_logits(x, Wg))


def test_gate_bf16_inputs_products_exact():
    # bf16 x bf16 products are exact in fp32, so an FMA chain gives the same
    # bits as the rounded-product chain for bf16 data.
    c = CONFIGS["moe_s_like"]
    x = rng.gen_rows(c, "x", np.arange(16))
    Wg = rng.gen(c, "Wg")
    l = oracle.gate_logits(x, Wg)
    acc = np.zeros((16, c.E), dtype=np.float32)
    for i in range(c.d):
        p64 = x[:, i:i + 1].astype(np.float64) * Wg[i:i + 1].astype(np.float64)
        assert np.array_equal(p64.astype(np.float32).astype(np.float64), p64)
        acc = (acc.astype(np.float64) + p64).astype(np.float32)
    assert np.array_equal(acc, l)
    # The exactness needs the product inside fp32's normal range: two bf16
    # values (8-bit significands) whose product lies below 2^-126 lose bits
    # to fp32's subnormal spacing, so there an FMA and a rounded product can
    # differ.  The gate's inputs stay far from that range.
    a = np.float32(np.ldexp(1.0078125, -70))      # 1 + 2^-7, a bf16 value
    assert np.float32(a).view(np.uint32) & 0xffff == 0
    exact = np.float64(a) * np.float64(a)
    assert np.float64(np.float32(exact)) != exact


def test_topk_brute_force_and_ties():
    g = np.random.default_rng(3)
    l = g.integers(-3, 4, size=(50, 9)).astype(np.float32)   # many ties
    for k in (1, 2, 4, 9):
        assert P.check_topk_brute(l, k) == 0.0
    # k = 1 is argmax (the first maximum wins)
    assert np.array_equal(oracle.topk_select(l, 1)[:, 0], np.argmax(l, axis=1))
    # -0.0 and +0.0 tie; lower index wins
    z = np.array([[-0.0, 0.0, -1.0]], dtype=np.float32)
    assert oracle.topk_select(z, 2).tolist() == [[0, 1]]


def test_weights_sum_to_one_and_special_cases():
    g = np.random.default_rng(4)
    l = (g.standard_normal((200, 16)) * 4).astype(np.float32)
    for k in (1, 2, 8):
        idx = oracle.topk_select(l, k)
        w = oracle.gate_weights(l, idx, 1)
        assert np.all(np.abs(w.sum(axis=1) - 1) <= 4 * k * 2.0 ** -53)
        assert np.all(np.diff(w, axis=1) <= 0)     # best slot first
        if k == 1:
            assert np.all(w == 1.0)
    # renorm=0 reads the full softmax (library routine) at the chosen experts
    idx = oracle.topk_select(l, 3)
    w0 = oracle.gate_weights(l, idx, 0)
    full = softmax(l.astype(np.float64), axis=1)
    assert np.allclose(w0, np.take_along_axis(full, idx, 1), rtol=1e-14,
                       atol=0)
    # renorm=1 equals the renormalised full softmax
    w1 = oracle.gate_weights(l, idx, 1)
    assert np.allclose(w1, w0 / w0.sum(axis=1, keepdims=True), rtol=1e-13,
                       atol=0)


# ---------------------------------------------------------------- permute

@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (13, 4, 2), (40, 7, 3),
                                   (25, 5, 5), (64, 16, 1)])
def test_permute_equals_brute_force_counting_sort(T, E, k):
    g = np.random.default_rng(T * 100 + E)
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    assert P.check_permute_brute(idx, E) == 0.0


def test_permute_invariants_and_skewed_routing():
    g = np.random.default_rng(5)
    E, k, T = 12, 2, 500
    # heavy skew: expert 3 in nearly every token, experts 9..11 never
    idx = np.stack([[3, int(g.integers(0, 9)) if g.random() < 0.9 else 3]
                    for _ in range(T)])
    idx[idx[:, 0] == idx[:, 1], 1] = 4
    counts, offsets, dest, src = oracle.permute(idx, E)
    assert counts.sum() == T * k and offsets[-1] == T * k
    assert np.all(counts[9:] == 0)
    flat = dest.reshape(-1)
    assert np.array_equal(np.sort(flat), np.arange(T * k))      # bijection
    for e in range(E):
        seg = src[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)                          # stable
    x = g.standard_normal((T, 3))
    xp = oracle.dispatch_rows(x, src)
    for j in range(k):
        assert np.array_equal(xp[dest[:, j]], x)


# ----------------------------------------------------------------- layer

@pytest.mark.parametrize("i", range(5))
def test_permuted_layer_equals_dense_masked_layer(i):
    L = P.all_small_layers()[i]
    assert P.check_dense_equivalence(L) <= 1e-12


def test_dense_equivalence_renorm0():
    L = P.rand_layer(11, 9, 4, 5, 5, 2, "gelu", True)
    assert P.check_dense_equivalence(L, renorm=0) <= 1e-12


def test_single_expert_reduces_to_plain_mlp():
    L = P.rand_layer(12, 10, 6, 7, 1, 1)
    fw = oracle.layer_forward(L["x"], L["Wg"], L["W1"], L["W2"], None, k=1)
    x = L["x"].astype(np.float64)
    mlp = oracle.gelu(x @ L["W1"][0]) @ L["W2"][0]
    assert np.abs(fw["y"] - mlp).max() <= 1e-13 * np.abs(mlp).max()


def test_activation_closed_forms():
    # standard normal table values
    assert math.isclose(oracle.gelu(1.0), 0.8413447460685429, rel_tol=1e-15)
    assert math.isclose(oracle.gelu(-1.0), -0.15865525393145707, rel_tol=1e-14)
    assert math.isclose(oracle.gelu(2.0), 1.9544997361036416, rel_tol=1e-15)
    assert oracle.gelu(0.0) == 0.0 and oracle.gelu_grad(0.0) == 0.5
    assert oracle.silu(0.0) == 0.0 and oracle.silu_grad(0.0) == 0.5
    z = np.linspace(-6, 6, 97)
    h = 1e-6
    for fn, gr in ((oracle.gelu, oracle.gelu_grad), (oracle.silu, oracle.silu_grad)):
        fd = (fn(z + h) - fn(z - h)) / (2 * h)
        assert np.abs(fd - gr(z)).max() < 1e-8


def test_golden_hand_worked_example():
    assert P.check_golden_hand_example() <= 1e-12


# ------------------------------------------------------------- gradients

@pytest.mark.parametrize("case", [
    ("gelu", 1, 2, 1), ("gelu", 2, 1, 1), ("swiglu", 2, 3, 1),
    ("gelu", 2, 3, 0), ("swiglu", 3, 4, 0)])
def test_finite_differences(case):
    act, k, E_extra, renorm = case
    L = P.rand_layer(20 + k, 6, 4, 5, k + E_extra, k, act, bias=True)
    assert P.check_finite_differences(L, renorm) < 1e-6


@pytest.mark.parametrize("case", [("gelu", 1, 1), ("gelu", 2, 1),
                                  ("swiglu", 2, 1), ("gelu", 3, 0)])
def test_torch_autograd_dense(case):
    act, k, renorm = case
    L = P.rand_layer(30 + k, 7, 5, 6, 4, k, act, bias=True)
    assert P.check_torch_autograd(L, renorm) < 1e-11


def test_top1_renormalised_gate_gradient_is_zero():
    L = P.rand_layer(40, 8, 4, 5, 3, 1)
    fw = oracle.layer_forward(L["x"], L["Wg"], L["W1"], L["W2"], None, k=1)
    gr = oracle.layer_backward(fw, L["dy"], L["x"], L["Wg"], L["W1"], L["W2"])
    assert np.all(gr["dlogits"] == 0) and np.all(gr["dWg"] == 0)


def test_zero_load_expert_has_zero_weight_grad():
    L = P.rand_layer(41, 6, 4, 5, 4, 1)
    idx = np.zeros((6, 1), dtype=np.int32)          # everyone to expert 0
    fw = oracle.layer_forward(L["x"], L["Wg"], L["W1"], L["W2"], None, k=1,
                              idx=idx)
    gr = oracle.layer_backward(fw, L["dy"], L["x"], L["Wg"], L["W1"], L["W2"])
    assert list(fw["counts"]) == [6, 0, 0, 0]
    for e in (1, 2, 3):
        assert np.all(gr["dW1"][e] == 0) and np.all(gr["dW2"][e] == 0)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_column_restricted_expert_grads_equal_full(act):
    # the restricted form is the full segment backward read at a few hidden
    # units (pinned here against ffn_bwd_segment, itself pinned by finite
    # differences and torch autograd above)
    g = np.random.default_rng(70)
    n, d, f = 13, 6, 9
    xs = g.standard_normal((n, d))
    dO = g.standard_normal((n, d))
    W1, W3 = g.standard_normal((d, f)), g.standard_normal((d, f))
    W2 = g.standard_normal((f, d))
    _, dW1, dW3, dW2 = oracle.ffn_bwd_segment(dO, xs, W1, W2, W3, act)
    cols = np.array([0, 4, 8, 5])
    c1, c3, c2 = oracle.ffn_bwd_columns(dO, xs, W1, W2, W3, act, cols)
    assert np.allclose(c1, dW1[:, cols], rtol=1e-13, atol=1e-13)
    assert np.allclose(c2, dW2[cols, :], rtol=1e-13, atol=1e-13)
    if act == "swiglu":
        assert np.allclose(c3, dW3[:, cols], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_column_restricted_expert_grads_torch(act):
    # the same quantities from torch float64 autograd of L = <dO, FFN(x)>
    import torch
    g = np.random.default_rng(71)
    n, d, f = 11, 5, 7
    xs = g.standard_normal((n, d))
    dO = g.standard_normal((n, d))
    t = lambda a: torch.tensor(a, requires_grad=True)
    W1, W3, W2 = t(g.standard_normal((d, f))), t(g.standard_normal((d, f))), \
        t(g.standard_normal((f, d)))
    X = torch.tensor(xs)
    h = X @ W1
    a = torch.nn.functional.gelu(h) if act == "gelu" else \
        torch.nn.functional.silu(h) * (X @ W3)
    ((a @ W2) * torch.tensor(dO)).sum().backward()
    cols = np.array([6, 1, 3])
    c1, c3, c2 = oracle.ffn_bwd_columns(dO, xs, W1.detach().numpy(),
                                        W2.detach().numpy(),
                                        W3.detach().numpy(), act, cols)
    assert np.allclose(c1, W1.grad.numpy()[:, cols], rtol=1e-12, atol=1e-12)
    assert np.allclose(c2, W2.grad.numpy()[cols, :], rtol=1e-12, atol=1e-12)
    if act == "swiglu":
        assert np.allclose(c3, W3.grad.numpy()[:, cols], rtol=1e-12, atol=1e-12)
