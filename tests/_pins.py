"""Checks that tie the oracle to things other than itself.

Each check returns the worst discrepancy it found (0 or a small number when
the oracle is right).  The oracle tests assert that every check passes; the
mutation tests plant plausible mistakes in the oracle and assert that some
check catches each one.
"""
import itertools
import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_layer(seed, T, d, f, E, k, act="gelu", bias=False, scale_gate=1.0):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, d))
    Wg = g.standard_normal((d, E)) * scale_gate / np.sqrt(d)
    W1 = g.standard_normal((E, d, f)) / np.sqrt(d)
    W3 = g.standard_normal((E, d, f)) / np.sqrt(d) if act == "swiglu" else None
    W2 = g.standard_normal((E, f, d)) / np.sqrt(f)
    b = g.standard_normal(E).astype(np.float32) if bias else None
    dy = g.standard_normal((T, d))
    f32 = lambda a: None if a is None else a.astype(np.float32)
    return dict(x=f32(x), Wg=f32(Wg), W1=f32(W1), W2=f32(W2), W3=f32(W3),
                bias=b, dy=f32(dy), k=k, act=act)


# ------------------------------------------------------------- brute force

def brute_topk(logits, k):
    T, E = logits.shape
    out = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))
        out[t] = order[:k]
    return out


def brute_counting_sort(idx, E):
    """Walk experts in order; inside each, walk tokens and slots in order."""
    T, k = idx.shape
    dest = np.full((T, k), -1, dtype=np.int64)
    src = []
    counts = []
    for e in range(E):
        n = 0
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    dest[t, j] = len(src)
                    src.append(t)
                    n += 1
        counts.append(n)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    return np.array(counts), offsets, dest, np.array(src, dtype=np.int64)


def dense_masked_layer(x, Wg, W1, W2, W3, bias, k, act, renorm=1):
    """All experts applied to all tokens, masked by the routing: the dense
    dispatch-mask formulation, written token by token, in float64."""
    x = np.asarray(x, np.float64)
    T, d = x.shape
    E = Wg.shape[1]
    l = oracle.gate_logits(x.astype(np.float32), Wg, bias)
    y = np.zeros((T, d))
    for t in range(T):
        row = l[t].astype(np.float64)
        chosen = sorted(range(E), key=lambda e: (-row[e], e))[:k]
        if renorm:
            z = {e: math.exp(row[e] - row[chosen[0]]) for e in chosen}
            s = sum(z.values())
            wt = {e: z[e] / s for e in chosen}
        else:
            m = max(row)
            s = sum(math.exp(v - m) for v in row)
            wt = {e: math.exp(row[e] - m) / s for e in chosen}
        for e in range(E):
            mask = 1.0 if e in wt else 0.0
            h = x[t] @ W1[e].astype(np.float64)
            if act == "gelu":
                a = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2)))
                              for v in h])
            else:
                h3 = x[t] @ W3[e].astype(np.float64)
                a = np.array([v / (1 + math.exp(-v)) for v in h]) * h3
            y[t] += mask * wt.get(e, 0.0) * (a @ W2[e].astype(np.float64))
    return y


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / den)


# ------------------------------------------------------------------ checks

def check_dense_equivalence(L, renorm=1):
    fw = oracle.layer_forward(L["x"], L["Wg"], L["W1"], L["W2"], L["W3"],
                              k=L["k"], act=L["act"], bias=L["bias"],
                              renorm=renorm)
    ref = dense_masked_layer(L["x"], L["Wg"], L["W1"], L["W2"], L["W3"],
                             L["bias"], L["k"], L["act"], renorm)
    return rel_err(fw["y"], ref)


def check_permute_brute(idx, E):
    counts, offsets, dest, src = oracle.permute(idx, E)
    bc, bo, bd, bs = brute_counting_sort(idx, E)
    ok = (np.array_equal(counts, bc) and np.array_equal(offsets, bo)
          and np.array_equal(dest, bd) and np.array_equal(src, bs))
    return 0.0 if ok else 1.0


def check_topk_brute(logits, k):
    return 0.0 if np.array_equal(oracle.topk_select(logits, k),
                                 brute_topk(logits, k)) else 1.0


def _loss(L, renorm, idx, **over):
    p = dict(L)
    p.update(over)
    fw = oracle.layer_forward(p["x"], p["Wg"], p["W1"], p["W2"], p["W3"],
                              k=L["k"], act=L["act"], bias=L["bias"],
                              renorm=renorm, exact_logits=True, idx=idx)
    return float((np.asarray(L["dy"], np.float64) * fw["y"]).sum())


def check_finite_differences(L, renorm=1, ncoord=12, eps=1e-6, seed=0):
    """Central differences of L = <dy, y> (float64 arithmetic, routing frozen)
    against the oracle's backward, on random coordinates of every input."""
    p = {n: (None if L[n] is None else np.asarray(L[n], np.float64))
         for n in ("x", "Wg", "W1", "W2", "W3")}
    L64 = dict(L)
    L64.update(p)
    fw = oracle.layer_forward(p["x"], p["Wg"], p["W1"], p["W2"], p["W3"],
                              k=L["k"], act=L["act"], bias=L["bias"],
                              renorm=renorm, exact_logits=True)
    idx = fw["idx"]
    gr = oracle.layer_backward(fw, L["dy"], p["x"], p["Wg"], p["W1"],
                               p["W2"], p["W3"], act=L["act"], renorm=renorm)
    names = {"x": "dx", "Wg": "dWg", "W1": "dW1", "W2": "dW2", "W3": "dW3"}
    g = np.random.default_rng(seed)
    worst = 0.0
    for n, gn in names.items():
        if p[n] is None:
            continue
        arr = p[n]
        scale = max(np.abs(gr[gn]).max(), 1e-12)
        for _ in range(ncoord):
            pos = tuple(int(g.integers(s)) for s in arr.shape)
            a_plus = arr.copy()
            a_plus[pos] += eps
            a_minus = arr.copy()
            a_minus[pos] -= eps
            fd = (_loss(L64, renorm, idx, **{n: a_plus})
                  - _loss(L64, renorm, idx, **{n: a_minus})) / (2 * eps)
            worst = max(worst, abs(fd - gr[gn][pos]) / scale)
    return worst


def check_torch_autograd(L, renorm=1):
    """torch float64 autograd of the dense masked formulation."""
    import torch
    t = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    x, Wg, W1, W2 = t(L["x"]), t(L["Wg"]), t(L["W1"]), t(L["W2"])
    W3 = t(L["W3"]) if L["act"] == "swiglu" else None
    bias = None if L["bias"] is None else torch.tensor(
        np.asarray(L["bias"], np.float64))
    logits = x @ Wg + (0 if bias is None else bias)
    fw = oracle.layer_forward(*(np.asarray(L[n], np.float64) if L[n] is not None
                                else None for n in ("x", "Wg", "W1", "W2", "W3")),
                              k=L["k"], act=L["act"], bias=L["bias"],
                              renorm=renorm, exact_logits=True)
    idx = torch.tensor(fw["idx"].astype(np.int64))
    if renorm:
        w = torch.softmax(torch.gather(logits, 1, idx), dim=1)
    else:
        w = torch.gather(torch.softmax(logits, dim=1), 1, idx)
    T, E = logits.shape
    mask = torch.zeros(T, E, dtype=torch.float64)
    wfull = mask.scatter(1, idx, w)
    y = torch.zeros_like(x)
    for e in range(E):
        h = x @ W1[e]
        if L["act"] == "gelu":
            a = torch.nn.functional.gelu(h)
        else:
            a = torch.nn.functional.silu(h) * (x @ W3[e])
        y = y + wfull[:, e:e + 1] * (a @ W2[e])
    dy = torch.tensor(np.asarray(L["dy"], np.float64))
    (y * dy).sum().backward()
    gr = oracle.layer_backward(fw, L["dy"], *(np.asarray(L[n], np.float64)
                                              if L[n] is not None else None
                                              for n in ("x", "Wg", "W1", "W2",
                                                        "W3")),
                               act=L["act"], renorm=renorm)
    worst = rel_err(fw["y"], y.detach().numpy())
    pairs = [("dx", x), ("dWg", Wg), ("dW1", W1), ("dW2", W2)]
    if W3 is not None:
        pairs.append(("dW3", W3))
    for gn, tv in pairs:
        worst = max(worst, rel_err(gr[gn], tv.grad.numpy()))
    return worst


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def check_golden_hand_example():
    """Returns the max abs deviation from the hand-worked values."""
    G = load_golden("hand_worked_top2_gelu.json")
    I, X = G["inputs"], G["expected"]
    f = lambda a: np.array(a, dtype=np.float32)
    x, Wg, W1, W2 = f(I["x"]), f(I["Wg"]), f(I["W1"]), f(I["W2"])
    fw = oracle.layer_forward(x, Wg, W1, W2, None, k=I["k"], act="gelu",
                              renorm=I["renorm"])
    gr = oracle.layer_backward(fw, f(I["dy"]), x, Wg, W1, W2, None,
                               act="gelu", renorm=I["renorm"])
    worst = 0.0
    for name in ("idx", "counts", "offsets", "dest", "src"):
        key = {"idx": "topk_idx"}.get(name, name)
        if not np.array_equal(np.asarray(fw[name]), np.array(X[key])):
            return float("inf")
    worst = max(worst, float(np.abs(fw["logits"] - np.array(X["logits"])).max()))
    for mine, key in ((fw["w"], "topk_w"), (fw["out_perm"], "out_perm"),
                      (fw["y"], "y"), (gr["d_out_perm"], "d_out_perm"),
                      (gr["dw"], "d_topk_w"), (gr["dx_perm"], "dx_perm"),
                      (gr["dx_unperm"], "dx_unperm"), (gr["dlogits"], "dlogits"),
                      (gr["dWg"], "dWg"), (gr["dx"], "dx"), (gr["dW1"], "dW1"),
                      (gr["dW2"], "dW2")):
        worst = max(worst, float(np.abs(np.asarray(mine, np.float64)
                                        - np.array(X[key], np.float64)).max()))
    return worst


def all_small_layers():
    """Small layers spanning top-1/2/3, GeLU/SwiGLU, bias on/off."""
    out = []
    for seed, (T, d, f, E, k, act, bias) in enumerate(itertools.chain(
            [(7, 4, 6, 3, 2, "gelu", False), (9, 5, 4, 4, 1, "gelu", True),
             (6, 3, 5, 5, 3, "swiglu", True), (8, 4, 4, 1, 1, "gelu", False),
             (10, 6, 3, 4, 4, "swiglu", False)])):
        out.append(rand_layer(100 + seed, T, d, f, E, k, act, bias))
    return out
