"""CPU oracle of the MoE layer forward and backward -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this module.  It shares no code with the HIP library: it
computes the plain definition of each step, slowly and visibly, in float64
(the gate logits alone are fp32 in a fixed order, because they decide the
integer routing; see ``gate_logits``).

The method (sources, by page and section):

* gate -> expert choice: ES-MoE review (xllm-io), 三 技术架构 /
  专家级卸载与处理 -- expert placement is only known after the gating network
  has run.  No gate formula is printed; reading: linear gate, top-k by logit,
  softmax weights over the selected k (GShard / Switch Transformer are the
  expert-parallel lineage named in 六 相关工作), no noise, no capacity factor,
  no token dropping, no auxiliary loss (the review lists those as the
  alternatives ES-MoE avoids, 六 相关工作, and wants zero padding removed,
  三 技术架构 / 自适应卸载).
* permutation: ES-MoE review, 三 技术架构 / 专家级卸载与处理 and 四 核心创新 --
  tokens are handed to their target experts in sequence, with no batched
  matmul over a dense dispatch mask; FastMoE review, 제안 방법 -- a
  scatter/gather layout batches the inputs of each expert together.
  Reading: a stable counting sort of (token, slot) pairs by expert, giving
  contiguous unpadded per-expert segments ordered by token index.
* expert FFN per segment: FastMoE review, 제안 방법 -- a dedicated expert FFN
  with a linear module that runs the experts' linear layers in parallel.
  Reading: GeLU experts A = GeLU(X W1), O = A W2 (exact erf GeLU); SwiGLU
  experts A = SiLU(X W1) * (X W3), O = A W2; no biases.
* combine: the gather back to token order weighted by the gate,
  y[t] = sum_j w[t,j] O[dest[t,j]], summed in slot order.
* backward: the exact derivative of the above (the long-context MoE paper,
  abstract, holds that reordering computation and data movement leaves loss
  and gradients exact -- the permuted layer must equal the dense masked one).

Pins (tests/test_oracle_*.py) tie every function to something other than
itself: a dense all-experts masked brute force, brute-force counting sort,
closed-form hand examples (tests/golden/), the recursive-summation error
bound, central finite differences and torch CPU autograd.
"""
import ctypes

import numpy as np

from . import _cbuild

F64 = np.float64


# ------------------------------------------------------------------- gate

def gate_logits(x, Wg, bias=None):
    """fp32 gate logits in fixed order (C helper, multi-threaded over t).

    l[t,e] = (sum_{i=0..d-1} x[t,i]*Wg[i,e], accumulated left to right in
    fp32, every product and sum rounded, no FMA) + bias[e] (also fp32).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    Wg = np.ascontiguousarray(Wg, dtype=np.float32)
    T, d = x.shape
    E = Wg.shape[1]
    out = np.empty((T, E), dtype=np.float32)
    fp = ctypes.POINTER(ctypes.c_float)
    b = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        b = bias.ctypes.data_as(fp)
    _cbuild.lib().oracle_gate_logits_f32(
        x.ctypes.data_as(fp), Wg.ctypes.data_as(fp), b, T, d, E,
        out.ctypes.data_as(fp))
    return out


def gate_logits_numpy(x, Wg, bias=None):
    """The same definition as ``gate_logits`` written with NumPy fp32 ops."""
    x = np.asarray(x, dtype=np.float32)
    Wg = np.asarray(Wg, dtype=np.float32)
    acc = np.zeros((x.shape[0], Wg.shape[1]), dtype=np.float32)
    for i in range(x.shape[1]):
        p = x[:, i:i + 1] * Wg[i:i + 1, :]         # fp32 product, rounded
        acc = acc + p                              # fp32 sum, rounded
    if bias is not None:
        acc = acc + np.asarray(bias, dtype=np.float32)[None, :]
    return acc


def gate_logits_f64(x, Wg, bias=None):
    """Exact-arithmetic logits (float64), for finite differences and bounds."""
    l = np.asarray(x, F64) @ np.asarray(Wg, F64)
    if bias is not None:
        l = l + np.asarray(bias, F64)[None, :]
    return l


def topk_select(logits, k):
    """Indices of the k largest logits per token, best first.

    Selection compares logits (not probabilities).  Equal logits: the lower
    expert index wins.  Slot j holds the j-th best.
    """
    order = np.argsort(-np.asarray(logits), axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def gate_weights(logits, idx, renorm=1):
    """Gate weights of the selected experts, float64 [T,k].

    renorm=1: softmax over the k selected logits (the full softmax
    renormalised over the top-k), w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0).
    renorm=0: full softmax over all E logits, read at the selected experts.
    """
    l = np.asarray(logits, F64)
    sel = np.take_along_axis(l, idx.astype(np.int64), axis=1)
    if renorm:
        z = np.exp(sel - sel[:, :1])
        return z / z.sum(axis=1, keepdims=True)
    m = l.max(axis=1, keepdims=True)
    den = np.exp(l - m).sum(axis=1, keepdims=True)
    return np.exp(sel - m) / den


# ---------------------------------------------------------------- permute

def permute(idx, E):
    """Stable counting sort of the (token, slot) pairs by expert.

    Returns counts[E], offsets[E+1] (exclusive prefix sum, offsets[E] = T*k),
    dest[T,k] (row of pair (t,j) in the permuted layout) and src[T*k] (token
    of each permuted row).  Inside a segment rows are ordered by token
    index; a token's k experts are distinct, so slot order never ties.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")          # stable sort by expert
    src = (order // k).astype(np.int32)
    dest = np.empty(T * k, dtype=np.int32)
    dest[order] = np.arange(T * k, dtype=np.int32)
    return counts, offsets, dest.reshape(T, k), src


def dispatch_rows(x, src):
    """x_perm[r] = x[src[r]]: the token rows in expert-segment order."""
    return np.asarray(x)[np.asarray(src, dtype=np.int64)]


# ------------------------------------------------------------- activations

def _erf(z):
    from scipy.special import erf
    return erf(z)


def gelu(z):
    """Exact GeLU, z * Phi(z) = z/2 * (1 + erf(z / sqrt 2))."""
    z = np.asarray(z, F64)
    return 0.5 * z * (1.0 + _erf(z / np.sqrt(2.0)))


def gelu_grad(z):
    """d GeLU / dz = Phi(z) + z * phi(z)."""
    z = np.asarray(z, F64)
    cdf = 0.5 * (1.0 + _erf(z / np.sqrt(2.0)))
    pdf = np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)
    return cdf + z * pdf


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    z = np.asarray(z, F64)
    return z * _sigmoid(z)


def silu_grad(z):
    """d SiLU / dz = s(z) * (1 + z * (1 - s(z)))."""
    z = np.asarray(z, F64)
    s = _sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


# ------------------------------------------------------------- expert FFN

def ffn_fwd_segment(xs, W1e, W2e, W3e=None, act="gelu"):
    """One expert on its rows.  Returns (H, H3 or None, A, O), float64."""
    xs = np.asarray(xs, F64)
    H = xs @ np.asarray(W1e, F64)
    if act == "gelu":
        H3 = None
        A = gelu(H)
    else:
        H3 = xs @ np.asarray(W3e, F64)
        A = silu(H) * H3
    O = A @ np.asarray(W2e, F64)
    return H, H3, A, O


def ffn_bwd_segment(dO, xs, W1e, W2e, W3e=None, act="gelu", saved=None):
    """Gradients of one expert: (dX, dW1, dW3 or None, dW2), float64.

    ``saved`` may pass (H, H3, A) from the forward to skip recomputation.
    """
    dO = np.asarray(dO, F64)
    xs = np.asarray(xs, F64)
    if saved is None:
        H, H3, A, _ = ffn_fwd_segment(xs, W1e, W2e, W3e, act)
    else:
        H, H3, A = saved
    W1e = np.asarray(W1e, F64)
    W2e = np.asarray(W2e, F64)
    dA = dO @ W2e.T
    dW2 = A.T @ dO
    if act == "gelu":
        dH = dA * gelu_grad(H)
        dW1 = xs.T @ dH
        dX = dH @ W1e.T
        return dX, dW1, None, dW2
    W3e = np.asarray(W3e, F64)
    dH1 = dA * H3 * silu_grad(H)
    dH3 = dA * silu(H)
    dW1 = xs.T @ dH1
    dW3 = xs.T @ dH3
    dX = dH1 @ W1e.T + dH3 @ W3e.T
    return dX, dW1, dW3, dW2


def ffn_bwd_columns(dO, xs, W1e, W2e, W3e=None, act="gelu", cols=None):
    """Weight gradients of one expert restricted to hidden units ``cols``.

    Hidden unit c of an expert touches only column c of W1 (and W3) and row c
    of W2, so dW1[:, c], dW3[:, c] and dW2[c, :] follow from the expert's
    rows exactly as in ``ffn_bwd_segment`` without forming the other units.
    Returns (dW1[:, cols], dW3[:, cols] or None, dW2[cols, :]), float64.
    """
    cols = np.asarray(cols, dtype=np.int64)
    dO = np.asarray(dO, F64)
    xs = np.asarray(xs, F64)
    H = xs @ np.asarray(W1e, F64)[:, cols]
    dA = dO @ np.asarray(W2e, F64)[cols, :].T
    if act == "gelu":
        A = gelu(H)
        dH = dA * gelu_grad(H)
        return xs.T @ dH, None, A.T @ dO
    H3 = xs @ np.asarray(W3e, F64)[:, cols]
    A = silu(H) * H3
    dH1 = dA * H3 * silu_grad(H)
    dH3 = dA * silu(H)
    return xs.T @ dH1, xs.T @ dH3, A.T @ dO


def _w(W, e):
    """Expert e's matrix from a stacked array or a mapping/callable."""
    if W is None:
        return None
    if callable(W):
        return W(e)
    return W[e]


def expert_ffn_fwd(x_perm, offsets, W1, W2, W3=None, act="gelu",
                   experts=None):
    """Per-segment FFN over the permuted rows.

    Returns dict with H [R,f], H3 [R,f] (SwiGLU) or None, A [R,f] and
    out [R,d] (float64).  With ``experts`` given, only those segments are
    computed and the other rows are left NaN.
    """
    x_perm = np.asarray(x_perm)
    R = x_perm.shape[0]
    E = len(offsets) - 1
    f = np.asarray(_w(W1, 0 if experts is None else experts[0])).shape[1]
    d = x_perm.shape[1]
    H = np.full((R, f), np.nan)
    H3 = np.full((R, f), np.nan) if act == "swiglu" else None
    A = np.full((R, f), np.nan)
    O = np.full((R, d), np.nan)
    for e in (range(E) if experts is None else experts):
        a, b = int(offsets[e]), int(offsets[e + 1])
        h, h3, aa, o = ffn_fwd_segment(x_perm[a:b], _w(W1, e), _w(W2, e),
                                       _w(W3, e), act)
        H[a:b] = h
        A[a:b] = aa
        O[a:b] = o
        if H3 is not None:
            H3[a:b] = h3
    return {"H": H, "H3": H3, "A": A, "out": O}


def expert_ffn_bwd(d_out_perm, x_perm, offsets, W1, W2, W3=None, act="gelu",
                   experts=None):
    """Per-segment FFN backward.  A zero-row expert gets dW = 0."""
    d_out_perm = np.asarray(d_out_perm)
    R, d = d_out_perm.shape
    E = len(offsets) - 1
    f = np.asarray(_w(W1, 0 if experts is None else experts[0])).shape[1]
    dXp = np.full((R, d), np.nan)
    dW1, dW3, dW2 = {}, {}, {}
    for e in (range(E) if experts is None else experts):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            dW1[e] = np.zeros((d, f))
            dW2[e] = np.zeros((f, d))
            if act == "swiglu":
                dW3[e] = np.zeros((d, f))
            continue
        dx, w1, w3, w2 = ffn_bwd_segment(d_out_perm[a:b], x_perm[a:b],
                                         _w(W1, e), _w(W2, e), _w(W3, e), act)
        dXp[a:b] = dx
        dW1[e] = w1
        dW2[e] = w2
        if act == "swiglu":
            dW3[e] = w3
    return {"dx_perm": dXp, "dW1": dW1, "dW3": dW3 if act == "swiglu" else None,
            "dW2": dW2}


# ---------------------------------------------------------------- combine

def combine(out_perm, dest, w):
    """y[t] = sum_j w[t,j] * out_perm[dest[t,j]], in slot order."""
    out_perm = np.asarray(out_perm, F64)
    dest = np.asarray(dest, dtype=np.int64)
    w = np.asarray(w, F64)
    T, k = dest.shape
    y = np.zeros((T, out_perm.shape[1]))
    for j in range(k):
        y = y + w[:, j:j + 1] * out_perm[dest[:, j]]
    return y


def combine_bwd(dy, out_perm, dest, w):
    """d_out_perm[dest[t,j]] = w[t,j] dy[t];  dw[t,j] = <dy[t], out_perm[dest[t,j]]>."""
    dy = np.asarray(dy, F64)
    out_perm = np.asarray(out_perm, F64)
    dest = np.asarray(dest, dtype=np.int64)
    w = np.asarray(w, F64)
    T, k = dest.shape
    d_out = np.zeros_like(out_perm)
    dw = np.zeros((T, k))
    for j in range(k):
        d_out[dest[:, j]] = w[:, j:j + 1] * dy
        dw[:, j] = np.einsum("td,td->t", dy, out_perm[dest[:, j]])
    return d_out, dw


def unpermute_grad(dx_perm, dest):
    """dx[t] = sum_j dx_perm[dest[t,j]]: the permutation's backward."""
    dx_perm = np.asarray(dx_perm, F64)
    dest = np.asarray(dest, dtype=np.int64)
    dx = np.zeros((dest.shape[0], dx_perm.shape[1]))
    for j in range(dest.shape[1]):
        dx = dx + dx_perm[dest[:, j]]
    return dx


# --------------------------------------------------------------- gate bwd

def gate_logits_grad(logits, idx, w, dw, renorm=1):
    """dL/dl [T,E] from the gradient dw of the selected weights.

    renorm=1: dl[t, idx_j] = w_j (dw_j - sum_j' w_j' dw_j'), zero elsewhere.
    renorm=0: dl[t, e] = p_e (g_e - sum_j w_j dw_j), p = softmax over all E,
    g_e = dw_j where e = idx_j, else 0.
    """
    w = np.asarray(w, F64)
    dw = np.asarray(dw, F64)
    T, E = np.asarray(logits).shape
    s = (w * dw).sum(axis=1, keepdims=True)
    dl = np.zeros((T, E))
    rows = np.arange(T)[:, None]
    if renorm:
        dl[rows, idx] = w * (dw - s)
        return dl
    l = np.asarray(logits, F64)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    g = np.zeros((T, E))
    g[rows, idx] = dw
    return p * (g - s)


def gate_bwd(x, Wg, logits, idx, w, dw, renorm=1):
    """(dl, dWg = x^T dl, dx_gate = dl Wg^T).  The workload bias gets no grad."""
    dl = gate_logits_grad(logits, idx, w, dw, renorm)
    dWg = np.asarray(x, F64).T @ dl
    dxg = dl @ np.asarray(Wg, F64).T
    return dl, dWg, dxg


# ------------------------------------------------------------- whole layer

def layer_forward(x, Wg, W1, W2, W3=None, *, k, act="gelu", bias=None,
                  renorm=1, exact_logits=False, idx=None, experts=None):
    """Gate -> permute -> expert FFN -> combine.  Returns a dict of all parts.

    exact_logits: use float64 logits (finite-difference checks).  idx: force
    the routing (frozen selection for finite differences).
    """
    E = np.asarray(Wg).shape[1] if not callable(Wg) else None
    if exact_logits:
        logits = gate_logits_f64(x, Wg, bias)
    else:
        logits = gate_logits(x, Wg, bias)
    if idx is None:
        idx = topk_select(logits, k)
    w = gate_weights(logits, idx, renorm)
    counts, offsets, dest, src = permute(idx, E)
    x_perm = dispatch_rows(x, src)
    ffn = expert_ffn_fwd(x_perm, offsets, W1, W2, W3, act, experts)
    y = combine(ffn["out"], dest, w) if experts is None else None
    return dict(logits=logits, idx=idx, w=w, counts=counts, offsets=offsets,
                dest=dest, src=src, x_perm=x_perm, H=ffn["H"], H3=ffn["H3"],
                A=ffn["A"], out_perm=ffn["out"], y=y)


def layer_backward(fw, dy, x, Wg, W1, W2, W3=None, *, act="gelu", renorm=1):
    """Full backward from the forward dict ``fw``.  Returns all gradients."""
    d_out, dw = combine_bwd(dy, fw["out_perm"], fw["dest"], fw["w"])
    g = expert_ffn_bwd(d_out, fw["x_perm"], fw["offsets"], W1, W2, W3, act)
    dx = unpermute_grad(g["dx_perm"], fw["dest"])
    dl, dWg, dxg = gate_bwd(x, Wg, fw["logits"], fw["idx"], fw["w"], dw,
                            renorm)
    E = len(fw["offsets"]) - 1
    stack = (lambda m: np.stack([m[e] for e in range(E)]))
    return dict(d_out_perm=d_out, dw=dw, dx_perm=g["dx_perm"],
                dx_unperm=dx, dx=dx + dxg, dlogits=dl, dWg=dWg,
                dW1=stack(g["dW1"]), dW2=stack(g["dW2"]),
                dW3=stack(g["dW3"]) if act == "swiglu" else None)
