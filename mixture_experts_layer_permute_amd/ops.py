"""Thin torch-tensor wrappers over the C entry points (marshalling only).

Shapes and meanings are those of include/moe.h.  Outputs not passed in are
allocated with torch on the inputs' device; workspaces likewise.  All calls
are asynchronous on torch's current HIP stream.
"""
import torch

from ._lib import (MOE_ACT_GELU, MOE_ACT_SWIGLU, MOE_BF16, MOE_F32, MoEError,
                   check, load)

_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}


def _dt(t):
    try:
        return _DT[t.dtype]
    except KeyError:
        raise MoEError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _p(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise MoEError("libmoe takes device tensors only")
        if t is not None and not t.is_contiguous():
            raise MoEError("libmoe takes contiguous tensors only")


def _act(act):
    if act in (MOE_ACT_GELU, "gelu"):
        return MOE_ACT_GELU
    if act in (MOE_ACT_SWIGLU, "swiglu"):
        return MOE_ACT_SWIGLU
    raise MoEError("unknown activation %r" % (act,))


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def moe_init(device=0):
    check(load().moe_init(int(device)), "moe_init")


def moe_set_overlap(enable=True):
    """Let the FFN backward run independent launches on a side stream (default)."""
    check(load().moe_set_overlap(1 if enable else 0), "moe_set_overlap")


def moe_gate_topk(x, Wg, k, logit_bias=None, renorm=1, logits=None,
                  topk_idx=None, topk_w=None):
    """-> (logits [T,E] f32, topk_idx [T,k] i32, topk_w [T,k] f32)."""
    _need_gpu(x, Wg, logit_bias)
    T, d = x.shape
    E = Wg.shape[1]
    dev = x.device
    if logits is None:
        logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty(T, k, dtype=torch.float32, device=dev)
    check(load().moe_gate_topk(_p(x), _p(Wg), _p(logit_bias), T, d, E, k, renorm,
                               _dt(x), _p(logits), _p(topk_idx), _p(topk_w),
                               _stream(dev)), "moe_gate_topk")
    return logits, topk_idx, topk_w


def moe_permute(topk_idx, x, E, out=None, ws=None, copy=True):
    """-> (counts [E], offsets [E+1], dest [T,k], src [T*k], x_perm [T*k,d]);
    copy=False: routing only, x_perm is None (for the *_gather FFN calls)."""
    _need_gpu(topk_idx, x)
    T, k = topk_idx.shape
    d = x.shape[1]
    dev = x.device
    L = load()
    if out is None:
        out = (torch.empty(E, dtype=torch.int32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(T, k, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev),
               torch.empty(T * k, d, dtype=x.dtype, device=dev) if copy else None)
    counts, offsets, dest, src, x_perm = out
    nb = L.moe_permute_workspace_bytes(T, E, k)
    if ws is None:
        ws = _ws(nb, dev)
    check(L.moe_permute(_p(topk_idx), _p(x), T, d, E, k, _dt(x), _p(counts),
                        _p(offsets), _p(dest), _p(src), _p(x_perm), _p(ws),
                        ws.numel(), _stream(dev)), "moe_permute")
    return counts, offsets, dest, src, x_perm


def moe_expert_ffn_fwd(x_perm, offsets, W1, W2, W3=None, act="gelu", out=None,
                       ws=None):
    """-> (h_save, a_save [R,f], out_perm [R,d]); h_save is the state the
    backward needs: GeLU'(H) [R,f], or [H3 SiLU'(H1) | SiLU(H1)] [R,2f]."""
    _need_gpu(x_perm, offsets, W1, W2, W3)
    a = _act(act)
    R, d = x_perm.shape
    E, _, f = W1.shape
    dev = x_perm.device
    L = load()
    if out is None:
        hw = 2 * f if a == MOE_ACT_SWIGLU else f
        out = (torch.empty(R, hw, dtype=x_perm.dtype, device=dev),
               torch.empty(R, f, dtype=x_perm.dtype, device=dev),
               torch.empty(R, d, dtype=x_perm.dtype, device=dev))
    h_save, a_save, out_perm = out
    if ws is None:
        ws = _ws(L.moe_ffn_workspace_bytes(R, E, d, f, a, _dt(x_perm), 0), dev)
    check(L.moe_expert_ffn_fwd(_p(x_perm), _p(offsets), R, E, d, f, a,
                               _dt(x_perm), _p(W1), _p(W3), _p(W2), _p(h_save),
                               _p(a_save), _p(out_perm), _p(ws), ws.numel(),
                               _stream(dev)), "moe_expert_ffn_fwd")
    return h_save, a_save, out_perm


def moe_expert_ffn_fwd_noalloc(x_perm, offsets, W1, W2, W3=None, act="gelu", out=None):
    """moe_expert_ffn_fwd with the library's static scratch instead of a
    workspace.  -> (h_save, a_save [R,f], out_perm [R,d]); pass ``out`` to
    allocate nothing at all."""
    _need_gpu(x_perm, offsets, W1, W2, W3)
    a = _act(act)
    R, d = x_perm.shape
    E, _, f = W1.shape
    dev = x_perm.device
    if out is None:
        hw = 2 * f if a == MOE_ACT_SWIGLU else f
        out = (torch.empty(R, hw, dtype=x_perm.dtype, device=dev),
               torch.empty(R, f, dtype=x_perm.dtype, device=dev),
               torch.empty(R, d, dtype=x_perm.dtype, device=dev))
    h_save, a_save, out_perm = out
    check(load().moe_expert_ffn_fwd_noalloc(_p(x_perm), _p(offsets), R, E, d, f, a,
                                            _dt(x_perm), _p(W1), _p(W3), _p(W2),
                                            _p(h_save), _p(a_save), _p(out_perm),
                                            _stream(dev)), "moe_expert_ffn_fwd_noalloc")
    return h_save, a_save, out_perm


def moe_expert_ffn_bwd(d_out_perm, x_perm, h_save, a_save, offsets, W1, W2,
                       W3=None, act="gelu", out=None, ws=None):
    """-> (dx_perm [R,d], dW1 [E,d,f], dW3 or None, dW2 [E,f,d])."""
    _need_gpu(d_out_perm, x_perm, h_save, a_save, offsets, W1, W2, W3)
    a = _act(act)
    R, d = x_perm.shape
    E, _, f = W1.shape
    dev = x_perm.device
    L = load()
    if out is None:
        out = (torch.empty(R, d, dtype=x_perm.dtype, device=dev),
               torch.empty_like(W1),
               torch.empty_like(W3) if a == MOE_ACT_SWIGLU else None,
               torch.empty_like(W2))
    dx_perm, dW1, dW3, dW2 = out
    if ws is None:
        ws = _ws(L.moe_ffn_workspace_bytes(R, E, d, f, a, _dt(x_perm), 1), dev)
    check(L.moe_expert_ffn_bwd(_p(d_out_perm), _p(x_perm), _p(h_save),
                               _p(a_save), _p(offsets), R, E, d, f, a,
                               _dt(x_perm), _p(W1), _p(W3), _p(W2), _p(dx_perm),
                               _p(dW1), _p(dW3), _p(dW2), _p(ws), ws.numel(),
                               _stream(dev)), "moe_expert_ffn_bwd")
    return dx_perm, dW1, dW3, dW2


def moe_expert_ffn_fwd_gather(x, src, offsets, W1, W2, W3=None, act="gelu",
                              out=None, ws=None):
    """moe_expert_ffn_fwd reading permuted row r as x[src[r]] (no x_perm).
    -> (h_save, a_save [R,f], out_perm [R,d]), R = src.numel()."""
    _need_gpu(x, src, offsets, W1, W2, W3)
    a = _act(act)
    T, d = x.shape
    R = src.numel()
    E, _, f = W1.shape
    dev = x.device
    L = load()
    if out is None:
        hw = 2 * f if a == MOE_ACT_SWIGLU else f
        out = (torch.empty(R, hw, dtype=x.dtype, device=dev),
               torch.empty(R, f, dtype=x.dtype, device=dev),
               torch.empty(R, d, dtype=x.dtype, device=dev))
    h_save, a_save, out_perm = out
    if ws is None:
        ws = _ws(L.moe_ffn_workspace_bytes(R, E, d, f, a, _dt(x), 0), dev)
    check(L.moe_expert_ffn_fwd_gather(_p(x), _p(src), _p(offsets), T, R, E, d, f, a,
                                      _dt(x), _p(W1), _p(W3), _p(W2), _p(h_save),
                                      _p(a_save), _p(out_perm), _p(ws), ws.numel(),
                                      _stream(dev)), "moe_expert_ffn_fwd_gather")
    return h_save, a_save, out_perm


def moe_expert_ffn_bwd_gather(d_out_perm, x, src, h_save, a_save, offsets, W1, W2,
                              W3=None, act="gelu", out=None, ws=None):
    """moe_expert_ffn_bwd reading permuted row r as x[src[r]] (no x_perm).
    -> (dx_perm [R,d], dW1 [E,d,f], dW3 or None, dW2 [E,f,d])."""
    _need_gpu(d_out_perm, x, src, h_save, a_save, offsets, W1, W2, W3)
    a = _act(act)
    T, d = x.shape
    R = src.numel()
    E, _, f = W1.shape
    dev = x.device
    L = load()
    if out is None:
        out = (torch.empty(R, d, dtype=x.dtype, device=dev),
               torch.empty_like(W1),
               torch.empty_like(W3) if a == MOE_ACT_SWIGLU else None,
               torch.empty_like(W2))
    dx_perm, dW1, dW3, dW2 = out
    if ws is None:
        ws = _ws(L.moe_ffn_workspace_bytes(R, E, d, f, a, _dt(x), 1), dev)
    check(L.moe_expert_ffn_bwd_gather(_p(d_out_perm), _p(x), _p(src), _p(h_save),
                                      _p(a_save), _p(offsets), T, R, E, d, f, a, _dt(x),
                                      _p(W1), _p(W3), _p(W2), _p(dx_perm), _p(dW1),
                                      _p(dW3), _p(dW2), _p(ws), ws.numel(),
                                      _stream(dev)), "moe_expert_ffn_bwd_gather")
    return dx_perm, dW1, dW3, dW2


def moe_combine(out_perm, dest, topk_w, y=None):
    """-> y [T,d]."""
    _need_gpu(out_perm, dest, topk_w)
    T, k = dest.shape
    d = out_perm.shape[1]
    if y is None:
        y = torch.empty(T, d, dtype=out_perm.dtype, device=out_perm.device)
    check(load().moe_combine(_p(out_perm), _p(dest), _p(topk_w), T, k, d,
                             _dt(out_perm), _p(y), _stream(out_perm.device)),
          "moe_combine")
    return y


def moe_combine_bwd(dy, out_perm, dest, topk_w, out=None):
    """-> (d_out_perm [T*k,d], d_topk_w [T,k] f32)."""
    _need_gpu(dy, out_perm, dest, topk_w)
    T, k = dest.shape
    d = dy.shape[1]
    dev = dy.device
    if out is None:
        out = (torch.empty(T * k, d, dtype=dy.dtype, device=dev),
               torch.empty(T, k, dtype=torch.float32, device=dev))
    d_out, dw = out
    check(load().moe_combine_bwd(_p(dy), _p(out_perm), _p(dest), _p(topk_w), T, k,
                                 d, _dt(dy), _p(d_out), _p(dw), _stream(dev)),
          "moe_combine_bwd")
    return d_out, dw


def moe_unpermute_grad(dx_perm, dest, dx=None, accumulate=0):
    """-> dx [T,d] (overwritten, or accumulated into when accumulate=1)."""
    _need_gpu(dx_perm, dest)
    T, k = dest.shape
    d = dx_perm.shape[1]
    if dx is None:
        dx = torch.empty(T, d, dtype=dx_perm.dtype, device=dx_perm.device)
    check(load().moe_unpermute_grad(_p(dx_perm), _p(dest), T, k, d, _dt(dx_perm),
                                    _p(dx), int(accumulate),
                                    _stream(dx_perm.device)), "moe_unpermute_grad")
    return dx


def moe_gate_topk_bwd(x, Wg, logits, topk_idx, topk_w, d_topk_w, dx, renorm=1,
                      dWg=None, ws=None, accumulate=True):
    """dx += dl Wg^T in place (dx = dl Wg^T with accumulate=False); -> dWg [d,E]."""
    _need_gpu(x, Wg, logits, topk_idx, topk_w, d_topk_w, dx)
    T, d = x.shape
    E = Wg.shape[1]
    k = topk_idx.shape[1]
    dev = x.device
    L = load()
    if dWg is None:
        dWg = torch.empty_like(Wg)
    if ws is None:
        ws = _ws(L.moe_gate_bwd_workspace_bytes(T, d, E), dev)
    check(L.moe_gate_topk_bwd(_p(x), _p(Wg), _p(logits), _p(topk_idx), _p(topk_w),
                              _p(d_topk_w), T, d, E, k, renorm, _dt(x), _p(dx),
                              int(bool(accumulate)), _p(dWg), _p(ws), ws.numel(),
                              _stream(dev)),
          "moe_gate_topk_bwd")
    return dWg
