"""MoELayer: every buffer of one layer shape allocated once, and the eight C
entry points chained into a forward and a backward pass.

forward:  moe_gate_topk -> moe_permute -> moe_expert_ffn_fwd -> moe_combine
backward: moe_combine_bwd -> moe_expert_ffn_bwd -> moe_unpermute_grad
          -> moe_gate_topk_bwd
"""
import torch

from ._lib import MOE_ACT_GELU, MOE_ACT_SWIGLU, MOE_BF16, MOE_F32, check, load
from .ops import _stream


class MoELayer:
    def __init__(self, T, d, f, E, k, act="gelu", dtype=torch.bfloat16,
                 renorm=1, device="cuda", fuse_gather=False):
        """fuse_gather: no x_perm buffer; the permute only routes and the FFN
        calls read rows of x through src (moe_expert_ffn_*_gather)."""
        self.T, self.d, self.f, self.E, self.k = T, d, f, E, k
        self.fuse_gather = bool(fuse_gather)
        self.act = MOE_ACT_SWIGLU if act == "swiglu" else MOE_ACT_GELU
        self.dtype = dtype
        self.dt = MOE_BF16 if dtype == torch.bfloat16 else MOE_F32
        self.renorm = renorm
        self.device = torch.device(device)
        L = self.lib = load()
        R = self.R = T * k
        dev = self.device
        e = lambda *s, dt=dtype: torch.empty(*s, dtype=dt, device=dev)
        i32, f32 = torch.int32, torch.float32
        hw = 2 * f if self.act == MOE_ACT_SWIGLU else f
        # forward activations
        self.logits = e(T, E, dt=f32)
        self.topk_idx = e(T, k, dt=i32)
        self.topk_w = e(T, k, dt=f32)
        self.counts = e(E, dt=i32)
        self.offsets = e(E + 1, dt=i32)
        self.dest = e(T, k, dt=i32)
        self.src = e(R, dt=i32)
        self.x_perm = None if self.fuse_gather else e(R, d)
        self.h_save = e(R, hw)
        self.a_save = e(R, f)
        self.out_perm = e(R, d)
        self.y = e(T, d)
        # backward
        self.d_out_perm = e(R, d)
        self.d_topk_w = e(T, k, dt=f32)
        self.dx_perm = e(R, d)
        self.dx = e(T, d)
        self.dW1 = e(E, d, f)
        self.dW3 = e(E, d, f) if self.act == MOE_ACT_SWIGLU else None
        self.dW2 = e(E, f, d)
        self.dWg = e(d, E)
        ws = lambda n: torch.empty(max(int(n), 1), dtype=torch.uint8, device=dev)
        self.ws_perm = ws(L.moe_permute_workspace_bytes(T, E, k))
        self.ws_ffn_f = ws(L.moe_ffn_workspace_bytes(R, E, d, f, self.act, self.dt, 0))
        self.ws_ffn_b = ws(L.moe_ffn_workspace_bytes(R, E, d, f, self.act, self.dt, 1))
        self.ws_gate = ws(L.moe_gate_bwd_workspace_bytes(T, d, E))

    def bind(self, x, Wg, W1, W2, W3=None, logit_bias=None, dy=None):
        """Remember the input tensors (device, contiguous, layer dtype)."""
        for t in (x, Wg, W1, W2, W3, dy):
            if t is not None:
                assert t.is_cuda and t.is_contiguous() and t.dtype == self.dtype
        self.x, self.Wg, self.W1, self.W2, self.W3 = x, Wg, W1, W2, W3
        self.bias = logit_bias
        self.dy = dy
        p = lambda t: None if t is None else t.data_ptr()
        T, d, f, E, k, R, dt, a = (self.T, self.d, self.f, self.E, self.k, self.R,
                                   self.dt, self.act)
        self._fwd = [
            ("moe_gate_topk", (p(x), p(Wg), p(logit_bias), T, d, E, k, self.renorm,
                               dt, p(self.logits), p(self.topk_idx), p(self.topk_w))),
            ("moe_permute", (p(self.topk_idx), p(x), T, d, E, k, dt, p(self.counts),
                             p(self.offsets), p(self.dest), p(self.src),
                             p(self.x_perm), p(self.ws_perm), self.ws_perm.numel())),
            ("moe_expert_ffn_fwd_gather", (p(x), p(self.src), p(self.offsets), T, R, E, d,
                                           f, a, dt, p(W1), p(W3), p(W2), p(self.h_save),
                                           p(self.a_save), p(self.out_perm),
                                           p(self.ws_ffn_f), self.ws_ffn_f.numel()))
            if self.fuse_gather else
            ("moe_expert_ffn_fwd", (p(self.x_perm), p(self.offsets), R, E, d, f, a, dt,
                                    p(W1), p(W3), p(W2), p(self.h_save),
                                    p(self.a_save), p(self.out_perm),
                                    p(self.ws_ffn_f), self.ws_ffn_f.numel())),
            ("moe_combine", (p(self.out_perm), p(self.dest), p(self.topk_w), T, k, d,
                             dt, p(self.y))),
        ]
        self._bwd = [
            ("moe_combine_bwd", (p(dy), p(self.out_perm), p(self.dest), p(self.topk_w),
                                 T, k, d, dt, p(self.d_out_perm), p(self.d_topk_w))),
            ("moe_expert_ffn_bwd_gather", (p(self.d_out_perm), p(x), p(self.src),
                                           p(self.h_save), p(self.a_save), p(self.offsets),
                                           T, R, E, d, f, a, dt, p(W1), p(W3), p(W2),
                                           p(self.dx_perm), p(self.dW1), p(self.dW3),
                                           p(self.dW2), p(self.ws_ffn_b),
                                           self.ws_ffn_b.numel()))
            if self.fuse_gather else
            ("moe_expert_ffn_bwd", (p(self.d_out_perm), p(self.x_perm), p(self.h_save),
                                    p(self.a_save), p(self.offsets), R, E, d, f, a, dt,
                                    p(W1), p(W3), p(W2), p(self.dx_perm),
                                    p(self.dW1), p(self.dW3), p(self.dW2),
                                    p(self.ws_ffn_b), self.ws_ffn_b.numel())),
            ("moe_unpermute_grad", (p(self.dx_perm), p(self.dest), T, k, d, dt,
                                    p(self.dx), 0)),
            ("moe_gate_topk_bwd", (p(x), p(Wg), p(self.logits), p(self.topk_idx),
                                   p(self.topk_w), p(self.d_topk_w), T, d, E, k,
                                   self.renorm, dt, p(self.dx), p(self.dWg),
                                   p(self.ws_gate), self.ws_gate.numel())),
        ]
        return self

    def _run(self, calls, stream=None):
        s = _stream(self.device) if stream is None else stream
        L = self.lib
        for name, args in calls:
            check(getattr(L, name)(*args, s), name)

    def forward(self, stream=None):
        self._run(self._fwd, stream)
        return self.y

    def backward(self, stream=None):
        assert self.dy is not None, "bind(dy=...) first"
        self._run(self._bwd, stream)
        return self.dx

    def step(self, stream=None):
        """One forward + backward pass."""
        self._run(self._fwd, stream)
        self._run(self._bwd, stream)

    def stage_calls(self):
        """[(name, callable)] of every entry point of one step, in order."""
        L = self.lib
        return [(n, (lambda n=n, a=a, s=None: check(
            getattr(L, n)(*a, _stream(self.device) if s is None else s), n)))
            for n, a in self._fwd + self._bwd]
