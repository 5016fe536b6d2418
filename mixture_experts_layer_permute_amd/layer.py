"""MoELayer: every buffer of one layer shape allocated once, and the eight C
entry points chained into a forward and a backward pass.

forward:  moe_gate_topk -> moe_permute -> moe_expert_ffn_fwd -> moe_combine
backward: moe_combine_bwd -> (moe_gate_topk_bwd on a second stream, writes
          dx) and moe_expert_ffn_bwd -> moe_unpermute_grad (adds to dx)
"""
import math

import torch

from ._lib import MOE_ACT_GELU, MOE_ACT_SWIGLU, MOE_BF16, MOE_F32, check, load
from .ops import _stream


def _torch_stream(handle, device):
    """torch's stream object for a raw stream handle.  The current and the
    default stream map to torch's own objects: an ExternalStream wrapped
    around handle 0 did not order events against work on the default stream
    (a dx computed on a second stream joined through it raced on the GPU)."""
    cur = torch.cuda.current_stream(device)
    if handle is None or handle == cur.cuda_stream:
        return cur
    dflt = torch.cuda.default_stream(device)
    if handle == dflt.cuda_stream:
        return dflt
    return torch.cuda.ExternalStream(handle, device=device)


class MoELayer:
    def __init__(self, T, d, f, E, k, act="gelu", dtype=torch.bfloat16,
                 renorm=1, device="cuda", fuse_gather=False, overlap_gate=True):
        """fuse_gather: no x_perm buffer; the permute only routes and the FFN
        calls read rows of x through src (moe_expert_ffn_*_gather).
        overlap_gate: the gate's backward on a second stream beside the
        expert GEMMs' backward."""
        self.T, self.d, self.f, self.E, self.k = T, d, f, E, k
        self.fuse_gather = bool(fuse_gather)
        self.overlap_gate = bool(overlap_gate)
        self._gstream = None
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
                                    p(self.dx), 1)),
        ]
        # the gate's backward needs only combine_bwd's d_topk_w: it runs on a
        # stream of its own beside the expert GEMMs; it writes dx, and
        # moe_unpermute_grad then adds the dispatch gradient to
        self._gate = ("moe_gate_topk_bwd", (p(x), p(Wg), p(self.logits), p(self.topk_idx),
                                            p(self.topk_w), p(self.d_topk_w), T, d, E, k,
                                            self.renorm, dt, p(self.dx), 0, p(self.dWg),
                                            p(self.ws_gate), self.ws_gate.numel()))
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
        """combine_bwd; then the gate backward (dx = dl Wg^T, dWg) on a second
        stream while moe_expert_ffn_bwd runs; then dx += the unpermuted
        dispatch gradient.  overlap_gate = False runs the same calls in the
        same order on one stream (identical bits)."""
        assert self.dy is not None, "bind(dy=...) first"
        s = _stream(self.device) if stream is None else stream
        ms = _torch_stream(stream, self.device)
        L = self.lib
        comb, ffn, unperm = self._bwd
        check(getattr(L, comb[0])(*comb[1], s), comb[0])
        # under HIP graph capture everything stays on the capturing stream
        # (plus the library's own side stream): capturing a second user
        # stream that shared that side stream once ended the capture with a
        # crash in the runtime, whose cause is not known.  The capture state
        # is that of the stream the step runs on, not of torch's current one
        with torch.cuda.stream(ms):
            capturing = torch.cuda.is_current_stream_capturing()
        if self.overlap_gate and not capturing:
            if self._gstream is None:
                self._gstream = torch.cuda.Stream(device=self.device)
            gs = self._gstream
            gs.wait_stream(ms)
            check(getattr(L, self._gate[0])(*self._gate[1], gs.cuda_stream), self._gate[0])
            check(getattr(L, ffn[0])(*ffn[1], s), ffn[0])
            ms.wait_stream(gs)
        else:
            check(getattr(L, self._gate[0])(*self._gate[1], s), self._gate[0])
            check(getattr(L, ffn[0])(*ffn[1], s), ffn[0])
        check(getattr(L, unperm[0])(*unperm[1], s), unperm[0])
        return self.dx

    def step(self, stream=None):
        """One forward + backward pass."""
        self._run(self._fwd, stream)
        self.backward(stream)

    def stage_calls(self):
        """[(name, callable)] of every step of one layer step, in order, on one
        stream."""
        L = self.lib
        mk = lambda n, a: (n, (lambda n=n, a=a, s=None: check(
            getattr(L, n)(*a, _stream(self.device) if s is None else s), n)))
        comb, ffn, unperm = self._bwd
        return ([mk(n, a) for n, a in self._fwd] + [mk(*comb)] +
                [mk(*self._gate), mk(*ffn), mk(*unperm)])


class ChunkedMoELayer:
    """The same layer step over the tokens in chunks of at most chunk_tokens,
    with the dispatch and activation buffers sized for one chunk and reused
    (MPipeMoE, 研究方法: buffers shared across micro-batches, recomputation;
    "Flattening Every Memory Peak in Long-Context MoE Training", English
    abstract: a token cap per dispatch chunk bounds the dispatch peak).

    forward:  moe_gate_topk over all tokens; per chunk moe_permute ->
              moe_expert_ffn_fwd -> moe_combine (out_perm is kept whole: the
              gate's backward needs it).
    backward: moe_combine_bwd of every chunk (d_topk_w), moe_gate_topk_bwd
              over all tokens, which writes dx; then chunks in reverse order,
              the last chunk's saved state still in the buffers, every other
              chunk re-permuted with GEMM1 recomputed (moe_expert_ffn_fwd with
              out_perm = NULL) and its d_out_perm remade; moe_expert_ffn_bwd
              (first) / _accumulate (rest) -> moe_unpermute_grad (adds to dx).

    y, dx, dWg and every routing output are bit-identical to MoELayer's; dW1,
    dW2, dW3 are the same sums taken chunk by chunk (one rounding per chunk
    in bf16).
    """

    def __init__(self, T, d, f, E, k, act="gelu", dtype=torch.bfloat16,
                 renorm=1, device="cuda", chunk_tokens=4096):
        self.T, self.d, self.f, self.E, self.k = T, d, f, E, k
        self.act = MOE_ACT_SWIGLU if act == "swiglu" else MOE_ACT_GELU
        self.dtype = dtype
        self.dt = MOE_BF16 if dtype == torch.bfloat16 else MOE_F32
        self.renorm = renorm
        self.device = torch.device(device)
        C = self.C = max(1, min(int(chunk_tokens), T)) if T > 0 else 1
        self.nch = (T + C - 1) // C
        L = self.lib = load()
        R = self.R = T * k
        Rc = self.Rc = C * k
        dev = self.device
        e = lambda *s, dt=dtype: torch.empty(*s, dtype=dt, device=dev)
        i32, f32 = torch.int32, torch.float32
        hw = 2 * f if self.act == MOE_ACT_SWIGLU else f
        # whole-batch tensors
        self.logits = e(T, E, dt=f32)
        self.topk_idx = e(T, k, dt=i32)
        self.topk_w = e(T, k, dt=f32)
        self.dest = e(T, k, dt=i32)            # rows within the token's chunk
        self.src = e(R, dt=i32)                # chunk-major; tokens within the chunk
        self.counts = e(self.nch, E, dt=i32)
        self.offsets = e(self.nch, E + 1, dt=i32)
        self.out_perm = e(R, d)                # chunk-major
        self.y = e(T, d)
        self.d_topk_w = e(T, k, dt=f32)
        self.dx = e(T, d)
        self.dW1 = e(E, d, f)
        self.dW3 = e(E, d, f) if self.act == MOE_ACT_SWIGLU else None
        self.dW2 = e(E, f, d)
        self.dWg = e(d, E)
        # one chunk's buffers, reused
        self.x_perm = e(Rc, d)
        self.h_save = e(Rc, hw)
        self.a_save = e(Rc, f)
        self.d_out_perm = e(Rc, d)
        self.dx_perm = e(Rc, d)
        ws = lambda n: torch.empty(max(int(n), 1), dtype=torch.uint8, device=dev)
        self.ws_perm = ws(L.moe_permute_workspace_bytes(C, E, k))
        self.ws_ffn_f = ws(L.moe_ffn_workspace_bytes(Rc, E, d, f, self.act, self.dt, 0))
        self.ws_ffn_b = ws(L.moe_ffn_workspace_bytes(Rc, E, d, f, self.act, self.dt, 1))
        self.ws_gate = ws(L.moe_gate_bwd_workspace_bytes(T, d, E))
        self._resident = -1                    # chunk whose state the buffers hold

    def bind(self, x, Wg, W1, W2, W3=None, logit_bias=None, dy=None):
        for t in (x, Wg, W1, W2, W3, dy):
            if t is not None:
                assert t.is_cuda and t.is_contiguous() and t.dtype == self.dtype
        self.x, self.Wg, self.W1, self.W2, self.W3 = x, Wg, W1, W2, W3
        self.bias, self.dy = logit_bias, dy
        self._resident = -1
        return self

    def _chunks(self):
        for c in range(self.nch):
            t0 = c * self.C
            tc = min(self.C, self.T - t0)
            yield c, t0, tc, c * self.Rc, tc * self.k

    def _permute(self, c, t0, tc, r0, s):
        p = lambda t: t.data_ptr()
        L = self.lib
        check(L.moe_permute(p(self.topk_idx[t0:]), p(self.x[t0:]), tc, self.d, self.E,
                            self.k, self.dt, p(self.counts[c]), p(self.offsets[c]),
                            p(self.dest[t0:]), p(self.src[r0:]), p(self.x_perm),
                            p(self.ws_perm), self.ws_perm.numel(), s), "moe_permute")

    def _ffn_fwd(self, c, rc, out, s):
        p = lambda t: None if t is None else t.data_ptr()
        check(self.lib.moe_expert_ffn_fwd(
            p(self.x_perm), p(self.offsets[c]), rc, self.E, self.d, self.f, self.act, self.dt,
            p(self.W1), p(self.W3), p(self.W2), p(self.h_save), p(self.a_save), p(out),
            p(self.ws_ffn_f), self.ws_ffn_f.numel(), s), "moe_expert_ffn_fwd")

    def forward(self, stream=None):
        s = _stream(self.device) if stream is None else stream
        p = lambda t: None if t is None else t.data_ptr()
        L, T, d, E, k = self.lib, self.T, self.d, self.E, self.k
        check(L.moe_gate_topk(p(self.x), p(self.Wg), p(self.bias), T, d, E, k, self.renorm,
                              self.dt, p(self.logits), p(self.topk_idx), p(self.topk_w), s),
              "moe_gate_topk")
        for c, t0, tc, r0, rc in self._chunks():
            self._permute(c, t0, tc, r0, s)
            self._ffn_fwd(c, rc, self.out_perm[r0:], s)
            self._resident = c
            check(L.moe_combine(p(self.out_perm[r0:]), p(self.dest[t0:]), p(self.topk_w[t0:]),
                                tc, k, d, self.dt, p(self.y[t0:]), s), "moe_combine")
        return self.y

    def backward(self, stream=None):
        assert self.dy is not None, "bind(dy=...) first"
        s = _stream(self.device) if stream is None else stream
        p = lambda t: None if t is None else t.data_ptr()
        L, T, d, f, E, k = self.lib, self.T, self.d, self.f, self.E, self.k

        def comb(t0, tc, r0):
            check(L.moe_combine_bwd(p(self.dy[t0:]), p(self.out_perm[r0:]), p(self.dest[t0:]),
                                    p(self.topk_w[t0:]), tc, k, d, self.dt,
                                    p(self.d_out_perm), p(self.d_topk_w[t0:]), s),
                  "moe_combine_bwd")
        # d_topk_w of every token first: the gate's backward (dx = dl Wg^T,
        # dWg) comes before the dispatch gradient is added, the order
        # MoELayer uses, so that dx has the same bits
        chunks = list(self._chunks())
        for c, t0, tc, r0, rc in chunks:
            comb(t0, tc, r0)
        dout = self.nch - 1                    # chunk whose d_out_perm is in place
        check(L.moe_gate_topk_bwd(p(self.x), p(self.Wg), p(self.logits), p(self.topk_idx),
                                  p(self.topk_w), p(self.d_topk_w), T, d, E, k, self.renorm,
                                  self.dt, p(self.dx), 0, p(self.dWg), p(self.ws_gate),
                                  self.ws_gate.numel(), s), "moe_gate_topk_bwd")
        first = True
        for c, t0, tc, r0, rc in reversed(chunks):
            if c != self._resident:        # the forward's last chunk is still in place
                self._permute(c, t0, tc, r0, s)
                self._ffn_fwd(c, rc, None, s)
                self._resident = c
            if c != dout:
                comb(t0, tc, r0)
                dout = c
            fn = L.moe_expert_ffn_bwd if first else L.moe_expert_ffn_bwd_accumulate
            check(fn(p(self.d_out_perm), p(self.x_perm), p(self.h_save), p(self.a_save),
                     p(self.offsets[c]), rc, E, d, f, self.act, self.dt, p(self.W1),
                     p(self.W3), p(self.W2), p(self.dx_perm), p(self.dW1), p(self.dW3),
                     p(self.dW2), p(self.ws_ffn_b), self.ws_ffn_b.numel(), s),
                  "moe_expert_ffn_bwd")
            first = False
            check(L.moe_unpermute_grad(p(self.dx_perm), p(self.dest[t0:]), tc, k, d, self.dt,
                                       p(self.dx[t0:]), 1, s), "moe_unpermute_grad")
        return self.dx

    def step(self, stream=None):
        self.forward(stream)
        self.backward(stream)


def offload_groups(E, G, pinned):
    """The expert calls of OffloadedMoELayer: offloaded groups (e0, ne), runs
    of unpinned experts cut into at most G, and resident runs (e0, ne, p0),
    maximal runs of consecutive pinned experts whose weights are rows
    p0 .. p0+ne-1 of the pinned tensors (pinned: increasing expert ids)."""
    pin = {e: j for j, e in enumerate(pinned)}
    groups, resident = [], []
    e = 0
    while e < E:
        e1 = e + 1
        if e in pin:
            while e1 < E and e1 in pin:
                e1 += 1
            resident.append((e, e1 - e, pin[e]))
        else:
            while e1 < E and e1 not in pin and e1 - e < G:
                e1 += 1
            groups.append((e, e1 - e))
        e = e1
    return groups, resident


class OffloadedMoELayer:
    """The layer step with the expert weights in pinned host memory and only
    the weights (and weight gradients) of G experts on the GPU at a time:
    experts are processed group by group, and the next group's parameters
    move in while the current group computes (ES-MoE review, 三 技术架构 /
    专家级卸载与处理: expert-wise processing with parameter transfers
    overlapped with expert compute).

    forward:  moe_gate_topk -> moe_permute -> per group of G experts: the
              group's W1/W2(/W3) uploaded on an upload stream into one of two
              staging slots (the next group's upload overlaps this group's
              GEMMs) -> moe_expert_ffn_fwd over the group's segments ->
              moe_combine
    backward: moe_combine_bwd -> moe_gate_topk_bwd (writes dx) -> per group,
              last first: the group's weights (uploaded again unless the
              forward left them in a slot) -> moe_expert_ffn_bwd over its
              segments -> its dW
              downloaded on a download stream -> moe_unpermute_grad (adds to dx)

    A group call passes offsets + e0 and the group's expert count; rows stay
    absolute, so every tile is the same fixed-order sum as in MoELayer and
    every output (y, dx, dWg, dW1, dW2, dW3) is bit-identical to it.

    Expert pinning (ES-MoE review, 三 技术架构 / 自适应卸载: the most
    frequently routed quarter of the experts is kept on the GPU to cut the
    transfers): the experts listed in `pinned` are copied to the GPU once, at
    bind(), into W1p/W2p/W3p [P, ...] (pinned order), and their weight
    gradients go to dW1p/dW2p/dW3p on the GPU (in the step's stream order;
    grads_ready covers the host gradients only); those two sets are the
    pinned experts' weights and gradients from then on (the host tensors'
    rows of pinned experts are neither read again nor written).  Runs of
    consecutive pinned experts are one call each.  They run first in the
    forward, while both staging slots fill, and right after the first
    offloaded group in the backward, while the slot that group frees is
    refilled: the most routed experts carry the most compute, and it hides
    those transfers.  (Dealing them in shares between all the groups was
    slower: skewed workload, 4 of 16 pinned, 40.6-44.4 against 32.6 ms.)
    The other experts form the offloaded groups of at most G.  Grouping
    changes no bits: every expert's rows are the same tiles in any call.
    most_routed(counts, frac) picks such a list from a routing histogram.
    Inputs: x, Wg, logit_bias, dy on the GPU; W1, W2, W3 as pinned host
    tensors (bind).  dW1, dW2, dW3 are pinned host tensors, final once the
    event grads_ready has completed (grads_ready.synchronize(), a stream that
    waits for it, or torch.cuda.synchronize()): the last downloads run beside
    the next step's uploads, not on the step's stream.  The host weights may
    change between steps (every forward uploads them again), not between a
    forward and its backward (which reuses the two groups still staged), and
    not while the step's uploads are in flight.
    """

    def __init__(self, T, d, f, E, k, act="gelu", dtype=torch.bfloat16, renorm=1,
                 device="cuda", group_experts=4, pinned=()):
        self.T, self.d, self.f, self.E, self.k = T, d, f, E, k
        self.act = MOE_ACT_SWIGLU if act == "swiglu" else MOE_ACT_GELU
        self.dtype = dtype
        self.dt = MOE_BF16 if dtype == torch.bfloat16 else MOE_F32
        self.renorm = renorm
        self.device = torch.device(device)
        self.G = G = max(1, min(int(group_experts), E))
        self.pinned = sorted({int(e) for e in pinned})
        assert all(0 <= e < E for e in self.pinned), "pinned experts out of range"
        self.groups, self.resident = offload_groups(E, G, self.pinned)
        gmax = max([ne for _, ne in self.groups] + [ne for _, ne, _ in self.resident])
        L = self.lib = load()
        R = self.R = T * k
        dev = self.device
        e = lambda *s, dt=dtype: torch.empty(*s, dtype=dt, device=dev)
        h = lambda *s: torch.empty(*s, dtype=dtype, pin_memory=True)
        i32, f32 = torch.int32, torch.float32
        sw = self.act == MOE_ACT_SWIGLU
        hw = 2 * f if sw else f
        self.logits = e(T, E, dt=f32)
        self.topk_idx = e(T, k, dt=i32)
        self.topk_w = e(T, k, dt=f32)
        self.counts = e(E, dt=i32)
        self.offsets = e(E + 1, dt=i32)
        self.dest = e(T, k, dt=i32)
        self.src = e(R, dt=i32)
        self.x_perm = e(R, d)
        self.h_save = e(R, hw)
        self.a_save = e(R, f)
        self.out_perm = e(R, d)
        self.y = e(T, d)
        self.d_out_perm = e(R, d)
        self.d_topk_w = e(T, k, dt=f32)
        self.dx_perm = e(R, d)
        self.dx = e(T, d)
        self.dWg = e(d, E)
        # the pinned experts' weights and weight gradients, on the GPU
        P = len(self.pinned)
        self.W1p = e(P, d, f) if P else None
        self.W2p = e(P, f, d) if P else None
        self.W3p = e(P, d, f) if P and sw else None
        self.dW1p = e(P, d, f) if P else None
        self.dW2p = e(P, f, d) if P else None
        self.dW3p = e(P, d, f) if P and sw else None
        # two staging slots of G experts' weights and weight gradients
        self.W1s = [e(G, d, f) for _ in range(2)]
        self.W2s = [e(G, f, d) for _ in range(2)]
        self.W3s = [e(G, d, f) if sw else None for _ in range(2)]
        self.dW1s = [e(G, d, f) for _ in range(2)]
        self.dW2s = [e(G, f, d) for _ in range(2)]
        self.dW3s = [e(G, d, f) if sw else None for _ in range(2)]
        # weight gradients on the host (pinned)
        self.dW1 = h(E, d, f)
        self.dW2 = h(E, f, d)
        self.dW3 = h(E, d, f) if sw else None
        ws = lambda n: torch.empty(max(int(n), 1), dtype=torch.uint8, device=dev)
        self.ws_perm = ws(L.moe_permute_workspace_bytes(T, E, k))
        self.ws_ffn_f = ws(L.moe_ffn_workspace_bytes(R, gmax, d, f, self.act, self.dt, 0))
        self.ws_ffn_b = ws(L.moe_ffn_workspace_bytes(R, gmax, d, f, self.act, self.dt, 1))
        self.ws_gate = ws(L.moe_gate_bwd_workspace_bytes(T, d, E))
        self._up_stream = torch.cuda.Stream(device=dev)
        self._dn_stream = torch.cuda.Stream(device=dev)
        ev = lambda: [torch.cuda.Event(), torch.cuda.Event()]
        self._up, self._free, self._dl = ev(), ev(), ev()
        self._slot = [-1, -1]          # group whose weights each slot holds
        self._pin_ready = torch.cuda.Event()
        # recorded on the download stream once a backward's weight gradients
        # are all on the host
        self.grads_ready = torch.cuda.Event()

    @staticmethod
    def most_routed(counts, frac=0.25):
        """The ceil(frac * E) experts with the most rows in a routing
        histogram (ties: lower index first), in increasing order."""
        c = [int(v) for v in torch.as_tensor(counts).detach().cpu().tolist()]
        n = min(len(c), math.ceil(frac * len(c)))
        return sorted(sorted(range(len(c)), key=lambda e: (-c[e], e))[:n])

    def bind(self, x, Wg, W1, W2, W3=None, logit_bias=None, dy=None):
        """x, Wg, logit_bias, dy on the GPU; W1 [E,d,f], W2 [E,f,d], W3 as
        pinned, contiguous host tensors of the layer's dtype."""
        for t in (x, Wg, dy):
            if t is not None:
                assert t.is_cuda and t.is_contiguous() and t.dtype == self.dtype
        for t in (W1, W2, W3):
            if t is not None:
                assert (not t.is_cuda and t.is_pinned() and t.is_contiguous()
                        and t.dtype == self.dtype)
        assert (W3 is not None) == (self.act == MOE_ACT_SWIGLU)
        self.x, self.Wg, self.bias, self.dy = x, Wg, logit_bias, dy
        self.W1h, self.W2h, self.W3h = W1, W2, W3
        self._slot = [-1, -1]
        if self.pinned:                # the pinned experts' weights, once
            # a step still in flight may read the pinned copies: let it finish
            torch.cuda.synchronize(self.device)
            us = self._up_stream
            with torch.cuda.stream(us):
                for j, e in enumerate(self.pinned):
                    self.W1p[j].copy_(W1[e], non_blocking=True)
                    self.W2p[j].copy_(W2[e], non_blocking=True)
                    if W3 is not None:
                        self.W3p[j].copy_(W3[e], non_blocking=True)
            self._pin_ready.record(us)
        return self

    def _upload(self, g):
        """The weights of group g into slot g % 2 on the upload stream, once
        the GEMMs that last read that slot are done."""
        b = g % 2
        if self._slot[b] == g:
            return
        e0, ne = self.groups[g]
        us = self._up_stream
        us.wait_event(self._free[b])
        with torch.cuda.stream(us):
            self.W1s[b][:ne].copy_(self.W1h[e0:e0 + ne], non_blocking=True)
            self.W2s[b][:ne].copy_(self.W2h[e0:e0 + ne], non_blocking=True)
            if self.W3h is not None:
                self.W3s[b][:ne].copy_(self.W3h[e0:e0 + ne], non_blocking=True)
        self._up[b].record(us)
        self._slot[b] = g

    def forward(self, stream=None):
        s = _stream(self.device) if stream is None else stream
        ms = _torch_stream(stream, self.device)
        p = lambda t: None if t is None else t.data_ptr()
        L, T, d, f, E, k, R = self.lib, self.T, self.d, self.f, self.E, self.k, self.R
        dt, a = self.dt, self.act
        check(L.moe_gate_topk(p(self.x), p(self.Wg), p(self.bias), T, d, E, k, self.renorm,
                              dt, p(self.logits), p(self.topk_idx), p(self.topk_w), s),
              "moe_gate_topk")
        check(L.moe_permute(p(self.topk_idx), p(self.x), T, d, E, k, dt, p(self.counts),
                            p(self.offsets), p(self.dest), p(self.src), p(self.x_perm),
                            p(self.ws_perm), self.ws_perm.numel(), s), "moe_permute")
        n = len(self.groups)
        # the host weights may have changed since the last step: upload all
        self._slot = [-1, -1]
        for g in range(min(n, 2)):     # both slots before any compute
            self._upload(g)
        if self.resident:
            ms.wait_event(self._pin_ready)

        def pinned_fwd(runs):
            for e0, ne, p0 in runs:
                check(L.moe_expert_ffn_fwd(p(self.x_perm), p(self.offsets) + 4 * e0, R, ne, d,
                                           f, a, dt, p(self.W1p[p0]),
                                           p(self.W3p[p0]) if self.W3p is not None else None,
                                           p(self.W2p[p0]), p(self.h_save), p(self.a_save),
                                           p(self.out_perm), p(self.ws_ffn_f),
                                           self.ws_ffn_f.numel(), s), "moe_expert_ffn_fwd")
        pinned_fwd(self.resident)
        for g, (e0, ne) in enumerate(self.groups):
            b = g % 2
            if g + 1 < n:
                self._upload(g + 1)
            ms.wait_event(self._up[b])
            check(L.moe_expert_ffn_fwd(p(self.x_perm), p(self.offsets) + 4 * e0, R, ne, d, f,
                                       a, dt, p(self.W1s[b]), p(self.W3s[b]), p(self.W2s[b]),
                                       p(self.h_save), p(self.a_save), p(self.out_perm),
                                       p(self.ws_ffn_f), self.ws_ffn_f.numel(), s),
                  "moe_expert_ffn_fwd")
            self._free[b].record(ms)
        check(L.moe_combine(p(self.out_perm), p(self.dest), p(self.topk_w), T, k, d, dt,
                            p(self.y), s), "moe_combine")
        return self.y

    def backward(self, stream=None):
        assert self.dy is not None, "bind(dy=...) first"
        s = _stream(self.device) if stream is None else stream
        ms = _torch_stream(stream, self.device)
        p = lambda t: None if t is None else t.data_ptr()
        L, T, d, f, E, k, R = self.lib, self.T, self.d, self.f, self.E, self.k, self.R
        dt, a = self.dt, self.act
        check(L.moe_combine_bwd(p(self.dy), p(self.out_perm), p(self.dest), p(self.topk_w),
                                T, k, d, dt, p(self.d_out_perm), p(self.d_topk_w), s),
              "moe_combine_bwd")
        check(L.moe_gate_topk_bwd(p(self.x), p(self.Wg), p(self.logits), p(self.topk_idx),
                                  p(self.topk_w), p(self.d_topk_w), T, d, E, k, self.renorm,
                                  dt, p(self.dx), 0, p(self.dWg), p(self.ws_gate),
                                  self.ws_gate.numel(), s), "moe_gate_topk_bwd")
        order = list(range(len(self.groups)))[::-1]   # the forward's last groups are staged
        if order:
            self._upload(order[0])

        def pinned_bwd(runs):          # pinned experts: gradients stay on the GPU
            for e0, ne, p0 in runs:
                check(L.moe_expert_ffn_bwd(p(self.d_out_perm), p(self.x_perm), p(self.h_save),
                                           p(self.a_save), p(self.offsets) + 4 * e0, R, ne, d,
                                           f, a, dt, p(self.W1p[p0]),
                                           p(self.W3p[p0]) if self.W3p is not None else None,
                                           p(self.W2p[p0]), p(self.dx_perm), p(self.dW1p[p0]),
                                           p(self.dW3p[p0]) if self.dW3p is not None else None,
                                           p(self.dW2p[p0]), p(self.ws_ffn_b),
                                           self.ws_ffn_b.numel(), s), "moe_expert_ffn_bwd")
        pending = [None, None]                # group whose dW a slot holds, not yet downloaded
        for i, g in enumerate(order):
            e0, ne = self.groups[g]
            b = g % 2
            if i + 1 < len(order):
                self._upload(order[i + 1])
            if pending[b] is not None:        # the slot's previous dW goes out first
                self._download(pending[b])
                pending[b] = None
            ms.wait_event(self._up[b])
            ms.wait_event(self._dl[b])        # slot b's previous dW is on the host
            check(L.moe_expert_ffn_bwd(p(self.d_out_perm), p(self.x_perm), p(self.h_save),
                                       p(self.a_save), p(self.offsets) + 4 * e0, R, ne, d, f,
                                       a, dt, p(self.W1s[b]), p(self.W3s[b]), p(self.W2s[b]),
                                       p(self.dx_perm), p(self.dW1s[b]), p(self.dW3s[b]),
                                       p(self.dW2s[b]), p(self.ws_ffn_b),
                                       self.ws_ffn_b.numel(), s), "moe_expert_ffn_bwd")
            self._free[b].record(ms)
            pending[b] = g
            if i == 0:                 # beside the refill of the slot just freed
                pinned_bwd(self.resident)
        if not order:
            pinned_bwd(self.resident)
        check(L.moe_unpermute_grad(p(self.dx_perm), p(self.dest), T, k, d, dt, p(self.dx), 1,
                                   s), "moe_unpermute_grad")
        # the last groups' gradients go out after the step's GEMMs: downloads
        # into pinned memory run as copy kernels on all compute units, and
        # beside a GEMM they slowed it several times over
        for g in order[-2:]:
            if pending[g % 2] == g:
                self._download(g)
        self.grads_ready.record(self._dn_stream)
        return self.dx

    def _download(self, g):
        """Group g's weight gradients from slot g % 2 to the host (download
        stream, after the GEMMs that wrote them)."""
        b = g % 2
        e0, ne = self.groups[g]
        ds = self._dn_stream
        ds.wait_event(self._free[b])
        with torch.cuda.stream(ds):
            self.dW1[e0:e0 + ne].copy_(self.dW1s[b][:ne], non_blocking=True)
            self.dW2[e0:e0 + ne].copy_(self.dW2s[b][:ne], non_blocking=True)
            if self.dW3 is not None:
                self.dW3[e0:e0 + ne].copy_(self.dW3s[b][:ne], non_blocking=True)
        self._dl[b].record(ds)

    def step(self, stream=None):
        self.forward(stream)
        self.backward(stream)
