"""One MoE expert-MLP layer driven through the C-ABI.

``MoEPath`` owns the device buffers of one problem size (allocated once
with torch, reused every step) and issues the library calls in order:

  forward : moe_router_logits -> moe_route -> moe_permute
            -> moe_grouped_mlp_fwd -> moe_unpermute
  backward: moe_permute_rows (dY) -> moe_grouped_mlp_bwd
            -> moe_router_backward (when the forward computed the router
               scores: dlogits with the balancing term, dW_g, db)
            -> moe_unpermute (dX, with the router's share added before its
               one rounding)

With a ``timers`` object (see ``StageTimers``) the GEMMs are issued
through the per-GEMM stage entry points instead of the fused ones, with
HIP events recorded around each stage on the stream it runs on.

``MoEPathMX`` is the same layer with MXFP8 GEMM operands: x is quantized
along d before the permutation, the weights along their rows once per step
(forward) and along their columns inside the backward, S and dAB inside the
GEMM epilogues that produce them (both along their GEMM axis and along each
expert's tokens, the latter for the weight gradients), and dO and Xp along
each expert's tokens in the backward.  No bf16 copy of S or dAB is kept.
With ``act_fp4`` the GEMMs stay MXFP8 but x is quantized to MXFP4 along d
(the dispatched payload, half the bytes), the gate_up GEMM widens it to
E4M3 on its way to LDS, and the backward converts that payload to MXFP4
blocks along each expert's tokens for the dW_gu GEMM (widened the same way)
instead of re-permuting bf16 x.

No arithmetic happens here: every step runs in the library's kernels.
"""

import contextlib

import torch

from . import moe
from .moe import (MOE_BF16, MOE_ENTRY_MLP_BWD, MOE_ENTRY_MLP_FWD,
                  MOE_ENTRY_PERMUTE, MOE_ENTRY_ROUTER_BWD, MOE_MXFP4,
                  MOE_MXFP8)


class StageTimers:
    """Pairs of HIP events recorded around named stages on the current
    stream; ``mean_ms()`` gives each stage's average duration."""

    def __init__(self):
        self.events = {}

    @contextlib.contextmanager
    def around(self, name):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        yield
        b.record()
        self.events.setdefault(name, []).append((a, b))

    def mean_ms(self):
        return {n: sum(a.elapsed_time(b) for a, b in ev) / len(ev)
                for n, ev in self.events.items()}

    def counts(self):
        return {n: len(ev) for n, ev in self.events.items()}


def _around(timers, name):
    return timers.around(name) if timers is not None else \
        contextlib.nullcontext()


class MoEPath:
    def __init__(self, T, d, f, E, k, renorm=True, prec=MOE_BF16,
                 device="cuda", y_fp32=False, aux_coef=0.01):
        if prec != MOE_BF16:
            raise NotImplementedError("use MoEPathMX for the MXFP8 path")
        self.T, self.d, self.f, self.E, self.k = T, d, f, E, k
        self.renorm = renorm
        self.aux_coef = aux_coef
        self._router = None
        self.prec = prec
        Tk = T * k
        dev = torch.device(device)
        i32, f32, bf = torch.int32, torch.float32, torch.bfloat16
        z = lambda *s, dt: torch.empty(*s, dtype=dt, device=dev)  # noqa: E731
        self.logits = z(T, E, dt=f32)
        self.topk_idx = z(T, k, dt=i32)
        self.topk_w = z(T, k, dt=f32)
        self.counts = z(E, dt=i32)
        self.offsets = z(E + 1, dt=i32)
        self.pos = z(T, k, dt=i32)
        self.src = z(Tk, dt=i32)
        self.w_perm = z(Tk, dt=f32)
        self.x_perm = z(Tk, d, dt=bf)
        self.ab = z(Tk, 2 * f, dt=bf)
        self.s = z(Tk, f, dt=bf)
        self.o = z(moe.row_planes(f), Tk, d, dt=f32)
        self.y = z(T, d, dt=f32 if y_fp32 else bf)
        ws_p = moe.moe_workspace_bytes(MOE_ENTRY_PERMUTE, prec, T, E, k, d, f)
        self.ws_permute = z(max(ws_p, 16), dt=torch.uint8)
        self._bwd_ready = False

    def _alloc_bwd(self):
        T, d, f, E, k = self.T, self.d, self.f, self.E, self.k
        Tk = T * k
        dev = self.x_perm.device
        bf = torch.bfloat16
        self.dout_perm = torch.empty(Tk, d, dtype=bf, device=dev)
        self.dx_perm = torch.empty(moe.row_planes(f), Tk, d,
                                   dtype=torch.float32, device=dev)
        self.dw_gu = torch.empty(E, 2 * f, d, dtype=bf, device=dev)
        self.dw2 = torch.empty(E, d, f, dtype=bf, device=dev)
        self.dp = torch.empty(T, k, dtype=torch.float32, device=dev)
        self.dx = torch.empty(T, d, dtype=bf, device=dev)
        self.dab = torch.empty(Tk, 2 * f, dtype=bf, device=dev)
        self.dp_part = torch.empty(Tk, moe.moe_dp_tiles(f),
                                   dtype=torch.float32, device=dev)
        ws_b = moe.moe_workspace_bytes(MOE_ENTRY_MLP_BWD, self.prec, T, E, k,
                                       d, f)
        self.ws_bwd = torch.empty(max(ws_b, 16), dtype=torch.uint8,
                                  device=dev)
        # router backward
        self.dlogits = torch.empty(T, E, dtype=torch.float32, device=dev)
        self.dw_g = torch.empty(E, d, dtype=torch.float32, device=dev)
        self.db = torch.empty(E, dtype=torch.float32, device=dev)
        self.aux_loss = torch.empty(1, dtype=torch.float32, device=dev)
        ws_r = moe.moe_workspace_bytes(MOE_ENTRY_ROUTER_BWD, MOE_BF16, T, E,
                                       k, d, f)
        self.ws_router = torch.empty(max(ws_r, 16), dtype=torch.uint8,
                                     device=dev)
        self._bwd_ready = True

    # ------------------------------------------------------------------
    def route(self, x=None, w_g=None, bias=None, logits=None, timers=None):
        if logits is None:
            with _around(timers, "router_logits"):
                moe.moe_router_logits(x, w_g, bias, self.logits)
            logits = self.logits
            self._router = (x, w_g, bias)
        else:
            self._router = None
        self._logits_used = logits
        with _around(timers, "route"):
            moe.moe_route(logits, self.k, self.renorm, self.topk_idx,
                          self.topk_w)

    def forward(self, x, w_gu, w2, w_g=None, bias=None, logits=None,
                timers=None):
        self.route(x, w_g, bias, logits, timers)
        with _around(timers, "permute"):
            moe.moe_permute(self.prec, self.topk_idx, self.topk_w, self.E, x,
                            None, self.counts, self.offsets, self.pos,
                            self.src, self.w_perm, self.x_perm, None,
                            self.ws_permute)
        if timers is None:
            moe.moe_grouped_mlp_fwd(self.prec, self.x_perm, None,
                                    self.offsets, w_gu, None, w2, None,
                                    self.w_perm, self.ab, self.s, self.o)
        else:
            with timers.around("gate_up_swiglu_fwd"):
                moe.moe_gate_up_swiglu_fwd(self.x_perm, self.offsets, w_gu,
                                           self.w_perm, self.ab, self.s)
            with timers.around("down_fwd"):
                moe.moe_down_fwd(self.s, self.offsets, w2, self.o)
        with _around(timers, "unpermute_y"):
            moe.moe_unpermute(self.o, self.pos, None, self.y)
        return self.y

    def backward(self, dy, w_gu, w2, timers=None):
        if not self._bwd_ready:
            self._alloc_bwd()
        with _around(timers, "permute_dy"):
            moe.moe_permute_rows(self.prec, self.pos, dy, None,
                                 self.dout_perm, None)
        if timers is None:
            moe.moe_grouped_mlp_bwd(self.prec, self.dout_perm, self.x_perm,
                                    self.offsets, self.pos, w_gu, w2, self.ab,
                                    self.s, self.w_perm, self.dx_perm,
                                    self.dw_gu, self.dw2, self.dp,
                                    self.ws_bwd)
        else:
            # the same kernels in the same order as moe_grouped_mlp_bwd
            with timers.around("down_swiglu_bwd"):
                moe.moe_down_swiglu_bwd(self.dout_perm, self.offsets, w2,
                                        self.ab, self.w_perm, self.dab,
                                        self.dp_part)
            with timers.around("dp_reduce"):
                moe.moe_dp_reduce(self.dp_part, self.pos, self.dp)
            with timers.around("wgrad_down"):
                moe.moe_grouped_wgrad(self.dout_perm, self.s, self.offsets,
                                      self.dw2)
            with timers.around("gate_up_dgrad"):
                moe.moe_gate_up_dgrad(self.dab, self.offsets, w_gu,
                                      self.dx_perm)
            with timers.around("wgrad_gate_up"):
                moe.moe_grouped_wgrad(self.dab, self.x_perm, self.offsets,
                                      self.dw_gu)
        self._finish_dx(timers)
        return self.dx, self.dw_gu, self.dw2, self.dp

    def _finish_dx(self, timers):
        """Combine dX; with a router, its backward runs first (score
        gradients, dW_g, db, the balancing loss) and the combine adds the
        router's share of dX before the one rounding."""
        if self._router is None:
            with _around(timers, "unpermute_dx"):
                moe.moe_unpermute(self.dx_perm, self.pos, None, self.dx)
            return
        x, w_g, bias = self._router
        with _around(timers, "router_backward"):
            moe.moe_router_backward(
                self._logits_used, self.topk_idx, self.topk_w, self.dp,
                self.counts, self.aux_coef, self.renorm, x, w_g,
                self.dlogits, self.dw_g, self.db if bias is not None else None,
                None, None, self.aux_loss, self.ws_router)
        with _around(timers, "unpermute_dx"):
            moe.moe_unpermute(self.dx_perm, self.pos, None, self.dx,
                              dlogits=self.dlogits, w_g=w_g)


class StepGraph:
    """A step (e.g. one forward and backward of a path) captured once as a
    HIP graph and replayed.  Every buffer and workspace belongs to the path
    and no entry point allocates, clears with a memset, synchronizes or
    reads back to the host, so the captured launches are the whole step.
    The step runs eagerly twice first: once to allocate what the path
    allocates lazily, once on the capture's side stream."""

    def __init__(self, step):
        step()
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            step()
        torch.cuda.synchronize()

    def replay(self):
        self.graph.replay()


class MoEPathMX(MoEPath):
    """The layer with MXFP8 GEMM operands (see the module docstring)."""

    def __init__(self, T, d, f, E, k, renorm=True, device="cuda",
                 y_fp32=False, aux_coef=0.01, act_fp4=False, training=True):
        super().__init__(T, d, f, E, k, renorm=renorm, prec=MOE_BF16,
                         device=device, y_fp32=y_fp32, aux_coef=aux_coef)
        # training: the forward quantizes each weight for both of its GEMMs
        # from one read (moe_mxfp8_quantize_weight) and the backward uses
        # those column-wise codes; otherwise only the forward's codes are
        # made and the backward quantizes the weights it is given
        self.training = training
        self.act_fp4 = act_fp4
        self.prec = MOE_MXFP4 if act_fp4 else MOE_MXFP8
        Tk = T * k
        dev = self.x_perm.device
        u8 = torch.uint8
        z = lambda *s: torch.empty(*s, dtype=u8, device=dev)  # noqa: E731
        dx = d // 2 if act_fp4 else d          # payload bytes a row
        self.xq, self.xs = z(T, dx), z(T, d // 32)
        self.xpq, self.xps = z(Tk, dx), z(Tk, d // 32)
        self.wguq, self.wgus = z(E, 2 * f, d), z(E, 2 * f, d // 32)
        self.w2q, self.w2s = z(E, d, f), z(E, d, f // 32)
        self.sq, self.ss = z(Tk, f), z(Tk, f // 32)
        # S along each expert's tokens, written by the gate_up epilogue and
        # read by the dW2 GEMM of the backward
        tp = moe.moe_mxfp8_padded_rows(Tk, E)
        self.tk_pad = tp
        self.st, self.sts = z(f, tp), z(f, tp // 32)
        self.s = None
        if training:
            self.w2tq, self.w2ts = z(f, E * d), z(f, E * d // 32)
            self.wgutq, self.wguts = z(d, E * 2 * f), z(d, E * 2 * f // 32)
        ws_f = moe.moe_workspace_bytes(MOE_ENTRY_MLP_FWD, MOE_MXFP8, T, E, k,
                                       d, f)
        self.ws_fwd = z(max(ws_f, 16))

    def _alloc_bwd(self):
        super()._alloc_bwd()
        T, d, f, E, k = self.T, self.d, self.f, self.E, self.k
        Tk = T * k
        dev = self.x_perm.device
        u8 = torch.uint8
        z = lambda *s: torch.empty(*s, dtype=u8, device=dev)  # noqa: E731
        tp = self.tk_pad
        self.doq, self.dos = z(Tk, d), z(Tk, d // 32)
        if not self.training:
            self.w2tq, self.w2ts = z(f, E * d), z(f, E * d // 32)
            self.wgutq, self.wguts = z(d, E * 2 * f), z(d, E * 2 * f // 32)
        self.dab = None
        self.dabq, self.dabs = z(Tk, 2 * f), z(Tk, 2 * f // 32)
        self.dot, self.dots = z(d, tp), z(d, tp // 32)
        self.dabt, self.dabts = z(2 * f, tp), z(2 * f, tp // 32)
        self.xpt = z(d, tp // 2 if self.act_fp4 else tp)
        self.xpts = z(d, tp // 32)
        ws_b = moe.moe_workspace_bytes(MOE_ENTRY_MLP_BWD, MOE_MXFP8, T, E, k,
                                       d, f)
        self.ws_bwd = z(max(ws_b, 16))

    def quantize_weights(self, w_gu, w2, timers=None):
        """MX codes of the weights (once per optimizer step): along their
        rows for the forward GEMMs and, when training, along their columns
        for the data-gradient GEMMs, from the same read."""
        E, d, f = self.E, self.d, self.f
        with _around(timers, "quant_weights"):
            if self.training:
                moe.moe_mxfp8_quantize_weight(
                    w_gu.view(E * 2 * f, d), self.wguq.view(E * 2 * f, d),
                    self.wgus.view(E * 2 * f, d // 32), self.wgutq,
                    self.wguts)
                moe.moe_mxfp8_quantize_weight(
                    w2.view(E * d, f), self.w2q.view(E * d, f),
                    self.w2s.view(E * d, f // 32), self.w2tq, self.w2ts)
            else:
                moe.moe_mxfp8_quantize(w_gu.view(E * 2 * f, d), 0, None,
                                       self.wguq.view(E * 2 * f, d),
                                       self.wgus.view(E * 2 * f, d // 32))
                moe.moe_mxfp8_quantize(w2.view(E * d, f), 0, None,
                                       self.w2q.view(E * d, f),
                                       self.w2s.view(E * d, f // 32))

    def forward(self, x, w_gu, w2, w_g=None, bias=None, logits=None,
                timers=None):
        self.route(x, w_g, bias, logits, timers)
        with _around(timers, "quant_x"):
            if self.act_fp4:
                moe.moe_mxfp4_quantize(x, 0, None, self.xq, self.xs)
            else:
                moe.moe_mxfp8_quantize(x, 0, None, self.xq, self.xs)
        with _around(timers, "permute"):
            moe.moe_permute(self.prec, self.topk_idx, self.topk_w, self.E,
                            self.xq, self.xs, self.counts, self.offsets,
                            self.pos, self.src, self.w_perm, self.xpq,
                            self.xps, self.ws_permute)
        self.quantize_weights(w_gu, w2, timers)
        if timers is None:
            moe.moe_grouped_mlp_fwd(self.prec, self.xpq, self.xps,
                                    self.offsets, self.wguq, self.wgus,
                                    self.w2q, self.w2s, self.w_perm, self.ab,
                                    None, self.o, self.ws_fwd,
                                    s_tok=self.st, s_tok_scales=self.sts)
        else:
            with timers.around("gate_up_swiglu_fwd"):
                moe.moe_mx_gate_up_swiglu_fwd(
                    self.xpq, self.xps, self.offsets, self.wguq, self.wgus,
                    self.w_perm, self.ab, None, self.sq, self.ss,
                    s_tok=self.st, s_tok_scales=self.sts,
                    x_fp4=self.act_fp4)
            with timers.around("down_fwd"):
                moe.moe_mx_down_fwd(self.sq, self.ss, self.offsets, self.w2q,
                                    self.w2s, self.o)
        with _around(timers, "unpermute_y"):
            moe.moe_unpermute(self.o, self.pos, None, self.y)
        self._x = x
        return self.y

    def backward(self, dy, w_gu, w2, timers=None):
        if not self._bwd_ready:
            self._alloc_bwd()
        E, d, f = self.E, self.d, self.f
        with _around(timers, "permute_dy"):
            moe.moe_permute_rows(MOE_BF16, self.pos, dy, None,
                                 self.dout_perm, None)
        if not self.act_fp4:
            # the MXFP4 variant reads the forward's payload instead
            with _around(timers, "permute_x"):
                moe.moe_permute_rows(MOE_BF16, self.pos, self._x, None,
                                     self.x_perm, None)
        xp, xps = ((self.xpq, self.xps) if self.act_fp4
                   else (self.x_perm, None))
        if timers is None:
            # when training, the forward's column-wise weight codes go in
            # ready-made
            cols = ({"w_gu_col": (self.wgutq, self.wguts),
                     "w2_col": (self.w2tq, self.w2ts)} if self.training
                    else {})
            moe.moe_grouped_mlp_bwd(self.prec, self.dout_perm, xp,
                                    self.offsets, self.pos, w_gu, w2, self.ab,
                                    None, self.w_perm, self.dx_perm,
                                    self.dw_gu, self.dw2, self.dp,
                                    self.ws_bwd, s_tok=self.st,
                                    s_tok_scales=self.sts,
                                    x_perm_scales=xps, **cols)
        else:
            # the kernels of moe_grouped_mlp_bwd in its order (when
            # training, the column-wise weight codes from the forward's
            # quantize_weights, as the fused call is given them)
            tp = self.tk_pad
            with timers.around("quant_bwd_operands"):
                moe.moe_mxfp8_quantize(self.dout_perm, 0, None, self.doq,
                                       self.dos)
                if not self.training:
                    moe.moe_mxfp8_quantize(w2.view(E * d, f), 1, None,
                                           self.w2tq, self.w2ts, E * d)
                    moe.moe_mxfp8_quantize(w_gu.view(E * 2 * f, d), 1, None,
                                           self.wgutq, self.wguts, E * 2 * f)
            with timers.around("down_swiglu_bwd"):
                moe.moe_mx_down_swiglu_bwd(
                    self.doq, self.dos, self.offsets, self.w2tq, self.w2ts,
                    self.ab, self.w_perm, None, self.dabq, self.dabs,
                    self.dp_part, dab_tok=self.dabt,
                    dab_tok_scales=self.dabts)
            with timers.around("dp_reduce"):
                moe.moe_dp_reduce(self.dp_part, self.pos, self.dp)
            with timers.around("gate_up_dgrad"):
                moe.moe_mx_gate_up_dgrad(self.dabq, self.dabs, self.offsets,
                                         self.wgutq, self.wguts, self.dx_perm)
            with timers.around("quant_tokens"):
                moe.moe_mxfp8_quantize(self.dout_perm, 1, self.offsets,
                                       self.dot, self.dots, tp)
                if self.act_fp4:
                    moe.moe_mxfp4_quantize(self.xpq, 1, self.offsets,
                                           self.xpt, self.xpts, tp,
                                           src_scales=self.xps)
                else:
                    moe.moe_mxfp8_quantize(self.x_perm, 1, self.offsets,
                                           self.xpt, self.xpts, tp)
            Tk = self.T * self.k
            with timers.around("wgrad_down"):
                moe.moe_mx_grouped_wgrad(self.dot, self.dots, self.st,
                                         self.sts, self.offsets, Tk, self.dw2)
            with timers.around("wgrad_gate_up"):
                moe.moe_mx_grouped_wgrad(self.dabt, self.dabts, self.xpt,
                                         self.xpts, self.offsets, Tk,
                                         self.dw_gu, b_fp4=self.act_fp4)
        self._finish_dx(timers)
        return self.dx, self.dw_gu, self.dw2, self.dp
