"""DeepSeekMoE layer forward composed from the C-ABI calls.

The steps, in the order the method applies them (aliyun study note
developer.aliyun.com/article/1776647 section 2.2; news.qq.com/rain/a/
20241229A05OQF00 sections DeepSeekMoE 架构, 无额外损耗的负载均衡 and
FP8 低精度训练):

  1. moe_route         sigmoid scores + selection bias, 4-of-8-group top-8
     (moe_route_scores + moe_seq_balance with seq_len: also the
     sequence-wise balance statistic, factor alpha = 0.0001)
  2. fp8_quant_1x128   x -> E4M3 with 1x128 scales
  3. moe_permute       expert-major dispatch order (no copy: GEMM 1 gathers)
  4. grouped_fp8_gemm_swiglu
                       gate+up of the 256 routed experts and the shared one,
                       SwiGLU and 1x128 requantisation in the epilogue
  5. grouped_fp8_gemm  down projection
  6. moe_combine       gate-weighted sum of routed outputs + shared output
  7. moe_bias_update   (optional) aux-loss-free bias step for the next batch

MoELayer.backward runs the backward of the expert path in FP8 (the pages'
backward-for-input and backward-for-weights chunks, section 工程 › DualPipe
流水线并行, with the FP8 formats of section FP8 低精度训练):

  1. moe_combine_backward   dD = w * dy per routed row, dy for the shared rows
                            (bf16, and its 1x128 E4M3 codes in the same pass);
                            dw = <dy, D> (the gate weights' gradient)
  2. grouped_fp8_gemm_dgrad on W_dn                   dh = dD W_dn
  3. grouped_fp8_gemm       the gate+up outputs again (bf16; the fused
                            forward keeps none)
  4. swiglu_backward_grouped  dGU = [dg | du] and h (bf16), dGU's 1x128
                            codes, the 128x1 chunk codes of dGU and h
  5. grouped_fp8_gemm_dgrad on W_gu                   dX = dGU W_gu
  6. moe_combine            dx = the sum of a token's rows of dX (unit weights)
  7. fp8_quant_128x1_grouped (dD, gathered x) + grouped_fp8_wgrad
                            dW_dn = dD^T h,
                            dW_gu = dGU^T x (x gathered through the permutation)
  8. moe_router_backward    dw -> the gate logits' gradient, dx += its part
     moe_router_dcentroids  the centroids' gradient (the bias has none)
     (with seq_len: moe_router_backward_dense - the balance term's gradient
     on every expert's logit joins the gate's, dx and dC as fp32 GEMMs)

The input gradients read the weights in their forward layout (LDS transpose
reads inside the GEMM), so the backward keeps nothing derived from the
weights: after a weight update (requantize_from_fp32, or any write to w_gu /
w_dn) the next forward and backward use the new weights as they are.

torch is only used to hold device memory and to name the stream; every step
runs in the library's HIP kernels.
"""
from __future__ import annotations

import dataclasses

import torch

from . import _lib as L


@dataclasses.dataclass(frozen=True)
class LayerShape:
    H: int
    E: int
    n_group: int
    topk_group: int
    k: int
    I: int
    n_shared: int = 1

    @property
    def G(self):
        return self.E + self.n_shared


class Buffers:
    """Device buffers of one forward at T tokens (reused across calls)."""

    def __init__(self, shape: LayerShape, T: int, device="cuda"):
        s = shape
        R = T * s.k + s.n_shared * T
        dev = torch.device(device)
        u8, i32, f32, bf = torch.uint8, torch.int32, torch.float32, torch.bfloat16
        self.T, self.R = T, R
        self.topk_idx = torch.empty((T, s.k), dtype=i32, device=dev)
        self.topk_w = torch.empty((T, s.k), dtype=f32, device=dev)
        self.topk_s = torch.empty((T, s.k), dtype=f32, device=dev)   # the chosen experts' scores
        self.counts = torch.empty((s.E,), dtype=i32, device=dev)
        self.route_ws_bytes = max(16, L.moe_route_workspace_bytes(T, s.H, s.E))
        self.route_ws = torch.empty((self.route_ws_bytes,), dtype=u8, device=dev)
        self.xq = torch.empty((T, s.H), dtype=u8, device=dev)
        self.xs = torch.empty((T, s.H // 128), dtype=f32, device=dev)
        self.offsets = torch.empty((s.G + 1,), dtype=i32, device=dev)
        self.perm_src = torch.empty((max(R, 1),), dtype=i32, device=dev)
        self.inv_perm = torch.empty((max(T * s.k, 1),), dtype=i32, device=dev)
        self.perm_ws_bytes = max(16, L.moe_permute_workspace_bytes(T, s.k, s.E))
        self.perm_ws = torch.empty((self.perm_ws_bytes,), dtype=u8, device=dev)
        self._hgu = None
        self._dev = dev
        self._shape = s
        self.hq = torch.empty((R, s.I), dtype=u8, device=dev)
        self.hs = torch.empty((R, s.I // 128), dtype=f32, device=dev)
        self.d = torch.empty((R, s.H), dtype=bf, device=dev)
        self.y = torch.empty((T, s.H), dtype=bf, device=dev)

    def balance(self, seq_len: int):
        """Buffers of the sequence-wise balance statistic (allocated on first
        use, again when seq_len changes): scores [T, E], score_sums [T],
        seq_f, seq_p [B, E], seq_loss [B], B = ceil(T / seq_len)."""
        s = self._shape
        if getattr(self, "_seq_len", None) != seq_len:
            T, dev, f32 = self.T, self._dev, torch.float32
            B = -(-T // seq_len)
            self.scores = torch.empty((max(T, 1), s.E), dtype=f32, device=dev)
            self.score_sums = torch.empty((max(T, 1),), dtype=f32, device=dev)
            self.seq_f = torch.empty((max(B, 1), s.E), dtype=f32, device=dev)
            self.seq_p = torch.empty((max(B, 1), s.E), dtype=f32, device=dev)
            self.seq_loss = torch.empty((max(B, 1),), dtype=f32, device=dev)
            self.seq_ws_bytes = max(16, L.moe_seq_balance_workspace_bytes(T, s.E, seq_len))
            self.seq_ws = torch.empty((self.seq_ws_bytes,), dtype=torch.uint8, device=dev)
            self._seq_len = seq_len
        return self

    @property
    def hgu(self):
        """bf16 gate+up outputs kept by forward(keep_gu=True) for the backward
        (allocated on first use)."""
        if self._hgu is None:
            self._hgu = torch.empty((self.R, 2 * self._shape.I), dtype=torch.bfloat16,
                                    device=self._dev)
        return self._hgu


class BackwardBuffers:
    """Device buffers of one layer backward at T tokens (reused across calls)."""

    def dense(self):
        """Buffers of the dense router backward (allocated on first use):
        dlogit [T, E] fp32 and its workspace."""
        if self.dlogit is None:
            s, T = self._shape, self.T
            self.dlogit = torch.empty((max(T, 1), s.E), dtype=torch.float32, device=self._dev)
            self.dense_ws_bytes = max(16, L.moe_router_backward_dense_workspace_bytes(T, s.H, s.E))
            self.dense_ws = torch.empty((self.dense_ws_bytes,), dtype=torch.uint8, device=self._dev)
        return self

    def intermediates(self):
        """Allocate the bf16 dGU [R, 2I] and h [R, I] that a backward with
        keep_intermediates writes (the GEMMs read only their FP8 codes)."""
        if self.dgu is None:
            I = self._shape.I
            self.dgu = torch.empty((self.R, 2 * I), dtype=torch.bfloat16, device=self._dev)
            self.h = torch.empty((self.R, I), dtype=torch.bfloat16, device=self._dev)
        return self

    def __init__(self, shape: LayerShape, T: int, device="cuda"):
        s = shape
        R = T * s.k + s.n_shared * T
        dev = torch.device(device)
        u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
        H, I = s.H, s.I
        self.T, self.R = T, R
        self.dD = torch.empty((R, H), dtype=bf, device=dev)
        self.dw = torch.empty((T, s.k), dtype=f32, device=dev)
        self.dDq = torch.empty((R, H), dtype=u8, device=dev)
        self.dDs = torch.empty((R, H // 128), dtype=f32, device=dev)
        self.dh = torch.empty((R, I), dtype=bf, device=dev)
        self.gu = torch.empty((R, 2 * I), dtype=bf, device=dev)
        self.dgu = self.h = None   # bf16 dGU and h: only with keep_intermediates
        self.dguq = torch.empty((R, 2 * I), dtype=u8, device=dev)
        self.dgus = torch.empty((R, 2 * I // 128), dtype=f32, device=dev)
        self.dxp = torch.empty((R, H), dtype=bf, device=dev)
        self.dx = torch.empty((T, H), dtype=bf, device=dev)
        self.ones = torch.ones((T, s.k), dtype=f32, device=dev)
        self.cap = L.wgrad_chunks(R, s.G)
        c = self.cap
        self.c_dD = torch.empty((c, H, 128), dtype=u8, device=dev)
        self.s_dD = torch.empty((c, H), dtype=f32, device=dev)
        self.c_h = torch.empty((c, I, 128), dtype=u8, device=dev)
        self.s_h = torch.empty((c, I), dtype=f32, device=dev)
        self.c_dgu = torch.empty((c, 2 * I, 128), dtype=u8, device=dev)
        self.s_dgu = torch.empty((c, 2 * I), dtype=f32, device=dev)
        self.c_x = torch.empty((c, H, 128), dtype=u8, device=dev)
        self.s_x = torch.empty((c, H), dtype=f32, device=dev)
        self.dW_gu = torch.empty((s.G, 2 * I, H), dtype=f32, device=dev)
        self.dW_dn = torch.empty((s.G, H, I), dtype=f32, device=dev)
        self.dx_total = torch.empty((T, H), dtype=bf, device=dev)
        self._shape, self._dev, self.dlogit = s, dev, None
        self.dlogit_rows = torch.empty((max(T * s.k, 1),), dtype=f32, device=dev)
        self.dC = torch.empty((s.E, H), dtype=f32, device=dev)


class MoELayer:
    """One MoE layer on one GPU: router state and FP8 expert weights.

    Weights are E4M3 with 128x128 scales:
      w_gu [G, 2I, H] (rows [0, I) gate, [I, 2I) up), w_gu_s [G, 2I/128, H/128]
      w_dn [G, H, I],                                  w_dn_s [G, H/128, I/128]
    Group E (the last) is the shared expert.
    """

    def __init__(self, shape: LayerShape, centroids, bias, w_gu, w_gu_s, w_dn, w_dn_s):
        self.shape = shape
        self.centroids = centroids
        self.bias = bias
        self.w_gu, self.w_gu_s, self.w_dn, self.w_dn_s = w_gu, w_gu_s, w_dn, w_dn_s
        self._bwd = {}
        self._bufs = {}
        self._side = None   # stream for x's quantisation beside the router (lazily made)

    @staticmethod
    def empty_weights(shape: LayerShape, device="cuda"):
        s = shape
        dev = torch.device(device)
        return (torch.empty((s.G, 2 * s.I, s.H), dtype=torch.uint8, device=dev),
                torch.empty((s.G, 2 * s.I // 128, s.H // 128), dtype=torch.float32, device=dev),
                torch.empty((s.G, s.H, s.I), dtype=torch.uint8, device=dev),
                torch.empty((s.G, s.H // 128, s.I // 128), dtype=torch.float32, device=dev))

    @staticmethod
    def quantize_into(w_f32, out_q, out_s, stream=None):
        """128x128 block quantisation of fp32 weights [G', N, K] into E4M3 + scales."""
        G, N, K = w_f32.shape
        L.fp8_quant_128x128(w_f32, G, N, K, out_q, out_s, stream)

    @classmethod
    def from_fp32_experts(cls, shape: LayerShape, centroids, bias, gu_fp32, dn_fp32,
                          device="cuda"):
        """Build a layer from per-expert fp32 weights, quantised on the GPU.

        gu_fp32 / dn_fp32: iterables of (expert, array [2I, H] / [H, I]) covering
        every group 0..G-1 (G-1 is the shared expert).  Each array is copied
        to the GPU and quantised in 128x128 blocks by fp8_quant_128x128.
        """
        w_gu, w_gu_s, w_dn, w_dn_s = cls.empty_weights(shape, device)
        stream = torch.cuda.current_stream()
        for src, q, s in ((gu_fp32, w_gu, w_gu_s), (dn_fp32, w_dn, w_dn_s)):
            for e, arr in src:
                t = torch.from_numpy(arr).to(device)
                cls.quantize_into(t[None], q[e:e + 1], s[e:e + 1], stream)
                stream.synchronize()
        return cls(shape, centroids, bias, w_gu, w_gu_s, w_dn, w_dn_s)

    def buffers(self, T: int) -> Buffers:
        b = self._bufs.get(T)
        if b is None:
            b = self._bufs[T] = Buffers(self.shape, T, self.centroids.device)
        return b

    def forward(self, x_bf16: torch.Tensor, bufs: Buffers | None = None, stream=None,
                update_bias: bool = False, gamma: float = 0.001,
                events: dict | None = None,
                seq_len: int | None = None, alpha: float = 0.0001,
                keep_gu: bool = False) -> torch.Tensor:
        """One layer forward.  With seq_len, also the sequence-wise balance
        statistic of the routing (factor alpha) over consecutive runs of
        seq_len tokens, into bufs.seq_f, seq_p and seq_loss.  keep_gu (for
        training): the fused gate+up kernel also writes its bf16 gate/up
        outputs into bufs.hgu (1.2 GB at T=16384), which the backward then
        reads instead of running the gate+up GEMM again; the layer's output
        is unchanged.  `events`, if
        given, maps a step name ("route", "seq_balance", "quant", "permute",
        "gate_up", "down", "combine", "bias") to a list that receives a
        (start, end) pair of torch.cuda.Event recorded on the launch stream
        around that step (quant: on the side stream it runs on); a dict that
        already holds keys times only those steps (each event pair adds a few
        microseconds to the step).

        x's 1x128 quantisation does not depend on the routing: it runs on a
        side stream (default priority) that forks from the launch stream
        before the router and joins it before the first expert GEMM, so the
        two overlap."""
        s = self.shape
        T = x_bf16.shape[0]
        b = bufs or self.buffers(T)
        R = b.R
        b.gu_kept = keep_gu
        st = stream if stream is not None else torch.cuda.current_stream()
        if self._side is None:
            self._side = torch.cuda.Stream(device=st.device)
        side = self._side
        only = set(events) if events else None

        def step(name, on, fn):
            if events is None or (only is not None and name not in only):
                fn()
                return
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(on)
            fn()
            e1.record(on)
            events.setdefault(name, []).append((e0, e1))

        side.wait_stream(st)
        step("quant", side, lambda: L.fp8_quant_1x128(x_bf16, T, s.H, s.H, 0, b.xq, b.xs, side))
        step("route", st, lambda: self._route(x_bf16, b, seq_len, st))
        if seq_len is not None:
            step("seq_balance", st, lambda: self._seq_balance(b, seq_len, alpha, st))
        step("permute", st, lambda: L.moe_permute(
            b.topk_idx, b.counts, T, s.k, s.E, s.n_shared, b.offsets, b.perm_src, b.inv_perm,
            None, None, s.H, None, None, b.perm_ws, b.perm_ws_bytes, st))
        st.wait_stream(side)
        if keep_gu:
            step("gate_up", st, lambda: L.grouped_fp8_gemm_swiglu_keep(
                b.xq, b.xs, b.perm_src, self.w_gu, self.w_gu_s, b.offsets, s.G, R, s.I, s.H,
                b.hq, b.hs, b.hgu, st))
        else:
            step("gate_up", st, lambda: L.grouped_fp8_gemm_swiglu(
                b.xq, b.xs, b.perm_src, self.w_gu, self.w_gu_s, b.offsets, s.G, R, s.I, s.H,
                b.hq, b.hs, st))
        step("down", st, lambda: L.grouped_fp8_gemm(
            b.hq, b.hs, None, self.w_dn, self.w_dn_s, b.offsets, s.G, R, s.H, s.I, b.d, st))
        shared = b.d[T * s.k:T * s.k + T] if s.n_shared else None
        step("combine", st, lambda: L.moe_combine(b.d, b.inv_perm, b.topk_w, shared, T, s.k,
                                                  s.H, b.y, st))
        if update_bias:
            step("bias", st, lambda: L.moe_bias_update(b.counts, self.bias, s.E, gamma, st))
        return b.y

    def requantize_from_fp32(self, gu_fp32, dn_fp32, stream=None):
        """Requantise both weight sets in place from fp32 master weights
        ([G, 2I, H] and [G, H, I] device tensors) in 128x128 blocks (the
        per-update cast after an optimizer step)."""
        s = self.shape
        L.fp8_quant_128x128(gu_fp32, s.G, 2 * s.I, s.H, self.w_gu, self.w_gu_s, stream)
        L.fp8_quant_128x128(dn_fp32, s.G, s.H, s.I, self.w_dn, self.w_dn_s, stream)

    def capture(self, x_bf16: torch.Tensor, bufs: Buffers | None = None, **forward_kw):
        """One forward captured as a HIP graph (torch.cuda.CUDAGraph); its
        replay() reruns the whole layer on the same buffers - write the next
        batch into x_bf16 first - with one launch.  The library only launches
        kernels (no allocation, no memset, no host synchronisation), so every
        step is capturable.  forward_kw as in forward (not events)."""
        T = x_bf16.shape[0]
        b = bufs or self.buffers(T)
        side = torch.cuda.Stream()   # default priority
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.forward(x_bf16, b, stream=side, **forward_kw)   # warm-up outside the capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.forward(x_bf16, b, stream=torch.cuda.current_stream(), **forward_kw)
        return graph

    def backward_buffers(self, T: int) -> BackwardBuffers:
        bb = self._bwd.get(T)
        if bb is None:
            bb = self._bwd[T] = BackwardBuffers(self.shape, T, self.centroids.device)
        return bb

    def backward(self, dy_bf16: torch.Tensor, x_bf16: torch.Tensor, bufs: Buffers | None = None,
                 bwd: BackwardBuffers | None = None, stream=None, events: dict | None = None,
                 seq_len: int | None = None, alpha: float = 0.0001,
                 keep_intermediates: bool = False):
        """Backward of the layer for the output gradient dy, after a forward of
        x on `bufs` (its routing, permutation, quantised x and D).  With
        seq_len (the forward's, which left the scores and f in `bufs`), the
        loss also holds the sequence-wise balance term alpha * sum_b L_bal,b
        and the router's backward is the dense one (bwd.dlogit [T, E]).
        After a forward with keep_gu the gate+up outputs are read from
        bufs.hgu; otherwise the gate+up GEMM runs again (into bwd.gu).
        Returns the BackwardBuffers: dx_total (the input gradient), dx (its
        expert-path part), dw (gate weights), dC (centroids), dW_gu, dW_dn.
        keep_intermediates: also write the bf16 dGU and h (bwd.dgu, bwd.h),
        which the step itself does not need (its GEMMs read their codes).
        `events` as in forward, keys "combine_bwd", "dgrad_down",
        "recompute_gate_up", "swiglu_bwd", "dgrad_gate_up", "unpermute",
        "wgrad_down", "wgrad_gate_up", "router_bwd"."""
        s = self.shape
        T = dy_bf16.shape[0]
        b = bufs or self.buffers(T)
        bb = bwd or self.backward_buffers(T)
        if keep_intermediates:
            bb.intermediates()
        R, G, H, I, k, cap = b.R, s.G, s.H, s.I, s.k, bb.cap
        st = stream if stream is not None else torch.cuda.current_stream()

        def step(name, fn):
            if events is None:
                fn()
                return
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            fn()
            e1.record(st)
            events.setdefault(name, []).append((e0, e1))

        # the combine and SwiGLU backward also write the 1x128 quantisation of
        # their bf16 gradients (the input-gradient GEMMs' operands)
        step("combine_bwd", lambda: L.moe_combine_backward(
            dy_bf16, b.inv_perm, b.topk_w, b.d, T, k, H, s.n_shared, bb.dD, bb.dw, st,
            d_expert_out_e4m3=bb.dDq, d_expert_out_scale=bb.dDs))
        step("dgrad_down", lambda: L.grouped_fp8_gemm_dgrad(
            bb.dDq, bb.dDs, self.w_dn, self.w_dn_s, b.offsets, G, R, H, I, bb.dh, st))
        if getattr(b, "gu_kept", False):
            gu = b.hgu   # kept by the forward (keep_gu): the same bf16 GEMM output
        else:
            gu = bb.gu
            step("recompute_gate_up", lambda: L.grouped_fp8_gemm(
                b.xq, b.xs, b.perm_src, self.w_gu, self.w_gu_s, b.offsets, G, R, 2 * I, H, gu,
                st))
        # the SwiGLU backward also writes dGU's 1x128 codes and the 128x1 chunk
        # codes of dGU and h that the input and weight gradients read
        step("swiglu_bwd", lambda: L.swiglu_backward_grouped(
            gu, bb.dh, b.offsets, G, R, I, bb.dgu if keep_intermediates else None,
            bb.h if keep_intermediates else None, bb.dguq, bb.dgus, cap, bb.c_dgu,
            bb.s_dgu, bb.c_h, bb.s_h, st))
        step("dgrad_gate_up", lambda: L.grouped_fp8_gemm_dgrad(
            bb.dguq, bb.dgus, self.w_gu, self.w_gu_s, b.offsets, G, R, 2 * I, H, bb.dxp, st))
        shared = bb.dxp[T * k:T * k + T] if s.n_shared else None
        step("unpermute", lambda: L.moe_combine(bb.dxp, b.inv_perm, bb.ones, shared, T, k, H,
                                                bb.dx, st))
        step("wgrad_down", lambda: (
            L.fp8_quant_128x1_grouped(bb.dD, H, None, b.offsets, G, R, H, bb.c_dD, bb.s_dD, cap, st),
            L.grouped_fp8_wgrad(bb.c_dD, bb.s_dD, bb.c_h, bb.s_h, cap, b.offsets, G, R, H, I,
                                bb.dW_dn, st)))
        step("wgrad_gate_up", lambda: (
            L.fp8_quant_128x1_grouped(x_bf16, H, b.perm_src, b.offsets, G, R, H, bb.c_x, bb.s_x,
                                      cap, st),
            L.grouped_fp8_wgrad(bb.c_dgu, bb.s_dgu, bb.c_x, bb.s_x, cap, b.offsets, G, R, 2 * I, H,
                                bb.dW_gu, st)))
        if seq_len is None:
            step("router_bwd", lambda: (
                L.moe_router_backward(x_bf16, self.centroids, b.topk_idx, bb.dw, b.inv_perm, bb.dx,
                                      T, H, s.E, k, bb.dx_total, bb.dlogit_rows, st,
                                      topk_s=b.topk_s),
                L.moe_router_dcentroids(x_bf16, b.perm_src, b.offsets, bb.dlogit_rows, T, H, s.E,
                                        bb.dC, st)))
        else:
            if getattr(b, "_seq_len", None) != seq_len:
                raise ValueError("backward with seq_len needs the forward run with the same seq_len")
            bb.dense()
            step("router_bwd", lambda: L.moe_router_backward_dense(
                x_bf16, self.centroids, b.topk_idx, bb.dw, b.scores, b.score_sums, b.seq_f, T, H,
                s.E, k, seq_len, alpha, bb.dx, bb.dx_total, bb.dC, bb.dlogit, bb.dense_ws,
                bb.dense_ws_bytes, st))
        return bb

    def _route(self, x_bf16, b, seq_len, stream):
        s = self.shape
        T = x_bf16.shape[0]
        if seq_len is None:
            L.moe_route(x_bf16, T, s.H, self.centroids, self.bias, s.E, s.n_group, s.topk_group,
                        s.k, b.topk_idx, b.topk_w, b.counts, b.route_ws, b.route_ws_bytes, stream,
                        topk_s=b.topk_s)
        else:
            b.balance(seq_len)
            L.moe_route_scores(x_bf16, T, s.H, self.centroids, self.bias, s.E, s.n_group,
                               s.topk_group, s.k, b.topk_idx, b.topk_w, b.counts, b.route_ws,
                               b.route_ws_bytes, b.scores, b.score_sums, stream, topk_s=b.topk_s)

    def _seq_balance(self, b, seq_len, alpha, stream):
        s = self.shape
        L.moe_seq_balance(b.scores, b.score_sums, b.topk_idx, b.T, s.E, s.k, seq_len, alpha,
                          b.seq_f, b.seq_p, b.seq_loss, b.seq_ws, b.seq_ws_bytes, stream)

