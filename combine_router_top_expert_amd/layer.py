"""Device buffers of one MoE layer instance, allocated with torch.

``MoELayer`` owns the caller-side memory the C ABI expects (configuration,
weights, forward state, staging rows, outputs, gradients, workspace, device
status word) and calls ``mok_layer_fwd`` / ``mok_layer_bwd``.  It does no
arithmetic of its own.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

from . import (MAX_SOURCES, AuxStream, make_config, make_state, make_weights, mok_layer_bwd, mok_layer_fwd,
               mok_prepare_bwd, mok_mx_quantize, mok_tune_fwd, mok_workspace_bytes, STATUS)


def _dt(prec: str):
    return torch.float32 if prec == "f32" else torch.bfloat16


def to_device(a: np.ndarray, prec: str, device) -> torch.Tensor:
    """Storage array from the input generator (fp32 values or bf16 bits) -> device tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class MoELayer:
    def __init__(self, S, T_src, d, E, k, I, E_local, prec, R_cap, own_lo, own_n, device="cuda",
                 ring_bytes=0, minibatch_rows=256, comm_wgs=0, gemm_wgs=0, with_bwd=True,
                 wait_limit_us=0, two_streams=True, bwd_ring_bytes=0, transposed_weights=True):
        assert S <= MAX_SOURCES
        self.S, self.T_src, self.d, self.E, self.k, self.I = S, T_src, d, E, k, I
        self.E_local, self.prec, self.R_cap = E_local, prec, R_cap
        self.own_lo, self.own_n = own_lo, own_n
        self.device = torch.device(device)
        self.cfg = make_config(S, T_src, d, E, k, I, E_local, prec, R_cap, minibatch_rows,
                               ring_bytes, comm_wgs, gemm_wgs, wait_limit_us, bwd_ring_bytes)
        dev = self.device
        act = _dt(prec)
        N = S * T_src * k
        self.topk_idx = torch.zeros(max(N, 1), dtype=torch.int32, device=dev)
        self.topk_gate = torch.zeros(max(N, 1), dtype=torch.float32, device=dev)
        self.counts = torch.zeros(E_local, dtype=torch.int32, device=dev)
        self.offsets = torch.zeros(E_local + 1, dtype=torch.int32, device=dev)
        self.row_src = torch.zeros(max(R_cap, 1), dtype=torch.int32, device=dev)
        self.dest_row = torch.zeros(max(N, 1), dtype=torch.int32, device=dev)
        if prec == "mxfp8":
            self.h = torch.zeros(max(R_cap, 1) * I, dtype=torch.uint8, device=dev)
        else:
            self.h = torch.zeros(max(R_cap, 1), I, dtype=act, device=dev)
        self.ab = torch.zeros(max(R_cap, 1), 2 * I, dtype=act, device=dev) if with_bwd or prec != "mxfp8" else None
        out_dt = torch.float32 if prec == "f32" else torch.bfloat16
        self.staging = [torch.zeros(T_src * k, d, dtype=out_dt, device=dev) for _ in range(S)]
        self.out = [torch.zeros(T_src, d, dtype=out_dt, device=dev) if own_lo <= s < own_lo + own_n
                    else None for s in range(S)]
        self.ws = torch.zeros(max(mok_workspace_bytes(self.cfg), 256), dtype=torch.uint8,
                              device=dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        # the bf16 backward runs its side work on a second stream (mok_aux)
        self.aux = None
        if two_streams and with_bwd and prec == "bf16" and not bwd_ring_bytes:
            self.aux = AuxStream(dev)
            self.aux.attach(self.cfg)
        # MXFP8: h holds E4M3 codes; its scales are kept for the backward
        self.h_scale = (torch.zeros(max(R_cap, 1) * I // 32, dtype=torch.uint8, device=dev)
                        if prec == "mxfp8" and with_bwd else None)
        self.state = make_state(self.topk_idx, self.topk_gate, self.counts, self.offsets,
                                self.row_src, self.dest_row, self.h, self.ab, self.h_scale)
        self.with_bwd = with_bwd
        # bf16 backward: the weights also transposed (mok_prepare_bwd), so dh
        # and dx read them k-contiguous (bit-identical either way)
        self.transposed_weights = transposed_weights
        if with_bwd:
            self.d_gate = torch.zeros(max(N, 1), dtype=torch.float32, device=dev)
            self.dx_stage = [torch.zeros(T_src * k, d, dtype=act, device=dev) for _ in range(S)]
            self.d_x = [torch.zeros(T_src, d, dtype=act, device=dev) if own_lo <= s < own_lo + own_n
                        else None for s in range(S)]
            self.dw_gate = torch.zeros(E_local, I, d, dtype=torch.float32, device=dev)
            self.dw_up = torch.zeros(E_local, I, d, dtype=torch.float32, device=dev)
            self.dw_down = torch.zeros(E_local, d, I, dtype=torch.float32, device=dev)
            self.dw_router = torch.zeros(E, d, dtype=torch.float32, device=dev)

    # ---------------------------------------------------------------- inputs
    def set_inputs(self, xs: List[torch.Tensor], w_router, bias, e2l, w_gate, w_up, w_down,
                   other_topk: Optional[List] = None):
        """xs: S device tensors [T_src, d]; other_topk: per non-own source
        (topk_idx [T_src, k] int32, topk_gate [T_src, k] fp32) numpy arrays."""
        self.xs = xs
        self.w_router = w_router
        self.bias = bias
        self.e2l = e2l
        self.w_gate, self.w_up, self.w_down = w_gate, w_up, w_down
        per = self.T_src * self.k
        for s in range(self.S):
            if self.own_lo <= s < self.own_lo + self.own_n:
                continue
            idx, g = other_topk[s]
            self.topk_idx[s * per:(s + 1) * per] = torch.from_numpy(idx.reshape(-1)).to(self.device)
            self.topk_gate[s * per:(s + 1) * per] = torch.from_numpy(g.reshape(-1)).to(self.device)
        if self.prec == "mxfp8":
            self._quantize_weights()
        elif self.prec == "bf16" and self.with_bwd and self.transposed_weights:
            E, d, I = self.E_local, self.d, self.I
            self.wt = [torch.empty(E * I * d, dtype=torch.bfloat16, device=self.device),
                       torch.empty(E * d * 2 * I, dtype=torch.bfloat16, device=self.device)]
            mok_prepare_bwd(self.cfg, w_gate, w_up, w_down, self.wt[0], None, self.wt[1], None)
            self.weights = make_weights(w_gate, w_up, w_down, wt_down=self.wt[0],
                                        wt_gu=self.wt[1])
        else:
            self.weights = make_weights(w_gate, w_up, w_down)

    def set_peer_slots(self, s: int, y: torch.Tensor, d_gate: torch.Tensor,
                       dx: Optional[torch.Tensor] = None):
        """What the GPUs holding remote experts write back to own source s:
        y [T_src*k, d] into its staging rows, d_gate [T_src*k] and dx
        [T_src*k, d] into its reverse-dispatch rows.  The layer overwrites the
        rows of local slots on every pass, so only remote slots keep them."""
        per = self.T_src * self.k
        self.staging[s].copy_(y)
        if self.with_bwd:
            self.d_gate[s * per:(s + 1) * per].copy_(d_gate)
            if dx is not None:
                self.dx_stage[s].copy_(dx)

    def _quantize_weights(self):
        """MX-quantise the expert weights once (off the timed path)."""
        q = []
        for w in (self.w_gate, self.w_up, self.w_down):
            rows = w.numel() // w.shape[-1]
            K = w.shape[-1]
            codes = torch.empty(w.numel(), dtype=torch.uint8, device=self.device)
            scales = torch.empty(w.numel() // 32, dtype=torch.uint8, device=self.device)
            mok_mx_quantize(rows, K, w, codes, scales)
            q.append((codes, scales))
        self.wq = q
        t = [None] * 4
        if self.with_bwd:
            # the backward's transposed operands: W_down^T and [W_gate; W_up]^T
            E, d, I = self.E_local, self.d, self.I
            t = [torch.empty(E * I * d, dtype=torch.uint8, device=self.device),
                 torch.empty(E * I * d // 32, dtype=torch.uint8, device=self.device),
                 torch.empty(E * d * 2 * I, dtype=torch.uint8, device=self.device),
                 torch.empty(E * d * 2 * I // 32, dtype=torch.uint8, device=self.device)]
            mok_prepare_bwd(self.cfg, self.w_gate, self.w_up, self.w_down, *t)
        self.wt = t
        self.weights = make_weights(q[0][0], q[1][0], q[2][0], q[0][1], q[1][1], q[2][1], *t)

    # ---------------------------------------------------------------- passes
    def forward(self, stream=None):
        mok_layer_fwd(self.cfg, self.own_lo, self.own_n, self.xs, self.w_router, self.bias,
                      self.e2l, self.weights, self.state, self.staging, self.out, self.ws,
                      self.status, stream)

    def tune(self, mbs=None, comms=None, reps=3, stream=None):
        """Pick the fused path's minibatch size and dispatch/GEMM split with
        mok_tune_fwd (off the timed path; synchronises).  The workspace grows
        to fit every candidate first.  Returns {(minibatch_rows, comm_wgs):
        ms per forward or None}; self.cfg holds the fastest pair after."""
        mbs = list(mbs) if mbs is not None else [64, 128, 256, 512, 1024, 2048, 4096]
        need = self.ws.numel()
        for mb in mbs:
            c = type(self.cfg).from_buffer_copy(self.cfg)
            c.minibatch_rows = mb
            need = max(need, mok_workspace_bytes(c))
        if need > self.ws.numel():
            self.ws = torch.zeros(need, dtype=torch.uint8, device=self.device)
        best, table = mok_tune_fwd(self.cfg, mbs, comms, reps, self.ws.numel(), self.own_lo,
                                   self.own_n, self.xs, self.w_router, self.bias, self.e2l,
                                   self.weights, self.state, self.staging, self.out, self.ws,
                                   self.status, stream)
        self.cfg.minibatch_rows = best.minibatch_rows
        self.cfg.comm_wgs = best.comm_wgs
        self.cfg.gemm_wgs = best.gemm_wgs
        return table

    def backward(self, d_out: List[torch.Tensor], stream=None, router_grad=True):
        mok_layer_bwd(self.cfg, self.own_lo, self.own_n, d_out, self.xs, self.w_router, self.e2l,
                      self.weights, self.state, self.staging, self.d_gate, self.dx_stage, self.d_x,
                      self.dw_gate, self.dw_up, self.dw_down,
                      self.dw_router if router_grad else None, self.ws, self.status, stream)

    def check_status(self):
        st = int(self.status.item())
        if st != 0:
            raise RuntimeError(f"device status {STATUS.get(st, st)}")
