"""Shared test fixtures: a workload's seeded inputs, the oracle's expected
values for them, and device copies for the HIP path.  Expected values come
only from ``oracle/`` applied to generator output, never from the HIP path."""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

import oracle
from combine_router_top_expert_amd import synth


@dataclasses.dataclass
class HostCase:
    w: synth.Workload
    x_store: List[np.ndarray]      # per source, storage dtype
    x_val: List[np.ndarray]        # per source, fp32 values
    wr_store: np.ndarray
    wr_val: np.ndarray
    bias: Optional[np.ndarray]
    wg_store: np.ndarray
    wg_val: np.ndarray
    wu_store: np.ndarray
    wu_val: np.ndarray
    wd_store: np.ndarray
    wd_val: np.ndarray
    e2l: np.ndarray
    other: Dict[int, tuple]        # non-own sources: (topk_idx, topk_gate)
    # own sources of a share: what the GPUs holding the remote experts write
    # back (synth.gen_peer_slots: y store, y values, d_gate, dx store, dx values)
    peer: Dict[int, tuple] = dataclasses.field(default_factory=dict)
    # oracle results
    topk_all: np.ndarray = None    # [S, T_src, k]
    gate_all: np.ndarray = None    # [S, T_src, k] float64 (own: oracle gates)
    layout: dict = None

    @property
    def own(self):
        return self.w.own

    def R_cap(self) -> int:
        return max(int(self.layout["R"]), 1)


def make_host_case(w: synth.Workload, route_own=True) -> HostCase:
    xs = [synth.gen_x(w, s) for s in range(w.S)]
    wr = synth.gen_router(w)
    bias = synth.load_bias(w)
    wg = synth.gen_expert_weights(w, "gate")
    wu = synth.gen_expert_weights(w, "up")
    wd = synth.gen_expert_weights(w, "down")
    other = {s: synth.gen_other_routing(w, s) for s in range(w.S) if s not in w.own}
    c = HostCase(w, [a for a, _ in xs], [b for _, b in xs], wr[0], wr[1], bias, wg[0], wg[1], wu[0],
                 wu[1], wd[0], wd[1], w.expert_to_local(), other)
    if w.E_local < w.E:
        c.peer = {s: synth.gen_peer_slots(w, s) for s in w.own}
    if route_own:
        oracle_routing(c)
    return c


def oracle_routing(c: HostCase):
    w = c.w
    topk = np.zeros((w.S, w.T_src, w.k), np.int32)
    gate = np.zeros((w.S, w.T_src, w.k), np.float64)
    for s in range(w.S):
        if s in w.own:
            topk[s], gate[s] = oracle.route(c.x_val[s], c.wr_val, c.bias, w.k, w.prec)
        else:
            topk[s], gate[s] = c.other[s][0], c.other[s][1].astype(np.float64)
    c.topk_all, c.gate_all = topk, gate
    c.layout = oracle.layout(topk, c.e2l, w.E_local)


def oracle_weights(c: HostCase, le=None):
    """Expert weights as the layer uses them (MX round trip for MXFP8); le:
    only local expert le's ([I, d], [I, d], [d, I])."""
    vals = (c.wg_val, c.wu_val, c.wd_val) if le is None else (c.wg_val[le], c.wu_val[le],
                                                             c.wd_val[le])
    if c.w.prec != "mxfp8":
        return vals
    out = []
    for v in vals:
        K = v.shape[-1]
        codes, scales = oracle.mx_quantize(v.reshape(-1, K).astype(np.float64))
        out.append(oracle.mx_dequantize(codes, scales).astype(np.float32).reshape(v.shape))
    return tuple(out)


def peer_rows(c: HostCase, toks, which: int):
    """Peer-written values of the tokens' k slots (which: 1 = y rows, 2 =
    d_gate, 4 = dx rows), or None when every expert is local."""
    if not c.peer:
        return None
    k = c.w.k
    return np.stack([c.peer[s][which][t * k:(t + 1) * k] for s, t in toks])


def oracle_fwd_tokens(c: HostCase, toks):
    """toks: list of (s, t) -> (y [n, k, d], out [n, d]) from the oracle."""
    tok_x = np.stack([c.x_val[s][t] for s, t in toks])
    idx = np.stack([c.topk_all[s, t] for s, t in toks])
    g = np.stack([c.gate_all[s, t] for s, t in toks])
    wg, wu, wd = oracle_weights(c)
    return oracle.fwd_tokens(tok_x, idx, g, c.e2l, wg, wu, wd, c.w.prec,
                             peer_y=peer_rows(c, toks, 1))


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def sample_tokens(w: synth.Workload, n: int, seed: int = 0):
    """n own tokens incl. the first and last ones of each own source."""
    rng = np.random.default_rng(seed)
    toks = set()
    for s in w.own:
        toks.add((s, 0))
        toks.add((s, w.T_src - 1))
    while len(toks) < n:
        s = int(rng.choice(w.own))
        toks.add((s, int(rng.integers(w.T_src))))
    return sorted(toks)
