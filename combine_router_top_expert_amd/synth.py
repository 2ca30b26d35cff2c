"""Seeded synthetic inputs for the MoE layer workloads.

This module is shared by the HIP path's tests/benchmark and by the CPU oracle's
tests.  It holds no arithmetic of the layer itself (no logits, no top-k over
logits, no softmax, no expert FFN): only random numbers, their rounding to the
storage dtype, and the shapes and distributions of the five workloads.

Generator: counter-based.  Value ``i`` of a tensor with seed ``s`` is built from
SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014: the 64-bit finaliser with constants 0x9E3779B97F4A7C15,
0xBF58476D1CE4E5B9 and 0x94D049BB133111EB), turned into a uniform in (0, 1)
from its top 53 bits, and into normals by the Box-Muller transform (one pair of
uniforms gives two normals).  Values are drawn in float64 and rounded once,
round-to-nearest-even, to the storage dtype (fp32 or bf16).

The workloads follow the configurations the layer is measured on (MoE layer of
the Mixture-of-Kittens write-ups: dispatch, SwiGLU expert FFN, combine).  Sizes,
distributions and the routing skew are restated in ``WORKLOADS``.
"""
from __future__ import annotations

import dataclasses
import math
import os
from typing import Dict, List, Optional

import numpy as np

_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)
_G = np.uint64(0x9E3779B97F4A7C15)
_C1 = np.uint64(0xBF58476D1CE4E5B9)
_C2 = np.uint64(0x94D049BB133111EB)

SEED_BASE = 0x4D6F4B00

REPO_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN_DIR = os.path.join(REPO_ROOT, "tests", "golden")


def _mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser on a uint64 array (wrapping arithmetic)."""
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _C1
        z = (z ^ (z >> np.uint64(27))) * _C2
        z = z ^ (z >> np.uint64(31))
    return z


def raw_u64(seed: int, start: int, n: int) -> np.ndarray:
    """Counter-based stream: word i = mix(mix(seed) + (i + 1) * golden)."""
    key = _mix64(np.array([seed & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))[0]
    ctr = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = key + ctr * _G
    return _mix64(z)


def uniform(seed: int, n: int, start: int = 0) -> np.ndarray:
    """Uniforms in the open interval (0, 1), float64."""
    u = raw_u64(seed, start, n)
    return ((u >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def normal(seed: int, n: int, std: float = 1.0, start: int = 0) -> np.ndarray:
    """N(0, std^2) float64 by Box-Muller over consecutive uniform pairs.

    ``start`` must be even so that pairs line up across chunked calls.
    """
    assert start % 2 == 0
    npair = (n + 1) // 2
    u = uniform(seed, 2 * npair, start=start)
    u1 = u[0::2]
    u2 = u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    th = (2.0 * math.pi) * u2
    out = np.empty(2 * npair, dtype=np.float64)
    out[0::2] = r * np.cos(th)
    out[1::2] = r * np.sin(th)
    return out[:n] * std


# ---------------------------------------------------------------- storage rounding
def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 bit patterns (uint16), via fp32 then RNE on the bits."""
    f = np.ascontiguousarray(v, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- workloads
@dataclasses.dataclass
class Workload:
    """Shapes and the recipe of one synthetic workload."""

    name: str
    index: int            # 1-based config number, part of every seed
    S: int                # simulated source-rank token buffers
    T_src: int            # tokens per source buffer
    d: int                # hidden size
    E: int                # experts in the layer
    k: int                # experts chosen per token
    I: int                # SwiGLU intermediate size per expert
    prec: str             # "f32" | "bf16" | "mxfp8"
    router_std: float     # std of the router weights
    own: List[int]        # source buffers routed and final-combined here
    local_experts: List[int]  # experts whose FFN runs here, in local order
    zipf_s: float = 0.0   # 0 => no bias; else popularity follows Zipf(s)
    ring_bytes: int = 0   # 0 => staged path
    minibatch_rows: int = 256

    @property
    def E_local(self) -> int:
        return len(self.local_experts)

    @property
    def T_total(self) -> int:
        return self.S * self.T_src

    @property
    def act_dtype(self) -> str:
        return "f32" if self.prec == "f32" else "bf16"

    def expert_to_local(self) -> np.ndarray:
        m = np.full(self.E, -1, dtype=np.int32)
        for i, e in enumerate(self.local_experts):
            m[e] = i
        return m

    def seed(self, tensor_id: int) -> int:
        return SEED_BASE + 16 * self.index + tensor_id

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


MiB = 1 << 20

# C1..C5 as stated for the measured layer; "N(0, s)" means std s, fan_in is d for
# the router, W_gate and W_up, and I for W_down.
WORKLOADS: Dict[str, Workload] = {
    # Tiny layer forward, fp32 throughout, one source buffer.
    "C1": Workload("C1", 1, S=1, T_src=512, d=256, E=8, k=2, I=512, prec="f32",
                   router_std=1.0 / math.sqrt(256), own=[0], local_experts=list(range(8))),
    # Mid layer, bf16, balanced routing, 8 source buffers of 2048 tokens.
    "C2": Workload("C2", 2, S=8, T_src=2048, d=2048, E=64, k=6, I=1408, prec="bf16",
                   router_std=1e-3, own=list(range(8)), local_experts=list(range(64)),
                   ring_bytes=256 * MiB, minibatch_rows=256),
    # One GPU's share of a 256-expert layer: 32 source buffers of 4096 tokens, this
    # GPU (rank 7) owns experts {7, 39, ..., 231}; Zipf(1.2) skew; 256 MiB ring.
    "C3": Workload("C3", 3, S=32, T_src=4096, d=7168, E=256, k=8, I=2048, prec="bf16",
                   router_std=1.0 / math.sqrt(7168), own=[7],
                   local_experts=[7 + 32 * i for i in range(8)], zipf_s=1.2,
                   ring_bytes=256 * MiB, minibatch_rows=256),
    # C2 in MXFP8 (e4m3 elements, one e8m0 scale per 32 along the contraction dim).
    "C4": Workload("C4", 4, S=8, T_src=2048, d=2048, E=64, k=6, I=1408, prec="mxfp8",
                   router_std=1e-3, own=list(range(8)), local_experts=list(range(64)),
                   ring_bytes=256 * MiB, minibatch_rows=256),
    # Backward of the C2-shaped layer with Zipf(1.2) skew over its 64 experts.
    "C5": Workload("C5", 5, S=8, T_src=2048, d=2048, E=64, k=6, I=1408, prec="bf16",
                   router_std=1e-3, own=list(range(8)),
                   local_experts=list(range(64)), zipf_s=1.2,
                   ring_bytes=256 * MiB, minibatch_rows=256),
}

# tensor ids inside a workload's seed space
TID_X, TID_WR, TID_WG, TID_WU, TID_WD, TID_DOUT, TID_OTHER, TID_CAL = 0, 1, 2, 3, 4, 5, 6, 7


def zipf_popularity(E: int, k: int, s: float) -> np.ndarray:
    """Per-expert probability that a token picks it: proportional to (e+1)^-s,
    capped at 1 (a token picks an expert at most once), summing to k."""
    w = (np.arange(E, dtype=np.float64) + 1.0) ** (-s)
    lo, hi = 0.0, float(k) / w.min()
    for _ in range(200):
        c = 0.5 * (lo + hi)
        if np.minimum(1.0, c * w).sum() < k:
            lo = c
        else:
            hi = c
    return np.minimum(1.0, hi * w)


def bias_file(w: Workload) -> str:
    return os.path.join(GOLDEN_DIR, f"zipf_bias_E{w.E}_k{w.k}_d{w.d}.txt")


def load_bias(w: Workload) -> Optional[np.ndarray]:
    """Router bias (fp32) for a skewed workload, from its stored calibration file.

    The file is written by tests/golden/make_zipf_bias.py (which calls only the
    CPU oracle).  Unskewed workloads have no bias (None).
    """
    if w.zipf_s == 0.0:
        return None
    path = bias_file(w)
    vals = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            vals.append(float.fromhex(line))
    b = np.array(vals, dtype=np.float32)
    assert b.shape == (w.E,), (path, b.shape)
    return b


def _round_store(v: np.ndarray, dtype: str):
    """Return (storage array, fp32 value array)."""
    if dtype == "f32":
        f = v.astype(np.float32)
        return f, f
    bits = f64_to_bf16_bits(v)
    return bits, bf16_bits_to_f32(bits)


def gen_tensor(w: Workload, tid: int, shape, std: float, dtype: str, start: int = 0):
    n = int(np.prod(shape))
    v = normal(w.seed(tid), n, std=std, start=start).reshape(shape)
    return _round_store(v, dtype)


def gen_x(w: Workload, s: int):
    """Source buffer s: [T_src, d] tokens ~ N(0, 1)."""
    n = w.T_src * w.d
    assert n % 2 == 0
    return gen_tensor(w, TID_X, (w.T_src, w.d), 1.0, w.act_dtype, start=s * n)


def gen_router(w: Workload):
    return gen_tensor(w, TID_WR, (w.E, w.d), w.router_std, w.act_dtype)


def gen_expert_weights(w: Workload, which: str, le: Optional[int] = None):
    """W_gate / W_up: [E_local, I, d] with std 1/sqrt(d); W_down: [E_local, d, I]
    with std 1/sqrt(I).  Expert weights are stored in the activation dtype (bf16
    for the MXFP8 workload too: they are quantised once, off the timed path).
    ``le`` selects one local expert (its slice of the same stream)."""
    tid = {"gate": TID_WG, "up": TID_WU, "down": TID_WD}[which]
    std = 1.0 / math.sqrt(w.d if which != "down" else w.I)
    shape = (w.I, w.d) if which != "down" else (w.d, w.I)
    per = shape[0] * shape[1]
    assert per % 2 == 0
    if le is None:
        return gen_tensor(w, tid, (w.E_local,) + shape, std, w.act_dtype)
    return gen_tensor(w, tid, shape, std, w.act_dtype, start=le * per)


def gen_dout(w: Workload, s: int):
    """Upstream gradient for source buffer s: [T_src, d] ~ N(0, 1)."""
    n = w.T_src * w.d
    assert n % 2 == 0
    return gen_tensor(w, TID_DOUT, (w.T_src, w.d), 1.0, w.act_dtype, start=s * n)


def gen_other_routing(w: Workload, s: int):
    """Routing of a source buffer that is not routed here (it stands for another
    rank's router output, an input to this GPU's share).

    Expert choices: k distinct experts per token by Gumbel-top-k sampling from the
    workload's popularity (Zipf when skewed, uniform otherwise).  Gate values: k
    uniforms sorted in descending order and divided by their sum.
    Returns (topk_idx [T_src, k] int32, topk_gate [T_src, k] fp32).
    """
    E, k, T = w.E, w.k, w.T_src
    if w.zipf_s:
        logp = np.log(zipf_popularity(E, k, w.zipf_s))
    else:
        logp = np.zeros(E)
    u = uniform(w.seed(TID_OTHER) + 1000 * s, T * E).reshape(T, E)
    key = logp[None, :] - np.log(-np.log(u))
    idx = np.argsort(-key, axis=1, kind="stable")[:, :k].astype(np.int32)
    g = np.sort(uniform(w.seed(TID_OTHER) + 1000 * s + 500, T * k).reshape(T, k), axis=1)[:, ::-1]
    g = (g / g.sum(axis=1, keepdims=True)).astype(np.float32)
    return np.ascontiguousarray(idx), np.ascontiguousarray(g)


def gen_calibration_tokens(w: Workload, n: int):
    """Separate token batch used only to calibrate the skew bias."""
    return gen_tensor(w, TID_CAL, (n, w.d), 1.0, w.act_dtype)


def scaled(w: Workload, **kw) -> Workload:
    """A smaller variant of a workload for parity tests (same recipe and dtype)."""
    return w.replace(**kw)
