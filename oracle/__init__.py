"""CPU oracle of the fused MoE layer (plain C, float64) -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never do; the two implementations share no code.  ``build()`` compiles
``mok_oracle.c`` with gcc into ``libmok_oracle.so`` next to it.

Every function here is a thin numpy wrapper over one C function of
``mok_oracle.c``; each C function cites the passage of the pages it follows.
The composite helpers at the bottom (``route``, ``layout``, ``layer_fwd`` ...)
only chain those calls in the layer's order.  Two functions are written
with numpy instead: ``ffn_rows_exact``, the exact expert FFN of many rows,
with numpy's float64 matrix product as its contraction step, for checks at
sizes where the row-by-row C loops are too slow; and ``gate_grads``, the
gate gradients of rows whose expert outputs are given (one float64 dot
product per row).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mok_oracle.c")
LIB = os.path.join(HERE, "libmok_oracle.so")

F32, BF16, MXFP8, EXACT = 0, 1, 2, 3
PREC = {"f32": F32, "bf16": BF16, "mxfp8": MXFP8, "exact": EXACT}

_lib = None


def build(out: str = LIB, sanitize: bool = False) -> str:
    """Compile the oracle (single-threaded C; fmaf must be the hardware fused op).
    sanitize: an AddressSanitizer + UndefinedBehaviorSanitizer build (every
    report fatal) for the host-side memory and UB check; it is loaded only
    through MOK_ORACLE_LIB, with libasan preloaded into the process."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-mfma", "-ffp-contract=off", "-fPIC", "-shared"]
    if sanitize:
        cmd += ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                "-fno-sanitize-recover=all"]
    cmd += ["-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def lib():
    global _lib
    if _lib is None:
        alt = os.environ.get("MOK_ORACLE_LIB")
        if alt:
            _lib = ctypes.CDLL(alt)
            _declare(_lib)
            return _lib
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = ctypes.CDLL(LIB)
        _declare(_lib)
    return _lib


_p = ctypes.c_void_p
_i = ctypes.c_int64
_d = ctypes.c_double
_int = ctypes.c_int


def _declare(L):
    L.mokref_round_bf16.argtypes = [_d]
    L.mokref_round_bf16.restype = _d
    L.mokref_e4m3_decode.argtypes = [_int]
    L.mokref_e4m3_decode.restype = _d
    L.mokref_e4m3_encode.argtypes = [_d]
    L.mokref_e4m3_encode.restype = _int
    L.mokref_mx_quantize.argtypes = [_i, _i, _p, _p, _p]
    L.mokref_mx_dequantize.argtypes = [_i, _i, _p, _p, _p]
    L.mokref_logits.argtypes = [_i, _i, _i, _p, _p, _p, _int, _p]
    L.mokref_topk.argtypes = [_i, _i, _i, _p, _p]
    L.mokref_gates.argtypes = [_i, _i, _i, _p, _p, _p]
    L.mokref_route.argtypes = [_i, _i, _i, _i, _p, _p, _p, _int, _p, _p]
    L.mokref_layout.argtypes = [_i, _i, _i, _i, _p, _p, _i, _i, _p, _p, _p, _p]
    L.mokref_layout.restype = _i
    L.mokref_ffn_row.argtypes = [_i, _i, _int, _p, _p, _p, _p, _p, _p, _p, _p]
    L.mokref_fwd_tokens.argtypes = [_i, _i, _i, _i, _i, _int, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                    _p]
    L.mokref_bwd_row.argtypes = [_i, _i, _p, _d, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]
    L.mokref_router_bwd_token.argtypes = [_i, _i, _p, _p, _p, _p, _p, _p]
    L.mokref_bwd_tokens.argtypes = [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                    _p, _p, _p]
    L.mokref_expert_wgrad.argtypes = [_i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p]
    L.mokref_router_wgrad.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p]
    L.mokref_expert_bwd_mx.argtypes = [_i, _i, _i, _int, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                       _p, _p, _p]
    L.mokref_expert_wgrad_cols.argtypes = [_i, _i, _i, _p, _p, _p, _p, _p, _p, _i, _p, _p, _p,
                                           _p]


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


# ------------------------------------------------------------------ scalars / MX
def round_bf16(v: float) -> float:
    return lib().mokref_round_bf16(float(v))


def e4m3_decode(code: int) -> float:
    return lib().mokref_e4m3_decode(int(code))


def e4m3_encode(v: float) -> int:
    return lib().mokref_e4m3_encode(float(v))


def mx_quantize(v: np.ndarray):
    """v: [rows, K] -> (codes uint8 [rows, K], scales uint8 [rows, K/32])."""
    v = _c(v, np.float64)
    rows, K = v.shape
    assert K % 32 == 0
    codes = np.empty((rows, K), np.uint8)
    scales = np.empty((rows, K // 32), np.uint8)
    lib().mokref_mx_quantize(rows, K, _ptr(v), _ptr(codes), _ptr(scales))
    return codes, scales


def mx_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows, K = codes.shape
    out = np.empty((rows, K), np.float64)
    lib().mokref_mx_dequantize(rows, K, _ptr(codes), _ptr(scales), _ptr(out))
    return out


# ------------------------------------------------------------------ routing
def logits(x, wr, bias, prec) -> np.ndarray:
    x = _c(x, np.float32)
    wr = _c(wr, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    T, d = x.shape
    E = wr.shape[0]
    z = np.empty((T, E), np.float64)
    lib().mokref_logits(T, d, E, _ptr(x), _ptr(wr), _ptr(b), PREC.get(prec, prec), _ptr(z))
    return z


def topk(z, k) -> np.ndarray:
    z = _c(z, np.float64)
    T, E = z.shape
    idx = np.empty((T, k), np.int32)
    lib().mokref_topk(T, E, k, _ptr(z), _ptr(idx))
    return idx


def gates(z, idx) -> np.ndarray:
    z = _c(z, np.float64)
    idx = _c(idx, np.int32)
    T, E = z.shape
    k = idx.shape[1]
    g = np.empty((T, k), np.float64)
    lib().mokref_gates(T, E, k, _ptr(z), _ptr(idx), _ptr(g))
    return g


def route(x, wr, bias, k, prec):
    """-> (topk_idx int32 [T, k], gates float64 [T, k])."""
    x = _c(x, np.float32)
    wr = _c(wr, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    T, d = x.shape
    E = wr.shape[0]
    idx = np.empty((T, k), np.int32)
    g = np.empty((T, k), np.float64)
    lib().mokref_route(T, d, E, k, _ptr(x), _ptr(wr), _ptr(b), PREC.get(prec, prec), _ptr(idx),
                       _ptr(g))
    return idx, g


# ------------------------------------------------------------------ layout
def layout(topk_all, e2l, E_local, R_cap=None):
    """topk_all: [S, T_src, k] -> dict(counts, offsets, row_src, dest_row, R)."""
    t = _c(topk_all, np.int32)
    S, T_src, k = t.shape
    e2l = _c(e2l, np.int32)
    E = e2l.shape[0]
    N = S * T_src * k
    if R_cap is None:
        R_cap = N
    counts = np.empty(E_local, np.int32)
    offsets = np.empty(E_local + 1, np.int32)
    row_src = np.full(max(R_cap, 1), -1, np.int32)
    dest_row = np.empty(N, np.int32)
    R = lib().mokref_layout(S, T_src, k, E, _ptr(t), _ptr(e2l), E_local, R_cap, _ptr(counts),
                            _ptr(offsets), _ptr(row_src), _ptr(dest_row))
    if R < 0:
        raise ValueError({-1: "expert id out of range", -2: "routed rows exceed R_cap"}[int(R)])
    return dict(counts=counts, offsets=offsets, row_src=row_src[:R], dest_row=dest_row, R=int(R))


# ------------------------------------------------------------------ FFN / forward
def ffn_row(x, wg, wu, wd, prec):
    """One row through one expert: -> (a, b, h, y) float64."""
    x = _c(x, np.float32)
    wg = _c(wg, np.float32)
    wu = _c(wu, np.float32)
    wd = _c(wd, np.float32)
    I, d = wg.shape
    a = np.empty(I)
    b = np.empty(I)
    h = np.empty(I)
    y = np.empty(d)
    lib().mokref_ffn_row(d, I, PREC.get(prec, prec), _ptr(x), _ptr(wg), _ptr(wu), _ptr(wd),
                         _ptr(a), _ptr(b), _ptr(h), _ptr(y))
    return a, b, h, y


def fwd_tokens(tok_x, topk_idx, gate, e2l, wg, wu, wd, prec, peer_y=None):
    """Forward of a list of tokens -> (y [n, k, d], out [n, d]) float64.
    peer_y [n, k, d]: rows pushed by the GPUs holding the remote experts
    (read at remote slots only; None = zeros)."""
    tok_x = _c(tok_x, np.float32)
    topk_idx = _c(topk_idx, np.int32)
    gate = _c(gate, np.float64)
    e2l = _c(e2l, np.int32)
    wg = _c(wg, np.float32)
    wu = _c(wu, np.float32)
    wd = _c(wd, np.float32)
    n, d = tok_x.shape
    k = topk_idx.shape[1]
    I = wg.shape[1]
    y = np.empty((n, k, d))
    out = np.empty((n, d))
    if peer_y is not None:
        peer_y = _c(np.asarray(peer_y).reshape(n, k, d), np.float64)
    lib().mokref_fwd_tokens(n, d, e2l.shape[0], k, I, PREC.get(prec, prec), _ptr(tok_x),
                            _ptr(topk_idx), _ptr(gate), _ptr(e2l), _ptr(wg), _ptr(wu), _ptr(wd),
                            _ptr(peer_y), _ptr(y), _ptr(out))
    return y, out


# ------------------------------------------------------------------ backward
def bwd_row(x, g, dout, wg, wu, wd):
    """-> dict(dx, dg, dy, h, da, db) float64 for one routed row."""
    x = _c(x, np.float32)
    dout = _c(dout, np.float32)
    wg = _c(wg, np.float32)
    wu = _c(wu, np.float32)
    wd = _c(wd, np.float32)
    I, d = wg.shape
    dx = np.empty(d)
    dg = np.empty(1)
    dy = np.empty(d)
    h = np.empty(I)
    da = np.empty(I)
    db = np.empty(I)
    lib().mokref_bwd_row(d, I, _ptr(x), float(g), _ptr(dout), _ptr(wg), _ptr(wu), _ptr(wd),
                         _ptr(dx), _ptr(dg), _ptr(dy), _ptr(h), _ptr(da), _ptr(db))
    return dict(dx=dx, dg=float(dg[0]), dy=dy, h=h, da=da, db=db)


def router_bwd_token(idx, g, dg, wr):
    idx = _c(idx, np.int32)
    g = _c(g, np.float64)
    dg = _c(dg, np.float64)
    wr = _c(wr, np.float32)
    k = idx.shape[0]
    d = wr.shape[1]
    dz = np.empty(k)
    dxr = np.empty(d)
    lib().mokref_router_bwd_token(d, k, _ptr(idx), _ptr(g), _ptr(dg), _ptr(wr), _ptr(dz),
                                  _ptr(dxr))
    return dz, dxr


def bwd_tokens(tok_x, tok_dout, topk_idx, gate, e2l, wr, wg, wu, wd, peer_dg=None, peer_dx=None):
    """Backward of a list of tokens -> (d_gate [n,k], dz [n,k], dx [n,d]).
    peer_dg [n, k], peer_dx [n, k, d]: gate gradients and input-gradient rows
    written back by the GPUs holding the remote experts (read at remote slots
    only; None = zeros)."""
    tok_x = _c(tok_x, np.float32)
    tok_dout = _c(tok_dout, np.float32)
    topk_idx = _c(topk_idx, np.int32)
    gate = _c(gate, np.float64)
    e2l = _c(e2l, np.int32)
    wr = _c(wr, np.float32)
    wg = _c(wg, np.float32)
    wu = _c(wu, np.float32)
    wd = _c(wd, np.float32)
    n, d = tok_x.shape
    k = topk_idx.shape[1]
    I = wg.shape[1]
    d_gate = np.empty((n, k))
    dz = np.empty((n, k))
    dx = np.empty((n, d))
    if peer_dg is not None:
        peer_dg = _c(np.asarray(peer_dg).reshape(n, k), np.float64)
    if peer_dx is not None:
        peer_dx = _c(np.asarray(peer_dx).reshape(n, k, d), np.float64)
    lib().mokref_bwd_tokens(n, d, e2l.shape[0], k, I, _ptr(tok_x), _ptr(tok_dout), _ptr(topk_idx),
                            _ptr(gate), _ptr(e2l), _ptr(wr), _ptr(wg), _ptr(wu), _ptr(wd),
                            _ptr(peer_dg), _ptr(peer_dx), _ptr(d_gate), _ptr(dz), _ptr(dx))
    return d_gate, dz, dx


def expert_wgrad(rows_x, rows_g, rows_dout, wg, wu, wd):
    """-> (dW_gate [I,d], dW_up [I,d], dW_down [d,I]) float64 for one expert."""
    rows_x = _c(rows_x, np.float32)
    rows_g = _c(rows_g, np.float64)
    rows_dout = _c(rows_dout, np.float32)
    wg = _c(wg, np.float32)
    wu = _c(wu, np.float32)
    wd = _c(wd, np.float32)
    n, d = rows_x.shape
    I = wg.shape[0]
    dwg = np.empty((I, d))
    dwu = np.empty((I, d))
    dwd = np.empty((d, I))
    lib().mokref_expert_wgrad(n, d, I, _ptr(rows_x), _ptr(rows_g), _ptr(rows_dout), _ptr(wg),
                              _ptr(wu), _ptr(wd), _ptr(dwg), _ptr(dwu), _ptr(dwd))
    return dwg, dwu, dwd


def router_wgrad(tok_x, topk_idx, dz, E):
    tok_x = _c(tok_x, np.float32)
    topk_idx = _c(topk_idx, np.int32)
    dz = _c(dz, np.float64)
    n, d = tok_x.shape
    k = topk_idx.shape[1]
    dwr = np.empty((E, d))
    lib().mokref_router_wgrad(n, d, E, k, _ptr(tok_x), _ptr(topk_idx), _ptr(dz), _ptr(dwr))
    return dwr


def expert_wgrad_cols(rows_x, rows_g, rows_dout, wg, wu, wd, sel):
    """Columns sel of one expert's weight gradients -> (dW_gate[sel] [n_sel, d],
    dW_up[sel] [n_sel, d], dW_down[:, sel] [d, n_sel]) float64."""
    rows_x = _c(rows_x, np.float32)
    rows_g = _c(rows_g, np.float64)
    rows_dout = _c(rows_dout, np.float32)
    wg = _c(wg, np.float32)
    wu = _c(wu, np.float32)
    wd = _c(wd, np.float32)
    sel = _c(sel, np.int32)
    n, d = rows_x.shape
    I = wg.shape[0]
    q = sel.shape[0]
    dwg = np.empty((q, d))
    dwu = np.empty((q, d))
    dwd = np.empty((d, q))
    lib().mokref_expert_wgrad_cols(n, d, I, _ptr(rows_x), _ptr(rows_g), _ptr(rows_dout), _ptr(wg),
                                   _ptr(wu), _ptr(wd), q, _ptr(sel), _ptr(dwg), _ptr(dwu),
                                   _ptr(dwd))
    return dwg, dwu, dwd


def ffn_rows_exact(rows_x, wg, wu, wd):
    """Exact expert FFN of many rows of one expert, float64 (no roundings):
    a = x W_gate^T, b = x W_up^T, h = silu(a) * b, y = h W_down^T, with
    silu(a) = a / (1 + exp(-a)).  The three contractions are numpy matrix
    products; nothing else is blocked or reordered.  -> y [n, d]."""
    x = np.asarray(rows_x, np.float64)
    a = x @ np.asarray(wg, np.float64).T
    b = x @ np.asarray(wu, np.float64).T
    h = a / (1.0 + np.exp(-a)) * b
    return h @ np.asarray(wd, np.float64).T


def router_dz(topk_idx, gate, d_gate):
    """dz [n, k] of many tokens from their gates and gate gradients (the
    router backward of each token, without the input-gradient part)."""
    topk_idx = _c(topk_idx, np.int32)
    gate = _c(gate, np.float64)
    d_gate = _c(d_gate, np.float64)
    n, k = topk_idx.shape
    dz = np.empty((n, k))
    L = lib()
    rowb = k * 8
    for t in range(n):
        L.mokref_router_bwd_token(0, k, topk_idx.ctypes.data + t * k * 4,
                                  gate.ctypes.data + t * rowb, d_gate.ctypes.data + t * rowb,
                                  None, dz.ctypes.data + t * rowb, None)
    return dz


def gate_grads(dout_rows, y_rows):
    """Gate gradients of routed rows from the expert outputs the forward
    produced: the final weighted combine sums g_j y_j into the token's output
    (kucoin article, section 03: the final weighted combine), so
    dL/dg_j = dout . y_j, a float64 dot product per row.  -> [n]."""
    d = np.asarray(dout_rows, np.float64)
    y = np.asarray(y_rows, np.float64)
    return (d * y).sum(axis=1)


def expert_bwd_mx(rows_x, rows_g, rows_dout, rows_a, rows_b, rows_h, wg, wu, wd, quant=True):
    """MXFP8 backward of one expert's rows -> (dx [n,d], dW_gate [I,d], dW_up [I,d],
    dW_down [d,I]) float64; quant=False: the exact backward."""
    rows_x = _c(rows_x, np.float32)
    rows_g = _c(rows_g, np.float64)
    rows_dout = _c(rows_dout, np.float32)
    rows_a = _c(rows_a, np.float64)
    rows_b = _c(rows_b, np.float64)
    rows_h = _c(rows_h, np.float64)
    wg = _c(wg, np.float32)
    wu = _c(wu, np.float32)
    wd = _c(wd, np.float32)
    n, d = rows_x.shape
    I = wg.shape[0]
    dx = np.empty((n, d))
    dwg = np.empty((I, d))
    dwu = np.empty((I, d))
    dwd = np.empty((d, I))
    lib().mokref_expert_bwd_mx(n, d, I, 1 if quant else 0, _ptr(rows_x), _ptr(rows_g),
                               _ptr(rows_dout), _ptr(rows_a), _ptr(rows_b), _ptr(rows_h),
                               _ptr(wg), _ptr(wu), _ptr(wd), _ptr(dx), _ptr(dwg), _ptr(dwu),
                               _ptr(dwd))
    return dx, dwg, dwu, dwd
