"""The MXFP8 backward (mok_layer_bwd with prec MOK_MXFP8) against the oracle.

The oracle's reading (oracle.expert_bwd_mx): every backward GEMM quantises
both operands to E4M3 with one E8M0 scale per 32 along its contraction axis,
from the stored bf16 values; the weight gradients' operands along the
expert's rows.  Its forward intermediates (a, b, h as GEMM2 read it, y) come
from the oracle's MXFP8 forward row.  Tolerance: max|err| / max|ref| <= 2e-2.

The two sides agree on every quantisation given the same bf16 values (the
codes of dy, [da|db] and of the transposed operands are the oracle
quantiser's codes of the kernel's own values), but not on every bf16 value:
the scaled matrix cores' sums differ from exact ones by about 2^-19 of the
sum of their terms' magnitudes, and the kernel computes in fp32 what the
oracle computes in float64, so about 1% of a, b, dh and [da|db] elements
round to the neighbouring bf16 value.  The MX scale rule amplifies a rare
few of those: a block whose largest magnitude sits just below a power of two
2^k saturates that element to 1.75 2^k, one just at or above it keeps 2^k,
so a one-ulp difference there moves one element by 2^k / 4.  In a weight
gradient that is one term of the n routed rows' sum, in an input-gradient
row one of 2I terms: relative to the largest result it shrinks as
1/sqrt(n) and 1/sqrt(2I).  Measured: 3e-2 with I = 128 and 150 rows per
expert, 2.1e-2 with I = 512 and 1000 rows.  The cases therefore use the
layer's own I (1408) and about 3000 rows per expert (the mid-size layer
routes about 1500 rows to each of its 64 experts; its own check samples
32-column slices of two experts).
"""
import numpy as np
import pytest
import torch

import oracle
from cases import make_host_case, oracle_weights, peer_rows, rel_err, sample_tokens
from combine_router_top_expert_amd import synth
from combine_router_top_expert_amd.layer import to_device
from test_gpu_parity import DEV, _layer, _log, _small

pytestmark = pytest.mark.gpu

TOL = 2e-2

BWD_MX_CASES = {
    # the layer's I (1408), about 3200 rows per expert (ragged 128-row stages
    # and 32-row blocks), every expert local
    "mx_all_local": _small("C4", S=2, T_src=1600, d=128, E=2, k=2, I=1408, own=[0, 1],
                           local_experts=[0, 1]),
    # remote experts: their slots' d_gate and dx rows are the peers'; about
    # 3000 rows per local expert from all three sources
    "mx_share": _small("C4", S=3, T_src=4000, d=128, E=8, k=2, I=1408, own=[1],
                       local_experts=[1, 4]),
}


def _rows_of(c, dout_store, rows):
    """Token rows, gates and upstream gradients of items `rows`."""
    w = c.w
    tt, jj = rows // w.k, rows % w.k
    rx = np.stack([c.x_val[t // w.T_src][t % w.T_src] for t in tt])
    rg = np.array([c.gate_all[t // w.T_src, t % w.T_src, j] for t, j in zip(tt, jj)])
    rd = np.stack([dout_store[t // w.T_src][1][t % w.T_src] for t in tt])
    return rx, rg, rd


def _fwd_rows(rx, wgq, wuq, wdq):
    """The oracle's MXFP8 forward of the rows -> a, b, h, y [n, .]."""
    out = [oracle.ffn_row(rx[r], wgq, wuq, wdq, "mxfp8") for r in range(rx.shape[0])]
    return [np.stack([o[i] for o in out]) for i in range(4)]


def _expert_ref(c, dout_store, le, sel=None):
    """Oracle MX backward of local expert le's rows: (items, dx rows, dg,
    dW_gate, dW_up, dW_down); sel (a 32-aligned block of I columns) restricts
    the weight gradients to those columns (dx and dg then not computed)."""
    lay = c.layout
    rows = lay["row_src"][lay["offsets"][le]:lay["offsets"][le + 1]]
    rx, rg, rd = _rows_of(c, dout_store, rows)
    wgq, wuq, wdq = oracle_weights(c, le)
    if sel is None:
        a, b, h, y = _fwd_rows(rx, wgq, wuq, wdq)
        dx, dwg, dwu, dwd = oracle.expert_bwd_mx(rx, rg, rd, a, b, h, c.wg_val[le], c.wu_val[le],
                                                 c.wd_val[le])
        return rows, dx, oracle.gate_grads(rd, y), dwg, dwu, dwd
    a, b, h, _ = _fwd_rows(rx, wgq[sel], wuq[sel], wdq[:, sel])
    _, dwg, dwu, dwd = oracle.expert_bwd_mx(rx, rg, rd, a, b, h, c.wg_val[le][sel],
                                            c.wu_val[le][sel], c.wd_val[le][:, sel])
    return rows, None, None, dwg, dwu, dwd


def _run(c):
    w = c.w
    L = _layer(c)
    dout_store = [synth.gen_dout(w, s) for s in range(w.S)]
    d_out = [to_device(a, w.prec, DEV) for a, _ in dout_store]
    for t in (L.dw_gate, L.dw_up, L.dw_down, L.dw_router):
        t.fill_(float("nan"))  # every element must be overwritten
    L.forward()
    L.backward(d_out)
    torch.cuda.synchronize()
    L.check_status()
    return L, dout_store, d_out


def _token_refs(c, toks, dout_store, slot_dg, slot_dx):
    """Reference d_gate / dz / d_x of own tokens from the rows' gate gradients
    and input-gradient rows (slot_dg[(s, t, j)], slot_dx[...] for local
    slots; the peers' values at remote slots): the oracle's token backward
    with every slot's values given."""
    w = c.w
    tok_x = np.stack([c.x_val[s][t] for s, t in toks])
    idx = np.stack([c.topk_all[s, t] for s, t in toks])
    g = np.stack([c.gate_all[s, t] for s, t in toks])
    pdg = peer_rows(c, toks, 2)
    pdx = peer_rows(c, toks, 4)
    dg = np.zeros((len(toks), w.k)) if pdg is None else np.array(pdg, np.float64)
    dx = np.zeros((len(toks), w.k, w.d)) if pdx is None else np.array(pdx, np.float64)
    for i, (s, t) in enumerate(toks):
        for j in range(w.k):
            if c.e2l[idx[i, j]] >= 0:
                dg[i, j] = slot_dg[(s, t, j)]
                dx[i, j] = slot_dx[(s, t, j)]
    none = np.full_like(c.e2l, -1)
    tok_d = np.stack([dout_store[s][1][t] for s, t in toks])
    d_gate, dz, d_x = oracle.bwd_tokens(tok_x, tok_d, idx, g, none, c.wr_val, c.wg_val, c.wu_val,
                                        c.wd_val, peer_dg=dg, peer_dx=dx)
    return tok_x, idx, d_gate, dz, d_x


@pytest.mark.parametrize("name", list(BWD_MX_CASES))
def test_layer_bwd_mx(name):
    w = BWD_MX_CASES[name]
    _log("layer_bwd_mx", name)
    c = make_host_case(w)
    L, dout_store, d_out = _run(c)
    lay = c.layout
    slot_dg, slot_dx = {}, {}
    e_w = e_row = 0.0
    dx_stage = [t.float().cpu().numpy() for t in L.dx_stage]
    for le in range(w.E_local):
        rows, dx, dg, dwg, dwu, dwd = _expert_ref(c, dout_store, le)
        if len(rows) == 0:
            assert float(L.dw_gate[le].abs().max()) == 0.0
            assert float(L.dw_down[le].abs().max()) == 0.0
            continue
        e_w = max(e_w, rel_err(L.dw_gate[le].cpu().numpy(), dwg),
                  rel_err(L.dw_up[le].cpu().numpy(), dwu),
                  rel_err(L.dw_down[le].cpu().numpy(), dwd))
        got = np.stack([dx_stage[n // w.k // w.T_src][(n // w.k) % w.T_src * w.k + n % w.k]
                        for n in rows])
        e_row = max(e_row, rel_err(got, dx))
        for r, n in enumerate(rows):
            tok = n // w.k
            slot_dg[(tok // w.T_src, tok % w.T_src, n % w.k)] = dg[r]
            slot_dx[(tok // w.T_src, tok % w.T_src, n % w.k)] = dx[r]
    toks = [(s, t) for s in w.own for t in range(w.T_src)]
    tok_x, idx, dg_ref, dz_ref, dx_ref = _token_refs(c, toks, dout_store, slot_dg, slot_dx)
    dg_all = L.d_gate.cpu().numpy().reshape(w.S, w.T_src, w.k)
    dg_got = np.stack([dg_all[s, t] for s, t in toks])
    local = c.e2l[idx] >= 0
    e_dg = rel_err(dg_got[local], dg_ref[local])
    np.testing.assert_array_equal(dg_got[~local], dg_ref[~local].astype(np.float32))
    dx_got = np.stack([L.d_x[s][t].float().cpu().numpy() for s, t in toks])
    e_dx = rel_err(dx_got, dx_ref)
    e_r = rel_err(L.dw_router.cpu().numpy(), oracle.router_wgrad(tok_x, idx, dz_ref, w.E))
    _log(f"  dx rows {e_row:.3e} dW {e_w:.3e} dg {e_dg:.3e} dx {e_dx:.3e} dWr {e_r:.3e}")
    assert max(e_row, e_w, e_dg, e_dx, e_r) <= TOL
    # run to run: a second backward gives the same bytes
    first = [t.clone() for t in (L.dw_gate, L.dw_up, L.dw_down, L.dw_router)]
    first_dx = [t.clone() for t in L.d_x if t is not None]
    L.backward(d_out)
    torch.cuda.synchronize()
    L.check_status()
    for a, b in zip(first, (L.dw_gate, L.dw_up, L.dw_down, L.dw_router)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    for a, b in zip(first_dx, [t for t in L.d_x if t is not None]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_layer_bwd_mx_empty_batch():
    """No tokens: the MXFP8 backward runs, latches no error and writes zero
    weight gradients (every expert's tiles contract over no rows)."""
    w = _small("C4", S=2, T_src=0, d=128, E=4, k=2, I=256, own=[0, 1],
               local_experts=list(range(4)))
    _log("layer_bwd_mx empty")
    c = make_host_case(w)
    L, _, _ = _run(c)
    assert int(L.offsets[-1].item()) == 0
    for t in (L.dw_gate, L.dw_up, L.dw_down, L.dw_router):
        assert float(t.abs().max()) == 0.0


def test_layer_bwd_mx_c4_full_sampled():
    """The mid-size MXFP8 layer (16384 tokens, 64 experts, top-6, d 2048,
    I 1408): sampled tokens' dx rows, gate gradients and input gradients, and
    two experts' weight gradients on a 32-column slice of I."""
    w = synth.WORKLOADS["C4"]
    _log("layer_bwd_mx c4_full")
    c = make_host_case(w)
    L, dout_store, _ = _run(c)
    toks = sample_tokens(w, 4)
    wq = {}
    slot_dg, slot_dx = {}, {}
    e_row = 0.0
    for s, t in toks:
        for j in range(w.k):
            n = np.array([(s * w.T_src + t) * w.k + j])
            le = int(c.e2l[c.topk_all[s, t, j]])
            if le not in wq:
                wq[le] = oracle_weights(c, le)
            rx, rg, rd = _rows_of(c, dout_store, n)
            a, b, h, y = _fwd_rows(rx, *wq[le])
            dx, _, _, _ = oracle.expert_bwd_mx(rx, rg, rd, a, b, h, c.wg_val[le], c.wu_val[le],
                                               c.wd_val[le])
            slot_dg[(s, t, j)] = oracle.gate_grads(rd, y)[0]
            slot_dx[(s, t, j)] = dx[0]
            got = L.dx_stage[s][t * w.k + j].float().cpu().numpy()
            e_row = max(e_row, rel_err(got, dx[0]))
    _, idx, dg_ref, _, dx_ref = _token_refs(c, toks, dout_store, slot_dg, slot_dx)
    dg_all = L.d_gate.cpu().numpy().reshape(w.S, w.T_src, w.k)
    e_dg = rel_err(np.stack([dg_all[s, t] for s, t in toks]), dg_ref)
    e_dx = rel_err(np.stack([L.d_x[s][t].float().cpu().numpy() for s, t in toks]), dx_ref)
    e_w = 0.0
    for le, blk in ((0, 0), (w.E_local - 1, w.I // 32 - 1)):
        sel = np.arange(32 * blk, 32 * blk + 32)
        rows, _, _, dwg, dwu, dwd = _expert_ref(c, dout_store, le, sel)
        assert len(rows) > 0
        e_w = max(e_w, rel_err(L.dw_gate[le][sel].cpu().numpy(), dwg),
                  rel_err(L.dw_up[le][sel].cpu().numpy(), dwu),
                  rel_err(L.dw_down[le][:, sel].cpu().numpy(), dwd))
    _log(f"  dx rows {e_row:.3e} dg {e_dg:.3e} dx {e_dx:.3e} dW slices {e_w:.3e}")
    assert max(e_row, e_dg, e_dx, e_w) <= TOL
    # the weight gradients are finite and overwritten everywhere
    for t in (L.dw_gate, L.dw_up, L.dw_down, L.dw_router):
        assert bool(torch.isfinite(t).all())
