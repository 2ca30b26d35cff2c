"""Parity of the HIP path (called through the C ABI) with the CPU oracle.

Bit-exact: routing indices, counts, offsets, row_src, dest_row, gathered
rows, MX codes.  Floating point: max|err| / max|ref| <= 1e-2 (fp32, bf16) and
2e-2 (MXFP8 against the MX-emulating oracle); gates within 2e-6."""
import numpy as np
import pytest
import torch

import oracle
from cases import (make_host_case, oracle_fwd_tokens, oracle_weights, peer_rows, rel_err,
                   sample_tokens)
from combine_router_top_expert_amd import (STATUS, make_config, make_weights, mok_combine,
                                           mok_dispatch, mok_expert_ffn, mok_layout,
                                           mok_mx_quantize, mok_mx_quantize_f32, mok_route,
                                           mok_workspace_bytes, synth)
from combine_router_top_expert_amd.layer import MoELayer, to_device

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {"f32": 1e-2, "bf16": 1e-2, "mxfp8": 2e-2}


def _log(*a):
    print(*a, flush=True)


def _layer(c, R_cap=None, with_bwd=True, **kw):
    w = c.w
    L = MoELayer(w.S, w.T_src, w.d, w.E, w.k, w.I, w.E_local, w.prec, R_cap or c.R_cap(),
                 own_lo=w.own[0], own_n=len(w.own), device=DEV, with_bwd=with_bwd, **kw)
    xs = [to_device(a, w.prec, DEV) for a in c.x_store]
    bias = None if c.bias is None else torch.from_numpy(c.bias).to(DEV)
    L.set_inputs(xs, to_device(c.wr_store, w.prec, DEV), bias, torch.from_numpy(c.e2l).to(DEV),
                 to_device(c.wg_store, w.prec, DEV), to_device(c.wu_store, w.prec, DEV),
                 to_device(c.wd_store, w.prec, DEV), other_topk=c.other)
    for s, (ys, _, dg, dxs, _) in c.peer.items():
        L.set_peer_slots(s, to_device(ys, w.prec, DEV), torch.from_numpy(dg).to(DEV),
                         to_device(dxs, w.prec, DEV))
    return L


def _small(name, **kw):
    return synth.WORKLOADS[name].replace(**kw)


ROUTE_CASES = {
    "c1": synth.WORKLOADS["C1"],
    "e1k1": _small("C2", S=1, T_src=70, d=128, E=1, k=1, I=64, own=[0], local_experts=[0]),
    "e3k2": _small("C2", S=1, T_src=129, d=64, E=3, k=2, I=64, own=[0], local_experts=[0, 1, 2]),
    "c2shape": _small("C2", S=1, T_src=1000, own=[0]),
    "c3shape": _small("C3", S=1, T_src=100, own=[0], local_experts=[0]),
    "e512k16": _small("C2", S=1, T_src=33, d=256, E=512, k=16, I=64, own=[0], local_experts=[0]),
    # two experts per lane, a ragged token count across two sources
    "e128": _small("C2", S=2, T_src=777, d=256, E=128, k=4, I=64, own=[0, 1], local_experts=[0]),
}


@pytest.mark.parametrize("name", list(ROUTE_CASES))
def test_route_bit_exact(name):
    w = ROUTE_CASES[name]
    _log("route", name, w.T_src, w.d, w.E, w.k)
    xs, xv = synth.gen_x(w, 0)
    wr, wrv = synth.gen_router(w)
    bias = synth.load_bias(w) if w.zipf_s else None
    if name == "c3shape":
        bias = synth.load_bias(synth.WORKLOADS["C3"])
    ref_idx, ref_g = oracle.route(xv, wrv, bias, w.k, w.prec)
    cfg = make_config(1, w.T_src, w.d, w.E, w.k, w.I, 1, w.prec, 1)
    x = to_device(xs, w.prec, DEV)
    wrd = to_device(wr, w.prec, DEV)
    b = None if bias is None else torch.from_numpy(bias).to(DEV)
    idx = torch.full((w.T_src, w.k), -1, dtype=torch.int32, device=DEV)
    g = torch.zeros((w.T_src, w.k), dtype=torch.float32, device=DEV)
    mok_route(cfg, w.T_src, x, wrd, b, idx, g)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_allclose(g.cpu().numpy(), ref_g, atol=2e-6, rtol=0)


def _special_route_inputs(kind):
    """Router inputs that exercise the selection rule: exact ties (small
    integer values, duplicated router rows, equal biases), k = E, and NaN /
    infinite logits.  -> (T, d, E, k, x values, router values, bias)."""
    rng = np.random.default_rng({"ties": 11, "k_eq_E": 12, "nan": 13}[kind])
    if kind == "k_eq_E":
        T, d, E, k = 300, 256, 16, 16
        x = rng.normal(size=(T, d))
        wr = rng.normal(size=(E, d)) / 16
        bias = None
    else:
        T, d, E, k = 333, 128, 24, 4
        # sums of small multiples of 1/4 are exact in fp32: many equal logits
        x = rng.integers(-2, 3, size=(T, d)).astype(np.float64)
        wr = rng.integers(-1, 2, size=(E, d)) * 0.25
        wr[5] = wr[2]
        wr[9] = wr[2]
        wr[E - 1] = wr[0]
        bias = np.zeros(E, np.float32)
        bias[[3, 4, 11]] = 0.5
        bias[[7, 8]] = -0.25
    if kind == "nan":
        x[0, :] = np.nan           # every logit of token 0 is NaN
        x[1, 17] = np.nan
        x[2, 3] = np.inf           # +-inf logits, NaN where a weight is 0
        x[3, :] = np.inf
        wr[6, 40] = np.nan         # expert 6 has a NaN logit for every token
    xs = synth.f64_to_bf16_bits(x)
    ws = synth.f64_to_bf16_bits(wr)
    return T, d, E, k, xs, ws, bias


@pytest.mark.parametrize("kind", ["ties", "k_eq_E", "nan"])
def test_route_selection_rule_bit_exact(kind):
    """Equal logits go to the lower expert id; k = E selects every expert in
    logit order; a NaN logit ranks after every number (-inf included), so a
    token with NaN logits still gets k distinct valid experts."""
    T, d, E, k, xs, ws, bias = _special_route_inputs(kind)
    _log("route rule", kind, T, d, E, k)
    xv = synth.bf16_bits_to_f32(xs)
    wv = synth.bf16_bits_to_f32(ws)
    ref_idx, ref_g = oracle.route(xv, wv, bias, k, "bf16")
    if kind == "ties":   # the inputs really produce ties that decide a slot
        z = oracle.logits(xv, wv, bias, "bf16")
        kth = np.sort(z, axis=1)[:, ::-1][:, k - 1:k + 1]
        assert np.sum(kth[:, 0] == kth[:, 1]) > 20
    cfg = make_config(1, T, d, E, k, 64, 1, "bf16", 1)
    x = to_device(xs, "bf16", DEV)
    wrd = to_device(ws, "bf16", DEV)
    b = None if bias is None else torch.from_numpy(bias).to(DEV)
    idx = torch.full((T, k), -1, dtype=torch.int32, device=DEV)
    g = torch.zeros((T, k), dtype=torch.float32, device=DEV)
    mok_route(cfg, T, x, wrd, b, idx, g)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    np.testing.assert_array_equal(gi, ref_idx)
    assert gi.min() >= 0 and gi.max() < E
    assert all(len(set(r)) == k for r in gi.tolist())
    np.testing.assert_allclose(g.cpu().numpy(), ref_g, atol=2e-6, rtol=0)  # NaN == NaN here


def test_layer_with_nan_token_keeps_valid_experts():
    """A token row holding NaN routes to valid experts (the k lowest ids), so
    the forward and the backward -- whose router term reads the router row
    of each chosen expert -- stay in bounds and latch nothing; the other
    tokens' outputs and input gradients are finite."""
    w = _small("C2", S=2, T_src=100, d=128, E=8, k=2, I=128, own=[0, 1],
               local_experts=list(range(8)))
    _log("nan token")
    c = make_host_case(w, route_own=False)
    v = synth.bf16_bits_to_f32(c.x_store[0]).astype(np.float64)
    v[7, :] = np.nan
    c.x_store[0] = synth.f64_to_bf16_bits(v)
    c.x_val[0] = synth.bf16_bits_to_f32(c.x_store[0])
    from cases import oracle_routing
    oracle_routing(c)
    L = _layer(c)
    d_out = [to_device(synth.gen_dout(w, s)[0], w.prec, DEV) for s in range(w.S)]
    L.forward()
    L.backward(d_out)
    torch.cuda.synchronize()
    L.check_status()
    gi = L.topk_idx.cpu().numpy().reshape(w.S, w.T_src, w.k)
    np.testing.assert_array_equal(gi, c.topk_all)
    np.testing.assert_array_equal(gi[0, 7], np.arange(w.k))
    out0 = L.out[0].float().cpu().numpy()
    dx0 = L.d_x[0].float().cpu().numpy()
    assert np.all(np.isnan(out0[7]))
    keep = np.arange(w.T_src) != 7
    assert np.all(np.isfinite(out0[keep])) and np.all(np.isfinite(dx0[keep]))


LAYOUT_CASES = {
    "c2": (synth.WORKLOADS["C2"], None),
    "c3": (synth.WORKLOADS["C3"], None),
    "tiny": (_small("C2", S=1, T_src=1, d=64, E=4, k=2, I=64, own=[0], local_experts=[2, 0]), None),
    "ragged": (_small("C2", S=3, T_src=999, d=64, E=40, k=5, I=64, own=[0],
                      local_experts=list(range(0, 40, 3))), None),
    "e256": (_small("C2", S=2, T_src=3000, d=64, E=256, k=8, I=64, own=[0],
                    local_experts=list(range(256))), None),
}


@pytest.mark.parametrize("name", list(LAYOUT_CASES))
def test_layout_bit_exact(name):
    w, _ = LAYOUT_CASES[name]
    _log("layout", name, w.S, w.T_src, w.k, w.E, w.E_local)
    topk = np.stack([synth.gen_other_routing(w.replace(own=[]), s)[0] for s in range(w.S)])
    e2l = w.expert_to_local()
    ref = oracle.layout(topk, e2l, w.E_local)
    R_cap = max(ref["R"], 1)
    cfg = make_config(w.S, w.T_src, w.d, w.E, w.k, w.I, w.E_local, w.prec, R_cap)
    ws = torch.zeros(mok_workspace_bytes(cfg), dtype=torch.uint8, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    counts = torch.zeros(w.E_local, dtype=torch.int32, device=DEV)
    offsets = torch.zeros(w.E_local + 1, dtype=torch.int32, device=DEV)
    row_src = torch.full((R_cap,), -7, dtype=torch.int32, device=DEV)
    dest_row = torch.full((topk.size,), -7, dtype=torch.int32, device=DEV)
    mok_layout(cfg, torch.from_numpy(topk.reshape(-1)).to(DEV), torch.from_numpy(e2l).to(DEV),
               counts, offsets, row_src, dest_row, ws, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    np.testing.assert_array_equal(counts.cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(offsets.cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(row_src.cpu().numpy()[:ref["R"]], ref["row_src"])
    np.testing.assert_array_equal(dest_row.cpu().numpy(), ref["dest_row"])


def test_layout_errors_latched():
    w = _small("C2", S=1, T_src=50, d=64, E=4, k=2, I=64, own=[0], local_experts=[0, 1, 2, 3])
    topk = synth.gen_other_routing(w.replace(own=[]), 0)[0]
    e2l = w.expert_to_local()
    for R_cap, bad, expect in ((99, False, "MOK_ECAPACITY"), (100, True, "MOK_EROUTE")):
        _log("layout error", expect)
        t = topk.copy()
        if bad:
            t[7, 1] = 9
        cfg = make_config(1, w.T_src, w.d, w.E, w.k, w.I, w.E_local, w.prec, R_cap)
        ws = torch.zeros(mok_workspace_bytes(cfg), dtype=torch.uint8, device=DEV)
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        counts = torch.zeros(4, dtype=torch.int32, device=DEV)
        offsets = torch.zeros(5, dtype=torch.int32, device=DEV)
        row_src = torch.zeros(R_cap, dtype=torch.int32, device=DEV)
        dest_row = torch.zeros(t.size, dtype=torch.int32, device=DEV)
        mok_layout(cfg, torch.from_numpy(t.reshape(-1)).to(DEV), torch.from_numpy(e2l).to(DEV),
                   counts, offsets, row_src, dest_row, ws, st)
        torch.cuda.synchronize()
        assert STATUS[int(st.item())] == expect
        rs = row_src.cpu().numpy()
        assert rs.min() >= 0 and rs.max() < t.size   # nothing written out of range
        if not bad:
            # the rows below R_cap as without a capacity; a dropped item keeps its
            # row number (>= R_cap) so that later steps skip it
            ref = oracle.layout(t.reshape(1, w.T_src, w.k), e2l, w.E_local)
            np.testing.assert_array_equal(rs, ref["row_src"][:R_cap])
            np.testing.assert_array_equal(dest_row.cpu().numpy(), ref["dest_row"])


def test_dispatch_tagged_rows_and_identity_combine():
    """Rows tagged with their (source, token) come back exactly where row_src
    says; combining the gathered rows with identity experts gives sum_j g_j x."""
    w = _small("C2", S=3, T_src=301, d=256, E=16, k=4, I=64, own=[1],
               local_experts=[1, 4, 7, 10, 13, 2])
    _log("dispatch", w.S, w.T_src)
    rng = np.random.default_rng(5)
    xs_val = []
    for s in range(w.S):
        v = rng.normal(size=(w.T_src, w.d))
        v[:, 0] = s
        v[:, 1] = np.arange(w.T_src) // 128
        v[:, 2] = np.arange(w.T_src) % 128
        xs_val.append(synth.f64_to_bf16_bits(v))
    topk = np.stack([synth.gen_other_routing(w.replace(own=[]), s)[0] for s in range(w.S)])
    gate = np.stack([synth.gen_other_routing(w.replace(own=[]), s)[1] for s in range(w.S)])
    e2l = w.expert_to_local()
    ref = oracle.layout(topk, e2l, w.E_local)
    R = ref["R"]
    cfg = make_config(w.S, w.T_src, w.d, w.E, w.k, w.I, w.E_local, "bf16", R)
    offsets = torch.from_numpy(ref["offsets"]).to(DEV)
    row_src = torch.from_numpy(ref["row_src"]).to(DEV)
    x = [to_device(a, "bf16", DEV) for a in xs_val]
    xp = torch.zeros(R, w.d, dtype=torch.bfloat16, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    mok_dispatch(cfg, x, row_src, offsets, xp, None, st)
    torch.cuda.synchronize()
    got = xp.view(torch.int16).cpu().numpy().view(np.uint16)
    toks = ref["row_src"] // w.k
    want = np.stack([xs_val[t // w.T_src][t % w.T_src] for t in toks])
    np.testing.assert_array_equal(got, want)
    # identity experts here and at the peers: y = the token's row in every
    # slot (the peers' pushes written up front); push + final combine for the
    # own source sums all k slots
    staging = [torch.zeros(w.T_src * w.k, w.d, dtype=torch.bfloat16, device=DEV) for _ in range(w.S)]
    staging[1].copy_(x[1].repeat_interleave(w.k, dim=0))
    out = [torch.zeros(w.T_src, w.d, dtype=torch.bfloat16, device=DEV) for _ in range(w.S)]
    mok_combine(cfg, xp, torch.from_numpy(ref["dest_row"]).to(DEV),
                torch.from_numpy(gate.reshape(-1)).to(DEV), staging, 1, 1, out, st)
    torch.cuda.synchronize()
    o = out[1].float().cpu().numpy()
    xv = synth.bf16_bits_to_f32(xs_val[1]).astype(np.float64)
    gsum = gate[1].astype(np.float64).sum(1)
    expect = xv * gsum[:, None]
    assert np.all(np.abs(o - expect) <= 2.0 ** -8 * np.abs(expect) + 1e-30)


def _ffn_case(prec):
    w = _small("C2", S=2, T_src=150, d=256, E=6, k=2, I=320, own=[0, 1],
               local_experts=list(range(6)), prec=prec)
    if prec == "f32":
        w = w.replace(prec="f32")
    return w


@pytest.mark.parametrize("prec", ["f32", "bf16"])
def test_expert_ffn_rows(prec):
    w = _ffn_case(prec)
    _log("expert_ffn", prec)
    c = make_host_case(w)
    R = c.layout["R"]
    cfg = make_config(w.S, w.T_src, w.d, w.E, w.k, w.I, w.E_local, prec, R)
    # inputs: the gathered rows, built on the host from the oracle layout
    toks = c.layout["row_src"] // w.k
    xs_rows = np.stack([c.x_store[t // w.T_src][t % w.T_src] for t in toks])
    xp = to_device(xs_rows, prec, DEV)
    dt = torch.float32 if prec == "f32" else torch.bfloat16
    h = torch.zeros(R, w.I, dtype=dt, device=DEV)
    ab = torch.zeros(R, 2 * w.I, dtype=dt, device=DEV)
    y = torch.zeros(R, w.d, dtype=dt, device=DEV)
    wts = [to_device(a, prec, DEV) for a in (c.wg_store, c.wu_store, c.wd_store)]
    W = make_weights(*wts)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    mok_expert_ffn(cfg, xp, None, torch.from_numpy(c.layout["offsets"]).to(DEV), W, h, None, ab, y,
                   st)
    torch.cuda.synchronize()
    yg = y.float().cpu().numpy()
    hg = h.float().cpu().numpy()
    abg = ab.float().cpu().numpy()
    offs = c.layout["offsets"]
    for r in range(R):
        le = int(np.searchsorted(offs, r, side="right") - 1)
        t = toks[r]
        a, b, hr, yr = oracle.ffn_row(c.x_val[t // w.T_src][t % w.T_src], c.wg_val[le], c.wu_val[le],
                                      c.wd_val[le], prec)
        assert rel_err(yg[r], yr) <= TOL[prec], r
        assert rel_err(hg[r], hr) <= TOL[prec], r
        assert rel_err(abg[r, :w.I], a) <= TOL[prec] and rel_err(abg[r, w.I:], b) <= TOL[prec]


def _mx_h_close(hq, hs, ref_codes, ref_scales):
    """GPU h (E4M3 codes + E8M0 scales) against the oracle's MX h.  h is
    quantised from fp32 on the GPU and from fp64 in the oracle, so a value
    lying within rounding noise of a code boundary may land one code step
    away: require at most one step per element (two if its block scale
    moved) and such elements to be rare."""
    got = oracle.mx_dequantize(hq, hs)
    ref = oracle.mx_dequantize(ref_codes, ref_scales)
    # one E4M3 step at value v in a block of shared exponent X: <= |v| 2^-3
    # (normal codes) or 2^(X-9) (subnormal codes)
    sub = np.repeat(np.exp2(ref_scales.astype(np.float64) - 127 - 9), 32, axis=1)
    one_step = np.maximum(np.abs(ref), np.abs(got)) * 2.0 ** -3 + sub
    assert np.all(np.abs(got - ref) <= 2 * one_step)
    frac = float(np.mean(hq != ref_codes))
    _log(f"  h codes differing: {frac:.2e}")
    assert frac <= 2e-3


def test_expert_ffn_rows_mx():
    w = _small("C4", S=2, T_src=150, d=256, E=6, k=2, I=384, own=[0, 1],
               local_experts=list(range(6)))
    _log("expert_ffn mxfp8")
    c = make_host_case(w)
    R = c.layout["R"]
    cfg = make_config(w.S, w.T_src, w.d, w.E, w.k, w.I, w.E_local, "mxfp8", R)
    toks = c.layout["row_src"] // w.k
    xs_rows = np.stack([c.x_store[t // w.T_src][t % w.T_src] for t in toks])
    xq = torch.zeros(R * w.d, dtype=torch.uint8, device=DEV)
    xsc = torch.zeros(R * w.d // 32, dtype=torch.uint8, device=DEV)
    mok_mx_quantize(R, w.d, to_device(xs_rows, "bf16", DEV), xq, xsc)
    q = []
    for a in (c.wg_store, c.wu_store, c.wd_store):
        K = a.shape[-1]
        cq = torch.zeros(a.size, dtype=torch.uint8, device=DEV)
        cs = torch.zeros(a.size // 32, dtype=torch.uint8, device=DEV)
        mok_mx_quantize(a.size // K, K, to_device(a, "bf16", DEV), cq, cs)
        q.append((cq, cs))
    W = make_weights(q[0][0], q[1][0], q[2][0], q[0][1], q[1][1], q[2][1])
    hq = torch.zeros(R * w.I, dtype=torch.uint8, device=DEV)
    hs = torch.zeros(R * w.I // 32, dtype=torch.uint8, device=DEV)
    y = torch.zeros(R, w.d, dtype=torch.bfloat16, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    mok_expert_ffn(cfg, xq, xsc, torch.from_numpy(c.layout["offsets"]).to(DEV), W, hq, hs, None,
                   y, st)
    torch.cuda.synchronize()
    wg, wu, wd = oracle_weights(c)
    yg = y.float().cpu().numpy()
    offs = c.layout["offsets"]
    h_ref = np.zeros((R, w.I))
    y_ref = np.zeros((R, w.d))
    for r in range(R):
        le = int(np.searchsorted(offs, r, side="right") - 1)
        t = toks[r]
        _, _, h_ref[r], y_ref[r] = oracle.ffn_row(c.x_val[t // w.T_src][t % w.T_src], wg[le],
                                                  wu[le], wd[le], "mxfp8")
    e_y = rel_err(yg, y_ref)
    _log(f"  y rel err {e_y:.3e}")
    assert e_y <= TOL["mxfp8"]
    # h: the oracle's MX h is exactly representable, so re-quantising it
    # returns its codes and scales
    rc, rs = oracle.mx_quantize(h_ref)
    _mx_h_close(hq.cpu().numpy().reshape(R, w.I), hs.cpu().numpy().reshape(R, w.I // 32), rc, rs)


FWD_CASES = {
    "c1": synth.WORKLOADS["C1"],
    "bf16_small": _small("C2", S=2, T_src=300, d=256, E=8, k=2, I=320, own=[0, 1],
                         local_experts=list(range(8))),
    "bf16_share": _small("C3", S=3, T_src=65, d=128, E=16, k=4, I=192, own=[1],
                         local_experts=[1, 4, 7, 10, 13], zipf_s=0.0),
    "c2_full": synth.WORKLOADS["C2"],
    "mx_small": _small("C4", S=2, T_src=300, d=256, E=8, k=2, I=256, own=[0, 1],
                       local_experts=list(range(8))),
    "mx_share": _small("C4", S=3, T_src=65, d=128, E=16, k=4, I=384, own=[1],
                       local_experts=[1, 4, 7, 10, 13]),
    "c4_full": synth.WORKLOADS["C4"],
}


def _check_fwd(c, L, toks):
    w = c.w
    per = w.T_src * w.k
    gi = L.topk_idx.cpu().numpy().reshape(w.S, w.T_src, w.k)
    gg = L.topk_gate.cpu().numpy().reshape(w.S, w.T_src, w.k)
    for s in w.own:
        np.testing.assert_array_equal(gi[s], c.topk_all[s])
        np.testing.assert_allclose(gg[s], c.gate_all[s], atol=2e-6, rtol=0)
    lay = c.layout
    np.testing.assert_array_equal(L.counts.cpu().numpy(), lay["counts"])
    np.testing.assert_array_equal(L.offsets.cpu().numpy(), lay["offsets"])
    np.testing.assert_array_equal(L.row_src.cpu().numpy()[:lay["R"]], lay["row_src"])
    np.testing.assert_array_equal(L.dest_row.cpu().numpy()[:w.S * per], lay["dest_row"])
    y_ref, out_ref = oracle_fwd_tokens(c, toks)
    ys, outs, ysr = [], [], []
    for i, (s, t) in enumerate(toks):
        o = L.out[s][t].float().cpu().numpy()
        outs.append(o)
        for j in range(w.k):
            if c.e2l[c.topk_all[s, t, j]] >= 0:
                ys.append(L.staging[s][t * w.k + j].float().cpu().numpy())
                ysr.append(y_ref[i, j])
            else:  # a remote slot keeps what its pusher wrote
                got = L.staging[s][t * w.k + j].float().cpu().numpy()
                np.testing.assert_array_equal(got, c.peer[s][1][t * w.k + j])
    e_out = rel_err(np.stack(outs), out_ref)
    e_y = rel_err(np.stack(ys), np.stack(ysr)) if ys else 0.0
    _log(f"  out rel err {e_out:.3e}  y rel err {e_y:.3e}")
    assert e_out <= TOL[w.prec] and e_y <= TOL[w.prec]


@pytest.mark.parametrize("name", list(FWD_CASES))
def test_layer_fwd(name):
    w = FWD_CASES[name]
    _log("layer_fwd", name)
    c = make_host_case(w)
    L = _layer(c, with_bwd=False)
    L.forward()
    torch.cuda.synchronize()
    L.check_status()
    full = name.endswith("_full")
    n = 24 if full else min(w.T_src * len(w.own), 64)
    toks = sample_tokens(w, n) if full else sorted(
        {(s, t) for s in w.own for t in range(w.T_src)})[:: max(1, (w.T_src * len(w.own)) // n)]
    _check_fwd(c, L, toks)


BWD_CASES = {
    "bf16_all_local": _small("C2", S=2, T_src=100, d=128, E=8, k=2, I=128, own=[0, 1],
                             local_experts=list(range(8))),
    "f32": _small("C1", S=1, T_src=90, d=64, E=4, k=2, I=192, own=[0], local_experts=[0, 1, 2, 3]),
    "bf16_share": _small("C3", S=3, T_src=65, d=128, E=16, k=4, I=192, own=[1],
                         local_experts=[1, 4, 7, 10, 13], zipf_s=0.0),
    # about 6000 rows per expert: the weight gradients run split over 4096-row chunks
    "bf16_split_k": _small("C2", S=2, T_src=6000, d=128, E=4, k=2, I=128, own=[0],
                           local_experts=[0, 1, 2, 3]),
    # the largest top-k the ABI takes (16): 16 slots per token through the
    # combine, the gate-gradient group of the dx sum and the router backward
    "bf16_k16": _small("C2", S=1, T_src=96, d=128, E=32, k=16, I=128, own=[0],
                       local_experts=list(range(32))),
    # 256 (gate/up) and 128 (down) weight-gradient tiles per expert: whole experts
    # spread over all XCDs, most routed expert first
    "bf16_spread": _small("C2", S=2, T_src=32, d=4096, E=4, k=2, I=2048, own=[0, 1],
                          local_experts=[0, 1, 2]),
}


@pytest.mark.parametrize("name", list(BWD_CASES))
def test_layer_bwd(name):
    w = BWD_CASES[name]
    _log("layer_bwd", name)
    c = make_host_case(w)
    L = _layer(c)
    dout_store = [synth.gen_dout(w, s) for s in range(w.S)]
    d_out = [to_device(a, w.prec, DEV) for a, _ in dout_store]
    for t in (L.dw_gate, L.dw_up, L.dw_down, L.dw_router):
        t.fill_(float("nan"))  # every element must be overwritten
    L.forward()
    L.backward(d_out)
    torch.cuda.synchronize()
    L.check_status()
    lay = c.layout
    tol = TOL[w.prec]
    # per own token: d_gate, dx (incl. router path)
    toks = [(s, t) for s in w.own for t in range(w.T_src)]
    tok_x = np.stack([c.x_val[s][t] for s, t in toks])
    tok_d = np.stack([dout_store[s][1][t] for s, t in toks])
    idx = np.stack([c.topk_all[s, t] for s, t in toks])
    g = np.stack([c.gate_all[s, t] for s, t in toks])
    dg_ref, dz_ref, dx_ref = oracle.bwd_tokens(tok_x, tok_d, idx, g, c.e2l, c.wr_val, c.wg_val,
                                               c.wu_val, c.wd_val, peer_dg=peer_rows(c, toks, 2),
                                               peer_dx=peer_rows(c, toks, 4))
    dg = L.d_gate.cpu().numpy().reshape(w.S, w.T_src, w.k)
    dg_got = np.stack([dg[s, t] for s, t in toks])
    local = c.e2l[idx] >= 0
    assert rel_err(dg_got[local], dg_ref[local]) <= tol
    # remote slots: the peers' gate gradients are read, never overwritten
    np.testing.assert_array_equal(dg_got[~local], dg_ref[~local].astype(np.float32))
    dx_got = np.stack([L.d_x[s][t].float().cpu().numpy() for s, t in toks])
    e_dx = rel_err(dx_got, dx_ref)
    # weight gradients per local expert (rows of all sources, in layout order)
    e_w = 0.0
    for le in range(w.E_local):
        rows = lay["row_src"][lay["offsets"][le]:lay["offsets"][le + 1]]
        if len(rows) == 0:
            assert float(L.dw_gate[le].abs().max()) == 0.0
            continue
        tt = rows // w.k
        jj = rows % w.k
        rx = np.stack([c.x_val[t // w.T_src][t % w.T_src] for t in tt])
        rg = np.array([c.gate_all[t // w.T_src, t % w.T_src, j] for t, j in zip(tt, jj)])
        rd = np.stack([dout_store[t // w.T_src][1][t % w.T_src] for t in tt])
        dwg, dwu, dwd = oracle.expert_wgrad(rx, rg, rd, c.wg_val[le], c.wu_val[le], c.wd_val[le])
        e_w = max(e_w, rel_err(L.dw_gate[le].cpu().numpy(), dwg),
                  rel_err(L.dw_up[le].cpu().numpy(), dwu), rel_err(L.dw_down[le].cpu().numpy(), dwd))
    dwr_ref = oracle.router_wgrad(tok_x, idx, dz_ref, w.E)
    e_r = rel_err(L.dw_router.cpu().numpy(), dwr_ref)
    _log(f"  dx {e_dx:.3e} dW {e_w:.3e} dWr {e_r:.3e}")
    assert e_dx <= tol and e_w <= tol and e_r <= tol


@pytest.mark.parametrize("two_streams", [False, True])
def test_layer_empty_batch(two_streams):
    """No tokens at all (T_src = 0, so no routed rows): forward and backward
    run, latch no error, and every weight gradient -- of experts that
    received no rows -- is exactly zero."""
    w = _small("C2", S=2, T_src=0, d=128, E=8, k=2, I=128, own=[0, 1],
               local_experts=list(range(8)))
    _log("empty batch", two_streams)
    c = make_host_case(w)
    L = _layer(c, two_streams=two_streams)
    for t in (L.dw_gate, L.dw_up, L.dw_down, L.dw_router):
        t.fill_(float("nan"))
    d_out = [to_device(synth.gen_dout(w, s)[0], w.prec, DEV) for s in range(w.S)]
    L.forward()
    L.backward(d_out)
    torch.cuda.synchronize()
    L.check_status()
    assert int(L.offsets[-1].item()) == 0
    for t in (L.dw_gate, L.dw_up, L.dw_down, L.dw_router):
        assert float(t.abs().max()) == 0.0


def test_layer_rows_beyond_capacity_dropped():
    """More routed rows than R_cap: the layer latches MOK_ECAPACITY, computes
    the rows below R_cap, and the combine and the dx sum leave out the
    dropped slots (a dropped slot adds nothing to the output and has a zero
    gate gradient).  Expected values: the oracle's forward with the dropped
    slots sent to a remote expert holding zeros, and the backward composed
    of the oracle's per-row backward over the kept slots plus its router
    backward with zero gate gradients at the dropped slots."""
    w = BWD_CASES["bf16_all_local"]
    _log("capacity")
    c = make_host_case(w)
    R = int(c.layout["R"])
    R_cap = R - 37  # the last rows of the last expert(s) are dropped
    L = _layer(c, R_cap=R_cap)
    dout_store = [synth.gen_dout(w, s) for s in range(w.S)]
    d_out = [to_device(a, w.prec, DEV) for a, _ in dout_store]
    # rows an earlier call could have left: a dropped slot must not be read
    for s in range(w.S):
        L.staging[s].fill_(float("nan"))
        L.dx_stage[s].fill_(float("nan"))
    L.d_gate.fill_(float("nan"))
    L.forward()
    L.backward(d_out)
    torch.cuda.synchronize()
    assert STATUS[int(L.status.item())] == "MOK_ECAPACITY"
    dest = c.layout["dest_row"].reshape(w.S, w.T_src, w.k)
    toks = [(s, t) for s in w.own for t in range(w.T_src)]
    dropped = np.stack([dest[s, t] >= R_cap for s, t in toks])
    assert dropped.sum() == 37
    tok_x = np.stack([c.x_val[s][t] for s, t in toks])
    idx = np.stack([c.topk_all[s, t] for s, t in toks])
    g = np.stack([c.gate_all[s, t] for s, t in toks])
    # forward: dropped slots -> an extra expert id that is remote, pushed rows 0
    e2l_x = np.concatenate([c.e2l, [-1]]).astype(np.int32)
    idx_x = np.where(dropped, w.E, idx)
    wg, wu, wd = oracle_weights(c)
    _, out_ref = oracle.fwd_tokens(tok_x, idx_x, g, e2l_x, wg, wu, wd, w.prec,
                                   peer_y=np.zeros((len(toks), w.k, w.d)))
    out = np.stack([L.out[s][t].float().cpu().numpy() for s, t in toks])
    e_out = rel_err(out, out_ref)
    # backward: per-row backward of the kept slots, router backward with dg = 0
    # at the dropped ones
    dx_ref = np.zeros((len(toks), w.d))
    for i, (s, t) in enumerate(toks):
        dg = np.zeros(w.k)
        for j in range(w.k):
            if dropped[i, j]:
                continue
            le = c.e2l[idx[i, j]]
            r = oracle.bwd_row(tok_x[i], g[i, j], dout_store[s][1][t], c.wg_val[le], c.wu_val[le],
                               c.wd_val[le])
            dg[j] = r["dg"]
            dx_ref[i] += r["dx"]
        _, dxr = oracle.router_bwd_token(idx[i], g[i], dg, c.wr_val)
        dx_ref[i] += dxr
    dx = np.stack([L.d_x[s][t].float().cpu().numpy() for s, t in toks])
    e_dx = rel_err(dx, dx_ref)
    # the weight gradients of the expert cut by the capacity cover its kept rows
    lay = c.layout
    le = int(np.searchsorted(lay["offsets"], R_cap - 1, side="right")) - 1
    rows = lay["row_src"][lay["offsets"][le]:min(lay["offsets"][le + 1], R_cap)]
    tt, jj = rows // w.k, rows % w.k
    rx = np.stack([c.x_val[q // w.T_src][q % w.T_src] for q in tt])
    rg = np.array([c.gate_all[q // w.T_src, q % w.T_src, j] for q, j in zip(tt, jj)])
    rd = np.stack([dout_store[q // w.T_src][1][q % w.T_src] for q in tt])
    dwg, dwu, dwd = oracle.expert_wgrad(rx, rg, rd, c.wg_val[le], c.wu_val[le], c.wd_val[le])
    e_w = max(rel_err(L.dw_gate[le].cpu().numpy(), dwg), rel_err(L.dw_up[le].cpu().numpy(), dwu),
              rel_err(L.dw_down[le].cpu().numpy(), dwd))
    _log(f"  out {e_out:.3e} dx {e_dx:.3e} dW(last expert) {e_w:.3e}")
    assert e_out <= TOL[w.prec] and e_dx <= TOL[w.prec] and e_w <= TOL[w.prec]


def _bwd_sampled(c, L, dout_store, toks):
    """d_gate and d_x of sampled own tokens against the oracle."""
    w = c.w
    tok_x = np.stack([c.x_val[s][t] for s, t in toks])
    tok_d = np.stack([dout_store[s][1][t] for s, t in toks])
    idx = np.stack([c.topk_all[s, t] for s, t in toks])
    g = np.stack([c.gate_all[s, t] for s, t in toks])
    dg_ref, _, dx_ref = oracle.bwd_tokens(tok_x, tok_d, idx, g, c.e2l, c.wr_val, c.wg_val,
                                          c.wu_val, c.wd_val, peer_dg=peer_rows(c, toks, 2),
                                          peer_dx=peer_rows(c, toks, 4))
    dg = L.d_gate.cpu().numpy().reshape(w.S, w.T_src, w.k)
    dg_got = np.stack([dg[s, t] for s, t in toks])
    local = c.e2l[idx] >= 0
    e_dg = rel_err(dg_got[local], dg_ref[local])
    np.testing.assert_array_equal(dg_got[~local], dg_ref[~local].astype(np.float32))
    dx_got = np.stack([L.d_x[s][t].float().cpu().numpy() for s, t in toks])
    e_dx = rel_err(dx_got, dx_ref)
    _log(f"  sampled d_gate {e_dg:.3e} dx {e_dx:.3e}")
    assert e_dg <= TOL[w.prec] and e_dx <= TOL[w.prec]


# full-size backward workloads: (workload, check the whole weight gradients of
# the least-routed local expert and the router weight gradient)
BWD_FULL = {
    "c5_full": (synth.WORKLOADS["C5"], True),
    "c3_full": (synth.WORKLOADS["C3"], False),
}


def _expert_rows(c, dout_store, le):
    """Token rows, gates and upstream gradients of local expert le's rows."""
    w = c.w
    lay = c.layout
    rows = lay["row_src"][lay["offsets"][le]:lay["offsets"][le + 1]]
    tt, jj = rows // w.k, rows % w.k
    rx = np.stack([c.x_val[t // w.T_src][t % w.T_src] for t in tt])
    rg = np.array([c.gate_all[t // w.T_src, t % w.T_src, j] for t, j in zip(tt, jj)])
    rd = np.stack([dout_store[t // w.T_src][1][t % w.T_src] for t in tt])
    return rx, rg, rd


def _check_wgrad_columns(c, L, dout_store, le, n_sel=6):
    """Sampled intermediate columns of local expert le's three weight
    gradients against the oracle (every d column of each)."""
    w = c.w
    rng = np.random.default_rng(le)
    sel = np.unique(np.concatenate([[0, w.I - 1, 255, 256],
                                    rng.integers(0, w.I, n_sel)])).astype(np.int32)
    sel = sel[sel < w.I]
    rx, rg, rd = _expert_rows(c, dout_store, le)
    cg, cu, cd = oracle.expert_wgrad_cols(rx, rg, rd, c.wg_val[le], c.wu_val[le], c.wd_val[le], sel)
    st = torch.from_numpy(sel.astype(np.int64)).to(DEV)
    e = max(rel_err(L.dw_gate[le][st].cpu().numpy(), cg), rel_err(L.dw_up[le][st].cpu().numpy(), cu),
            rel_err(L.dw_down[le][:, st].cpu().numpy(), cd))
    _log(f"  expert {le} ({len(rx)} rows) dW columns {sel.tolist()}: rel err {e:.3e}")
    assert e <= TOL[w.prec]


def _check_router_wgrad_full(c, L, dout_store):
    """The whole router weight gradient over every own token: the oracle's
    gate gradients of every routed row come from its exact FFN of all rows
    (numpy matrix products), then dz and dW_router from the oracle."""
    w = c.w
    assert w.E_local == w.E and w.own == list(range(w.S))
    lay = c.layout
    dg = np.zeros(w.S * w.T_src * w.k)
    for le in range(w.E_local):
        rows = lay["row_src"][lay["offsets"][le]:lay["offsets"][le + 1]]
        if len(rows) == 0:
            continue
        tt = rows // w.k
        rx = np.stack([c.x_val[t // w.T_src][t % w.T_src] for t in tt])
        rd = np.stack([dout_store[t // w.T_src][1][t % w.T_src] for t in tt]).astype(np.float64)
        y = oracle.ffn_rows_exact(rx, c.wg_val[le], c.wu_val[le], c.wd_val[le])
        dg[rows] = np.einsum("rc,rc->r", rd, y)
    n_tok = w.S * w.T_src
    idx = c.topk_all.reshape(n_tok, w.k)
    dz = oracle.router_dz(idx, c.gate_all.reshape(n_tok, w.k), dg.reshape(n_tok, w.k))
    tok_x = np.concatenate([c.x_val[s] for s in range(w.S)])
    ref = oracle.router_wgrad(tok_x, idx, dz, w.E)
    e = rel_err(L.dw_router.cpu().numpy(), ref)
    _log(f"  dW_router (all {n_tok} tokens) rel err {e:.3e}")
    assert e <= TOL[w.prec]


@pytest.mark.parametrize("name", list(BWD_FULL))
def test_layer_bwd_full_sampled(name):
    """Full-size forward + backward in the launch configuration bench.py
    times, checked on sampled tokens (forward: routing and layout bit-exact,
    outputs and pushed rows; backward: d_gate and d_x; for the skewed
    mid-size layer also one expert's weight gradients)."""
    w, check_dw = BWD_FULL[name]
    _log("layer_bwd_full", name)
    c = make_host_case(w)
    L = _layer(c)
    dout_store = [synth.gen_dout(w, s) for s in range(w.S)]
    d_out = [to_device(a, w.prec, DEV) for a, _ in dout_store]
    L.forward()
    L.backward(d_out)
    torch.cuda.synchronize()
    L.check_status()
    toks = sample_tokens(w, 16)
    _check_fwd(c, L, toks)
    _bwd_sampled(c, L, dout_store, toks)
    lay = c.layout
    cnt = np.diff(lay["offsets"])
    # the most-routed expert's weight gradients, on sampled columns (the
    # chunked split-K schedule or the spread schedule, whichever the device
    # picks for these counts, at their longest contraction)
    _check_wgrad_columns(c, L, dout_store, int(np.argmax(cnt)))
    if not check_dw:
        return
    le = int(np.argmin(np.where(cnt > 0, cnt, np.iinfo(np.int64).max)))
    rx, rg, rd = _expert_rows(c, dout_store, le)
    _log(f"  expert {le}: {len(rx)} rows")
    dwg, dwu, dwd = oracle.expert_wgrad(rx, rg, rd, c.wg_val[le], c.wu_val[le], c.wd_val[le])
    e_w = max(rel_err(L.dw_gate[le].cpu().numpy(), dwg), rel_err(L.dw_up[le].cpu().numpy(), dwu),
              rel_err(L.dw_down[le].cpu().numpy(), dwd))
    _log(f"  dW rel err {e_w:.3e}")
    assert e_w <= TOL[w.prec]
    _check_router_wgrad_full(c, L, dout_store)


def test_fwd_bwd_run_to_run_bit_identical():
    w = BWD_CASES["bf16_all_local"].replace(T_src=400)
    _log("determinism")
    c = make_host_case(w)
    L = _layer(c)
    d_out = [to_device(synth.gen_dout(w, s)[0], w.prec, DEV) for s in range(w.S)]
    snaps = []
    for _ in range(2):
        L.forward()
        L.backward(d_out)
        torch.cuda.synchronize()
        snaps.append([t.clone() for t in (L.out[0], L.out[1], L.staging[0], L.h, L.ab, L.d_gate,
                                          L.d_x[0], L.d_x[1], L.dw_gate, L.dw_up, L.dw_down,
                                          L.dw_router)])
    for a, b in zip(*snaps):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                           b.view(torch.uint8) if b.dtype != torch.uint8 else b)


@pytest.mark.parametrize("name", ["bf16_all_local", "bf16_share", "bf16_split_k"])
def test_bwd_two_streams_bit_identical_to_one(name):
    """The backward with its side work on a second stream (mok_aux) gives the
    same bytes as the one-stream backward, twice in a row."""
    w = BWD_CASES[name]
    _log("two streams", name)
    c = make_host_case(w)
    d_out = [to_device(synth.gen_dout(w, s)[0], w.prec, DEV) for s in range(w.S)]
    snaps = []
    for two in (False, True, True):
        L = _layer(c, two_streams=two)
        assert (L.aux is not None) == two
        L.forward()
        L.backward(d_out)
        torch.cuda.synchronize()
        L.check_status()
        snaps.append([t.clone() for t in [L.d_gate, L.dw_gate, L.dw_up, L.dw_down, L.dw_router] +
                      [L.d_x[s] for s in w.own] + [L.dx_stage[s] for s in range(w.S)]])
        del L
    for snap in snaps[1:]:
        for a, b in zip(snaps[0], snap):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("name", ["bf16_all_local", "bf16_share", "bf16_spread"])
def test_bwd_transposed_weights_bit_identical(name):
    """dh and dx reading the prepared W^T (k-contiguous, mok_prepare_bwd) give
    the same bytes as reading W itself through the transposing LDS loads."""
    w = BWD_CASES[name]
    _log("transposed weights", name)
    c = make_host_case(w)
    d_out = [to_device(synth.gen_dout(w, s)[0], w.prec, DEV) for s in range(w.S)]
    snaps = []
    for tw in (False, True):
        L = _layer(c, transposed_weights=tw)
        assert (L.weights.wt_down is not None) == tw
        L.forward()
        L.backward(d_out)
        torch.cuda.synchronize()
        L.check_status()
        snaps.append([t.clone() for t in [L.d_gate, L.dw_gate, L.dw_up, L.dw_down, L.dw_router] +
                      [L.d_x[s] for s in w.own] + [L.dx_stage[s] for s in range(w.S)]])
        del L
    for a, b in zip(*snaps):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_mx_quantize_bit_exact():
    w = synth.WORKLOADS["C2"].replace(E=2, local_experts=[0, 1], I=256, d=512)
    _log("mx_quantize")
    store, val = synth.gen_expert_weights(w, "gate")
    rows, K = w.E_local * w.I, w.d
    codes = torch.zeros(rows * K, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(rows * K // 32, dtype=torch.uint8, device=DEV)
    mok_mx_quantize(rows, K, to_device(store, "bf16", DEV), codes, scales)
    torch.cuda.synchronize()
    rc, rs = oracle.mx_quantize(val.reshape(rows, K).astype(np.float64))
    np.testing.assert_array_equal(codes.cpu().numpy().reshape(rows, K), rc)
    np.testing.assert_array_equal(scales.cpu().numpy().reshape(rows, K // 32), rs)


def test_mx_quantize_every_bf16_value():
    """The E4M3 conversion (gfx950's packed fp8 conversion of the clamped
    value) against the oracle's bit-level rule on every finite bf16 value
    below 2 in magnitude, each in 32-blocks whose leader (the block maximum)
    is 1, 1.5, 1.75, 1.875 or 1.9921875: the scaled values then reach every
    E4M3 normal and subnormal, exact ties, and the saturation above 448."""
    _log("mx_quantize every bf16 value")
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 2.0)]
    blocks = []
    for lead in (1.0, 1.5, 1.75, 1.875, 1.9921875):
        v = f[np.abs(f) <= lead]
        n = -(-len(v) // 31) * 31
        v = np.concatenate([v, np.zeros(n - len(v), np.float32)]).reshape(-1, 31)
        blocks.append(np.concatenate([np.full((len(v), 1), lead, np.float32), v], axis=1))
    blk = np.concatenate(blocks)                        # [blocks, 32]
    K = 512
    nb = -(-len(blk) // (K // 32)) * (K // 32)
    blk = np.concatenate([blk, np.zeros((nb - len(blk), 32), np.float32)])
    val = blk.reshape(-1, K)
    rows = val.shape[0]
    codes = torch.zeros(rows * K, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(rows * K // 32, dtype=torch.uint8, device=DEV)
    src = torch.from_numpy(val).to(torch.bfloat16).to(DEV)  # exact: every value is a bf16
    mok_mx_quantize(rows, K, src, codes, scales)
    torch.cuda.synchronize()
    rc, rs = oracle.mx_quantize(val.astype(np.float64))
    np.testing.assert_array_equal(codes.cpu().numpy().reshape(rows, K), rc)
    np.testing.assert_array_equal(scales.cpu().numpy().reshape(rows, K // 32), rs)


def test_mx_quantize_f32_rounding_cases():
    """The E4M3 conversion of fp32 values (the GEMM1 epilogue's path for h)
    against the oracle's bit-level rule: every fp32 exponent below 2^10 with
    every top-7 mantissa pattern and the low mantissa bits that decide the
    rounding (0, 1, just below, at and above the half-way point of the
    dropped bits, all ones), both signs, in blocks of 31 under leaders that
    put their scaled values across the whole E4M3 range (subnormals, ties,
    saturation above 448)."""
    _log("mx_quantize_f32 rounding cases")
    hi = np.arange(0x4480, dtype=np.uint32) << 16            # sign 0, exponent <= 136, top 7 mantissa bits
    low = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    pat = (hi[:, None] | low[None, :]).reshape(-1)
    f = np.concatenate([pat, pat | 0x80000000]).view(np.float32)
    blocks = []
    for lead in (1.0, 1.75, 1.9921875, 512.0, 1000.0):
        v = f[np.abs(f) <= lead]
        n = -(-len(v) // 31) * 31
        v = np.concatenate([v, np.zeros(n - len(v), np.float32)]).reshape(-1, 31)
        blocks.append(np.concatenate([np.full((len(v), 1), lead, np.float32), v], axis=1))
    blk = np.concatenate(blocks)
    K = 512
    nb = -(-len(blk) // (K // 32)) * (K // 32)
    val = np.concatenate([blk, np.zeros((nb - len(blk), 32), np.float32)]).reshape(-1, K)
    rows = val.shape[0]
    codes = torch.zeros(rows * K, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(rows * K // 32, dtype=torch.uint8, device=DEV)
    mok_mx_quantize_f32(rows, K, torch.from_numpy(val).to(DEV), codes, scales)
    torch.cuda.synchronize()
    rc, rs = oracle.mx_quantize(val.astype(np.float64))
    np.testing.assert_array_equal(codes.cpu().numpy().reshape(rows, K), rc)
    np.testing.assert_array_equal(scales.cpu().numpy().reshape(rows, K // 32), rs)


def _mx_rows_ref(c, rows):
    """The oracle's MX codes and scales of the token rows behind routed rows."""
    w = c.w
    toks = c.layout["row_src"][rows] // w.k
    v = np.stack([c.x_val[t // w.T_src][t % w.T_src] for t in toks]).astype(np.float64)
    return oracle.mx_quantize(v)


@pytest.mark.parametrize("name", ["mx_share", "c4_full"])
def test_dispatch_mx_bytes_bit_exact(name):
    """The MXFP8 pull dispatch quantises each gathered row: its E4M3 codes and
    E8M0 scales equal the oracle's MX quantisation of the token rows, byte
    for byte (every row of the small share; at full size the first and last
    rows of every expert plus 3000 sampled rows)."""
    w = FWD_CASES[name]
    _log("dispatch mx bytes", name)
    c = make_host_case(w)
    lay = c.layout
    R = int(lay["R"])
    cfg = make_config(w.S, w.T_src, w.d, w.E, w.k, w.I, w.E_local, "mxfp8", R)
    xq = torch.zeros(R * w.d, dtype=torch.uint8, device=DEV)
    xs = torch.zeros(R * w.d // 32, dtype=torch.uint8, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    mok_dispatch(cfg, [to_device(a, "bf16", DEV) for a in c.x_store],
                 torch.from_numpy(lay["row_src"]).to(DEV), torch.from_numpy(lay["offsets"]).to(DEV),
                 xq, xs, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    if name.endswith("_full"):
        rng = np.random.default_rng(9)
        offs = lay["offsets"]
        rows = set(rng.integers(0, R, 3000).tolist())
        for e in range(w.E_local):
            if offs[e + 1] > offs[e]:
                rows |= {int(offs[e]), int(offs[e + 1]) - 1}
        rows = np.array(sorted(rows))
    else:
        rows = np.arange(R)
    rc, rs = _mx_rows_ref(c, rows)
    got_c = xq.view(R, w.d)[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    got_s = xs.view(R, w.d // 32)[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    np.testing.assert_array_equal(got_c, rc)
    np.testing.assert_array_equal(got_s, rs)
