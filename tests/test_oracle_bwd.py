"""Pins of the oracle's backward by float64 central finite differences of the
oracle's own exact forward on tiny shapes (the selection is checked to stay
fixed under every perturbation), plus closed-form properties."""
import numpy as np
import pytest

import oracle
from combine_router_top_expert_amd import synth

H = 2.0 ** -12  # exact in fp32 for the bf16-valued inputs used here


def _bf16(a):
    return synth.bf16_bits_to_f32(synth.f64_to_bf16_bits(np.asarray(a, np.float64)))


def _setup(seed, T=6, d=16, E=4, k=2, I=12, local=None):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.normal(size=(T, d)))
    wr = _bf16(rng.normal(size=(E, d)) / np.sqrt(d))
    bias = _bf16(rng.normal(size=E) * 0.3)
    E_l = E if local is None else len(local)
    wg = _bf16(rng.normal(size=(E_l, I, d)) / np.sqrt(d))
    wu = _bf16(rng.normal(size=(E_l, I, d)) / np.sqrt(d))
    wd = _bf16(rng.normal(size=(E_l, d, I)) / np.sqrt(I))
    dout = _bf16(rng.normal(size=(T, d)))
    e2l = np.full(E, -1, np.int32)
    for i, e in enumerate(range(E) if local is None else local):
        e2l[e] = i
    return dict(x=x, wr=wr, bias=bias, wg=wg, wu=wu, wd=wd, dout=dout, e2l=e2l, k=k)


def _loss(p):
    idx, g = oracle.route(p["x"], p["wr"], p["bias"], p["k"], "exact")
    _, out = oracle.fwd_tokens(p["x"], idx, g, p["e2l"], p["wg"], p["wu"], p["wd"], "exact")
    return float((out * p["dout"].astype(np.float64)).sum()), idx


def _fd(p, name, pos):
    base_idx = _loss(p)[1]
    vals = []
    for sgn in (1, -1):
        q = dict(p)
        q[name] = p[name].copy()
        q[name][pos] += np.float32(sgn * H)
        L, idx = _loss(q)
        assert np.array_equal(idx, base_idx), "selection changed under perturbation"
        vals.append(L)
    return (vals[0] - vals[1]) / (2 * H)


def _analytic(p):
    idx, g = oracle.route(p["x"], p["wr"], p["bias"], p["k"], "exact")
    d_gate, dz, dx = oracle.bwd_tokens(p["x"], p["dout"], idx, g, p["e2l"], p["wr"], p["wg"],
                                       p["wu"], p["wd"])
    dwr = oracle.router_wgrad(p["x"], idx, dz, p["wr"].shape[0])
    E_l = p["wg"].shape[0]
    dW = []
    for le in range(E_l):
        rows = [(t, j) for t in range(idx.shape[0]) for j in range(idx.shape[1])
                if p["e2l"][idx[t, j]] == le]
        if rows:
            tt = [t for t, _ in rows]
            gg = [g[t, j] for t, j in rows]
            dW.append(oracle.expert_wgrad(p["x"][tt], np.array(gg), p["dout"][tt], p["wg"][le],
                                          p["wu"][le], p["wd"][le]))
        else:
            dW.append(tuple(np.zeros_like(w[le], dtype=np.float64)
                            for w in (p["wg"], p["wu"], p["wd"])))
    return dict(dx=dx, dwr=dwr, dW=dW, d_gate=d_gate, idx=idx, g=g)


@pytest.mark.parametrize("seed,local", [(0, None), (1, None), (2, [3, 1])])
def test_backward_matches_finite_differences(seed, local):
    p = _setup(seed, local=local)
    A = _analytic(p)
    rng = np.random.default_rng(seed + 50)
    T, d = p["x"].shape
    for _ in range(12):
        t, c = rng.integers(T), rng.integers(d)
        np.testing.assert_allclose(A["dx"][t, c], _fd(p, "x", (t, c)), rtol=1e-5, atol=1e-8)
    for _ in range(8):
        e, c = rng.integers(p["wr"].shape[0]), rng.integers(d)
        np.testing.assert_allclose(A["dwr"][e, c], _fd(p, "wr", (e, c)), rtol=1e-5, atol=1e-8)
    I = p["wg"].shape[1]
    for le in range(p["wg"].shape[0]):
        for _ in range(4):
            i, c = rng.integers(I), rng.integers(d)
            np.testing.assert_allclose(A["dW"][le][0][i, c], _fd(p, "wg", (le, i, c)), rtol=1e-5,
                                       atol=1e-8)
            np.testing.assert_allclose(A["dW"][le][1][i, c], _fd(p, "wu", (le, i, c)), rtol=1e-5,
                                       atol=1e-8)
            np.testing.assert_allclose(A["dW"][le][2][c, i], _fd(p, "wd", (le, c, i)), rtol=1e-5,
                                       atol=1e-8)


def test_gate_gradient_is_derivative_wrt_gate():
    p = _setup(3)
    A = _analytic(p)
    idx, g = A["idx"], A["g"]
    for t in range(idx.shape[0]):
        for j in range(idx.shape[1]):
            vals = []
            for sgn in (1, -1):
                gg = g.copy()
                gg[t, j] += sgn * H
                _, out = oracle.fwd_tokens(p["x"], idx, gg, p["e2l"], p["wg"], p["wu"], p["wd"],
                                           "exact")
                vals.append((out * p["dout"]).sum())
            np.testing.assert_allclose(A["d_gate"][t, j], (vals[0] - vals[1]) / (2 * H),
                                       rtol=1e-7, atol=1e-10)


def test_router_bwd_closed_form_properties():
    rng = np.random.default_rng(9)
    k, d, E = 4, 8, 6
    idx = np.array([4, 0, 2, 5], np.int32)
    g = rng.dirichlet(np.ones(k))
    dg = rng.normal(size=k)
    wr = rng.normal(size=(E, d)).astype(np.float32)
    dz, dxr = oracle.router_bwd_token(idx, g, dg, wr)
    assert abs(dz.sum()) < 1e-15           # softmax gradient sums to zero
    dz2, _ = oracle.router_bwd_token(idx, g, dg + 3.0, wr)   # invariant to a shift of dg
    np.testing.assert_allclose(dz, dz2, atol=1e-14)
    # FD through the softmax of the chosen logits
    z = rng.normal(size=k)
    gz = np.exp(z - z.max()); gz /= gz.sum()
    dz3, _ = oracle.router_bwd_token(idx, gz, dg, wr)
    for j in range(k):
        zp, zm = z.copy(), z.copy()
        zp[j] += 1e-6; zm[j] -= 1e-6
        f = lambda zz: (np.exp(zz - zz.max()) / np.exp(zz - zz.max()).sum() * dg).sum()
        np.testing.assert_allclose(dz3[j], (f(zp) - f(zm)) / 2e-6, rtol=1e-6, atol=1e-10)


def _split(p, mine):
    """Experts split between this GPU (`mine`) and a peer holding the rest:
    (e2l here, e2l at the peer, weights here, weights at the peer)."""
    E = p["e2l"].shape[0]
    theirs = [e for e in range(E) if e not in mine]
    e2l_a = np.full(E, -1, np.int32)
    e2l_b = np.full(E, -1, np.int32)
    for i, e in enumerate(mine):
        e2l_a[e] = i
    for i, e in enumerate(theirs):
        e2l_b[e] = i
    pick = lambda es: tuple(p[n][[p["e2l"][e] for e in es]] for n in ("wg", "wu", "wd"))
    return e2l_a, e2l_b, pick(mine), pick(theirs)


@pytest.mark.parametrize("mine", [[0, 2], [1], [0, 1, 3]])
def test_share_with_peer_slots_equals_all_local(mine):
    """Expert parallelism over two GPUs: the source's combine and backward
    sum over all k slots, the remote ones filled by the peer's push and its
    reverse-combine (pull, then push back).  With the peer's values taken from
    the same oracle run on the peer's experts, the share reproduces the
    all-local result exactly (same values, same slot order)."""
    p = _setup(21, T=7, d=16, E=4, k=3, I=12)
    idx, g = oracle.route(p["x"], p["wr"], p["bias"], p["k"], "exact")
    e2l_a, e2l_b, wa, wb = _split(p, mine)
    y_all, out_all = oracle.fwd_tokens(p["x"], idx, g, p["e2l"], p["wg"], p["wu"], p["wd"], "exact")
    y_b, _ = oracle.fwd_tokens(p["x"], idx, g, e2l_b, *wb, "exact")
    y_a, out_a = oracle.fwd_tokens(p["x"], idx, g, e2l_a, *wa, "exact", peer_y=y_b)
    np.testing.assert_array_equal(y_a, y_all)
    np.testing.assert_array_equal(out_a, out_all)
    # without the peer's rows the share misses exactly the remote slots' terms
    _, out_0 = oracle.fwd_tokens(p["x"], idx, g, e2l_a, *wa, "exact")
    remote = e2l_a[idx] < 0
    miss = np.einsum("tj,tjd->td", g * remote, y_all)
    np.testing.assert_allclose(out_all - out_0, miss, rtol=0, atol=1e-12)
    assert np.abs(miss).max() > 0.01
    # backward: the peer's gate gradients and dx rows of its slots
    dg_all, dz_all, dx_all = oracle.bwd_tokens(p["x"], p["dout"], idx, g, p["e2l"], p["wr"],
                                               p["wg"], p["wu"], p["wd"])
    T, k, d = idx.shape[0], idx.shape[1], p["x"].shape[1]
    peer_dg = np.zeros((T, k))
    peer_dx = np.zeros((T, k, d))
    for t in range(T):
        for j in range(k):
            lb = e2l_b[idx[t, j]]
            if lb >= 0:
                r = oracle.bwd_row(p["x"][t], g[t, j], p["dout"][t], wb[0][lb], wb[1][lb], wb[2][lb])
                peer_dg[t, j], peer_dx[t, j] = r["dg"], r["dx"]
    dg_a, dz_a, dx_a = oracle.bwd_tokens(p["x"], p["dout"], idx, g, e2l_a, p["wr"], *wa,
                                         peer_dg=peer_dg, peer_dx=peer_dx)
    np.testing.assert_array_equal(dg_a, dg_all)
    np.testing.assert_array_equal(dz_a, dz_all)
    np.testing.assert_array_equal(dx_a, dx_all)
    assert remote.any() and (~remote).any()


def test_expert_wgrad_cols_equal_the_whole_gradient_at_those_columns():
    """The sampled-column weight gradients are the same sums as the whole
    gradients (pinned by finite differences above), restricted to the
    selected intermediate indices."""
    rng = np.random.default_rng(21)
    n, d, I = 37, 24, 20
    x = rng.normal(size=(n, d)).astype(np.float32)
    g = rng.random(n)
    dout = rng.normal(size=(n, d)).astype(np.float32)
    wg = (rng.normal(size=(I, d)) / 5).astype(np.float32)
    wu = (rng.normal(size=(I, d)) / 5).astype(np.float32)
    wd = (rng.normal(size=(d, I)) / 5).astype(np.float32)
    dwg, dwu, dwd = oracle.expert_wgrad(x, g, dout, wg, wu, wd)
    sel = np.array([0, 7, 19, 3], np.int32)
    cg, cu, cd = oracle.expert_wgrad_cols(x, g, dout, wg, wu, wd, sel)
    np.testing.assert_allclose(cg, dwg[sel], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(cu, dwu[sel], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(cd, dwd[:, sel], rtol=1e-12, atol=1e-14)


def test_ffn_rows_exact_matches_the_row_oracle():
    """The matrix-product form of the exact FFN gives the row-by-row C
    oracle's exact y (float64, summation order aside)."""
    rng = np.random.default_rng(22)
    n, d, I = 19, 64, 96
    x = rng.normal(size=(n, d)).astype(np.float32)
    wg = (rng.normal(size=(I, d)) / 8).astype(np.float32)
    wu = (rng.normal(size=(I, d)) / 8).astype(np.float32)
    wd = (rng.normal(size=(d, I)) / 10).astype(np.float32)
    y = oracle.ffn_rows_exact(x, wg, wu, wd)
    for r in range(n):
        _, _, _, yr = oracle.ffn_row(x[r], wg, wu, wd, "exact")
        np.testing.assert_allclose(y[r], yr, rtol=1e-11, atol=1e-13)


def test_router_dz_matches_the_token_backward():
    rng = np.random.default_rng(23)
    n, k, E, d = 30, 3, 9, 16
    idx = np.stack([rng.permutation(E)[:k] for _ in range(n)]).astype(np.int32)
    g = rng.random((n, k))
    g /= g.sum(1, keepdims=True)
    dg = rng.normal(size=(n, k))
    wr = rng.normal(size=(E, d)).astype(np.float32)
    dz = oracle.router_dz(idx, g, dg)
    for t in range(n):
        ref, _ = oracle.router_bwd_token(idx[t], g[t], dg[t], wr)
        np.testing.assert_array_equal(dz[t], ref)
    # closed form: sum_j dz_j = sum_j g_j dg_j (1 - sum_i g_i) = 0 for gates summing to 1
    assert np.all(np.abs(dz.sum(1)) < 1e-12)


def _mx_bwd_case(seed, n=45, d=64, I=64):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.normal(size=(n, d)))
    g = rng.random(n)
    dout = _bf16(rng.normal(size=(n, d)))
    wg = _bf16(rng.normal(size=(I, d)) / np.sqrt(d))
    wu = _bf16(rng.normal(size=(I, d)) / np.sqrt(d))
    wd = _bf16(rng.normal(size=(d, I)) / np.sqrt(I))
    a = np.zeros((n, I))
    b = np.zeros((n, I))
    h = np.zeros((n, I))
    for r in range(n):
        a[r], b[r], h[r], _ = oracle.ffn_row(x[r], wg, wu, wd, "exact")
    return x, g, dout, a, b, h, wg, wu, wd


def test_mx_backward_without_quantisation_is_the_exact_backward():
    """With every MX quantisation and bf16 rounding off, the MXFP8 backward is
    the exact backward (pinned above by finite differences): the same rows'
    input gradients and the same weight gradients."""
    x, g, dout, a, b, h, wg, wu, wd = _mx_bwd_case(31)
    dx, dwg, dwu, dwd = oracle.expert_bwd_mx(x, g, dout, a, b, h, wg, wu, wd, quant=False)
    for r in range(x.shape[0]):
        ref = oracle.bwd_row(x[r], g[r], dout[r], wg, wu, wd)
        np.testing.assert_allclose(dx[r], ref["dx"], rtol=1e-10, atol=1e-12)
    rg, ru, rd = oracle.expert_wgrad(x, g, dout, wg, wu, wd)
    np.testing.assert_allclose(dwg, rg, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dwu, ru, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dwd, rd, rtol=1e-10, atol=1e-12)


def test_mx_backward_error_is_that_of_e4m3():
    """With quantisation on, the result stays within the error of E4M3
    operands (3 mantissa bits: each quantised factor carries at most 2^-4
    relative error) of the exact backward, and is not the exact backward."""
    x, g, dout, a, b, h, wg, wu, wd = _mx_bwd_case(32)
    qx, qg, qu, qd = oracle.expert_bwd_mx(x, g, dout, a, b, h, wg, wu, wd, quant=True)
    ex, eg, eu, ed = oracle.expert_bwd_mx(x, g, dout, a, b, h, wg, wu, wd, quant=False)
    for got, ref in ((qx, ex), (qg, eg), (qu, eu), (qd, ed)):
        err = np.abs(got - ref).max() / np.abs(ref).max()
        assert 1e-4 < err < 0.1, err


def test_mx_weight_gradient_quantises_along_the_rows():
    """One routed row: every column of the weight-gradient operands is a
    block holding that row's value and 31 zero paddings, so dW_down[c][i] is
    the product of the single-value MX round trips of dy[c] = bf16(g dout[c])
    and h[i] -- not of their row-wise (along d, along I) blocks."""
    x, g, dout, a, b, h, wg, wu, wd = _mx_bwd_case(33, n=1)

    def q1(v):
        blk = np.zeros((1, 32))
        blk[0, 0] = v
        c, s = oracle.mx_quantize(blk)
        return oracle.mx_dequantize(c, s)[0, 0]
    _, _, _, dwd = oracle.expert_bwd_mx(x, g, dout, a, b, h, wg, wu, wd, quant=True)
    dy = np.array([oracle.round_bf16(g[0] * float(v)) for v in dout[0]])
    want = np.array([[q1(dy[c]) * q1(h[0, i]) for i in range(h.shape[1])] for c in range(dy.size)])
    np.testing.assert_array_equal(dwd, want)


def test_gate_grads_match_the_rows_backward():
    """gate_grads on the exact forward's y equals the gate gradient the
    row backward derives (dout . y of the same row)."""
    rng = np.random.default_rng(41)
    d, I = 16, 24
    x = rng.standard_normal((3, d)).astype(np.float32)
    dout = rng.standard_normal((3, d)).astype(np.float32)
    wg, wu = (rng.standard_normal((I, d)) * 0.2).astype(np.float32), (rng.standard_normal((I, d)) * 0.2).astype(np.float32)
    wd = (rng.standard_normal((d, I)) * 0.2).astype(np.float32)
    y = np.stack([oracle.ffn_row(x[r], wg, wu, wd, "exact")[3] for r in range(3)])
    got = oracle.gate_grads(dout, y)
    for r in range(3):
        assert got[r] == pytest.approx(oracle.bwd_row(x[r], 0.5, dout[r], wg, wu, wd)["dg"],
                                       rel=1e-12, abs=1e-12)
