"""The persistent ring kernel (mok_layer_fwd with ring_bytes > 0) against the
one-launch-per-GEMM path and the oracle.

The ring path must give bit-identical h, a | b, staging rows and outputs for
every ring size (down to one slot, so slots are recycled), minibatch size and
split of workgroups between the dispatch and GEMM sides.  A wait bound set
from the host (1 microsecond) must end in MOK_ETIMEOUT with every workgroup
returning, after which the layer runs normally again."""
import numpy as np
import pytest
import torch

from cases import make_host_case, sample_tokens
from combine_router_top_expert_amd import synth
from combine_router_top_expert_amd.layer import to_device
from test_gpu_parity import BWD_CASES, DEV, _check_fwd, _layer, _log, _small

pytestmark = pytest.mark.gpu

MiB = 1 << 20


def _slot_bytes(w, mb):
    b = mb * w.d * 2 if w.prec != "mxfp8" else mb * w.d + mb * (w.d // 32)
    return (b + 255) // 256 * 256


BF16_SMALL = _small("C2", S=2, T_src=300, d=256, E=8, k=2, I=320, own=[0, 1],
                    local_experts=list(range(8)))
SHARE = _small("C3", S=3, T_src=65, d=128, E=16, k=4, I=192, own=[1],
               local_experts=[1, 4, 7, 10, 13], zipf_s=0.0)
MX_SMALL = _small("C4", S=2, T_src=300, d=256, E=8, k=2, I=256, own=[0, 1],
                  local_experts=list(range(8)))

# name -> (workload, minibatch rows, ring slots or bytes, comm_wgs, gemm_wgs, oracle check)
RING_CASES = {
    "bf16_mb64_2slots_split4x12": (BF16_SMALL, 64, 2, 4, 12, True),
    "bf16_mb256_1slot_auto": (BF16_SMALL, 256, 1, 0, 0, True),
    "bf16_mb512_3slots_split2x30": (BF16_SMALL, 512, 3, 2, 30, False),
    "bf16_mb32_1slot_split1x1": (BF16_SMALL, 32, 1, 1, 1, False),
    "share_mb64_2slots": (SHARE, 64, 2, 3, 9, True),
    "mx_mb128_2slots": (MX_SMALL, 128, 2, 4, 28, True),
    "mx_mb256_1slot_auto": (MX_SMALL, 256, 1, 0, 0, False),
    "c2_full_256MiB": (synth.WORKLOADS["C2"], 256, 256 * MiB, 0, 0, False),
    "c4_full_64MiB": (synth.WORKLOADS["C4"], 256, 64 * MiB, 0, 0, False),
    # the one-GPU share of the 256-expert layer through its 256 MiB ring: 18,724
    # bf16 rows of d = 7168, so the ring's slots are recycled about twice over
    # the ~38.8k routed rows; the smallest minibatch of the sweep and the one
    # the tuner picks (with 16 dispatch workgroups)
    "c3_full_mb64_256MiB": (synth.WORKLOADS["C3"], 64, 256 * MiB, 0, 0, "sampled"),
    "c3_full_mb512_256MiB": (synth.WORKLOADS["C3"], 512, 256 * MiB, 16, 0, "sampled"),
}

_CASES = {}


def _host_case(w):
    """Host inputs and oracle routing of a workload, built once per module
    (the full share takes about a minute)."""
    key = repr(w)
    if key not in _CASES:
        _CASES.clear()
        _CASES[key] = make_host_case(w)
    return _CASES[key]


def _ring_bytes(w, mb, ring):
    return ring if ring >= MiB else ring * _slot_bytes(w, mb)


def _same(a, b):
    a = a.view(torch.uint8) if a.dtype != torch.uint8 else a
    b = b.view(torch.uint8) if b.dtype != torch.uint8 else b
    return torch.equal(a, b)


@pytest.mark.parametrize("name", list(RING_CASES))
def test_ring_bit_identical_to_staged(name):
    w, mb, ring, comm, gemm, check = RING_CASES[name]
    _log("ring", name)
    c = _host_case(w)
    ref = _layer(c, with_bwd=False)
    ref.forward()
    rb = _ring_bytes(w, mb, ring)
    L = _layer(c, with_bwd=False, ring_bytes=rb, minibatch_rows=mb, comm_wgs=comm,
               gemm_wgs=gemm)
    L.forward()
    torch.cuda.synchronize()
    ref.check_status()
    L.check_status()
    R = int(c.layout["R"])
    _log(f"  R={R} slots={rb // _slot_bytes(w, mb)} minibatches>={-(-R // mb)}")
    if w.prec == "mxfp8":
        n = R * w.I
        assert _same(L.h[:n], ref.h[:n])
    else:
        assert _same(L.h[:R], ref.h[:R])
        assert _same(L.ab[:R], ref.ab[:R])
    for s in range(w.S):
        assert _same(L.staging[s], ref.staging[s]), s
    for s in w.own:
        assert _same(L.out[s], ref.out[s]), s
    if check == "sampled":
        _check_fwd(c, L, sample_tokens(w, 16))
    elif check:
        toks = sorted({(s, t) for s in w.own for t in range(w.T_src)})[::5]
        _check_fwd(c, L, toks)


def test_ring_repeated_calls_bit_identical():
    """Counters are re-armed on every call: three calls in a row agree."""
    w = BF16_SMALL
    _log("ring repeat")
    c = make_host_case(w)
    L = _layer(c, with_bwd=False, ring_bytes=2 * _slot_bytes(w, 64), minibatch_rows=64)
    outs = []
    for _ in range(3):
        L.forward()
        torch.cuda.synchronize()
        L.check_status()
        outs.append([t.clone() for t in L.staging] + [L.out[0].clone(), L.out[1].clone()])
    for a, b in zip(outs[0], outs[2]):
        assert _same(a, b)


def test_ring_tuner_picks_a_candidate_and_keeps_results():
    """mok_tune_fwd times every (minibatch rows, dispatch workgroups) pair the
    ring can take, skips the others (a minibatch larger than the ring, a
    split beyond the CUs), returns the fastest, and leaves the outputs of one
    forward call: bit-identical to the staged path."""
    w = BF16_SMALL
    _log("ring tuner")
    c = make_host_case(w)
    ref = _layer(c, with_bwd=False)
    ref.forward()
    rb = 2 * _slot_bytes(w, 128)  # two 128-row slots: a 512-row minibatch does not fit
    L = _layer(c, with_bwd=False, ring_bytes=rb, minibatch_rows=64)
    table = L.tune(mbs=[64, 128, 512], comms=[4, 8, 100000], reps=2)
    torch.cuda.synchronize()
    L.check_status()
    ran = {key: v for key, v in table.items() if v is not None}
    assert set(ran) == {(64, 4), (64, 8), (128, 4), (128, 8)}, table
    assert all(v > 0 for v in ran.values())
    best = (L.cfg.minibatch_rows, L.cfg.comm_wgs)
    assert ran[best] == min(ran.values())
    for s in range(w.S):
        assert _same(L.staging[s], ref.staging[s]), s
    for s in w.own:
        assert _same(L.out[s], ref.out[s]), s
    L.forward()
    torch.cuda.synchronize()
    L.check_status()
    for s in w.own:
        assert _same(L.out[s], ref.out[s]), s


def test_ring_wait_bound_latches_timeout():
    """A 1 us bound on every wait: the kernel ends with MOK_ETIMEOUT (the
    waits of a C2-sized forward cannot all be met that fast) and every
    workgroup returns; a normal call afterwards is correct."""
    w = synth.WORKLOADS["C2"]
    _log("ring timeout")
    c = make_host_case(w)
    rb = 4 * _slot_bytes(w, 256)
    L = _layer(c, with_bwd=False, ring_bytes=rb, minibatch_rows=256, wait_limit_us=1)
    L.forward()
    torch.cuda.synchronize()
    assert int(L.status.item()) == -5  # MOK_ETIMEOUT
    ok = _layer(c, with_bwd=False, ring_bytes=rb, minibatch_rows=256)
    ok.forward()
    torch.cuda.synchronize()
    ok.check_status()
    ref = _layer(c, with_bwd=False)
    ref.forward()
    torch.cuda.synchronize()
    for s in w.own:
        assert _same(ok.out[s], ref.out[s])
    toks = sample_tokens(w, 12)
    _check_fwd(c, ok, toks)


@pytest.mark.parametrize("name", ["mx_small", "c4_full"])
def test_ring_mx_fill_bytes_bit_exact(name):
    """The MXFP8 ring's dispatch side quantises each pulled row into its slot:
    with a ring that holds every minibatch (no slot reused), each slot's E4M3
    codes and E8M0 scales equal the oracle's MX quantisation of the rows'
    tokens, byte for byte (all rows of the small case; at full size the
    first, last and 3000 sampled rows)."""
    from combine_router_top_expert_amd import mok_ring_layout
    from test_gpu_parity import _mx_rows_ref
    w = MX_SMALL if name == "mx_small" else synth.WORKLOADS["C4"]
    mb = 128 if name == "mx_small" else 256
    _log("ring mx fill", name)
    c = _host_case(w)
    lay = c.layout
    R = int(lay["R"])
    offs = lay["offsets"]
    # minibatches in expert order: (first row, rows)
    mbs = [(r0, min(mb, int(offs[e + 1]) - r0)) for e in range(w.E_local)
           for r0 in range(int(offs[e]), int(offs[e + 1]), mb)]
    rb = (len(mbs) + 1) * _slot_bytes(w, mb)
    L = _layer(c, with_bwd=False, ring_bytes=rb, minibatch_rows=mb)
    off, sb, nslot = mok_ring_layout(L.cfg)
    assert nslot >= len(mbs)
    L.forward()
    torch.cuda.synchronize()
    L.check_status()
    ring = L.ws[off:off + nslot * sb].view(nslot, sb)
    codes = ring[:, :mb * w.d].reshape(nslot, mb, w.d)
    scales = ring[:, mb * w.d:mb * w.d + mb * w.d // 32].reshape(nslot, mb, w.d // 32)
    slot_of_row = np.empty(R, np.int64)
    q_of_row = np.empty(R, np.int64)
    for m, (r0, n) in enumerate(mbs):
        slot_of_row[r0:r0 + n] = m
        q_of_row[r0:r0 + n] = np.arange(n)
    if name.endswith("_full"):
        rng = np.random.default_rng(3)
        rows = set(rng.integers(0, R, 3000).tolist()) | {0, R - 1}
        rows = np.array(sorted(rows))
    else:
        rows = np.arange(R)
    rc, rs = _mx_rows_ref(c, rows)
    si = torch.from_numpy(slot_of_row[rows]).to(DEV)
    qi = torch.from_numpy(q_of_row[rows]).to(DEV)
    np.testing.assert_array_equal(codes[si, qi].cpu().numpy(), rc)
    np.testing.assert_array_equal(scales[si, qi].cpu().numpy(), rs)


def _second_call(c):
    """Host inputs of a second layer call with the first one's weights and
    router: new token rows (and new routing of the other sources), from the
    generator with other seeds."""
    from cases import oracle_routing
    w = c.w
    d = make_host_case(w.replace(index=w.index + 40), route_own=False)
    d.w = w
    d.wr_store, d.wr_val, d.bias = c.wr_store, c.wr_val, c.bias
    d.wg_store, d.wg_val, d.wu_store, d.wu_val = c.wg_store, c.wg_val, c.wu_store, c.wu_val
    d.wd_store, d.wd_val = c.wd_store, c.wd_val
    oracle_routing(d)
    return d


def _state_bytes(L, R):
    outs = [L.topk_idx, L.topk_gate, L.counts, L.offsets, L.row_src[:R], L.dest_row]
    if L.prec == "mxfp8":
        outs.append(L.h[:R * L.I])
    else:
        outs += [L.h[:R], L.ab[:R]]
    return outs + list(L.staging) + [L.out[s] for s in range(L.S) if L.out[s] is not None]


# name -> (workload, calls, minibatch rows, ring slots or bytes, comm_wgs, gemm_wgs)
MACRO_CASES = {
    "bf16_2calls_2slots_split4x12": (BF16_SMALL, 2, 64, 2, 4, 12),
    "bf16_3calls_256MiB_auto": (BF16_SMALL, 3, 256, 256 * MiB, 0, 0),
    "share_2calls_3slots": (SHARE, 2, 64, 3, 3, 9),
    "mx_2calls_2slots": (MX_SMALL, 2, 128, 2, 4, 28),
    "c2_full_2calls_256MiB": (synth.WORKLOADS["C2"], 2, 256, 256 * MiB, 0, 0),
}


@pytest.mark.parametrize("name", list(MACRO_CASES))
def test_macro_calls_bit_identical_to_separate_calls(name):
    """mok_layer_fwd_macro over several layer calls (one ring launch, the
    combine of call i beside the pull of call i + 1) leaves every call's
    state, staging rows and outputs byte-identical to separate staged
    mok_layer_fwd calls, and oracle-correct on sampled tokens."""
    from combine_router_top_expert_amd import mok_layer_fwd_macro
    w, n_calls, mb, ring, comm, gemm = MACRO_CASES[name]
    _log("macro", name)
    cases = [_host_case(w)]
    while len(cases) < n_calls:
        cases.append(_second_call(cases[-1]))
    R_cap = max(int(c.layout["R"]) for c in cases)
    refs, want = [], []
    for c in cases:
        ref = _layer(c, R_cap=R_cap, with_bwd=False)
        ref.forward()
        torch.cuda.synchronize()
        ref.check_status()
        want.append([t.clone() for t in _state_bytes(ref, int(c.layout["R"]))])
        del ref
    rb = _ring_bytes(w, mb, ring)
    Ls = [_layer(c, R_cap=R_cap, with_bwd=False, ring_bytes=rb, minibatch_rows=mb, comm_wgs=comm,
                 gemm_wgs=gemm) for c in cases]
    for L in Ls:  # outputs and layout must be written by the call
        for s in range(L.own_lo, L.own_lo + L.own_n):
            L.out[s].fill_(float("nan"))
        L.row_src.fill_(-7)
    L0 = Ls[0]
    calls = [dict(own_lo=L.own_lo, own_n=L.own_n, src_x=L.xs, state=L.state, staging=L.staging,
                  out=L.out) for L in Ls]
    mok_layer_fwd_macro(L0.cfg, calls, L0.w_router, L0.bias, L0.e2l, L0.weights, L0.ws, L0.status)
    torch.cuda.synchronize()
    L0.check_status()
    for i, (c, L) in enumerate(zip(cases, Ls)):
        got = _state_bytes(L, int(c.layout["R"]))
        for j, (a, b) in enumerate(zip(want[i], got)):
            assert _same(a, b), (i, j)
        if w.T_src * len(w.own) <= 2000:
            toks = sorted({(s, t) for s in w.own for t in range(w.T_src)})[::7]
        else:
            toks = sample_tokens(w, 8, seed=i)
        _check_fwd(c, L, toks)


def _bwd_ring_bytes(w, mb, slots):
    """Bytes of a backward ring of `slots` minibatch slots (dy, da | db and the
    transposed token rows of mb rows each, plus the column padding)."""
    slot = mb * (2 * w.d + 2 * w.I) * 2
    fixed = (64 * w.E_local + 64) * w.d * 2 + 3 * 256
    return fixed + slots * slot


def _bwd_bytes(L, w):
    outs = [L.d_gate, L.dw_gate, L.dw_up, L.dw_down, L.dw_router] + list(L.dx_stage)
    return outs + [L.d_x[s] for s in w.own]


# name -> (workload, minibatch rows, ring slots or bytes, oracle check)
BWD_RING_CASES = {
    # 64-row minibatches in 3 slots: many windows, experts cut across windows
    "all_local_mb64_3slots": (BWD_CASES["bf16_all_local"], 64, 3, "all"),
    # ~6000 rows per expert on the split-K schedule: 4096-row chunks cut by windows
    "split_k_mb256_2slots": (BWD_CASES["bf16_split_k"], 256, 2, None),
    # the spread schedule (whole experts, d = 4096, I = 2048) cut by windows
    "spread_mb64_5slots": (BWD_CASES["bf16_spread"], 64, 5, None),
    # a share with peer-written slots
    "share_mb64_2slots": (BWD_CASES["bf16_share"], 64, 2, "all"),
    # the skewed mid-size layer's backward through its 256 MiB ring
    "c5_full_256MiB": (synth.WORKLOADS["C5"], 256, 256 * MiB, "sampled"),
    # the 256-expert share's backward through a 256 MiB ring
    "c3_full_256MiB": (synth.WORKLOADS["C3"], 512, 256 * MiB, "sampled"),
}


@pytest.mark.parametrize("name", list(BWD_RING_CASES))
def test_ring_backward_bit_identical_to_staged(name):
    """The backward through the ring -- windows of whole minibatches whose dy,
    da | db and transposed token rows occupy the ring's slots, weight
    gradients carried over exactly from window to window -- gives the same
    bytes as the one-launch backward (d_gate, pushed dx rows, d_x, every
    weight gradient, the router gradient), and matches the oracle."""
    from test_gpu_parity import _bwd_sampled, _check_wgrad_columns, peer_rows, TOL
    import oracle
    from cases import rel_err
    w, mb, ring, check = BWD_RING_CASES[name]
    _log("ring backward", name)
    c = _host_case(w)
    dout_store = [synth.gen_dout(w, s) for s in range(w.S)]
    d_out = [to_device(a, w.prec, DEV) for a, _ in dout_store]
    ref = _layer(c)
    ref.forward()
    ref.backward(d_out)
    torch.cuda.synchronize()
    ref.check_status()
    want = [t.clone() for t in _bwd_bytes(ref, w)]
    del ref
    rb = ring if ring >= MiB else _bwd_ring_bytes(w, mb, ring)
    L = _layer(c, minibatch_rows=mb, bwd_ring_bytes=rb)
    for t in (L.dw_gate, L.dw_up, L.dw_down, L.dw_router):
        t.fill_(float("nan"))
    L.forward()
    L.backward(d_out)
    torch.cuda.synchronize()
    L.check_status()
    R = int(c.layout["R"])
    slot = mb * (2 * w.d + 2 * w.I) * 2
    slots = (rb - ((64 * w.E_local + 64) * w.d * 2 + 768)) // slot
    _log(f"  R={R} window rows={slots * mb} windows>={-(-R // (slots * mb))}")
    for j, (a, b) in enumerate(zip(want, _bwd_bytes(L, w))):
        assert _same(a, b), j
    if check == "all":
        toks = [(s, t) for s in w.own for t in range(w.T_src)]
        _bwd_sampled(c, L, dout_store, toks)
    elif check == "sampled":
        _bwd_sampled(c, L, dout_store, sample_tokens(w, 12))
        cnt = np.diff(c.layout["offsets"])
        _check_wgrad_columns(c, L, dout_store, int(np.argmax(cnt)))
