"""The no-allocation forward entry point, mok_layer_fwd_noalloc, called
through the C ABI, against mok_layer_fwd on the same inputs: routing, layout,
h, a | b, staging rows and outputs byte for byte (the same kernels run; the
only difference is where the layout's scratch lives).  Two calls in a row,
the second on a smaller input, so the static scratch holds the first call's
values when the second starts."""
import pytest
import torch

from cases import make_host_case
from combine_router_top_expert_amd import make_config, mok_layer_fwd_noalloc, MokError
from test_gpu_parity import DEV, _layer, _log, _small

pytestmark = pytest.mark.gpu

FIRST = _small("C2", S=8, T_src=1024, d=512, E=64, k=6, I=256, own=list(range(8)),
               local_experts=list(range(64)))
SECOND = _small("C3", S=3, T_src=65, d=128, E=16, k=4, I=192, own=[1],
                local_experts=[1, 4, 7, 10, 13], zipf_s=0.0)


def _snapshot(L, w):
    outs = [L.topk_idx, L.topk_gate, L.counts, L.offsets, L.row_src, L.dest_row, L.h, L.ab]
    outs += list(L.staging) + [L.out[s] for s in w.own]
    return [t.clone() for t in outs]


def _same(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_noalloc_forward_matches_layer_fwd_on_two_calls():
    for w in (FIRST, SECOND):
        _log("noalloc", w.S, w.T_src, w.d, w.E, w.k)
        c = make_host_case(w)
        ref = _layer(c, with_bwd=False)
        ref.forward()
        torch.cuda.synchronize()
        ref.check_status()
        want = _snapshot(ref, w)
        del ref
        L = _layer(c, with_bwd=False)
        # poison the outputs so that each must be written by the call (the
        # staging rows of remote slots are the peers' and are never written)
        for t in [L.h, L.ab] + [L.out[s] for s in w.own]:
            t.fill_(float("nan"))
        for t in (L.row_src, L.dest_row):
            t.fill_(-7)
        mok_layer_fwd_noalloc(L.cfg, L.own_lo, L.own_n, L.xs, L.w_router, L.bias, L.e2l,
                              L.weights, L.state, L.staging, L.out, L.status)
        torch.cuda.synchronize()
        L.check_status()
        got = _snapshot(L, w)
        R = int(c.layout["R"])
        for i, (a, b) in enumerate(zip(want, got)):
            if i == 4:  # row_src: the rows past R are not part of the layout
                a, b = a[:R], b[:R]
            assert _same(a, b), i


def test_noalloc_rejects_what_it_cannot_run():
    """Another precision, a ring, or a configuration whose layout counts do
    not fit the static scratch are refused before anything is enqueued."""
    w = FIRST
    c = make_host_case(w.replace(T_src=64))
    L = _layer(c, with_bwd=False)
    for bad, code in ((dict(prec="f32"), -1), (dict(ring_bytes=1 << 24), -1),
                      (dict(S=64, T_src=8192, k=16, E=256, E_local=256), -7)):
        base = dict(S=L.S, T_src=L.T_src, d=L.d, E=L.E, k=L.k, I=L.I, E_local=L.E_local,
                    prec="bf16", R_cap=L.R_cap)
        base.update(bad)
        cfg = make_config(**base)
        with pytest.raises(MokError) as ei:
            mok_layer_fwd_noalloc(cfg, 0, 1, L.xs, L.w_router, L.bias, L.e2l, L.weights, L.state,
                                  L.staging, L.out, L.status)
        assert ei.value.code == code
