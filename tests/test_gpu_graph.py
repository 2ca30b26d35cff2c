"""A whole layer step (forward + backward, the backward over two streams)
captured once in a HIP graph and replayed: every replay gives the bytes of
the eager step.  Eager work and synchronisations run between the replays,
and each replay is checked, so a node that only behaves on its first replay
would show.  The library enqueues no memset and no host synchronisation on
these paths, so the whole step can be captured."""
import pytest
import torch

from cases import make_host_case
from combine_router_top_expert_amd import synth
from combine_router_top_expert_amd.layer import to_device
from test_gpu_parity import BWD_CASES, DEV, _layer, _log, _small

pytestmark = pytest.mark.gpu

GRAPH_CASES = {
    "bf16_all_local": BWD_CASES["bf16_all_local"],
    "bf16_share": BWD_CASES["bf16_share"],
    "f32_c1_shape": _small("C1", T_src=256),
}


def _outputs(L, w):
    outs = [L.out[s] for s in w.own] + [L.staging[s] for s in range(w.S)] + [L.h]
    if L.with_bwd:
        outs += [L.d_gate, L.dw_gate, L.dw_up, L.dw_down, L.dw_router]
        outs += [L.d_x[s] for s in w.own] + [L.dx_stage[s] for s in range(w.S)]
    return [t.clone() for t in outs]


def _same(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("name", list(GRAPH_CASES))
def test_graph_replay_matches_eager(name):
    w = GRAPH_CASES[name]
    _log("graph", name)
    c = make_host_case(w)
    d_out = [to_device(synth.gen_dout(w, s)[0], w.prec, DEV) for s in range(w.S)]
    L = _layer(c)

    def step():
        L.forward()
        L.backward(d_out)

    step()
    torch.cuda.synchronize()
    L.check_status()
    ref = _outputs(L, w)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capturing stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device=DEV)
    for rep in range(3):
        # clobber the outputs eagerly, then replay
        for t in [L.out[s] for s in w.own] + ([L.dw_gate, L.dw_down] if L.with_bwd else []):
            t.fill_(float("nan"))
        scratch.add_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        L.check_status()
        got = _outputs(L, w)
        for i, (a, b) in enumerate(zip(ref, got)):
            assert _same(a, b), (rep, i)
    del g
