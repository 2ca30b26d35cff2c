"""The C-ABI library loads, exports every symbol include/mok.h declares, and
rejects invalid arguments on the host (no GPU work is enqueued here)."""
import ctypes
import os
import re

import pytest

import combine_router_top_expert_amd as mok
from combine_router_top_expert_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mok.LIB_PATH):
        build.build()
    return mok.lib()


def _declared():
    src = open(os.path.join(ROOT, "include", "mok.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|size_t|mok_status)\s+(mok_\w+)\(", src, re.M)))


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert set(names) == set(mok.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_version(L):
    assert mok.mok_version().startswith("mok ")


def _cfg(**kw):
    base = dict(S=2, T_src=100, d=256, E=8, k=2, I=128, E_local=8, prec="bf16", R_cap=400)
    base.update(kw)
    return mok.make_config(**base)


def test_workspace_bytes_host_logic(L):
    a = mok.mok_workspace_bytes(_cfg())
    b = mok.mok_workspace_bytes(_cfg(R_cap=4000))
    assert a > 0 and b > a
    assert mok.mok_workspace_bytes(_cfg(d=100)) == 0       # d % 64 != 0
    assert mok.mok_workspace_bytes(_cfg(k=9)) == 0         # k > E
    assert mok.mok_workspace_bytes(_cfg(S=65)) == 0        # too many sources


@pytest.mark.parametrize("bad", [dict(d=96), dict(I=100), dict(E=0), dict(k=0), dict(E_local=9),
                                 dict(prec=7), dict(R_cap=-1), dict(S=0)])
def test_invalid_config_rejected_before_any_launch(L, bad):
    cfg = _cfg(**bad)
    rc = L.mok_route(ctypes.byref(cfg), 10, 1, 1, None, 1, 1, None)
    assert rc == -1
    rc = L.mok_layout(ctypes.byref(cfg), 1, 1, 1, 1, 1, 1, 1, None, None)
    assert rc == -1


def test_null_pointers_rejected(L):
    cfg = _cfg()
    assert L.mok_route(ctypes.byref(cfg), 10, None, 1, None, 1, 1, None) == -1
    assert L.mok_layout(ctypes.byref(cfg), None, 1, 1, 1, 1, 1, 1, None, None) == -1
    assert L.mok_mx_quantize(4, 48, 1, 1, 1, None) == -1       # K % 32 != 0
    assert L.mok_combine(ctypes.byref(cfg), None, 1, 1, None, 0, 3, None, None, None) == -1


def _layer_fwd_rc(L, cfg):
    """mok_layer_fwd with dummy (never dereferenced) non-null pointers."""
    S = cfg.S
    tab = (ctypes.c_void_p * S)(*([1] * S))
    w = mok.mok_expert_weights(1, 1, 1, 1, 1, 1)
    st = mok.mok_fwd_state(*([1] * 8))
    return L.mok_layer_fwd(ctypes.byref(cfg), 0, S, ctypes.cast(tab, ctypes.c_void_p), 1, None, 1,
                           ctypes.byref(w), ctypes.byref(st), ctypes.cast(tab, ctypes.c_void_p),
                           ctypes.cast(tab, ctypes.c_void_p), 1, 1, None)


def test_ring_workspace_and_rejections(L):
    base = mok.mok_workspace_bytes(_cfg())
    ring = 3 << 20
    assert mok.mok_workspace_bytes(_cfg(ring_bytes=ring)) >= max(base, ring)  # fwd and bwd share
    assert mok.mok_workspace_bytes(_cfg(ring_bytes=ring, minibatch_rows=0)) == 0
    assert mok.mok_workspace_bytes(_cfg(ring_bytes=ring, comm_wgs=-1)) == 0
    assert mok.mok_workspace_bytes(_cfg(wait_limit_us=-5)) == 0
    # the ring path takes bf16 or MXFP8 (rejected before any launch)
    assert _layer_fwd_rc(L, _cfg(prec="f32", ring_bytes=ring)) == -1
    # a ring smaller than one minibatch of rows (256 rows x 256 x 2 bytes)
    assert _layer_fwd_rc(L, _cfg(ring_bytes=256 * 256 * 2 - 1, minibatch_rows=256)) == -1
    # MXFP8 expert GEMMs need d and I multiples of 128
    assert _layer_fwd_rc(L, _cfg(prec="mxfp8", I=192, ring_bytes=ring)) == -2


def _tune_rc(L, cfg, best=True, reps=1, n_mb=1):
    """mok_tune_fwd with dummy (never dereferenced) non-null pointers."""
    S = cfg.S
    tab = (ctypes.c_void_p * S)(*([1] * S))
    w = mok.mok_expert_weights(1, 1, 1, 1, 1, 1)
    st = mok.mok_fwd_state(*([1] * 8))
    mbs = (ctypes.c_int32 * 1)(64)
    out = mok.mok_config()
    return L.mok_tune_fwd(ctypes.byref(cfg), ctypes.cast(mbs, ctypes.c_void_p), n_mb, None, 0,
                          reps, 1 << 30, 0, S, ctypes.cast(tab, ctypes.c_void_p), 1, None, 1,
                          ctypes.byref(w), ctypes.byref(st), ctypes.cast(tab, ctypes.c_void_p),
                          ctypes.cast(tab, ctypes.c_void_p), 1, 1, None,
                          ctypes.byref(out) if best else None, None)


def test_tuner_rejects_bad_arguments_on_the_host(L):
    ring = _cfg(ring_bytes=1 << 20, minibatch_rows=64)
    assert _tune_rc(L, _cfg()) == -1                   # staged path: nothing to tune
    assert _tune_rc(L, ring, best=False) == -1         # no place for the result
    assert _tune_rc(L, ring, reps=0) == -1             # no timed call
    assert _tune_rc(L, ring, n_mb=65) == -1            # too many candidates
    assert _tune_rc(L, _cfg(ring_bytes=1 << 20, minibatch_rows=64, R_cap=0)) == -1


def test_backward_second_stream_checked_on_the_host(L):
    """mok_aux must name its own stream and three events (MOK_EINVAL before any launch)."""
    S = 2
    tab = (ctypes.c_void_p * S)(*([1] * S))
    tp = ctypes.cast(tab, ctypes.c_void_p)
    w = mok.mok_expert_weights(1, 1, 1, 1, 1, 1)
    st = mok.mok_fwd_state(*([1] * 8))
    for aux in (mok.mok_aux(None, (ctypes.c_void_p * 3)(1, 1, 1)),      # no stream
                mok.mok_aux(7, (ctypes.c_void_p * 3)(1, None, 1)),      # an event missing
                mok.mok_aux(7, (ctypes.c_void_p * 3)(1, 1, 1))):        # the call's own stream
        cfg = _cfg()
        cfg.aux = ctypes.addressof(aux)
        rc = L.mok_layer_bwd(ctypes.byref(cfg), 0, S, tp, tp, 1, 1, ctypes.byref(w),
                             ctypes.byref(st), tp, 1, tp, tp, 1, 1, 1, None, 1, 1,
                             7 if aux.stream == 7 and aux.events[1] else None)
        assert rc == -1
