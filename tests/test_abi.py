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


def test_every_export_declares_its_arguments(L):
    """Each binding gives ctypes the argument types of its C declaration, as
    many as the header lists: without them ctypes passes Python ints as
    32-bit C ints, and a 64-bit parameter then reads whatever the upper half
    of its register holds."""
    src = open(os.path.join(ROOT, "include", "mok.h")).read()
    for n in _declared():
        params = re.search(n + r"\(([^)]*)\);", src, re.S).group(1).strip()
        count = 0 if params in ("", "void") else params.count(",") + 1
        argtypes = getattr(L, n).argtypes
        assert argtypes is not None, n
        assert len(argtypes) == count, n


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
    # misaligned values (16-byte loads) or codes (8-byte stores), never dereferenced
    for f in (L.mok_mx_quantize, L.mok_mx_quantize_f32):
        assert f(4, 64, 0x1008, 0x2000, 0x3000, None) == -1
        assert f(4, 64, 0x1000, 0x2004, 0x3000, None) == -1
        assert f(0, 64, 0x1008, 0x2004, 0x3000, None) == 0  # nothing to do
    assert L.mok_combine(ctypes.byref(cfg), None, 1, 1, None, 0, 3, None, None, None) == -1
    # the matrix-core probe: kind, data flag, counts and output checked on the host
    assert L.mok_mfma_probe(2, 0, 10, 1, 0x1000, None) == -1
    assert L.mok_mfma_probe(0, 2, 10, 1, 0x1000, None) == -1
    assert L.mok_mfma_probe(1, 0, 0, 1, 0x1000, None) == -1
    assert L.mok_mfma_probe(1, 0, 10, 0, 0x1000, None) == -1
    assert L.mok_mfma_probe(0, 1, 10, 1, None, None) == -1


def _layer_fwd_rc(L, cfg):
    """mok_layer_fwd with dummy (never dereferenced) non-null pointers."""
    S = cfg.S
    tab = (ctypes.c_void_p * S)(*([1] * S))
    w = mok.mok_expert_weights(*([1] * 10))
    st = mok.mok_fwd_state(*([1] * 9))
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
    w = mok.mok_expert_weights(*([1] * 10))
    st = mok.mok_fwd_state(*([1] * 9))
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
    w = mok.mok_expert_weights(*([1] * 10))
    st = mok.mok_fwd_state(*([1] * 9))
    for aux in (mok.mok_aux(None, (ctypes.c_void_p * 3)(1, 1, 1)),      # no stream
                mok.mok_aux(7, (ctypes.c_void_p * 3)(1, None, 1)),      # an event missing
                mok.mok_aux(7, (ctypes.c_void_p * 3)(1, 1, 1))):        # the call's own stream
        cfg = _cfg()
        cfg.aux = ctypes.addressof(aux)
        rc = L.mok_layer_bwd(ctypes.byref(cfg), 0, S, tp, tp, 1, 1, ctypes.byref(w),
                             ctypes.byref(st), tp, 1, tp, tp, 1, 1, 1, None, 1, 1,
                             7 if aux.stream == 7 and aux.events[1] else None)
        assert rc == -1


def _tab(S, null_at=None):
    tab = (ctypes.c_void_p * S)(*([1] * S))
    if null_at is not None:
        tab[null_at] = None
    return ctypes.cast(tab, ctypes.c_void_p), tab


@pytest.mark.parametrize("which", ["src_x", "staging", "out_own"])
def test_layer_fwd_rejects_null_source_pointers(L, which):
    """The pull and the push may reach any source (which ones is known on the
    device only), so every src_x[s] and staging[s] must be set; out[s] only
    for the own sources.  MOK_EINVAL comes back before anything is enqueued."""
    S = 3
    cfg = _cfg(S=S)
    w = mok.mok_expert_weights(*([1] * 10))
    st = mok.mok_fwd_state(*([1] * 9))
    full, _k1 = _tab(S)
    bad, _k2 = _tab(S, 2 if which != "out_own" else 0)
    src = bad if which == "src_x" else full
    stg = bad if which == "staging" else full
    out = bad if which == "out_own" else full
    # own source 0 only: sources 1 and 2 are other ranks'
    rc = L.mok_layer_fwd(ctypes.byref(cfg), 0, 1, src, 1, None, 1, ctypes.byref(w),
                         ctypes.byref(st), stg, out, 1, 1, None)
    assert rc == -1


def test_layer_fwd_out_of_non_own_source_may_be_null(L):
    """out[s] of a source this GPU does not combine is never touched: a NULL
    there passes validation (the call then fails only at launch on a host
    without a GPU, with MOK_EDEVICE, never with MOK_EINVAL)."""
    S = 3
    cfg = _cfg(S=S, R_cap=0)
    w = mok.mok_expert_weights(*([1] * 10))
    st = mok.mok_fwd_state(*([1] * 9))
    full, _k1 = _tab(S)
    out, _k2 = _tab(S, 2)
    rc = L.mok_layer_fwd(ctypes.byref(cfg), 0, 1, full, 1, None, 1, ctypes.byref(w),
                         ctypes.byref(st), full, out, 1, 1, None)
    assert rc != -1


def test_combine_and_dispatch_reject_null_source_pointers(L):
    S = 3
    cfg = _cfg(S=S)
    full, _k1 = _tab(S)
    bad, _k2 = _tab(S, 1)
    # push (y given) into a NULL staging buffer of a non-own source
    assert L.mok_combine(ctypes.byref(cfg), 1, 1, 1, bad, 0, 1, full, 1, None) == -1
    # gather from a NULL source buffer
    assert L.mok_dispatch(ctypes.byref(cfg), bad, 1, 1, 1, None, 1, None) == -1


@pytest.mark.parametrize("which", ["d_out", "src_x", "staging", "dx_stage"])
def test_layer_bwd_rejects_null_source_pointers(L, which):
    S = 3
    cfg = _cfg(S=S)
    w = mok.mok_expert_weights(*([1] * 10))
    st = mok.mok_fwd_state(*([1] * 9))
    full, _k1 = _tab(S)
    bad, _k2 = _tab(S, 2)
    args = {k: (bad if k == which else full) for k in ("d_out", "src_x", "staging", "dx_stage")}
    rc = L.mok_layer_bwd(ctypes.byref(cfg), 0, 1, args["d_out"], args["src_x"], 1, 1,
                         ctypes.byref(w), ctypes.byref(st), args["staging"], 1, args["dx_stage"],
                         full, 1, 1, 1, None, 1, 1, None)
    assert rc == -1


def test_ring_layout_host_logic(L):
    """Where the ring sits in the workspace: past the forward's other pieces,
    slots of minibatch_rows rows (256-byte aligned), as many as fit."""
    cfg = _cfg(ring_bytes=10 * 64 * 256 * 2 + 100, minibatch_rows=64)
    off, sb, n = mok.mok_ring_layout(cfg)
    assert sb == 64 * 256 * 2 and n == 10
    assert off % 256 == 0 and off + n * sb <= mok.mok_workspace_bytes(cfg)
    cm = _cfg(prec="mxfp8", ring_bytes=1 << 20, minibatch_rows=128)
    off, sb, n = mok.mok_ring_layout(cm)
    assert sb == (128 * 256 + 128 * 8 + 255) // 256 * 256 and n == (1 << 20) // sb
    with pytest.raises(mok.MokError):
        mok.mok_ring_layout(_cfg())                         # no ring
    with pytest.raises(mok.MokError):
        mok.mok_ring_layout(_cfg(prec="f32", ring_bytes=1 << 20))


def test_noalloc_forward_rejections_on_the_host(L):
    """mok_layer_fwd_noalloc runs the bf16 staged layer only, and refuses a
    configuration whose layout counts outgrow its static scratch
    (MOK_ESCRATCH) -- both before any device call."""
    S = 2
    full, _k = _tab(S)
    w = mok.mok_expert_weights(*([1] * 10))
    st = mok.mok_fwd_state(*([1] * 9))

    def rc(cfg):
        return L.mok_layer_fwd_noalloc(ctypes.byref(cfg), 0, 1, full, 1, None, 1, ctypes.byref(w),
                                       ctypes.byref(st), full, full, 1, None)
    assert rc(_cfg(prec="f32")) == -1
    assert rc(_cfg(prec="mxfp8")) == -1
    assert rc(_cfg(ring_bytes=1 << 24)) == -1
    # ceil(64 * 8192 * 16 / 1024) chunks x 256 local experts x 4 bytes = 32 MiB > 4 MiB
    assert rc(_cfg(S=64, T_src=8192, k=16, E=256, E_local=256)) == -7


def test_macro_forward_rejections_on_the_host(L):
    """mok_layer_fwd_macro needs the ring, bf16 or MXFP8, 1..MOK_MAX_CALLS
    calls and every call's pointers (MOK_EINVAL before anything runs)."""
    S = 2
    full, _k1 = _tab(S)
    bad, _k2 = _tab(S, 1)
    w = mok.mok_expert_weights(*([1] * 10))
    st = mok.mok_fwd_state(*([1] * 9))

    def rc(cfg, n=2, src=full):
        arr = (mok.mok_layer_call * max(n, 1))()
        for i in range(max(n, 1)):
            arr[i] = mok.mok_layer_call(0, 1, src, ctypes.pointer(st), full, full)
        return L.mok_layer_fwd_macro(ctypes.byref(cfg), n, arr, 1, None, 1, ctypes.byref(w), 1, 1,
                                     None)
    ring = dict(ring_bytes=1 << 24, minibatch_rows=64)
    assert rc(_cfg()) == -1                        # no ring
    assert rc(_cfg(prec="f32", **ring)) == -1      # fp32 has no ring path
    assert rc(_cfg(**ring), n=0) == -1
    assert rc(_cfg(**ring), n=9) == -1             # more than MOK_MAX_CALLS
    assert rc(_cfg(**ring), src=bad) == -1         # a call's NULL source pointer


def test_mxfp8_backward_rejections_on_the_host(L):
    """The MXFP8 backward needs the transposed MX weights and h's scales, and
    d % 128 == 0; the weight preparation checks its pointers and shapes."""
    S = 2
    full, _k = _tab(S)

    def bwd(cfg, w, st):
        return L.mok_layer_bwd(ctypes.byref(cfg), 0, S, full, full, 1, 1, ctypes.byref(w),
                               ctypes.byref(st), full, 1, full, full, 1, 1, 1, None, 1, 1, None)

    cfg = _cfg(S=S, prec="mxfp8")
    st = mok.mok_fwd_state(*([1] * 9))
    for i in range(6, 10):  # wt_down, st_down, wt_gu, st_gu
        p = [1] * 10
        p[i] = None
        assert bwd(cfg, mok.mok_expert_weights(*p), st) == -1
    st0 = mok.mok_fwd_state(*([1] * 8), None)  # no h scales kept
    assert bwd(cfg, mok.mok_expert_weights(*([1] * 10)), st0) == -1
    assert bwd(_cfg(S=S, prec="mxfp8", d=192), mok.mok_expert_weights(*([1] * 10)), st) == -2
    assert L.mok_prepare_bwd(ctypes.byref(cfg), 1, 1, 1, 1, 1, 1, None, None) == -1
    assert L.mok_prepare_bwd(ctypes.byref(_cfg(prec="mxfp8", d=192)), 1, 1, 1, 1, 1, 1, 1,
                             None) == -2
    assert L.mok_prepare_bwd(ctypes.byref(_cfg(prec="f32")), 1, 1, 1, 1, None, 1, None,
                             None) == -1
    # bf16: the scales are unused, the transposes both required
    assert L.mok_prepare_bwd(ctypes.byref(_cfg()), 1, 1, 1, None, None, 1, None, None) == -1
