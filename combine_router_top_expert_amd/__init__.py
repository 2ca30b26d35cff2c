"""Python binding of the gfx950 MoE layer library (``libmok.so``).

Argument marshalling only: every function below has the name of a C entry
point declared in ``include/mok.h``, turns torch tensors into device pointers
(PyTorch provides device memory and streams) and raises ``MokError`` on a
negative status.  Every step of the layer runs in the library's HIP kernels;
there is no fallback: importing the binding works without a GPU, but calling
into it needs the built library (``build.build()``) and a gfx950 device.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
# MOK_LIB: another build of the library to load instead (the host-sanitizer
# build that the CPU tests run the argument checks through)
LIB_PATH = os.environ.get("MOK_LIB") or os.path.join(HERE, "libmok.so")

MOK_F32, MOK_BF16, MOK_MXFP8 = 0, 1, 2
PREC = {"f32": MOK_F32, "bf16": MOK_BF16, "mxfp8": MOK_MXFP8}
MAX_SOURCES = 64

STATUS = {
    0: "MOK_OK", -1: "MOK_EINVAL", -2: "MOK_ESHAPE", -3: "MOK_EDEVICE", -4: "MOK_ECAPACITY",
    -5: "MOK_ETIMEOUT", -6: "MOK_EROUTE", -7: "MOK_ESCRATCH",
}

# every symbol include/mok.h declares
EXPORTS = ("mok_workspace_bytes", "mok_route", "mok_layout", "mok_dispatch", "mok_expert_ffn",
           "mok_combine", "mok_layer_fwd", "mok_layer_bwd", "mok_mx_quantize", "mok_tune_fwd",
           "mok_ring_layout", "mok_hbm_stream", "mok_layer_fwd_noalloc", "mok_layer_fwd_macro",
           "mok_prepare_bwd", "mok_mx_quantize_f32", "mok_mfma_probe", "mok_version")


class MokError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}")
        self.code = code


class mok_config(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int32), ("T_src", ctypes.c_int32), ("d", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E_local", ctypes.c_int32), ("prec", ctypes.c_int32), ("R_cap", ctypes.c_int32),
                ("minibatch_rows", ctypes.c_int32), ("ring_bytes", ctypes.c_int64),
                ("comm_wgs", ctypes.c_int32), ("gemm_wgs", ctypes.c_int32),
                ("wait_limit_us", ctypes.c_int32), ("trace", ctypes.c_void_p),
                ("aux", ctypes.c_void_p), ("bwd_ring_bytes", ctypes.c_int64)]


class mok_trace(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)),
                ("names", ctypes.POINTER(ctypes.c_char_p)),
                ("capacity", ctypes.c_int32), ("count", ctypes.c_int32),
                ("from_", ctypes.POINTER(ctypes.c_int32)),
                ("last_stream", ctypes.c_void_p * 2), ("last_idx", ctypes.c_int32 * 2)]


class mok_aux(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("events", ctypes.c_void_p * 3)]


def _hip_runtime():
    """The HIP runtime instance this process already uses (torch's copy when
    torch is loaded), with the event functions' signatures declared."""
    path = None
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
    except OSError:
        pass
    hip = ctypes.CDLL(path or "libamdhip64.so.7")
    P = ctypes.c_void_p
    hip.hipEventCreate.argtypes = [ctypes.POINTER(P)]
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P), ctypes.c_uint]
    hip.hipEventCreateWithFlags.restype = ctypes.c_int
    hip.hipEventSynchronize.argtypes = [P]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
    hip.hipEventDestroy.argtypes = [P]
    for fn in (hip.hipEventCreate, hip.hipEventSynchronize, hip.hipEventElapsedTime,
               hip.hipEventDestroy):
        fn.restype = ctypes.c_int
    return hip


class Trace:
    """Caller-owned kernel timing: `capacity` hipEvents (created through the HIP
    runtime) handed to the library through mok_config.trace."""

    def __init__(self, capacity: int):
        self.hip = _hip_runtime()
        self.capacity = capacity
        self.events = (ctypes.c_void_p * capacity)()
        for i in range(capacity):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            self.events[i] = ev
        self.names = (ctypes.c_char_p * capacity)()
        self.from_ = (ctypes.c_int32 * capacity)()
        self.t = mok_trace(self.events, self.names, capacity, 0, self.from_)

    def attach(self, cfg: "mok_config"):
        cfg.trace = ctypes.addressof(self.t)

    @staticmethod
    def detach(cfg: "mok_config"):
        cfg.trace = None

    def reset(self):
        self.t.count = 0
        self.t.last_stream[0] = self.t.last_stream[1] = None
        self.t.last_idx[0] = self.t.last_idx[1] = 0

    def records(self):
        """[(name, ms since the previous event on the same stream)] for every
        recorded event but the 'start' marks of each call and stream."""
        if self.t.count == 0:
            return []
        rc = self.hip.hipEventSynchronize(self.events[self.t.count - 1])
        if rc != 0:
            raise RuntimeError(f"hipEventSynchronize failed: {rc}")
        out = []
        for i in range(1, self.t.count):
            name = self.names[i].decode()
            if name == "start" or self.from_[i] < 0:
                continue
            ms = ctypes.c_float()
            rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.events[self.from_[i]],
                                              self.events[i])
            if rc != 0:
                raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
            out.append((name, float(ms.value)))
        return out

    def __del__(self):
        try:
            for i in range(self.capacity):
                self.hip.hipEventDestroy(self.events[i])
        except Exception:
            pass


class AuxStream:
    """A second stream for the backward pass (a torch stream of default
    priority) and the three events mok_aux asks for; attach() points a
    mok_config at it."""

    def __init__(self, device):
        import torch
        self.hip = _hip_runtime()
        self.stream = torch.cuda.Stream(device=device)
        evs = []
        for _ in range(3):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(ev), 2)  # hipEventDisableTiming
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
            evs.append(ev.value)
        self.a = mok_aux(self.stream.cuda_stream, (ctypes.c_void_p * 3)(*evs))

    def attach(self, cfg: "mok_config"):
        cfg.aux = ctypes.addressof(self.a)

    def __del__(self):
        try:
            for i in range(3):
                self.hip.hipEventDestroy(self.a.events[i])
        except Exception:
            pass


class mok_expert_weights(ctypes.Structure):
    _fields_ = [("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
                ("wt_down", ctypes.c_void_p), ("st_down", ctypes.c_void_p),
                ("wt_gu", ctypes.c_void_p), ("st_gu", ctypes.c_void_p)]


class mok_fwd_state(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_gate", ctypes.c_void_p),
                ("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("row_src", ctypes.c_void_p), ("dest_row", ctypes.c_void_p),
                ("h", ctypes.c_void_p), ("ab", ctypes.c_void_p), ("h_scale", ctypes.c_void_p)]


class mok_layer_call(ctypes.Structure):
    _fields_ = [("own_lo", ctypes.c_int32), ("own_n", ctypes.c_int32),
                ("src_x", ctypes.c_void_p), ("st", ctypes.POINTER(mok_fwd_state)),
                ("staging", ctypes.c_void_p), ("out", ctypes.c_void_p)]


MAX_CALLS = 8

_lib = None


def lib():
    """Load libmok.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m combine_router_top_expert_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        cfgp = ctypes.POINTER(mok_config)
        L.mok_workspace_bytes.argtypes = [cfgp]
        L.mok_workspace_bytes.restype = ctypes.c_size_t
        L.mok_route.argtypes = [cfgp, I32, P, P, P, P, P, P]
        L.mok_layout.argtypes = [cfgp, P, P, P, P, P, P, P, P, P]
        L.mok_dispatch.argtypes = [cfgp, P, P, P, P, P, P, P]
        L.mok_expert_ffn.argtypes = [cfgp, P, P, P, ctypes.POINTER(mok_expert_weights), P, P, P, P,
                                     P, P]
        L.mok_combine.argtypes = [cfgp, P, P, P, P, I32, I32, P, P, P]
        L.mok_layer_fwd.argtypes = [cfgp, I32, I32, P, P, P, P,
                                    ctypes.POINTER(mok_expert_weights),
                                    ctypes.POINTER(mok_fwd_state), P, P, P, P, P]
        L.mok_layer_bwd.argtypes = [cfgp, I32, I32, P, P, P, P, ctypes.POINTER(mok_expert_weights),
                                    ctypes.POINTER(mok_fwd_state), P, P, P, P, P, P, P, P, P, P, P]
        L.mok_mx_quantize.argtypes = [I64, I64, P, P, P, P]
        L.mok_tune_fwd.argtypes = [cfgp, P, I32, P, I32, I32, ctypes.c_size_t, I32, I32, P, P, P, P,
                                   ctypes.POINTER(mok_expert_weights),
                                   ctypes.POINTER(mok_fwd_state), P, P, P, P, P, cfgp, P]
        L.mok_ring_layout.argtypes = [cfgp, ctypes.POINTER(ctypes.c_size_t),
                                      ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(I32)]
        L.mok_hbm_stream.argtypes = [I32, P, P, I64, P]
        L.mok_mfma_probe.argtypes = [I32, I32, I64, I32, P, P]
        L.mok_layer_fwd_noalloc.argtypes = [cfgp, I32, I32, P, P, P, P,
                                            ctypes.POINTER(mok_expert_weights),
                                            ctypes.POINTER(mok_fwd_state), P, P, P, P]
        L.mok_layer_fwd_macro.argtypes = [cfgp, I32, ctypes.POINTER(mok_layer_call), P, P, P,
                                          ctypes.POINTER(mok_expert_weights), P, P, P]
        L.mok_prepare_bwd.argtypes = [cfgp, P, P, P, P, P, P, P, P]
        L.mok_mx_quantize_f32.argtypes = [I64, I64, P, P, P, P]
        L.mok_version.argtypes = []
        L.mok_version.restype = ctypes.c_char_p
        for name in EXPORTS[1:-1]:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


# ------------------------------------------------------------------ marshalling helpers
def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _table(tensors: Sequence) -> ctypes.Array:
    arr = (ctypes.c_void_p * MAX_SOURCES)()
    for i, t in enumerate(tensors):
        arr[i] = _ptr(t)
    return arr


def _check(fn: str, rc: int):
    if rc != 0:
        raise MokError(fn, rc)


def make_config(S, T_src, d, E, k, I, E_local, prec, R_cap, minibatch_rows=256, ring_bytes=0,
                comm_wgs=0, gemm_wgs=0, wait_limit_us=0, bwd_ring_bytes=0) -> mok_config:
    return mok_config(S, T_src, d, E, k, I, E_local, PREC.get(prec, prec), R_cap, minibatch_rows,
                      ring_bytes, comm_wgs, gemm_wgs, wait_limit_us, None, None, bwd_ring_bytes)


def make_weights(w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None, wt_down=None,
                 st_down=None, wt_gu=None, st_gu=None) -> mok_expert_weights:
    return mok_expert_weights(_ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up),
                              _ptr(s_down), _ptr(wt_down), _ptr(st_down), _ptr(wt_gu),
                              _ptr(st_gu))


def make_state(topk_idx, topk_gate, counts, offsets, row_src, dest_row, h, ab,
               h_scale=None) -> mok_fwd_state:
    return mok_fwd_state(_ptr(topk_idx), _ptr(topk_gate), _ptr(counts), _ptr(offsets),
                         _ptr(row_src), _ptr(dest_row), _ptr(h), _ptr(ab), _ptr(h_scale))


# ------------------------------------------------------------------ entry points
def mok_version() -> str:
    return lib().mok_version().decode()


def mok_workspace_bytes(cfg: mok_config) -> int:
    return int(lib().mok_workspace_bytes(ctypes.byref(cfg)))


def mok_route(cfg, T, x, w_router, bias, topk_idx, topk_gate, stream=None):
    _check("mok_route", lib().mok_route(ctypes.byref(cfg), T, _ptr(x), _ptr(w_router), _ptr(bias),
                                        _ptr(topk_idx), _ptr(topk_gate), _stream(stream)))


def mok_layout(cfg, topk_idx_all, expert_to_local, counts, offsets, row_src, dest_row, ws,
               dev_status, stream=None):
    _check("mok_layout", lib().mok_layout(ctypes.byref(cfg), _ptr(topk_idx_all),
                                          _ptr(expert_to_local), _ptr(counts), _ptr(offsets),
                                          _ptr(row_src), _ptr(dest_row), _ptr(ws), _ptr(dev_status),
                                          _stream(stream)))


def mok_dispatch(cfg, src_x, row_src, offsets, x_perm, x_scale, dev_status, stream=None):
    _check("mok_dispatch", lib().mok_dispatch(ctypes.byref(cfg), _table(src_x), _ptr(row_src),
                                              _ptr(offsets), _ptr(x_perm), _ptr(x_scale),
                                              _ptr(dev_status), _stream(stream)))


def mok_expert_ffn(cfg, x_perm, x_scale, offsets, weights: mok_expert_weights, h, h_scale, ab, y,
                   dev_status, stream=None):
    _check("mok_expert_ffn", lib().mok_expert_ffn(ctypes.byref(cfg), _ptr(x_perm), _ptr(x_scale),
                                                  _ptr(offsets), ctypes.byref(weights), _ptr(h),
                                                  _ptr(h_scale), _ptr(ab), _ptr(y), _ptr(dev_status),
                                                  _stream(stream)))


def mok_combine(cfg, y, dest_row, topk_gate, staging, own_lo, own_n, out, dev_status,
                stream=None):
    _check("mok_combine", lib().mok_combine(ctypes.byref(cfg), _ptr(y), _ptr(dest_row),
                                            _ptr(topk_gate), _table(staging), own_lo, own_n,
                                            _table(out) if out is not None else None,
                                            _ptr(dev_status), _stream(stream)))


def mok_layer_fwd(cfg, own_lo, own_n, src_x, w_router, bias, expert_to_local,
                  weights: mok_expert_weights, state: mok_fwd_state, staging, out, ws, dev_status,
                  stream=None):
    _check("mok_layer_fwd", lib().mok_layer_fwd(
        ctypes.byref(cfg), own_lo, own_n, _table(src_x), _ptr(w_router), _ptr(bias),
        _ptr(expert_to_local), ctypes.byref(weights), ctypes.byref(state), _table(staging),
        _table(out) if out is not None else None, _ptr(ws), _ptr(dev_status), _stream(stream)))


def mok_layer_bwd(cfg, own_lo, own_n, d_out, src_x, w_router, expert_to_local,
                  weights: mok_expert_weights, state: mok_fwd_state, staging, d_gate, dx_stage,
                  d_x, dw_gate, dw_up, dw_down, dw_router, ws, dev_status, stream=None):
    _check("mok_layer_bwd", lib().mok_layer_bwd(
        ctypes.byref(cfg), own_lo, own_n, _table(d_out), _table(src_x), _ptr(w_router),
        _ptr(expert_to_local), ctypes.byref(weights), ctypes.byref(state), _table(staging),
        _ptr(d_gate), _table(dx_stage), _table(d_x) if d_x is not None else None, _ptr(dw_gate),
        _ptr(dw_up), _ptr(dw_down), _ptr(dw_router), _ptr(ws), _ptr(dev_status), _stream(stream)))


def mok_tune_fwd(cfg, mbs, comms, reps, ws_bytes, own_lo, own_n, src_x, w_router, bias,
                 expert_to_local, weights: mok_expert_weights, state: mok_fwd_state, staging, out,
                 ws, dev_status, stream=None):
    """Returns (best mok_config, {(minibatch_rows, comm_wgs): mean ms or None if skipped})."""
    mbs = list(mbs) if mbs is not None else [64, 128, 256, 512, 1024, 2048, 4096]
    if comms is None:
        import torch
        cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
        comms = [max(cus * q // 16, 1) for q in (1, 2, 3, 4)]
    comms = list(comms)
    mb_arr = (ctypes.c_int32 * len(mbs))(*mbs)
    cm_arr = (ctypes.c_int32 * len(comms))(*comms)
    times = (ctypes.c_float * (len(mbs) * len(comms)))()
    best = mok_config()
    _check("mok_tune_fwd", lib().mok_tune_fwd(
        ctypes.byref(cfg), ctypes.cast(mb_arr, ctypes.c_void_p), len(mbs),
        ctypes.cast(cm_arr, ctypes.c_void_p), len(comms), reps, ws_bytes, own_lo, own_n,
        _table(src_x), _ptr(w_router), _ptr(bias), _ptr(expert_to_local), ctypes.byref(weights),
        ctypes.byref(state), _table(staging), _table(out) if out is not None else None, _ptr(ws),
        _ptr(dev_status), _stream(stream), ctypes.byref(best), ctypes.cast(times, ctypes.c_void_p)))
    table = {}
    for i, mb in enumerate(mbs):
        for j, c in enumerate(comms):
            v = times[i * len(comms) + j]
            table[(mb, c)] = float(v) if v >= 0 else None
    return best, table


def mok_mx_quantize(rows, K, src, codes, scales, stream=None):
    _check("mok_mx_quantize", lib().mok_mx_quantize(rows, K, _ptr(src), _ptr(codes), _ptr(scales),
                                                    _stream(stream)))


def mok_mx_quantize_f32(rows, K, src, codes, scales, stream=None):
    _check("mok_mx_quantize_f32", lib().mok_mx_quantize_f32(rows, K, _ptr(src), _ptr(codes),
                                                            _ptr(scales), _stream(stream)))


def mok_prepare_bwd(cfg, w_gate, w_up, w_down, wt_down, st_down, wt_gu, st_gu, stream=None):
    _check("mok_prepare_bwd", lib().mok_prepare_bwd(
        ctypes.byref(cfg), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(wt_down), _ptr(st_down),
        _ptr(wt_gu), _ptr(st_gu), _stream(stream)))


def mok_ring_layout(cfg):
    """-> (offset, slot_bytes, nslot) of the fused path's ring inside the workspace."""
    off, sb, n = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int32()
    _check("mok_ring_layout", lib().mok_ring_layout(ctypes.byref(cfg), ctypes.byref(off),
                                                    ctypes.byref(sb), ctypes.byref(n)))
    return int(off.value), int(sb.value), int(n.value)


def mok_hbm_stream(mode, dst, src, nbytes, stream=None):
    """HBM streaming probe: mode 0 read src, 1 write dst, 2 copy src -> dst."""
    _check("mok_hbm_stream", lib().mok_hbm_stream(mode, _ptr(dst), _ptr(src), nbytes,
                                                  _stream(stream)))


def mok_mfma_probe(kind, constant, iters, workgroups, out, stream=None):
    """Matrix-core rate probe: kind 0 bf16, 1 E4M3; constant 0 hashed data, 1 ones."""
    _check("mok_mfma_probe", lib().mok_mfma_probe(kind, constant, iters, workgroups, _ptr(out),
                                                  _stream(stream)))


def mok_layer_fwd_noalloc(cfg, own_lo, own_n, src_x, w_router, bias, expert_to_local,
                          weights: mok_expert_weights, state: mok_fwd_state, staging, out,
                          dev_status, stream=None):
    _check("mok_layer_fwd_noalloc", lib().mok_layer_fwd_noalloc(
        ctypes.byref(cfg), own_lo, own_n, _table(src_x), _ptr(w_router), _ptr(bias),
        _ptr(expert_to_local), ctypes.byref(weights), ctypes.byref(state), _table(staging),
        _table(out) if out is not None else None, _ptr(dev_status), _stream(stream)))


def mok_layer_fwd_macro(cfg, calls, w_router, bias, expert_to_local, weights: mok_expert_weights,
                        ws, dev_status, stream=None):
    """calls: list of dicts with own_lo, own_n, src_x, state (mok_fwd_state),
    staging, out -- one per layer call (macrobatch)."""
    keep = []
    arr = (mok_layer_call * len(calls))()
    for i, c in enumerate(calls):
        src, stg = _table(c["src_x"]), _table(c["staging"])
        out = _table(c["out"]) if c["out"] is not None else None
        keep += [src, stg, out, c["state"]]
        arr[i] = mok_layer_call(c["own_lo"], c["own_n"], ctypes.cast(src, ctypes.c_void_p),
                                ctypes.pointer(c["state"]), ctypes.cast(stg, ctypes.c_void_p),
                                ctypes.cast(out, ctypes.c_void_p) if out is not None else None)
    _check("mok_layer_fwd_macro", lib().mok_layer_fwd_macro(
        ctypes.byref(cfg), len(calls), arr, _ptr(w_router), _ptr(bias), _ptr(expert_to_local),
        ctypes.byref(weights), _ptr(ws), _ptr(dev_status), _stream(stream)))
