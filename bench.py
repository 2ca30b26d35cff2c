"""Benchmark of the MoE layer hot path on one MI355X.

One step = the whole layer over one batch of synthetic input resident in HBM:
route -> layout -> gather -> SwiGLU grouped GEMMs -> push + final weighted
combine, then (where the workload has a backward pass) reverse-combine pull
-> dgrad GEMMs with the SwiGLU derivative -> wgrad GEMMs -> reverse-dispatch
push + router backward.

Workloads (--workload; default: all four, one JSON line each, the headline
last):
  C2  the mid-size layer: T = 16384 tokens in 8 source buffers of 2048,
      d = 2048, E = 64 experts all local, top-6, SwiGLU I = 1408, bf16 with
      fp32 accumulation, balanced routing; forward + backward;
  C4  the same layer in MXFP8, forward only (the MXFP8 layer has no backward);
  C5  the mid-size layer with Zipf 1.2 skew, forward + backward;
  C3  one GPU's share of a 256-expert layer (own 4096 tokens of 32 source
      buffers, 8 local experts, d = 7168, I = 2048, top-8, Zipf 1.2 skew),
      forward + backward -- the largest configuration that one GPU holds, and
      the headline (printed last).

Each JSON line: layer tokens/s, the forward-only rate, per-kernel average
times (HIP events recorded by the library between its kernels on the
layer's streams, during the timed steps), the roofline of the dominant
kernel, and the CPU oracle's rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/sec fwd & fwd+bwd on 1 MI355X; % MFMA peak, % HBM peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 / MXFP8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# fp32 fmaf on the vector ALU: 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz.
# (The 157.3 TFLOP/s headline counts packed two-wide fp32, which this library
# does not use.)
PEAK_FP32_FMA_TFLOPS = 78.6


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_work(name, w, R, T_pull=None):
    """Algorithmic work of one launch: ('mfma', flops), ('alu', flops) or ('hbm', bytes).
    R: routed rows computed here; T_pull: tokens with at least one of them
    (the tokens whose upstream gradient the reverse-combine pull reads)."""
    d, I, k = w.d, w.I, w.k
    if T_pull is None:
        T_pull = R
    T = len(w.own) * w.T_src  # tokens combined / summed here (own sources)
    eb = 2 if w.prec != "f32" else 4
    gemm = {
        "ffn1_gate_up_swiglu": 2.0 * R * d * 2 * I,
        "ffn2_down": 2.0 * R * I * d,
        "ffn1_gate_up_swiglu_mx": 2.0 * R * d * 2 * I,
        "ffn2_down_mx": 2.0 * R * I * d,
        # persistent ring kernel: pull into ring slots + GEMM1/SwiGLU + GEMM2 + push
        "ring_fused_ffn": 2.0 * R * d * 2 * I + 2.0 * R * I * d,
        "bwd_dh": 2.0 * R * d * I,
        "bwd_dh_swiglu": 2.0 * R * d * I,
        "bwd_dx_push": 2.0 * R * 2 * I * d,
        "bwd_wgrad_gate_up": 2.0 * R * 2 * I * d,
        "bwd_wgrad_down": 2.0 * R * d * I,
        "bwd_dh_mx": 2.0 * R * d * I,
        "bwd_dx_push_mx": 2.0 * R * 2 * I * d,
        "bwd_wgrad_gate_up_mx": 2.0 * R * 2 * I * d,
        "bwd_wgrad_down_mx": 2.0 * R * d * I,
    }
    if name in gemm:
        fp8 = name.endswith("_mx") or (name == "ring_fused_ffn" and w.prec == "mxfp8")
        return ("mfma_fp8" if fp8 else "mfma"), gemm[name]
    moves = {
        # read each pulled token's row once (its other routed rows hit the
        # caches), write every slot row (MX: d E4M3 codes + d/32 scales)
        "gather": T_pull * d * 2.0 + (R * d * (1 + 1 / 32) if w.prec == "mxfp8" else R * d * eb),
        "bwd_regather_x": (T_pull + R) * d * eb,
        # the token rows (each pulled token read once) and h, written
        # transposed per expert
        "bwd_transpose_x_h": ((T_pull + R) * d + 2.0 * R * I) * eb,
        "combine": (T * k * d + T * d) * eb,              # read k pushed rows, write out
        # read each pulled token's dout once and every row's pushed y, write dy
        "bwd_reverse_combine_pull": (T_pull + 2.0 * R) * d * eb,
        "bwd_swiglu": 5.0 * R * I * eb,                   # read dh, a, b; write da, db
        "bwd_dx_sum_router": (T * k * d + T * d) * eb,    # read k dx rows, write dX
        # MX packs (E4M3 codes + one scale byte per 32 = 33/32 bytes a value):
        # dy read once, quantised along d and along the rows
        "bwd_pack_dy_mx": R * d * (2 + 2 * 33 / 32),
        # dh, a, b read; da | db quantised along 2I and along the rows
        "bwd_swiglu_pack_mx": R * I * (3 * 2 + 2 * 2 * 33 / 32),
        # h's codes read and re-quantised along the rows; token rows likewise
        "bwd_pack_h_x_mx": R * I * 2 * 33 / 32 + R * d * (2 + 33 / 32),
    }
    if name in moves:
        return "hbm", moves[name]
    if name == "route":  # fp32 fmaf chains over d for every (own token, expert)
        return "alu", 2.0 * T * w.E * d
    return None, None


def cpu_baseline(w, host, n_tok):
    """Time the CPU oracle (single thread) on n_tok tokens of the workload:
    routing, forward, and -- where the workload has one -- backward with the
    tokens' share of the weight gradients."""
    import numpy as np

    import oracle
    own = w.own
    has_bwd = host["dout_val"] is not None
    toks = [(own[i % len(own)], (i * 7919) % w.T_src) for i in range(n_tok)]
    tok_x = np.stack([host["x_val"][s][t] for s, t in toks])
    e2l = w.expert_to_local()
    t0 = time.perf_counter()
    idx, g = oracle.route(tok_x, host["wr_val"], host["bias"], w.k, w.prec)
    # (MXFP8: the FFN rows take the weights as given; their cost does not
    # depend on whether the values were rounded to MX first)
    oracle.fwd_tokens(tok_x, idx, g, e2l, host["wg_val"], host["wu_val"], host["wd_val"], w.prec)
    if has_bwd:
        tok_d = np.stack([host["dout_val"][s][t] for s, t in toks])
        _, dz, _ = oracle.bwd_tokens(tok_x, tok_d, idx, g, e2l, host["wr_val"], host["wg_val"],
                                     host["wu_val"], host["wd_val"])
        for le in range(w.E_local):
            sel = [(i, j) for i in range(n_tok) for j in range(w.k) if e2l[idx[i, j]] == le]
            if sel:
                ii = [i for i, _ in sel]
                oracle.expert_wgrad(tok_x[ii], np.array([g[i, j] for i, j in sel]), tok_d[ii],
                                    host["wg_val"][le], host["wu_val"][le], host["wd_val"][le])
        oracle.router_wgrad(tok_x, idx, dz, w.E)
    dt = time.perf_counter() - t0
    what = ("forward + backward (routing, FFN rows, combine, backward rows, their "
            "weight-gradient rows, router gradient)" if has_bwd else
            "forward (routing, MX FFN rows, combine)")
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_tok} tokens of the workload, {what}; {dt:.1f} s single-threaded "
                      f"float64 C"}


def measure(args, w, L, d_out, has_bwd, mb, np, torch, Trace):
    """Warm up, time args.steps steps of the layer, and build the JSON record."""
    def step():
        L.forward()
        if has_bwd:
            L.backward(d_out)

    # warm-up: args.warmup steps, continued until 0.5 s have passed, so that
    # the clocks have left the idle state the host-side input generation left
    # them in (untimed)
    t_w = time.perf_counter()
    i = 0
    while i < args.warmup or time.perf_counter() - t_w < 0.5:
        step()
        if i % 4 == 3:
            torch.cuda.synchronize()
        i += 1
    torch.cuda.synchronize()
    L.check_status()
    R = int(L.offsets[-1].item())
    T_pull = int(torch.unique(L.row_src[:R].long() // w.k).numel()) if R > 0 else 0

    # (through the backward ring, every window adds its kernels' events)
    trace = Trace(capacity=512 * (args.steps + 1))
    trace.attach(L.cfg)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    Trace.detach(L.cfg)
    L.check_status()
    ms_per_step = (t_end - t_start) * 1e3 / args.steps
    T_tok = w.T_total if len(w.own) == w.S else len(w.own) * w.T_src

    recs = trace.records()
    per_kernel = {}
    for name, ms in recs:
        per_kernel.setdefault(name, []).append(ms)
    fwd_names = {"route", "layout_count", "layout_scan", "layout_place", "gather",
                 "ffn1_gate_up_swiglu", "ffn2_down", "ffn1_gate_up_swiglu_mx", "ffn2_down_mx",
                 "ring_init", "ring_fused_ffn", "combine"}
    fwd_ms = sum(sum(v) for n, v in per_kernel.items() if n in fwd_names) / args.steps
    # the backward's side work runs on a second stream beside its GEMMs, so
    # its time is the step's wall time less the forward's kernels
    bwd_ms = ms_per_step - fwd_ms
    kernels = {n: {"avg_ms": float(np.mean(v)), "launches_per_step": len(v) // args.steps,
                   "ms_per_step": float(np.sum(v)) / args.steps}
               for n, v in per_kernel.items()}
    # dominant kernel: largest time per step among kernels with a work model
    modeled = [n for n in per_kernel if kernel_work(n, w, R, T_pull)[0] is not None]
    dom = max(modeled, key=lambda n: sum(per_kernel[n]))
    kind, work = kernel_work(dom, w, R, T_pull)
    # the work of a step over the kernel's time in the step: per launch for a
    # kernel launched once per step (through the backward ring, several
    # windows each launch the kernel over their rows)
    avg_s = float(np.sum(per_kernel[dom])) / args.steps * 1e-3
    if kind == "alu":
        achieved = work / avg_s / 1e12
        roof = {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_FMA_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_FP32_FMA_TFLOPS, "traffic": None, "kernel": dom,
                "algorithmic_flops_per_launch": work}
    elif kind in ("mfma", "mfma_fp8"):
        achieved = work / avg_s / 1e12
        peak = PEAK_FP8_TFLOPS if kind == "mfma_fp8" else PEAK_BF16_TFLOPS
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": None, "kernel": dom,
                "algorithmic_flops_per_launch": work}
    else:
        achieved = work / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": None, "kernel": dom,
                "algorithmic_bytes_per_launch": work}
    from combine_router_top_expert_amd.profiling import recorded_traffic
    roof["traffic"] = recorded_traffic(dom, w.name, "ring" if args.ring_mib else "staged")
    # per-kernel roofline fractions, for the record
    for n, v in kernels.items():
        kd, wk = kernel_work(n, w, R, T_pull)
        t_s = v["ms_per_step"] * 1e-3
        if kd in ("mfma", "mfma_fp8"):
            v["tflops"] = wk / t_s / 1e12
            v["frac_mfma_peak"] = v["tflops"] / (PEAK_FP8_TFLOPS if kd == "mfma_fp8"
                                                 else PEAK_BF16_TFLOPS)
        elif kd == "hbm":
            v["gbs"] = wk / t_s / 1e9
            v["frac_hbm_peak"] = v["gbs"] / PEAK_HBM_GBS
        elif kd == "alu":
            v["tflops"] = wk / t_s / 1e12
            v["frac_alu_peak"] = v["tflops"] / PEAK_FP32_FMA_TFLOPS

    # run-to-run identity at full size: every output of two consecutive
    # untimed steps compared byte for byte on the device; the digest covers
    # the combined outputs (and input gradients) of the own tokens
    def outputs():
        outs = [L.out[s] for s in w.own] + list(L.staging) + [L.h]
        if has_bwd:
            outs += [L.d_x[s] for s in w.own] + [L.d_gate, L.dw_gate, L.dw_up, L.dw_down,
                                                 L.dw_router] + list(L.dx_stage)
        return outs

    step()
    torch.cuda.synchronize()
    L.check_status()
    first = [t.clone() for t in outputs()]
    step()
    torch.cuda.synchronize()
    L.check_status()
    identical = all(torch.equal(a.view(torch.uint8), b.view(torch.uint8))
                    for a, b in zip(first, outputs()))
    import hashlib
    h = hashlib.sha256()
    for t in [L.out[s] for s in w.own] + ([L.d_x[s] for s in w.own] if has_bwd else []):
        h.update(t.contiguous().view(torch.uint8).cpu().numpy().tobytes())
    del first
    torch.cuda.empty_cache()

    graph = None
    if args.graph:
        # the whole step captured once and replayed: no host launch cost
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(max(args.warmup, 1)):
            g.replay()
        torch.cuda.synchronize()
        L.check_status()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        g_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        L.check_status()
        graph = {"ms_per_step": g_ms, "tokens_per_s": T_tok / (g_ms * 1e-3)}
        del g

    result = {
        "metric": METRIC,
        "value": T_tok / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.prec == "bf16" else w.prec,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: T={T_tok} tokens ({w.S} sources x {w.T_src}), d={w.d}, "
                               f"E={w.E} ({w.E_local} local), top-{w.k}, SwiGLU I={w.I}, {w.prec}, "
                               f"{'Zipf %.1f skew' % w.zipf_s if w.zipf_s else 'balanced routing'}; "
                               f"step = {'forward + backward' if has_bwd else 'forward'}",
                   "routed_rows": R,
                   "pulled_tokens": T_pull,
                   "backward_streams": 2 if (has_bwd and L.aux is not None) else 1,
                   "path": ("ring %d MiB, minibatch %d rows, comm/gemm workgroups %s/%s"
                            % (args.ring_mib, mb, args.comm_wgs or "auto",
                               args.gemm_wgs or "auto")) if args.ring_mib else "staged",
                   "backward_path": (("ring %d MiB in windows of whole %d-row minibatches"
                                      % (args.bwd_ring_mib, mb)) if args.bwd_ring_mib
                                     else "one launch per step") if has_bwd else None},
        "fwd_tokens_per_s": T_tok / (fwd_ms * 1e-3),
        "fwd_ms": fwd_ms,
        "bwd_ms": bwd_ms if has_bwd else None,
        "roofline": roof,
        "kernels": kernels,
    }
    if graph is not None:
        result["graph"] = graph
    result["determinism"] = {"two_steps_identical": identical,
                             "own_outputs_sha256": h.hexdigest()}
    return result


def hbm_copy_line(args, torch):
    """A plain device-to-device copy of args.hbm_copy_gib GiB (the runtime's
    copy kernel), args.steps times: the reference of known size that scales
    the profiler's byte counters."""
    n = int(args.hbm_copy_gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(max(args.warmup, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"metric": "device copy (bytes read + written per second)",
                      "value": 8 * n / dt / 1e9, "unit": "GB/s", "bytes_per_copy": 4 * n,
                      "steps": args.steps}), flush=True)


def hbm_stream_lines(args, torch):
    """The HBM streaming probe (16-byte loads and stores over a grid-stride
    loop, the access of the layer's data-movement kernels): read-only,
    write-only and copy rates, one JSON line each."""
    from combine_router_top_expert_amd import mok_hbm_stream
    n = int(args.hbm_stream_gib * (1 << 30)) // 256 * 256
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for mode, name, moved in ((0, "read", n), (1, "write", n), (2, "copy", 2 * n)):
        # warm-up: at least args.warmup calls and 0.5 s of streaming, so that
        # the clocks have left their idle state
        t_w = time.perf_counter()
        i = 0
        while i < args.warmup or time.perf_counter() - t_w < 0.5:
            mok_hbm_stream(mode, dst, src, n)
            if i % 8 == 7:
                torch.cuda.synchronize()
            i += 1
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            mok_hbm_stream(mode, dst, src, n)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"metric": f"HBM streaming probe, {name} (bytes moved per second)",
                          "value": moved / dt / 1e9, "unit": "GB/s", "bytes_per_call": moved,
                          "ms_per_call": dt * 1e3, "frac_hbm_peak": moved / dt / 1e9 / PEAK_HBM_GBS,
                          "steps": args.steps}), flush=True)


def mfma_probe_lines(args, torch):
    """The matrix-core rate probe (MFMAs on register operands, one wave per
    SIMD, no memory traffic) for bf16 and E4M3, on hashed and on constant
    operands: one JSON line each, with the fraction of the published peak."""
    from combine_router_top_expert_amd import mok_mfma_probe
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 256, dtype=torch.float32, device="cuda:0")
    iters = 4000
    for kind, name, flops, peak in ((0, "bf16 32x32x16", 32768.0, PEAK_BF16_TFLOPS),
                                    (1, "E4M3 scaled 32x32x64", 131072.0, PEAK_FP8_TFLOPS)):
        for constant, data in ((0, "hashed"), (1, "ones")):
            for _ in range(max(args.warmup, 1)):
                mok_mfma_probe(kind, constant, iters, cus, out)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                mok_mfma_probe(kind, constant, iters, cus, out)
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) / args.steps
            tf = cus * 4 * iters * 16 * flops / dt / 1e12
            exact = None
            if constant:
                exact = bool(torch.all(out == 256.0 * (16 if kind == 0 else 64) * iters).item())
            print(json.dumps({"metric": f"matrix-core rate probe, {name}, {data} operands",
                              "value": tf, "unit": "TFLOP/s", "frac_peak": tf / peak,
                              "ms_per_call": dt * 1e3, "workgroups": cus, "steps": args.steps,
                              "sums_exact": exact}), flush=True)


def run_workload(args, name, np, torch):
    """Inputs, layer, timed steps and the CPU baseline of one workload -> records."""
    from combine_router_top_expert_amd import Trace, synth
    from combine_router_top_expert_amd.layer import MoELayer, to_device

    dev = "cuda:0"
    w = synth.WORKLOADS[name]
    has_bwd = w.prec != "mxfp8"
    t0 = time.time()
    xs = [synth.gen_x(w, s) for s in range(w.S)]
    wr = synth.gen_router(w)
    bias = synth.load_bias(w)
    wg = synth.gen_expert_weights(w, "gate")
    wu = synth.gen_expert_weights(w, "up")
    wd = synth.gen_expert_weights(w, "down")
    dout = [synth.gen_dout(w, s) for s in range(w.S)] if has_bwd else None
    other = {s: synth.gen_other_routing(w, s) for s in range(w.S) if s not in w.own}
    log(f"{name}: inputs generated in {time.time() - t0:.1f} s")
    N = w.S * w.T_src * w.k
    # row capacity: every item when all experts are local, else twice the
    # balanced share (a layer latches MOK_ECAPACITY if routing exceeds it)
    R_cap = N if w.E_local == w.E else min(N, 2 * N * w.E_local // w.E)
    dev_in = dict(xs=[to_device(a, w.prec, dev) for a, _ in xs], wr=to_device(wr[0], w.prec, dev),
                  bias=None if bias is None else torch.from_numpy(bias).to(dev),
                  e2l=torch.from_numpy(w.expert_to_local()).to(dev),
                  wg=to_device(wg[0], w.prec, dev), wu=to_device(wu[0], w.prec, dev),
                  wd=to_device(wd[0], w.prec, dev))
    d_out = [to_device(a, w.prec, dev) for a, _ in dout] if has_bwd else None

    def make_layer(mb):
        L = MoELayer(w.S, w.T_src, w.d, w.E, w.k, w.I, w.E_local, w.prec, R_cap, w.own[0],
                     len(w.own), device=dev, with_bwd=has_bwd, ring_bytes=args.ring_mib << 20,
                     minibatch_rows=mb, comm_wgs=args.comm_wgs, gemm_wgs=args.gemm_wgs,
                     bwd_ring_bytes=(args.bwd_ring_mib << 20) if has_bwd else 0,
                     two_streams=args.bwd_streams == 2)
        L.set_inputs(dev_in["xs"], dev_in["wr"], dev_in["bias"], dev_in["e2l"], dev_in["wg"],
                     dev_in["wu"], dev_in["wd"], other_topk=other)
        return L

    # the share of the 256-expert layer runs its forward through the 256 MiB
    # ring of token slots its configuration names, with the minibatch size and
    # dispatch split the tuner picks (untimed); the others run staged
    if args.path == "auto" and name == "C3" and not args.ring_mib and not args.mb_sweep:
        args = argparse.Namespace(**{**vars(args), "ring_mib": 256, "tune": True})
    elif args.path == "staged":
        args = argparse.Namespace(**{**vars(args), "ring_mib": 0, "tune": False})
    mbs = [int(v) for v in args.mb_sweep.split(",")] if args.mb_sweep else [args.mb]
    results = []
    for mb in mbs:
        L = make_layer(mb)
        tuned = None
        comm = args.comm_wgs
        if args.tune:
            table = L.tune(reps=10)
            log("tuner (minibatch rows, dispatch workgroups) -> ms per forward:",
                {f"{m}/{c}": (round(v, 3) if v is not None else None) for (m, c), v in table.items()})
            mb, comm = L.cfg.minibatch_rows, L.cfg.comm_wgs
            tuned = {f"{m}/{c}": v for (m, c), v in table.items()}
        a = argparse.Namespace(**{**vars(args), "comm_wgs": comm})
        results.append(measure(a, w, L, d_out, has_bwd, mb, np, torch, Trace))
        if tuned is not None:
            results[-1]["config"]["tuner_ms_per_forward"] = tuned
        del L
        torch.cuda.empty_cache()
    # the skewed mid-size layer's configuration names a 256 MiB ring for its
    # backward: the same step with the backward through that ring (windows of
    # whole minibatches) is measured beside the one-launch backward
    if (args.path == "auto" and name == "C5" and not args.bwd_ring_mib and not args.mb_sweep
            and not args.ring_mib):
        a = argparse.Namespace(**{**vars(args), "bwd_ring_mib": 256})
        L = MoELayer(w.S, w.T_src, w.d, w.E, w.k, w.I, w.E_local, w.prec, R_cap, w.own[0],
                     len(w.own), device=dev, with_bwd=True, minibatch_rows=args.mb,
                     bwd_ring_bytes=256 << 20)
        L.set_inputs(dev_in["xs"], dev_in["wr"], dev_in["bias"], dev_in["e2l"], dev_in["wg"],
                     dev_in["wu"], dev_in["wd"], other_topk=other)
        rr = measure(a, w, L, d_out, True, args.mb, np, torch, Trace)
        results[-1]["ring_backward"] = {
            "ms_per_step": rr["ms_per_step"], "tokens_per_s": rr["value"],
            "bwd_ms": rr["bwd_ms"], "backward_path": rr["config"]["backward_path"],
            "determinism": rr["determinism"],
            "kernels": {n: v for n, v in rr["kernels"].items() if n.startswith("bwd")}}
        del L
        torch.cuda.empty_cache()
    # the MXFP8 layer: its backward in MXFP8, measured beside the forward line
    if args.path == "auto" and name == "C4" and not args.mb_sweep and not args.ring_mib:
        dmx = [to_device(synth.gen_dout(w, s)[0], w.prec, dev) for s in range(w.S)]
        L = MoELayer(w.S, w.T_src, w.d, w.E, w.k, w.I, w.E_local, w.prec, R_cap, w.own[0],
                     len(w.own), device=dev, with_bwd=True, minibatch_rows=args.mb)
        L.set_inputs(dev_in["xs"], dev_in["wr"], dev_in["bias"], dev_in["e2l"], dev_in["wg"],
                     dev_in["wu"], dev_in["wd"], other_topk=other)
        rr = measure(args, w, L, dmx, True, args.mb, np, torch, Trace)
        results[-1]["mxfp8_backward"] = {
            "ms_per_step": rr["ms_per_step"], "tokens_per_s": rr["value"],
            "bwd_ms": rr["bwd_ms"], "roofline": rr["roofline"],
            "determinism": rr["determinism"],
            "kernels": {n: v for n, v in rr["kernels"].items() if n.startswith("bwd")}}
        del L, dmx
        torch.cuda.empty_cache()
    for r in results:
        r["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        host = {"x_val": [b for _, b in xs], "dout_val": [b for _, b in dout] if has_bwd else None,
                "wr_val": wr[1], "bias": bias, "wg_val": wg[1], "wu_val": wu[1], "wd_val": wd[1]}
        base = cpu_baseline(w, host, args.cpu_tokens or CPU_TOKENS.get(name, 20))
        for r in results:
            r["cpu_baseline"] = base
    del dev_in, d_out
    torch.cuda.empty_cache()
    return results


def run_macro(args, name, np, torch):
    """Macrobatch pipelining: args.macro layer calls of the workload's
    forward through one ring launch (mok_layer_fwd_macro) against the same
    calls one mok_layer_fwd (ring) after the other.  The calls take the same
    inputs, each with its own state, staging rows and outputs."""
    from combine_router_top_expert_amd import mok_layer_fwd_macro, synth
    from combine_router_top_expert_amd.layer import MoELayer, to_device

    dev = "cuda:0"
    w = synth.WORKLOADS[name]
    xs = [synth.gen_x(w, s) for s in range(w.S)]
    wr = synth.gen_router(w)
    bias = synth.load_bias(w)
    wts = [synth.gen_expert_weights(w, p_) for p_ in ("gate", "up", "down")]
    other = {s: synth.gen_other_routing(w, s) for s in range(w.S) if s not in w.own}
    N = w.S * w.T_src * w.k
    R_cap = N if w.E_local == w.E else min(N, 2 * N * w.E_local // w.E)
    xs_d = [to_device(a, w.prec, dev) for a, _ in xs]
    wr_d = to_device(wr[0], w.prec, dev)
    bias_d = None if bias is None else torch.from_numpy(bias).to(dev)
    e2l = torch.from_numpy(w.expert_to_local()).to(dev)
    wts_d = [to_device(a[0], w.prec, dev) for a in wts]
    ring = (args.ring_mib or 256) << 20
    Ls = []
    for _ in range(args.macro):
        L = MoELayer(w.S, w.T_src, w.d, w.E, w.k, w.I, w.E_local, w.prec, R_cap, w.own[0],
                     len(w.own), device=dev, with_bwd=False, ring_bytes=ring,
                     minibatch_rows=args.mb, comm_wgs=args.comm_wgs, gemm_wgs=args.gemm_wgs)
        L.set_inputs(xs_d, wr_d, bias_d, e2l, *wts_d, other_topk=other)
        Ls.append(L)
    L0 = Ls[0]
    calls = [dict(own_lo=L.own_lo, own_n=L.own_n, src_x=L.xs, state=L.state, staging=L.staging,
                  out=L.out) for L in Ls]

    def macro():
        mok_layer_fwd_macro(L0.cfg, calls, L0.w_router, L0.bias, L0.e2l, L0.weights, L0.ws,
                            L0.status)

    def separate():
        for L in Ls:
            L.forward()

    res = {}
    for label, fn in (("separate", separate), ("macro", macro)):
        t_w = time.perf_counter()
        i = 0
        while i < args.warmup or time.perf_counter() - t_w < 0.5:
            fn()
            torch.cuda.synchronize()
            i += 1
        for L in Ls:
            L.check_status()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        res[label] = (time.perf_counter() - t0) * 1e3 / args.steps
    for L in Ls:
        L.check_status()
    T_tok = len(w.own) * w.T_src * args.macro
    print(json.dumps({
        "metric": "MoE layer forward tokens/sec, macrobatch pipelining on 1 MI355X",
        "value": T_tok / (res["macro"] * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["macro"],
        "higher_is_better": True, "dtype": "bf16" if w.prec == "bf16" else w.prec,
        "data": "synthetic",
        "config": {"workload": f"{name}: {args.macro} layer calls of {len(w.own) * w.T_src} own "
                               f"tokens (the same inputs), forward",
                   "path": f"ring {ring >> 20} MiB, minibatch {args.mb} rows, comm/gemm "
                           f"workgroups {args.comm_wgs or 'auto'}/{args.gemm_wgs or 'auto'}"},
        "separate_calls_ms": res["separate"],
        "separate_tokens_per_s": T_tok / (res["separate"] * 1e-3),
        "speedup": res["separate"] / res["macro"]}), flush=True)


# the CPU oracle's sample per workload: about 10 s of single-threaded work
CPU_TOKENS = {"C1": 512, "C2": 36, "C3": 160, "C4": 600, "C5": 36}

# the default run: every configuration one GPU holds, the largest (the
# headline) last
DEFAULT_ORDER = ["C2", "C4", "C5", "C3"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all",
                    help="C1..C5, or 'all' (C2, C4, C5, then C3, one JSON line each)")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of the CPU oracle's sample (0: per workload, about 10 s of "
                         "single-threaded work)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ring-mib", type=int, default=0,
                    help="forward through the persistent ring kernel with a ring of this many "
                         "MiB (0 = one launch per step)")
    ap.add_argument("--mb", type=int, default=256, help="ring path: rows per minibatch")
    ap.add_argument("--bwd-streams", type=int, choices=[1, 2], default=2,
                    help="bf16 backward: side work on a second stream (2) or all on one (1)")
    ap.add_argument("--bwd-ring-mib", type=int, default=0,
                    help="backward through a ring of this many MiB (windows of whole "
                         "minibatches; 0 = one launch per step over all rows)")
    ap.add_argument("--comm-wgs", type=int, default=0, help="ring path: dispatch workgroups")
    ap.add_argument("--gemm-wgs", type=int, default=0, help="ring path: GEMM workgroups")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one step in a HIP graph and time its replays "
                         "(reported under 'graph'; the headline stays the eager step)")
    ap.add_argument("--tune", action="store_true",
                    help="ring path: choose minibatch rows and dispatch workgroups with "
                         "mok_tune_fwd before the timed steps (untimed)")
    ap.add_argument("--mb-sweep", default="",
                    help="ring path: comma-separated minibatch sizes, one JSON line each")
    ap.add_argument("--path", choices=["auto", "staged"], default="auto",
                    help="auto: the 256-expert share (C3) through its 256 MiB ring with the "
                         "tuned minibatch and split, the others staged; staged: all staged "
                         "(--ring-mib sets the ring for every workload)")
    ap.add_argument("--macro", type=int, default=0,
                    help="instead of the step: this many forward calls through one ring launch "
                         "(mok_layer_fwd_macro) against the same calls one after the other")
    ap.add_argument("--hbm-copy-gib", type=float, default=0.0,
                    help="only a plain device copy of this many GiB (profiler byte-counter "
                         "reference)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="instead of the layer: the matrix-core rate probe (bf16 and E4M3, "
                         "hashed and constant operands)")
    ap.add_argument("--hbm-stream-gib", type=float, default=0.0,
                    help="instead of the layer: the HBM streaming probe (read, write, copy) "
                         "over this many GiB")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one MI355X: the library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    if args.mfma_probe:
        mfma_probe_lines(args, torch)
        return
    if args.hbm_stream_gib > 0:
        hbm_stream_lines(args, torch)
        return
    if args.hbm_copy_gib > 0:
        hbm_copy_line(args, torch)
        return
    if args.tune and (not args.ring_mib or args.mb_sweep):
        sys.exit("--tune needs --ring-mib and no --mb-sweep")
    names = DEFAULT_ORDER if args.workload == "all" else [args.workload]
    if args.macro > 0:
        for name in names:
            run_macro(args, name, np, torch)
        return
    for name in names:
        for r in run_workload(args, name, np, torch):
            print(json.dumps(r), flush=True)


if __name__ == "__main__":
    main()
