"""Summaries of rocprofv3 output for the layer's kernels.

``python -m combine_router_top_expert_amd.profiling OUT_DIR WORKLOAD PATH [BENCH ARGS...]``
reads, from OUT_DIR (the folder the rocprofv3 runs below wrote to; BENCH ARGS
are the bench.py arguments they were run with, e.g. ``--workload C3
--ring-mib 256 --mb 1024 --comm-wgs 16``):
  kt/kt_kernel_stats.csv                  rocprofv3 --kernel-trace --stats of bench.py
  pf/pf_counter_collection.csv            rocprofv3 --pmc FETCH_SIZE of bench.py
  pw/pw_counter_collection.csv            rocprofv3 --pmc WRITE_SIZE of bench.py
  cf/cf_counter_collection.csv            rocprofv3 --pmc FETCH_SIZE of bench.py --hbm-copy-gib 1
  cw/cw_counter_collection.csv            rocprofv3 --pmc WRITE_SIZE of bench.py --hbm-copy-gib 1
and writes ``profiles/<workload>_<path>_kernel_trace.md``,
``profiles/<workload>_<path>_hbm_traffic.md`` and that workload and path's
record in ``profiles/hbm_traffic.json``.

The byte counters are scaled by what they read for the plain 1 GiB device copy
(``FETCH_SIZE`` and ``WRITE_SIZE`` are in KiB; the factor maps the copy's
reading onto its known 1 GiB).  ``hbm_traffic.json`` records the traffic of one
launch of each kernel (its last profiled launch) under the name ``bench.py``
reports, together with a hash of each kernel's sources (the .hip file that
defines it, every header under csrc/ and include/): ``bench.py`` reports a
kernel's traffic only while its sources still hash to that value.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
PROFILES = os.path.join(ROOT, "profiles")

# HIP kernel (as named in the profiler) -> the name bench.py's trace uses
TRACE_NAME = {
    "route_kernel": "route", "layout_count": "layout_count", "layout_scan": "layout_scan",
    "layout_place": "layout_place", "gather_kernel": "gather", "gather_mx_kernel": "gather",
    "ffn1_g2": "ffn1_gate_up_swiglu", "ffn2_g2": "ffn2_down", "ffn1_mx": "ffn1_gate_up_swiglu_mx",
    "ffn2_mx": "ffn2_down_mx", "combine_kernel": "combine", "rc_pull_kernel": "bwd_reverse_combine_pull",
    "dh_g2": "bwd_dh", "swiglu_bwd_kernel": "bwd_swiglu", "dx_g2": "bwd_dx_push",
    "wgrad_g2<0>": "bwd_wgrad_gate_up", "wgrad_g2<1>": "bwd_wgrad_down",
    "wgrad_reduce<0>": "bwd_wgrad_gate_up_reduce", "wgrad_reduce<1>": "bwd_wgrad_down_reduce",
    "dx_final_kernel": "bwd_dx_sum_router", "dwr_part_kernel": "bwd_dw_router_part",
    "dwr_reduce_kernel": "bwd_dw_router_reduce", "ring_kernel": "ring_fused_ffn",
    "gather_t_kernel": "bwd_transpose_x_h", "rc_pull_rows_kernel": "bwd_reverse_combine_pull",
    "mx_pack_kernel<0>": "bwd_pack_dy_mx", "mx_pack_kernel<1>": "bwd_swiglu_pack_mx",
    "mx_pack_kernel<2>": "bwd_pack_h_x_mx", "mx_pack_kernel<3>": "bwd_pack_h_x_mx",
    "wgrad_mx_kernel<0>": "bwd_wgrad_gate_up_mx",
    "wgrad_mx_kernel<1>": "bwd_wgrad_down_mx", "mx_quantize_kernel": "mx_quantize",
}


def source_hash() -> str:
    """sha256 over the kernel sources (csrc/*.hip, csrc/*.h, include/*.h)."""
    h = hashlib.sha256()
    files = []
    for d, exts in ((CSRC, (".hip", ".h")), (os.path.join(ROOT, "include"), (".h",))):
        files += sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(exts))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def kernel_source_hash(key: str):
    """sha256 over the .hip file that defines kernel ``key`` (a name as
    kernel_key returns it, template arguments dropped) and every header, or
    None if no source defines it."""
    base = key.split("<")[0]
    pat = re.compile(r"__global__[^;{]*\b%s\s*\(" % re.escape(base))
    hip = [f for f in sorted(os.listdir(CSRC)) if f.endswith(".hip")
           and pat.search(open(os.path.join(CSRC, f)).read())]
    if len(hip) != 1:
        return None
    h = hashlib.sha256()
    files = [os.path.join(CSRC, hip[0])]
    files += sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h"))
    inc = os.path.join(ROOT, "include")
    files += sorted(os.path.join(inc, f) for f in os.listdir(inc) if f.endswith(".h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def kernel_key(name: str) -> str:
    m = re.search(r"mok::\(anonymous namespace\)::(\w+)", name)
    if not m:
        m = re.search(r"^(?:void\s+)?([\w:]+)", name)
        return m.group(1) if m else name
    key = m.group(1)
    if key in ("wgrad_g2", "wgrad_reduce", "wgrad_mx_kernel", "mx_pack_kernel"):
        # the MODE / KIND argument: the first integer argument after the
        # optional tile configuration
        t = re.search(r"%s<(?:[\w:]*Cfg<[^>]*>,\s*)?(\d)" % key, name)
        key += "<%s>" % (t.group(1) if t else "?")
    return key


def counters(path: str):
    """kernel key -> list of counter values (one per dispatch, in order)."""
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            out.setdefault(kernel_key(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return out


def copy_factor(path: str, expect_kib: float) -> float:
    vals = counters(path).get("__amd_rocclr_copyBuffer")
    if not vals:
        raise SystemExit(f"{path}: no copy kernel dispatches")
    return expect_kib / (sum(vals) / len(vals))


WHAT = {
    "C2": ("mid-size layer (forward + backward)",
           "T=16384 tokens (8 x 2048), d=2048, E=64 all local, top-6, SwiGLU I=1408, bf16"),
    "C3": ("one GPU's share of the 256-expert layer (forward through the ring + backward)",
           "T=131072 tokens (32 x 4096), d=7168, E=256 with 8 local, top-8, SwiGLU I=2048, "
           "bf16, Zipf 1.2 skew"),
    "C4": ("mid-size layer in MXFP8 (forward; backward in MXFP8 beside it)",
           "T=16384 tokens (8 x 2048), d=2048, E=64 all local, top-6, SwiGLU I=1408, MXFP8"),
    "C5": ("mid-size layer with skewed routing (forward + backward)",
           "T=16384 tokens (8 x 2048), d=2048, E=64 all local, top-6, SwiGLU I=1408, bf16, "
           "Zipf 1.2 skew"),
}


def main(out_dir: str, workload: str = "C2", path: str = "staged", *bench_args: str):
    # the traffic record is written only from counter passes of this
    # folder (run post-processing before any source changes: the record
    # takes the kernels' current source hashes)
    args = " ".join(bench_args) if bench_args else f"--workload {workload}"
    if os.path.exists(os.path.join(out_dir, "pf", "pf_counter_collection.csv")):
        traffic_main(out_dir, workload, path, args)
    trace_main(out_dir, workload, path, args)


def _stem(workload: str, path: str) -> str:
    return f"{workload.lower()}_{path}"


def traffic_main(out_dir: str, workload: str, path: str, args: str):
    fs = copy_factor(os.path.join(out_dir, "cf", "cf_counter_collection.csv"), 1 << 20)
    ws = copy_factor(os.path.join(out_dir, "cw", "cw_counter_collection.csv"), 1 << 20)
    fetch = counters(os.path.join(out_dir, "pf", "pf_counter_collection.csv"))
    write = counters(os.path.join(out_dir, "pw", "pw_counter_collection.csv"))
    traffic = {}
    title, shape = WHAT.get(workload, (workload, ""))
    lines = [f"# HBM traffic per launch, {title}", "", shape + ".", "",
             "Byte counters from two rocprofv3 passes over one timed step of `bench.py`",
             "(`FETCH_SIZE`, then `WRITE_SIZE`, in KiB per dispatch), each scaled by what the",
             f"same counter reads for a plain 1 GiB device copy: FETCH_SIZE x {fs:.3f},",
             f"WRITE_SIZE x {ws:.3f}.  Values are for the last profiled launch of each kernel.", "",
             "Commands (from the repository root; OUT = the output folder):", "",
             f"    rocprofv3 --pmc FETCH_SIZE -f csv -d OUT/pf -o pf -- python3 bench.py {args} --steps 1 --warmup 1 --no-cpu-baseline",
             f"    rocprofv3 --pmc WRITE_SIZE -f csv -d OUT/pw -o pw -- python3 bench.py {args} --steps 1 --warmup 1 --no-cpu-baseline",
             "    rocprofv3 --pmc FETCH_SIZE -f csv -d OUT/cf -o cf -- python3 bench.py --hbm-copy-gib 1 --steps 3 --warmup 1",
             "    rocprofv3 --pmc WRITE_SIZE -f csv -d OUT/cw -o cw -- python3 bench.py --hbm-copy-gib 1 --steps 3 --warmup 1",
             f"    python3 -m combine_router_top_expert_amd.profiling OUT {workload} {path} {args}", "",
             "| kernel | trace name | read MB | written MB | total MB |", "|---|---|---|---|---|"]
    for k, fv in fetch.items():
        name = TRACE_NAME.get(k)
        if name is None:
            continue
        rb = fv[-1] * 1024 * fs
        wb = write.get(k, [0.0])[-1] * 1024 * ws
        traffic[name] = {"read_bytes": rb, "write_bytes": wb, "bytes": rb + wb,
                         "source_sha256": kernel_source_hash(k)}
        lines.append(f"| {k} | {name} | {rb / 1e6:.1f} | {wb / 1e6:.1f} | {(rb + wb) / 1e6:.1f} |")
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, _stem(workload, path) + "_hbm_traffic.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    jf = os.path.join(PROFILES, "hbm_traffic.json")
    rec = {}
    if os.path.exists(jf):
        with open(jf) as fh:
            rec = json.load(fh)
        if "records" not in rec:
            rec = {}
    rec.setdefault("records", {})[f"{workload}/{path}"] = {
        "source_sha256": source_hash(), "bench_args": args, "fetch_factor": fs,
        "write_factor": ws, "kernels": traffic}
    with open(jf, "w") as f:
        json.dump(rec, f, indent=1)


def trace_main(out_dir: str, workload: str, path: str, args: str):
    stats = os.path.join(out_dir, "kt", "kt_kernel_stats.csv")
    if os.path.exists(stats):
        rows = list(csv.DictReader(open(stats)))
        title, shape = WHAT.get(workload, (workload, ""))
        t = [f"# Kernel trace summary, {title}", "",
             "Command (from the repository root):", "",
             f"    rocprofv3 --kernel-trace --stats -f csv -d OUT/kt -o kt -- python3 bench.py {args} --steps 3 --warmup 2 --no-cpu-baseline",
             "", "Seven or more steps (2 warm-up, 3 timed, 2 for the run-to-run identity check, whose",
             "byte comparisons and host copies are the torch kernels below) of: " + shape + ".", "",
             "| kernel | trace name | calls | average us | share % |", "|---|---|---|---|---|"]
        for r in rows:
            k = kernel_key(r["Name"])
            t.append(f"| {k} | {TRACE_NAME.get(k, '')} | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
        with open(os.path.join(PROFILES, _stem(workload, path) + "_kernel_trace.md"), "w") as f:
            f.write("\n".join(t) + "\n")
    print("written under", PROFILES)


def last_counters(path: str):
    """kernel key -> {counter: value of its last profiled dispatch}."""
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            out.setdefault(kernel_key(r["Kernel_Name"]), {})[r["Counter_Name"]] = \
                float(r["Counter_Value"])
    return out


def mfma_main(out_dir: str):
    """MFMA utilisation of the GEMMs from three rocprofv3 passes:
    mfma/c2 (MfmaUtil, SQ_INSTS_VALU_MFMA_MOPS_BF16), mfma/c2l
    (SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE) and mfma/c4 (MfmaUtil,
    SQ_INSTS_VALU_MFMA_MOPS_F8) -> profiles/mfma_util.md.  Executed flops are
    the MOPS counter x 512; the algorithmic flops are those bench.py uses."""
    sys.path.insert(0, ROOT)
    from bench import kernel_work  # noqa: E402  (the work model of the bench line)
    from combine_router_top_expert_amd import synth  # noqa: E402
    c2 = last_counters(os.path.join(out_dir, "c2", "c2_counter_collection.csv"))
    c2l = last_counters(os.path.join(out_dir, "c2l", "c2l_counter_collection.csv"))
    c4 = last_counters(os.path.join(out_dir, "c4", "c4_counter_collection.csv"))
    R = 98304
    lines = ["# MFMA utilisation of the expert GEMMs (mid-size layer, bf16 and MXFP8)", "",
             "rocprofv3 counters of one profiled step (forward + backward in bf16; forward in",
             "MXFP8).  `MfmaUtil` is rocprofv3's derived metric: MFMA busy cycles summed over",
             "the SIMDs / (active cycles x SIMDs).  Executed flops are the MFMA op counter x 512,",
             "against the algorithmic flops of the launch (R = 98304 routed rows); the excess is",
             "the work on padding (rows past an expert's last tile, columns past I).  LDS bank",
             "conflicts are the share of LDS-active cycles spent in conflicts.", "",
             "Commands (from the repository root; OUT = the output folder):", "",
             "    rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 -f csv -d OUT/c2 -o c2 -- python3 bench.py --workload C2 --steps 1 --warmup 1 --no-cpu-baseline",
             "    rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE -f csv -d OUT/c2l -o c2l -- python3 bench.py --workload C2 --steps 1 --warmup 1 --no-cpu-baseline",
             "    rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_INSTS_VALU_MFMA_MOPS_F6F4 -f csv -d OUT/c4 -o c4 -- python3 bench.py --workload C4 --path staged --steps 1 --warmup 1 --no-cpu-baseline",
             "    python3 -m combine_router_top_expert_amd.profiling --mfma OUT", "",
             "| kernel | trace name | MfmaUtil % | executed TFLOP | algorithmic TFLOP | padding % | LDS bank-conflict % |",
             "|---|---|---|---|---|---|---|"]
    w2 = synth.WORKLOADS["C2"]
    w4 = synth.WORKLOADS["C4"]
    for table, mops, w in ((c2, "SQ_INSTS_VALU_MFMA_MOPS_BF16", w2), (c4, "SQ_INSTS_VALU_MFMA_MOPS_F8", w4)):
        for k, v in table.items():
            name = TRACE_NAME.get(k)
            if name is None or v.get("MfmaUtil", 0.0) == 0.0:
                continue
            kind, work = kernel_work(name, w, R)
            ex = v.get(mops, 0.0) * 512
            lds = c2l.get(k, {}) if w is w2 else {}
            act = lds.get("SQ_LDS_IDX_ACTIVE", 0.0)
            conf = 100.0 * lds["SQ_LDS_BANK_CONFLICT"] / act if act else None
            lines.append(f"| {k} | {name} | {v['MfmaUtil']:.1f} | {ex / 1e12:.3f} | "
                         f"{(work or 0) / 1e12:.3f} | {100.0 * (ex / work - 1) if work else 0:.1f} | "
                         + (f"{conf:.1f}" if conf is not None else "-") + " |")
    with open(os.path.join(PROFILES, "mfma_util.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("written", os.path.join(PROFILES, "mfma_util.md"))


def recorded_traffic(kernel: str, workload: str, path: str):
    """HBM bytes of one launch of ``kernel`` as profiled, or None when the
    record is missing, was taken on another workload or path, or the kernel
    sources have changed since."""
    f = os.path.join(PROFILES, "hbm_traffic.json")
    if not os.path.exists(f):
        return None
    with open(f) as fh:
        rec = json.load(fh).get("records", {}).get(f"{workload}/{path}")
    if rec is None:
        return None
    k = rec["kernels"].get(kernel)
    if k is None:
        return None
    keys = [key for key, n in TRACE_NAME.items() if n == kernel]
    now = {kernel_source_hash(key) for key in keys} - {None}
    if k.get("source_sha256") is None or k["source_sha256"] not in now:
        return None
    return k["bytes"]


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--mfma":
        mfma_main(sys.argv[2])
    else:
        main(*sys.argv[1:])
