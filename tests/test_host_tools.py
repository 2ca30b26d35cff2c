"""Host-side logic of the measurement tools (no GPU): every kernel the
profiles name is defined in exactly one source file (its traffic record is
hashed against that file), the traffic record is well-formed, and bench.py
has a work model for every GEMM and streaming kernel the library traces."""
import json
import os
import re

from combine_router_top_expert_amd import profiling
from combine_router_top_expert_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_profiled_kernel_has_one_source():
    for key in profiling.TRACE_NAME:
        h = profiling.kernel_source_hash(key)
        assert h is not None and re.fullmatch(r"[0-9a-f]{64}", h), key


def test_traffic_record_well_formed():
    recs = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))["records"]
    assert recs
    names = set(profiling.TRACE_NAME.values())
    for key, rec in recs.items():
        workload, path = key.split("/")
        assert workload in synth.WORKLOADS and path in ("staged", "ring")
        assert rec["fetch_factor"] > 0 and rec["write_factor"] > 0
        for name, k in rec["kernels"].items():
            assert name in names, name
            assert k["bytes"] == k["read_bytes"] + k["write_bytes"] >= 0
            assert k["source_sha256"] is None or re.fullmatch(r"[0-9a-f]{64}", k["source_sha256"])


def test_bench_work_model_covers_the_traced_kernels():
    import bench
    traced = set()
    for f in os.listdir(os.path.join(ROOT, "combine_router_top_expert_amd", "csrc")):
        src = open(os.path.join(ROOT, "combine_router_top_expert_amd", "csrc", f)).read()
        for call in re.findall(r'trace_mark\(([^;]*)\);', src):
            traced |= set(re.findall(r'"(\w+)"', call))
        # (the MX row GEMM launcher takes its trace name as its last argument)
        traced |= set(re.findall(r'launch_mx_rows_gemm\([^;]*?"(\w+)"\);', src))
    traced.discard("start")
    w = synth.WORKLOADS["C2"]
    modeled = {n for n in traced if bench.kernel_work(n, w, 98304)[0] is not None}
    # the expert GEMMs and the HBM-bound copies must be priced against a roofline
    for n in ("ffn1_gate_up_swiglu", "ffn2_down", "bwd_dh", "bwd_dx_push", "bwd_wgrad_gate_up",
              "bwd_wgrad_down", "combine", "bwd_reverse_combine_pull", "bwd_swiglu",
              "bwd_regather_x", "bwd_transpose_x_h", "bwd_dx_sum_router", "route", "bwd_dh_mx", "bwd_dx_push_mx",
              "bwd_wgrad_gate_up_mx", "bwd_wgrad_down_mx", "bwd_pack_dy_mx",
              "bwd_swiglu_pack_mx", "bwd_pack_h_x_mx"):
        assert n in traced and n in modeled, n
