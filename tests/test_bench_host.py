"""Host logic of bench.py (no GPU): the multi-GPU refusal, the dtype label, and the
lookup of committed traffic counters, which must match both the workload and the
kernel source they were taken on."""
import importlib.util
import json
import os
import subprocess
import sys

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(spec)
spec.loader.exec_module(bench)

IDX_SRC = ["long_context_attention_19_amd/csrc/index_score.hip"]
ATT_SRC = ["long_context_attention_19_amd/csrc/attention.hip"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU only" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_dtype_names_every_format():
    assert bench._dtype(workloads.get("hybrid_decode_1m")) == "bf16+int8"
    assert bench._dtype(workloads.get("hybrid_decode_1m_fp4")) == "bf16+fp4"
    assert bench._dtype(workloads.get("hybrid_decode_1m_kv8")) == "bf16+fp8+int8"
    assert bench._dtype(workloads.get("hca_decode_128k")) == "bf16"


def test_traffic_record_needs_its_workload_and_source():
    recs = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for tag, rec in recs.items():
        wl = rec["workload"].split(" ")[0]
        workloads.get(wl)   # every record names a workload that exists
        src = ATT_SRC if tag == "csa_sparse_attn" else IDX_SRC
        got = bench.traffic_from_profile(tag, src, wl)
        if rec["source_sha256"] == bench._src_hash(src):
            assert got == rec["bytes_per_launch"]
            want = round(rec["fetch_kib_raw"] * rec["fetch_scale"] * 1024
                         + rec["write_kib_raw"] * rec["write_scale"] * 1024)
            assert abs(got - want) <= 1024
        else:
            assert got is None
        # a record never stands in for another workload of the same kernel
        assert bench.traffic_from_profile(tag, src, "csa_decode_8k") is None
    assert bench.traffic_from_profile("no_such_kernel", IDX_SRC, "hybrid_decode_1m") is None
