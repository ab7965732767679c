"""The benchmark's CPU leg (the oracle timed on the host) runs and reports the
agreed fields, on shrunk copies of each kind of workload (no GPU needed)."""
import os

import numpy as np
import pytest

import bench
from kv_cache_vector_randomized_amd import synth


@pytest.mark.parametrize("mode", ["gqa_decode", "qjl", "polar3", "prefill_append", "dequant_layer", "gqa_d256",
                                  "gqa_group8"])
def test_cpu_baseline_reports_the_contract_fields(mode):
    wname, kind = bench.MODES[mode]
    base = bench.generic_workloads(synth).get(wname) or synth.WORKLOADS[wname]
    w = synth.shrink(base, batch=2, context=48)
    lay = synth.paged_layout(w.batch, [w.context] * w.batch, w.seed)
    k = synth.kv_tensor(w, w.batch * w.context, "k")
    v = synth.kv_tensor(w, w.batch * w.context, "v")
    q = synth.query_tensor(w)
    rec = bench.cpu_baseline(w, kind, k, v, q, lay, np)
    assert set(rec) == {"value", "unit", "cores", "kind", "sample"}
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s" and rec["value"] > 0 and rec["cores"] >= 1
    assert isinstance(rec["sample"], str) and rec["sample"]


def test_more_than_one_gpu_is_refused():
    """bench.py runs on one GPU: --gpus N > 1 exits with a message before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
