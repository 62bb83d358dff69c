"""The workload registry (swa_inputs.WORKLOADS) holds the five measured
workloads exactly as they are specified: shapes, sinks and window, dtype,
value scale, the sink construction, chunking, RoPE base, decode steps and
the checked-row stride."""
import numpy as np

import swa_inputs as si

# id: (kind, dtype, B, Hq, Hkv, d, L, s, r, value scale, sink factor, rope base, chunk, steps, check stride)
SPEC = {
    1: ("prefill", "f32", 1, 1, 1, 64, 256, 4, 28, 1.0, 0.0, 0.0, 0, 0, 1),
    2: ("prefill", "bf16", 1, 32, 8, 128, 8192, 0, 4096, float(np.float32(1 / np.sqrt(2))), 0.0, 0.0, 0, 0, 1),
    3: ("prefill", "bf16", 4, 32, 32, 128, 16384, 4, 1020, 1.0, 3.0, 0.0, 0, 0, 1),
    4: ("decode", "bf16", 64, 32, 8, 128, 8192, 4, 4092, 1.0, 0.0, 0.0, 0, 1024, 1),
    5: ("chunked", "bf16", 1, 32, 32, 128, 131072, 4, 4092, 1.0, 0.0, 10000.0, 4096, 0, 64),
}


def test_registry_matches_the_specified_workloads():
    assert sorted(si.WORKLOADS) == [1, 2, 3, 4, 5]
    for wid, spec in SPEC.items():
        w = si.WORKLOADS[wid]
        got = (w.kind, w.dtype, w.B, w.Hq, w.Hkv, w.d, w.L, w.s, w.r, w.value_scale, w.sink_from_mean_q,
               w.rope_base, w.chunk, w.steps, w.check_every)
        assert got == spec, (wid, got)
        assert w.wid == wid and w.scale == 1 / np.sqrt(w.d)


def test_derived_budgets():
    """Window plus sinks is the key budget of each workload (32 for the fp32
    case, 1024 for the StreamingLLM split, 4096 otherwise); the chunked
    workload is 32 chunks; GQA groups of 4 where the heads differ."""
    budgets = {wid: w.s + w.r for wid, w in si.WORKLOADS.items()}
    assert budgets == {1: 32, 2: 4096, 3: 1024, 4: 4096, 5: 4096}
    assert si.WORKLOADS[5].L // si.WORKLOADS[5].chunk == 32
    assert {wid: w.Hq // w.Hkv for wid, w in si.WORKLOADS.items()} == {1: 1, 2: 4, 3: 1, 4: 4, 5: 1}
