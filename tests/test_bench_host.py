"""bench.py's host-side accounting, on the CPU: the FLOP and byte counts the
roofline and the JSON line are computed from, the per-call summary, the
sustained-clock record, and the lookup of counter-derived traffic, which must
refuse a figure taken from other kernel sources."""
import json
import os

import numpy as np
import pytest

import bench
import moe_inputs

W = {w.name: w for w in moe_inputs.WORKLOADS}
STEP = W["step_T32768_D768_F1536_E8_top2_shared_zipf"]
SMALL = W["smallchunk_T512_D768_F1536_E8_top2"]


def test_stage_flops_add_up_to_the_layer():
    counts = np.array([22947, 13239, 8606, 6192, 4743, 3892, 3165, 2752])
    work = bench.stage_work(STEP, counts)
    rows = STEP.T * STEP.k + STEP.T
    assert work["up_swiglu"]["flop"] == 4 * STEP.D * STEP.F * rows
    assert work["down"]["flop"] == 2 * STEP.D * STEP.F * rows
    assert work["up_swiglu"]["flop"] + work["down"]["flop"] == STEP.flops()
    # the routed W1/W3 products alone: about 309 GFLOP per layer and step at 32,768
    # tokens and top-2 ("Triton MoE Kernels & Memory Checkpointing", Part A, section 2)
    routed_up = 4 * STEP.D * STEP.F * STEP.T * STEP.k
    assert abs(routed_up / 1e9 - 309.2) < 0.1


def test_stage_bytes_count_each_operand_once():
    counts = np.array([64] * 8)
    w = SMALL
    b = 2
    work = bench.stage_work(w, counts)
    rows = w.T * w.k
    weights = w.D * w.F * b
    assert work["up_swiglu"]["bytes"] == w.T * w.D * b + 2 * weights * 8 + rows * w.F * b
    assert work["down"]["bytes"] == rows * w.F * b + weights * 8 + rows * w.D * b
    # an expert without rows reads no weights
    counts0 = counts.copy()
    counts0[3] = 0
    assert bench.stage_work(w, counts0)["down"]["bytes"] == work["down"]["bytes"] - weights
    # the whole path: x and y, routing, three matrices per active expert
    assert bench.path_bytes(w, counts) == 2 * w.T * w.D * b + w.T * w.k * 8 + 3 * weights * 8
    assert abs(bench.path_bytes(w, counts) / 1e6 - 58.2) < 0.1


def test_percentiles():
    p = bench.percentiles([1.0, 2.0, 3.0, 4.0, 100.0])
    assert p["median"] == 3.0 and p["mean"] == 22.0
    assert p["p10"] == pytest.approx(1.4) and p["p90"] == pytest.approx(61.6)


def test_sustained_record():
    assert bench.sustained_record({"sustained": None}, STEP) is None
    m = {"sustained": {"ms_per_step": 0.75, "calls_before": 200, "clocks": {(0, 0): 1.8, (1, 0): 1.9}}}
    r = bench.sustained_record(m, STEP)
    assert r["tflops"] == pytest.approx(STEP.flops() / 0.75e-3 / 1e12, rel=1e-6)
    assert r["pct_of_bf16_peak"] == pytest.approx(100 * r["tflops"] / bench.PEAK_BF16_TFLOPS, abs=0.01)
    assert r["sclk_ghz_median"] == pytest.approx(1.85)
    assert r["calls_before"] == 200


def test_traffic_lookup_refuses_stale_figures(tmp_path, monkeypatch):
    key = "unfused:up_swiglu"
    good = bench.source_hash("up_swiglu", "unfused", False)
    rec = {STEP.name: {key: {"bytes_per_launch": 123, "source_sha": good}},
           "other": {key: {"bytes_per_launch": 456, "source_sha": "0" * 16}}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    # the hash of the real sources, computed above; ROOT now points at the temp record
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash",
                        lambda st, var="unfused", small=False: good if st == "up_swiglu" else "x")
    assert bench.load_traffic(STEP.name, key) == 123
    assert bench.load_traffic("other", key) is None
    assert bench.load_traffic(STEP.name, "unfused:down") is None
    assert bench.load_traffic("absent", key) is None


def test_source_hash_covers_the_kernels_headers():
    # the small-chunk up GEMM is built with the permute's device code (its sort workgroup)
    import hashlib
    h = hashlib.sha256()
    for rel in ("gemm_bf16_slab.hip", "permute_device.h", "mfma_common.h", "moe_internal.h"):
        with open(os.path.join(bench.ROOT, "grouped_gemm_permute_amd", "csrc", rel), "rb") as f:
            h.update(f.read())
    assert bench.source_hash("up_swiglu", "unfused", True) == h.hexdigest()[:16]
    assert bench.source_hash("up_swiglu", "unfused", False) != bench.source_hash("up_swiglu", "unfused", True)


def test_back_to_back_record():
    assert bench.back_to_back_record({"sustained": None}, 58_204_160) is None
    m = {"sustained": {"ms_per_step": 0.0291, "calls_before": 5000, "clocks": {}}}
    r = bench.back_to_back_record(m, 58_204_160)
    assert r["ms_per_call"] == 0.0291 and r["calls_before"] == 5000
    assert r["gbs"] == pytest.approx(58_204_160 / 29.1e-6 / 1e9, abs=0.05)
    assert r["frac_of_8tbs"] == pytest.approx(r["gbs"] / 8000.0, abs=1e-4)
