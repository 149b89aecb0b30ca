"""Host-side checks of bench.py on the CPU: the one-GPU refusal, the
algorithmic work behind the roofline figure, the counter records it reads and
its CPU-baseline leg. No GPU call is made."""
import json
import os
import subprocess
import sys

import pytest

import bench
from dsa_top_token_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "8"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       env=dict(os.environ, **env), capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_decode_indexer_work_is_one_pass_over_the_keys():
    # 64 sequences whose queries sit at position 131071: every key's 128
    # fp8 bytes are read once, plus the 64 query rows
    w = synth.WORKLOADS["decode_128k_clustered"]
    bound, amount, unit, peak = bench.stage_work(w, "indexer")
    assert (bound, unit, peak) == ("hbm", "GB/s", 8000.0)
    assert round(amount * 1e9) == 64 * 131072 * 128 + 64 * 128


def test_prefill_indexer_work_counts_the_causal_pairs():
    # L queries at positions 0 .. L-1 score L (L + 1) / 2 pairs, 2 d flops each
    for name, peak in (("prefill_64k", 5000.0), ("prefill_128k", 2500.0)):
        w = synth.WORKLOADS[name]
        L = w.n_q
        bound, amount, unit, pk = bench.stage_work(w, "indexer")
        assert (bound, unit, pk) == ("mfma", "TFLOP/s", peak)
        assert amount * 1e12 == pytest.approx(2 * w.d_idx * L * (L + 1) / 2, rel=1e-12)


def test_attention_work_is_the_selected_rows():
    # each query gathers min(top_k, pos + 1) K and V rows of 256 bytes, and
    # reads Q and writes O (16 heads x 128 bf16 each)
    w = synth.WORKLOADS["decode_128k_clustered"]
    _, amount, _, _ = bench.stage_work(w, "attn")
    assert round(amount * 1e9) == 64 * 2048 * 512 + 2 * 64 * 16 * 128 * 2
    tiny = synth.Workload("tiny", "prefill", 1, 40, 40, 0, 64, "fp8", 8, 4)
    # positions 0..39: 1 + 2 + ... + 8 rows for the first eight, then 8 each
    assert tiny.n_selected() == 36 + 32 * 8


def test_counter_records_are_keyed_to_the_current_sources():
    # a record whose kernel sources changed since the counters were taken is
    # not used (the bench line then reports traffic null); the default
    # workload's record must be current
    recs = json.load(open(bench.TRAFFIC_FILE))
    rec = recs["decode_128k_clustered/indexer"]
    assert rec["source_sha256_16"] == bench.source_hash("decode", "indexer")
    for key, rec in recs.items():
        assert rec["bytes_per_step"] > 0 and rec["algorithmic_bytes_per_step"] > 0
        assert rec["fetch_scale"] == pytest.approx(2.0, rel=1e-3)


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_cpu_baseline_leg(mode):
    if mode == "decode":
        w = synth.Workload("tiny_decode", "decode", 4, 1, 2048, 2047, 64, "fp8", 128, 4)
    else:
        w = synth.Workload("tiny_prefill", "prefill", 1, 256, 256, 0, 64, "bf16", 32, 4)
    x = synth.make_inputs(w, 0, "cpu")
    r = bench.cpu_baseline(w, x, target_s=0.3)
    assert r["kind"] == "oracle" and r["unit"] == "queries/s"
    assert r["value"] > 0 and r["cores"] >= 1 and r["seconds"] > 0
    if mode == "decode":
        assert r["sample"].startswith("4 of 4 sequences")
    else:
        assert "of the prefill's 256" in r["sample"] and "strided sweep" in r["sample"]
