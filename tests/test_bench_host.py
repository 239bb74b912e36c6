"""Host logic of bench.py (no GPU): the one-GPU refusal, the algorithmic byte counts of the roofline, the choice
of the dominant kernel and the match between the committed profile summaries and the kernel sources."""
import json
import os
import subprocess
import sys

import pytest

import bench
from linear_rnn_layers_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
WL = bench.WORKLOADS(inputs)
MEASURED = (bench.HEADLINE,) + tuple(bench.NESTED)


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    rec = json.loads(res.stdout.strip().splitlines()[-1])
    assert rec["n_gpus"] == 2 and "one GPU" in rec["error"]


def test_byte_counts_of_the_long_workload():
    # bf16 (2 bytes), D = M = 64, 2^20 token-heads: the per-token-head figures of each tensor read or written
    w, th = WL["long"], 1 << 20
    assert (w.B * w.H * w.N, w.D, w.M) == (th, 64, 64)
    pb = bench.pass_bytes(w, 2)
    assert pb["fwd"] == 4 * 64 * 2 + 4 and pb["bwd"] == 8 * 64 * 2 + 4
    assert bench.kernel_bytes("fwd_causal", w, 2) == th * (4 * 128 + 4)    # Q, K, V read; O written; den
    assert bench.kernel_bytes("seg_state", w, 2) == th * 2 * 128           # K, V read
    assert bench.kernel_bytes("bwd_query", w, 2) == th * 5 * 128           # Q, K, V, dO read; dQ written
    assert bench.kernel_bytes("bwd_kv", w, 2) == th * 6 * 128              # Q, K, V, dO read; dK, dV written
    assert bench.dominant_bytes("long", "bwd_query", w, 2) == bench.kernel_bytes("bwd_query", w, 2)
    step, _ = bench.step_work("long", w, 2)
    assert step == th * (pb["fwd"] + pb["bwd"])


def test_byte_counts_of_wide_features():
    # the attention on C = 256 features sees C-wide vectors; the maps read X (Din wide) and write C features
    w = WL["mnist-rf256"]
    th = w.B * w.H * w.N
    assert bench.kernel_bytes("bwd_query", w, 4) == th * (3 * 256 + 2 * 32) * 4
    assert bench.kernel_bytes("feat_rf", w, 4) == th * (32 + 256) * 4


@pytest.mark.parametrize("wl", MEASURED)
def test_committed_profiles_match_the_sources(wl):
    ks = bench._profile_json(f"{wl}_kernels.json")
    assert ks is not None, f"profiles/{wl}_kernels.json is missing or was taken at other kernel sources"
    assert bench._profile_json(f"{wl}_mfma.json") is not None
    dom = bench.dominant_kernel(wl)
    assert dom in ks["kernels"]
    assert bench.traffic_from_profiles(dom, wl) is not None


@pytest.mark.parametrize("wl", MEASURED)
def test_dominant_kernel_has_the_largest_share(wl):
    ks = bench._profile_json(f"{wl}_kernels.json")
    tot = {k: v["total_us"] for k, v in ks["kernels"].items()}
    dom = bench.dominant_kernel(wl)
    assert tot[dom] == max(tot.values())
    assert bench.DOMINANT[wl] == dom  # the fallback table agrees with the committed statistics


def test_dominant_kernel_falls_back_without_matching_statistics(monkeypatch):
    monkeypatch.setattr(bench, "source_hash", lambda: "0" * 16)
    for wl in MEASURED:
        assert bench.dominant_kernel(wl) == bench.DOMINANT[wl]
        assert bench.traffic_from_profiles(bench.DOMINANT[wl], wl) is None
