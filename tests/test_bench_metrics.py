"""The benchmark's efficiency metrics (eqs. (7)-(10) of the DiffusionGemma
Technical Report, part 3, section 3.4), computed in bench.py's own code,
against the oracle's metrics and the pages' closed forms.  CPU only."""
import json
import os

import numpy as np
import pytest

import bench
from oracle import dg_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_generation_metrics_match_the_oracle_on_random_generations():
    rng = np.random.default_rng(4)
    for _ in range(50):
        K = int(rng.integers(1, 6))
        N = rng.integers(1, 49, size=K).tolist()
        Cv = rng.integers(0, 257, size=K).tolist()
        if sum(Cv) == 0:
            Cv[0] = 1
        got = bench.generation_metrics(N, Cv)
        ref = O.metrics(N, Cv)
        assert got["total_tokens"] == ref["total_tokens"]
        assert got["total_denoising_steps"] == ref["total_steps"]
        assert got["effective_denoising_steps"] == pytest.approx(ref["effective_steps"], rel=1e-15)
        assert got["tokens_per_forward"] == pytest.approx(ref["tpf"], rel=1e-15)


def test_generation_metrics_closed_forms():
    # no adaptive stop: EDS = N; the long-context generation (4 canvases of
    # 48 steps, 3 appends) has TPF 1024 / 195
    m = bench.generation_metrics([48] * 4, [256] * 4)
    assert m["effective_denoising_steps"] == 48
    assert m["tokens_per_forward"] == pytest.approx(1024 / 195)
    assert m["total_tokens"] == 1024 and m["total_denoising_steps"] == 192
    # one canvas: TPF = C_k / N_k; a canvas cut at its EOS keeps C_k tokens
    m = bench.generation_metrics([12], [256])
    assert m["tokens_per_forward"] == pytest.approx(256 / 12)
    # EDS weights step counts by the tokens each canvas kept
    m = bench.generation_metrics([10, 40], [200, 50])
    assert m["effective_denoising_steps"] == pytest.approx((10 * 200 + 40 * 50) / 250)


def test_pages_numbers_through_the_bench_metrics():
    """The pages' canvas figures through the bench's metric code: 256 tokens
    in about 12 forwards give about 20 tokens per forward; the SFT sampler's
    full 48-step budget gives about 5."""
    pages = json.load(open(os.path.join(GOLDEN, "pages_numbers.json")))
    cv = pages["canvas"]
    m = bench.generation_metrics([cv["forwards_per_canvas"]], [cv["canvas_tokens"]])
    assert m["tokens_per_forward"] == pytest.approx(cv["approx_tpf"], rel=0.1)
    m = bench.generation_metrics([pages["adaptive_stop"]["budget_N"]], [cv["canvas_tokens"]])
    assert m["tokens_per_forward"] == pytest.approx(pages["sft_tpf"]["approx_tpf"], rel=0.1)
    assert m["effective_denoising_steps"] == pages["adaptive_stop"]["budget_N"]


def test_kernel_work_counts():
    from block_discrete_diffusion_amd import synth
    wl = synth.workload("single_canvas")
    w = bench.kernel_work(wl, [1024.0], 125.33, 256)
    by, fl, bound = w["lmhead_sampler"]
    assert bound == "hbm" and fl == pytest.approx(2 * 125.33 * 2048 * 32768)
    assert by == pytest.approx(32768 * 2048 * 2 + 125.33 * (2048 * 2 + 8) + 256 * 125.33 * 16, abs=1)
    by, fl, bound = w["attention"]
    assert bound == "mfma" and fl == pytest.approx(4 * 256 * 1280 * 128 * 16)
    by, fl, _ = w["qkv_rope"]
    assert fl == pytest.approx(2 * 256 * 2048 * 3072)


def test_bench_refuses_more_than_one_gpu(capsys):
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_committed_traffic_files_match_the_current_sources():
    """The committed counter files (LM head, bf16 and e4m3; attention at
    long context) were taken on the current kernel sources, so the bench
    line carries their bytes as roofline.traffic."""
    from block_discrete_diffusion_amd import synth
    cases = [(synth.workload("single_canvas"), "lmhead_sampler"),
             (synth.workload("single_canvas").with_(lm_fp8=True), "lmhead_sampler"),
             (synth.workload("long_context"), "attention")]
    for wl, kind in cases:
        b = bench.measured_traffic(wl, kind)
        assert b is not None, (wl.name, wl.lm_fp8, kind)
        with open(bench.traffic_file(bench.traffic_key(wl.name, wl.lm_fp8), kind)) as f:
            t = json.load(f)
        assert t["kernel"] == bench.traffic_kernel(wl, kind)
        # the total and its two parts are rounded separately
        assert abs(b - t["fetch_bytes_per_launch"] - t["write_bytes_per_launch"]) <= 1
    # no counters for other kinds or workloads
    assert bench.measured_traffic(synth.workload("single_canvas"), "attention") is None
    assert bench.measured_traffic(synth.workload("single_canvas"), "qkv_rope") is None


def test_traffic_is_dropped_when_the_sources_change(monkeypatch):
    from block_discrete_diffusion_amd import synth
    wl = synth.workload("long_context")
    assert bench.measured_traffic(wl, "attention") is not None
    monkeypatch.setattr(bench, "source_hash", lambda kind: "0" * 64)
    assert bench.measured_traffic(wl, "attention") is None
    assert bench.measured_traffic(synth.workload("single_canvas")) is None
