"""Benchmark of the canvas denoising hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload single_canvas]

One bench step = one whole canvas of the workload: reset to all-MASK, the N
denoising steps (embed/norm, QKV + RoPE, block-bidirectional attention,
output projection, LM head with the fused vocabulary sampler, commit /
re-mask / adaptive stop), then the KV-append pass.  Before every canvas the
cache length is set back to the prefix length, so each canvas sees the same
prefix and the work per step is fixed.

Prints one JSON line: canvas tokens denoised per second (sum of C_k over the
timed canvases divided by the time, eq. (7) of the DiffusionGemma Technical
Report, section 3.4), the roofline position of the LM-head sampler kernel
(HIP events around each of its launches in the timed region) and the CPU
oracle timed on the host cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lmhead_single_canvas_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5, help="timed canvases")
    ap.add_argument("--warmup", type=int, default=2, help="untimed canvases")
    ap.add_argument("--workload", default="single_canvas")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true", help="also time every kernel kind (extra canvas)")
    return ap.parse_args()


def lmhead_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("k_gemm.hip", "dg_device.hpp", "dg_internal.hpp"):
        with open(os.path.join(ROOT, "block_discrete_diffusion_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(wl):
    """HBM bytes per LM-head launch from the committed rocprofv3 counter runs,
    if they were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != lmhead_source_hash() or t.get("workload") != wl.name:
        return None
    return float(t["bytes_per_launch"])


def cpu_baseline(inp, wl, budget_s: float):
    """Time the oracle as it stands on this host: free-running denoising steps
    of the same canvas from its initial state until the budget is used, plus
    one append pass; scale to canvas tokens per second."""
    import numpy as np
    from oracle import dg_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = sum(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas") or 1
    except Exception:
        threads = os.cpu_count() or 1
    m = O.model_from_inputs(inp)
    reqs = O.requests_from_inputs(m, inp)
    times = []
    t_start = time.perf_counter()
    for _ in range(wl.n_steps):
        t0 = time.perf_counter()
        for r in reqs:
            O.denoise_step(m, r, wl.n_steps, wl.stop_conf)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s:
            break
    t0 = time.perf_counter()
    for r in reqs:
        O.kv_rows(m, r.ids, r.P + np.arange(len(r.ids)))
    t_app = time.perf_counter() - t0
    t_step = sum(times) / len(times)
    t_canvas = wl.n_steps * t_step + t_app
    tokens = wl.batch * wl.canvas
    return {"value": tokens / t_canvas, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(times)} denoising steps of the {wl.name} canvas from its initial state "
                      f"(mean {t_step:.3f} s/step) and one append pass ({t_app:.3f} s), scaled to "
                      f"{wl.n_steps} steps + 1 append per canvas"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path is built for a single "
              f"MI355X and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from block_discrete_diffusion_amd import binding as B
    from block_discrete_diffusion_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    B.lib()                                   # fails loudly without the HIP library
    wl = synth.workload(args.workload)
    inp = synth.make_inputs(wl, args.seed)
    dw = B.device_workload(inp)
    cv = B.Canvas(dw.model, dw.caches, wl.canvas, wl.n_steps, stop_conf=wl.stop_conf,
                  init_ids=dw.init_ids, init_committed=dw.init_committed)
    P = list(inp.prefix_len)

    def one_canvas():
        for b in range(wl.batch):
            cv.set_cache_len(b, P[b])
        cv.dg_canvas_reset(dw.init_ids, dw.init_committed)
        cv.dg_run_canvas(stats=False)
        cv.dg_append_canvas_kv()

    for _ in range(args.warmup):
        one_canvas()
    torch.cuda.synchronize()

    cv.dg_profile_enable(["lmhead_sampler"])
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    n_valid = []
    n_steps = []
    for _ in range(args.steps):
        one_canvas()
    ev1.record()
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    prof = cv.dg_profile_read()
    cv.dg_profile_enable([])
    st = cv.state
    n_steps = st.n_steps_done.cpu().tolist()
    n_valid = st.n_valid.cpu().tolist()
    assert int(cv.error_word()[0]) == 0, "append found an unfinished canvas"

    tokens_per_canvas = sum(n_valid)
    steps_per_canvas = max(n_steps)
    ms_per_canvas = total_ms / args.steps
    value = tokens_per_canvas * args.steps / (total_ms / 1e3)

    # roofline of the dominant kernel: LM head + fused vocabulary sampler
    lm_ms, lm_n = prof.get("lmhead_sampler", (0.0, 0))
    avg_ms = lm_ms / max(lm_n, 1)
    M = wl.batch * wl.canvas
    n_slices = (wl.vocab + 127) // 128
    alg_bytes = wl.vocab * wl.d_model * 2 + M * wl.d_model * 2 + M * 4 + n_slices * M * 16
    alg_flops = 2.0 * M * wl.d_model * wl.vocab
    achieved = alg_bytes / (avg_ms / 1e3) / 1e9
    traffic = measured_traffic(wl)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "lmhead_sampler", "avg_launch_us": round(avg_ms * 1e3, 2), "launches": lm_n,
            "alg_bytes_per_launch": alg_bytes,
            "mfma_tflops": round(alg_flops / (avg_ms / 1e3) / 1e12, 1),
            "mfma_frac": round(alg_flops / (avg_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)}

    line = {
        "metric": "canvas tokens denoised/sec", "value": round(value, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_canvas, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded random weights and prefix K/V; no trained model)",
        "config": {"workload": wl.name, "vocab": wl.vocab, "d_model": wl.d_model, "q_heads": wl.n_q_heads,
                   "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "prefix": P if wl.batch > 1 else P[0],
                   "canvas": wl.canvas, "batch": wl.batch, "denoise_budget": wl.n_steps,
                   "adaptive_stop": wl.stop_conf, "step": "one canvas: reset + denoising steps + KV append"},
        "denoise_steps_per_s": round(steps_per_canvas * args.steps / (total_ms / 1e3), 1),
        "us_per_denoise_step": round(ms_per_canvas * 1e3 / steps_per_canvas, 2),
        "effective_steps": steps_per_canvas, "tokens_per_canvas": tokens_per_canvas,
        "roofline": roof,
    }
    if args.breakdown:
        cv.dg_profile_enable(None)
        one_canvas()
        torch.cuda.synchronize()
        br = cv.dg_profile_read()
        cv.dg_profile_enable([])
        line["kernel_us_per_canvas"] = {k: round(v[0] * 1e3, 1) for k, v in br.items()}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
