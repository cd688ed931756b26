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
PROFILES = os.path.join(ROOT, "profiles")
LM_KERNELS = {False: "k_lmhead_bf16", True: "k_lmhead_fp8"}   # by lm_fp8
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def traffic_key(workload: str, lm_fp8: bool) -> str:
    return workload + ("_fp8head" if lm_fp8 else "")


def traffic_file(key: str) -> str:
    return os.path.join(PROFILES, f"lmhead_{key}_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5, help="timed canvases")
    ap.add_argument("--warmup", type=int, default=2, help="untimed canvases")
    ap.add_argument("--workload", default="single_canvas")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--fill", type=int, default=0, choices=(0, 1),
                    help="1: candidate canvas (uncommitted positions fed their candidate tokens)")
    ap.add_argument("--commit-conf", type=float, default=None,
                    help="threshold commit: also commit every position with confidence >= this value")
    ap.add_argument("--stop-entropy", type=float, default=None,
                    help="entropy stop: end the canvas once every position left open has entropy <= this "
                         "bound (nats); replaces the workload's confidence stop")
    ap.add_argument("--lm-fp8", action="store_true",
                    help="vocabulary head stored as e4m3 bytes with one fp32 scale per row")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true", help="also time every kernel kind (extra canvas)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of the bench, then of "
                         "--copy-calibration) into the LM-head traffic file under profiles/ and exit")
    ap.add_argument("--calibration-mib", type=int, default=256, help="size the calibration copy was run with")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="turn a rocprofv3 --kernel-trace --stats run of the default bench command into the "
                         "per-kernel summary under profiles/ and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 launches), the reference "
                         "kernel whose FETCH_SIZE / WRITE_SIZE counters scale the HBM traffic figures")
    return ap.parse_args()


def copy_calibration(mib: int):
    """A plain copy kernel of known size: reads and writes exactly mib MiB per launch."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert torch.equal(dst[:1024], src[:1024])
    print(json.dumps({"copy_calibration_bytes_per_launch": n * 4, "launches": 5}), flush=True)


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
        with open(traffic_file(traffic_key(wl.name, wl.lm_fp8))) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != lmhead_source_hash() or t.get("workload") != wl.name or \
            bool(t.get("lm_fp8")) != wl.lm_fp8:
        return None
    return float(t["bytes_per_launch"])


def counter_values(run_dir: str, kernel_substr: str):
    """Per-dispatch values (KiB) of the one counter of a rocprofv3 --pmc run,
    for the kernels whose name contains kernel_substr."""
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if kernel_substr in (row.get("Kernel_Name") or ""):
                    vals.append(float(row["Counter_Value"]))
    return vals


def summarize_trace(args):
    """Per-kernel launches / average / min / max from rocprofv3's kernel_stats.csv."""
    import csv
    import glob
    files = glob.glob(os.path.join(args.summarize_trace, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        sys.exit("no kernel_stats.csv")
    rows = list(csv.DictReader(open(files[0])))
    wl = args.workload
    from block_discrete_diffusion_amd import synth
    n_steps = synth.workload(wl).n_steps
    flag = " --lm-fp8" if args.lm_fp8 else ""
    lines = [f"# rocprofv3 kernel trace of the bench run, workload {wl}" +
             (" with the e4m3 vocabulary head" if args.lm_fp8 else ""),
             "# command: cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o bench -- "
             f"python3 <repo>/bench.py --workload {wl}{flag} --no-cpu-baseline",
             f"# (2 warm-up + 5 timed canvases + the profiled LM-head pass; {n_steps} denoising steps per canvas)",
             "# columns: launches, avg_us, min_us, max_us, share_of_gpu_time_%, kernel"]
    for r in rows:
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                     f"{float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}  {r['Name'][:110]}")
    out = os.path.join(PROFILES, f"step_{traffic_key(wl, args.lm_fp8)}_kernel_trace.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def write_traffic(args):
    """LM-head HBM bytes per launch = counter KiB x 1024 x (known bytes of the
    calibration copy / what the same counter reads for it)."""
    known = args.calibration_mib * (1 << 20)
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = args.write_traffic
    cf = [v for v in counter_values(cfetch_dir, COPY_KERNEL) if v * 1024 > known / 4]
    cw = [v for v in counter_values(cwrite_dir, COPY_KERNEL) if v * 1024 > known / 4]
    kernel = LM_KERNELS[args.lm_fp8]
    lf = counter_values(fetch_dir, kernel)
    lw = counter_values(write_dir, kernel)
    if not (cf and cw and lf and lw):
        sys.exit("missing counter values")
    f_scale = known / (sum(cf) / len(cf) * 1024)
    w_scale = known / (sum(cw) / len(cw) * 1024)
    fetch_b = sum(lf) / len(lf) * 1024 * f_scale
    write_b = sum(lw) / len(lw) * 1024 * w_scale
    flag = " --lm-fp8" if args.lm_fp8 else ""
    out = {"workload": args.workload, "lm_fp8": bool(args.lm_fp8), "kernel": kernel,
           "source_sha256": lmhead_source_hash(),
           "bytes_per_launch": round(fetch_b + write_b), "fetch_bytes_per_launch": round(fetch_b),
           "write_bytes_per_launch": round(write_b), "launches_counted": [len(lf), len(lw)],
           "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
           "calibration": f"plain device copy of {args.calibration_mib} MiB ({COPY_KERNEL}): FETCH_SIZE reads "
                          f"{sum(cf) / len(cf):.1f} KiB, WRITE_SIZE {sum(cw) / len(cw):.1f} KiB per launch",
           "commands": [f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- python3 bench.py "
                        f"--workload {args.workload}{flag} --steps 1 --warmup 0 --no-cpu-baseline",
                        "the same with --pmc WRITE_SIZE",
                        f"rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d <dir> -o run -- "
                        f"python3 bench.py --copy-calibration {args.calibration_mib}"]}
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_file(traffic_key(args.workload, args.lm_fp8)), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def open_rows_per_step(wl, init_committed, n_steps_done):
    """Open (uncommitted) positions summed over requests at the start of
    each denoising step of a canvas: the commit schedule takes
    ceil(|U| / (N - s + 1)) positions at step s; a request that stopped at
    step n_k has none left after it."""
    per_req = []
    for b in range(wl.batch):
        u = int(wl.canvas - int(init_committed[b].sum()))
        seq = []
        for s in range(1, wl.n_steps + 1):
            if s > n_steps_done[b] or u == 0:
                break
            seq.append(u)
            u -= -(-u // (wl.n_steps - s + 1))
        per_req.append(seq)
    n = max(len(x) for x in per_req)
    return [sum(x[s] for x in per_req if s < len(x)) for s in range(n)]


def measured_open_rows(cv, dw, wl, P):
    """Open positions summed over requests at the start of each step, read
    back step by step from an extra untimed canvas (for samplers whose commit
    counts depend on the run)."""
    import torch
    for b in range(wl.batch):
        cv.set_cache_len(b, P[b])
    cv.dg_canvas_reset(dw.init_ids, dw.init_committed)
    rows = []
    for _ in range(wl.n_steps):
        st = cv.state
        open_ = ((st.committed == 0) & (st.done.view(-1, 1) == 0)).sum().item()
        if open_ == 0:
            break
        rows.append(int(open_))
        cv.dg_denoise_step()
        torch.cuda.synchronize()
    cv.dg_append_canvas_kv()
    torch.cuda.synchronize()
    return rows


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
            O.denoise_step(m, r, wl.n_steps, wl.stop_conf, wl.commit_conf, wl.fill, wl.stop_entropy)
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

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.write_traffic:
        write_traffic(args)
        return
    if args.summarize_trace:
        summarize_trace(args)
        return

    import numpy as np
    import torch
    from block_discrete_diffusion_amd import binding as B
    from block_discrete_diffusion_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    B.lib()                                   # fails loudly without the HIP library
    wl = synth.workload(args.workload)
    if args.fill or args.commit_conf is not None:
        wl = wl.with_(fill=args.fill, commit_conf=args.commit_conf)
    if args.stop_entropy is not None:
        wl = wl.with_(stop_conf=None, stop_entropy=args.stop_entropy)
    if args.lm_fp8:
        wl = wl.with_(lm_fp8=True)
    inp = synth.make_inputs(wl, args.seed)
    dw = B.device_workload(inp)
    cv = B.Canvas(dw.model, dw.caches, wl.canvas, wl.n_steps, stop_conf=wl.stop_conf,
                  init_ids=dw.init_ids, init_committed=dw.init_committed,
                  commit_conf=wl.commit_conf, fill=wl.fill, stop_entropy=wl.stop_entropy)
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

    # roofline of the dominant kernel: LM head + fused vocabulary sampler.
    # Per launch it streams the whole head (V x d bf16) and works on the
    # positions still open at the start of the step: R_s rows of fp16 h
    # (d x 2 bytes), their row scale and index (8 bytes) and one 16-byte
    # record per 128-id slice (and a 4-byte entropy term per slice under the
    # entropy stop); 2 R_s d V flops.
    lm_ms, lm_n = prof.get("lmhead_sampler", (0.0, 0))
    avg_ms = lm_ms / max(lm_n, 1)
    if wl.commit_conf is None:
        rows = open_rows_per_step(wl, inp.init_committed, n_steps)
    else:
        rows = measured_open_rows(cv, dw, wl, P)     # the threshold decides the counts at run time
    R = sum(rows) / max(len(rows), 1)
    n_slices = (wl.vocab + 127) // 128
    rec_bytes = 16 + (4 if wl.stop_entropy is not None else 0)
    # e4m3 head: one byte per weight plus a 4-byte scale per row
    head_bytes = wl.vocab * wl.d_model + wl.vocab * 4 if wl.lm_fp8 else wl.vocab * wl.d_model * 2
    alg_bytes = int(head_bytes + R * (wl.d_model * 2 + 8) + n_slices * R * rec_bytes)
    alg_flops = 2.0 * R * wl.d_model * wl.vocab
    achieved = alg_bytes / (avg_ms / 1e3) / 1e9
    traffic = measured_traffic(wl)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "lmhead_sampler", "avg_launch_us": round(avg_ms * 1e3, 2), "launches": lm_n,
            "alg_bytes_per_launch": alg_bytes, "mean_open_rows": round(R, 2),
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
                   "adaptive_stop": wl.stop_conf, "stop_entropy": wl.stop_entropy,
                   "commit_conf": wl.commit_conf, "canvas_fill": wl.fill,
                   "lm_head": "e4m3 + fp32 row scales" if wl.lm_fp8 else "bf16",
                   "step": "one canvas: reset + denoising steps + KV append"},
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
