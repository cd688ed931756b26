"""Benchmark of the canvas denoising hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload single_canvas]

One bench step = one generation of the workload: its K canvases (K = 4 for
the long-context workload, else 1), each reset to all-MASK and denoised
until every request is done or the budget N is spent (embed/norm, QKV +
RoPE, block-bidirectional attention, output projection, LM head with the
fused vocabulary sampler, commit / re-mask / adaptive stop), with the KV
append pass between consecutive canvases (K - 1 appends, the extra forwards
that eq. (10) of the DiffusionGemma Technical Report, part 3, section 3.4
counts).  Before every generation the cache lengths go back to the prefix
lengths, so each bench step does the same work.

Prints one JSON line:
  * value: canvas tokens denoised per second, the sum of the valid lengths
    C_k (eq. (7)) over the timed generations divided by their time;
  * the efficiency metrics of eqs. (7)-(10) (Total Tokens, Total Denoising
    Steps, Effective Denoising Steps, tokens per forward), from the device's
    per-request step counts and valid lengths, per request for batches;
  * roofline: the dominant step kernel against its roof, and every step
    kernel in roofline_kernels, from HIP events around each launch in one
    extra generation run after the timed region;
  * cpu_baseline: the CPU oracle timed on the host cores on a bounded sample
    of the same workload.
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
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 (matrix / vector), published
PROFILES = os.path.join(ROOT, "profiles")
LM_KERNELS = {False: "k_lmhead_bf16", True: "k_lmhead_fp8"}   # by lm_fp8
ATTN_KERNELS = {64: "k_attn_bf16<64>", 128: "k_attn_q16<128>", 256: "k_attn_q16<256>"}   # by head_dim
COPY_KERNEL = "__amd_rocclr_copyBuffer"
# kernel kinds with committed HBM traffic counters, and the sources each
# kind's counts depend on
TRAFFIC_SOURCES = {"lmhead_sampler": ("k_gemm.hip", "dg_gemm.hpp", "dg_device.hpp", "dg_internal.hpp"),
                   "attention": ("k_attn.hip", "dg_device.hpp", "dg_internal.hpp")}
STEP_KINDS = ("qkv_rope", "attention", "attn_merge", "out_proj", "ffn", "moe", "lmhead_sampler", "sample_commit")


def traffic_key(workload: str, lm_fp8: bool) -> str:
    return workload + ("_fp8head" if lm_fp8 else "")


def traffic_file(key: str, kind: str = "lmhead_sampler") -> str:
    prefix = "lmhead" if kind == "lmhead_sampler" else kind
    return os.path.join(PROFILES, f"{prefix}_{key}_traffic.json")


def traffic_kernel(wl, kind: str) -> str:
    return LM_KERNELS[wl.lm_fp8] if kind == "lmhead_sampler" else ATTN_KERNELS[wl.head_dim]


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5, help="timed generations")
    ap.add_argument("--warmup", type=int, default=2, help="untimed generations")
    ap.add_argument("--workload", default="single_canvas")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--batch", type=int, default=None,
                    help="requests per canvas handle instead of the workload's (its prefix length each)")
    ap.add_argument("--budget", type=int, default=None,
                    help="denoising budget N instead of the workload's (e.g. 12: the pages' effective steps)")
    ap.add_argument("--fill", type=int, default=0, choices=(0, 1),
                    help="1: candidate canvas (uncommitted positions fed their candidate tokens)")
    ap.add_argument("--commit-conf", type=float, default=None,
                    help="threshold commit: also commit every position with confidence >= this value")
    ap.add_argument("--stop-conf", type=float, default=None,
                    help="confidence stop threshold instead of the workload's")
    ap.add_argument("--stop-entropy", type=float, default=None,
                    help="entropy stop: end the canvas once every position left open has entropy <= this "
                         "bound (nats); replaces the workload's confidence stop")
    ap.add_argument("--lm-fp8", action="store_true",
                    help="vocabulary head stored as e4m3 bytes with one fp32 scale per row")
    ap.add_argument("--graph", action="store_true",
                    help="issue each denoising step as one recorded HIP graph launch (dg_canvas_set_graph)")
    ap.add_argument("--proj-fp8", action="store_true",
                    help="every layer's projection weights as e4m3 bytes with one fp32 scale per output row")
    ap.add_argument("--temperature", type=float, nargs=2, default=None, metavar=("T0", "T1"),
                    help="temperature sampling, annealed linearly from T0 at step 1 to T1 at step N (seed 1)")
    ap.add_argument("--stop-tail", action="store_true",
                    help="also measure what the steps enqueued after an adaptive stop cost (extra runs)")
    ap.add_argument("--serve", type=str, default=None, metavar="SLOTS",
                    help="continuous-batching sweep instead of the bench line: comma-separated slot counts "
                         "(e.g. 1,2,4,8,16,32); prints one JSON line of serving throughput per count")
    ap.add_argument("--serve-requests", type=int, default=4, metavar="X",
                    help="requests per slot in each serving run")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of the bench, then of "
                         "--copy-calibration) into the traffic file of --traffic-kind under profiles/ and exit")
    ap.add_argument("--traffic-kind", default="lmhead_sampler", choices=("lmhead_sampler", "attention"),
                    help="the kernel whose counters --write-traffic reads")
    ap.add_argument("--calibration-mib", type=int, default=256, help="size the calibration copy was run with")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="turn a rocprofv3 --kernel-trace --stats run of the default bench command into the "
                         "per-kernel summary under profiles/ and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 launches), the reference "
                         "kernel whose FETCH_SIZE / WRITE_SIZE counters scale the HBM traffic figures")
    return ap.parse_args(argv)


# ----------------------------------------------------------------------------
# efficiency metrics of a generation (DiffusionGemma Technical Report, part 3,
# section 3.4): K canvases, canvas k taking N_k denoising steps and keeping
# C_k valid tokens
# ----------------------------------------------------------------------------

def generation_metrics(n_steps, n_valid) -> dict:
    """Total Tokens (7), Total Denoising Steps (8), Effective Denoising Steps
    (9: step counts weighted by the tokens each canvas kept) and tokens per
    forward (10: the K - 1 append forwards count as forwards)."""
    K = len(n_steps)
    tokens = sum(n_valid)
    steps = sum(n_steps)
    eds = sum(n * c for n, c in zip(n_steps, n_valid)) / tokens if tokens else float("nan")
    return {"total_tokens": tokens, "total_denoising_steps": steps,
            "effective_denoising_steps": eds, "tokens_per_forward": tokens / (steps + K - 1)}


# ----------------------------------------------------------------------------
# algorithmic work of the step kernels (bytes that must move, flops that
# must be done), per launch
# ----------------------------------------------------------------------------

def kernel_work(wl, P_mean, R, n_batch_rows, experts=None):
    """Per-launch algorithmic (bytes, flops, bound) of each step kernel kind.
    P_mean: mean prefix length per request over the generation; R: mean open
    positions summed over requests per step; n_batch_rows: B * C."""
    V, d, Hq, Hkv, hd, C, B = wl.vocab, wl.d_model, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.canvas, wl.batch
    M = n_batch_rows
    nqkv = (Hq + 2 * Hkv) * hd
    w = 2 if wl.dtype == "bf16" else 4
    ww = 1 if wl.proj_fp8 else w               # bytes per projection weight
    out = {}
    # E rows gathered, q written fp32, canvas K / V rows written
    out["qkv_rope"] = (nqkv * d * ww + M * d * w + M * Hq * hd * 4 + M * 2 * Hkv * hd * w, 2.0 * M * d * nqkv, "hbm")
    keys = sum(p + C for p in P_mean)
    att_flops = 4.0 * C * keys * hd * Hq
    # every prefix and canvas key / value once, q in and o out in fp32
    out["attention"] = (keys * Hkv * hd * 2 * w + M * Hq * hd * 8, att_flops, "mfma")
    out["attn_merge"] = (M * Hq * hd * 8, 0.0, "latency")
    # Wo, o in fp32, e in, h out in fp32
    out["out_proj"] = (d * Hq * hd * ww + M * Hq * hd * 4 + M * d * w + M * d * 4, 2.0 * M * Hq * hd * d, "hbm")
    n_slices = (V + 127) // 128
    head = (V * d + V * 4) if wl.lm_fp8 else V * d * w
    rec = 16 + (4 if wl.stop_entropy is not None else 0)
    out["lmhead_sampler"] = (head + R * (d * 2 + 8) + n_slices * R * rec, 2.0 * R * d * V, "hbm")
    # slice records in, the fp32 rows and two head rows of the exact leading logits
    out["sample_commit"] = (n_slices * R * rec + R * d * 4 + R * 2 * d * w, 4.0 * R * d, "latency")
    out["append"] = (2 * Hkv * hd * d * ww + B * C * d * w + B * C * 2 * Hkv * hd * w,
                     2.0 * B * C * d * 2 * Hkv * hd, "hbm")
    if wl.d_ff:
        # gate, up and down weights; x in and out in fp32, the activation out and in in fp32
        ff = wl.d_ff
        out["ffn"] = (3 * d * ff * ww + 2 * M * d * 4 + 2 * M * ff * 4, 6.0 * M * d * ff, "hbm")
    if wl.n_experts and experts is not None:
        # per layer: the router, the weights of the experts some token chose
        # (mean count over the steps), x's planes gathered, the activation
        # planes out and in, the gated outputs out (fp32)
        E, k, de = wl.n_experts, wl.top_k, wl.d_expert
        out["moe"] = (E * d * w + experts * 3 * d * de * w + M * d * 4 + 2 * M * k * de * 4 + M * k * d * 4,
                      2.0 * M * E * d + 6.0 * M * k * d * de, "hbm")
    return out


def measured_experts(cv, dw, wl, P):
    """Distinct experts chosen per layer per step (mean over the steps of one
    untimed canvas, read back from the routing dump step by step)."""
    import torch
    for b in range(wl.batch):
        cv.set_cache_len(b, P[b])
    cv.dg_canvas_reset(dw.init_ids, dw.init_committed)
    M = wl.batch * wl.canvas
    sel = torch.empty((wl.n_layers, M, wl.top_k), dtype=torch.int32, device="cuda")
    counts = []
    for _ in range(wl.n_steps):
        st = cv.state
        live = (st.done == 0).repeat_interleave(wl.canvas)
        if not bool(live.any()):
            break
        cv.dg_denoise_step(moe_sel=sel)
        torch.cuda.synchronize()
        for l in range(wl.n_layers):
            counts.append(int(torch.unique(sel[l][live]).numel()))
    return sum(counts) / max(len(counts), 1), counts


def roof_entry(bytes_, flops, bound, avg_us, peak_tflops):
    """Achieved fractions of HBM and matrix peak and of the binding roof
    (the larger of the two floors, bytes / BW and flops / peak)."""
    t = avg_us * 1e-6
    hbm = bytes_ / t / 1e9 / HBM_PEAK_GBS
    mfma = flops / t / 1e12 / peak_tflops
    t_hbm, t_mfma = bytes_ / (HBM_PEAK_GBS * 1e9), flops / (peak_tflops * 1e12)
    floor = max(t_hbm, t_mfma)
    if bound != "latency":
        bound = "mfma" if t_mfma > t_hbm else "hbm"
    return {"avg_us": round(avg_us, 2), "bound": bound, "alg_bytes": int(bytes_), "alg_flops": flops,
            "hbm_frac": round(hbm, 4), "mfma_frac": round(mfma, 4), "roof_frac": round(floor / t, 4)}


# ----------------------------------------------------------------------------
# counter and trace summaries (rocprofv3 outputs -> profiles/)
# ----------------------------------------------------------------------------

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
    return source_hash("lmhead_sampler")


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[kind]:
        with open(os.path.join(ROOT, "block_discrete_diffusion_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(wl, kind: str = "lmhead_sampler"):
    """HBM bytes per launch of the kernel kind (the LM head, or attention)
    from the committed rocprofv3 counter runs, if they were taken on the
    current kernel source; else None."""
    if kind not in TRAFFIC_SOURCES:
        return None
    try:
        with open(traffic_file(traffic_key(wl.name, wl.lm_fp8), kind)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_hash(kind) or t.get("workload") != wl.name or \
            bool(t.get("lm_fp8")) != wl.lm_fp8 or t.get("kernel") != traffic_kernel(wl, kind):
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
    w = synth.workload(wl)
    flag = " --lm-fp8" if args.lm_fp8 else ""
    lines = [f"# rocprofv3 kernel trace of the bench run, workload {wl}" +
             (" with the e4m3 vocabulary head" if args.lm_fp8 else ""),
             "# command: cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o bench -- "
             f"python3 <repo>/bench.py --workload {wl}{flag} --no-cpu-baseline --steps {args.steps} --warmup {args.warmup}",
             f"# ({args.warmup} warm-up + {args.steps} timed generations + the profiled generation; "
             f"{w.n_canvases} canvas(es) of up to {w.n_steps} denoising steps each)",
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
    from block_discrete_diffusion_amd import synth
    kind = args.traffic_kind
    wl = synth.workload(args.workload).with_(lm_fp8=bool(args.lm_fp8))
    kernel = traffic_kernel(wl, kind)
    lf = counter_values(fetch_dir, kernel)
    lw = counter_values(write_dir, kernel)
    if not (cf and cw and lf and lw):
        sys.exit("missing counter values")
    f_scale = known / (sum(cf) / len(cf) * 1024)
    w_scale = known / (sum(cw) / len(cw) * 1024)
    fetch_b = sum(lf) / len(lf) * 1024 * f_scale
    write_b = sum(lw) / len(lw) * 1024 * w_scale
    flag = " --lm-fp8" if args.lm_fp8 else ""
    extra = f" --budget {args.budget}" if args.budget else ""
    out = {"workload": args.workload, "lm_fp8": bool(args.lm_fp8), "kernel": kernel, "kind": kind,
           "source_sha256": source_hash(kind),
           "bytes_per_launch": round(fetch_b + write_b), "fetch_bytes_per_launch": round(fetch_b),
           "write_bytes_per_launch": round(write_b), "launches_counted": [len(lf), len(lw)],
           "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
           "calibration": f"plain device copy of {args.calibration_mib} MiB ({COPY_KERNEL}): FETCH_SIZE reads "
                          f"{sum(cf) / len(cf):.1f} KiB, WRITE_SIZE {sum(cw) / len(cw):.1f} KiB per launch",
           "commands": [f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- python3 bench.py "
                        f"--workload {args.workload}{flag}{extra} --steps 1 --warmup 0 --no-cpu-baseline",
                        "the same with --pmc WRITE_SIZE",
                        f"rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d <dir> -o run -- "
                        f"python3 bench.py --copy-calibration {args.calibration_mib}"]}
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_file(traffic_key(args.workload, args.lm_fp8), kind), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


# ----------------------------------------------------------------------------
# open rows of the vocabulary head
# ----------------------------------------------------------------------------

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
    return rows


def cpu_baseline(inp, wl, budget_s: float):
    """Time the oracle as it stands on this host: free-running denoising steps
    of the first canvas from its initial state until the budget is used, plus
    one append pass; scale to canvas tokens per second of a whole generation
    (K canvases of N steps, K - 1 appends)."""
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
            O.denoise_step(m, r, wl.n_steps, wl.stop_conf, wl.commit_conf, wl.fill, wl.stop_entropy, wl.temperature)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s:
            break
    t0 = time.perf_counter()
    for r in reqs:
        O.kv_rows(m, r.ids, r.P + np.arange(len(r.ids)), r.Ks, r.Vs)
    t_app = time.perf_counter() - t0
    t_step = sum(times) / len(times)
    K = wl.n_canvases
    t_gen = K * wl.n_steps * t_step + (K - 1) * t_app
    tokens = K * wl.batch * wl.canvas
    return {"value": tokens / t_gen, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(times)} denoising steps of the first {wl.name} canvas from its initial state "
                      f"(mean {t_step:.3f} s/step) and one append pass ({t_app:.3f} s), scaled to {K} canvas(es) "
                      f"of {wl.n_steps} steps and {K - 1} append(s)"}


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
    if args.serve:
        serve_sweep(args, B, synth, torch, np)
        return
    wl = synth.workload(args.workload)
    if args.budget is not None:
        wl = wl.with_(n_steps=args.budget)
    if args.batch is not None:
        wl = wl.with_(batch=args.batch)
    if args.fill or args.commit_conf is not None:
        wl = wl.with_(fill=args.fill, commit_conf=args.commit_conf)
    if args.stop_conf is not None:
        wl = wl.with_(stop_conf=args.stop_conf, stop_entropy=None)
    if args.stop_entropy is not None:
        wl = wl.with_(stop_conf=None, stop_entropy=args.stop_entropy)
    if args.lm_fp8:
        wl = wl.with_(lm_fp8=True)
    if args.proj_fp8:
        wl = wl.with_(proj_fp8=True)
    if args.temperature:
        wl = wl.with_(temperature=(args.temperature[0], args.temperature[1], 1))
    inp = synth.make_inputs(wl, args.seed)
    dw = B.device_workload(inp)
    K = wl.n_canvases

    def canvas_for(w):
        return B.Canvas(dw.model, dw.caches, w.canvas, w.n_steps, stop_conf=w.stop_conf,
                        init_ids=dw.init_ids, init_committed=dw.init_committed,
                        commit_conf=w.commit_conf, fill=w.fill, stop_entropy=w.stop_entropy,
                        temperature=w.temperature)

    cv = canvas_for(wl)
    if args.graph:
        cv.dg_canvas_set_graph(True)
    P = list(inp.prefix_len)

    def generation(c=cv, k_canvases=K):
        """K canvases with the K - 1 appends between them; returns, per
        canvas, per request (N_k, C_k) (dg_run_canvas waits once per canvas)."""
        for b in range(wl.batch):
            c.set_cache_len(b, P[b])
        stats = []
        for k in range(k_canvases):
            c.dg_canvas_reset(dw.init_ids, dw.init_committed)
            stats.append(c.dg_run_canvas(stats=True))
            if k + 1 < k_canvases:
                c.dg_append_canvas_kv()
        return stats

    for _ in range(args.warmup):
        generation()
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    t_wall0 = time.perf_counter()
    all_stats = []
    for _ in range(args.steps):
        all_stats.append(generation())
    ev1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    total_ms = ev0.elapsed_time(ev1)
    err = [int(x) for x in cv.error_word().cpu().tolist()[:3]]
    assert err == [0, 0, 0], f"device error word {err} (appends skipped, bad ids, vocabulary groups over bound)"

    stats = all_stats[-1]                        # [K][B] of (N_k, C_k)
    tokens = sum(c for st in all_stats for k in st for (_, c) in k)
    value = tokens / (total_ms / 1e3)
    fwd_steps = sum(max(n for (n, _) in k) for k in stats)       # denoising forwards of the batch
    ms_per_gen = total_ms / args.steps
    per_req = []
    for b in range(wl.batch):
        per_req.append(generation_metrics([k[b][0] for k in stats], [k[b][1] for k in stats]))
    if wl.batch == 1:
        metrics = per_req[0]
    else:
        metrics = {"per_request_tokens_per_forward": [round(m["tokens_per_forward"], 3) for m in per_req],
                   "per_request_total_tokens": [m["total_tokens"] for m in per_req],
                   "per_request_total_denoising_steps": [m["total_denoising_steps"] for m in per_req],
                   "total_tokens": sum(m["total_tokens"] for m in per_req)}

    # per-kernel timing: HIP events around every launch of one extra
    # generation (the LM head's are stamped by its own dispatch), outside
    # the timed region
    cv.dg_profile_enable(None)
    generation()
    torch.cuda.synchronize()
    prof = cv.dg_profile_read()
    cv.dg_profile_enable([])

    if wl.commit_conf is None:
        rows = []
        for k in stats:
            rows += open_rows_per_step(wl, inp.init_committed, [n for (n, _) in k])
    else:
        rows = measured_open_rows(cv, dw, wl, P)     # the threshold decides the counts at run time
    R = sum(rows) / max(len(rows), 1)
    P_mean = [p + wl.canvas * (K - 1) / 2.0 for p in P]
    experts, expert_counts = (measured_experts(cv, dw, wl, P) if wl.n_experts else (None, None))
    work = kernel_work(wl, P_mean, R, wl.batch * wl.canvas, experts)
    peak = BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS
    kernels = {}
    for kind, (ms, n) in prof.items():
        if kind not in work or n == 0:
            continue
        by, fl, bound = work[kind]
        e = roof_entry(by, fl, bound, ms * 1e3 / n, peak)
        e["launches"] = n
        e["us_per_generation"] = round(ms * 1e3, 1)
        if kind == "attention" and wl.dtype == "bf16":
            # q enters the scores as a hi + lo pair (two MFMAs per product), P
            # the P.V product as one fp16 operand (one MFMA): half the flops
            # are issued twice
            e["issued_mfma_frac"] = round(1.5 * e["mfma_frac"], 4)
        kernels[kind] = e
    step_kinds = [k for k in STEP_KINDS if k in kernels]
    dom = max(step_kinds, key=lambda k: kernels[k]["us_per_generation"])
    d = kernels[dom]
    if d["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": round(d["alg_flops"] / (d["avg_us"] * 1e-6) / 1e12, 1),
                "peak": peak, "unit": "TFLOP/s", "frac": d["mfma_frac"], "traffic": measured_traffic(wl, dom)}
    else:
        roof = {"bound": "hbm", "achieved": round(d["alg_bytes"] / (d["avg_us"] * 1e-6) / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": d["hbm_frac"],
                "traffic": measured_traffic(wl, dom)}
    roof.update({"kernel": dom, "avg_launch_us": d["avg_us"], "launches": d["launches"],
                 "alg_bytes_per_launch": d["alg_bytes"], "alg_flops_per_launch": d["alg_flops"],
                 "mean_open_rows": round(R, 2), "timing": "HIP events of one generation after the timed region"})

    line = {
        "metric": "canvas tokens denoised/sec", "value": round(value, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_gen, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded random weights and prefix K/V; no trained model)",
        "config": {"workload": wl.name, "vocab": wl.vocab, "d_model": wl.d_model, "q_heads": wl.n_q_heads,
                   "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "prefix": P if wl.batch > 1 else P[0],
                   "canvas": wl.canvas, "batch": wl.batch, "canvases": K, "denoise_budget": wl.n_steps,
                   "layers": wl.n_layers, "d_ff": wl.d_ff, "temperature": wl.temperature,
                   "experts": ({"n": wl.n_experts, "top_k": wl.top_k, "d_expert": wl.d_expert}
                               if wl.n_experts else None),
                   "adaptive_stop": wl.stop_conf, "stop_entropy": wl.stop_entropy,
                   "commit_conf": wl.commit_conf, "canvas_fill": wl.fill,
                   "lm_head": "e4m3 + fp32 row scales" if wl.lm_fp8 else ("bf16" if wl.dtype == "bf16" else "f32"),
                   "projections": "e4m3 + fp32 row scales" if wl.proj_fp8 else ("bf16" if wl.dtype == "bf16" else "f32"),
                   "step": f"one generation: {K} canvas(es) to done or N steps, {K - 1} KV append(s) between",
                   "launches": "one recorded graph per step" if args.graph else "separate kernel launches"},
        "denoise_steps_per_s": round(fwd_steps * args.steps / (total_ms / 1e3), 1),
        "us_per_denoise_step": round(ms_per_gen * 1e3 / fwd_steps, 2),
        "metrics_eq7_10": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in metrics.items()},
        "host_wall_s": round(t_wall, 4),
        "roofline": roof,
        "roofline_kernels": kernels,
        "experts_per_layer_step": ({"mean": round(experts, 2), "min": min(expert_counts),
                                    "max": max(expert_counts)} if experts is not None else None),
        "error_word": err,
    }
    if args.stop_tail:
        line["stop_tail"] = stop_tail(B, dw, wl, P, canvas_for)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def serve_requests(n, seed):
    """Output lengths of a serving run: each request asks for 1 to 4
    canvases (256 to 1024 tokens), drawn uniformly from a seeded stream, so
    that slots fall out of step."""
    import numpy as np
    return [int(k) for k in np.random.default_rng(seed).integers(1, 5, size=n)]


def serve_run(B, torch, cv, caches, P, wanted, continuous):
    """Serve the requests (canvases wanted per request) through the handle's
    slots, queue order, all queued at the start.  Continuous: a slot whose
    request is done takes the next one at once, while the others carry on;
    static: a batch of slots is refilled only once every slot in it is done.
    A request's next canvas follows in its slot either way (its canvas is
    appended to its cache first).  Returns (tokens, denoising steps
    enqueued)."""
    S = cv.B
    queue = list(range(len(wanted)))
    slot_req = [None] * S
    left = [0] * S
    tokens = 0
    steps = 0

    def admit(b):
        r = queue.pop(0)
        caches[b].len = P[b]
        cv.dg_canvas_admit(b, caches[b])
        slot_req[b], left[b] = r, wanted[r]

    for b in range(S):
        if queue:
            admit(b)
    while any(r is not None for r in slot_req):
        running = sum(1 << b for b in range(S) if slot_req[b] is not None)
        n, done = cv.dg_run_steps(1 << 30, running)
        steps += n
        for b in range(S):
            if slot_req[b] is None or not (done >> b) & 1:
                continue
            tokens += cv.C
            left[b] -= 1
            if left[b] > 0:
                cv.dg_append_request_kv(b)
            elif continuous and queue:
                admit(b)
            else:
                slot_req[b] = None
        if not continuous and all(r is None for r in slot_req):
            for b in range(S):
                if queue:
                    admit(b)
    return tokens, steps


def serve_sweep(args, B, synth, torch, np):
    """Serving throughput against concurrency: for each slot count, the same
    kind of request stream served with continuous batching and with static
    batches, on the single-canvas shapes (greedy, budget N, no adaptive
    stop).  Time is the host's wall clock over the whole run, every wait and
    host decision included."""
    counts = [int(x) for x in args.serve.split(",")]
    if max(counts) > B.DG_MAX_BATCH or min(counts) < 1:
        raise SystemExit(f"slot counts must lie in [1, {B.DG_MAX_BATCH}]")
    wl = synth.workload(args.workload).with_(batch=max(counts))
    if args.budget is not None:
        wl = wl.with_(n_steps=args.budget)
    inp = synth.make_inputs(wl, args.seed)
    dw = B.device_workload(inp, extra_canvases=4)
    points = []
    for S in counts:
        caches = dw.caches[:S]
        P = list(inp.prefix_len[:S])
        row = {"slots": S}
        for mode in ("continuous", "static"):
            cv = B.Canvas(dw.model, caches, wl.canvas, wl.n_steps, stop_conf=wl.stop_conf,
                          init_ids=dw.init_ids[:S].contiguous(), init_committed=dw.init_committed[:S].contiguous())
            wanted = serve_requests(args.serve_requests * S, args.seed + S)
            serve_run(B, torch, cv, caches, P, serve_requests(S, 99), mode == "continuous")     # warm-up
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            tokens, steps = serve_run(B, torch, cv, caches, P, wanted, mode == "continuous")
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            err = [int(x) for x in cv.error_word().cpu().tolist()[:3]]
            assert err == [0, 0, 0], f"device error word {err}"
            assert tokens == wl.canvas * sum(wanted)
            row[mode] = {"tokens_per_s": round(tokens / dt, 1), "wall_ms": round(dt * 1e3, 2),
                         "steps": steps, "us_per_step": round(dt * 1e6 / steps, 2),
                         "requests": len(wanted), "tokens": tokens}
            cv.dg_canvas_destroy()
        row["continuous_over_static"] = round(row["continuous"]["tokens_per_s"] / row["static"]["tokens_per_s"], 3)
        points.append(row)
        print(json.dumps({"serving_point": row}), flush=True)
    print(json.dumps({
        "metric": "canvas tokens denoised/sec", "unit": "tokens/s", "mode": "serving sweep",
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded random weights and prefix K/V; no trained model)",
        "config": {"workload": wl.name, "vocab": wl.vocab, "d_model": wl.d_model, "q_heads": wl.n_q_heads,
                   "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "prefix": wl.prefix, "canvas": wl.canvas,
                   "denoise_budget": wl.n_steps, "requests_per_slot": args.serve_requests,
                   "canvases_per_request": "uniform 1..4 (seeded)"},
        "points": points}), flush=True)


def stop_tail(B, dw, wl, P, canvas_for, reps=20):
    """What the steps enqueued after an adaptive stop cost: a canvas whose
    stop fires at step 1 (threshold below every confidence; dg_run_canvas
    then has 2 more steps in flight, which exit early on the device) against
    a canvas with a one-step budget (the same one live step, nothing after
    it), each timed over reps canvases, next to one live denoising step."""
    import torch

    def timed(c):
        for _ in range(3):
            for b in range(wl.batch):
                c.set_cache_len(b, P[b])
            c.dg_canvas_reset(dw.init_ids, dw.init_committed)
            c.dg_run_canvas(stats=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            c.dg_canvas_reset(dw.init_ids, dw.init_committed)
            st = c.dg_run_canvas(stats=True)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps, st

    stop1 = canvas_for(wl.with_(stop_conf=1e-9, stop_entropy=None))
    t_stop, st = timed(stop1)
    assert all(n == 1 for (n, _) in st), st
    stop1.dg_profile_enable(["sample_commit"])
    stop1.dg_canvas_reset(dw.init_ids, dw.init_committed)
    stop1.dg_run_canvas(stats=True)
    enq = stop1.dg_profile_read()["sample_commit"][1]
    one = canvas_for(wl.with_(n_steps=1, stop_conf=None, stop_entropy=None))
    t_one, _ = timed(one)
    two = canvas_for(wl.with_(n_steps=2, stop_conf=None, stop_entropy=None))
    t_two, _ = timed(two)
    live = t_two - t_one
    dead = (t_stop - t_one) / max(enq - 1, 1)
    return {"canvas_us_stop_at_step1": round(t_stop, 1), "steps_enqueued": enq,
            "canvas_us_one_step_budget": round(t_one, 1), "live_step_us": round(live, 1),
            "us_per_step_after_stop": round(dead, 1), "after_stop_over_live_step": round(dead / live, 4)}


if __name__ == "__main__":
    main()
