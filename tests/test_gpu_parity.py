"""HIP path vs CPU oracle, element by element on the same seeded inputs.

Small shapes span several tiles and ragged tails (canvas rows not a multiple
of the 128-row tile, vocabularies not a multiple of the 128-id slice, key
counts not a multiple of the 32-key block).  The five registered workloads
are covered at their full sizes in test_gpu_full_size.py.
"""
import math

import numpy as np
import pytest
import torch

from block_discrete_diffusion_amd import binding as B
from block_discrete_diffusion_amd import synth
from oracle import dg_oracle as O

from dgparity import GAP, Pair, first_divergence, teacher_forced, to_np, tol

pytestmark = pytest.mark.gpu


def small_bf16(hd=64, **kw):
    base = dict(vocab=1000, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=hd, canvas=40, n_steps=6,
                prefix=100)
    base.update(kw)
    return synth.workload("single_canvas", **base)


def test_tiny_f32_teacher_forced():
    pair = Pair(synth.workload("tiny_f32"))
    assert pair.dw.caches[0].len == 32
    # prefill rows against the oracle's prompt encoding
    K, V = pair.dw.caches[0].rows(0, 32)
    np.testing.assert_allclose(to_np(K), pair.reqs[0].K, atol=1e-5)
    np.testing.assert_allclose(to_np(V), pair.reqs[0].V, atol=1e-5)
    ex = teacher_forced(pair, 8, check_logits_first=True)
    assert all(r.done for r in pair.reqs)
    print("exempted steps:", ex)


@pytest.mark.parametrize("hd,d", [(64, 256), (128, 256), (256, 256), (128, 512), (64, 1024)])
def test_small_bf16_teacher_forced(hd, d):
    """d = 512 / 1024 also exercise the split-K projections (K cut in 2 / 4)."""
    pair = Pair(small_bf16(hd=hd, d_model=d))
    teacher_forced(pair, 6, check_logits_first=True)
    assert all(r.done for r in pair.reqs)


@pytest.mark.parametrize("hd,d,V", [(64, 256, 1000), (128, 512, 1000), (64, 256, 130)])
def test_small_bf16_fp8_head_teacher_forced(hd, d, V):
    """e4m3 vocabulary head with per-row scales: logits at step 1 and every
    stage of 6 steps against the oracle on the decoded head (V = 1000 and 130
    end in a ragged 128-id slice)."""
    wl = small_bf16(hd=hd, d_model=d, vocab=V, lm_fp8=True)
    pair = Pair(wl)
    assert pair.dw.model.lm_head.dtype == torch.uint8
    teacher_forced(pair, 6, check_logits_first=True)


def _first_step_conf_quantile(wl, q):
    """tau_c at the q-quantile of the oracle's first-step confidences, so that
    the threshold commits a real share of the positions at step 1."""
    pair = Pair(wl)
    st = O.sampler_stats(O.forward(pair.m, pair.reqs[0], wl.fill)["z"])
    return float(np.quantile(st["conf"], q))


@pytest.mark.parametrize("fill", [0, 1])
def test_tiny_f32_sampler_variants(fill):
    """Threshold commit and candidate canvas on the fp32 path."""
    wl = synth.workload("tiny_f32").with_(fill=fill)
    wl = wl.with_(commit_conf=_first_step_conf_quantile(wl, 0.6))
    pair = Pair(wl)
    ex = teacher_forced(pair, 8)
    assert all(r.done for r in pair.reqs)
    print("exempted steps:", ex)


@pytest.mark.parametrize("fill,threshold", [(1, False), (0, True), (1, True)])
def test_small_bf16_sampler_variants(fill, threshold):
    """Candidate canvas (uncommitted positions fed their candidate tokens)
    and threshold commit, teacher-forced on the bf16 path."""
    wl = small_bf16(hd=128, d_model=512, n_steps=6, fill=fill)
    if threshold:
        wl = wl.with_(commit_conf=_first_step_conf_quantile(wl, 0.5))
    pair = Pair(wl)
    teacher_forced(pair, 6, check_logits_first=True)
    assert all(r.done for r in pair.reqs)


@pytest.mark.parametrize("canvas,n_steps", [(1, 3), (40, 1)])
def test_small_bf16_degenerate_schedules(canvas, n_steps):
    """A one-position canvas (one row in every tile, one query per head), and
    a budget of one step (every position commits at step 1)."""
    pair = Pair(small_bf16(hd=64, d_model=256, canvas=canvas, n_steps=n_steps))
    teacher_forced(pair, n_steps, check_logits_first=True)
    assert all(r.done for r in pair.reqs)


def test_small_bf16_canvas_committed_before_the_first_step():
    """Every position committed before the first step: nothing is open, so
    the vocabulary head and the sampler see zero rows; the forward pass still
    runs over the canvas and the step only marks the request done with its
    valid length."""
    wl = small_bf16(hd=64, d_model=256, canvas=40, n_steps=4)
    pair = Pair(wl)
    rng = np.random.default_rng(5)
    for r in pair.reqs:
        r.ids = rng.integers(0, wl.vocab - 1, size=wl.canvas).astype(np.int64)
        r.committed = np.ones(wl.canvas, dtype=np.uint8)
    teacher_forced(pair, 1)
    assert all(r.done for r in pair.reqs)
    assert int(pair.canvas.state.done.cpu()[0]) == 1
    assert int(pair.canvas.state.n_valid.cpu()[0]) == pair.reqs[0].n_valid


def test_small_bf16_candidate_canvas_free_running_commits_match():
    """Free-running candidate canvas: the GPU's own trajectory, checked by
    re-running the oracle's commit rule on the GPU's statistics."""
    wl = small_bf16(hd=64, d_model=256, n_steps=5, fill=1)
    pair = Pair(wl)
    c = pair.canvas
    for s in range(wl.n_steps):
        before_ids = c.state.ids.cpu().numpy()[0].copy()
        before_c = c.state.committed.cpu().numpy()[0].copy()
        rs = torch.empty((wl.canvas, 4), dtype=torch.float32, device="cuda")
        c.dg_denoise_step(row_stats=rs)
        torch.cuda.synchronize()
        r = rs.cpu().numpy()
        ids = c.state.ids.cpu().numpy()[0]
        com = c.state.committed.cpu().numpy()[0]
        U = before_c == 0
        am = r[:, 3].copy().view(np.int32)
        # every open position now holds its greedy token; committed ones keep theirs
        np.testing.assert_array_equal(ids[U], am[U])
        np.testing.assert_array_equal(ids[~U], before_ids[~U])
        k = O.commit_count(int(U.sum()), s + 1, wl.n_steps)
        assert int(com.sum() - before_c.sum()) == k
    assert bool(c.state.done.cpu().numpy()[0])


def test_small_bf16_canvas_kv_rows_and_append():
    wl = small_bf16(hd=128, canvas=72, n_steps=4, prefix=61)
    pair = Pair(wl)
    teacher_forced(pair, 4)
    P, C = 61, 72
    # last step's scratch rows hold the K/V of the canvas as fed in that step
    pair.force_state()
    pair.canvas.dg_append_canvas_kv()
    torch.cuda.synchronize()
    assert int(pair.canvas.error_word()[0]) == 0
    r = pair.reqs[0]
    (k,), (v,) = O.append_canvas(pair.m, r)
    Kg, Vg = pair.dw.caches[0].rows(P, P + C)
    np.testing.assert_allclose(to_np(Kg), k, atol=tol(wl), rtol=0)
    np.testing.assert_allclose(to_np(Vg), v, atol=tol(wl), rtol=0)
    assert pair.dw.caches[0].len == P + C
    with pytest.raises(B.DGError):
        pair.canvas.dg_denoise_step()


def test_append_of_unfinished_canvas_is_refused():
    """dg_append_canvas_kv reads the done flags first: with a request not
    done it returns STATE and enqueues nothing (no row, no length changes)."""
    wl = small_bf16(canvas=32, n_steps=4, prefix=40)
    pair = Pair(wl, extra_canvases=1)
    before = pair.dw.caches[0].k.clone()
    with pytest.raises(B.DGError) as ei:
        pair.canvas.dg_append_canvas_kv()
    assert ei.value.status == B.DG_ERR_STATE
    torch.cuda.synchronize()
    assert pair.dw.caches[0].len == 40
    assert torch.equal(before, pair.dw.caches[0].k)
    assert int(pair.canvas.error_word()[0]) == 0
    # the handle still steps and appends once the canvas is done
    assert pair.canvas.dg_run_canvas() == [(4, 32)]
    pair.canvas.dg_append_canvas_kv()
    assert pair.dw.caches[0].len == 72


def test_ragged_batch_small_with_eos():
    wl = synth.workload("ragged_batch", vocab=1000, d_model=256, n_q_heads=4, n_kv_heads=1, head_dim=128,
                        canvas=48, n_steps=5, batch=3, prefix_range=(20, 300), n_eos_requests=1)
    pair = Pair(wl)
    assert len(set(pair.inp.prefix_len)) > 1
    teacher_forced(pair, 5, check_logits_first=True)
    assert all(r.done for r in pair.reqs)
    n_valid = pair.canvas.state.n_valid.cpu().numpy()
    for b, r in enumerate(pair.reqs):
        assert n_valid[b] == O.valid_length(pair.canvas.state.ids[b].cpu().numpy(), wl.eos_id)
    # the vocabulary head took two requests per workgroup (48-position
    # canvases), the last group holding one; no group exceeded its bound
    assert int(pair.canvas.error_word()[2]) == 0


@pytest.mark.parametrize("proj_fp8", [False, True])
def test_many_requests_take_256_row_projection_tiles(proj_fp8):
    """12 requests of 256 rows (3072 token rows) over 24 heads of 128: the
    projections take 256-row tiles over whole K (576 q / k / v tiles); q, o,
    h, the statistics, the commits and the canvas K / V rows against the
    oracle."""
    wl = synth.workload("ragged_batch", vocab=1000, d_model=256, n_q_heads=16, n_kv_heads=4, head_dim=128,
                        canvas=256, n_steps=2, batch=12, prefix_range=(20, 120), n_eos_requests=0, stop_conf=None,
                        proj_fp8=proj_fp8)
    pair = Pair(wl)
    teacher_forced(pair, 2, check_logits_first=True)
    assert int(pair.canvas.error_word()[0]) == 0


def _oracle_trajectory(wl, seed=0, stop=None):
    inp = synth.make_inputs(wl, seed)
    m = O.model_from_inputs(inp)
    reqs = O.requests_from_inputs(m, inp)
    trace = O.run_canvas(m, reqs, wl.n_steps, stop)
    return m, reqs, trace


def test_adaptive_stop_fires_where_the_oracle_stops():
    """tau is chosen from the oracle's own trajectory so that the stop fires at
    a step after the first, with every earlier step clearly below it."""
    wl = small_bf16(hd=64, n_steps=8)
    inp = synth.make_inputs(wl, 0)
    mo = O.model_from_inputs(inp)
    rq = O.requests_from_inputs(mo, inp)[0]
    mins = []
    for s in range(1, wl.n_steps):
        fw, st, cr = O.denoise_step(mo, rq, wl.n_steps, None)
        mins.append(st["logconf"][cr.committed == 0].min())   # positions left open by step s
    choice = None
    for s in range(1, len(mins)):
        t = mins[s] - 0.01
        if all(mins[j] < t - 0.005 for j in range(s)):
            choice = (s + 1, t)
    if choice is None:
        pytest.skip("no step after the first gives a clean stop for this seed")
    stop_step, ln_tau = choice
    tau = float(np.float32(math.exp(ln_tau)))
    pair = Pair(wl, stop_conf=tau)
    teacher_forced(pair, wl.n_steps)
    assert pair.reqs[0].n_steps == stop_step
    assert int(pair.canvas.state.n_steps_done[0]) == stop_step
    assert bool(pair.canvas.state.committed.all())


def test_entropy_stop_fires_where_the_oracle_stops():
    """Entropy stop: h_max is chosen from the oracle's own trajectory so that
    the stop fires at a step after the first, with every earlier step's
    largest left-out entropy clearly above it.  Each step also checks the
    per-position entropies against the oracle's.  The LM head is drawn with a
    larger spread so that the distributions are peaked and their entropies
    far apart."""
    wl = small_bf16(hd=64, n_steps=8, lm_std=0.3)
    inp = synth.make_inputs(wl, 0)
    mo = O.model_from_inputs(inp)
    rq = O.requests_from_inputs(mo, inp)[0]
    maxs = []
    for s in range(1, wl.n_steps):
        fw, st, cr = O.denoise_step(mo, rq, wl.n_steps, None)
        maxs.append(st["entropy"][cr.committed == 0].max())   # positions left open by step s
    choice = None
    for s in range(1, len(maxs)):
        h = maxs[s] + 0.02
        if all(maxs[j] > h + 0.02 for j in range(s)):
            choice = (s + 1, h)
            break
    if choice is None:
        pytest.skip("no step after the first gives a clean entropy stop for this seed")
    stop_step, h_max = choice
    pair = Pair(wl, stop_conf=None, stop_entropy=float(np.float32(h_max)))
    teacher_forced(pair, wl.n_steps)
    assert pair.reqs[0].n_steps == stop_step
    assert int(pair.canvas.state.n_steps_done[0]) == stop_step
    assert bool(pair.canvas.state.committed.all())


@pytest.mark.parametrize("fill", [0, 1])
def test_tiny_f32_entropy_stop_and_dump(fill):
    """fp32 path: entropy dump within 1e-4 of the oracle and the entropy stop
    rule, teacher-forced (h_max at the median first-step entropy)."""
    wl = synth.workload("tiny_f32").with_(fill=fill, stop_conf=None, lm_std=0.3)
    pair = Pair(wl)
    st = O.sampler_stats(O.forward(pair.m, pair.reqs[0], fill)["z"])
    wl = wl.with_(stop_entropy=float(np.float32(np.median(st["entropy"]))))
    teacher_forced(Pair(wl), wl.n_steps)


def test_entropy_stop_extremes():
    wl = small_bf16(hd=64, n_steps=5)
    pair = Pair(wl, stop_conf=None, stop_entropy=math.log(wl.vocab))   # above every entropy: step 1
    assert pair.canvas.dg_run_canvas() == [(1, wl.canvas)]
    assert bool(pair.canvas.state.committed.all())
    pair = Pair(wl, stop_conf=None, stop_entropy=-1.0)                 # never reachable
    assert pair.canvas.dg_run_canvas() == [(5, wl.canvas)]


def test_stop_threshold_extremes():
    wl = small_bf16(hd=64, n_steps=5)
    pair = Pair(wl, stop_conf=1e-9)                  # every confidence exceeds it: stop at step 1
    stats = pair.canvas.dg_run_canvas()
    assert stats == [(1, wl.canvas)]
    assert bool(pair.canvas.state.committed.all())
    pair = Pair(wl, stop_conf=2.0)                   # never reachable: the full budget
    assert pair.canvas.dg_run_canvas() == [(5, wl.canvas)]


def test_free_running_matches_oracle_until_first_near_tie():
    """GPU and oracle each run free from the same start; their committed ids
    and flags must agree at every step, or first differ at a step whose
    oracle margins exempt it (a near-tie below 1e-3)."""
    wl = small_bf16(hd=128, canvas=64, n_steps=8, prefix=200)
    pair = Pair(wl)
    s, exempt = first_divergence(pair, wl.n_steps)
    if s is not None:
        assert exempt, f"free-running trajectory first differs at step {s} without a near-tie"
        print(f"first divergence at exempted step {s}")
    else:
        assert int(pair.canvas.state.n_steps_done[0]) == wl.n_steps


def test_free_running_single_canvas_shape_small_vocab():
    """Free-running at the single-canvas layer shapes (d 2048, 16/4/128,
    prefix 1024, 256 positions) with a smaller vocabulary, 12 steps."""
    wl = synth.workload("single_canvas", vocab=4096, n_steps=12)
    pair = Pair(wl)
    s, exempt = first_divergence(pair, wl.n_steps)
    assert s is None or exempt, f"free-running trajectory first differs at step {s} without a near-tie"


def test_multi_canvas_loop_matches_oracle():
    """K consecutive canvases: run, append, reset; the cache grows by C per canvas."""
    wl = small_bf16(hd=64, canvas=32, n_steps=4, prefix=50, n_canvases=3)
    pair = Pair(wl)
    P0 = 50
    for k in range(3):
        teacher_forced(pair, 4)
        r = pair.reqs[0]
        assert r.done
        pair.force_state()
        pair.canvas.dg_append_canvas_kv()
        (kk,), (vv,) = O.append_canvas(pair.m, r)
        start = P0 + 32 * k
        Kg, Vg = pair.dw.caches[0].rows(start, start + 32)
        torch.cuda.synchronize()
        np.testing.assert_allclose(to_np(Kg), kk, atol=tol(wl), rtol=0)
        np.testing.assert_allclose(to_np(Vg), vv, atol=tol(wl), rtol=0)
        if k < 2:
            O.reset_canvas(r, np.full(32, wl.mask_id), np.zeros(32, np.uint8))
            pair.canvas.dg_canvas_reset()
    assert pair.dw.caches[0].len == P0 + 96
    mt = O.metrics([4, 4, 4], [32, 32, 32])
    assert mt["effective_steps"] == 4 and mt["tpf"] == pytest.approx(96 / 14)


def test_deterministic_bits():
    """Two handles over the same inputs: every stage dump (q, o, h, row
    statistics, entropies, logits at step 1) and the canvas state are
    bit-identical step by step (fixed reduction orders; a race or an
    order-dependent reduction would show here)."""
    wl = small_bf16(hd=128, d_model=512, canvas=64, n_steps=5)
    runs = []
    for _ in range(2):
        pair = Pair(wl)
        M = wl.canvas
        steps = []
        for s in range(wl.n_steps):
            lg = torch.full((M, wl.vocab), float("nan"), dtype=torch.float32, device="cuda") if s == 0 else None
            for t in (pair.q, pair.o, pair.h, pair.rs, pair.ent):
                t.fill_(float("nan"))
            pair.canvas.dg_denoise_step(q=pair.q, o=pair.o, h=pair.h, row_stats=pair.rs, logits=lg,
                                        entropy=pair.ent)
            torch.cuda.synchronize()
            st = pair.canvas.state
            steps.append([x.clone() for x in (pair.q, pair.o, pair.h, pair.rs, pair.ent, st.ids, st.committed)] +
                         ([lg.clone()] if lg is not None else []))
        runs.append(steps)
    for s, (a, b) in enumerate(zip(*runs)):
        for i, (x, y) in enumerate(zip(a, b)):
            assert torch.equal(x.view(torch.int32) if x.is_floating_point() else x,
                               y.view(torch.int32) if y.is_floating_point() else y), f"step {s + 1}, dump {i}"


def test_resume_after_destroy_equals_uninterrupted_run():
    """Checkpoint / resume: run 3 steps, destroy the handle, build a new one
    over the same state buffers and caches with DG_INIT_RESUME, finish; the
    canvas equals the one of an uninterrupted run, bit for bit."""
    wl = small_bf16(hd=128, canvas=64, n_steps=7, prefix=90)
    ref = Pair(wl)
    assert ref.canvas.dg_run_canvas() == [(7, 64)]
    pair = Pair(wl)
    for _ in range(3):
        pair.canvas.dg_denoise_step()
    torch.cuda.synchronize()
    state = pair.canvas.state
    pair.canvas.dg_canvas_destroy()
    c2 = pair.make_canvas(state=state, flags=B.DG_INIT_RESUME)
    assert c2.dg_run_canvas() == [(7, 64)]
    for name in ("ids", "committed", "step", "n_steps_done", "n_valid", "done"):
        assert torch.equal(getattr(c2.state, name), getattr(ref.canvas.state, name)), name


def test_run_canvas_stops_enqueueing_after_the_stop():
    """With a stop at step 1, dg_run_canvas enqueues at most 1 more step
    (it reads the done flags 2 steps behind) instead of the whole budget."""
    wl = small_bf16(hd=64, n_steps=12)
    pair = Pair(wl, stop_conf=1e-9)
    pair.canvas.dg_profile_enable(["sample_commit"])
    assert pair.canvas.dg_run_canvas() == [(1, wl.canvas)]
    n = pair.canvas.dg_profile_read()["sample_commit"][1]
    assert 1 <= n <= 2, n


def test_profile_counts_launches():
    wl = small_bf16(hd=64, n_steps=3)
    pair = Pair(wl)
    pair.canvas.dg_profile_enable()
    pair.canvas.dg_run_canvas()
    prof = pair.canvas.dg_profile_read()
    assert prof["lmhead_sampler"][1] == 3 and prof["sample_commit"][1] == 3
    assert all(ms >= 0 for ms, n in prof.values())


@pytest.mark.parametrize("L,d_ff,hd,d", [(2, 0, 64, 256), (1, 512, 128, 256), (3, 256, 64, 512), (2, 512, 256, 256)])
def test_deep_model_teacher_forced(L, d_ff, hd, d):
    """Stacked layers and dense SwiGLU FFNs: every layer's canvas K / V rows,
    the last layer's q and o, h, the statistics and the commits of every
    step against the oracle, logits at step 1."""
    wl = small_bf16(hd=hd, d_model=d, n_layers=L, d_ff=d_ff, n_steps=5)
    pair = Pair(wl)
    teacher_forced(pair, 5, check_logits_first=True)
    assert all(r.done for r in pair.reqs)


@pytest.mark.parametrize("L,d_ff,hd", [(2, 256, 64), (3, 0, 64), (2, 256, 128), (2, 0, 256)])
def test_deep_append_is_causal_context_encoding(L, d_ff, hd):
    """The append pass of a deep model: every layer's rows against the
    oracle's causal encoding of the finished canvas over the prefix, then a
    teacher-forced step of the next canvas over the longer caches (head_dim
    64: the 32-query attention form; 128 and 256: the 16-query form, whose
    causal mask cuts inside the 32-key blocks at 70 + 48 keys)."""
    wl = small_bf16(hd=hd, d_model=256, canvas=48, n_steps=3, prefix=70, n_layers=L, d_ff=d_ff)
    pair = Pair(wl, extra_canvases=1)
    teacher_forced(pair, 3)
    r = pair.reqs[0]
    assert r.done
    pair.force_state()
    pair.canvas.dg_append_canvas_kv()
    torch.cuda.synchronize()
    ks, vs = O.append_canvas(pair.m, r)
    cache = pair.dw.caches[0]
    for l in range(L):
        K, V = cache.rows(70, 70 + 48, layer=l)
        np.testing.assert_allclose(to_np(K), ks[l], atol=tol(wl), rtol=0, err_msg=f"layer {l} K rows")
        np.testing.assert_allclose(to_np(V), vs[l], atol=tol(wl), rtol=0, err_msg=f"layer {l} V rows")
    assert cache.len == 70 + 48
    O.reset_canvas(r, pair.inp.init_ids[0], pair.inp.init_committed[0])
    pair.canvas.dg_canvas_reset(pair.dw.init_ids, pair.dw.init_committed)
    teacher_forced(pair, 1)


@pytest.mark.parametrize("hd,d,V,fp8", [(64, 256, 1000, False), (128, 512, 130, False), (64, 256, 1000, True)])
def test_temperature_sampling_teacher_forced(hd, d, V, fp8):
    """Temperature sampling with annealing (T 1.5 -> 0.5): the drawn ids, the
    draws' log-probabilities and the commits of every step against the
    oracle's Philox4x64-10 Gumbel-max draws (ids exact unless the two largest
    perturbed values are within 1e-3)."""
    wl = small_bf16(hd=hd, d_model=d, vocab=V, n_steps=6, lm_fp8=fp8, temperature=(1.5, 0.5, 20241203))
    pair = Pair(wl)
    teacher_forced(pair, 6, check_logits_first=True)
    assert all(r.done for r in pair.reqs)


def test_temperature_sampling_draws_differ_from_greedy_and_repeat():
    """The same seed gives the same canvas twice; another seed another one;
    the drawn canvas is not the greedy one."""
    wl = small_bf16(hd=64, n_steps=4, temperature=(2.0, 1.0, 7))
    runs = []
    for seed in (7, 7, 8):
        pair = Pair(wl.with_(temperature=(2.0, 1.0, seed)))
        pair.canvas.dg_run_canvas()
        runs.append(pair.canvas.state.ids.cpu().clone())
    greedy = Pair(wl.with_(temperature=None))
    greedy.canvas.dg_run_canvas()
    assert torch.equal(runs[0], runs[1])
    assert not torch.equal(runs[0], runs[2])
    assert not torch.equal(runs[0], greedy.canvas.state.ids.cpu())


@pytest.mark.parametrize("L,d_ff,hd,prompt", [(1, 0, 128, 0), (2, 256, 64, 0), (1, 0, 64, 40)])
def test_fp8_projections_teacher_forced(L, d_ff, hd, prompt):
    """e4m3 projection weights with per-output-row scales (the bf16 weights
    quantised row by row): every layer's canvas K / V rows, q, o, h, the
    statistics and the commits of every step against the oracle on the
    dequantised weights, logits at step 1; with a prompt, the prefill's rows
    through the same weights."""
    wl = small_bf16(hd=hd, n_layers=L, d_ff=d_ff, n_steps=4, proj_fp8=True, prompt_tokens=prompt)
    pair = Pair(wl)
    if prompt:
        ks, vs = O.kv_rows(pair.m, pair.inp.prompt, np.arange(prompt))
        K, V = pair.dw.caches[0].rows(0, prompt)
        np.testing.assert_allclose(to_np(K), ks[0], atol=tol(wl), rtol=0, err_msg="prefill K rows")
        np.testing.assert_allclose(to_np(V), vs[0], atol=tol(wl), rtol=0, err_msg="prefill V rows")
    teacher_forced(pair, 4, check_logits_first=True)
    assert all(r.done for r in pair.reqs)


def test_fp8_projection_append_of_a_deep_model():
    wl = small_bf16(hd=64, canvas=48, n_steps=3, prefix=70, n_layers=2, d_ff=256, proj_fp8=True)
    pair = Pair(wl, extra_canvases=1)
    teacher_forced(pair, 3)
    r = pair.reqs[0]
    pair.force_state()
    pair.canvas.dg_append_canvas_kv()
    torch.cuda.synchronize()
    ks, vs = O.append_canvas(pair.m, r)
    for l in range(2):
        K, V = pair.dw.caches[0].rows(70, 70 + 48, layer=l)
        np.testing.assert_allclose(to_np(K), ks[l], atol=tol(wl), rtol=0, err_msg=f"layer {l} K rows")
        np.testing.assert_allclose(to_np(V), vs[l], atol=tol(wl), rtol=0, err_msg=f"layer {l} V rows")


@pytest.mark.parametrize("L,E,k,hd", [(1, 8, 2, 64), (2, 16, 4, 128), (2, 32, 8, 64)])
def test_experts_teacher_forced(L, E, k, hd):
    """Routed experts beside the shared FFN: every layer's expert choices
    (exact outside the oracle's 1e-3 near-tie band of the router margin;
    inside it the oracle takes the GPU's choice), every layer's canvas K / V
    rows, q, o, h, the statistics and the commits of every step, logits at
    step 1."""
    wl = small_bf16(hd=hd, n_layers=L, d_ff=256, n_experts=E, top_k=k, d_expert=256, n_steps=4)
    pair = Pair(wl)
    teacher_forced(pair, 4, check_logits_first=True)
    assert all(r.done for r in pair.reqs)


def test_experts_in_a_ragged_batch_and_the_append():
    """Three requests of different prefix lengths share the experts' lists;
    then the causal append pass of the finished canvases through two routed
    layers (a token's layer-1 rows depend on its own layer-0 routing only:
    rows of tokens inside the near-tie band are not compared)."""
    wl = synth.workload("ragged_batch", vocab=1000, d_model=256, n_q_heads=4, n_kv_heads=1, head_dim=64,
                        canvas=40, n_steps=3, batch=3, prefix_range=(20, 120), n_eos_requests=0, stop_conf=None,
                        n_layers=2, d_ff=256, n_experts=16, top_k=4, d_expert=256)
    pair = Pair(wl, extra_canvases=1)
    teacher_forced(pair, 3)
    assert all(r.done for r in pair.reqs)
    pair.force_state()
    pair.canvas.dg_append_canvas_kv()
    torch.cuda.synchronize()
    for b, r in enumerate(pair.reqs):
        P = r.P
        margins = []
        ks, vs = O.kv_rows(pair.m, r.ids, P + np.arange(wl.canvas), r.Ks, r.Vs, margins=margins)
        ok = margins[0] >= O.ROUTE_GAP
        for l in range(2):
            K, V = pair.dw.caches[b].rows(P, P + wl.canvas, layer=l)
            keep = ok if l == 1 else np.ones_like(ok)
            np.testing.assert_allclose(to_np(K)[:, keep], ks[l][:, keep], atol=tol(wl), rtol=0,
                                       err_msg=f"req {b} layer {l} K rows")
            np.testing.assert_allclose(to_np(V)[:, keep], vs[l][:, keep], atol=tol(wl), rtol=0,
                                       err_msg=f"req {b} layer {l} V rows")
