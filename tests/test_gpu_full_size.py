"""GPU parity at the full workload sizes, through the C-ABI, in the launch
configuration bench.py times (one canvas handle over the workload's batch).

The oracle is cheap enough at these sizes to compute every row, so the
checks compare all positions, not a sample:
  * single_canvas (V 32768, d 2048, 16/4/128, prefix 1024): the whole
    48-step canvas teacher-forced, full logits at step 1; with an e4m3 head,
    the first three steps;
  * full_vocab (V 262144, d 2816, 16/8/256, prefix 8192, stop 0.9): the
    first two steps, full logits at step 1;
  * long_context (V 32768, d 2816, 16/8/256, prefix 65536): first step,
    append of a finished canvas (rows checked against the oracle's fresh K/V
    of the same ids), then the first step of the next canvas over the longer
    prefix;
  * ragged_batch (8 requests, V 65536, prefixes 512..16384, two with a
    pre-committed EOS): the first two steps;
  * seeded mid-canvas states with few open positions, which reach the
    vocabulary head's narrower wave layouts (<= 128 and <= 64 open rows at
    d_model 2816) and its request groups (4 and 8 requests per workgroup
    in the ragged batch);
  * long_context through its 4 canvases (append, reset, a step each);
  * full_vocab with a stop threshold taken from the oracle's own margins, so
    that the adaptive stop fires at step 2 at this shape.
"""
import numpy as np
import pytest
import torch

from block_discrete_diffusion_amd import synth
from oracle import dg_oracle as O

from dgparity import Pair, inputs, seed_state, teacher_forced, to_np, tol

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def banner(msg):
    print(msg, flush=True)


def test_single_canvas_whole_trajectory():
    wl = synth.workload("single_canvas")
    banner(f"full size {wl.name}: {wl.n_steps} teacher-forced steps")
    pair = Pair(wl)
    ex = teacher_forced(pair, wl.n_steps, check_logits_first=True)
    r = pair.reqs[0]
    assert r.done and r.n_steps == wl.n_steps
    st = pair.canvas.state
    assert int(st.done[0]) == 1 and int(st.step[0]) == wl.n_steps
    assert int(st.committed.sum()) == wl.canvas
    print(f"exempted steps: {ex}")


def test_single_canvas_fp8_head_first_steps():
    wl = synth.workload("single_canvas", lm_fp8=True)
    banner(f"full size {wl.name} with an e4m3 head: 3 teacher-forced steps")
    pair = Pair(wl)
    teacher_forced(pair, 3, check_logits_first=True)


def test_full_vocab_first_steps():
    wl = synth.workload("full_vocab")
    banner(f"full size {wl.name}: 2 teacher-forced steps")
    pair = Pair(wl)
    teacher_forced(pair, 2, check_logits_first=True)


def test_ragged_batch_first_steps():
    wl = synth.workload("ragged_batch")
    banner(f"full size {wl.name}: 2 teacher-forced steps")
    pair = Pair(wl)
    assert sum(int(c.sum()) for c in pair.inp.init_committed) == wl.n_eos_requests
    teacher_forced(pair, 2)


def test_ragged_batch_short_budget_groups_requests():
    """Full ragged shapes with a budget of 4 steps: the open rows per request
    fall to 128 and then 64, so the vocabulary head takes 2 and then 4
    requests per workgroup at steps 3 and 4."""
    wl = synth.workload("ragged_batch").with_(n_steps=4)
    banner(f"full size {wl.name}, budget 4: 4 teacher-forced steps")
    pair = Pair(wl)
    teacher_forced(pair, 4)
    assert all(r.done for r in pair.reqs)
    assert int(pair.canvas.error_word()[2]) == 0


@pytest.mark.parametrize("name", ["full_vocab", "long_context"])
@pytest.mark.parametrize("n_open", [100, 40])
def test_few_open_rows_at_d2816(name, n_open):
    """A seeded state with 100 (<= 128: two id tiles per wave) or 40 (<= 64:
    one id tile per wave) open positions at d_model 2816, two steps."""
    wl = synth.workload(name)
    banner(f"full size {wl.name}: {n_open} open positions, 2 teacher-forced steps")
    pair = Pair(wl)
    seed_state(pair, [n_open], step=40, seed=n_open)
    teacher_forced(pair, 2)


@pytest.mark.parametrize("hi", [32, 64])
def test_ragged_batch_request_groups(hi):
    """Seeded states with at most 32 (8 requests per vocabulary-head
    workgroup) or at most 64 (4 per workgroup) open positions per request,
    counts differing per request; two steps; no group over its bound."""
    wl = synth.workload("ragged_batch")
    banner(f"full size {wl.name}: <= {hi} open positions per request, 2 teacher-forced steps")
    pair = Pair(wl)
    rng = np.random.default_rng(hi)
    counts = rng.integers(hi // 2, hi + 1, size=wl.batch)
    counts[0] = hi
    seed_state(pair, counts, step=44, seed=hi)
    teacher_forced(pair, 2)
    assert int(pair.canvas.error_word()[2]) == 0


def test_long_context_four_canvases():
    """The long-context loop of 4 canvases: each finished canvas (seeded
    clean ids) is appended (rows against the oracle's fresh K/V), the next
    canvas starts 256 positions further and its first step is checked."""
    wl = synth.workload("long_context")
    banner(f"full size {wl.name}: 4 canvases, a step and an append each")
    pair = Pair(wl)
    req = pair.reqs[0]
    cache = pair.dw.caches[0]
    rng = np.random.default_rng(7)
    t = tol(wl)
    for k in range(wl.n_canvases):
        teacher_forced(pair, 1)
        P = req.P
        assert P == 65536 + 256 * k and cache.len == P
        req.ids = rng.integers(0, wl.vocab - 1, size=wl.canvas).astype(np.int64)
        req.committed = np.ones(wl.canvas, dtype=np.uint8)
        req.step = wl.n_steps
        req.done = True
        pair.force_state()
        pair.canvas.dg_append_canvas_kv()
        torch.cuda.synchronize()
        assert cache.len == P + wl.canvas
        (k_ref,), (v_ref,) = O.append_canvas(pair.m, req)
        gk, gv = cache.rows(P, P + wl.canvas)
        np.testing.assert_allclose(to_np(gk), k_ref, atol=t, rtol=0, err_msg=f"appended K rows, canvas {k + 1}")
        np.testing.assert_allclose(to_np(gv), v_ref, atol=t, rtol=0, err_msg=f"appended V rows, canvas {k + 1}")
        if k + 1 < wl.n_canvases:
            O.reset_canvas(req, pair.inp.init_ids[0], pair.inp.init_committed[0])
            pair.canvas.dg_canvas_reset(pair.dw.init_ids, pair.dw.init_committed)
    assert cache.len == 65536 + 4 * 256


@pytest.mark.parametrize("side", [-1, 1])
def test_full_vocab_stop_decision_at_the_oracle_margin(side):
    """tau from the oracle's own step: 0.01 in log-confidence under (side -1)
    or over (side +1) the smallest confidence that step 1's schedule leaves
    open.  Under it every position left open is sure and the stop fires at
    step 1 (all 256 positions committed, N_k = 1); over it the step commits
    its schedule only.  (With these random weights the smallest confidence
    left open falls from step to step, so a stop can only fire first at
    step 1.)"""
    wl = synth.workload("full_vocab")
    mo = O.model_from_inputs(inputs(wl))
    rq = O.requests_from_inputs(mo, inputs(wl))[0]
    fw, st, cr = O.denoise_step(mo, rq, wl.n_steps, None)
    lo = float(st["logconf"][cr.committed == 0].min())
    del mo, rq, fw
    tau = float(np.float32(np.exp(lo + 0.01 * side)))
    banner(f"full size {wl.name}: stop threshold {side:+d}0 mlog from the step-1 margin")
    pair = Pair(wl, stop_conf=tau)
    teacher_forced(pair, 1)
    r = pair.reqs[0]
    st = pair.canvas.state
    if side < 0:
        assert r.done and r.n_steps == 1
        assert int(st.n_steps_done[0]) == 1 and int(st.done[0]) == 1 and bool(st.committed.all())
    else:
        assert not r.done and int(st.done[0]) == 0
        assert int(st.committed.sum()) == O.commit_count(wl.canvas, 1, wl.n_steps)


def test_long_context_append_and_next_canvas():
    wl = synth.workload("long_context")
    banner(f"full size {wl.name}: step, append, next canvas")
    pair = Pair(wl, extra_canvases=1)
    teacher_forced(pair, 1)

    # a finished canvas: seeded clean ids, every position committed
    rng = np.random.default_rng(7)
    req = pair.reqs[0]
    P = req.P
    req.ids = rng.integers(0, wl.vocab - 1, size=wl.canvas).astype(np.int64)
    req.committed = np.ones(wl.canvas, dtype=np.uint8)
    req.step = wl.n_steps
    req.done = True
    pair.force_state()
    pair.canvas.dg_append_canvas_kv()
    torch.cuda.synchronize()
    assert int(pair.canvas.error_word()[0]) == 0
    cache = pair.dw.caches[0]
    assert cache.len == P + wl.canvas
    (k_ref,), (v_ref,) = O.append_canvas(pair.m, req)
    gk, gv = cache.rows(P, P + wl.canvas)
    t = tol(wl)
    np.testing.assert_allclose(to_np(gk), k_ref, atol=t, rtol=0, err_msg="appended K rows")
    np.testing.assert_allclose(to_np(gv), v_ref, atol=t, rtol=0, err_msg="appended V rows")
    # rows before the canvas are untouched
    k0, _ = cache.rows(P - 8, P)
    np.testing.assert_array_equal(to_np(k0), O.decode(pair.inp.prefix_k[0][:, P - 8:P], "bf16"))

    # next canvas over the prefix + appended canvas
    O.reset_canvas(req, pair.inp.init_ids[0], pair.inp.init_committed[0])
    pair.canvas.dg_canvas_reset(pair.dw.init_ids, pair.dw.init_committed)
    teacher_forced(pair, 1)


def test_deep_canvas_steps_and_append():
    """Two layers with SwiGLU FFNs (d_ff 8192) at the single-canvas shapes:
    three teacher-forced steps (logits at step 1), then a finished canvas
    appended through the causal two-layer pass (both layers' rows against the
    oracle) and the first step of the next canvas."""
    wl = synth.workload("deep_canvas")
    banner(f"full size {wl.name}: 3 steps, append, next canvas")
    pair = Pair(wl, extra_canvases=1)
    teacher_forced(pair, 3, check_logits_first=True)
    rng = np.random.default_rng(8)
    req = pair.reqs[0]
    P = req.P
    req.ids = rng.integers(0, wl.vocab - 1, size=wl.canvas).astype(np.int64)
    req.committed = np.ones(wl.canvas, dtype=np.uint8)
    req.step = wl.n_steps
    req.done = True
    pair.force_state()
    pair.canvas.dg_append_canvas_kv()
    torch.cuda.synchronize()
    ks, vs = O.append_canvas(pair.m, req)
    cache = pair.dw.caches[0]
    t = tol(wl)
    for l in range(wl.n_layers):
        gk, gv = cache.rows(P, P + wl.canvas, layer=l)
        np.testing.assert_allclose(to_np(gk), ks[l], atol=t, rtol=0, err_msg=f"appended K rows, layer {l}")
        np.testing.assert_allclose(to_np(gv), vs[l], atol=t, rtol=0, err_msg=f"appended V rows, layer {l}")
    O.reset_canvas(req, pair.inp.init_ids[0], pair.inp.init_committed[0])
    pair.canvas.dg_canvas_reset(pair.dw.init_ids, pair.dw.init_committed)
    teacher_forced(pair, 1)


def test_single_canvas_temperature_sampling_first_steps():
    """Temperature sampling at the single-canvas shapes: three teacher-forced
    steps of Gumbel-max draws against the oracle."""
    wl = synth.workload("single_canvas", temperature=(1.0, 0.3, 42))
    banner(f"full size {wl.name} with temperature sampling: 3 teacher-forced steps")
    pair = Pair(wl)
    teacher_forced(pair, 3, check_logits_first=True)


@pytest.mark.parametrize("name", ["single_canvas", "deep_canvas"])
def test_fp8_projections_first_steps(name):
    """e4m3 projections (and FFN weights) at full size: three teacher-forced
    steps, logits at step 1."""
    wl = synth.workload(name, proj_fp8=True)
    banner(f"full size {wl.name} with e4m3 projections: 3 teacher-forced steps")
    pair = Pair(wl)
    teacher_forced(pair, 3, check_logits_first=True)


def test_moe_canvas_first_steps():
    """Two layers with 128 routed experts (8 per token) beside the shared
    FFN at the single-canvas shapes: two teacher-forced steps, every layer's
    expert choices, logits at step 1."""
    wl = synth.workload("moe_canvas")
    banner(f"full size {wl.name}: 2 teacher-forced steps")
    pair = Pair(wl)
    teacher_forced(pair, 2, check_logits_first=True)
