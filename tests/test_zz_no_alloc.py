"""The allocation-free handle (dg_canvas_init_static: library-owned device
scratch, no workspace argument) against the workspace handle of
dg_canvas_init on the same inputs: two calls in a row, the second on a
smaller input, each stage dump and the canvas state bit-identical (same
kernels, same inputs).  Also the refusals: shapes beyond the scratch, and a
second live handle on the device."""
import numpy as np
import pytest
import torch

from block_discrete_diffusion_amd import binding as B
from block_discrete_diffusion_amd import synth

pytestmark = pytest.mark.gpu


def run(wl, static, n_steps):
    inp = synth.make_inputs(wl, 0)
    dw = B.device_workload(inp)
    cv = B.Canvas(dw.model, dw.caches, wl.canvas, wl.n_steps, stop_conf=wl.stop_conf, init_ids=dw.init_ids,
                  init_committed=dw.init_committed, static_scratch=static)
    M = wl.batch * wl.canvas
    out = []
    for s in range(n_steps):
        q = torch.full((M, wl.n_q_heads * wl.head_dim), float("nan"), device="cuda")
        o = torch.full_like(q, float("nan"))
        h = torch.full((M, wl.d_model), float("nan"), device="cuda")
        rs = torch.full((M, 4), float("nan"), device="cuda")
        ent = torch.full((M,), float("nan"), device="cuda")
        cv.dg_denoise_step(q=q, o=o, h=h, row_stats=rs, entropy=ent)
        torch.cuda.synchronize()
        st = cv.state
        out.append([x.cpu() for x in (q, o, h, rs, ent, st.ids, st.committed, st.step, st.done)])
    err = cv.error_word()
    cv.dg_canvas_destroy()
    return out, err


def bits(x):
    return x.view(torch.int32) if x.is_floating_point() else x


@pytest.mark.parametrize("order", ["large_then_small"])
def test_static_scratch_handle_matches_workspace_handle(order):
    large = synth.workload("single_canvas", n_steps=48)
    small = synth.workload("single_canvas", vocab=1000, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                           canvas=40, n_steps=6, prefix=100)
    for wl, n in ((large, 3), (small, 6)):
        print(f"{wl.name} V {wl.vocab} d {wl.d_model} C {wl.canvas}: {n} steps", flush=True)
        ref, ref_err = run(wl, False, n)
        got, got_err = run(wl, True, n)
        assert torch.equal(ref_err, got_err) and int(got_err[:3].abs().sum()) == 0
        for s, (a, b) in enumerate(zip(ref, got)):
            for i, (x, y) in enumerate(zip(a, b)):
                assert torch.equal(bits(x), bits(y)), f"{wl.name} step {s + 1} dump {i}"


def test_static_scratch_refusals():
    wl = synth.workload("ragged_batch", vocab=1000, d_model=256, n_q_heads=16, n_kv_heads=4, head_dim=128,
                        canvas=256, n_steps=4, batch=16, prefix_range=(2048, 2048), n_eos_requests=0)
    inp = synth.make_inputs(wl, 0)
    dw = B.device_workload(inp)
    with pytest.raises(B.DGError) as ei:
        B.Canvas(dw.model, dw.caches, wl.canvas, wl.n_steps, static_scratch=True)
    assert ei.value.status == B.DG_ERR_WORKSPACE
    small = synth.workload("single_canvas", vocab=1000, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                           canvas=40, n_steps=3, prefix=100)
    dws = B.device_workload(synth.make_inputs(small, 0))
    c1 = B.Canvas(dws.model, dws.caches, small.canvas, small.n_steps, static_scratch=True)
    with pytest.raises(B.DGError) as ei:
        B.Canvas(dws.model, dws.caches, small.canvas, small.n_steps, static_scratch=True)
    assert ei.value.status == B.DG_ERR_STATE
    assert c1.dg_run_canvas() == [(3, 40)]
    c1.dg_canvas_destroy()
    c2 = B.Canvas(dws.model, dws.caches, small.canvas, small.n_steps, static_scratch=True)
    assert c2.dg_run_canvas() == [(3, 40)]
    c2.dg_canvas_destroy()
