"""Recorded steps (dg_canvas_set_graph) against separate launches, on the
GPU, through the C-ABI.

Two handles are built over identical inputs (each with its own caches,
since the steps write their canvas rows into the caches): one issues every
step as separate kernel launches, the other replays a recorded graph of the
step.  Their state (ids, committed flags, step counters, done flags, valid
lengths) and every cache row must agree bit for bit:

  * several canvases in a row on one recording (every step a replay), with
    the program's own eager work and synchronisations between them;
  * one step at a time over a batch whose vocabulary-head grouping changes
    as the open rows shrink (the step is recorded again), checked after every
    step;
  * across an append (the cache lengths change: recorded again), and after
    switching the recording off in the middle of a canvas.
"""
import pytest
import torch

from block_discrete_diffusion_amd import binding as B
from block_discrete_diffusion_amd import synth

pytestmark = pytest.mark.gpu

STATE_FIELDS = ("ids", "committed", "step", "done", "n_steps_done", "n_valid")


def small(**kw):
    base = dict(vocab=1000, d_model=256, n_q_heads=4, n_kv_heads=1, head_dim=128, canvas=128, n_steps=8,
                batch=3, prefix_range=(20, 300), n_eos_requests=0, stop_conf=None)
    base.update(kw)
    return synth.workload("ragged_batch", **base)


class Twin:
    """A handle issuing separate launches and a handle replaying recorded
    steps, over the same inputs."""

    def __init__(self, wl, seed=0, extra_canvases=0):
        self.wl = wl
        inp = synth.make_inputs(wl, seed)
        self.dws = [B.device_workload(inp, extra_canvases=extra_canvases) for _ in range(2)]
        self.c = [B.Canvas(dw.model, dw.caches, wl.canvas, wl.n_steps, stop_conf=wl.stop_conf,
                           init_ids=dw.init_ids, init_committed=dw.init_committed) for dw in self.dws]
        self.c[1].dg_canvas_set_graph(True)

    def assert_same(self, what):
        torch.cuda.synchronize()
        for f in STATE_FIELDS:
            a, b = getattr(self.c[0].state, f), getattr(self.c[1].state, f)
            assert torch.equal(a, b), f"{what}: {f} differs"
        for r, (ka, kb) in enumerate(zip(self.dws[0].caches, self.dws[1].caches)):
            assert ka.len == kb.len, f"{what}: cache {r} length"
            n = min(ka.capacity, ka.len + self.wl.canvas)
            for l in range(self.wl.n_layers):
                (k0, v0), (k1, v1) = ka.rows(0, n, layer=l), kb.rows(0, n, layer=l)
                assert torch.equal(k0, k1) and torch.equal(v0, v1), f"{what}: cache {r} layer {l} rows"
        for i in range(3):
            assert int(self.c[0].error_word()[i]) == int(self.c[1].error_word()[i]) == 0, f"{what}: error word"


def eager_work():
    """The program's own work between replays: a product and a reduction on
    the same device, then a synchronisation."""
    x = torch.randn(512, 512, device="cuda")
    y = (x @ x.T).sum()
    torch.cuda.synchronize()
    return float(y)


@pytest.mark.parametrize("name", ["single_canvas", "small"])
def test_canvases_replayed_equal_separate_launches(name):
    wl = synth.workload("single_canvas") if name == "single_canvas" else small()
    t = Twin(wl)
    for canvas in range(3):
        for c in t.c:
            c.dg_run_canvas()
        t.assert_same(f"canvas {canvas}")
        assert int(t.c[1].state.n_steps_done.min()) == wl.n_steps
        eager_work()
        for c in t.c:
            c.dg_canvas_reset()
        eager_work()


def test_steps_recorded_again_when_the_head_grouping_changes():
    wl = small()
    t = Twin(wl)
    for s in range(wl.n_steps):
        for c in t.c:
            c.dg_denoise_step()
        t.assert_same(f"step {s + 1}")
        eager_work()


def test_recording_follows_an_append_and_can_be_switched_off():
    wl = small(n_steps=6)
    t = Twin(wl, extra_canvases=2)
    for c in t.c:
        c.dg_run_canvas()
    t.assert_same("first canvas")
    for c in t.c:
        c.dg_append_canvas_kv()
    t.assert_same("append")
    for c in t.c:
        c.dg_canvas_reset()
    # half a canvas recorded (over the grown caches), the rest as separate launches
    for s in range(3):
        for c in t.c:
            c.dg_denoise_step()
        eager_work()
    t.c[1].dg_canvas_set_graph(False)
    for s in range(3, wl.n_steps):
        for c in t.c:
            c.dg_denoise_step()
    t.assert_same("second canvas")
    assert B.lib().dg_canvas_set_graph(t.c[1]._h, 2) == B.DG_ERR_SHAPE
