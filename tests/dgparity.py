"""Helpers of the GPU parity tests: run the HIP path and the CPU oracle on the
same seeded inputs and compare them under the parity contract.

Contract (per teacher-forced step; both sides start from the oracle's state):
  * floating outputs (q, o, h, canvas K/V rows, logits, log-confidence)
    within max abs error 2e-2 (bf16) or 1e-4 (fp32);
  * greedy ids bit-exact except where the oracle's top-2 logit gap < 1e-3;
  * the committed set bit-exact except where the oracle's confidence
    cutoff margin (log-confidence of the k-th minus the (k+1)-th ranked
    position) or its stop margin (min log-confidence left out minus ln tau,
    or h_max minus the max entropy left out) is below 1e-3; then the GPU's
    choice must still be one the oracle's ordering allows: every position
    that differs lies within 1e-3 plus twice the step's measured
    log-confidence error of the oracle's cut;
  * the done flag and valid length exact unless that request's commit was
    exempted;
  * the canvas K / V rows the step wrote into the cache scratch rows within
    the float tolerance of the oracle's.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from block_discrete_diffusion_amd import binding as B
from block_discrete_diffusion_amd import synth
from oracle import dg_oracle as O

GAP = 1e-3


def id_margin(wl, st):
    """The oracle's margin of each position's proposed id: the top-2 logit
    gap (greedy), or the gap of the two largest perturbed values z / T + g
    (temperature sampling)."""
    return st["key_gap"] if wl.temperature else st["m"] - st["m2"]


def tol(wl) -> float:
    return 2e-2 if wl.dtype == "bf16" else 1e-4


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


_INPUTS = {}


def inputs(wl, seed=0):
    """synth.make_inputs, memoised for the two most recent (workload, seed)
    pairs: the full-vocabulary inputs take tens of seconds to draw."""
    key = (wl, seed)
    if key not in _INPUTS:
        while len(_INPUTS) >= 2:
            _INPUTS.pop(next(iter(_INPUTS)))
        _INPUTS[key] = synth.make_inputs(wl, seed)
    return _INPUTS[key]


class Pair:
    """Oracle requests and a GPU canvas built from the same inputs."""

    def __init__(self, wl, seed=0, extra_canvases=0, stop_conf="workload", stop_entropy="workload"):
        self.wl = wl
        self.inp = inputs(wl, seed)
        self.m = O.model_from_inputs(self.inp)
        self.reqs = O.requests_from_inputs(self.m, self.inp)
        self.dw = B.device_workload(self.inp, extra_canvases=extra_canvases)
        self.stop = wl.stop_conf if stop_conf == "workload" else stop_conf
        self.hstop = wl.stop_entropy if stop_entropy == "workload" else stop_entropy
        self.canvas = self.make_canvas()
        M = wl.batch * wl.canvas
        dt = self.dw.model.tdtype
        self.q = torch.empty((M, wl.n_q_heads * wl.head_dim), dtype=torch.float32, device="cuda")
        self.o = torch.empty(self.q.shape, dtype=torch.float32, device="cuda")
        self.h = torch.empty((M, wl.d_model), dtype=torch.float32, device="cuda")
        self.rs = torch.empty((M, 4), dtype=torch.float32, device="cuda")
        self.ent = torch.empty((M,), dtype=torch.float32, device="cuda")
        self.sel = (torch.empty((wl.n_layers, M, wl.top_k), dtype=torch.int32, device="cuda")
                    if wl.n_experts else None)

    def make_canvas(self, state=None, flags=0):
        wl = self.wl
        return B.Canvas(self.dw.model, self.dw.caches, wl.canvas, wl.n_steps, stop_conf=self.stop,
                        init_ids=self.dw.init_ids, init_committed=self.dw.init_committed,
                        commit_conf=wl.commit_conf, fill=wl.fill, stop_entropy=self.hstop, state=state,
                        flags=flags, temperature=wl.temperature)

    def force_state(self):
        """Copy the oracle's canvas state into the GPU state buffers."""
        st = self.canvas.state
        ids = np.stack([r.ids for r in self.reqs]).astype(np.int32)
        com = np.stack([r.committed for r in self.reqs]).astype(np.uint8)
        st.ids.copy_(torch.from_numpy(ids))
        st.committed.copy_(torch.from_numpy(com))
        st.step.copy_(torch.tensor([r.step for r in self.reqs], dtype=torch.int32))
        st.done.copy_(torch.tensor([int(r.done) for r in self.reqs], dtype=torch.int32))
        self.canvas.dg_canvas_resume()

    def gpu_step(self, logits: bool = False):
        lg = None
        if logits:
            lg = torch.empty((self.wl.batch * self.wl.canvas, self.wl.vocab), dtype=torch.float32, device="cuda")
        self.canvas.dg_denoise_step(q=self.q, o=self.o, h=self.h, row_stats=self.rs, logits=lg, entropy=self.ent,
                                    moe_sel=self.sel)
        torch.cuda.synchronize()
        st = self.canvas.state
        rs = self.rs.cpu().numpy()
        out = dict(q=to_np(self.q), o=to_np(self.o), h=to_np(self.h),
                   m=rs[:, 0].astype(np.float64), S=rs[:, 1].astype(np.float64), m2=rs[:, 2].astype(np.float64),
                   argmax=rs[:, 3].copy().view(np.int32).astype(np.int64),
                   ids=st.ids.cpu().numpy(), committed=st.committed.cpu().numpy(),
                   step=st.step.cpu().numpy(), done=st.done.cpu().numpy(), n_valid=st.n_valid.cpu().numpy())
        with np.errstate(divide="ignore", invalid="ignore"):
            out["logconf"] = -np.log(out["S"])     # rows never sampled hold stale or unset values
        out["entropy"] = self.ent.cpu().numpy().astype(np.float64)
        if lg is not None:
            out["logits"] = lg.cpu().numpy().astype(np.float64)
        if self.sel is not None:
            out["moe_sel"] = self.sel.cpu().numpy()
        # canvas K / V rows of this step (cache scratch rows [len, len + C)),
        # per request, per layer
        ks, vs = [], []
        for c in self.dw.caches:
            rows = [c.rows(c.len, c.len + self.wl.canvas, layer=l) for l in range(self.wl.n_layers)]
            ks.append([to_np(k) for k, _ in rows])
            vs.append([to_np(v) for _, v in rows])
        out["kv"] = (ks, vs)
        return out

    def oracle_step(self, g=None):
        """The oracle's step of every request; with experts, tokens whose
        router margin is below the oracle's near-tie band take the GPU's
        choice of experts (g["moe_sel"])."""
        C = self.wl.canvas
        out = []
        for b, r in enumerate(self.reqs):
            routes = None
            if g is not None and "moe_sel" in g:
                routes = [g["moe_sel"][l, b * C:(b + 1) * C] for l in range(self.wl.n_layers)]
            out.append(O.denoise_step(self.m, r, self.wl.n_steps, self.stop, self.wl.commit_conf, self.wl.fill,
                                      self.hstop, self.wl.temperature, b, routes))
        return out


def report(b, g, fw, st, rows, open_, with_logits):
    """Print per-stage error statistics (shown by pytest on failure or with -s).
    Vocabulary statistics exist on the GPU only for the positions still open
    (uncommitted) at the start of the step."""
    C = rows.stop - rows.start
    items = []
    for name, ref in (("q", fw["q"].reshape(C, -1)), ("o", fw["o"].reshape(C, -1)), ("h", fw["h"])):
        d = np.abs(g[name][rows] - ref)
        items.append(f"{name}: max {d.max():.2e} diff-frac {np.mean(d > 0):.3f}")
    items.append(f"open: {int(open_.sum())}")
    if open_.any():
        items.append(f"m: {np.abs(g['m'][rows][open_] - st['m'][open_]).max():.2e}")
        items.append(f"logconf: {np.abs(g['logconf'][rows][open_] - st['logconf'][open_]).max():.2e}")
        items.append(f"entropy: {np.abs(g['entropy'][rows][open_] - st['entropy'][open_]).max():.2e}")
        if with_logits:
            z = fw["z"][open_]
            fin = np.isfinite(z)
            items.append(f"logits: {np.abs(g['logits'][rows][open_][fin] - z[fin]).max():.2e}")
    print(f"[req {b}] " + "; ".join(items))


def check_forward(pair: Pair, g: dict, res: list, before_c, check_logits=False):
    """Stage outputs of one step against the oracle's forward pass.  The
    vocabulary head and sampler run on the positions still open at the start
    of the step (before_c == 0); their statistics are compared there."""
    wl = pair.wl
    C = wl.canvas
    t = tol(wl)
    for b, r in enumerate(res):
        if r is None:
            continue
        fw, st, cr = r
        rows = slice(b * C, (b + 1) * C)
        open_ = before_c[b] == 0
        report(b, g, fw, st, rows, open_, check_logits)
        np.testing.assert_allclose(g["q"][rows], fw["q"].reshape(C, -1), atol=t, rtol=0, err_msg=f"q req {b}")
        np.testing.assert_allclose(g["o"][rows], fw["o"].reshape(C, -1), atol=t, rtol=0, err_msg=f"o req {b}")
        np.testing.assert_allclose(g["h"][rows], fw["h"], atol=t, rtol=0, err_msg=f"h req {b}")
        gm, glc, gam = g["m"][rows][open_], g["logconf"][rows][open_], g["argmax"][rows][open_]
        np.testing.assert_allclose(gm, st["m"][open_], atol=t, rtol=0, err_msg=f"max logit req {b}")
        np.testing.assert_allclose(glc, st["logconf"][open_], atol=t, rtol=0, err_msg=f"logconf req {b}")
        np.testing.assert_allclose(g["entropy"][rows][open_], st["entropy"][open_], atol=t, rtol=0,
                                   err_msg=f"entropy req {b}")
        gm2 = g["m2"][rows][open_]
        np.testing.assert_allclose(gm2, st["m2"][open_], atol=t, rtol=0, err_msg=f"second logit req {b}")
        sure = id_margin(wl, st)[open_] >= GAP
        np.testing.assert_array_equal(gam[sure], st["argmax"][open_][sure], err_msg=f"argmax req {b}")
        # the canvas K / V rows as fed at this step, every layer (requests not
        # done write them)
        for l in range(wl.n_layers):
            gk, gv = g["kv"][0][b][l], g["kv"][1][b][l]
            np.testing.assert_allclose(gk, fw["ks"][l].transpose(1, 0, 2), atol=t, rtol=0,
                                       err_msg=f"canvas K rows req {b} layer {l}")
            np.testing.assert_allclose(gv, fw["vs"][l].transpose(1, 0, 2), atol=t, rtol=0,
                                       err_msg=f"canvas V rows req {b} layer {l}")
        if check_logits:
            z = fw["z"][open_]
            gz = g["logits"][rows][open_]
            fin = np.isfinite(z)
            assert np.array_equal(fin, np.isfinite(gz)), "MASK column handling differs"
            np.testing.assert_allclose(gz[fin], z[fin], atol=t, rtol=0, err_msg=f"logits req {b}")


def check_commit(pair: Pair, g: dict, res: list, before_ids, before_c):
    """Commit decisions of one step against the oracle's (teacher-forced)."""
    wl = pair.wl
    C = wl.canvas
    n_exempt = 0
    for b, r in enumerate(res):
        if r is None:
            continue
        fw, st, cr = r
        gsel = (g["committed"][b] == 1) & (before_c[b] == 0)
        osel = cr.selected
        U = before_c[b] == 0
        exempt = False
        if not np.array_equal(gsel, osel):
            # allowed only across a near-tie of the ranking, of the stop test
            # or of the commit threshold
            near_cut = cr.cutoff_margin < GAP
            near_stop = cr.stop_margin is not None and abs(cr.stop_margin) < GAP
            near_thr = cr.commit_margin < GAP
            assert near_cut or near_stop or near_thr, \
                f"req {b}: committed set differs with margins {cr.cutoff_margin}, {cr.stop_margin}, {cr.commit_margin}"
            n_exempt += 1
            exempt = True
            if not (near_stop or near_thr):
                assert gsel.sum() == osel.sum(), "schedule size differs"
                lc = st["logconf"]
                cut = lc[osel].min()
                # the step's own measured log-confidence error over the open positions
                err = float(np.abs(g["logconf"][b * C:(b + 1) * C][U] - lc[U]).max())
                diff = np.flatnonzero(gsel != osel)
                band = GAP + 2 * err
                assert np.all(np.abs(lc[diff] - cut) < band), \
                    f"GPU choice outside the near-tie band {band:.2e}: {np.abs(lc[diff] - cut)}"
        # committed ids: previous ids kept, new ones = GPU greedy ids
        keep = before_c[b] == 1
        np.testing.assert_array_equal(g["ids"][b][keep], before_ids[b][keep])
        sel = np.flatnonzero(gsel)
        np.testing.assert_array_equal(g["ids"][b][sel], g["argmax"][b * C:(b + 1) * C][sel])
        sure = id_margin(wl, st) >= GAP
        both = gsel & osel & sure
        np.testing.assert_array_equal(g["ids"][b][both], cr.ids[both])
        if wl.fill:
            # candidate canvas: every position left open takes its greedy
            # token as its new candidate
            still = (before_c[b] == 0) & ~gsel
            np.testing.assert_array_equal(g["ids"][b][still], g["argmax"][b * C:(b + 1) * C][still])
            np.testing.assert_array_equal(g["ids"][b][still & ~osel & sure], cr.ids[still & ~osel & sure])
        assert g["step"][b] == pair.reqs[b].step
        assert bool(g["done"][b]) == cr.done or exempt, f"req {b}: done flag differs"
        if cr.done and g["done"][b]:
            exp = O.valid_length(g["ids"][b], pair.m.eos_id)
            assert g["n_valid"][b] == exp
    return n_exempt


def check_routes(pair: Pair, g: dict, res: list):
    """Every layer's expert choices: the GPU's set of chosen experts equals
    the oracle's for every token of a running request whose router margin
    (k-th against (k+1)-th logit) is at least the near-tie band; inside it
    the oracle took the GPU's choice (and checked it lies in the band).  The
    order among the chosen experts is not compared: two chosen experts with
    near-equal logits may swap ranks, which only reorders the fp32 sum of
    their gated outputs (the gates are a softmax over the set)."""
    if "moe_sel" not in g:
        return
    C = pair.wl.canvas
    for b, r in enumerate(res):
        if r is None:
            continue
        fw = r[0]
        for l, mg in enumerate(fw["route_margin"]):
            gsel = g["moe_sel"][l, b * C:(b + 1) * C]
            osel = fw["route_sel"][l]
            far = mg >= O.ROUTE_GAP
            np.testing.assert_array_equal(np.sort(gsel[far], axis=1), np.sort(osel[far], axis=1),
                                          err_msg=f"experts req {b} layer {l}")


def teacher_forced(pair: Pair, n_steps: int, check_logits_first=False):
    """Run n_steps teacher-forced steps, checking each; returns exemptions."""
    ex = 0
    for s in range(n_steps):
        if all(r.done for r in pair.reqs):
            break
        pair.force_state()
        before_ids = [r.ids.copy() for r in pair.reqs]
        before_c = [r.committed.copy() for r in pair.reqs]
        g = pair.gpu_step(logits=check_logits_first and s == 0)
        res = pair.oracle_step(g)
        check_routes(pair, g, res)
        check_forward(pair, g, res, before_c, check_logits=check_logits_first and s == 0)
        ex += check_commit(pair, g, res, before_ids, before_c)
    return ex


def seed_state(pair: Pair, open_counts, step: int, seed: int = 11):
    """Put every request of the oracle side in a seeded mid-canvas state:
    open_counts[b] positions left open (chosen at random), every other
    position committed to a random id (never MASK), step counter ``step``.
    The GPU side takes the same state at the next force_state()."""
    rng = np.random.default_rng(seed)
    wl = pair.wl
    for b, r in enumerate(pair.reqs):
        u = int(open_counts[b])
        ids = rng.integers(0, wl.vocab - 1, size=wl.canvas).astype(np.int64)
        com = np.ones(wl.canvas, dtype=np.uint8)
        com[rng.choice(wl.canvas, size=u, replace=False)] = 0
        ids[com == 0] = pair.m.mask_id
        r.ids, r.committed = ids, com
        r.step = step
        r.n_steps = step
        r.done = u == 0
        r.n_valid = wl.canvas


def first_divergence(pair: Pair, n_steps: int):
    """Free-running GPU steps beside free-running oracle steps from the same
    start.  Returns (step, exempt) of the first step whose committed ids or
    flags differ, with exempt telling whether the oracle's margins allowed
    it (a top-2 gap among the positions committed, the cutoff margin or the
    stop margin below 1e-3); (None, False) if the trajectories agree."""
    wl = pair.wl
    st = pair.canvas.state
    for s in range(1, n_steps + 1):
        if all(r.done for r in pair.reqs):
            return None, False
        pair.canvas.dg_denoise_step()
        res = pair.oracle_step()
        torch.cuda.synchronize()
        gids, gcom = st.ids.cpu().numpy(), st.committed.cpu().numpy()
        for b, r in enumerate(pair.reqs):
            if np.array_equal(gids[b], r.ids) and np.array_equal(gcom[b], r.committed):
                continue
            x = res[b]
            if x is None:
                return s, False
            _, o, cr = x
            gaps = id_margin(wl, o)[cr.selected]
            near = (gaps.size and gaps.min() < GAP) or cr.cutoff_margin < GAP or \
                (cr.stop_margin is not None and abs(cr.stop_margin) < GAP)
            return s, bool(near)
    return None, False
