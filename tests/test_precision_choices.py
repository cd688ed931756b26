"""Operand precision of the attention products, decided by emulation.

The attention kernel multiplies P (the softmax numerators, at most 2^8) as a
single fp16 operand against the fp16 values, and q as two bf16 operands (hi
and lo) against the bf16 keys.  These tests emulate the candidate operand
roundings in float64 on the oracle's own step-1 state, carry the attention
output through the output projection and the vocabulary head, and measure
how far the logits of each row's leading ids move.  The step's discrete
decisions are exact only outside a near-tie band of 1e-3 (greedy id, top-k
cut, stop), so an operand choice is acceptable when it moves those logits by
well under half the band; a move of more than the band can flip decisions
the contract does not exempt.

Kept: single fp16 P (the bound below).  Rejected: a single bf16 q (moves the
logits by more than the band) and a single fp16 q together with the fp16 P
(above half the band at head_dim 256).
"""
import math

import numpy as np
import pytest

from block_discrete_diffusion_amd import synth
from oracle import dg_oracle as O

BAND = 1e-3


def step_state(name):
    # the attention shapes of the workload (head_dim, heads, prefix, canvas);
    # the vocabulary is cut to 32768 ids, which leaves the leading logits'
    # sensitivity to o unchanged and keeps the test to seconds
    wl = synth.workload(name, vocab=min(32768, synth.workload(name).vocab))
    inp = synth.make_inputs(wl, 0)
    m = O.model_from_inputs(inp)
    req = O.requests_from_inputs(m, inp)[0]
    out = O.forward(m, req)
    K = np.concatenate([req.Ks[0], out["k"].transpose(1, 0, 2)], axis=1)
    Vv = np.concatenate([req.Vs[0], out["v"].transpose(1, 0, 2)], axis=1)
    top = np.argsort(-out["z"], axis=1)[:, :8]
    return m, out, K, Vv, top


def emulated_attention(m, q, K, Vv, qmode, pmode):
    """Block-bidirectional attention with q and P rounded as a kernel would
    feed them to its products; the row sums l add the unrounded p."""
    G = m.Hq // m.Hkv
    C = q.shape[0]
    o = np.empty((C, m.Hq, m.hd))
    sc = math.log2(math.e) / math.sqrt(m.hd)
    for h in range(m.Hq):
        g = h // G
        qq = q[:, h, :] * sc
        if qmode == "bf16":
            qe = O.round_bf16(qq)
        elif qmode == "f16":
            qe = O.round_f16(qq)
        else:                                   # two bf16 parts
            hi = O.round_bf16(qq)
            qe = hi + O.round_bf16(qq - hi)
        s = qe @ K[g].T
        p = np.exp2(s - s.max(axis=1, keepdims=True))
        l = p.sum(axis=1, keepdims=True)
        pe = O.round_f16(p) if pmode == "f16" else p
        o[:, h, :] = (pe @ Vv[g]) / l
    return o


def leading_logit_move(m, out, K, Vv, top, qmode, pmode):
    o = emulated_attention(m, out["q"], K, Vv, qmode, pmode)
    C = o.shape[0]
    h = out["e"] + o.reshape(C, -1) @ m.Wo.T
    r = O.rms_scale(h, m.eps)[:, None]
    z = r * np.einsum("cd,ckd->ck", h, m.Wlm[top])
    return np.abs(z - np.take_along_axis(out["z"], top, 1)).max()


_STATES = {}


def cached_state(name):
    if name not in _STATES:
        _STATES[name] = step_state(name)
    return _STATES[name]


@pytest.fixture(params=["single_canvas", "full_vocab"])
def state(request):
    return cached_state(request.param)


def test_single_fp16_p_moves_the_leading_logits_by_under_half_the_band(state):
    d = leading_logit_move(*state, "bf16x2", "f16")
    assert d < 0.5 * BAND, d


def test_two_part_q_and_exact_p_are_far_inside_the_band(state):
    d = leading_logit_move(*state, "bf16x2", "exact")
    assert d < 0.02 * BAND, d


def test_a_single_bf16_q_would_exceed_the_band(state):
    d = leading_logit_move(*state, "bf16", "f16")
    assert d > BAND, d


def test_a_single_fp16_q_has_no_margin_at_head_dim_256():
    m, out, K, Vv, top = cached_state("full_vocab")
    d = leading_logit_move(m, out, K, Vv, top, "f16", "f16")
    assert d > 0.5 * BAND, d
