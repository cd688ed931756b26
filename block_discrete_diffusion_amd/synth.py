"""Seeded synthetic inputs for the canvas denoising step.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the HIP path and the CPU oracle receive exactly the
arrays produced here, so the two never depend on each other.

Workloads follow the problem statement of the DiffusionGemma Technical Report:
a canvas of C tokens over a vocabulary of V ids (section 2.1), denoised for at
most N steps (section 3.3, N=48) against a read-only KV cache of earlier
context (blog retelling, "Once Written, a Prefix Becomes History").  The layer
shapes are synthetic stand-ins: the pages publish no weights, so every weight
is N(0, 0.02^2) random and every prefix K/V row is N(0, 1).

Draw order (numpy PCG64 ``default_rng(seed)``):
  1. E, Wq, Wk, Wv, Wo, then Wlm when the head is untied; each is
     ``standard_normal(shape, float32) * 0.02`` in nn.Linear ``[out, in]`` shape
     (Wlm: ``* lm_std``, 0.02 unless a test asks for peakier distributions).
     FP8 head (``lm_fp8``): Wlm is drawn as ``standard_normal * 16`` and
     stored as e4m3 codes, then its per-row scales
     ``lm_std / 16 * 2^uniform(-1/2, 1/2)`` in float32.
  1b. Deeper models: layer 0's FFN Wg, Wu, Wd (if d_ff > 0), then for each
     further layer Wq, Wk, Wv, Wo and its Wg, Wu, Wd, the same way.
  2. tiny workload: the prompt ``integers(0, V - 1, n_prompt)``.
     Other workloads: one prefix length per request (fixed, or
     ``integers(lo, hi + 1)`` for ragged batches), then the EOS requests
     ``choice(B, n_eos, replace=False)`` and their canvas positions
     ``integers(0, C)``, then for every request its prefix K then V as
     ``standard_normal([Hkv, P_b, hd], float32)`` (for each layer in turn).
fp32 values are converted to bf16 by round-to-nearest-even on the bit pattern.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"


@dataclass(frozen=True)
class Workload:
    """Shapes and sampler settings of one synthetic canvas workload."""
    name: str
    dtype: str                 # "bf16" or "f32": storage / arithmetic type of the path
    vocab: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    canvas: int                # C
    n_steps: int               # N, the denoising budget
    batch: int = 1             # B concurrent requests, one canvas each
    tied: bool = False         # LM head shares the embedding matrix
    prefix: int = 0            # P for every request (ignored when prefix_range is set)
    prefix_range: Optional[tuple] = None   # (lo, hi) inclusive, drawn per request
    prompt_tokens: int = 0     # >0: the prefix is built from this many prompt ids (prefill)
    stop_conf: Optional[float] = None      # adaptive stop threshold tau, None = no stop
    eos_id: int = -1           # <0: no EOS handling
    n_eos_requests: int = 0    # requests that carry a pre-committed EOS in their canvas
    n_canvases: int = 1        # K consecutive canvases
    commit_conf: Optional[float] = None    # threshold commit tau_c, None = schedule only
    fill: int = 0              # 1: uncommitted positions carry candidate tokens (drawn uniformly at start)
    stop_entropy: Optional[float] = None   # entropy stop bound h_max (nats), None = off
    lm_std: float = 0.02       # std of the untied LM head's entries (larger: peakier distributions)
    lm_fp8: bool = False       # LM head as OCP e4m3 codes + one fp32 scale per row (bf16 models)
    proj_fp8: bool = False     # every layer's projections as e4m3 codes + one fp32 scale per output row
    temperature: Optional[tuple] = None    # (T0, T1, seed): temperature sampling, None = greedy
    n_layers: int = 1          # transformer layers (each with its own KV cache)
    d_ff: int = 0              # dense SwiGLU feed-forward width per layer, 0 = no FFN
    n_experts: int = 0         # routed SwiGLU experts per layer beside the dense (shared) FFN, 0 = none
    top_k: int = 0             # experts per token
    d_expert: int = 0          # width of each expert
    router_std: float = 0.02   # std of the router's entries
    rope_base: float = 10000.0
    norm_eps: float = 1e-6

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: shapes are the pages' 256-token canvas with N=48
# (report section 3.3) at several vocabulary / context sizes.
WORKLOADS = {
    "tiny_f32": Workload(
        name="tiny_f32", dtype=F32, vocab=256, d_model=64, n_q_heads=4, n_kv_heads=2,
        head_dim=16, canvas=16, n_steps=8, tied=True, prompt_tokens=32),
    "single_canvas": Workload(
        name="single_canvas", dtype=BF16, vocab=32768, d_model=2048, n_q_heads=16,
        n_kv_heads=4, head_dim=128, canvas=256, n_steps=48, prefix=1024),
    "full_vocab": Workload(
        name="full_vocab", dtype=BF16, vocab=262144, d_model=2816, n_q_heads=16,
        n_kv_heads=8, head_dim=256, canvas=256, n_steps=48, prefix=8192, stop_conf=0.9),
    "long_context": Workload(
        name="long_context", dtype=BF16, vocab=32768, d_model=2816, n_q_heads=16,
        n_kv_heads=8, head_dim=256, canvas=256, n_steps=48, prefix=65536, n_canvases=4),
    "ragged_batch": Workload(
        name="ragged_batch", dtype=BF16, vocab=65536, d_model=2048, n_q_heads=16,
        n_kv_heads=4, head_dim=128, canvas=256, n_steps=48, batch=8,
        prefix_range=(512, 16384), stop_conf=0.9, eos_id=1, n_eos_requests=2),
    # depth: two layers, each with a dense SwiGLU FFN of width 4 d, at the
    # single-canvas shapes
    "deep_canvas": Workload(
        name="deep_canvas", dtype=BF16, vocab=32768, d_model=2048, n_q_heads=16,
        n_kv_heads=4, head_dim=128, canvas=256, n_steps=48, prefix=1024, n_layers=2, d_ff=8192),
    # mixture of experts: two layers, each with a shared SwiGLU expert of
    # width d and 128 routed experts of width 256, 8 per token, at the
    # single-canvas shapes
    "moe_canvas": Workload(
        name="moe_canvas", dtype=BF16, vocab=32768, d_model=2048, n_q_heads=16,
        n_kv_heads=4, head_dim=128, canvas=256, n_steps=48, prefix=1024, n_layers=2, d_ff=2048,
        n_experts=128, top_k=8, d_expert=256),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (inputs hold no NaN)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP FP8 E4M3 ("fn") byte, round to nearest even, magnitudes
    beyond 448 saturated to 448 (inputs hold no NaN).  Normal values keep 3
    fraction bits (spacing 2^(e-3) for 2^e <= |x| < 2^(e+1)); below 2^-6 the
    spacing stays 2^-9 (subnormals)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, ex = np.frexp(a)                       # a = f 2^ex, 1/2 <= f < 1
    e = np.maximum(ex - 1, -6)                # exponent of the leading bit, subnormals pinned at -6
    q = np.rint(a / np.exp2(e - 3.0)) * np.exp2(e - 3.0)   # rint: ties to even
    q = np.minimum(q, 448.0)
    _, ex2 = np.frexp(q)
    e2 = np.maximum(ex2 - 1, -6)
    sub = q < 2.0 ** -6
    field_e = np.where(sub, 0, e2 + 7)
    mant = np.where(sub, q / 2.0 ** -9, q / np.exp2(e2 - 3.0) - 8.0)
    code = (field_e.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = np.where(q == 0, 0, code)
    return (code | np.where(np.signbit(np.asarray(x, dtype=np.float64)), 0x80, 0)).astype(np.uint8)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Inputs:
    """Materialised inputs.  Weights are uint16 bf16 bit patterns (bf16
    workloads) or float32 arrays (f32 workloads), in [out, in] layout."""
    wl: Workload
    embed: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray
    lm_head: np.ndarray                     # same object as embed when tied; uint8 e4m3 codes when lm_fp8
    lm_scale: Optional[np.ndarray] = None   # float32 [V] per-row scales of an FP8 head
    layers: Optional[list] = None           # deeper models / FFN / FP8 projections: per layer dict of wq, wk,
                                            # wv, wo[, wg, wu, wd] (FP8: uint8 codes, plus <name>_scale rows)
    prefix_len: list = field(default_factory=list)       # P_b per request
    prefix_k: list = field(default_factory=list)         # per request [Hkv, P_b, hd] (not for prompt workloads)
    prefix_v: list = field(default_factory=list)
    prompt: Optional[np.ndarray] = None     # int32 [n_prompt] for prefill workloads
    init_ids: np.ndarray = None             # int32 [B, C]
    init_committed: np.ndarray = None       # uint8 [B, C]


def _weights(rng, shape, dtype, std=0.02):
    w = rng.standard_normal(shape, dtype=np.float32)
    w *= np.float32(std)
    return f32_to_bf16_bits(w) if dtype == BF16 else w


def make_inputs(wl: Workload, seed: int = 0) -> Inputs:
    """Draw every input of ``wl`` from ``default_rng(seed)`` in the documented order."""
    rng = np.random.default_rng(seed)
    V, d, Hq, Hkv, hd = wl.vocab, wl.d_model, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    embed = _weights(rng, (V, d), wl.dtype)
    wq = _weights(rng, (Hq * hd, d), wl.dtype)
    wk = _weights(rng, (Hkv * hd, d), wl.dtype)
    wv = _weights(rng, (Hkv * hd, d), wl.dtype)
    wo = _weights(rng, (d, Hq * hd), wl.dtype)
    lm_scale = None
    if wl.lm_fp8:
        # codes of N(0, 16^2) values (using the e4m3 range), then per-row
        # scales lm_std / 16 * 2^u, u ~ U[-1/2, 1/2): the decoded head has
        # entries of spread ~ lm_std, as the bf16 head
        lm_head = f32_to_e4m3_bits(rng.standard_normal((V, d), dtype=np.float32) * np.float32(16.0))
        lm_scale = (np.float32(wl.lm_std / 16.0) *
                    np.exp2(rng.uniform(-0.5, 0.5, size=V)).astype(np.float32)).astype(np.float32)
    else:
        lm_head = embed if wl.tied else _weights(rng, (V, d), wl.dtype, wl.lm_std)
    inp = Inputs(wl, embed, wq, wk, wv, wo, lm_head, lm_scale)
    if wl.n_layers > 1 or wl.d_ff > 0:
        def ffn_weights():
            if wl.d_ff <= 0:
                return {}
            return dict(wg=_weights(rng, (wl.d_ff, d), wl.dtype), wu=_weights(rng, (wl.d_ff, d), wl.dtype),
                        wd=_weights(rng, (d, wl.d_ff), wl.dtype))
        inp.layers = [dict(wq=wq, wk=wk, wv=wv, wo=wo, **ffn_weights())]
        for _ in range(1, wl.n_layers):
            Ly = dict(wq=_weights(rng, (Hq * hd, d), wl.dtype), wk=_weights(rng, (Hkv * hd, d), wl.dtype),
                      wv=_weights(rng, (Hkv * hd, d), wl.dtype), wo=_weights(rng, (d, Hq * hd), wl.dtype))
            Ly.update(ffn_weights())
            inp.layers.append(Ly)
    if wl.proj_fp8:
        # the same bf16 weights, quantised row by row (no extra draws): scale
        # = max |w| / 448 over the row, codes = e4m3(w / scale) (RNE)
        if inp.layers is None:
            inp.layers = [dict(wq=wq, wk=wk, wv=wv, wo=wo)]
        inp.layers = [{k2: v2 for k, w in Ly.items() for k2, v2 in _fp8_rows(k, w).items()} for Ly in inp.layers]
    B, C = wl.batch, wl.canvas
    inp.init_ids = np.full((B, C), wl.mask_id, dtype=np.int32)
    inp.init_committed = np.zeros((B, C), dtype=np.uint8)
    if wl.prompt_tokens > 0:
        # uniform ids in [0, V-1): the MASK id never appears in the prompt
        inp.prompt = rng.integers(0, V - 1, size=wl.prompt_tokens).astype(np.int32)
        inp.prefix_len = [wl.prompt_tokens] * B
        _candidates(rng, wl, inp)
        _experts(rng, wl, inp)
        return inp
    if wl.prefix_range is not None:
        lo, hi = wl.prefix_range
        inp.prefix_len = [int(p) for p in rng.integers(lo, hi + 1, size=B)]
    else:
        inp.prefix_len = [wl.prefix] * B
    if wl.n_eos_requests > 0:
        reqs = rng.choice(B, wl.n_eos_requests, replace=False)
        poss = rng.integers(0, C, size=wl.n_eos_requests)
        for b, p in zip(reqs, poss):
            inp.init_ids[b, p] = wl.eos_id
            inp.init_committed[b, p] = 1
    for b in range(B):
        shape = (Hkv, inp.prefix_len[b], hd)
        ks, vs = [], []
        for _ in range(wl.n_layers):
            kf = rng.standard_normal(shape, dtype=np.float32)
            vf = rng.standard_normal(shape, dtype=np.float32)
            ks.append(f32_to_bf16_bits(kf) if wl.dtype == BF16 else kf)
            vs.append(f32_to_bf16_bits(vf) if wl.dtype == BF16 else vf)
        # one layer: the arrays themselves; deeper: a list per layer
        inp.prefix_k.append(ks[0] if wl.n_layers == 1 else ks)
        inp.prefix_v.append(vs[0] if wl.n_layers == 1 else vs)
    _candidates(rng, wl, inp)
    _experts(rng, wl, inp)
    return inp


def _experts(rng, wl: Workload, inp: Inputs):
    """Routed experts of every layer (router [E, d], gate / up [E, d_e, d],
    down [E, d, d_e]), drawn last so that the other inputs do not change."""
    if wl.n_experts <= 0:
        return
    E, d, de = wl.n_experts, wl.d_model, wl.d_expert
    for Ly in inp.layers:
        Ly["wr"] = _weights(rng, (E, d), wl.dtype, wl.router_std)
        Ly["wge"] = _weights(rng, (E, de, d), wl.dtype)
        Ly["wue"] = _weights(rng, (E, de, d), wl.dtype)
        Ly["wde"] = _weights(rng, (E, d, de), wl.dtype)


def _fp8_rows(name: str, w: np.ndarray) -> dict:
    """{name: e4m3 codes, name_scale: fp32 per-row scales} of a bf16 weight."""
    f = bf16_bits_to_f32(w)
    amax = np.abs(f).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    return {name: f32_to_e4m3_bits(f / scale[:, None]), name + "_scale": scale}


def _candidates(rng, wl: Workload, inp: Inputs):
    """Candidate canvas: the uncommitted positions start as uniform draws
    over [0, V-1) (MASK excluded), drawn last so that the other inputs of a
    workload do not change with the fill mode."""
    if not wl.fill:
        return
    for b in range(wl.batch):
        draw = rng.integers(0, wl.vocab - 1, size=wl.canvas).astype(np.int32)
        open_ = inp.init_committed[b] == 0
        inp.init_ids[b, open_] = draw[open_]


def workload(name: str, **overrides) -> Workload:
    """Registered workload, optionally with shapes overridden (small parity cases)."""
    wl = WORKLOADS[name]
    return wl.with_(**overrides) if overrides else wl
