"""CPU oracle of one block-discrete-diffusion denoising step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
calls it.  It shares no code with the HIP library: it decodes its own inputs,
rounds with its own bf16 routine and recomputes every stage from the
definitions below, in float64, one plain step after another.

Sources (the pages this follows):
  [TR1] DiffusionGemma Technical Report, part 1: Abstract, section 1
        (causal context encoding + bidirectional attention inside a 256-token
        canvas), section 2.1 (the canvas x_t over vocabulary V of length C).
  [TR3] DiffusionGemma Technical Report, part 3: section 3.3 (adaptive
        stopping, N=48 budget), section 3.4 eqs. (7)-(10) (efficiency
        metrics), section 4 (block-diagonal mask, clean context through the
        encoder KV cache, p_theta = softmax of the output logits, eq. (11)),
        section 5 (adaptive stop triggered by low predictive entropy,
        "Improved speed-to-intelligence Pareto frontier": a collapse of the
        entropy fires the stop early).
  [BLOG] "Google Releases DiffusionGemma: When Language Models No Longer Write
        Only Left to Right", section "Once Written, a Prefix Becomes History":
        high-confidence positions lock first, a finished canvas is written into
        the KV cache as a read-only prefix.

Where the pages are silent the oracle takes these readings (the HIP path takes
the same ones):
  * absorbing MASK canvas: uncommitted positions are fed as MASK = V-1 and
    the sampler never proposes MASK (its logit is -inf);
  * one pre-norm attention layer with RMSNorm of unit gain folded into a row
    scale r = (mean(x^2) + eps)^-1/2 applied to the projection outputs, RoPE
    (half-split pairs, base 1e4) on q and k at absolute positions, GQA with
    contiguous head groups, residual h = e + o Wo^T, logits z = r_h (h Wlm^T);
  * deeper models ([TR1] Abstract and section 1: the backbone is a stack of
    transformer layers; [TR3] section 6 names the FFN among the step's
    costs): L such layers, each optionally followed by a pre-norm dense
    SwiGLU feed-forward block x <- x + (silu(r x Wg^T) * (r x Wu^T)) Wd^T
    (r the row scale of x), every layer with its own KV cache; the logits
    read the residual stream after the last layer;
  * the append pass encodes the finished canvas as context: causal
    attention ([TR1] section 1: context encoding is causal), canvas position
    i seeing the prefix and canvas positions 0..i; with one layer the K/V
    rows do not depend on attention at all;
  * confidence = max softmax probability; commit k_s = ceil(|U|/(N-s+1)) of
    the uncommitted positions, ranked by confidence (ties: lower position);
    argmax ties go to the lower token id; unselected positions are re-masked;
  * adaptive stop: the canvas stops when every uncommitted position left
    out of this step's selection is already sure; two readings of "sure":
    confidence >= tau, or predictive entropy -sum_v p_v ln p_v (nats, of the
    position's softmax over the vocabulary) <= h_max ([TR3] section 5 names
    the entropy as the trigger but gives no threshold or aggregation; the
    per-position bound over every position left open is the reading that
    matches the confidence rule);
  * two sampler variants (off by default):
      - threshold commit: every uncommitted position whose confidence is
        >= tau_c is committed, and at least the schedule's k_s most confident
        ones (so the canvas still ends by step N);
      - candidate canvas: an uncommitted position is fed its current
        candidate token instead of MASK: the caller's initial id (a uniform
        draw over the vocabulary, the multinomial prior of [BLOG] section
        "Text Cannot Directly Take Gaussian Noise"), then the greedy token it
        received at the previous step (the interim canvas of [BLOG] section
        "Once Written, a Prefix Becomes History", where an interim digit is
        corrected by the next forward pass);
  * temperature sampling (an option; [TR3] section 5, "Training setup": the
    online teacher samples with mild temperature annealing): at step s of N
    the temperature is T_s = T0 + (T1 - T0)(s - 1)/(N - 1); an open position
    proposes the Gumbel-max sample argmax_v z_v / T_s + g_v (lowest id on a
    tie) instead of its greedy token, and its confidence is the probability
    p_theta of that sample (the max probability when the sample is the
    greedy token); g_v = -ln(-ln u_v), u_v the 24 top bits (plus a half) of a
    Philox4x64-10 output with key (seed, 0) and counter (v >> 2, position,
    step, request), word v & 3 (Salmon, Moraes, Dror and Shaw, SC'11);
  * FP8 vocabulary head (an option; the pages serve the model in FP8 but
    give no format or scale convention): the head is stored as OCP E4M3
    codes with one fp32 scale per vocabulary row, z_v = r_h s_v
    (h . e4m3(W_v)); the activations stay as in the bf16 model;
  * mixture of experts (an option; [TR3] section 6 names the MoE layer, its
    experts chosen per token, and a shared expert among the step's costs;
    the pages give no router or expert shapes): a layer's FFN is then a
    shared expert (the dense SwiGLU block above) plus E routed SwiGLU experts
    on the same normed input a = r x: router logits l = a Wr^T, the top_k
    experts by logit (ties to the lower expert id), gates g = softmax of the
    selected logits, x <- x + shared(a) + sum_j g_j expert_{e_j}(a), each
    expert's activation held like the dense one;
  * FP8 projections (an option, same convention): every layer's projection
    weights (Wq, Wk, Wv, Wo and the FFN's Wg, Wu, Wd) are OCP E4M3 codes
    with one fp32 scale per output row, W[n, :] = s_n e4m3(codes[n, :]);
    the activations stay as in the bf16 model;
  * precision points: the canvas K / V rows are rounded to the cache's type
    (the model dtype, bf16 RNE or fp32), since they are stored in the cache;
    the step's own activations q, o, the residual stream x (h after the
    last layer) and the FFN activation are held in fp32 and enter their
    products as held (the pages fix no operand precision; p_theta is the
    softmax of the logits of h, [TR3] section 4); everything else is float64.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------

def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values (bf16 is the top half of fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits and fp32's exponent range, so a value with
    binary exponent e (x = m 2^e, 1/2 <= |m| < 1) is rounded to a multiple of
    2^(e-8); below the smallest normal (2^-126) the spacing stays 2^-133.
    np.rint rounds half-way cases to even.  Values beyond the largest finite
    bf16 become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)
    quantum = np.ldexp(1.0, e - 8)
    y = np.rint(x / quantum) * quantum
    big = np.abs(y) > 3.3895313892515355e38        # largest finite bf16
    return np.where(big, np.copysign(np.inf, x), y)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 (the "fn" variant: no infinities) bytes -> exact float64.
    Bit layout s eeee mmm, exponent bias 7: e = 0 encodes the subnormals
    (m / 8) 2^-6, e = 1..15 the normals (1 + m / 8) 2^(e - 7); the two codes
    with e = 15 and m = 7 are NaN, so the largest finite value is 448."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    mant = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, mant / 8.0 * 2.0 ** -6, (1.0 + mant / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)
    return sign * mag


def round_f16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest IEEE binary16 value, ties to even
    (numpy's float64 -> float16 conversion; subnormals below 2^-14, +-inf
    beyond 65504)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float64 tensor to the storage type of the path.  "f64" keeps
    every value exact; the pins use it to compare stages with library code."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f16":
        return round_f16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


def held(dtype: str) -> str:
    """Type in which a step holds its own activations (q, o, h): fp32, or
    exact values for the "f64" pin models."""
    return "f64" if dtype == "f64" else "f32"


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_decode(a)
    return np.asarray(a).astype(np.float64)


def dequant_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """FP8 projection weight: row n is s_n times the E4M3 values of its codes."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float32).astype(np.float64)[:, None]


# ----------------------------------------------------------------------------
# model
# ----------------------------------------------------------------------------

@dataclass
class Model:
    dtype: str
    V: int
    d: int
    Hq: int
    Hkv: int
    hd: int
    mask_id: int
    eos_id: int
    rope_base: float
    eps: float
    E: np.ndarray      # [V, d]
    Wq: np.ndarray     # [Hq*hd, d]
    Wk: np.ndarray     # [Hkv*hd, d]
    Wv: np.ndarray     # [Hkv*hd, d]
    Wo: np.ndarray     # [d, Hq*hd]
    Wlm: np.ndarray    # [V, d]; with an FP8 head the decoded e4m3 values (unscaled)
    lm_scale: Optional[np.ndarray] = None   # [V] per-row scale of an FP8 head, else None
    layers: Optional[list] = None           # [L] Layer; None: one layer of Wq, Wk, Wv, Wo, no FFN


@dataclass
class Layer:
    """One transformer layer: attention projections and, when Wg is given, a
    dense SwiGLU feed-forward block ([d_ff, d], [d_ff, d], [d, d_ff]); when
    Wr is given also E routed experts: router [E, d], expert gate / up
    [E, d_e, d], down [E, d, d_e], top_k experts per token."""
    Wq: np.ndarray
    Wk: np.ndarray
    Wv: np.ndarray
    Wo: np.ndarray
    Wg: Optional[np.ndarray] = None
    Wu: Optional[np.ndarray] = None
    Wd: Optional[np.ndarray] = None
    Wr: Optional[np.ndarray] = None
    Wge: Optional[np.ndarray] = None
    Wue: Optional[np.ndarray] = None
    Wde: Optional[np.ndarray] = None
    top_k: int = 0


def layer_list(m: Model) -> list:
    if m.layers is not None:
        return m.layers
    return [Layer(m.Wq, m.Wk, m.Wv, m.Wo)]


def model_from_inputs(inp) -> Model:
    wl = inp.wl
    dt = wl.dtype
    E = decode(inp.embed, dt)
    scale = None
    if getattr(wl, "lm_fp8", False):
        Wlm = e4m3_decode(inp.lm_head)
        scale = np.asarray(inp.lm_scale, dtype=np.float32).astype(np.float64)
    else:
        Wlm = E if wl.tied else decode(inp.lm_head, dt)
    layers = None
    if getattr(inp, "layers", None):
        fp8 = getattr(wl, "proj_fp8", False)

        def weight(Ly, name):
            w = Ly.get(name)
            if w is None:
                return None
            return dequant_rows(w, Ly[name + "_scale"]) if fp8 else decode(w, dt)
        layers = [Layer(*[weight(Ly, n) for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")],
                        *[decode(Ly[n], dt) if n in Ly else None for n in ("wr", "wge", "wue", "wde")],
                        getattr(wl, "top_k", 0)) for Ly in inp.layers]
    m = Model(dt, wl.vocab, wl.d_model, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
              wl.vocab - 1, wl.eos_id, float(wl.rope_base), float(wl.norm_eps),
              E, decode(inp.wq, dt), decode(inp.wk, dt), decode(inp.wv, dt),
              decode(inp.wo, dt), Wlm, scale, layers)
    if layers is not None:
        # layer 0 is the one the top-level fields describe
        m.Wq, m.Wk, m.Wv, m.Wo = layers[0].Wq, layers[0].Wk, layers[0].Wv, layers[0].Wo
    return m


# ----------------------------------------------------------------------------
# stages of one forward pass over a canvas
# ----------------------------------------------------------------------------

def canvas_input_ids(ids: np.ndarray, committed: np.ndarray, mask_id: int, fill: int = 0) -> np.ndarray:
    """Canvas fed to the network ([TR1] section 2.1, the canvas x_t).
    fill 0 (absorbing mask): committed ids as they are, every other slot MASK.
    fill 1 (candidate canvas): every slot its current id; an uncommitted
    slot's id is its candidate token."""
    if fill:
        return np.asarray(ids, dtype=np.int64).copy()
    return np.where(committed != 0, ids, mask_id).astype(np.int64)


def rms_scale(x: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm with unit gain as a per-row scale: (mean_j x_j^2 + eps)^(-1/2)."""
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)


def rope_cos_sin(positions: np.ndarray, hd: int, base: float):
    """Rotation of pair j at absolute position p: angle p * base^(-2j/hd).
    Angle, cos and sin are computed in float64; cos and sin are then held in
    float32, the precision the tables of the HIP path keep."""
    j = np.arange(hd // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * j / hd)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    c = np.cos(ang).astype(np.float32).astype(np.float64)
    s = np.sin(ang).astype(np.float32).astype(np.float64)
    return c, s


def rotate(x: np.ndarray, c: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Half-split rotary embedding of x [n, H, hd]: pair (j, j + hd/2)."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    c = c[:, None, :]
    s = s[:, None, :]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def project_qkv(m: Model, tok: np.ndarray, positions: np.ndarray):
    """Pre-norm QKV projection of token ids at absolute positions.

    e = E[tok]; r = rms_scale(e); q = RoPE(r * e Wq^T), k = RoPE(r * e Wk^T),
    v = r * e Wv^T.  k and v are rounded to the cache type (the model dtype);
    q is held in fp32.  Returns e too (the residual stream input)."""
    e = m.E[tok]
    r = rms_scale(e, m.eps)[:, None]
    n = len(tok)
    q = (r * (e @ m.Wq.T)).reshape(n, m.Hq, m.hd)
    k = (r * (e @ m.Wk.T)).reshape(n, m.Hkv, m.hd)
    v = (r * (e @ m.Wv.T)).reshape(n, m.Hkv, m.hd)
    c, s = rope_cos_sin(positions, m.hd, m.rope_base)
    q = store(rotate(q, c, s), held(m.dtype))
    k = store(rotate(k, c, s), m.dtype)
    v = store(v, m.dtype)
    return e, q, k, v


def project_qkv_x(m: Model, Ly: Layer, x: np.ndarray, positions: np.ndarray):
    """The same pre-norm projection of layer Ly applied to a residual stream
    x [n, d] (held values): r = rms_scale(x); q = RoPE(r x Wq^T), k =
    RoPE(r x Wk^T), v = r x Wv^T; k, v rounded to the cache type, q held."""
    r = rms_scale(x, m.eps)[:, None]
    n = x.shape[0]
    q = (r * (x @ Ly.Wq.T)).reshape(n, m.Hq, m.hd)
    k = (r * (x @ Ly.Wk.T)).reshape(n, m.Hkv, m.hd)
    v = (r * (x @ Ly.Wv.T)).reshape(n, m.Hkv, m.hd)
    c, s = rope_cos_sin(positions, m.hd, m.rope_base)
    return store(rotate(q, c, s), held(m.dtype)), store(rotate(k, c, s), m.dtype), store(v, m.dtype)


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x)."""
    return x / (1.0 + np.exp(-x))


def ffn(m: Model, Ly: Layer, x: np.ndarray, force: Optional[np.ndarray] = None) -> np.ndarray:
    """Pre-norm dense SwiGLU block with its residual: with r = rms_scale(x),
    a = silu(r x Wg^T) * (r x Wu^T) (held), x + a Wd^T (held).  A layer with
    experts adds their output (moe) to the shared block's before the
    residual.  force: see moe."""
    r = rms_scale(x, m.eps)[:, None]
    a = store(silu(r * (x @ Ly.Wg.T)) * (r * (x @ Ly.Wu.T)), held(m.dtype))
    delta = a @ Ly.Wd.T
    if Ly.Wr is not None:
        delta = delta + moe(m, Ly, x, force)
    return store(x + delta, held(m.dtype))


# Near-tie band of the router's top-k: the same absolute band as the step's
# token decisions (a margin below it can flip under the 16-bit operands of
# either side's arithmetic).
ROUTE_GAP = 1e-3


def moe_route(m: Model, Ly: Layer, x: np.ndarray):
    """Router of a layer with experts, on the normed input a = r x: logits
    l = a Wr^T [n, E]; each token's top_k experts in (logit desc, expert id
    asc) order; gates = softmax of their logits.  Also the margin l_(k) -
    l_(k+1) between the last chosen and the first left out (inf when every
    expert is chosen).  Returns (sel [n, k], gates [n, k], logits, margin)."""
    r = rms_scale(x, m.eps)[:, None]
    logits = r * (x @ Ly.Wr.T)
    n, E = logits.shape
    k = Ly.top_k
    order = np.array([sorted(range(E), key=lambda e: (-logits[t, e], e)) for t in range(n)], dtype=np.int64)
    sel = order[:, :k]
    ls = np.take_along_axis(logits, sel, axis=1)
    g = np.exp(ls - ls[:, :1])
    g /= g.sum(axis=1, keepdims=True)
    if k < E:
        margin = ls[:, -1] - np.take_along_axis(logits, order[:, k:k + 1], axis=1)[:, 0]
    else:
        margin = np.full(n, np.inf)
    return sel, g, logits, margin


def moe(m: Model, Ly: Layer, x: np.ndarray, force: Optional[np.ndarray] = None) -> np.ndarray:
    """Routed experts' output sum_j g_j expert_{e_j}(a), a = r x, expert_e(a)
    = (silu(a Wge[e]^T) * (a Wue[e]^T)) (held) Wde[e]^T.
    force [n, k]: a selection made elsewhere (by another evaluation of the
    same logits), taken for the tokens whose margin is below ROUTE_GAP; it
    must then agree with this router's order except among experts whose
    logits lie within ROUTE_GAP of the last chosen one.  Its gates are the
    softmax of this router's logits of the forced experts."""
    sel, g, logits, margin = moe_route(m, Ly, x)
    if force is not None:
        force = np.asarray(force, dtype=np.int64)
        for t in np.flatnonzero(margin < ROUTE_GAP):
            f = force[t]
            if set(f.tolist()) == set(sel[t].tolist()):
                continue
            cut = logits[t, sel[t, -1]]
            for e in set(f.tolist()) ^ set(sel[t].tolist()):
                assert abs(logits[t, e] - cut) < ROUTE_GAP, "forced routing outside the near-tie band"
            ls = logits[t, f]
            o = np.array(sorted(range(len(f)), key=lambda j: (-ls[j], f[j])))
            sel[t] = f[o]
            gt = np.exp(ls[o] - ls[o].max())
            g[t] = gt / gt.sum()
    a = rms_scale(x, m.eps)[:, None] * x
    y = np.zeros_like(x)
    for e in np.unique(sel):
        tt, jj = np.nonzero(sel == e)
        h = store(silu(a[tt] @ Ly.Wge[e].T) * (a[tt] @ Ly.Wue[e].T), held(m.dtype))
        y[tt] += g[tt, jj][:, None] * (h @ Ly.Wde[e].T)
    return y


def attend(m: Model, q: np.ndarray, K: np.ndarray, Vv: np.ndarray, causal_from: Optional[int] = None) -> np.ndarray:
    """Block-bidirectional attention ([TR1] section 1; [TR3] section 4).

    q [n, Hq, hd]; K, Vv [Hkv, L, hd] hold the read-only prefix rows followed by
    the canvas rows.  Every canvas query sees every prefix key and every canvas
    key (no mask inside the canvas).  Query head h reads KV head
    h // (Hq / Hkv).  Scores are scaled by hd^-1/2; exact softmax in float64.
    The output is held in fp32 whatever the model dtype.
    causal_from = P (context encoding, [TR1] section 1): query i sees keys
    0 .. P + i only.
    """
    G = m.Hq // m.Hkv
    n = q.shape[0]
    o = np.empty((n, m.Hq, m.hd))
    scale = 1.0 / math.sqrt(m.hd)
    for h in range(m.Hq):
        g = h // G
        s = (q[:, h, :] @ K[g].T) * scale
        if causal_from is not None:
            i = np.arange(n)[:, None]
            j = np.arange(K.shape[1])[None, :]
            s = np.where(j <= causal_from + i, s, NEG_INF)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        o[:, h, :] = p @ Vv[g]
    return store(o, held(m.dtype))


def residual_out(m: Model, e: np.ndarray, o: np.ndarray, Wo: Optional[np.ndarray] = None) -> np.ndarray:
    """h = e + o Wo^T, held in fp32 (Wo: the layer's, default the model's)."""
    n = e.shape[0]
    Wo = m.Wo if Wo is None else Wo
    return store(e + o.reshape(n, m.Hq * m.hd) @ Wo.T, held(m.dtype))


def vocab_logits(m: Model, h: np.ndarray, chunk: int = 16384) -> np.ndarray:
    """z = rms_scale(h) * (h Wlm^T) with the MASK column set to -inf; with an
    FP8 head, z_v = rms_scale(h) * s_v * (h . e4m3(W_v)).  h enters as the
    step holds it.

    p_theta is the softmax of these logits ([TR3] section 4, eq. (11)).  The
    product is evaluated in vocabulary chunks only to bound memory; each
    entry is the same full dot product."""
    r = rms_scale(h, m.eps)[:, None]
    z = np.empty((h.shape[0], m.V))
    for v0 in range(0, m.V, chunk):
        v1 = min(m.V, v0 + chunk)
        z[:, v0:v1] = r * (h @ m.Wlm[v0:v1].T)
        if m.lm_scale is not None:
            z[:, v0:v1] *= m.lm_scale[v0:v1]
    z[:, m.mask_id] = NEG_INF
    return z


def sampler_stats(z: np.ndarray) -> dict:
    """Per-row statistics of softmax(z): greedy token, confidence and margins.

    argmax: lowest id attaining the maximum m; m2: second largest logit (equal
    to m on a tie); lse = m + ln sum exp(z - m); confidence = exp(m - lse), the
    largest softmax probability; entropy = -sum_v p_v ln p_v over the ids with
    p_v > 0 (a -inf logit has p_v = 0 and adds nothing)."""
    n, V = z.shape
    argmax = np.argmax(z, axis=1)                # first index of the maximum
    m = z[np.arange(n), argmax]
    z2 = z.copy()
    z2[np.arange(n), argmax] = NEG_INF
    m2 = z2.max(axis=1)
    ssum = np.exp(z - m[:, None]).sum(axis=1)
    lse = m + np.log(ssum)
    logconf = m - lse
    p = np.exp(z - lse[:, None])
    logp = np.where(p > 0, z - lse[:, None], 0.0)
    entropy = -(p * logp).sum(axis=1)
    return dict(argmax=argmax.astype(np.int64), m=m, m2=m2, lse=lse,
                logconf=logconf, conf=np.exp(logconf), sumexp=ssum, entropy=entropy)


def softmax_rows(z: np.ndarray) -> np.ndarray:
    zz = z - z.max(axis=1, keepdims=True)
    p = np.exp(zz)
    return p / p.sum(axis=1, keepdims=True)


# ----------------------------------------------------------------------------
# temperature sampling: counter-based random numbers and the Gumbel-max draw
# ----------------------------------------------------------------------------

_PH_M = (np.uint64(0xD2E7470EE14C6C93), np.uint64(0xCA5A826395121157))   # round multipliers
_PH_W = (np.uint64(0x9E3779B97F4A7C15), np.uint64(0xBB67AE8584CAA73B))   # key increments (golden ratio, sqrt 3)
_M32, _S32 = np.uint64(0xFFFFFFFF), np.uint64(32)


def _mulhilo64(a, b):
    """High and low 64-bit halves of the 128-bit product a * b (uint64
    arrays), from four 32 x 32-bit partial products."""
    a = np.asarray(a, np.uint64)
    b = np.asarray(b, np.uint64)
    al, ah, bl, bh = a & _M32, a >> _S32, b & _M32, b >> _S32
    ll, hl, lh, hh = al * bl, ah * bl, al * bh, ah * bh
    cross = (ll >> _S32) + (hl & _M32) + (lh & _M32)
    lo = (ll & _M32) | ((cross & _M32) << _S32)
    hi = hh + (hl >> _S32) + (lh >> _S32) + (cross >> _S32)
    return hi, lo


def philox4x64_10(counter, key):
    """Philox4x64 with 10 rounds: each round multiplies words 0 and 2 by the
    round multipliers and recombines the halves with words 1, 3 and the key;
    the key advances by the Weyl increments between rounds.  counter: four
    uint64 arrays (broadcast), key: two uint64.  Returns four uint64 arrays."""
    c0, c1, c2, c3 = [np.asarray(x, np.uint64) for x in counter]
    k0, k1 = np.uint64(key[0]), np.uint64(key[1])
    with np.errstate(over="ignore"):
        for r in range(10):
            if r:
                k0, k1 = k0 + _PH_W[0], k1 + _PH_W[1]
            h0, l0 = _mulhilo64(_PH_M[0], c0)
            h1, l1 = _mulhilo64(_PH_M[1], c2)
            c0, c1, c2, c3 = h1 ^ c1 ^ k0, l1, h0 ^ c3 ^ k1, l0
    return c0, c1, c2, c3


def gumbel_noise(seed: int, b: int, step: int, positions, V: int) -> np.ndarray:
    """g [len(positions), V]: -ln(-ln u) with u = (top 24 bits + 1/2) / 2^24 of
    word v & 3 of Philox4x64-10(counter (v >> 2, position, step, b), key
    (seed, 0))."""
    pos = np.asarray(positions, dtype=np.uint64)[:, None]
    v = np.arange(V, dtype=np.uint64)[None, :]
    words = philox4x64_10((v >> np.uint64(2), pos, np.uint64(step), np.uint64(b)),
                          (np.uint64(seed & 0xFFFFFFFFFFFFFFFF), np.uint64(0)))
    sel = (v & np.uint64(3)).astype(np.int64) + np.zeros(pos.shape, dtype=np.int64)
    w = np.choose(sel, words)
    u = ((w >> np.uint64(40)).astype(np.float64) + 0.5) / 2.0 ** 24
    return -np.log(-np.log(u))


def temperature_at(s: int, N: int, t0: float, t1: float) -> float:
    """T_s, linear in the step from T0 at step 1 to T1 at step N."""
    return float(t0) if N <= 1 else float(t0) + (float(t1) - float(t0)) * (s - 1) / (N - 1)


def sample_stats(st: dict, z: np.ndarray, T: float, seed: int, b: int, step: int, positions) -> dict:
    """Gumbel-max draw at temperature T for rows z [n, V] at canvas positions
    ``positions`` of request b: sample = argmax_v z_v / T + g_v (lowest id on
    a tie), its log-probability under p_theta = softmax(z) and the gap of the
    two largest perturbed values (the draw's own near-tie margin)."""
    g = gumbel_noise(seed, b, step, positions, z.shape[1])
    key = z / T + g
    sample = np.argmax(key, axis=1)
    n = np.arange(z.shape[0])
    k1 = key[n, sample]
    k2 = key.copy()
    k2[n, sample] = NEG_INF
    out = dict(st)
    out["sample"] = sample.astype(np.int64)
    out["sample_logconf"] = z[n, sample] - st["lse"]
    out["key_gap"] = k1 - k2.max(axis=1)
    return out


# ----------------------------------------------------------------------------
# sampler: commit / re-mask / adaptive stop
# ----------------------------------------------------------------------------

def commit_count(n_uncommitted: int, s: int, N: int) -> int:
    """Positions committed at step s (1-based) of an N-step budget:
    ceil(|U| / (N - s + 1)); at s = N this is |U|, so the canvas always ends."""
    return -(-n_uncommitted // (N - s + 1))


@dataclass
class CommitResult:
    ids: np.ndarray
    committed: np.ndarray
    selected: np.ndarray        # bool [C]: committed at this step
    k: int                      # scheduled commit count
    stopped: bool               # adaptive stop fired
    done: bool
    n_valid: int
    cutoff_margin: float        # logconf(k-th ranked) - logconf((k+1)-th ranked)
    stop_margin: float          # min over unselected of (logconf - ln tau),
                                # or of (h_max - entropy) under the entropy stop
    commit_margin: float = math.inf   # threshold rule: min over U of |logconf - ln tau_c|


def commit(ids, committed, st: dict, s: int, N: int, stop_conf: Optional[float],
           eos_id: int, commit_conf: Optional[float] = None, fill: int = 0,
           stop_entropy: Optional[float] = None) -> CommitResult:
    """One sampler update of a single canvas after the forward pass of step s.

    High-confidence positions lock first ([BLOG], "Once Written, a Prefix
    Becomes History"); the rest are re-masked (fill 0) or take their new
    greedy token as candidate (fill 1).  With adaptive stopping the canvas
    ends as soon as every remaining position is already confident ([TR3]
    sections 3.3 and 5): confidence >= stop_conf, or entropy <= stop_entropy
    (at most one of the two is given).  commit_conf (threshold rule): every
    uncommitted position with confidence >= commit_conf is committed as well."""
    if stop_conf is not None and stop_entropy is not None:
        raise ValueError("give stop_conf or stop_entropy, not both")
    C = len(ids)
    conf = st["conf"]
    logconf = st["logconf"]
    U = [i for i in range(C) if committed[i] == 0]
    nU = len(U)
    k = commit_count(nU, s, N) if nU else 0
    ranked = sorted(U, key=lambda i: (-conf[i], i))
    commit_margin = math.inf
    if commit_conf is not None and nU > 0:
        tau_c = float(np.float32(commit_conf))
        ln_c = math.log(tau_c) if tau_c > 0 else -math.inf
        above = sum(1 for i in U if conf[i] >= tau_c)
        commit_margin = float(min(abs(logconf[i] - ln_c) for i in U))
        k = max(k, above)
    sel = ranked[:k]
    rest = ranked[k:]
    cutoff = math.inf
    if 0 < k < nU:
        cutoff = float(logconf[ranked[k - 1]] - logconf[ranked[k]])
    stop_margin = math.inf
    stopped = False
    if stop_conf is not None and nU > 0:
        tau = float(np.float32(stop_conf))
        if rest:
            ln_tau = math.log(tau) if tau > 0 else -math.inf
            stop_margin = float(min(logconf[i] for i in rest) - ln_tau)
        if all(conf[i] >= tau for i in rest):
            stopped = len(rest) > 0
            sel = ranked
    if stop_entropy is not None and nU > 0:
        h_max = float(np.float32(stop_entropy))
        ent = st["entropy"]
        if rest:
            stop_margin = float(h_max - max(ent[i] for i in rest))
        if all(ent[i] <= h_max for i in rest):
            stopped = len(rest) > 0
            sel = ranked
    new_ids = np.array(ids, dtype=np.int64).copy()
    new_c = np.array(committed, dtype=np.uint8).copy()
    selected = np.zeros(C, dtype=bool)
    for i in sel:
        new_ids[i] = st["argmax"][i]
        new_c[i] = 1
        selected[i] = True
    if fill:
        for i in U:
            if not selected[i]:
                new_ids[i] = st["argmax"][i]       # the position's new candidate
    done = bool(np.all(new_c != 0))
    n_valid = valid_length(new_ids, eos_id) if done else C
    return CommitResult(new_ids, new_c, selected, k, stopped, done, n_valid, cutoff, stop_margin, commit_margin)


def valid_length(ids: np.ndarray, eos_id: int) -> int:
    """C_k: all C tokens, or the tokens before the first end-of-sequence id
    ([TR3] section 3.4)."""
    if eos_id < 0:
        return len(ids)
    hits = np.flatnonzero(np.asarray(ids) == eos_id)
    return int(hits[0]) if len(hits) else len(ids)


# ----------------------------------------------------------------------------
# one request: cache, step, append
# ----------------------------------------------------------------------------

class Request:
    """A single canvas with its read-only KV cache (prefix rows only)."""

    def __init__(self, m: Model, K, Vv, ids, committed):
        self.m = m
        # per layer [Hkv, P, hd] float64, keys post-RoPE (one array: one layer)
        self.Ks = list(K) if isinstance(K, (list, tuple)) else [K]
        self.Vs = list(Vv) if isinstance(Vv, (list, tuple)) else [Vv]
        self.ids = np.array(ids, dtype=np.int64)
        self.committed = np.array(committed, dtype=np.uint8)
        self.step = 0
        self.done = False
        self.n_steps = 0
        self.n_valid = len(self.ids)

    @property
    def K(self) -> np.ndarray:
        return self.Ks[0]

    @property
    def V(self) -> np.ndarray:
        return self.Vs[0]

    @property
    def P(self) -> int:
        return self.Ks[0].shape[1]


def forward(m: Model, req: Request, fill: int = 0, routes: Optional[list] = None):
    """Network forward of the current canvas of ``req`` (one denoising pass):
    every layer attends block-bidirectionally over its own prefix rows and the
    canvas rows of this pass, then its FFN (if any); the logits read the last
    residual stream.  Returns layer 0's k, v, the last layer's q, o, the
    per-layer lists ks, vs, os, the residual h after the last layer and the
    logits.  routes: per layer, a forced expert selection (see moe) or None."""
    C = len(req.ids)
    tok = canvas_input_ids(req.ids, req.committed, m.mask_id, fill)
    pos = req.P + np.arange(C)
    e = m.E[tok]
    x = e
    out = dict(tok=tok, e=e, ks=[], vs=[], os=[])
    for l, Ly in enumerate(layer_list(m)):
        q, k, v = project_qkv_x(m, Ly, x, pos)
        K = np.concatenate([req.Ks[l], k.transpose(1, 0, 2)], axis=1)
        Vv = np.concatenate([req.Vs[l], v.transpose(1, 0, 2)], axis=1)
        o = attend(m, q, K, Vv)
        x = residual_out(m, x, o, Ly.Wo)
        if Ly.Wr is not None:
            sel_l, _, _, margin_l = moe_route(m, Ly, x)
            out.setdefault("route_margin", []).append(margin_l)
            out.setdefault("route_sel", []).append(sel_l)
        if Ly.Wg is not None:
            x = ffn(m, Ly, x, routes[l] if routes is not None else None)
        if l == 0:
            out.update(k=k, v=v)
        out.update(q=q, o=o)                   # the last layer's (what a device dump holds)
        out["ks"].append(k)
        out["vs"].append(v)
        out["os"].append(o)
    out["h"] = x
    out["z"] = vocab_logits(m, x)
    return out


def denoise_step(m: Model, req: Request, N: int, stop_conf: Optional[float],
                 commit_conf: Optional[float] = None, fill: int = 0,
                 stop_entropy: Optional[float] = None, temp: Optional[tuple] = None, b: int = 0,
                 routes: Optional[list] = None):
    """Step s = req.step + 1: forward, sampler statistics, commit.  A finished
    request is left untouched.  temp = (T0, T1, seed): temperature sampling
    (the proposal is the Gumbel-max sample, its probability the confidence);
    b: the request's index in its batch (part of the sampling counter);
    routes: see forward.  Returns (forward dict, stats, CommitResult)."""
    if req.done:
        return None
    s = req.step + 1
    fw = forward(m, req, fill, routes)
    st = sampler_stats(fw["z"])
    if temp is not None and temp[0] > 0:
        T = temperature_at(s, N, temp[0], temp[1])
        st = sample_stats(st, fw["z"], T, temp[2], b, s, np.arange(len(req.ids)))
        st["argmax"] = st["sample"]
        st["logconf"] = st["sample_logconf"]
        st["conf"] = np.exp(st["sample_logconf"])
    cr = commit(req.ids, req.committed, st, s, N, stop_conf, m.eos_id, commit_conf, fill, stop_entropy)
    req.ids, req.committed = cr.ids, cr.committed
    req.step = s
    req.n_steps = s
    if cr.done:
        req.done = True
        req.n_valid = cr.n_valid
    return fw, st, cr


def kv_rows(m: Model, tok: np.ndarray, positions: np.ndarray, prefix_Ks=None, prefix_Vs=None,
            margins: Optional[list] = None):
    """Per-layer K (post-RoPE) and V rows of clean tokens at absolute
    positions P .. P + n - 1, as lists of [Hkv, n, hd].  This is the extra
    forward that encodes a finished canvas (or a prompt) as context and
    appends its key-value pairs ([TR3] section 3.4, the K-1 term of eq. (10)).
    Context encoding is causal ([TR1] section 1): in every layer but the
    last, token i attends to the prefix rows (prefix_Ks / prefix_Vs, per
    layer, P rows each; none: P = 0) and to tokens 0 .. i; the last layer's
    attention feeds nothing that is kept.  With one layer the rows depend
    only on each token and its position.  margins (a list): gets each
    routed layer's per-token router margins."""
    tok = np.asarray(tok, dtype=np.int64)
    positions = np.asarray(positions)
    layers = layer_list(m)
    L = len(layers)
    if prefix_Ks is None:
        prefix_Ks = [np.zeros((m.Hkv, 0, m.hd)) for _ in range(L)]
        prefix_Vs = [np.zeros((m.Hkv, 0, m.hd)) for _ in range(L)]
    P = prefix_Ks[0].shape[1]
    x = m.E[tok]
    ks, vs = [], []
    for l, Ly in enumerate(layers):
        q, k, v = project_qkv_x(m, Ly, x, positions)
        ks.append(k.transpose(1, 0, 2))
        vs.append(v.transpose(1, 0, 2))
        if l + 1 == L:
            break
        K = np.concatenate([prefix_Ks[l], ks[-1]], axis=1)
        Vv = np.concatenate([prefix_Vs[l], vs[-1]], axis=1)
        o = attend(m, q, K, Vv, causal_from=P)
        x = residual_out(m, x, o, Ly.Wo)
        if Ly.Wr is not None and margins is not None:
            margins.append(moe_route(m, Ly, x)[3])
        if Ly.Wg is not None:
            x = ffn(m, Ly, x)
    return ks, vs


def append_canvas(m: Model, req: Request):
    """Write the finished canvas into every layer's cache as read-only prefix
    ([BLOG], "Once Written, a Prefix Becomes History"); returns the appended
    per-layer rows (lists of [Hkv, C, hd])."""
    C = len(req.ids)
    ks, vs = kv_rows(m, req.ids, req.P + np.arange(C), req.Ks, req.Vs)
    req.Ks = [np.concatenate([K, k], axis=1) for K, k in zip(req.Ks, ks)]
    req.Vs = [np.concatenate([V, v], axis=1) for V, v in zip(req.Vs, vs)]
    return ks, vs


def reset_canvas(req: Request, ids, committed):
    req.ids = np.array(ids, dtype=np.int64)
    req.committed = np.array(committed, dtype=np.uint8)
    req.step = 0
    req.done = False
    req.n_steps = 0
    req.n_valid = len(req.ids)


def requests_from_inputs(m: Model, inp) -> List[Request]:
    """Per-request caches from materialised inputs.  Prompt workloads prefill
    the cache with the prompt's K/V rows at positions 0..n-1."""
    reqs = []
    for b in range(inp.wl.batch):
        if inp.prompt is not None:
            K, Vv = kv_rows(m, inp.prompt, np.arange(len(inp.prompt)))
        else:
            # per layer [Hkv, P_b, hd] (a single array: one layer)
            pk, pv = inp.prefix_k[b], inp.prefix_v[b]
            if isinstance(pk, (list, tuple)):
                K = [decode(x, m.dtype) for x in pk]
                Vv = [decode(x, m.dtype) for x in pv]
            else:
                K = decode(pk, m.dtype)
                Vv = decode(pv, m.dtype)
        reqs.append(Request(m, K, Vv, inp.init_ids[b], inp.init_committed[b]))
    return reqs


def run_canvas(m: Model, reqs: List[Request], N: int, stop_conf: Optional[float],
               commit_conf: Optional[float] = None, fill: int = 0,
               stop_entropy: Optional[float] = None, temp: Optional[tuple] = None):
    """Denoise every request's canvas until it is done (at most N steps)."""
    trace = []
    for _ in range(N):
        if all(r.done for r in reqs):
            break
        trace.append([denoise_step(m, r, N, stop_conf, commit_conf, fill, stop_entropy, temp, b)
                      for b, r in enumerate(reqs)])
    return trace


# ----------------------------------------------------------------------------
# efficiency metrics ([TR3] section 3.4)
# ----------------------------------------------------------------------------

def metrics(n_steps: List[int], n_valid: List[int]) -> dict:
    """Eqs. (7)-(10) over K canvases with N_k steps and C_k valid tokens."""
    K = len(n_steps)
    total_tokens = sum(n_valid)                                   # eq. (7)
    total_steps = sum(n_steps)                                    # eq. (8)
    eds = (sum(nk * ck for nk, ck in zip(n_steps, n_valid)) / total_tokens
           if total_tokens else float("nan"))                     # eq. (9)
    tpf = total_tokens / (total_steps + K - 1)                    # eq. (10)
    return dict(total_tokens=total_tokens, total_steps=total_steps,
                effective_steps=eds, tpf=tpf)
