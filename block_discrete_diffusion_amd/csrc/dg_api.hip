// Host side of the C-ABI: argument validation, workspace layout, the launch
// sequence of a denoising step, the append pass, prefill and per-launch
// timing.  Nothing here allocates device memory; every buffer is the caller's.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "dg_internal.hpp"

using namespace dg;

static thread_local std::string g_err;

static dg_status fail(dg_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

extern "C" const char *dg_last_error(void) { return g_err.c_str(); }

namespace dg {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int lm_slice_width(int dtype) { return dtype == DG_BF16 ? 128 : 64; }

int attn_base_wgs(int dtype, int B, int Hq, int Hkv, int C) {
    (void)dtype;
    const int G = Hq / Hkv;
    return B * Hkv * ((G * C + 127) / 128);
}

// Key-axis splits of the bf16 attention.  One request: about one workgroup
// per CU (256) in total, at least 4 blocks of 32 keys per split, at most 64
// splits.  (Measured on 1024- and 65536-row prefixes: one wave of
// workgroups beats both fewer, longer splits and a second round of shorter
// ones, whose partial sums cost more than they save.)  Several requests:
// a budget of 1024 workgroups (two per CU are resident at head_dim <= 128)
// shared in proportion to each request's key count, so that a long prefix
// does not leave the other requests' CUs idle while it finishes; at most
// 16 splits per request, at least 4 blocks per split.  (Measured on the
// ragged batch, prefixes of 1340 to 14210 keys: attention 302 us per step
// against 320 us with a budget of 512 and 491 us with one split each.)
static const int ATTN_SPLIT_MAX_BATCHED = 16;

int attn_n_split(int dtype, int B, int Hq, int Hkv, int C, int64_t total_keys) {
    if (dtype != DG_BF16) return 1;
    const int base = attn_base_wgs(dtype, 1, Hq, Hkv, C);
    const int64_t nblk = (total_keys + 31) / 32;
    if (B > 1)                                          // bound of attn_splits for any length mix
        return (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)ATTN_SPLIT_MAX_BATCHED, nblk / 4,
                                                             (int64_t)((1024 + base - 1) / base)}));
    const int want = std::max(1, (256 + base / 2) / base);
    return (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)want, nblk / 4, (int64_t)64}));
}

int attn_splits(int dtype, int B, int Hq, int Hkv, int C, const int64_t *len, int *split) {
    if (B == 1) {
        split[0] = attn_n_split(dtype, 1, Hq, Hkv, C, len[0] + C);
        return split[0];
    }
    const int base = attn_base_wgs(dtype, 1, Hq, Hkv, C);
    int64_t total = 0;
    for (int b = 0; b < B; ++b) total += (len[b] + C + 31) / 32;
    int smax = 1;
    for (int b = 0; b < B; ++b) {
        const int64_t nblk = (len[b] + C + 31) / 32;
        const int64_t want = (1024 * nblk + (int64_t)base * total - 1) / ((int64_t)base * total);   // ceil
        split[b] = dtype != DG_BF16 ? 1 : (int)std::max<int64_t>(1, std::min<int64_t>({want, nblk / 4,
                                                            (int64_t)ATTN_SPLIT_MAX_BATCHED}));
        smax = std::max(smax, split[b]);
    }
    return smax;
}

// Token rows per QKV workgroup: 128 (TM = 1) up to one full canvas of 256
// rows (measured faster: twice the tiles, half the split), 256 beyond.
int gemm_tm(int M) { return M > 256 ? 2 : 1; }

// Split of the K axis: each chunk holds a multiple of 4 stages of 64 (the
// depth of the weight ring), at least 8 stages, and the split stops once the
// grid has >= 160 workgroups.
int gemm_splitk(int tiles, int K) {
    const int nst = K / 64;
    int S = 1;
    while (tiles * S < 160 && nst % (2 * S) == 0 && (nst / (2 * S)) % 4 == 0 && nst / (2 * S) >= 8) S *= 2;
    return S;
}

// 64-row tiles with two K parts per workgroup where 128-row tiles give
// fewer than 256 tiles and K <= 4096 (the long K of a wide FFN's down
// projection keeps 128 rows: there the doubled weight reads cost more than
// the smaller partial sums save); then chunks, each part a multiple of 4
// stages (at least 8 stages with one part, 4 with two), until the grid has
// >= 160 workgroups.  Either weight format takes the same shape.
ProjShape oproj_shape(int M, int d, int K) {
    ProjShape p{4, 1, 1};
    if (K <= 4096 && (d / 64) * ((M + 127) / 128) < 256) {
        p.wpg = 2;
        p.kh = 2;
    }
    const int tiles = (d / 64) * ((M + 32 * p.wpg - 1) / (32 * p.wpg));
    const int nst = K / 64;
    auto fits = [&](int s2) {
        if (nst % (s2 * p.kh)) return false;
        const int per = nst / (s2 * p.kh);
        return per % 4 == 0 && per >= (p.kh == 1 ? 8 : 4);
    };
    while (tiles * p.S < 160 && fits(2 * p.S)) p.S *= 2;
    return p;
}

// fp32 partial sums of the split-K projections (QKV and output projection
// use the buffer one after the other).
size_t gemm_part_bytes(int dtype, int d, int Hq, int Hkv, int hd, int M, int d_ff) {
    if (dtype != DG_BF16) return 0;
    const int mt = (M + 128 * gemm_tm(M) - 1) / (128 * gemm_tm(M));
    const int n_all = (Hq + 2 * Hkv) * hd;
    const int s_qkv = gemm_splitk((n_all / 64) * mt, d);
    const int s_kv = gemm_splitk((2 * Hkv * hd / 64) * mt, d);
    int s_o = oproj_shape(M, d, Hq * hd).S;            // output and FFN down projections
    if (d_ff > 0) s_o = std::max(s_o, oproj_shape(M, d, d_ff).S);
    const size_t q = (std::max(s_qkv, s_kv) > 1) ? (size_t)std::max(s_qkv, s_kv) * M * n_all : 0;
    const size_t o = (size_t)s_o * M * d;
    return std::max(q, o) * 4;
}

Layout make_layout(int dtype, int V, int d, int Hq, int Hkv, int hd, int B, int C, int64_t max_prefix, int d_ff,
                   bool deep, MoeShape moe) {
    Layout L{};
    const size_t M = (size_t)B * C;
    const size_t A = 256;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, A); return o; };
    L.inp = take(M * 4);
    L.r_e = take(M * 4);
    L.r_h = take(M * 4);
    L.rope = take(M * (hd / 2) * 8);
    L.m_pad = (int)((M + 31) / 32 * 32);
    const size_t MP = dtype == DG_BF16 ? (size_t)L.m_pad : M;
    L.q = take(M * Hq * hd * 4);           // queries, fp32 for every dtype
    L.o = take(MP * Hq * hd * 4);         // attention output: bf16 path fp16 hi + lo planes, f32 path fp32
    L.cp = (C + 31) / 32 * 32;
    L.rows_c = B * L.cp;
    // bf16: fp16 vocabulary-head operand over the compact rows; f32: row-major h
    L.h = take(dtype == DG_BF16 ? (size_t)L.rows_c * d * 2 : M * d * 4);
    L.hf = take(dtype == DG_BF16 ? (size_t)L.rows_c * d * 4 : 0);   // fp32 h of the compact rows
    L.ulist = take((size_t)L.rows_c * 4);
    L.uidx = take(M * 4);
    L.ucount = take((size_t)B * 4);
    L.sample_cnt = take((size_t)B * 4);
    L.escale = take(dtype == DG_BF16 ? (size_t)V * 4 : 0);
    L.has_escale = dtype == DG_BF16 ? 1 : 0;
    L.n_split_max = attn_n_split(dtype, B, Hq, Hkv, C, max_prefix + C);
    const size_t QV = (size_t)B * Hq * C;
    if (dtype == DG_BF16) {
        L.attn_ml = take(L.n_split_max * QV * 8);
        L.attn_acc = take(L.n_split_max * QV * hd * 4);
    } else {
        L.attn_ml = L.attn_acc = take(0);
    }
    L.slice_width = lm_slice_width(dtype);
    L.n_slices = (V + L.slice_width - 1) / L.slice_width;
    L.lm_part = take((size_t)L.n_slices * L.rows_c * 16);
    L.lm_tpart = take((size_t)L.n_slices * L.rows_c * 4);
    L.lm_kpart = take(dtype == DG_BF16 ? (size_t)L.n_slices * L.rows_c * 16 : 0);
    L.rowstats = take(M * 16);
    L.rowent = take(M * 4);
    L.gemm_part = take(gemm_part_bytes(dtype, d, Hq, Hkv, hd, (int)M, d_ff));
    const bool resid = dtype == DG_BF16 && (deep || d_ff > 0);
    L.x = take(resid ? M * d * 4 : 0);
    L.xp = take(resid ? (size_t)L.m_pad * d * 4 : 0);
    L.r_x = take(resid ? M * 4 : 0);
    L.act = take(dtype == DG_BF16 && d_ff > 0 ? (size_t)L.m_pad * d_ff * 4 : 0);
    {
        const bool on = dtype == DG_BF16 && moe.E > 0;
        const size_t mk = on ? M * moe.k : 0;
        L.mk_pad = on ? (int)(mk + 32 * (size_t)moe.E) : 0;
        L.xr = take(on ? M * d * 4 : 0);
        L.moe_logit = take(on ? (size_t)(d / 128) * M * moe.E * 4 : 0);   // split-K partials [d/128][M][E]
        L.moe_sel = take(on ? (size_t)moe.n_layers * mk * 4 : 0);
        L.moe_gate = take(mk * 4);
        L.moe_cnt = take(on ? (size_t)moe.E * 4 : 0);
        L.moe_off = take(on ? (size_t)moe.E * 4 : 0);
        L.moe_ids = take(on ? (size_t)(moe.E + 1) * 4 : 0);
        L.moe_xg = take((size_t)L.mk_pad * d * 4);
        L.moe_list = take((size_t)L.mk_pad * 4);
        L.moe_act = take((size_t)L.mk_pad * moe.de * 4);
        L.moe_y = take(mk * d * 4);
    }
    L.err = take(16);
    L.total = off;
    return L;
}

}  // namespace dg

// ---------------------------------------------------------------------------
// validation
// ---------------------------------------------------------------------------
static MoeShape moe_shape(const dg_model *m) {
    MoeShape s;
    s.n_layers = m->n_layers > 0 ? m->n_layers : 1;
    if (m->n_experts > 0) { s.E = m->n_experts; s.k = m->top_k; s.de = m->d_expert; }
    return s;
}

static dg_status check_model(const dg_model *m) {
    if (!m) return fail(DG_ERR_NULL, "model is NULL");
    if (!m->embed || !m->wq || !m->wk || !m->wv || !m->wo || !m->lm_head)
        return fail(DG_ERR_NULL, "a weight pointer is NULL");
    if (m->dtype != DG_BF16 && m->dtype != DG_F32) return fail(DG_ERR_UNSUPPORTED, "unknown dtype %d", m->dtype);
    if (m->vocab < 2 || m->d_model < 1 || m->n_q_heads < 1 || m->n_kv_heads < 1 || m->head_dim < 2)
        return fail(DG_ERR_SHAPE, "non-positive model size");
    if (m->n_q_heads % m->n_kv_heads) return fail(DG_ERR_SHAPE, "n_q_heads %% n_kv_heads != 0");
    if (m->mask_id < 0 || m->mask_id >= m->vocab) return fail(DG_ERR_SHAPE, "mask_id outside [0, V)");
    if (m->eos_id >= m->vocab) return fail(DG_ERR_SHAPE, "eos_id >= V");
    if (m->eos_id == m->mask_id) return fail(DG_ERR_SHAPE, "eos_id == mask_id");
    if (!(m->rope_base > 0.f) || !(m->norm_eps >= 0.f)) return fail(DG_ERR_SHAPE, "bad rope_base / norm_eps");
    if (m->lm_format != DG_LM_NATIVE && m->lm_format != DG_LM_FP8)
        return fail(DG_ERR_UNSUPPORTED, "unknown lm_format %d", m->lm_format);
    if (m->lm_format == DG_LM_FP8) {
        if (m->dtype != DG_BF16) return fail(DG_ERR_UNSUPPORTED, "an e4m3 LM head needs a bf16 model");
        if (!m->lm_scale) return fail(DG_ERR_NULL, "lm_scale is NULL with an e4m3 LM head");
    }
    if (m->n_layers < 0 || m->n_layers > DG_MAX_LAYERS)
        return fail(DG_ERR_SHAPE, "n_layers %d outside [0, %d]", m->n_layers, DG_MAX_LAYERS);
    if (m->d_ff < 0) return fail(DG_ERR_SHAPE, "d_ff < 0");
    if (m->n_layers == 0 && m->d_ff != 0) return fail(DG_ERR_SHAPE, "an FFN needs n_layers >= 1 and layers[]");
    if (m->n_layers > 0) {
        if (m->dtype != DG_BF16) return fail(DG_ERR_UNSUPPORTED, "stacked layers and FFNs need a bf16 model");
        if (!m->layers) return fail(DG_ERR_NULL, "layers is NULL with n_layers = %d", m->n_layers);
        if (m->d_ff % 256) return fail(DG_ERR_SHAPE, "d_ff %% 256 != 0");
        for (int l = 0; l < m->n_layers; ++l) {
            const dg_layer &y = m->layers[l];
            if (!y.wq || !y.wk || !y.wv || !y.wo) return fail(DG_ERR_NULL, "layer %d: an attention weight is NULL", l);
            if (m->d_ff > 0 && (!y.w_gate || !y.w_up || !y.w_down))
                return fail(DG_ERR_NULL, "layer %d: an FFN weight is NULL", l);
            if (m->proj_format == DG_LM_FP8) {
                if (!y.wq_scale || !y.wk_scale || !y.wv_scale || !y.wo_scale)
                    return fail(DG_ERR_NULL, "layer %d: an attention weight scale is NULL", l);
                if (m->d_ff > 0 && (!y.w_gate_scale || !y.w_up_scale || !y.w_down_scale))
                    return fail(DG_ERR_NULL, "layer %d: an FFN weight scale is NULL", l);
            }
        }
    }
    if (m->n_experts < 0) return fail(DG_ERR_SHAPE, "n_experts < 0");
    if (m->n_experts > 0) {
        if (m->dtype != DG_BF16 || m->n_layers < 1)
            return fail(DG_ERR_UNSUPPORTED, "experts need a bf16 model with layers[] (n_layers >= 1)");
        if (m->d_ff <= 0) return fail(DG_ERR_SHAPE, "experts need the shared FFN (d_ff > 0)");
        if (m->n_experts > 256) return fail(DG_ERR_SHAPE, "n_experts %d > 256", m->n_experts);
        if (m->top_k < 1 || m->top_k > 16 || m->top_k > m->n_experts)
            return fail(DG_ERR_SHAPE, "top_k %d outside [1, min(n_experts, 16)]", m->top_k);
        if (m->d_expert <= 0 || m->d_expert % 256) return fail(DG_ERR_SHAPE, "d_expert %% 256 != 0");
        for (int l = 0; l < m->n_layers; ++l) {
            const dg_layer &y = m->layers[l];
            if (!y.w_router || !y.w_expert_gate || !y.w_expert_up || !y.w_expert_down)
                return fail(DG_ERR_NULL, "layer %d: an expert weight is NULL", l);
        }
    }
    if (m->proj_format != DG_LM_NATIVE && m->proj_format != DG_LM_FP8)
        return fail(DG_ERR_UNSUPPORTED, "unknown proj_format %d", m->proj_format);
    if (m->proj_format == DG_LM_FP8 && (m->dtype != DG_BF16 || m->n_layers < 1))
        return fail(DG_ERR_UNSUPPORTED, "e4m3 projections need a bf16 model with layers[] (n_layers >= 1)");
    if (m->dtype == DG_BF16) {
        if (m->d_model % 256) return fail(DG_ERR_SHAPE, "bf16 path needs d_model %% 256 == 0");
        if (m->head_dim != 64 && m->head_dim != 128 && m->head_dim != 256)
            return fail(DG_ERR_SHAPE, "bf16 path needs head_dim in {64, 128, 256}");
    } else {
        if (m->head_dim % 2 || m->head_dim > 256) return fail(DG_ERR_SHAPE, "f32 path needs even head_dim <= 256");
    }
    return DG_OK;
}

static dg_status check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DG_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return fail(DG_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    if (strncmp(p.gcnArchName, "gfx950", 6) != 0)
        return fail(DG_ERR_UNSUPPORTED, "device %d is %s, not gfx950", dev, p.gcnArchName);
    return DG_OK;
}

static const int F32_MAX_KEYS = 8192;

// ---------------------------------------------------------------------------
// handle
// ---------------------------------------------------------------------------
// Steps dg_run_canvas keeps in flight ahead of the done flags it reads: it
// waits for step s - RUN_LAG to finish before it enqueues step s, so a
// canvas that stops at step s' is followed by at most RUN_LAG - 1 enqueued
// steps (each a few early-exit launches) while the GPU never runs dry.
static const int RUN_LAG = 2;

struct dg_canvas {
    StepArgs a;
    dg_kv_cache *slot_cache[DG_MAX_BATCH];   // the caller's cache of each request slot
    hipStream_t stream;
    bool appended;
    int steps;            // steps enqueued since the last reset or resume
    // Host upper bounds of each request's open positions at its next step
    // and of its step counter (reset: C and 0; resume: read from the
    // device; each enqueued step applies the commit schedule, which a
    // threshold commit or a stop can only undercut).  The vocabulary head
    // groups requests by the largest bound.
    int open_bound[DG_MAX_BATCH];
    int step_idx[DG_MAX_BATCH];
    uint32_t prof;        // bit k: time launches of kernel kind k
    std::vector<hipEvent_t> pool;
    struct Rec { int kind; hipEvent_t e0, e1; };
    std::vector<Rec> rec;
    int32_t *done_host;   // pinned host [DG_MAX_BATCH], written by the kernels (null: no early exit)
    hipEvent_t run_ev[RUN_LAG];
    bool is_static;       // file-scope handle of dg_canvas_init_static (never deleted)
    int device;
    // Captured step (dg_canvas_set_graph): the launches of one step recorded
    // on a private stream and replayed on `stream`; re-recorded whenever the
    // step's launch arguments (its StepArgs bytes, the head's group size)
    // differ from the recorded ones.
    bool graph_on;
    hipStream_t cap_stream;
    hipGraphExec_t graph_exec;
    StepArgs graph_args;
    int graph_bp;
    dg_layer layers[DG_MAX_LAYERS];   // per-layer weights (layer 0 = the model's top-level ones if n_layers == 0)
};

// Arguments of the launches of layer l: its weights and its cache planes.
static StepArgs layer_args(const dg_canvas *c, const StepArgs &base, int l) {
    StepArgs a = base;
    const dg_layer &y = c->layers[l];
    a.layer = l;
    a.wq = y.wq; a.wk = y.wk; a.wv = y.wv; a.wo = y.wo;
    a.wg = y.w_gate; a.wu = y.w_up; a.wd = y.w_down;
    a.sq = y.wq_scale; a.sk = y.wk_scale; a.sv = y.wv_scale; a.so = y.wo_scale;
    a.sg = y.w_gate_scale; a.su = y.w_up_scale; a.sd = y.w_down_scale;
    a.wr = y.w_router; a.wge = y.w_expert_gate; a.wue = y.w_expert_up; a.wde = y.w_expert_down;
    const size_t esz = a.dtype == DG_BF16 ? 2 : 4;
    for (int b = 0; b < a.B; ++b) {
        const size_t plane = (size_t)a.Hkv * a.reqs.cap[b] * a.hd * esz;
        a.reqs.k[b] = (char *)base.reqs.k[b] + plane * l;
        a.reqs.v[b] = (char *)base.reqs.v[b] + plane * l;
    }
    return a;
}

// Enqueues one kernel kind.  When that kind is being timed, the events
// e0 / e1 bracket its launch on the stream, except for kinds whose launcher
// takes the events itself (launch_owns_events): those stamp them with the
// kernel's own start and end (hipExtLaunchKernelGGL), so the interval holds
// no dispatch gap.
static bool launch_owns_events(int kind) { return kind == K_LMHEAD; }

template <class F>
static dg_status run_ev(dg_canvas *c, int kind, F &&launch) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    const bool timed = (c->prof >> kind) & 1u;
    const bool owns = launch_owns_events(kind);
    if (timed) {
        for (hipEvent_t *e : {&e0, &e1}) {
            if (!c->pool.empty()) { *e = c->pool.back(); c->pool.pop_back(); }
            else if (hipEventCreate(e) != hipSuccess) return fail(DG_ERR_DEVICE, "hipEventCreate failed");
        }
        if (!owns) (void)hipEventRecord(e0, c->stream);
    }
    hipError_t err = launch(e0, e1);
    if (timed) {
        if (!owns) (void)hipEventRecord(e1, c->stream);
        c->rec.push_back({kind, e0, e1});
    }
    if (err != hipSuccess) return fail(DG_ERR_DEVICE, "launch (kind %d): %s", kind, hipGetErrorString(err));
    return DG_OK;
}

template <class F>
static dg_status run(dg_canvas *c, int kind, F &&launch) {
    return run_ev(c, kind, [&](hipEvent_t, hipEvent_t) { return launch(); });
}

#define RUN(kind, expr)                                              \
    do {                                                             \
        dg_status st_ = run(c, kind, [&]() { return (expr); });      \
        if (st_ != DG_OK) return st_;                                \
    } while (0)


static dg_status check_caches(const dg_kv_cache *caches, int B, int C, int dtype) {
    for (int b = 0; b < B; ++b) {
        const dg_kv_cache &k = caches[b];
        if (!k.k || !k.v) return fail(DG_ERR_NULL, "cache %d has a NULL buffer", b);
        if (k.capacity <= 0 || k.capacity % 8) return fail(DG_ERR_CAPACITY, "cache %d capacity %lld not a positive multiple of 8", b, (long long)k.capacity);
        if (k.len < 0 || k.len + C > k.capacity)
            return fail(DG_ERR_CAPACITY, "cache %d: len %lld + canvas %d > capacity %lld", b, (long long)k.len, C, (long long)k.capacity);
        if (dtype == DG_F32 && k.len + C > F32_MAX_KEYS)
            return fail(DG_ERR_SHAPE, "f32 path holds at most %d keys per query", F32_MAX_KEYS);
    }
    return DG_OK;
}

static int64_t max_capacity_prefix(const dg_kv_cache *caches, int B, int C) {
    int64_t m = 0;
    for (int b = 0; b < B; ++b) m = std::max<int64_t>(m, caches[b].capacity - C);
    return m;
}

extern "C" size_t dg_workspace_bytes(const dg_model *m, int32_t batch, int32_t canvas_len, int64_t max_prefix) {
    if (check_model(m) != DG_OK) return 0;
    if (batch < 1 || batch > DG_MAX_BATCH || canvas_len < 1 || canvas_len > DG_MAX_CANVAS || max_prefix < 0) return 0;
    return make_layout(m->dtype, m->vocab, m->d_model, m->n_q_heads, m->n_kv_heads, m->head_dim, batch,
                       canvas_len, max_prefix, m->d_ff, m->n_layers > 1, moe_shape(m)).total;
}

// Open positions and step counters of every request as the device holds
// them (waits for the stream): the exact bounds after a resume.
static dg_status read_bounds(dg_canvas *c) {
    int32_t cnt[DG_MAX_BATCH], stp[DG_MAX_BATCH];
    const int B = c->a.B;
    hipError_t e = hipMemcpyAsync(cnt, c->a.ws + c->a.L.ucount, B * 4, hipMemcpyDeviceToHost, c->stream);
    if (e == hipSuccess) e = hipMemcpyAsync(stp, c->a.step, B * 4, hipMemcpyDeviceToHost, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return fail(DG_ERR_DEVICE, "reading the canvas state: %s", hipGetErrorString(e));
    for (int b = 0; b < B; ++b) {
        c->open_bound[b] = std::max(0, std::min(cnt[b], c->a.C));
        c->step_idx[b] = std::max(0, stp[b]);
    }
    return DG_OK;
}

static dg_status enqueue_reset(dg_canvas *c, const int32_t *init_ids, const uint8_t *init_committed, bool state_too) {
    if (state_too) RUN(K_RESET, launch_reset(c->a, init_ids, init_committed, c->stream));   // also lists the open positions
    else RUN(K_RESET, launch_ulist(c->a, c->stream));
    RUN(K_RESET, launch_rope_table(c->a, c->stream));
    c->appended = false;
    c->steps = 0;
    if (state_too) {
        for (int b = 0; b < c->a.B; ++b) {
            c->open_bound[b] = c->a.C;
            c->step_idx[b] = 0;
            // the reset kernel clears them too; clearing here keeps a stale
            // set flag from being read before it runs
            if (c->done_host) __atomic_store_n(&c->done_host[b], 0, __ATOMIC_RELEASE);
        }
        return DG_OK;
    }
    return read_bounds(c);   // waits: the flags the list kernel copied are current
}

// Host checks of dg_canvas_init's arguments; the layout the workspace must hold.
static dg_status check_init(const dg_model *m, const dg_sampler *smp, const dg_kv_cache *caches, int32_t batch,
                            int32_t canvas_len, const dg_canvas_state *state, Layout *L, int64_t *maxp) {
    if (!smp || !caches || !state) return fail(DG_ERR_NULL, "sampler, caches or state is NULL");
    dg_status st = check_model(m);
    if (st != DG_OK) return st;
    if (batch < 1 || batch > DG_MAX_BATCH) return fail(DG_ERR_SHAPE, "batch %d outside [1, %d]", batch, DG_MAX_BATCH);
    if (canvas_len < 1 || canvas_len > DG_MAX_CANVAS)
        return fail(DG_ERR_SHAPE, "canvas_len %d outside [1, %d]", canvas_len, DG_MAX_CANVAS);
    if (!state->ids || !state->committed || !state->step || !state->n_steps_done || !state->n_valid || !state->done)
        return fail(DG_ERR_NULL, "a canvas-state buffer is NULL");
    if (smp->n_steps < 1) return fail(DG_ERR_SHAPE, "n_steps must be >= 1");
    if (smp->adaptive_stop < 0 || smp->adaptive_stop > 2) return fail(DG_ERR_SHAPE, "adaptive_stop must be 0, 1 or 2");
    if (smp->adaptive_stop == 1 && !std::isfinite(smp->stop_conf)) return fail(DG_ERR_SHAPE, "stop_conf not finite");
    if (smp->adaptive_stop == 2 && !std::isfinite(smp->stop_entropy)) return fail(DG_ERR_SHAPE, "stop_entropy not finite");
    if (smp->commit_rule != 0 && smp->commit_rule != 1) return fail(DG_ERR_SHAPE, "commit_rule must be 0 or 1");
    if (smp->commit_rule == 1 && !std::isfinite(smp->commit_conf)) return fail(DG_ERR_SHAPE, "commit_conf not finite");
    if (smp->canvas_fill != 0 && smp->canvas_fill != 1) return fail(DG_ERR_SHAPE, "canvas_fill must be 0 or 1");
    if (!std::isfinite(smp->temperature) || smp->temperature < 0.f)
        return fail(DG_ERR_SHAPE, "temperature must be finite and >= 0");
    if (smp->temperature > 0.f) {
        if (!std::isfinite(smp->temperature_end) || smp->temperature_end <= 0.f)
            return fail(DG_ERR_SHAPE, "temperature_end must be finite and > 0 when sampling");
        if (m->dtype != DG_BF16) return fail(DG_ERR_UNSUPPORTED, "temperature sampling needs a bf16 model");
    }
    st = check_caches(caches, batch, canvas_len, m->dtype);
    if (st != DG_OK) return st;
    *maxp = max_capacity_prefix(caches, batch, canvas_len);
    *L = make_layout(m->dtype, m->vocab, m->d_model, m->n_q_heads, m->n_kv_heads, m->head_dim, batch, canvas_len,
                     *maxp, m->d_ff, m->n_layers > 1, moe_shape(m));
    return DG_OK;
}

// Fills a handle (validated arguments) and enqueues the error-word clear,
// the embedding row scales and the canvas reset (or the resume).
static dg_status start_handle(dg_canvas *c, const dg_model *m, const dg_sampler *smp, dg_kv_cache *caches,
                              int32_t batch, int32_t canvas_len, const dg_canvas_state *state,
                              const int32_t *init_ids, const uint8_t *init_committed, uint32_t flags, char *ws,
                              const Layout &L, void *stream) {
    StepArgs &a = c->a;
    a = StepArgs{};
    a.dtype = m->dtype;
    a.V = m->vocab; a.d = m->d_model; a.Hq = m->n_q_heads; a.Hkv = m->n_kv_heads; a.hd = m->head_dim;
    a.mask_id = m->mask_id; a.eos_id = m->eos_id;
    a.rope_base = m->rope_base; a.eps = m->norm_eps;
    a.embed = m->embed; a.wq = m->wq; a.wk = m->wk; a.wv = m->wv; a.wo = m->wo; a.lm = m->lm_head;
    a.lm_scale = m->lm_scale; a.lm_fp8 = m->lm_format == DG_LM_FP8 ? 1 : 0;
    a.proj_fp8 = m->proj_format == DG_LM_FP8 ? 1 : 0;
    a.n_experts = m->n_experts > 0 ? m->n_experts : 0;
    a.top_k = m->top_k;
    a.d_e = m->d_expert;
    a.B = batch; a.C = canvas_len; a.M = batch * canvas_len;
    a.N = smp->n_steps; a.adaptive = smp->adaptive_stop; a.tau = smp->stop_conf; a.h_max = smp->stop_entropy;
    a.ent = smp->adaptive_stop == 2 ? 1 : 0;
    a.commit_rule = smp->commit_rule; a.tau_c = smp->commit_conf; a.fill = smp->canvas_fill;
    a.temp0 = smp->temperature; a.temp1 = smp->temperature_end; a.seed = smp->seed;
    a.only_req = -1;
    a.n_layers = m->n_layers > 0 ? m->n_layers : 1;
    a.d_ff = m->d_ff;
    a.phase = PH_STEP;
    for (int l = 0; l < DG_MAX_LAYERS; ++l) c->layers[l] = dg_layer{};
    if (m->n_layers > 0)
        for (int l = 0; l < m->n_layers; ++l) c->layers[l] = m->layers[l];
    else
        c->layers[0] = dg_layer{m->wq, m->wk, m->wv, m->wo, nullptr, nullptr, nullptr};
    a.ids = state->ids; a.committed = state->committed; a.step = state->step;
    a.n_steps_done = state->n_steps_done; a.n_valid = state->n_valid; a.done = state->done;
    a.done_host = c->done_host;
    a.ws = ws;
    a.L = L;
    for (int b = 0; b < DG_MAX_BATCH; ++b) {
        const bool on = b < batch;
        a.reqs.k[b] = on ? caches[b].k : nullptr;
        a.reqs.v[b] = on ? caches[b].v : nullptr;
        a.reqs.cap[b] = on ? caches[b].capacity : 0;
        a.reqs.len[b] = on ? caches[b].len : 0;
    }
    for (int b = 0; b < DG_MAX_BATCH; ++b) c->slot_cache[b] = b < batch ? &caches[b] : nullptr;
    c->stream = (hipStream_t)stream;
    c->prof = 0;
    c->appended = false;
    c->steps = 0;
    dg_status st;
    if ((st = run(c, K_RESET, [&]() { return launch_clear_err(c->a, c->stream); })) != DG_OK ||
        (a.dtype == DG_BF16 && (st = run(c, K_RESET, [&]() { return launch_escale(c->a, c->stream); })) != DG_OK) ||
        (st = enqueue_reset(c, init_ids, init_committed, !(flags & DG_INIT_RESUME))) != DG_OK)
        return st;
    return DG_OK;
}

extern "C" dg_status dg_canvas_init(dg_canvas **out, const dg_model *m, const dg_sampler *smp,
                                    dg_kv_cache *caches, int32_t batch, int32_t canvas_len,
                                    const dg_canvas_state *state, const int32_t *init_ids,
                                    const uint8_t *init_committed, uint32_t flags, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    if (!out) return fail(DG_ERR_NULL, "out is NULL");
    *out = nullptr;
    if (!workspace) return fail(DG_ERR_NULL, "workspace is NULL");
    Layout L;
    int64_t maxp = 0;
    dg_status st = check_init(m, smp, caches, batch, canvas_len, state, &L, &maxp);
    if (st != DG_OK) return st;
    if (workspace_bytes < L.total)
        return fail(DG_ERR_WORKSPACE, "workspace %zu bytes < %zu needed (dg_workspace_bytes with max_prefix = %lld)",
                    workspace_bytes, L.total, (long long)maxp);
    st = check_device();
    if (st != DG_OK) return st;

    dg_canvas *c = new (std::nothrow) dg_canvas();
    if (!c) return fail(DG_ERR_DEVICE, "host allocation failed");
    c->done_host = nullptr;
    for (int i = 0; i < RUN_LAG; ++i) c->run_ev[i] = nullptr;
    {
        // early exit of dg_run_canvas: a pinned, coherent host copy of the
        // done flags and a ring of events to wait on
        void *hp = nullptr;
        hipError_t e = hipHostMalloc(&hp, DG_MAX_BATCH * sizeof(int32_t), hipHostMallocCoherent);
        for (int i = 0; e == hipSuccess && i < RUN_LAG; ++i) e = hipEventCreateWithFlags(&c->run_ev[i], hipEventDisableTiming);
        if (e != hipSuccess) {
            for (int i = 0; i < RUN_LAG; ++i)
                if (c->run_ev[i]) (void)hipEventDestroy(c->run_ev[i]);
            if (hp) (void)hipHostFree(hp);
            delete c;
            return fail(DG_ERR_DEVICE, "pinned host flags: %s", hipGetErrorString(e));
        }
        c->done_host = (int32_t *)hp;
        for (int b = 0; b < DG_MAX_BATCH; ++b) c->done_host[b] = 0;
    }
    st = start_handle(c, m, smp, caches, batch, canvas_len, state, init_ids, init_committed, flags,
                      (char *)workspace, L, stream);
    if (st != DG_OK) {
        (void)dg_canvas_destroy(c);
        return st;
    }
    *out = c;
    return DG_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free handles: the workspace is the file-scope device array
// `scratch` (each GPU holds its own copy for the life of the process), and
// the handle itself is a file-scope host object, one per device.  Host code
// never uses the array's name as an address: hipGetSymbolAddress gives the
// device address of this GPU's copy, once per device, at the first init on
// it, with that device current.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[DG_STATIC_SCRATCH_BYTES];

static const int STATIC_MAX_DEVICES = 64;
static dg_canvas g_static_handle[STATIC_MAX_DEVICES];
static bool g_static_live[STATIC_MAX_DEVICES];
static void *g_scratch_ptr[STATIC_MAX_DEVICES];

extern "C" dg_status dg_canvas_init_static(dg_canvas **out, const dg_model *m, const dg_sampler *smp,
                                           dg_kv_cache *caches, int32_t batch, int32_t canvas_len,
                                           const dg_canvas_state *state, const int32_t *init_ids,
                                           const uint8_t *init_committed, uint32_t flags, void *stream) {
    if (!out) return fail(DG_ERR_NULL, "out is NULL");
    *out = nullptr;
    Layout L;
    int64_t maxp = 0;
    dg_status st = check_init(m, smp, caches, batch, canvas_len, state, &L, &maxp);
    if (st != DG_OK) return st;
    if (L.total > (size_t)DG_STATIC_SCRATCH_BYTES)
        return fail(DG_ERR_WORKSPACE, "these shapes need %zu bytes of workspace; the static scratch holds %zu "
                    "(use dg_canvas_init with a workspace)", L.total, (size_t)DG_STATIC_SCRATCH_BYTES);
    st = check_device();
    if (st != DG_OK) return st;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DG_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= STATIC_MAX_DEVICES) return fail(DG_ERR_UNSUPPORTED, "device %d beyond %d", dev, STATIC_MAX_DEVICES);
    if (g_static_live[dev]) return fail(DG_ERR_STATE, "device %d already has a live static-scratch handle", dev);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(DG_ERR_DEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    dg_canvas *c = &g_static_handle[dev];
    c->rec.clear();
    c->done_host = nullptr;              // no pinned flags: dg_run_canvas enqueues the whole budget
    for (int i = 0; i < RUN_LAG; ++i) c->run_ev[i] = nullptr;
    c->is_static = true;
    c->device = dev;
    g_static_live[dev] = true;
    st = start_handle(c, m, smp, caches, batch, canvas_len, state, init_ids, init_committed, flags,
                      (char *)g_scratch_ptr[dev], L, stream);
    if (st != DG_OK) {
        (void)dg_canvas_destroy(c);
        return st;
    }
    *out = c;
    return DG_OK;
}

// The launches of one denoising step with the step's arguments a (key
// splits set), n_split the largest split count and bp the head's group
// size.
static dg_status enqueue_step(dg_canvas *c, const StepArgs &a, int n_split, int bp, const dg_debug *dbg) {
    if (a.dtype != DG_BF16) RUN(K_PREP, launch_prep(a, 0, c->stream));
    // every layer: QKV + RoPE (layer 0 from the fed ids' embedding rows,
    // deeper layers from the residual stream), attention over its own cache
    // plane, output projection with the residual, then its FFN; the last
    // projection of the last layer hands h to the vocabulary head
    float *hdump = (dbg && a.dtype == DG_BF16) ? (float *)dbg->h : nullptr;
    for (int l = 0; l < a.n_layers; ++l) {
        const StepArgs al = layer_args(c, a, l);
        const bool last = l + 1 == a.n_layers;
        const int src = l == 0 ? SRC_EMBED : SRC_RESID;
        RUN(K_QKV, launch_qkv(al, 0, WRITE_STEP, c->stream, src));
        RUN(K_ATTN, launch_attention(al, n_split, c->stream));
        if (a.dtype == DG_BF16)
            RUN(K_ATTN_MERGE, launch_attn_merge(al, n_split, dbg ? (float *)dbg->o : nullptr, c->stream));
        const int o_out = (last && a.d_ff == 0) ? OUT_LMHEAD : OUT_RESID;
        RUN(K_OPROJ, launch_oproj(al, o_out == OUT_LMHEAD ? hdump : nullptr, c->stream, src, o_out));
        if (a.n_experts > 0) RUN(K_MOE, launch_moe(al, c->stream));
        if (a.d_ff > 0) RUN(K_FFN, launch_ffn(al, last ? hdump : nullptr, c->stream, last ? OUT_LMHEAD : OUT_RESID));
    }
    if (a.dtype != DG_BF16) RUN(K_ROWSCALE, launch_rowscale_h(a, c->stream));
    {
        dg_status st_ = run_ev(c, K_LMHEAD, [&](hipEvent_t e0, hipEvent_t e1) {
            return launch_lmhead(a, dbg ? dbg->logits : nullptr, bp, c->stream, e0, e1);
        });
        if (st_ != DG_OK) return st_;
    }
    RUN(K_SAMPLE, launch_sample_commit(a, c->stream));
    if (dbg) {
        const size_t M = (size_t)a.M;
        if (dbg->q) RUN(K_DEBUG, hipMemcpyAsync(dbg->q, a.ws + a.L.q, M * a.Hq * a.hd * 4, hipMemcpyDeviceToDevice, c->stream));
        if (dbg->row_stats) RUN(K_DEBUG, hipMemcpyAsync(dbg->row_stats, a.ws + a.L.rowstats, M * 16, hipMemcpyDeviceToDevice, c->stream));
        if (dbg->entropy) RUN(K_DEBUG, hipMemcpyAsync(dbg->entropy, a.ws + a.L.rowent, M * 4, hipMemcpyDeviceToDevice, c->stream));
        if (dbg->moe_sel && a.n_experts > 0)
            RUN(K_DEBUG, hipMemcpyAsync(dbg->moe_sel, a.ws + a.L.moe_sel, (size_t)a.n_layers * M * a.top_k * 4,
                                        hipMemcpyDeviceToDevice, c->stream));
        // the bf16 path writes its o and h dumps from the attention merge and
        // the output projection's finish
        if (a.dtype != DG_BF16) {
            if (dbg->o) RUN(K_DEBUG, hipMemcpyAsync(dbg->o, a.ws + a.L.o, M * a.Hq * a.hd * 4, hipMemcpyDeviceToDevice, c->stream));
            if (dbg->h) RUN(K_DEBUG, hipMemcpyAsync(dbg->h, a.ws + a.L.h, M * a.d * 4, hipMemcpyDeviceToDevice, c->stream));
        }
    }
    return DG_OK;
}

// The step as a graph: recorded on the private capture stream (the handle's
// stream may be the legacy default stream, which cannot be captured) the
// first time and whenever the arguments change, replayed on the handle's
// stream.  Nothing in a step allocates, copies or sets memory, so the graph
// holds kernel nodes only.
static dg_status step_graph(dg_canvas *c, const StepArgs &a, int n_split, int bp) {
    const bool same = c->graph_exec && bp == c->graph_bp && std::memcmp(&a, &c->graph_args, sizeof(StepArgs)) == 0;
    if (!same) {
        if (c->graph_exec) {
            (void)hipGraphExecDestroy(c->graph_exec);
            c->graph_exec = nullptr;
        }
        if (!c->cap_stream) {
            const hipError_t e = hipStreamCreate(&c->cap_stream);
            if (e != hipSuccess) return fail(DG_ERR_DEVICE, "hipStreamCreate: %s", hipGetErrorString(e));
        }
        hipStream_t user = c->stream;
        c->stream = c->cap_stream;
        hipError_t e = hipStreamBeginCapture(c->stream, hipStreamCaptureModeThreadLocal);
        if (e != hipSuccess) {
            c->stream = user;
            return fail(DG_ERR_DEVICE, "hipStreamBeginCapture: %s", hipGetErrorString(e));
        }
        const dg_status st = enqueue_step(c, a, n_split, bp, nullptr);
        hipGraph_t g = nullptr;
        e = hipStreamEndCapture(c->stream, &g);
        c->stream = user;
        if (st != DG_OK) {
            if (g) (void)hipGraphDestroy(g);
            return st;
        }
        if (e != hipSuccess) return fail(DG_ERR_DEVICE, "hipStreamEndCapture: %s", hipGetErrorString(e));
        e = hipGraphInstantiate(&c->graph_exec, g, nullptr, nullptr, 0);
        (void)hipGraphDestroy(g);
        if (e != hipSuccess) {
            c->graph_exec = nullptr;
            return fail(DG_ERR_DEVICE, "hipGraphInstantiate: %s", hipGetErrorString(e));
        }
        std::memcpy(&c->graph_args, &a, sizeof(StepArgs));
        c->graph_bp = bp;
    }
    const hipError_t e = hipGraphLaunch(c->graph_exec, c->stream);
    if (e != hipSuccess) return fail(DG_ERR_DEVICE, "hipGraphLaunch: %s", hipGetErrorString(e));
    return DG_OK;
}

extern "C" dg_status dg_denoise_step(dg_canvas *c, const dg_debug *dbg) {
    if (!c) return fail(DG_ERR_NULL, "handle is NULL");
    if (c->appended) return fail(DG_ERR_STATE, "canvas already appended; call dg_canvas_reset");
    StepArgs a;
    std::memcpy(&a, &c->a, sizeof(StepArgs));         // bytewise, so that a recorded step compares exactly
    a.ent = (a.adaptive == 2 || (dbg && dbg->entropy)) ? 1 : 0;
    const int n_split = std::min(attn_splits(a.dtype, a.B, a.Hq, a.Hkv, a.C, a.reqs.len, a.attn_split), a.L.n_split_max);
    for (int b = 0; b < a.B; ++b) a.attn_split[b] = std::min(a.attn_split[b], n_split);
    // At most open_bound[b] positions of request b are open at this step.
    // The LM head takes as many requests per workgroup as fit 8 row tiles
    // of 32 under the largest bound.
    int open_max = 0;
    for (int b = 0; b < a.B; ++b) open_max = std::max(open_max, c->open_bound[b]);
    int bp = 1;
    while (2 * bp <= std::min(a.B, DG_LM_GROUP_MAX) && 2 * bp * ((open_max + 31) / 32) <= 8) bp *= 2;
    const dg_status st = (c->graph_on && !dbg && c->prof == 0) ? step_graph(c, a, n_split, bp)
                                                                : enqueue_step(c, a, n_split, bp, dbg);
    if (st != DG_OK) return st;
    c->steps++;
    // the schedule of this step (s = step_idx + 1) commits at least
    // ceil(|U| / (N - s + 1)) of |U| open positions
    for (int b = 0; b < a.B; ++b) {
        const int s = ++c->step_idx[b];
        const int left = a.N - s + 1;
        int &u = c->open_bound[b];
        u -= left <= 1 ? u : (u + left - 1) / left;
    }
    return DG_OK;
}

// Steps until max_steps, until every request's budget is spent, until every
// request is done or until a request of stop_mask is done.  Before step
// k + RUN_LAG of the call is enqueued, step k has finished and the done
// flags the sampler copies to pinned host memory are read; *done_mask gets
// the flags of the last such read (or of a final synchronisation).
static dg_status run_steps(dg_canvas *c, int max_steps, uint32_t stop_mask, int *n_run, uint32_t *done_mask) {
    auto budget_left = [&]() {
        for (int b = 0; b < c->a.B; ++b)
            if (c->step_idx[b] < c->a.N) return true;
        return false;
    };
    auto read_flags = [&]() {
        uint32_t m = 0;
        for (int b = 0; b < c->a.B; ++b)
            if (__atomic_load_n(&c->done_host[b], __ATOMIC_ACQUIRE) != 0) m |= 1u << b;
        return m;
    };
    const uint32_t all = c->a.B == 32 ? 0xffffffffu : (1u << c->a.B) - 1;
    int k = 0;
    bool stopped = false;
    uint32_t mask = 0;
    while (k < max_steps && budget_left()) {
        if (c->done_host && k >= RUN_LAG) {
            hipError_t e = hipEventSynchronize(c->run_ev[k % RUN_LAG]);
            if (e != hipSuccess) return fail(DG_ERR_DEVICE, "hipEventSynchronize: %s", hipGetErrorString(e));
            mask = read_flags();
            if ((stopped = mask == all || (mask & stop_mask) != 0)) break;
        }
        dg_status st = dg_denoise_step(c, nullptr);
        if (st != DG_OK) return st;
        if (c->done_host) {
            hipError_t e = hipEventRecord(c->run_ev[k % RUN_LAG], c->stream);
            if (e != hipSuccess) return fail(DG_ERR_DEVICE, "hipEventRecord: %s", hipGetErrorString(e));
        }
        ++k;
    }
    if (n_run) *n_run = k;
    if (done_mask && !stopped) {
        // the loop ended on max_steps or the budget: the flags as of the
        // last enqueued step
        if (c->done_host) {
            hipError_t e = hipStreamSynchronize(c->stream);
            if (e != hipSuccess) return fail(DG_ERR_DEVICE, "hipStreamSynchronize: %s", hipGetErrorString(e));
            mask = read_flags();
        } else {
            std::vector<int32_t> dn(c->a.B);
            hipError_t e = hipMemcpyAsync(dn.data(), c->a.done, c->a.B * 4, hipMemcpyDeviceToHost, c->stream);
            if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
            if (e != hipSuccess) return fail(DG_ERR_DEVICE, "reading done flags: %s", hipGetErrorString(e));
            mask = 0;
            for (int b = 0; b < c->a.B; ++b)
                if (dn[b]) mask |= 1u << b;
        }
    }
    if (done_mask) *done_mask = mask;
    return DG_OK;
}

extern "C" dg_status dg_run_steps(dg_canvas *c, int32_t max_steps, uint32_t stop_mask, int32_t *n_run,
                                  uint32_t *done_mask) {
    if (!c) return fail(DG_ERR_NULL, "handle is NULL");
    if (c->appended) return fail(DG_ERR_STATE, "canvas already appended; call dg_canvas_reset");
    if (max_steps < 0) return fail(DG_ERR_SHAPE, "max_steps %d < 0", max_steps);
    int k = 0;
    dg_status st = run_steps(c, max_steps, stop_mask, &k, done_mask);
    if (n_run) *n_run = k;
    return st;
}

extern "C" dg_status dg_run_canvas(dg_canvas *c, dg_canvas_stats *out) {
    if (!c) return fail(DG_ERR_NULL, "handle is NULL");
    if (c->appended) return fail(DG_ERR_STATE, "canvas already appended; call dg_canvas_reset");
    dg_status st = run_steps(c, 0x7fffffff, 0, nullptr, nullptr);
    if (st != DG_OK) return st;
    if (out) {
        std::vector<int32_t> ns(c->a.B), nv(c->a.B);
        hipError_t e = hipMemcpyAsync(ns.data(), c->a.n_steps_done, c->a.B * 4, hipMemcpyDeviceToHost, c->stream);
        if (e == hipSuccess) e = hipMemcpyAsync(nv.data(), c->a.n_valid, c->a.B * 4, hipMemcpyDeviceToHost, c->stream);
        if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
        if (e != hipSuccess) return fail(DG_ERR_DEVICE, "reading canvas stats: %s", hipGetErrorString(e));
        for (int b = 0; b < c->a.B; ++b) out[b] = dg_canvas_stats{ns[b], nv[b]};
    }
    return DG_OK;
}

// The append pass of every done request (only_req < 0) or of one.
// Context encoding of the clean canvas (causal: canvas position i sees the
// prefix and positions 0 .. i): every layer's K / V rows; each layer but the
// last also runs its attention, output projection and FFN to produce the
// next layer's input.
static dg_status enqueue_append(dg_canvas *c, int only_req) {
    StepArgs a = c->a;
    a.only_req = only_req;
    RUN(K_APPEND, launch_prep(a, 1, c->stream));
    a.phase = PH_APPEND;
    a.causal = 1;
    const int n_split = std::min(attn_splits(a.dtype, a.B, a.Hq, a.Hkv, a.C, a.reqs.len, a.attn_split), a.L.n_split_max);
    for (int b = 0; b < a.B; ++b) a.attn_split[b] = std::min(a.attn_split[b], n_split);
    for (int l = 0; l < a.n_layers; ++l) {
        const StepArgs al = layer_args(c, a, l);
        const int src = l == 0 ? SRC_EMBED : SRC_RESID;
        if (l + 1 == a.n_layers) {
            RUN(K_APPEND, launch_qkv(al, 1, WRITE_APPEND, c->stream, src));
            break;
        }
        RUN(K_APPEND, launch_qkv(al, 0, WRITE_APPEND, c->stream, src));
        RUN(K_APPEND, launch_attention(al, n_split, c->stream));
        RUN(K_APPEND, launch_attn_merge(al, n_split, nullptr, c->stream));
        RUN(K_APPEND, launch_oproj(al, nullptr, c->stream, src, OUT_RESID));
        if (a.n_experts > 0) RUN(K_APPEND, launch_moe(al, c->stream));
        if (a.d_ff > 0) RUN(K_APPEND, launch_ffn(al, nullptr, c->stream, OUT_RESID));
    }
    return DG_OK;
}

// Slot b starts a fresh canvas at its cache's length (the rest of the
// batch carries on): its state, open-position list and fed ids, the RoPE
// table (all rows; the others' are rewritten with the same values) and its
// host bounds.
static dg_status restart_slot(dg_canvas *c, int b, const int32_t *init_ids, const uint8_t *init_committed) {
    if (c->done_host) __atomic_store_n(&c->done_host[b], 0, __ATOMIC_RELEASE);
    RUN(K_RESET, launch_reset(c->a, init_ids, init_committed, c->stream, b));
    RUN(K_RESET, launch_rope_table(c->a, c->stream));
    c->open_bound[b] = c->a.C;
    c->step_idx[b] = 0;
    return DG_OK;
}

extern "C" dg_status dg_append_request_kv(dg_canvas *c, int32_t b, const int32_t *init_ids,
                                         const uint8_t *init_committed) {
    if (!c) return fail(DG_ERR_NULL, "handle is NULL");
    if (c->appended) return fail(DG_ERR_STATE, "canvas already appended; call dg_canvas_reset");
    if (b < 0 || b >= c->a.B) return fail(DG_ERR_SHAPE, "request %d outside [0, %d)", b, c->a.B);
    // done flags only rise within a request and are cleared on the host and
    // on the stream when the slot restarts, so a set pinned flag is final;
    // without pinned flags the device flag is read after the stream drains
    int32_t dn = 0;
    if (c->done_host) {
        dn = __atomic_load_n(&c->done_host[b], __ATOMIC_ACQUIRE);
        if (!dn) {
            hipError_t e = hipStreamSynchronize(c->stream);
            if (e != hipSuccess) return fail(DG_ERR_DEVICE, "hipStreamSynchronize: %s", hipGetErrorString(e));
            dn = __atomic_load_n(&c->done_host[b], __ATOMIC_ACQUIRE);
        }
    } else {
        hipError_t e = hipMemcpyAsync(&dn, c->a.done + b, 4, hipMemcpyDeviceToHost, c->stream);
        if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
        if (e != hipSuccess) return fail(DG_ERR_DEVICE, "reading the done flag: %s", hipGetErrorString(e));
    }
    if (!dn) return fail(DG_ERR_STATE, "request %d is not done; nothing appended", b);
    if (c->a.reqs.len[b] + 2 * c->a.C > c->a.reqs.cap[b])
        return fail(DG_ERR_CAPACITY, "cache %d cannot hold this canvas and the next", b);
    dg_status st = enqueue_append(c, b);
    if (st != DG_OK) return st;
    c->a.reqs.len[b] += c->a.C;
    c->slot_cache[b]->len = c->a.reqs.len[b];
    return restart_slot(c, b, init_ids, init_committed);
}

extern "C" dg_status dg_canvas_admit(dg_canvas *c, int32_t b, dg_kv_cache *cache, const int32_t *init_ids,
                                     const uint8_t *init_committed) {
    if (!c || !cache) return fail(DG_ERR_NULL, "handle or cache is NULL");
    if (c->appended) return fail(DG_ERR_STATE, "canvas already appended; call dg_canvas_reset");
    if (b < 0 || b >= c->a.B) return fail(DG_ERR_SHAPE, "request %d outside [0, %d)", b, c->a.B);
    dg_status st = check_caches(cache, 1, c->a.C, c->a.dtype);
    if (st != DG_OK) return st;
    // A longer cache than those at init needs no more workspace: the
    // attention split count is clamped to what the workspace holds.
    c->slot_cache[b] = cache;
    c->a.reqs.k[b] = cache->k;
    c->a.reqs.v[b] = cache->v;
    c->a.reqs.cap[b] = cache->capacity;
    c->a.reqs.len[b] = cache->len;
    return restart_slot(c, b, init_ids, init_committed);
}

extern "C" const volatile int32_t *dg_done_flags(const dg_canvas *c) { return c ? c->done_host : nullptr; }

extern "C" dg_status dg_append_canvas_kv(dg_canvas *c) {
    if (!c) return fail(DG_ERR_NULL, "handle is NULL");
    if (c->appended) return fail(DG_ERR_STATE, "canvas already appended");
    for (int b = 0; b < c->a.B; ++b)
        if (c->a.reqs.len[b] + c->a.C > c->a.reqs.cap[b]) return fail(DG_ERR_CAPACITY, "cache %d full", b);
    {
        // every request must be done: read the flags once (waits for the stream)
        int32_t dn[DG_MAX_BATCH];
        hipError_t e = hipMemcpyAsync(dn, c->a.done, c->a.B * 4, hipMemcpyDeviceToHost, c->stream);
        if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
        if (e != hipSuccess) return fail(DG_ERR_DEVICE, "reading the done flags: %s", hipGetErrorString(e));
        for (int b = 0; b < c->a.B; ++b)
            if (!dn[b]) return fail(DG_ERR_STATE, "request %d is not done; nothing appended", b);
    }
    dg_status st = enqueue_append(c, -1);
    if (st != DG_OK) return st;
    for (int b = 0; b < c->a.B; ++b) {
        c->a.reqs.len[b] += c->a.C;
        c->slot_cache[b]->len = c->a.reqs.len[b];
    }
    c->appended = true;
    return DG_OK;
}

extern "C" dg_status dg_canvas_reset(dg_canvas *c, const int32_t *init_ids, const uint8_t *init_committed) {
    if (!c) return fail(DG_ERR_NULL, "handle is NULL");
    for (int b = 0; b < c->a.B; ++b) {
        const int64_t len = c->slot_cache[b]->len;
        if (len < 0) return fail(DG_ERR_CAPACITY, "cache %d has a negative length", b);
        if (len + c->a.C > c->a.reqs.cap[b]) return fail(DG_ERR_CAPACITY, "cache %d cannot hold another canvas", b);
        if (c->a.dtype == DG_F32 && len + c->a.C > F32_MAX_KEYS)
            return fail(DG_ERR_SHAPE, "f32 path holds at most %d keys per query", F32_MAX_KEYS);
    }
    for (int b = 0; b < c->a.B; ++b) c->a.reqs.len[b] = c->slot_cache[b]->len;
    return enqueue_reset(c, init_ids, init_committed, true);
}

extern "C" dg_status dg_canvas_resume(dg_canvas *c) {
    if (!c) return fail(DG_ERR_NULL, "handle is NULL");
    if (c->appended) return fail(DG_ERR_STATE, "canvas already appended; call dg_canvas_reset");
    RUN(K_RESET, launch_ulist(c->a, c->stream));
    c->steps = 0;
    return read_bounds(c);
}

extern "C" size_t dg_prefill_workspace_bytes(const dg_model *m, int32_t n) {
    if (check_model(m) != DG_OK || n < 1) return 0;
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
    L.inp = take((size_t)n * 4);
    L.r_e = take((size_t)n * 4);
    L.rope = take((size_t)n * (m->head_dim / 2) * 8);
    L.gemm_part = take(gemm_part_bytes(m->dtype, m->d_model, m->n_q_heads, m->n_kv_heads, m->head_dim, n));
    L.err = take(16);
    return off;
}

extern "C" dg_status dg_prefill_kv(const dg_model *m, dg_kv_cache *cache, const int32_t *ids, int32_t n,
                                   void *workspace, size_t workspace_bytes, void *stream) {
    if (!cache || !ids || !workspace) return fail(DG_ERR_NULL, "cache, ids or workspace is NULL");
    dg_status st = check_model(m);
    if (st != DG_OK) return st;
    if (m->n_layers > 1 || m->d_ff > 0)
        return fail(DG_ERR_UNSUPPORTED, "prefill of a model with stacked layers or an FFN: encode the context with "
                    "dg_append_canvas_kv");
    if (n < 1) return fail(DG_ERR_SHAPE, "n must be >= 1");
    if (!cache->k || !cache->v) return fail(DG_ERR_NULL, "cache buffer is NULL");
    if (cache->capacity <= 0 || cache->capacity % 8) return fail(DG_ERR_CAPACITY, "capacity not a positive multiple of 8");
    if (cache->len < 0 || cache->len + n > cache->capacity) return fail(DG_ERR_CAPACITY, "len + n > capacity");
    const size_t need = dg_prefill_workspace_bytes(m, n);
    if (workspace_bytes < need) return fail(DG_ERR_WORKSPACE, "workspace %zu < %zu", workspace_bytes, need);
    st = check_device();
    if (st != DG_OK) return st;
    StepArgs a{};
    a.only_req = -1;
    a.dtype = m->dtype;
    a.V = m->vocab; a.d = m->d_model; a.Hq = m->n_q_heads; a.Hkv = m->n_kv_heads; a.hd = m->head_dim;
    a.mask_id = m->mask_id; a.eos_id = m->eos_id; a.rope_base = m->rope_base; a.eps = m->norm_eps;
    a.embed = m->embed; a.wq = m->wq; a.wk = m->wk; a.wv = m->wv; a.wo = m->wo; a.lm = m->lm_head;
    a.lm_scale = m->lm_scale; a.lm_fp8 = m->lm_format == DG_LM_FP8 ? 1 : 0;
    if (m->n_layers == 1) {                            // the one layer given through layers[]
        const dg_layer &y = m->layers[0];
        a.wq = y.wq; a.wk = y.wk; a.wv = y.wv; a.wo = y.wo;
        a.sq = y.wq_scale; a.sk = y.wk_scale; a.sv = y.wv_scale; a.so = y.wo_scale;
    }
    a.proj_fp8 = m->proj_format == DG_LM_FP8 ? 1 : 0;
    a.B = 1; a.C = n; a.M = n; a.N = 1;
    a.ids = (int32_t *)ids;
    a.ws = (char *)workspace;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
    a.L.inp = take((size_t)n * 4);
    a.L.r_e = take((size_t)n * 4);
    a.L.rope = take((size_t)n * (m->head_dim / 2) * 8);
    a.L.m_pad = (n + 31) / 32 * 32;
    a.L.gemm_part = take(gemm_part_bytes(m->dtype, m->d_model, m->n_q_heads, m->n_kv_heads, m->head_dim, n));
    a.L.err = take(16);
    a.reqs.k[0] = cache->k; a.reqs.v[0] = cache->v;
    a.reqs.cap[0] = cache->capacity; a.reqs.len[0] = cache->len;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_clear_err(a, s);
    if (e == hipSuccess) e = launch_rope_table(a, s);
    if (e == hipSuccess) e = launch_prep(a, 2, s);
    if (e == hipSuccess) e = launch_qkv(a, 1, WRITE_ALWAYS, s);
    if (e != hipSuccess) return fail(DG_ERR_DEVICE, "prefill launch: %s", hipGetErrorString(e));
    cache->len += n;
    return DG_OK;
}

extern "C" const int32_t *dg_error_word(const dg_canvas *c) {
    return c ? (const int32_t *)(c->a.ws + c->a.L.err) : nullptr;
}

static const char *kind_names[DG_NUM_KERNEL_KINDS] = {
    "reset", "prep_rows", "qkv_rope", "attention", "attn_merge", "out_proj",
    "rowscale_h", "lmhead_sampler", "sample_commit", "append", "debug_copy", "ffn", "moe"};

extern "C" const char *dg_kernel_kind_name(int32_t kind) {
    return (kind >= 0 && kind < DG_NUM_KERNEL_KINDS) ? kind_names[kind] : "?";
}

extern "C" dg_status dg_profile_enable(dg_canvas *c, uint32_t kind_mask) {
    if (!c) return fail(DG_ERR_NULL, "handle is NULL");
    c->prof = kind_mask & ((1u << DG_NUM_KERNEL_KINDS) - 1u);
    return DG_OK;
}

extern "C" dg_status dg_profile_read(dg_canvas *c, double *ms, int64_t *launches) {
    if (!c || !ms || !launches) return fail(DG_ERR_NULL, "NULL argument");
    for (int k = 0; k < DG_NUM_KERNEL_KINDS; ++k) { ms[k] = 0; launches[k] = 0; }
    hipError_t e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return fail(DG_ERR_DEVICE, "hipStreamSynchronize: %s", hipGetErrorString(e));
    for (auto &r : c->rec) {
        float t = 0.f;
        if (hipEventElapsedTime(&t, r.e0, r.e1) == hipSuccess) {
            ms[r.kind] += t;
            launches[r.kind] += 1;
        }
        c->pool.push_back(r.e0);
        c->pool.push_back(r.e1);
    }
    c->rec.clear();
    return DG_OK;
}

extern "C" dg_status dg_canvas_set_graph(dg_canvas *c, int32_t on) {
    if (!c) return fail(DG_ERR_NULL, "handle is NULL");
    if (on != 0 && on != 1) return fail(DG_ERR_SHAPE, "on must be 0 or 1, got %d", on);
    c->graph_on = on != 0;
    if (!c->graph_on && c->graph_exec) {
        const hipError_t e = hipStreamSynchronize(c->stream);   // the recorded step may still run
        if (e != hipSuccess) return fail(DG_ERR_DEVICE, "hipStreamSynchronize: %s", hipGetErrorString(e));
        (void)hipGraphExecDestroy(c->graph_exec);
        c->graph_exec = nullptr;
    }
    return DG_OK;
}

extern "C" dg_status dg_canvas_destroy(dg_canvas *c) {
    if (!c) return fail(DG_ERR_NULL, "handle is NULL");
    // the kernels write the pinned flags: nothing may still run when they go
    if (!c->rec.empty() || c->done_host || c->graph_exec) (void)hipStreamSynchronize(c->stream);
    if (c->graph_exec) (void)hipGraphExecDestroy(c->graph_exec);
    if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
    c->graph_exec = nullptr;
    c->cap_stream = nullptr;
    c->graph_on = false;
    for (auto &r : c->rec) { (void)hipEventDestroy(r.e0); (void)hipEventDestroy(r.e1); }
    for (auto e : c->pool) (void)hipEventDestroy(e);
    for (int i = 0; i < RUN_LAG; ++i)
        if (c->run_ev[i]) (void)hipEventDestroy(c->run_ev[i]);
    if (c->done_host) (void)hipHostFree(c->done_host);
    if (c->is_static) {
        if (c->a.ws) (void)hipStreamSynchronize(c->stream);     // the scratch is free once nothing runs on it
        c->rec.clear();
        c->pool.clear();
        c->done_host = nullptr;
        g_static_live[c->device] = false;
        return DG_OK;
    }
    delete c;
    return DG_OK;
}
