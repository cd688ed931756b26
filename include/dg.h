/*
 * dg.h — C-ABI of the MI355X (gfx950) block-discrete-diffusion canvas step.
 *
 * The problem these calls implement is the one the DiffusionGemma pages state:
 *   - a canvas of C tokens over a vocabulary of V ids is refined in parallel
 *     by repeated forward passes (DiffusionGemma Technical Report, Abstract
 *     and section 2.1);
 *   - canvas queries attend bidirectionally to every canvas position and to
 *     a read-only KV cache of the prompt and earlier canvases (report
 *     section 1; section 4, block-diagonal mask with the clean context read
 *     through the encoder KV cache);
 *   - confident positions lock first while the rest stay open (blog
 *     "Google Releases DiffusionGemma ...", section "Once Written, a Prefix
 *     Becomes History"), for at most N steps, with adaptive stopping
 *     (report section 3.3);
 *   - a finished canvas costs one more forward that appends its K/V to the
 *     cache (report section 3.4, the K-1 term of eq. (10)), and its valid
 *     length ends at the first end-of-sequence id (same section, C_k).
 *
 * Conventions common to every call:
 *   - All device buffers (weights, caches, canvas state, workspace) are
 *     allocated and owned by the caller and must outlive the handle.  The
 *     library never allocates or frees device memory; a handle holds a few
 *     bytes of pinned host memory for the done flags (dg_run_canvas).
 *   - Calls enqueue work on the stream given at init and return without
 *     waiting, except where stated: dg_run_canvas (keeps at most 2 steps in
 *     flight; with a stats pointer it waits at the end), dg_append_canvas_kv
 *     and dg_canvas_resume (and dg_canvas_init with DG_INIT_RESUME) wait
 *     once.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     non-OK status means nothing was enqueued (except DG_ERR_DEVICE, which
 *     reports a HIP error raised while enqueueing).  No call aborts or
 *     throws; dg_last_error() describes the last non-OK status of the
 *     calling thread.
 *   - A handle must be used from one thread at a time.
 *   - Only gfx950 devices are supported.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DG_MAX_BATCH 32      /* requests (slots) per handle                 */
#define DG_MAX_CANVAS 256    /* canvas positions per request                */

typedef enum {
    DG_OK = 0,
    DG_ERR_NULL = -1,        /* a required pointer is NULL                  */
    DG_ERR_SHAPE = -2,       /* sizes inconsistent or outside what the kernels support */
    DG_ERR_CAPACITY = -3,    /* a cache cannot hold the rows to be written  */
    DG_ERR_STATE = -4,       /* call not allowed in the handle's state      */
    DG_ERR_DEVICE = -5,      /* HIP error while enqueueing                  */
    DG_ERR_UNSUPPORTED = -6, /* device is not gfx950, or unknown dtype      */
    DG_ERR_WORKSPACE = -7    /* workspace smaller than dg_*_workspace_bytes */
} dg_status;

typedef enum { DG_F32 = 0, DG_BF16 = 1 } dg_dtype;

/* Storage of the vocabulary head. */
typedef enum {
    DG_LM_NATIVE = 0,        /* lm_head in the model dtype                   */
    DG_LM_FP8 = 1            /* lm_head as OCP FP8 E4M3 bytes ("fn": no inf,
                                largest finite 448) [V, d] plus one fp32 scale
                                per vocabulary row in lm_scale [V]; bf16 models
                                only.  z_v = r(h) * lm_scale[v] * (h .
                                e4m3(W_v)).  The pages serve the model in FP8
                                without fixing a format; this is one.        */
} dg_lm_format;

/* Model weights, device pointers, nn.Linear layout [out, in], row-major,
 * element type `dtype` (bf16 as raw 16-bit patterns).  One attention layer
 * with a vocabulary head:
 *   embed   [V, d]          token embedding E
 *   wq      [Hq*hd, d]      query projection
 *   wk, wv  [Hkv*hd, d]     key / value projections
 *   wo      [d, Hq*hd]      attention output projection
 *   lm_head [V, d]          vocabulary head (may equal embed: tied)
 * Uncommitted canvas slots are fed as mask_id and the sampler never proposes
 * mask_id.  eos_id < 0 disables end-of-sequence handling.  RMSNorm has unit
 * gain: r(x) = (mean(x^2) + norm_eps)^-1/2; RoPE uses half-split pairs with
 * angle pos * rope_base^(-2j/hd).
 * Supported: 1 <= Hkv, Hq % Hkv == 0; bf16: d % 256 == 0 and hd in {64,128,256};
 * f32: hd even, hd <= 256.
 *   lm_format / lm_scale: see dg_lm_format (zero: lm_head in `dtype`, and
 *   lm_scale is ignored).  Errors: UNSUPPORTED (unknown format, FP8 head in
 *   an f32 model), NULL (FP8 head without lm_scale). */
typedef struct dg_layer dg_layer;
typedef struct dg_model {
    int32_t vocab, d_model, n_q_heads, n_kv_heads, head_dim;
    int32_t mask_id;
    int32_t eos_id;
    int32_t dtype;            /* dg_dtype */
    float rope_base;
    float norm_eps;
    const void *embed;
    const void *wq, *wk, *wv;
    const void *wo;
    const void *lm_head;
    int32_t lm_format;        /* dg_lm_format */
    const float *lm_scale;    /* DG_LM_FP8: device fp32 [V] */
    int32_t n_layers;         /* 0: the one layer above, no FFN; >= 1: layers[] */
    int32_t d_ff;             /* width of every layer's SwiGLU FFN, 0 = none */
    const dg_layer *layers;   /* host [n_layers] (read at init), see dg_layer */
    int32_t proj_format;      /* dg_lm_format values for every layer's projection
                                 weights (wq, wk, wv, wo, w_gate, w_up, w_down):
                                 DG_LM_FP8 stores each as E4M3 bytes [out, in]
                                 with one fp32 scale per output row in the
                                 layer's *_scale arrays, W[n, :] = s_n e4m3(row n),
                                 the convention of the FP8 head; bf16 models
                                 with n_layers >= 1 only (the weights are read
                                 from layers[]).  Errors: UNSUPPORTED, NULL
                                 (a scale array missing). */
    int32_t n_experts;        /* routed experts per layer beside the FFN, 0 = none */
    int32_t top_k;            /* experts per token */
    int32_t d_expert;         /* width of each expert's SwiGLU block */
} dg_model;

/* One transformer layer of a deeper model (device pointers, [out, in]
 * row-major, model dtype; the backbone is a stack of such layers:
 * DiffusionGemma Technical Report, Abstract and section 1):
 *   wq, wk, wv, wo   as in dg_model;
 *   w_gate, w_up [d_ff, d], w_down [d, d_ff]: a pre-norm dense SwiGLU block
 *   after the attention, x <- x + (silu(r x Wg^T) * (r x Wu^T)) Wd^T with
 *   r = (mean(x^2) + norm_eps)^-1/2 (NULL when d_ff == 0).
 * Layer l attends over its own KV cache plane (dg_kv_cache); the logits
 * read the residual stream after the last layer.  Deeper models and FFNs
 * need the bf16 path, d_ff % 256 == 0 and L <= DG_MAX_LAYERS. */
#define DG_MAX_LAYERS 16
struct dg_layer {
    const void *wq, *wk, *wv;
    const void *wo;
    const void *w_gate, *w_up;
    const void *w_down;
    /* proj_format DG_LM_FP8: device fp32 per-output-row scales of the
     * weights above ([Hq*hd], [Hkv*hd], [Hkv*hd], [d], [d_ff], [d_ff], [d]);
     * ignored otherwise */
    const float *wq_scale, *wk_scale, *wv_scale;
    const float *wo_scale;
    const float *w_gate_scale, *w_up_scale;
    const float *w_down_scale;
    /* n_experts > 0: a mixture of experts beside the FFN, which is then its
     * shared expert (DiffusionGemma Technical Report, part 3, section 6: the
     * MoE layer, its experts chosen per token, and the shared expert).  On
     * the FFN's normed input a = r x: router logits l = a w_router^T, each
     * token's top_k experts by logit (ties to the lower expert id), gates =
     * softmax of the chosen logits, and
     *   x <- x + shared(a) + sum_j g_j (silu(a Wge[e_j]^T) * (a Wue[e_j]^T)) Wde[e_j]^T.
     * Model dtype (bf16), row-major:
     *   w_router      [E, d]
     *   w_expert_gate [E, d_expert, d],  w_expert_up [E, d_expert, d]
     *   w_expert_down [E, d, d_expert]
     * Needs d_ff > 0 (the shared expert), 1 <= top_k <= min(E, 16),
     * E <= 256, d_expert % 256 == 0.  The pages fix none of these shapes. */
    const void *w_router;
    const void *w_expert_gate, *w_expert_up;
    const void *w_expert_down;
};

/* KV cache of one request (device memory, element type = model dtype).
 *   k: [L][Hkv][capacity][hd]   keys after RoPE, one row per position
 *   v: [L][Hkv][hd][capacity]   values stored transposed (position fastest)
 * (L = max(1, n_layers) planes, one per layer, back to back.)
 * Rows [0, len) hold the read-only prefix.  capacity must be a multiple of 8.
 * During denoising the library uses rows [len, len + C) as scratch for the
 * canvas keys/values of the current step. */
typedef struct dg_kv_cache {
    void *k;
    void *v;
    int64_t capacity;
    int64_t len;
} dg_kv_cache;

/* Sampler: N-step budget.  Adaptive stop: a step commits every open
 * position (and the canvas ends) once every position its schedule leaves
 * open is sure:
 *   adaptive_stop 0: off;
 *                 1: sure = confidence (max probability) >= stop_conf;
 *                 2: sure = entropy of the position's distribution over the
 *                    vocabulary (nats) <= stop_entropy.
 *   commit_rule 0: step s commits the k_s = ceil(|U| / (N - s + 1)) most
 *                  confident uncommitted positions (the schedule);
 *               1: it commits every uncommitted position with confidence
 *                  >= commit_conf, and at least the schedule's k_s.
 *   canvas_fill 0: uncommitted positions are fed MASK;
 *               1: uncommitted positions are fed their candidate token: the
 *                  id the state holds for them at init/reset (e.g. a uniform
 *                  draw), then the greedy token of their previous step, which
 *                  the sampler writes into ids (committed stays 0).
 *   temperature > 0: temperature sampling with annealing (report section 5,
 *                  the online teacher's sampler): at step s the temperature
 *                  is T_s = temperature + (temperature_end - temperature)
 *                  (s - 1) / (N - 1); an open position proposes the
 *                  Gumbel-max draw argmax_v z_v / T_s + g_v (lowest id on a
 *                  tie) instead of its greedy token, and its confidence (for
 *                  the ranking, the threshold and the stop) is the draw's
 *                  probability under softmax(z).  g_v = -ln(-ln u), u = (the
 *                  top 24 bits of word v & 3 of Philox4x64-10 with counter
 *                  (v >> 2, position, step, request index) and key (seed, 0)
 *                  + 1/2) / 2^24; bf16 models only.  0: greedy.
 * Zero-initialised fields give the schedule and the MASK canvas. */
typedef struct dg_sampler {
    int32_t n_steps;
    int32_t adaptive_stop;
    float stop_conf;
    int32_t commit_rule;
    float commit_conf;
    int32_t canvas_fill;
    float stop_entropy;
    float temperature;
    float temperature_end;
    uint64_t seed;
} dg_sampler;

/* Canvas state, device memory owned by the caller:
 *   ids        int32 [B, C]   token ids (meaningful where committed)
 *   committed  uint8 [B, C]   1 = locked
 *   step, n_steps_done, n_valid, done   int32 [B]
 * step = steps executed on the canvas; n_valid = C_k once done.  The
 * handle reads and writes them on its stream; a caller that changes them
 * between steps calls dg_canvas_resume before the next step. */
typedef struct dg_canvas_state {
    int32_t *ids;
    uint8_t *committed;
    int32_t *step;
    int32_t *n_steps_done;
    int32_t *n_valid;
    int32_t *done;
} dg_canvas_state;

typedef struct dg_canvas_stats {   /* host, one per request */
    int32_t n_steps_done;
    int32_t n_valid;
} dg_canvas_stats;

/* Optional stage dumps for checking (device pointers, NULL = skip):
 *   q        [B*C, Hq*hd]  float32, queries after RoPE
 *   o        [B*C, Hq*hd]  float32, attention output
 *   h        [B*C, d]      float32, residual stream after the layer
 * Precision of the bf16 path: the canvas K / V rows are stored in the cache
 * as bf16; q, o and h are held in fp32.  The vocabulary head multiplies h
 * rounded to fp16 with the LM-head rows (converted from bf16 to fp16, exact
 * for magnitudes in [2^-14, 65504]) and scales by the RMS of the fp32 h;
 * the logits of each row's two leading ids are then recomputed from the
 * fp32 h, and the max logit, second logit, greedy id, sum of exponentials
 * and entropy are corrected with them.  The full-logits dump holds the
 * fp16-operand logits.
 *   row_stats float32 [B*C, 4] per position: max logit m, sum_v exp(z_v - m),
 *            second largest logit, greedy id (int32 bit pattern)
 *   logits   float32 [B*C, V] full logits (MASK column = -inf); slow path
 *   entropy  float32 [B*C]   per position: -sum_v p_v ln p_v of softmax(z)
 * The vocabulary head and the sampler run only on the positions still
 * uncommitted at the start of the step (a committed position's logits are
 * never read); row_stats, entropy and logits rows of committed positions
 * are left as they were.  The dumps are copies of what the step computed; they do
 * not change it. */
typedef struct dg_debug {
    void *q;
    void *o;
    void *h;
    float *row_stats;
    float *logits;
    float *entropy;
    int32_t *moe_sel;   /* int32 [n_layers, B*C, top_k]: each layer's chosen experts
                           per position, in (logit desc, id asc) order (models
                           with experts; rows of finished requests as they were) */
} dg_debug;

typedef struct dg_canvas dg_canvas;   /* opaque host handle */

#define DG_INIT_RESUME 1u   /* keep the state buffers as they are (resume) */

/* Bytes of workspace a handle needs for `batch` canvases of `canvas_len`
 * positions whose caches hold at most `max_prefix` rows before the canvas.
 * Returns 0 if the shapes are unsupported. */
size_t dg_workspace_bytes(const dg_model *m, int32_t batch, int32_t canvas_len,
                          int64_t max_prefix);

/* Bind buffers and enqueue the canvas reset.
 *   caches      [batch] array, caller-owned, must outlive the handle; the
 *               library updates caches[b].len when it appends
 *   init_ids / init_committed: device [batch, C] or NULL (all MASK, nothing
 *               committed).  Pre-committed positions (e.g. an EOS already
 *               fixed) are kept and never re-sampled.
 *   flags       DG_INIT_RESUME: leave the state buffers untouched
 *   stream      hipStream_t to enqueue on (NULL = default stream)
 *   workspace   device, owned by the handle until dg_canvas_destroy; it
 *               keeps per-row state from one step to the next (the input
 *               rows of the next step, written as positions are committed),
 *               so neither it nor the weights may change while the handle
 *               lives (reset and resume rebuild that state)
 * Errors: NULL, SHAPE (batch outside [1,16], C outside [1,256], model
 * unsupported), CAPACITY (len + C > capacity, capacity % 8 != 0), WORKSPACE,
 * UNSUPPORTED (not gfx950), DEVICE. */
dg_status dg_canvas_init(dg_canvas **out, const dg_model *m, const dg_sampler *smp,
                         dg_kv_cache *caches, int32_t batch, int32_t canvas_len,
                         const dg_canvas_state *state, const int32_t *init_ids,
                         const uint8_t *init_committed, uint32_t flags,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Allocation-free variant of dg_canvas_init, for callers that cannot
 * allocate memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments and behaviour except:
 *   - no workspace argument: the handle uses a device array inside the
 *     library of DG_STATIC_SCRATCH_BYTES bytes (each GPU holds its own copy
 *     from the library's first use on it until the process ends); shapes
 *     whose dg_workspace_bytes exceed it are refused with WORKSPACE;
 *   - the handle is a library-owned object, one per device: while it lives,
 *     another dg_canvas_init_static on the same device returns STATE;
 *     dg_canvas_destroy releases it (and frees nothing);
 *   - the call allocates nothing, device or host (dg_profile_enable on such
 *     a handle may allocate host memory for its event records);
 *   - without a pinned host buffer, dg_run_canvas on this handle enqueues
 *     the whole budget N (steps of finished requests exit early on the
 *     device) instead of stopping after the done flags.
 * The array keeps the contents of the last handle that used it; init clears
 * and rebuilds everything the step reads from it.  Work of two handles that
 * overlap in time on one GPU would race on it; the STATE check above keeps
 * handles of this process apart, not work still running from a destroyed
 * handle on another stream (destroy waits for the handle's own stream). */
#define DG_STATIC_SCRATCH_BYTES (64u << 20)
dg_status dg_canvas_init_static(dg_canvas **out, const dg_model *m, const dg_sampler *smp,
                                dg_kv_cache *caches, int32_t batch, int32_t canvas_len,
                                const dg_canvas_state *state, const int32_t *init_ids,
                                const uint8_t *init_committed, uint32_t flags, void *stream);

/* Enqueue one denoising step for every request that is not done: forward
 * pass over (prefix || canvas), vocabulary statistics, commit / re-mask /
 * adaptive stop.  A finished request is left untouched.  dbg may be NULL.
 * Errors: NULL, STATE (canvas already appended), DEVICE. */
dg_status dg_denoise_step(dg_canvas *c, const dg_debug *dbg);

/* Enqueue steps until every request is done (adaptive stop or the last
 * position committed; report section 3.3) or has had N steps since its
 * canvas (re)started.
 * To see the done flags without a round trip per step it keeps at most 3
 * steps in flight: before enqueueing a step it waits for the step 2 before
 * it and reads the done flags that step's sampler wrote into a pinned host
 * buffer of the handle; after a stop at most 1 step follows, as early-exit
 * launches.  With out != NULL, waits for the stream and fills out[b].
 * Errors: NULL, STATE (canvas already appended), DEVICE. */
dg_status dg_run_canvas(dg_canvas *c, dg_canvas_stats *out);

/* Enqueue the append pass: the K/V rows of each finished canvas are computed
 * from its clean ids at positions len .. len+C-1 and written into its cache;
 * then len += C (report section 3.4: one more forward per finished canvas,
 * the K-1 term of eq. (10); blog section "Once Written, a Prefix Becomes
 * History": the canvas becomes read-only prefix).  It first reads the done
 * flags (waits for the stream once): if any request is not done it returns
 * STATE and enqueues nothing, so no cache row or length changes.
 * Afterwards the handle accepts only dg_canvas_reset or dg_canvas_destroy.
 * Errors: NULL, STATE (already appended, or a request not done), CAPACITY,
 * DEVICE. */
dg_status dg_append_canvas_kv(dg_canvas *c);

/* ---- continuous batching ------------------------------------------------
 * The B requests of a handle are slots that finish at different steps.  A
 * serving loop keeps them busy: it runs steps until some watched slot is
 * done, then either appends that request's canvas to its cache and starts
 * its next canvas in the same slot, or hands the slot a new request; the
 * other slots carry on without a pause (blog "Google Releases
 * DiffusionGemma ...", section "Test Conditions Behind 1,456 Tokens per
 * Second ...": several requests batched together, with the ~32-request
 * crossover against autoregressive decoding; DG_MAX_BATCH is 32 to reach
 * it).  A slot's step counter, open positions, statistics and done flag
 * restart with it; the schedule of eq. (8) and the budget N then count from
 * its own restart.  These calls and dg_append_canvas_kv / dg_canvas_reset
 * (which act on every slot at once) may be mixed. */

/* Enqueue steps as dg_run_canvas does, and stop early also once a request
 * whose bit b is set in stop_mask is seen done; at most max_steps steps.
 * Flags are seen with the lag of dg_run_canvas (checks start at the
 * call's third step, each after waiting for the step 2 before it).  n_run
 * (may be NULL) gets the number of steps enqueued; done_mask (may be NULL)
 * gets bit b set for each done request, as of the last check when the call
 * stopped on one, else after waiting for the stream.
 * Errors: NULL, STATE (canvas already appended), SHAPE (max_steps < 0),
 * DEVICE. */
dg_status dg_run_steps(dg_canvas *c, int32_t max_steps, uint32_t stop_mask, int32_t *n_run,
                       uint32_t *done_mask);

/* Append request b's finished canvas to its cache (the pass of
 * dg_append_canvas_kv for that request alone; report section 3.4) and start
 * its next canvas in the same slot at the new length: ids from init_ids
 * [C] / init_committed [C] (device, may be NULL: every position masked and
 * open).  The done check reads the handle's pinned flag (a flag once seen
 * set is final for the request) and otherwise waits for the stream once.
 * Errors: NULL, STATE (request b not done, or canvas already appended),
 * SHAPE (b outside [0, B)), CAPACITY (len + 2C > capacity: no room for this
 * canvas and the next), DEVICE. */
dg_status dg_append_request_kv(dg_canvas *c, int32_t b, const int32_t *init_ids,
                               const uint8_t *init_committed);

/* Give slot b a new request: its cache (the caller's struct, which must
 * outlive the slot's use; len is its prefix length, capacity at least
 * len + C) and its first canvas (init_ids / init_committed as for
 * dg_append_request_kv).  The slot's previous request, done or not, is
 * dropped: a request still running is pre-empted, and its done flag may
 * read set until the reset enqueued here has run.  A cache longer than
 * those given at init needs no more workspace (the attention split count
 * is bounded by what the workspace holds).
 * Errors: NULL, STATE (canvas already appended), SHAPE (b outside [0, B)),
 * CAPACITY / SHAPE (cache checks of dg_canvas_init), DEVICE. */
dg_status dg_canvas_admit(dg_canvas *c, int32_t b, dg_kv_cache *cache, const int32_t *init_ids,
                          const uint8_t *init_committed);

/* The handle's pinned host array of done flags ([B] int32, written by the
 * sampler as requests finish, cleared when a slot restarts), or NULL for a
 * handle without one (dg_canvas_init_static).  Valid until destroy. */
const volatile int32_t *dg_done_flags(const dg_canvas *c);

/* Start the next canvas after an append (or restart the current one):
 * state reset as in dg_canvas_init.  The canvas starts at the len of slot
 * b's cache struct (caches[b] of init, or the one given to dg_canvas_admit)
 * as the caller holds it now (normally the length after the append; a
 * caller may set a shorter length to drop rows, e.g. to redo a canvas).
 * Errors: NULL, CAPACITY (len + C > capacity), SHAPE. */
dg_status dg_canvas_reset(dg_canvas *c, const int32_t *init_ids, const uint8_t *init_committed);

/* The caller has written the state buffers (ids, committed, step, done)
 * since the last call on the handle: rebuild what the handle derives from
 * them (the list of open positions, the input rows of the next step) and
 * read back each request's open-position count and step counter (waits
 * for the stream once), from which the host bounds the open positions of
 * later steps.  Between calls the state buffers belong to the handle; a
 * caller that writes them must call this before the next dg_denoise_step
 * or dg_run_canvas.  dg_run_canvas afterwards enqueues steps until each
 * request's step counter reaches N (steps of finished requests are no-ops).
 * Errors: NULL, STATE (canvas already appended), DEVICE. */
dg_status dg_canvas_resume(dg_canvas *c);

/* Prefill: encode n prompt ids (device int32 [n]) at positions len..len+n-1
 * and append their K/V rows to one cache; cache->len += n.  Uses its own
 * workspace of dg_prefill_workspace_bytes(m, n) bytes.  One-layer models
 * only (a token's K/V rows then depend on the token and its position
 * alone); deeper models encode context through dg_append_canvas_kv, whose
 * causal pass this call would need.  Errors: UNSUPPORTED for n_layers > 1
 * or d_ff > 0, and those of dg_canvas_init. */
size_t dg_prefill_workspace_bytes(const dg_model *m, int32_t n);
dg_status dg_prefill_kv(const dg_model *m, dg_kv_cache *cache, const int32_t *ids,
                        int32_t n, void *workspace, size_t workspace_bytes, void *stream);

/* Device error word of the handle (device int32 [4]): [0] append requests
 * skipped on the device because their canvas was not done (the host check
 * of dg_append_canvas_kv leaves this at zero); [1] canvas ids outside the
 * vocabulary (fed as MASK); [2] vocabulary-head workgroups whose group of
 * requests held more open rows than the step's bound (not computed; zero
 * unless the state was changed behind the handle's back without
 * dg_canvas_resume). */
const int32_t *dg_error_word(const dg_canvas *c);

/* Recorded steps.  The step's time is its kernels' time plus the host's
 * cost of issuing them (DiffusionGemma Technical Report, part 3, section 6,
 * "GPU time breakdown", which separates the two).  on = 1: every later
 * dg_denoise_step without a debug dump and without kernel timing (and every
 * step of dg_run_steps / dg_run_canvas) issues one HIP graph launch on the
 * handle's stream instead of the step's separate kernel launches.  The graph
 * is recorded on a private stream of the handle at the first such step and
 * recorded again whenever the step's launch arguments change (an append, a
 * slot restart or admission, a different key split or vocabulary-head
 * group); its results are those of the separate launches, bit for bit.  on =
 * 0 waits for the handle's stream and frees the recorded graph.
 * Errors: NULL, SHAPE (on not 0 or 1), DEVICE (recording or launching the
 * graph failed; the step was not enqueued). */
dg_status dg_canvas_set_graph(dg_canvas *c, int32_t on);

/* Per-kernel timing with HIP events on the handle's stream.  Bit k of
 * kind_mask records every later launch of kernel kind k between two events
 * (0 stops recording); dg_profile_read waits for the stream and returns, per
 * kernel kind, the summed milliseconds and the launch count (arrays of
 * length DG_NUM_KERNEL_KINDS), then clears the record. */
#define DG_NUM_KERNEL_KINDS 13
#define DG_KIND_LMHEAD 7
const char *dg_kernel_kind_name(int32_t kind);
dg_status dg_profile_enable(dg_canvas *c, uint32_t kind_mask);
dg_status dg_profile_read(dg_canvas *c, double *ms, int64_t *launches);

dg_status dg_canvas_destroy(dg_canvas *c);

/* Message for the last non-OK status returned to this thread. */
const char *dg_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
