// Internal declarations shared by the HIP kernels and the host orchestrator.
// gfx950 only: 64-lane waves, bf16 MFMA 32x32x16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dg.h"

namespace dg {

typedef uint16_t bf16_t;   // raw bf16 bit pattern in memory

// Most requests whose open rows one LM-head workgroup takes together.
constexpr int DG_LM_GROUP_MAX = 8;

// Per-request cache pointers and prefix lengths, passed by value to kernels.
struct Reqs {
    void *k[DG_MAX_BATCH];
    void *v[DG_MAX_BATCH];
    int64_t cap[DG_MAX_BATCH];
    int64_t len[DG_MAX_BATCH];
};

// Which requests a launch works on: denoising steps take the requests not
// done, the append pass the done ones, the prompt prefill every row.
enum Phase : int { PH_STEP = 0, PH_APPEND = 1, PH_PREFILL = 2 };

// Which rows a K/V-writing projection may write.
enum WriteMode : int {
    WRITE_STEP = 0,     // requests that are not done (canvas scratch rows)
    WRITE_APPEND = 1,   // requests that are done (clean canvas rows)
    WRITE_ALWAYS = 2    // prefill
};

// Workspace layout: offsets in bytes from the workspace base.
// q is fp32 [M][Hq][hd] in both paths.  inp[t]: id fed at canvas row t (the
// QKV projection gathers its embedding row).  bf16 path: o (fp16 hi plane
// then fp16 lo plane) is fragment-major (frag_index) over M_pad = M rounded
// up to 32 rows; h (the fp16 operand of the vocabulary product) is
// fragment-major over the compact rows, and hf holds the same rows of h in
// fp32, row-major (the sampler's exact logits of the leading ids).  The f32
// path keeps o and h row-major in fp32.
struct Layout {
    size_t inp, r_e, r_h, rope, q, o, h, hf, attn_ml, attn_acc, lm_part, rowstats, gemm_part, err, total;
    // Deeper models (bf16): the residual stream x between layers, fp32
    // [M][d]; its fp16 hi and lo planes, fragment-major over m_pad rows
    // (operand of the next QKV and FFN projections); its row scale r_x; the
    // FFN activation's fp16 hi and lo planes, fragment-major [m_pad][d_ff].
    size_t x, xp, r_x, act;
    // Positions still uncommitted at the start of a step, per request: the
    // vocabulary head and sampler work on these compact rows only (row
    // r = b * cp + j, j < ucount[b]).  ulist[r]: canvas position of compact
    // row r; uidx[t]: compact index of canvas row t, -1 if committed.
    size_t ulist, uidx, ucount;
    size_t sample_cnt;  // int32 [B]: workgroups of the sampler kernel that have arrived
    size_t escale;      // float [V], RMSNorm scale of every embedding row (if has_escale)
    int has_escale;     // bf16 canvas handles: the QKV projection takes row scales from escale
    int cp;             // C rounded up to 32: compact rows per request
    int rows_c;         // B * cp
    int m_pad;
    int n_split_max;
    int n_slices;       // vocabulary slices of the LM-head kernel; lm_part holds
                        // float4 records [rows_c][n_slices] (a row's records
                        // contiguous): (m, sum exp, m2, ids of m and m2 as
                        // 16-bit offsets from the slice's first id); lm_tpart holds
                        // the matching t = sum (z - m) exp(z - m) as floats
                        // (written only under the entropy stop)
    size_t lm_tpart;
    size_t lm_kpart;    // temperature sampling: float4 records [rows_c][n_slices] of the two
                        // largest perturbed logits z / T + g and their ids (packed as in lm_part)
    size_t rowent;      // float [M]: entropy of softmax(z) per canvas row (open rows)
    // Routed experts (models with experts): x as row-major fp16 hi and lo
    // planes [2][M][d] (the experts gather their tokens' rows from it); the
    // router logits [M][E]; each layer's choices [L][M][k] and the current
    // layer's gates [M][k]; per expert its token count, the start of its
    // rows (multiples of 32) in the expert-grouped slot list [mk_pad] (slot
    // t k + j, -1 past the count); the experts' activations, fp16 hi and lo
    // planes fragment-major [2][mk_pad][d_e]; their gated outputs, fp32
    // [M k][d] (slot order).
    size_t xr, moe_logit, moe_sel, moe_gate, moe_cnt, moe_off, moe_list, moe_act, moe_y;
    size_t moe_ids;     // int32 [1 + E]: the count of chosen experts, then their ids (ascending)
    size_t moe_xg;      // x of the chosen slots, fp16 hi / lo planes, fragment-major [2][mk_pad][d]
    int mk_pad;
    int slice_width;
};

// Everything a step's kernels need; built once per handle.
struct StepArgs {
    int dtype;
    int V, d, Hq, Hkv, hd, mask_id, eos_id;
    float rope_base, eps;
    const void *embed, *wq, *wk, *wv, *wo, *lm;
    const float *lm_scale;  // per-row scales of an e4m3 head (lm_fp8)
    int lm_fp8;
    int B, C, M;
    int N;
    int adaptive;       // 1: stop on max-probability >= tau; 2: on entropy <= h_max
    float tau;
    float h_max;
    int ent;            // the step computes per-row entropies (entropy stop or dump)
    int n_layers, d_ff; // layers (1: the one layer of wq..wo) and FFN width (0: none)
    int layer;          // the layer this launch works on (its weights and cache plane)
    int phase;          // Phase: which requests are active
    int causal;         // attention: canvas position i sees keys 0 .. len + i only (context encoding)
    int only_req;       // >= 0: the launch works on this request alone (per-request append); -1: all
    const void *wg, *wu, *wd;   // the layer's FFN weights
    int n_experts, top_k, d_e;  // routed experts beside the FFN (0: none), experts per token, width
    const void *wr, *wge, *wue, *wde;   // the layer's router and expert weights
    int proj_fp8;       // the layer's projections are e4m3 bytes with per-output-row scales
    const float *sq, *sk, *sv, *so, *sg, *su, *sd;   // those scales (proj_fp8)
    int commit_rule;    // 1: also commit every open position with conf >= tau_c
    float tau_c;
    int fill;           // 1: uncommitted positions are fed their candidate id
    float temp0, temp1; // temperature sampling (temp0 > 0): T_s linear from temp0 to temp1
    uint64_t seed;      // key of the Philox draws
    int32_t *ids;
    uint8_t *committed;
    int32_t *step, *n_steps_done, *n_valid, *done;
    int32_t *done_host;   // [B] pinned host copy of done (written by the kernels), or null
    char *ws;
    Layout L;
    Reqs reqs;
    int attn_split[DG_MAX_BATCH];   // key splits of each request's attention (bf16), set per step
};

// Kernel kinds for per-launch timing.
enum Kind : int {
    K_RESET = 0, K_PREP, K_QKV, K_ATTN, K_ATTN_MERGE, K_OPROJ, K_ROWSCALE,
    K_LMHEAD, K_SAMPLE, K_APPEND, K_DEBUG, K_FFN, K_MOE, K_NUM
};
static_assert(K_NUM == DG_NUM_KERNEL_KINDS, "kind count");

// ---- layout helpers (host) ----
size_t align_up(size_t x, size_t a);
int lm_slice_width(int dtype);
int attn_base_wgs(int dtype, int B, int Hq, int Hkv, int C);
int attn_n_split(int dtype, int B, int Hq, int Hkv, int C, int64_t total_keys);
// Key splits per request for the current cache lengths (len[b] + C keys);
// returns the largest, which sizes the grid.
int attn_splits(int dtype, int B, int Hq, int Hkv, int C, const int64_t *len, int *split);
// d_ff > 0 or deep: the buffers of stacked layers (x, its planes, r_x) and
// of the FFN (activation planes, the down projection's partial sums).
struct MoeShape {
    int n_layers = 1, E = 0, k = 0, de = 0;
};
Layout make_layout(int dtype, int V, int d, int Hq, int Hkv, int hd, int B, int C, int64_t max_prefix,
                   int d_ff = 0, bool deep = false, MoeShape moe = MoeShape{});
// Skinny bf16 GEMMs: token tiles of 128*TM rows and a K split into S chunks
// of whole 64-wide stages, chosen so that the grid covers the 256 CUs.
int gemm_tm(int M);
int gemm_splitk(int tiles, int K);
// Output / down projection to d features over K inputs: token tiles of
// 32 wpg rows, kh parts of a chunk inside a workgroup, S chunks across
// workgroups (fp32 partial sums, added by the residual finish).
struct ProjShape {
    int wpg, kh, S;
};
ProjShape oproj_shape(int M, int d, int K);
size_t gemm_part_bytes(int dtype, int d, int Hq, int Hkv, int hd, int M, int d_ff = 0);

// ---- launchers (return hipGetLastError of the launch) ----
// Source of a projection's token operand, and destination of a residual.
enum Src : int { SRC_EMBED = 0, SRC_RESID = 1 };
enum Out : int { OUT_LMHEAD = 0, OUT_RESID = 1 };
// slot >= 0: reset request `slot` alone, its initial ids / flags given as
// [C] rows (NULL: all MASK, nothing committed); slot < 0: every request,
// [B, C].
hipError_t launch_reset(const StepArgs &a, const int32_t *init_ids, const uint8_t *init_committed,
                        hipStream_t s, int slot = -1);
hipError_t launch_rope_table(const StepArgs &a, hipStream_t s);
hipError_t launch_prep(const StepArgs &a, int force_committed, hipStream_t s);
hipError_t launch_qkv(const StepArgs &a, int kv_only, int mode, hipStream_t s, int src = SRC_EMBED);
// n_split: the largest of a.attn_split (grid depth).
hipError_t launch_attention(const StepArgs &a, int n_split, hipStream_t s);
// odump: optional fp32 [M][Hq*hd] copy of the attention output (bf16 path).
hipError_t launch_attn_merge(const StepArgs &a, int n_split, float *odump, hipStream_t s);
// hdump: optional fp32 [M][d] copy of the residual stream h (bf16 path).
// src: residual the projection adds to (the embedding rows or x); out: the
// vocabulary head's operand (last layer) or the next projection's planes.
hipError_t launch_oproj(const StepArgs &a, float *hdump, hipStream_t s, int src = SRC_EMBED, int out = OUT_LMHEAD);
// SwiGLU FFN of layer a.layer: up / gate projection with the activation,
// then the down projection with the residual.
hipError_t launch_ffn(const StepArgs &a, float *hdump, hipStream_t s, int out);
hipError_t launch_moe(const StepArgs &a, hipStream_t s);
hipError_t launch_rowscale_h(const StepArgs &a, hipStream_t s);
// ev0/ev1 (optional, both or neither): events stamped with the kernel's own
// start and end (hipExtLaunchKernelGGL; recorded around the launch on the
// fp32 path).
// bp: requests per workgroup (1, 2, 4 or 8), chosen by the host so that
// bp open-row counts fit 8 row tiles of 32; a group over that is counted in
// error-word slot 2 and left uncomputed.
hipError_t launch_lmhead(const StepArgs &a, float *logits_dump, int bp, hipStream_t s,
                         hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
// Vocabulary-statistics merge and, in its last workgroup per request, the
// commit / re-mask / stop update.
hipError_t launch_sample_commit(const StepArgs &a, hipStream_t s);
// Compact lists of uncommitted positions from the committed flags as they
// are (used when a handle resumes caller-provided state).
hipError_t launch_ulist(const StepArgs &a, hipStream_t s);
hipError_t launch_escale(const StepArgs &a, hipStream_t s);
hipError_t launch_clear_err(const StepArgs &a, hipStream_t s);


}  // namespace dg
