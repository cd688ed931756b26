// Row-wise kernels of the canvas step: state reset, RoPE table, canvas input
// assembly with the RMS row scale, vocabulary-statistics merge, the sampler's
// commit / re-mask / adaptive stop (with the input rows of the next step),
// and the split-attention merge.
#include <float.h>
#include <limits.h>

#include "dg_device.hpp"
#include "dg_internal.hpp"

namespace dg {

template <typename T> __device__ __forceinline__ float ldx(const T *p, size_t i);
template <> __device__ __forceinline__ float ldx<uint16_t>(const uint16_t *p, size_t i) { return bf2f(p[i]); }
template <> __device__ __forceinline__ float ldx<float>(const float *p, size_t i) { return p[i]; }

template <typename T> __device__ __forceinline__ T stx(float v);
template <> __device__ __forceinline__ uint16_t stx<uint16_t>(float v) { return f2bf(v); }
template <> __device__ __forceinline__ float stx<float>(float v) { return v; }

__device__ __forceinline__ int block_sum_int_256(int v, int *sh) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    int t = sh[0] + sh[1] + sh[2] + sh[3];
    __syncthreads();
    return t;
}

__device__ __forceinline__ int block_min_int_256(int v, int *sh) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    int t = min(min(sh[0], sh[1]), min(sh[2], sh[3]));
    __syncthreads();
    return t;
}

// Id fed at a canvas row: the committed id, else MASK.  An id no embedding
// row exists for is counted in the error word (slot 1) and fed as MASK.
__device__ __forceinline__ int fed_id(const StepArgs &a, int committed, int id, bool count) {
    int tok = committed ? id : a.mask_id;
    if (tok < 0 || tok >= a.V) {
        if (count) atomicAdd((int *)(a.ws + a.L.err) + 1, 1);
        tok = a.mask_id;
    }
    return tok;
}

// ---------------------------------------------------------------------------
// reset: canvas ids/committed from the caller's initial state (or all MASK)
// ---------------------------------------------------------------------------
// Compact list of the positions of request b that the next step samples
// (open != 0), in position order: ulist[b*cp + j] = i, uidx[b*C + i] = j
// (-1 where closed), ucount[b].  One workgroup of 256 threads per request,
// thread i = canvas position i (C <= 256).
__device__ __forceinline__ void build_ulist(const StepArgs &a, int b, int i, int open) {
    __shared__ int wcnt[4];
    const int w = i >> 6, lane = i & 63;
    const uint64_t m = __ballot(open);
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    __syncthreads();
    if (lane == 0) wcnt[w] = __popcll(m);
    __syncthreads();
    int off = 0;
    for (int x = 0; x < w; ++x) off += wcnt[x];
    const int j = off + before;
    if (i < a.C) ((int32_t *)(a.ws + a.L.uidx))[b * a.C + i] = open ? j : -1;
    if (open) ((int32_t *)(a.ws + a.L.ulist))[b * a.L.cp + j] = i;
    if (i == 0) ((int32_t *)(a.ws + a.L.ucount))[b] = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
}

__global__ __launch_bounds__(256) void k_reset(StepArgs a, const int32_t *init_ids,
                                               const uint8_t *init_committed, int slot) {
    const int b = slot >= 0 ? slot : blockIdx.x;
    const int i = threadIdx.x;
    int open = 0;
    if (i < a.C) {
        const int t = b * a.C + i;
        const int ti = slot >= 0 ? i : t;             // a single slot's initial rows are [C]
        const int id = init_ids ? init_ids[ti] : a.mask_id;
        const uint8_t c = init_committed ? (init_committed[ti] ? 1 : 0) : 0;
        a.ids[t] = id;
        a.committed[t] = c;
        // bf16: the fed id, kept up to date by the sampler; f32: nothing fed
        // yet (the input kernel assembles every row at the first step)
        ((int32_t *)(a.ws + a.L.inp))[t] = a.L.has_escale ? fed_id(a, c || a.fill, id, true) : -1;
        open = !c;
    }
    if (i == 0) {
        a.step[b] = 0;
        a.n_steps_done[b] = 0;
        a.n_valid[b] = a.C;
        a.done[b] = 0;
        if (a.done_host) __hip_atomic_store(a.done_host + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        ((int *)(a.ws + a.L.sample_cnt))[b] = 0;
    }
    build_ulist(a, b, i, open);
}

// Lists from the committed flags as the caller left them (resumed state).
__global__ __launch_bounds__(256) void k_ulist(StepArgs a) {
    const int b = blockIdx.x;
    const int i = threadIdx.x;
    const int open = (i < a.C && !a.done[b] && !a.committed[b * a.C + i]) ? 1 : 0;
    if (i < a.C) {
        const int t = b * a.C + i;
        ((int32_t *)(a.ws + a.L.inp))[t] = a.L.has_escale ? fed_id(a, a.committed[t] || a.fill, a.ids[t], true) : -1;
    }
    if (i == 0) {
        ((int *)(a.ws + a.L.sample_cnt))[b] = 0;
        if (a.done_host) __hip_atomic_store(a.done_host + b, a.done[b] ? 1 : 0, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_SYSTEM);
    }
    build_ulist(a, b, i, open);
}

__global__ void k_clear_err(int32_t *err) {
    if (threadIdx.x < 4) err[threadIdx.x] = 0;
}

// ---------------------------------------------------------------------------
// RoPE table: row t of the canvas sits at absolute position len_b + (t % C).
// Angle, cos and sin in double precision, kept as float.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void k_rope_table(StepArgs a) {
    const int t = blockIdx.x;
    const int b = t / a.C;
    const int64_t pos = a.reqs.len[b] + (t % a.C);
    float2 *tab = (float2 *)(a.ws + a.L.rope) + (size_t)t * (a.hd / 2);
    for (int j = threadIdx.x; j < a.hd / 2; j += blockDim.x) {
        const double inv = pow((double)a.rope_base, -2.0 * (double)j / (double)a.hd);
        const double ang = (double)pos * inv;
        double s, c;
        sincos(ang, &s, &c);
        tab[j] = make_float2((float)c, (float)s);
    }
}

// ---------------------------------------------------------------------------
// Canvas input assembly: token fed at row t (MASK where not committed) and
// the RMSNorm row scale of its embedding.
//   force = 0: denoising step; 1: append (only done requests); 2: prefill.
// ---------------------------------------------------------------------------
// Sum of squares of a row of d values with 16-byte loads (d % 8 == 0 for
// bf16, d % 4 == 0 for fp32 is not required: the tail is read one by one).
// ss + the squares of 8 bf16 values, in order, with explicit fmas.
__device__ __forceinline__ float sumsq_bf16x8(float ss, const uint4 &w) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(u[i] << 16), hi = __uint_as_float(u[i] & 0xffff0000u);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
    }
    return ss;
}

template <typename T>
__device__ __forceinline__ float row_sumsq(const T *row, int d) {
    constexpr int V = 16 / sizeof(T);
    float ss = 0.f;
    const int nv = d / V;
    for (int c = threadIdx.x; c < nv; c += 256) {
        const uint4 w = *(const uint4 *)(row + (size_t)c * V);
        if constexpr (sizeof(T) == 2) {
            ss = sumsq_bf16x8(ss, w);
        } else {
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = __uint_as_float(u[i]);
                ss += x * x;
            }
        }
    }
    for (int k = nv * V + threadIdx.x; k < d; k += 256) {
        const float x = ldx<T>(row, k);
        ss += x * x;
    }
    return ss;
}

// With a per-id scale table (bf16 canvas) only the fed id is written; else
// the row scale is computed from the embedding row.  A denoising step
// (force 0, f32 path) skips rows whose fed id is the one fed last time (inp
// keeps it; reset and resume set it to -1).
template <typename T>
__global__ __launch_bounds__(256) void k_prep(StepArgs a, int force) {
    __shared__ float sh[4];
    const int t = blockIdx.x;
    const int b = t / a.C;
    if (a.only_req >= 0 && b != a.only_req) return;   // a per-request append leaves the others alone
    const int tok = fed_id(a, force != 0 || a.committed[t] || a.fill, a.ids[t], threadIdx.x == 0);
    if (force == 1 && threadIdx.x == 0 && (t % a.C) == 0 && !a.done[b])
        atomicAdd((int *)(a.ws + a.L.err), 1);
    if (force == 0 && tok == ((const int32_t *)(a.ws + a.L.inp))[t]) return;
    if (a.L.has_escale) {
        if (threadIdx.x == 0) ((int32_t *)(a.ws + a.L.inp))[t] = tok;
        return;
    }
    const T *row = (const T *)a.embed + (size_t)tok * a.d;
    const float ss = block_sum_256(row_sumsq<T>(row, a.d), sh);
    if (threadIdx.x == 0) {
        ((int32_t *)(a.ws + a.L.inp))[t] = tok;
        ((float *)(a.ws + a.L.r_e))[t] = 1.0f / sqrtf(ss / (float)a.d + a.eps);
    }
}

// RMSNorm scale of every embedding row (bf16 path), once per handle: the
// sampler reads the scale of a committed id from this table.  Same
// arithmetic as the input assembly.
__global__ __launch_bounds__(256) void k_escale(StepArgs a) {
    __shared__ float sh[4];
    const int v = blockIdx.x;
    const uint16_t *row = (const uint16_t *)a.embed + (size_t)v * a.d;
    const float ss = block_sum_256(row_sumsq<uint16_t>(row, a.d), sh);
    if (threadIdx.x == 0) ((float *)(a.ws + a.L.escale))[v] = 1.0f / sqrtf(ss / (float)a.d + a.eps);
}

// RMSNorm row scale of the residual stream h (input of the vocabulary head).
template <typename T>
__global__ __launch_bounds__(256) void k_rowscale_h(StepArgs a) {
    __shared__ float sh[4];
    const int t = blockIdx.x;
    const T *row = (const T *)(a.ws + a.L.h) + (size_t)t * a.d;
    const float ss = block_sum_256(row_sumsq<T>(row, a.d), sh);
    if (threadIdx.x == 0) ((float *)(a.ws + a.L.r_h))[t] = 1.0f / sqrtf(ss / (float)a.d + a.eps);
}

// ---------------------------------------------------------------------------
// Sampler update of one request, run by the last workgroup of the request
// to finish its merge (256 threads).  Commits the k most confident positions
// among the open ones (k = ceil(|U| / (N - s + 1)); confidence = 1 / sum
// exp(z - m), ties to the lower position), re-masks the rest, applies the
// adaptive stop, does the end-of-canvas bookkeeping (C_k = first EOS
// position, else C) and lists the positions the next step samples.  On the
// bf16 path it also records the id fed at each committed row.
//   Inputs loaded by the caller before the merge (no merge changes them):
//   c0 = compact index of position threadIdx.x at step start (-1: closed or
//   padding), id0 = its id, step0 = the request's step counter, cnt = |U|.
// ---------------------------------------------------------------------------
constexpr int KEY_PAD = 32;            // keys past the last one read by the pipelined rank loop

// Row statistics cross from the merging workgroups to the committing one
// through device-scope relaxed atomic stores and loads: the stores write
// through to the device's coherence point and the loads read from it, so a
// completed store (waited for before the counter is incremented) is seen
// by a load issued after the counter says every group has arrived.  No
// cache writeback or invalidation is needed around the counter.
__device__ __forceinline__ void st_dev_f4(float4 *p, const float4 &v) {
    uint64_t *q = (uint64_t *)p;
    __hip_atomic_store(q, ((uint64_t)__float_as_uint(v.y) << 32) | __float_as_uint(v.x), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, ((uint64_t)__float_as_uint(v.w) << 32) | __float_as_uint(v.z), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float4 ld_dev_f4(const float4 *p) {
    const uint64_t *q = (const uint64_t *)p;
    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float4(__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                       __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32)));
}

struct CommitSmem {
    uint64_t key[DG_MAX_CANVAS + KEY_PAD];   // per compact row: S bits << 32 | compact index
    int selc[DG_MAX_CANVAS];           // per compact row: among the k smallest keys
    float ent[DG_MAX_CANVAS];          // per compact row: entropy (entropy stop)
    int shi[4];
};

__device__ __forceinline__ void commit_request(const StepArgs &a, int b, CommitSmem &sm, int cnt, int c0,
                                               int id0, int step0) {
    const int i = threadIdx.x;
    const int t = b * a.C + i;
    const bool unc = c0 >= 0;
    // 1. keys of the open positions, at their compact index (compact order is
    //    position order, so the low word breaks ties to the lower position);
    //    the unused tail reads as +inf
    const float4 st = unc ? ld_dev_f4((const float4 *)(a.ws + a.L.rowstats) + t) : make_float4(0, 0, 0, 0);
    const int arg = __float_as_int(st.w);
    if (unc) sm.key[c0] = ((uint64_t)__float_as_uint(st.y) << 32) | (uint32_t)c0;
    if (unc && a.adaptive == 2)
        sm.ent[c0] = __hip_atomic_load((const float *)(a.ws + a.L.rowent) + t, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    if (i >= cnt) sm.key[i] = ~0ull;
    if (i < KEY_PAD) sm.key[DG_MAX_CANVAS + i] = ~0ull;
    __syncthreads();
    // 2. thread j = compact row j: rank among the cnt keys (S > 0, so its bit
    //    pattern orders like the value).  8 keys per round, the next round's
    //    reads issued before this round's compares.
    const int s = step0 + 1;
    const int left = a.N - s + 1;
    const int k = (left <= 1) ? cnt : (cnt + left - 1) / left;
    int rank = 0;
    float conf = 0.f;
    if (64 * (i >> 6) < cnt) {                         // wave-uniform
        const uint64_t mine = sm.key[i];
        const ulonglong2 *kp = (const ulonglong2 *)sm.key;
        ulonglong2 q[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) q[u] = kp[u];
        for (int j = 0; j < cnt; j += 8) {
            ulonglong2 nx[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) nx[u] = kp[j / 2 + 4 + u];
#pragma unroll
            for (int u = 0; u < 4; ++u) rank += (q[u].x < mine ? 1 : 0) + (q[u].y < mine ? 1 : 0);
#pragma unroll
            for (int u = 0; u < 4; ++u) q[u] = nx[u];
        }
        conf = 1.0f / __uint_as_float((uint32_t)(mine >> 32));
    }
    // threshold rule: the k' = max(k, #{conf >= tau_c}) most confident
    int kk = k;
    if (a.commit_rule) kk = max(k, block_sum_int_256((i < cnt && conf >= a.tau_c) ? 1 : 0, sm.shi));
    const int selc = (i < cnt && rank < kk) ? 1 : 0;
    // adaptive stop: a position left out counts as unsure below tau (max
    // probability) or above h_max (entropy)
    const int low = (i < cnt && !selc && (a.adaptive == 2 ? sm.ent[i] > a.h_max : conf < a.tau)) ? 1 : 0;
    sm.selc[i] = selc;
    bool all = false;
    if (a.adaptive) all = block_sum_int_256(low, sm.shi) == 0;   // nobody left unsure: commit all
    else __syncthreads();
    const int nsel = all ? cnt : kk;
    const bool finished = (cnt - nsel == 0);
    // 3. thread i = position i: commit, re-mask, next step's list
    const int sel = (unc && (all || sm.selc[c0])) ? 1 : 0;
    if (sel || (unc && a.fill)) {
        // committed: the final id; candidate canvas: the position's new
        // candidate (committed stays 0).  bf16: the id fed at this row from
        // the next step on (an argmax is always a valid id; the check only
        // guards the gather)
        a.ids[t] = arg;
        if (sel) a.committed[t] = 1;
        if (a.L.has_escale) ((int32_t *)(a.ws + a.L.inp))[t] = (arg >= 0 && arg < a.V) ? arg : a.mask_id;
    }
    const int id_now = sel ? arg : id0;
    build_ulist(a, b, i, unc && !sel);
    if (i == 0) {
        a.step[b] = s;
        a.n_steps_done[b] = s;
    }
    if (finished) {
        const int e = (i < a.C && a.eos_id >= 0 && id_now == a.eos_id) ? i : a.C;
        const int first = block_min_int_256(e, sm.shi);
        if (i == 0) {
            a.n_valid[b] = first;
            a.done[b] = 1;
            if (a.done_host) __hip_atomic_store(a.done_host + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
}

// ---------------------------------------------------------------------------
// Exact leading logits (bf16 path).  The vocabulary head multiplies fp16(h)
// (~11 significant bits), so its logits z~ differ from the logits z of the
// fp32 h by up to r_h 2^-11 sum_k |h_k| |W_vk|.  The decisions of the step
// hang on the two leading entries of a row (greedy id, max logit, second
// logit) and the sum of exponentials is dominated by them, so the wave that
// merged row r recomputes z for the ids a and a2 from the fp32 h (fp32 FMA,
// fixed-order butterfly: every lane ends with the same bits) and replaces
// their z~ terms:
//   S~ = 1 + e^(m2~ - m~) + R (R: every other id, relative to m~);
//   S  = R e^(m~ - M) + sum over {a, a2} of e^(z - M),  M = max z of the two;
//   T  = e^(m~ - M) (R_t + (m~ - M) R) + sum over {a, a2} of (z - M) e^(z - M)
// with R_t the rest of t~.  Everything but the two leading ids keeps its
// fp16-operand logit, whose errors enter S and T only through the rest R
// (weights e^(z - M) << 1 apart from near-ties).  An id whose true logit
// ranks first or second but whose z~ ranks third or lower would need two
// z~ errors across its gap, which is below 2 r_h 2^-11 sum |h| |W|.
// ---------------------------------------------------------------------------
// FX 8-float chunks of the fp32 row per lane are loaded with the slice
// records, before the merge (d <= 512 FX); wider rows read the rest inside.
constexpr int FX = 6;

__device__ __forceinline__ void load_hrow(const StepArgs &a, int r, int lane, float4 (&hv)[FX][2]) {
    const float *hr = (const float *)(a.ws + a.L.hf) + (size_t)r * a.d;
#pragma unroll
    for (int u = 0; u < FX; ++u) {
        const int k = min(8 * lane + 512 * u, a.d - 8);   // clamped: chunks past d are not used
        hv[u][0] = *(const float4 *)(hr + k);
        hv[u][1] = *(const float4 *)(hr + k + 4);
    }
}

// r_h-free dot products of the fp32 row r of h with head rows i1 and i2
// (fp32 FMA per lane in chunk order, then a fixed butterfly: every lane ends
// with the same bits); the head rows of an e4m3 head are scaled by their
// row scales.
__device__ __forceinline__ void head_dots2(const StepArgs &a, int r, int i1, int i2, int lane,
                                           const float4 (&hv)[FX][2], float &o1, float &o2) {
    const float *hr = (const float *)(a.ws + a.L.hf) + (size_t)r * a.d;
    float d1 = 0.f, d2 = 0.f;
    // 8 products of chunk k (fp32 h values x[0..7]) with both rows
    auto fma8 = [&](const float (&x)[8], const float (&y1)[8], const float (&y2)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            d1 = fmaf(x[e], y1[e], d1);
            d2 = fmaf(x[e], y2[e], d2);
        }
    };
    // the two head rows' values of chunk k, as floats (exact)
    auto rows8 = [&](int k, float (&y1)[8], float (&y2)[8]) __attribute__((always_inline)) {
        if (a.lm_fp8) {
            const uint8_t *w1 = (const uint8_t *)a.lm + (size_t)i1 * a.d;
            const uint8_t *w2 = (const uint8_t *)a.lm + (size_t)i2 * a.d;
            const u32x2 c1 = *(const u32x2 *)(w1 + k), c2 = *(const u32x2 *)(w2 + k);
            // codes 2e, 2e + 1 -> two floats; the pair is shifted into the
            // low half instead of selecting the high half in the conversion,
            // whose half select this compiler drops once the result feeds
            // mixed-precision FMAs
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x1 = (e & 1) ? (c1[e >> 1] >> 16) : c1[e >> 1];
                const uint32_t x2 = (e & 1) ? (c2[e >> 1] >> 16) : c2[e >> 1];
                const f32x2 f1 = __builtin_convertvector(
                    __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x1, 1.0f, false)), f32x2);
                const f32x2 f2 = __builtin_convertvector(
                    __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x2, 1.0f, false)), f32x2);
                y1[2 * e] = f1.x; y1[2 * e + 1] = f1.y;
                y2[2 * e] = f2.x; y2[2 * e + 1] = f2.y;
            }
        } else {
            const uint16_t *w1 = (const uint16_t *)a.lm + (size_t)i1 * a.d;
            const uint16_t *w2 = (const uint16_t *)a.lm + (size_t)i2 * a.d;
            const u32x4 c1 = *(const u32x4 *)(w1 + k), c2 = *(const u32x4 *)(w2 + k);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                y1[2 * e] = bf_lo(c1[e]); y1[2 * e + 1] = bf_hi(c1[e]);
                y2[2 * e] = bf_lo(c2[e]); y2[2 * e + 1] = bf_hi(c2[e]);
            }
        }
    };
    {
        // every row chunk's loads first, then the products
        float y1[FX][8], y2[FX][8];
#pragma unroll
        for (int u = 0; u < FX; ++u) rows8(min(8 * lane + 512 * u, a.d - 8), y1[u], y2[u]);
#pragma unroll
        for (int u = 0; u < FX; ++u) {
            if (8 * lane + 512 * u < a.d) {
                const float x[8] = {hv[u][0].x, hv[u][0].y, hv[u][0].z, hv[u][0].w,
                                    hv[u][1].x, hv[u][1].y, hv[u][1].z, hv[u][1].w};
                fma8(x, y1[u], y2[u]);
            }
        }
    }
    for (int k = 8 * lane + 512 * FX; k < a.d; k += 512) {
        const float4 h0 = *(const float4 *)(hr + k), h1 = *(const float4 *)(hr + k + 4);
        const float x[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
        float y1[8], y2[8];
        rows8(k, y1, y2);
        fma8(x, y1, y2);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        d1 += shfl_xor_f(d1, o);
        d2 += shfl_xor_f(d2, o);
    }
    if (a.lm_fp8) {
        d1 *= a.lm_scale[i1];
        d2 *= a.lm_scale[i2];
    }
    o1 = d1;
    o2 = d2;
}

__device__ __forceinline__ void exact_leading(const StepArgs &a, int r, int t, VStat &acc, int lane, bool ent,
                                              const float4 (&hv)[FX][2]) {
    if (acc.a < 0 || acc.a >= a.V) return;             // no valid id (cannot happen for V >= 2)
    const bool has2 = acc.m2 != -INFINITY && acc.a2 >= 0 && acc.a2 < a.V;   // a second id exists (V > 2)
    const int i1 = acc.a, i2 = has2 ? acc.a2 : acc.a;
    float d1, d2;
    head_dots2(a, r, i1, i2, lane, hv, d1, d2);
    const float rs = ((const float *)(a.ws + a.L.r_h))[t];
    float e1 = rs * d1, e2 = has2 ? rs * d2 : -INFINITY;
    int j1 = i1, j2 = has2 ? i2 : INT_MAX;
    if (!vbefore(e1, j1, e2, j2)) {
        const float te = e1; e1 = e2; e2 = te;
        const int tj = j1; j1 = j2; j2 = tj;
    }
    const float w2 = has2 ? __expf(acc.m2 - acc.m) : 0.f;
    const float rest = fmaxf(acc.s - 1.f - w2, 0.f);
    const float g = __expf(acc.m - e1);
    const float x2 = has2 ? __expf(e2 - e1) : 0.f;
    const float s = fmaf(rest, g, 1.f + x2);
    if (ent) {
        const float rest_t = acc.t - (has2 ? (acc.m2 - acc.m) * w2 : 0.f);
        acc.t = g * fmaf(acc.m - e1, rest, rest_t) + (has2 ? (e2 - e1) * x2 : 0.f);
    }
    acc.m = e1;
    acc.a = j1;
    acc.m2 = e2;
    acc.a2 = j2;
    acc.s = s;
}

// ---------------------------------------------------------------------------
// Temperature sampling (bf16 path): the draw of row r.  The vocabulary head
// kept, per slice, the two largest z~ / T + g of the fp16-operand logits;
// the two largest over all slices are the candidates, whose keys are
// recomputed from the exact logits (fp32 h) and double-precision Gumbel
// noise.  The draw is the larger (lower id on a tie); it replaces the
// greedy id in the row statistics, and the sum slot becomes
// S e^(M - z_draw) = 1 / p_theta(draw), so that the ranking, the threshold
// and the stop read the draw's probability.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void exact_draw(const StepArgs &a, int b, int r, int t, int pos, VStat &acc, int lane,
                                           const float4 (&hv)[FX][2], const float4 (&kq)[4]) {
    const int ns = a.L.n_slices, sw = a.L.slice_width;
    const float4 *kp = (const float4 *)(a.ws + a.L.lm_kpart) + (size_t)r * ns;
    Top2 kt{-INFINITY, -INFINITY, INT_MAX, INT_MAX};
    auto fold = [&](const float4 &x, int sl) __attribute__((always_inline)) {
        if (sl >= ns) return;
        const uint32_t w = __float_as_uint(x.z);
        kt = top2_merge(kt, Top2{x.x, x.y, unpack_id(w & 0xffffu, sl * sw), unpack_id(w >> 16, sl * sw)});
    };
#pragma unroll
    for (int u = 0; u < 4; ++u) fold(kq[u], 64 * u + lane);          // loaded with the slice records
    for (int sl = 256 + lane; sl < ns; sl += 64) fold(kp[sl], sl);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) kt = top2_merge(kt, top2_shfl_xor(kt, o));
    if (kt.i1 < 0 || kt.i1 >= a.V) return;              // no candidate (cannot happen for V >= 2)
    const bool has2 = kt.k2 != -INFINITY && kt.i2 >= 0 && kt.i2 < a.V;
    const int j1 = kt.i1, j2 = has2 ? kt.i2 : kt.i1;
    float d1, d2;
    head_dots2(a, r, j1, j2, lane, hv, d1, d2);
    const float rs = ((const float *)(a.ws + a.L.r_h))[t];
    const float z1 = rs * d1, z2 = rs * d2;
    const int s = a.step[b] + 1;
    const double T = a.N <= 1 ? (double)a.temp0
                              : (double)a.temp0 + ((double)a.temp1 - (double)a.temp0) * (double)(s - 1) / (double)(a.N - 1);
    auto key = [&](int v, float z) __attribute__((always_inline)) {
        const Philox4 ph = philox4x64_10((uint64_t)(v >> 2), (uint64_t)pos, (uint64_t)s, (uint64_t)b, a.seed, 0ull);
        return (double)z / T + gumbel_f64(ph.word(v & 3));
    };
    const double e1 = key(j1, z1), e2 = has2 ? key(j2, z2) : -INFINITY;
    const bool second = has2 && (e2 > e1 || (e2 == e1 && j2 < j1));
    const int draw = second ? j2 : j1;
    const float zd = second ? z2 : z1;
    acc.s = acc.s * __expf(acc.m - zd);
    acc.a = draw;
}

// ---------------------------------------------------------------------------
// Merge of the per-slice vocabulary statistics, then the sampler update.
// Workgroup (request b, group q) merges compact rows 4q .. 4q+3 of b, one
// wave each: lane l folds slices l, l + 64, ... in order (the records of a
// row are contiguous, part[row * n_slices + slice]), then a xor butterfly.
// The workgroups of a request count themselves on a per-request counter
// once their statistics stores have completed; the last to arrive (all
// statistics of the request visible) runs the commit and clears the counter.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_sample_commit(StepArgs a) {
    __shared__ __align__(16) CommitSmem sm;
    __shared__ int last;
    const int G = a.L.cp / 4;
    const int b = blockIdx.x / G, q = blockIdx.x - (blockIdx.x / G) * G;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int jr = 4 * q + w;                          // compact row of this wave (< cp)
    const int r = b * a.L.cp + jr;
    const int ns = a.L.n_slices;
    const float4 *part = (const float4 *)(a.ws + a.L.lm_part) + (size_t)r * ns;
    const float *tpart = (const float *)(a.ws + a.L.lm_tpart) + (size_t)r * ns;
    const bool ent = a.ent != 0;
    const int sw = a.L.slice_width;
    // Every load this workgroup needs before the counter is issued here, at
    // once: the request's flags, the commit's inputs that no merge changes,
    // and the first 256 slice records of the row (read whether or not the
    // row is open; a closed row's records are discarded).
    const int done = a.done[b];
    const int cnt = ((const int32_t *)(a.ws + a.L.ucount))[b];
    const int step0 = a.step[b];
    const int tp = b * a.C + threadIdx.x;
    const bool vp = threadIdx.x < a.C;
    const int c0 = vp ? ((const int32_t *)(a.ws + a.L.uidx))[tp] : -1;
    const int id0 = vp ? a.ids[tp] : 0;
    const int pos = ((const int32_t *)(a.ws + a.L.ulist))[r];
    // (clamped addresses, identity records selected afterwards: no branch
    // and no wait between the loads)
    const float4 ident = make_float4(-INFINITY, 0.f, -INFINITY, __uint_as_float(0xffffffffu));
    float4 p[4];
    float pt[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] = part[min(64 * u + lane, ns - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) pt[u] = 0.f;
    if (ent) {
#pragma unroll
        for (int u = 0; u < 4; ++u) pt[u] = tpart[min(64 * u + lane, ns - 1)];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
        if (64 * u + lane >= ns) {
            p[u] = ident;
            pt[u] = 0.f;
        }
    float4 hv[FX][2];                                  // fp32 row of h for the exact leading logits
    if (a.dtype == DG_BF16) load_hrow(a, r, lane, hv);
    // temperature sampling: the first 256 slices' candidate records as well
    float4 kq[4];
    if (a.temp0 > 0.f) {
        const float4 *kp = (const float4 *)(a.ws + a.L.lm_kpart) + (size_t)r * ns;
#pragma unroll
        for (int u = 0; u < 4; ++u) kq[u] = kp[min(64 * u + lane, ns - 1)];
    }
    const int nwg = max(1, (cnt + 3) / 4);             // group 0 also runs for an empty list
    if (done || q >= nwg) return;
    if (jr < cnt) {
        const int t = b * a.C + pos;
        // lane folds slices lane, lane + 64, ... in order
        auto rec = [&](const float4 &x, float tt, int slice) __attribute__((always_inline)) {
            const uint32_t w = __float_as_uint(x.w);
            return VStat{x.x, x.y, x.z, unpack_id(w & 0xffffu, slice * sw), tt, unpack_id(w >> 16, slice * sw)};
        };
        VStat acc{-INFINITY, 0.f, -INFINITY, INT_MAX, 0.f, INT_MAX};
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = vmerge(acc, rec(p[u], pt[u], 64 * u + lane));
        for (int base = 256; base < ns; base += 256) {
#pragma unroll
            for (int u = 0; u < 4; ++u) p[u] = part[min(base + 64 * u + lane, ns - 1)];
            if (ent) {
#pragma unroll
                for (int u = 0; u < 4; ++u) pt[u] = tpart[min(base + 64 * u + lane, ns - 1)];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (base + 64 * u + lane >= ns) {
                    p[u] = ident;
                    pt[u] = 0.f;
                }
#pragma unroll
            for (int u = 0; u < 4; ++u) acc = vmerge(acc, rec(p[u], pt[u], base + 64 * u + lane));
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) acc = vmerge(acc, vshfl_xor(acc, o));
        if (a.dtype == DG_BF16) exact_leading(a, r, t, acc, lane, ent, hv);
        const float entropy = __logf(acc.s) - acc.t / acc.s;   // of softmax(z): ln s - t / s
        if (a.temp0 > 0.f) exact_draw(a, b, r, t, pos, acc, lane, hv, kq);
        if (lane == 0) {
            st_dev_f4((float4 *)(a.ws + a.L.rowstats) + t, make_float4(acc.m, acc.s, acc.m2, __int_as_float(acc.a)));
            if (ent)
                __hip_atomic_store((float *)(a.ws + a.L.rowent) + t, entropy, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);                     // this wave's statistics stores have completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    int *counter = (int *)(a.ws + a.L.sample_cnt) + b;
    if (threadIdx.x == 0) {
        const int old = atomicAdd(counter, 1);
        last = (old == nwg - 1) ? 1 : 0;
        if (last) *counter = 0;                        // ready for the next step
    }
    __syncthreads();
    if (!last) return;
    commit_request(a, b, sm, cnt, c0, id0, step0);   // reads the statistics with device-scope loads
}

// ---------------------------------------------------------------------------
// Split-KV merge: o = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s in
// fp32, stored as the output projection's operand: an fp16 hi plane and an
// fp16 lo plane (o - hi), fragment-major; odump (optional) gets fp32 o
// row-major.  One wave per query vector (b, h, i); lane covers hd/64
// channels.
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(256) void k_attn_merge(StepArgs a, int n_split, float *odump) {
    constexpr int PER = HD / 64;
    constexpr int SB = 8;                              // splits whose loads are in flight together
    const int QV = a.B * a.Hq * a.C;
    const int qvg = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (qvg >= QV) return;
    const int b = qvg / (a.Hq * a.C);
    const int h = (qvg / a.C) % a.Hq;
    const int ic = qvg % a.C;
    const float2 *ml = (const float2 *)(a.ws + a.L.attn_ml);
    const float *acc = (const float *)(a.ws + a.L.attn_acc);
    // Loads first (the request's flag, split s's (max, sum) in lane s, the
    // first SB splits' partial outputs), then the weights.  An empty split
    // wrote no partial output: its weight is 0 and its values are dropped
    // by a select, never multiplied.
    const int done = ((a.only_req >= 0 && b != a.only_req) ||
                      (a.phase == PH_APPEND ? a.done[b] == 0 : a.done[b] != 0)) ? 1 : 0;   // not taking part
    n_split = a.attn_split[b];                         // this request's splits
    const float2 p = (lane < n_split) ? ml[(size_t)lane * QV + qvg] : make_float2(-INFINITY, 0.f);
    float x[SB][PER];
#pragma unroll
    for (int u = 0; u < SB; ++u) {
        const float *src = acc + ((size_t)min(u, n_split - 1) * QV + qvg) * HD + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) x[u][e] = src[e];
    }
    if (done) return;
    float M = p.x;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, shfl_xor_f(M, o));
    const float w = (p.x == -INFINITY) ? 0.f : exp2f(p.x - M);
    float den = w * p.y;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) den += shfl_xor_f(den, o);
    float o_[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) o_[e] = 0.f;
    for (int s0 = 0; s0 < n_split; s0 += SB) {
        if (s0 > 0) {
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                const float *src = acc + ((size_t)min(s0 + u, n_split - 1) * QV + qvg) * HD + lane * PER;
#pragma unroll
                for (int e = 0; e < PER; ++e) x[u][e] = src[e];
            }
        }
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            const float ws = (s0 + u < n_split) ? __shfl(w, s0 + u, 64) : 0.f;
#pragma unroll
            for (int e = 0; e < PER; ++e) o_[e] += (ws != 0.f) ? ws * x[u][e] : 0.f;
        }
    }
    const float inv = 1.0f / den;
#pragma unroll
    for (int e = 0; e < PER; ++e) o_[e] *= inv;
    const int t = b * a.C + ic;
    const int K = a.Hq * HD;
    const size_t plane = (size_t)a.L.m_pad * K;
    uint16_t *dst = (uint16_t *)(a.ws + a.L.o) + frag_index(t, h * HD + lane * PER, K);
    if constexpr (PER == 1) {                          // hd 64: one channel per lane
        const _Float16 hi = (_Float16)o_[0];
        dst[0] = __builtin_bit_cast(uint16_t, hi);
        dst[plane] = __builtin_bit_cast(uint16_t, (_Float16)(o_[0] - (float)hi));
    } else {
#pragma unroll
        for (int e = 0; e < PER; e += 2) {
            const uint32_t hi = pack_h2(o_[e], o_[e + 1]);
            const f32x2 hf = __builtin_convertvector(__builtin_bit_cast(f16x2, hi), f32x2);
            *(uint32_t *)(dst + e) = hi;
            *(uint32_t *)(dst + plane + e) = pack_h2(o_[e] - hf.x, o_[e + 1] - hf.y);
        }
    }
    if (odump) {
#pragma unroll
        for (int e = 0; e < PER; ++e) odump[(size_t)t * K + h * HD + lane * PER + e] = o_[e];
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_reset(const StepArgs &a, const int32_t *init_ids, const uint8_t *init_committed,
                        hipStream_t s, int slot) {
    hipLaunchKernelGGL(k_reset, dim3(slot >= 0 ? 1 : a.B), dim3(256), 0, s, a, init_ids, init_committed, slot);
    return hipGetLastError();
}

hipError_t launch_clear_err(const StepArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_clear_err, dim3(1), dim3(64), 0, s, (int32_t *)(a.ws + a.L.err));
    return hipGetLastError();
}

hipError_t launch_rope_table(const StepArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_rope_table, dim3(a.M), dim3(128), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_prep(const StepArgs &a, int force, hipStream_t s) {
    if (a.dtype == DG_BF16)
        hipLaunchKernelGGL(k_prep<uint16_t>, dim3(a.M), dim3(256), 0, s, a, force);
    else
        hipLaunchKernelGGL(k_prep<float>, dim3(a.M), dim3(256), 0, s, a, force);
    return hipGetLastError();
}


hipError_t launch_rowscale_h(const StepArgs &a, hipStream_t s) {
    if (a.dtype == DG_BF16)
        hipLaunchKernelGGL(k_rowscale_h<uint16_t>, dim3(a.M), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(k_rowscale_h<float>, dim3(a.M), dim3(256), 0, s, a);
    return hipGetLastError();
}


hipError_t launch_escale(const StepArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_escale, dim3(a.V), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_ulist(const StepArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_ulist, dim3(a.B), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_sample_commit(const StepArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_sample_commit, dim3(a.B * (a.L.cp / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attn_merge(const StepArgs &a, int n_split, float *odump, hipStream_t s) {
    const int QV = a.B * a.Hq * a.C;
    const dim3 g((QV + 3) / 4);
    switch (a.hd) {
        case 64: hipLaunchKernelGGL(k_attn_merge<64>, g, dim3(256), 0, s, a, n_split, odump); break;
        case 128: hipLaunchKernelGGL(k_attn_merge<128>, g, dim3(256), 0, s, a, n_split, odump); break;
        case 256: hipLaunchKernelGGL(k_attn_merge<256>, g, dim3(256), 0, s, a, n_split, odump); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dg
