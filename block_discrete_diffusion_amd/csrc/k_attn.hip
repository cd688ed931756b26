// Block-bidirectional GQA attention of the canvas queries over
// (prefix keys || canvas keys), split over the key axis (flash-decoding
// style partials, merged by k_attn_merge).  Request b's keys are cut into
// a.attn_split[b] splits; grid z covers the largest count.
//
// Every canvas query sees every prefix key and every canvas key: no causal
// mask inside the canvas (DiffusionGemma Technical Report, section 1 and
// section 4: bidirectional attention within the 256-token block, clean
// context through the KV cache).  Query head h reads KV head h / (Hq/Hkv).
//
// A workgroup takes 128 query vectors of one KV group and one key split;
// its waves work transposed:
//   S^T = K Q^T       A = K rows (LDS), B = Q (registers)
//   O^T += V^T P^T    A = V^T rows (LDS, the cache stores V key-fastest),
//                     B = P^T straight from the S^T registers
// so every lane holds scores, softmax state and output channels of one
// query, and the online softmax needs only cross-lane reductions per key
// block.  The key rows of the A operand of S^T are permuted so that each
// lane's score registers are runs of consecutive keys, exactly the k-slot
// layout its P^T operand needs.  Two forms:
//   k_attn_q16 (head_dim 128 and 256): 16 query vectors per wave on 16x16x32
//     MFMAs, 8 waves;
//   k_attn_bf16 (head_dim 64): 32 query vectors per wave on 32x32x16 MFMAs,
//     4 waves.
//
// Precision: q is held in fp32 and enters S^T as two bf16 operands, hi and
// lo (~16 significant bits), against the bf16 keys of the cache: two MFMAs
// per k-slice of the head.  The PV product uses single fp16 operands:
// V is converted exactly from bf16 while it is staged in LDS, and P (at most
// 2^8, see m_ref) is rounded to fp16 (11 significant bits); the row sums l
// add the fp32 p.  The attention output stays in fp32.  Emulated in float64
// at the workloads' shapes, the fp16 P moves the logits of each row's
// leading ids by at most 4e-4, under half of the 1e-3 near-tie band of the
// step's decisions; a single bf16 q would move them by 2.4e-3 and a single
// fp16 q (with the fp16 P) by 6.7e-4, so q keeps its two parts.
#include "dg_device.hpp"
#include "dg_internal.hpp"

namespace dg {

hipError_t launch_attention_f32(const StepArgs &a, hipStream_t s);

// 32x32 form: MFMA row i of the S^T tile is key sigma(i) of the block.
__device__ __forceinline__ int key_perm(int i) {
    const int a = i >> 3, b = (i >> 2) & 1, c = i & 3;
    return 16 * (a >> 1) + 8 * b + 4 * (a & 1) + c;
}

// LDS swizzles of the 32x32 form.  A 16-byte read of a quarter-wave (16 lanes) is free of
// bank conflicts when its 16 addresses fall in 16 different 16-byte units of
// a 256-byte bank cycle.  K tile rows are HD * 2 bytes: from 256 bytes up,
// every row starts at unit 0, so chunk c of row r goes to unit c ^ (r & 15)
// (16 consecutive key rows, one chunk column); 128-byte rows pair up, and
// the XOR takes (r / 2) & 7.  V^T rows are 64 bytes (4 per cycle): chunk kc
// of channel row ch goes to kc ^ ((ch / 4) & 3), so 16 consecutive channels
// cover all 16 units.
template <int KC>
__device__ __forceinline__ int kswz(int r) { return KC >= 16 ? (r & 15) : ((r >> 1) & 7); }
__device__ __forceinline__ int vswz(int ch) { return (ch >> 2) & 3; }

template <int HD>
__global__ __launch_bounds__(256, 2) void k_attn_bf16(StepArgs a) {
    constexpr int NTHR = 256;
    constexpr int KC = HD / 8;                    // 16-byte chunks per K row
    constexpr int NK = (32 * KC) / NTHR;          // K-tile chunks per thread
    constexpr int NV = (HD * 4) / NTHR;           // V^T-tile chunks per thread
    constexpr int NKS = HD / 16;                  // k-steps of the score product
    constexpr int NVT = HD / 32;                  // 32-channel output tiles
    __shared__ u32x4 kl[2][32 * KC];              // K tiles [32 keys][HD], swizzled
    __shared__ u32x4 vl[2][HD * 4];               // V^T tiles [HD][32 keys] in fp16, swizzled

    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, row32 = lane & 31;
    const int wave = tid >> 6;                    // query tile of the workgroup
    const int b = blockIdx.y / a.Hkv;
    const int g = blockIdx.y - b * a.Hkv;
    // the request takes part (not done in a step, done in the append pass);
    // tested once the first loads are in flight
    const int done = ((a.only_req >= 0 && b != a.only_req) ||
                      (a.phase == PH_APPEND ? a.done[b] == 0 : a.done[b] != 0)) ? 1 : 0;
    const int G = a.Hq / a.Hkv;
    const int nqv = G * a.C;
    const int QV = a.B * a.Hq * a.C;
    const int split = blockIdx.z;
    const int64_t P = a.reqs.len[b];
    const int L = (int)(P + a.C);
    const bool causal = a.causal != 0;
    const int nblk = (L + 31) >> 5;
    const int ns = a.attn_split[b];               // this request's splits (<= n_split, the grid depth)
    if (split >= ns) return;
    const int bps = (nblk + ns - 1) / ns;
    const int blk0 = split * bps;
    const int blk1 = min(nblk, blk0 + bps);

    const int qv = blockIdx.x * 128 + wave * 32 + row32;
    const bool vq = qv < nqv;
    const int qvc = min(qv, nqv - 1);             // rows past the end read a valid row, results dropped
    const int hl = qvc / a.C;
    const int ic = qvc - hl * a.C;
    const int h = g * G + hl;
    const int t = b * a.C + ic;
    const int qvg = (b * a.Hq + h) * a.C + ic;
    float2 *mlp = (float2 *)(a.ws + a.L.attn_ml) + (size_t)split * QV;
    float *accp = (float *)(a.ws + a.L.attn_acc) + (size_t)split * QV * HD;

    if (blk0 >= blk1) {                           // empty split: neutral partial
        if (!done && vq && half == 0) mlp[qvg] = make_float2(-INFINITY, 0.f);
        return;
    }

    const int64_t cap = a.reqs.cap[b];
    const uint16_t *Kg = (const uint16_t *)a.reqs.k[b] + (size_t)g * cap * HD;
    const uint16_t *Vg = (const uint16_t *)a.reqs.v[b] + (size_t)g * HD * cap;

    // global -> registers for one 32-key block: plain 16-byte loads from
    // addresses clamped into [0, L) (a V^T chunk starting below L ends at or
    // before capacity since capacity % 8 == 0).  Nothing here uses the loaded
    // data, so the loads stay in flight until the block is staged one
    // iteration later.
    u32x4 rk[NK], rv[NV];
    auto fetch_to = [&](int blk, u32x4 (&rk)[NK], u32x4 (&rv)[NV]) __attribute__((always_inline)) {
        const int key0 = blk * 32;
#pragma unroll
        for (int x = 0; x < NK; ++x) {
            const int c = tid + NTHR * x;
            const int r = c / KC, col = c - r * KC;
            rk[x] = *(const u32x4 *)(Kg + (size_t)min(key0 + r, L - 1) * HD + col * 8);
        }
#pragma unroll
        for (int x = 0; x < NV; ++x) {
            const int c = tid + NTHR * x;
            const int ch = c >> 2, kc = c & 3;
            const int k8c = min(key0 + kc * 8, (L - 1) & ~7);
            rv[x] = *(const u32x4 *)(Vg + (size_t)ch * cap + k8c);
        }
    };
    // registers -> LDS buffer for block blk.  Key rows at or past L need no
    // mask (their scores are replaced by -inf before the softmax); values
    // at or past L are zeroed, since p = 0 times whatever the cache holds
    // there (possibly not finite) must contribute nothing.  V goes to fp16.
    auto fetch = [&](int blk) __attribute__((always_inline)) { fetch_to(blk, rk, rv); };
    auto stage_from = [&](int buf, int blk, const u32x4 (&rk)[NK], const u32x4 (&rv)[NV])
                          __attribute__((always_inline)) {
        const int key0 = blk * 32;
#pragma unroll
        for (int x = 0; x < NK; ++x) {
            const int c = tid + NTHR * x;
            const int r = c / KC, col = c - r * KC;
            kl[buf][r * KC + (col ^ kswz<KC>(r))] = rk[x];
        }
#pragma unroll
        for (int x = 0; x < NV; ++x) {
            const int c = tid + NTHR * x;
            const int ch = c >> 2, kc = c & 3;
            u32x4 v = rv[x];
            if (key0 + 32 > L) {                   // only the last block of the sequence
                const int nv = L - (key0 + kc * 8);    // valid keys in this chunk (may be <= 0 or >= 8)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t keep_lo = (2 * w < nv) ? 0x0000ffffu : 0u;
                    const uint32_t keep_hi = (2 * w + 1 < nv) ? 0xffff0000u : 0u;
                    v[w] &= keep_lo | keep_hi;
                }
            }
            vl[buf][ch * 4 + (kc ^ vswz(ch))] = bf8_to_h8(v);
        }
    };
    auto stage = [&](int buf, int blk) __attribute__((always_inline)) { stage_from(buf, blk, rk, rv); };

    // q of this lane's query is loaded first (loads complete in issue order,
    // so its split below waits for q alone), then the key/value blocks.
    // HD <= 128: blocks blk0 and blk0 + 1 are fetched together (second
    // register set rk1 / rv1, staged by the first iteration), so the first
    // iteration does not wait for a fetch issued just before it.
    u32x4 qh[NKS], ql[NKS];                       // raw fp32 q first, then its bf16 hi / lo parts
    {
        const float *qrow = (const float *)(a.ws + a.L.q) + ((size_t)t * a.Hq + h) * HD + 8 * half;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            qh[ks] = *(const u32x4 *)(qrow + 16 * ks);
            ql[ks] = *(const u32x4 *)(qrow + 16 * ks + 4);
        }
    }
    constexpr bool TWO = HD <= 128;
    u32x4 rk1[NK], rv1[NV];                       // unused when !TWO
    fetch(blk0);
    if constexpr (TWO) fetch_to(min(blk0 + 1, blk1 - 1), rk1, rv1);
    // q pre-scaled by log2(e)/sqrt(hd) so that the scores come out in the
    // exp2 domain, as a bf16 hi/lo pair
    {
        const float scale = 1.4426950408889634f / sqrtf((float)HD);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            u32x4 x0 = qh[ks], x1 = ql[ks];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x0[e] = __float_as_uint(__uint_as_float(x0[e]) * scale);
                x1[e] = __float_as_uint(__uint_as_float(x1[e]) * scale);
            }
            split2_bf16(x0, x1, qh[ks], ql[ks]);
        }
    }
    if (done) return;
    stage(0, blk0);
    fetch(min(blk0 + (TWO ? 2 : 1), blk1 - 1));
    __syncthreads();

    f32x16 acc[NVT];
#pragma unroll
    for (int i = 0; i < NVT; ++i) acc[i] = zero16();
    // m_ref: reference of the exponentials, raised only when a block's max
    // exceeds it by more than 8 (so p <= 2^8, well inside fp16); l_run: sum
    // of p over this lane's keys
    float m_ref = -INFINITY, l_run = 0.f;
    const int krow = key_perm(row32);

    auto body = [&](int blk, auto FIRST) __attribute__((always_inline)) {
        constexpr bool first = decltype(FIRST)::value;
        const int cur = (blk - blk0) & 1;
        const int key0 = blk * 32;
        f32x16 s = zero16();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int c = 2 * ks + half;
            const u32x4 kf = kl[cur][krow * KC + (c ^ kswz<KC>(krow))];
            s = mfma32(kf, qh[ks], s);
            s = mfma32(kf, ql[ks], s);
        }
        // register r holds key key0 + 16*(r/8) + 8*half + r%8 for query row32;
        // only the last block of the sequence can reach past L.  Causal
        // (context encoding): canvas position ic sees keys up to P + ic.
        const int lim = causal ? min(L, (int)P + ic + 1) : L;
        if (key0 + 32 > lim) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + 16 * (r >> 3) + 8 * half + (r & 7);
                s[r] = (key < lim) ? s[r] : -INFINITY;
            }
        }
        float mloc = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mloc = fmaxf(mloc, s[r]);
        mloc = fmaxf(mloc, shfl_xor_f(mloc, 32));     // both halves: same query, same value
        const bool up = mloc > m_ref + 8.f;
        if (__ballot(up)) {
            const float m_new = up ? mloc : m_ref;
            const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);   // 0 on the first block, 1 if kept
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < NVT; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][r] *= alpha;
            m_ref = m_new;
        }
        float psum = 0.f;
        uint32_t pk[8];
        // a causal query that has seen no key yet keeps m_ref = -inf: p = 0
        const float mexp = (causal && m_ref == -INFINITY) ? INFINITY : m_ref;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = __builtin_amdgcn_exp2f(s[r] - mexp);
            const float p1 = __builtin_amdgcn_exp2f(s[r + 1] - mexp);
            psum += p0 + p1;
            pk[r >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p0, p1}, f16x2));
        }
        l_run += psum;
        const u32x4 pf0 = {pk[0], pk[1], pk[2], pk[3]};
        const u32x4 pf1 = {pk[4], pk[5], pk[6], pk[7]};
#pragma unroll
        for (int i = 0; i < NVT; ++i) {
            const int ch = 32 * i + row32;
            const int sw = vswz(ch);
            const u32x4 v0 = vl[cur][ch * 4 + ((0 + half) ^ sw)];
            const u32x4 v1 = vl[cur][ch * 4 + ((2 + half) ^ sw)];
            acc[i] = mfma32_f16(v0, pf0, acc[i]);
            acc[i] = mfma32_f16(v1, pf1, acc[i]);
        }
        // block blk+1 (fetched one iteration ago, or with the first block)
        // into the other buffer, and the fetch of blk+2; past the end both
        // repeat the last block, so every iteration issues the same loads
        if constexpr (first && TWO) {
            stage_from(cur ^ 1, min(blk + 1, blk1 - 1), rk1, rv1);
        } else {
            stage(cur ^ 1, min(blk + 1, blk1 - 1));
            fetch(min(blk + 2, blk1 - 1));
        }
        __syncthreads();
    };
    body(blk0, std::true_type{});
    for (int blk = blk0 + 1; blk < blk1; ++blk) body(blk, std::false_type{});

    const float l_tot = l_run + shfl_xor_f(l_run, 32);
    if (!vq) return;
    if (half == 0) mlp[qvg] = make_float2(m_ref, l_tot);
    float *dst = accp + (size_t)qvg * HD;
#pragma unroll
    for (int i = 0; i < NVT; ++i)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int ch = 32 * i + 8 * rg + 4 * half;
            *(float4 *)(dst + ch) = make_float4(acc[i][4 * rg], acc[i][4 * rg + 1], acc[i][4 * rg + 2], acc[i][4 * rg + 3]);
        }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// D = A B + C for one 16x16 tile, K = 32.  Lane l holds, for A, row l%16 and
// the 8 k-slots 8*(l/16)..+7; for B, column l%16 and the same k-slots; the
// result register r of lane l is D[4*(l/16) + r][l%16].
__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_f16(const u32x4 &a, const u32x4 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// 16 query vectors per wave on 16x16x32 MFMAs, 8 waves (128 query vectors
// of one KV group) per workgroup.  With 16 query vectors a wave's q (bf16 hi
// and lo) and output take 2 * head_dim / 4 registers, so a whole head of 256
// channels fits at two waves per SIMD (four at head_dim 128), and each score
// and exponential is computed by one wave only.  The price is twice the LDS
// fragment bytes per MAC of the 32x32 form.  (Measured against the 32x32
// form with the head dimension split over two waves, whose partial scores
// meet through LDS: 417 against 476 us per long-context step at head_dim
// 256; at head_dim 128, 16.1 against 17.8 us per single-canvas step.)
//
// Per 32-key block a wave computes two S^T tiles of 16 keys; tile t row i is
// key 8 (i / 4) + 4 t + i % 4, so that lane l holds keys 8 (l / 16) .. +7 of
// query l % 16 (tile 0 registers, then tile 1): exactly the k-slots of its
// P^T operand.  K chunk col of key row r sits at col ^ kq(r), which spreads
// the 16 key rows of a quarter-wave read over 16 units of a bank cycle.
// (Measured nonetheless: SQ_LDS_BANK_CONFLICT reads about one extra pass per
// K-fragment read, some 2% of a block; swizzles built for other lane
// groupings kept or doubled it.)
__device__ __forceinline__ int kq(int r) { return ((r >> 3) & 3) * 4 + (r & 3); }

// Lane exchanges across rows of 16 lanes (xor 16) and across wave halves
// (xor 32) as VALU lane swaps instead of LDS permutes.  Swapping a value
// with itself leaves each lane its own value in one result and its partner's
// in the other; max and sum of the two are then the same bits in both lanes
// (fmax and IEEE addition commute).
__device__ __forceinline__ float2 pair16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float2 pair32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max16(float v) { const float2 p = pair16(v); return fmaxf(p.x, p.y); }
__device__ __forceinline__ float max32(float v) { const float2 p = pair32(v); return fmaxf(p.x, p.y); }
__device__ __forceinline__ float sum16(float v) { const float2 p = pair16(v); return p.x + p.y; }
__device__ __forceinline__ float sum32(float v) { const float2 p = pair32(v); return p.x + p.y; }

template <int HD>
__global__ __launch_bounds__(512, HD <= 128 ? 2 : 1) void k_attn_q16(StepArgs a) {
    constexpr int NTHR = 512;
    constexpr int KC = HD / 8;                    // 16-byte chunks per K row
    constexpr int NK = (32 * KC) / NTHR;          // K-tile chunks per thread
    constexpr int NV = (HD * 4) / NTHR;           // V^T-tile chunks per thread
    constexpr int NKS = HD / 32;                  // k-steps of the score product
    constexpr int NCT = HD / 16;                  // 16-channel output tiles
    static_assert(NK >= 1 && NV >= 1, "head_dim 128 or 256");
    __shared__ u32x4 kl[2][32 * KC];
    __shared__ u32x4 vl[2][HD * 4];

    const int tid = threadIdx.x, lane = tid & 63, g16 = lane >> 4, c16 = lane & 15;
    const int wave = tid >> 6;
    const int b = blockIdx.y / a.Hkv;
    const int g = blockIdx.y - b * a.Hkv;
    const int done = ((a.only_req >= 0 && b != a.only_req) ||
                      (a.phase == PH_APPEND ? a.done[b] == 0 : a.done[b] != 0)) ? 1 : 0;
    const int G = a.Hq / a.Hkv;
    const int nqv = G * a.C;
    const int QV = a.B * a.Hq * a.C;
    const int split = blockIdx.z;
    const int64_t P = a.reqs.len[b];
    const int L = (int)(P + a.C);
    const bool causal = a.causal != 0;
    const int nblk = (L + 31) >> 5;
    const int ns = a.attn_split[b];
    if (split >= ns) return;
    const int bps = (nblk + ns - 1) / ns;
    const int blk0 = split * bps;
    const int blk1 = min(nblk, blk0 + bps);

    const int qv = blockIdx.x * 128 + wave * 16 + c16;
    const bool vq = qv < nqv;
    const int qvc = min(qv, nqv - 1);
    const int hl = qvc / a.C;
    const int ic = qvc - hl * a.C;
    const int h = g * G + hl;
    const int t = b * a.C + ic;
    const int qvg = (b * a.Hq + h) * a.C + ic;
    float2 *mlp = (float2 *)(a.ws + a.L.attn_ml) + (size_t)split * QV;
    float *accp = (float *)(a.ws + a.L.attn_acc) + (size_t)split * QV * HD;

    if (blk0 >= blk1) {
        if (!done && vq && g16 == 0) mlp[qvg] = make_float2(-INFINITY, 0.f);
        return;
    }

    const int64_t cap = a.reqs.cap[b];
    const uint16_t *Kg = (const uint16_t *)a.reqs.k[b] + (size_t)g * cap * HD;
    const uint16_t *Vg = (const uint16_t *)a.reqs.v[b] + (size_t)g * HD * cap;

    // global -> registers -> LDS as in k_attn_bf16 (clamped addresses, V
    // past L zeroed, V to fp16)
    u32x4 rk[NK], rv[NV];
    auto fetch = [&](int blk) __attribute__((always_inline)) {
        const int key0 = blk * 32;
#pragma unroll
        for (int x = 0; x < NK; ++x) {
            const int c = tid + NTHR * x;
            const int r = c / KC, col = c - r * KC;
            rk[x] = *(const u32x4 *)(Kg + (size_t)min(key0 + r, L - 1) * HD + col * 8);
        }
#pragma unroll
        for (int x = 0; x < NV; ++x) {
            const int c = tid + NTHR * x;
            const int ch = c >> 2, kc = c & 3;
            const int k8c = min(key0 + kc * 8, (L - 1) & ~7);
            rv[x] = *(const u32x4 *)(Vg + (size_t)ch * cap + k8c);
        }
    };
    auto stage = [&](int buf, int blk) __attribute__((always_inline)) {
        const int key0 = blk * 32;
#pragma unroll
        for (int x = 0; x < NK; ++x) {
            const int c = tid + NTHR * x;
            const int r = c / KC, col = c - r * KC;
            kl[buf][r * KC + (col ^ kq(r))] = rk[x];
        }
#pragma unroll
        for (int x = 0; x < NV; ++x) {
            const int c = tid + NTHR * x;
            const int ch = c >> 2, kc = c & 3;
            u32x4 v = rv[x];
            if (key0 + 32 > L) {
                const int nv = L - (key0 + kc * 8);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t keep_lo = (2 * w < nv) ? 0x0000ffffu : 0u;
                    const uint32_t keep_hi = (2 * w + 1 < nv) ? 0xffff0000u : 0u;
                    v[w] &= keep_lo | keep_hi;
                }
            }
            vl[buf][ch * 4 + (kc ^ vswz(ch))] = bf8_to_h8(v);
        }
    };

    // q: lane l takes dims 32 ks + 8 (l / 16) .. +7 of its query vector
    u32x4 qh[NKS], ql[NKS];
    {
        const float *qrow = (const float *)(a.ws + a.L.q) + ((size_t)t * a.Hq + h) * HD + 8 * g16;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            qh[ks] = *(const u32x4 *)(qrow + 32 * ks);
            ql[ks] = *(const u32x4 *)(qrow + 32 * ks + 4);
        }
    }
    fetch(blk0);
    {
        const float scale = 1.4426950408889634f / sqrtf((float)HD);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            u32x4 x0 = qh[ks], x1 = ql[ks];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x0[e] = __float_as_uint(__uint_as_float(x0[e]) * scale);
                x1[e] = __float_as_uint(__uint_as_float(x1[e]) * scale);
            }
            split2_bf16(x0, x1, qh[ks], ql[ks]);
        }
    }
    if (done) return;
    stage(0, blk0);
    fetch(min(blk0 + 1, blk1 - 1));
    __syncthreads();

    f32x4 acc[NCT];
#pragma unroll
    for (int i = 0; i < NCT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY, l_run = 0.f;
    // key rows of this lane's A operand in the two S^T tiles
    const int kr0 = 8 * (c16 >> 2) + (c16 & 3), kr1 = kr0 + 4;
    const int lim = causal ? min(L, (int)P + ic + 1) : L;

    for (int blk = blk0; blk < blk1; ++blk) {
        const int cur = (blk - blk0) & 1;
        const int key0 = blk * 32;
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int c = 4 * ks + g16;
            const u32x4 k0 = kl[cur][kr0 * KC + (c ^ kq(kr0))];
            const u32x4 k1 = kl[cur][kr1 * KC + (c ^ kq(kr1))];
            s0 = mfma16(k0, qh[ks], s0);
            s1 = mfma16(k1, qh[ks], s1);
            s0 = mfma16(k0, ql[ks], s0);
            s1 = mfma16(k1, ql[ks], s1);
        }
        // register r of tile t: key key0 + 8 g16 + 4 t + r of query c16
        float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
        if (key0 + 32 > lim) {
#pragma unroll
            for (int r = 0; r < 8; ++r) sv[r] = (key0 + 8 * g16 + r < lim) ? sv[r] : -INFINITY;
        }
        float mloc = sv[0];
#pragma unroll
        for (int r = 1; r < 8; ++r) mloc = fmaxf(mloc, sv[r]);
        mloc = max32(max16(mloc));
        const bool up = mloc > m_ref + 8.f;
        if (__ballot(up)) {
            const float m_new = up ? mloc : m_ref;
            const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < NCT; ++i) acc[i] *= alpha;
            m_ref = m_new;
        }
        const float mexp = (causal && m_ref == -INFINITY) ? INFINITY : m_ref;
        float psum = 0.f;
        uint32_t pk[4];
#pragma unroll
        for (int r = 0; r < 8; r += 2) {
            const float p0 = __builtin_amdgcn_exp2f(sv[r] - mexp);
            const float p1 = __builtin_amdgcn_exp2f(sv[r + 1] - mexp);
            psum += p0 + p1;
            pk[r >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p0, p1}, f16x2));
        }
        l_run += psum;
        const u32x4 pf = {pk[0], pk[1], pk[2], pk[3]};
#pragma unroll
        for (int i = 0; i < NCT; ++i) {
            const int ch = 16 * i + c16;
            const u32x4 vf = vl[cur][ch * 4 + (g16 ^ vswz(ch))];
            acc[i] = mfma16_f16(vf, pf, acc[i]);
        }
        stage(cur ^ 1, min(blk + 1, blk1 - 1));
        fetch(min(blk + 2, blk1 - 1));
        __syncthreads();
    }

    const float l_tot = sum32(sum16(l_run));
    if (!vq) return;
    if (g16 == 0) mlp[qvg] = make_float2(m_ref, l_tot);
    float *dst = accp + (size_t)qvg * HD;
#pragma unroll
    for (int i = 0; i < NCT; ++i)
        *(float4 *)(dst + 16 * i + 4 * g16) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
}

hipError_t launch_attention(const StepArgs &a, int n_split, hipStream_t s) {
    if (a.dtype != DG_BF16) return launch_attention_f32(a, s);
    const int G = a.Hq / a.Hkv;
    const dim3 grid((G * a.C + 127) / 128, a.B * a.Hkv, n_split);
    switch (a.hd) {
        case 64: hipLaunchKernelGGL((k_attn_bf16<64>), grid, dim3(256), 0, s, a); break;
        case 128: hipLaunchKernelGGL((k_attn_q16<128>), grid, dim3(512), 0, s, a); break;
        case 256: hipLaunchKernelGGL((k_attn_q16<256>), grid, dim3(512), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dg
