// bf16 MFMA projections of the canvas step, all of the form
//     Y^T[n, t] = sum_k W[n, k] X[t, k]          (W: [out, in], X: token rows)
// computed as 32x32x16 MFMA tiles with the weight rows as the A operand and
// the token rows as the B operand, so that one lane ends up holding one token
// and 16 output features of a tile.  The epilogues then work per lane:
//   * QKV: RMS row scale, RoPE (the tile pairs features j and j + hd/2 so that
//     both halves of a rotation pair sit in the same lane), stores of q and of
//     the canvas K / V rows into the caller's cache;
//   * O-proj: residual add of the token embedding;
//   * LM head: RMS row scale and per-(token, 128-id slice) softmax statistics
//     (max, sum of exp, second max, argmax), so the logits never reach memory.
//
// Work split: a workgroup of 4 waves owns BN = 32*NT weight rows and
// 4 * 32*TM token rows.  The weight tile of each 64-wide K stage is staged in
// LDS (shared by the 4 waves, XOR-swizzled 16-byte chunks); each wave reads
// its own token rows straight from global memory into registers (they are
// small and L2-resident).  Register queues of depth PF keep PF stages of
// global loads in flight.  Workgroups that share a weight tile are placed on
// the same XCD (blockIdx % 8) so the tile is fetched from HBM once.
#include <limits.h>

#include <type_traits>

#include <hip/hip_ext.h>

#include "dg_device.hpp"
#include "dg_gemm.hpp"
#include "dg_internal.hpp"

namespace dg {

hipError_t launch_qkv_f32(const StepArgs &a, int kv_only, int mode, hipStream_t s);
hipError_t launch_oproj_f32(const StepArgs &a, hipStream_t s);
hipError_t launch_lmhead_f32(const StepArgs &a, float *logits, hipStream_t s);


// Stores one rotated / scaled (j, j + hd/2) pair group of row t, head hh:
// 4 consecutive features starting at jj0 of each half.  Queries are held in
// fp32 (they never leave the step); canvas K / V rows go to the cache in
// bf16, V transposed.
__device__ __forceinline__ void qkv_store4(const StepArgs &a, int t, int hh, int jj0, const float (&y0)[4],
                                           const float (&y1)[4]) {
    const int b = t / a.C;
    const int ic = t - b * a.C;
    const int hd2 = a.hd / 2;
    const int64_t pos = a.reqs.len[b] + ic;
    const uint2 lo = make_uint2(pack_bf2(y0[0], y0[1]), pack_bf2(y0[2], y0[3]));
    const uint2 hi = make_uint2(pack_bf2(y1[0], y1[1]), pack_bf2(y1[2], y1[3]));
    if (hh < a.Hq) {
        float *q = (float *)(a.ws + a.L.q) + ((size_t)t * a.Hq + hh) * a.hd;
        *(float4 *)(q + jj0) = make_float4(y0[0], y0[1], y0[2], y0[3]);
        *(float4 *)(q + jj0 + hd2) = make_float4(y1[0], y1[1], y1[2], y1[3]);
    } else if (hh < a.Hq + a.Hkv) {
        const int g = hh - a.Hq;
        uint16_t *kr = (uint16_t *)a.reqs.k[b] + ((size_t)g * a.reqs.cap[b] + pos) * a.hd;
        *(uint2 *)(kr + jj0) = lo;
        *(uint2 *)(kr + jj0 + hd2) = hi;
    } else {
        const int g = hh - a.Hq - a.Hkv;
        const int64_t cap = a.reqs.cap[b];
        uint16_t *vt = (uint16_t *)a.reqs.v[b] + (size_t)g * a.hd * cap + pos;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vt[(size_t)(jj0 + e) * cap] = f2bf(y0[e]);
            vt[(size_t)(jj0 + hd2 + e) * cap] = f2bf(y1[e]);
        }
    }
}

// Row scale and RoPE of 4 pairs (features jj0..jj0+3 and their partners),
// with the pairs' (cos, sin) given (cs01, cs23: pairs 0,1 and 2,3).
__device__ __forceinline__ void qkv_finish4_cs(bool rotate, float (&y0)[4], float (&y1)[4], float re,
                                               const float4 &cs01, const float4 &cs23) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        y0[e] *= re;
        y1[e] *= re;
    }
    if (rotate) {
        const float c[4] = {cs01.x, cs01.z, cs23.x, cs23.z};
        const float sn[4] = {cs01.y, cs01.w, cs23.y, cs23.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x1 = y0[e], x2 = y1[e];
            y0[e] = x1 * c[e] - x2 * sn[e];
            y1[e] = x1 * sn[e] + x2 * c[e];
        }
    }
}

__device__ __forceinline__ const float4 *rope_pairs(const StepArgs &a, int t, int jj0) {
    return (const float4 *)((const float2 *)(a.ws + a.L.rope) + (size_t)t * (a.hd / 2) + jj0);
}

// The same, loading the pairs' (cos, sin) from the RoPE table.
__device__ __forceinline__ void qkv_finish4(const StepArgs &a, int t, int hh, int jj0, float (&y0)[4],
                                            float (&y1)[4], float re) {
    const bool rotate = hh < a.Hq + a.Hkv;
    float4 cs01 = make_float4(0, 0, 0, 0), cs23 = cs01;
    if (rotate) {
        const float4 *rp = rope_pairs(a, t, jj0);
        cs01 = rp[0];
        cs23 = rp[1];
    }
    qkv_finish4_cs(rotate, y0, y1, re, cs01, cs23);
}

__device__ __forceinline__ bool row_writable(const StepArgs &a, int t, int mode) {
    if (mode == WRITE_ALWAYS) return true;
    if (a.only_req >= 0 && t / a.C != a.only_req) return false;
    const bool dn = a.done[t / a.C] != 0;
    return (mode == WRITE_STEP) ? !dn : dn;
}

// ---------------------------------------------------------------------------
// QKV projection.  Tile nt = (head hh, pair block u) covers features j in
// [32u, 32u+32) (MFMA tile 0) and j + hd/2 (tile 1) of head hh; the K axis
// is cut into S chunks.  S == 1: RMS scale + RoPE + scatter in the epilogue.
// S > 1: fp32 partial sums [S][M][(Hq+2Hkv)*hd], finished by k_qkv_finish.
// KH = 2 or 4 (S == 1, TM == 1): 256 KH threads, KH groups of four waves
// each take one part of the K axis (own LDS staging buffers, same barriers);
// the other groups hand their accumulators to group 0 through LDS, which
// adds them in a fixed order ((g0 + g2) + (g1 + g3) for four parts) and runs
// the epilogue, so no partial sums leave the CU.
// ---------------------------------------------------------------------------
// WPG: waves per K part (4: 128 token rows per workgroup; 2: 64 rows, twice
// the workgroups over the same weights, each staging thread carrying four
// weight rows per stage instead of two).
template <int TM, int PW, int PA, bool PARTIAL, int NSTC, int KH = 1, int SRC = SRC_EMBED, bool W8 = false,
          int WPG = 4>
__global__ __launch_bounds__(64 * WPG * KH) void k_qkv_bf16(StepArgs a, int kv_only, int mode, int n_mt, int S) {
    static_assert(KH == 1 || ((KH == 2 || KH == 4) && TM == 1 && !PARTIAL), "K parts: one row tile, no partials");
    static_assert(WPG == 4 || (WPG == 2 && TM == 1), "64-row workgroups: one row tile");
    constexpr int NTH = 64 * WPG;                      // threads per K part
    constexpr int NL = 8 / WPG;                        // weight rows per staging thread and stage (64 in all)
    constexpr int ROWS = 32 * WPG * TM;                // token rows per workgroup
    __shared__ u32x4 lds[KH][2 * NL * NTH];
    const int kh = (KH > 1) ? (int)(threadIdx.x / NTH) : 0;
    const int pph = a.hd / 64;
    const int n_heads = kv_only ? 2 * a.Hkv : a.Hq + 2 * a.Hkv;
    const int n_nt = n_heads * pph;
    int j;
    if (!xcd_index(S * n_nt * n_mt, j)) return;
    const int kc = j / (n_nt * n_mt);
    const int rem = j - kc * n_nt * n_mt;
    const int nt = rem / n_mt, mt = rem - (rem / n_mt) * n_mt;
    const int tid = threadIdx.x % NTH, wave = tid >> 6, lane = tid & 63, half = lane >> 5, row32 = lane & 31;
    const int tok_wg = mt * ROWS;
    if (mode != WRITE_ALWAYS && none_active(a, tok_wg, tok_wg + ROWS)) return;
    const int hh = nt / pph + (kv_only ? a.Hq : 0);
    const int u = nt % pph;
    const int kchunk = a.d / S / KH;
    const int k0 = kc * (a.d / S) + kh * kchunk;
    const uint16_t *W;
    int base;
    if (hh < a.Hq) { W = (const uint16_t *)a.wq; base = hh * a.hd; }
    else if (hh < a.Hq + a.Hkv) { W = (const uint16_t *)a.wk; base = (hh - a.Hq) * a.hd; }
    else { W = (const uint16_t *)a.wv; base = (hh - a.Hq - a.Hkv) * a.hd; }

    // staged row r = tid / 8 + x NTH / 8 of the 64: rows 0..31 are tile 0
    // (features 32 u ..), rows 32..63 tile 1 (the same plus hd / 2)
    const uint16_t *wp[NL];
#pragma unroll
    for (int x = 0; x < NL; ++x) {
        const int r = (tid >> 3) + x * (NTH / 8);
        const size_t off = (size_t)(base + 32 * u + (r >> 5) * (a.hd / 2) + (r & 31)) * a.d + k0 + (tid & 7) * 8;
        wp[x] = W8 ? (const uint16_t *)((const uint8_t *)W + off) : W + off;
    }
    // SRC_EMBED: activations gathered straight from the embedding rows of
    // the fed ids: lane (row32, half) streams features k0 + 16 kk + 8 half ..
    // + 7 of its row, the operand layout of the MFMA.  Rows past M read row
    // M - 1 (their results are not stored).  The row's RMSNorm scale comes
    // from the per-id table when there is one, else from r_e.
    // SRC_RESID (a deeper layer): the residual stream x as its fp16 hi and lo
    // planes (fragment-major, ~22 significant bits, two MFMAs against the
    // weights converted to fp16 in LDS); the row scale is r_x.
    const void *ap[TM];
    float re[TM];
    const int tok0 = tok_wg + wave * 32 * TM;
    const int32_t *inp = (const int32_t *)(a.ws + a.L.inp);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int t = min(tok0 + tm * 32 + row32, a.M - 1);
        if constexpr (SRC == SRC_RESID) {
            const int tb = min(tok0 / 32 + tm, a.L.m_pad / 32 - 1);
            ap[tm] = (const uint16_t *)(a.ws + a.L.xp) + ((size_t)tb * (a.d / 16) + k0 / 16) * 512 + lane * 8;
            re[tm] = ((const float *)(a.ws + a.L.r_x))[t];
        } else {
            const int tok = inp[t];
            ap[tm] = (const uint16_t *)a.embed + (size_t)tok * a.d + k0 + half * 8;
            re[tm] = a.L.has_escale ? ((const float *)(a.ws + a.L.escale))[tok] : ((const float *)(a.ws + a.L.r_e))[t];
        }
    }
    // K parts in the workgroup (up to 512 threads): the parts are summed
    // scattered, each group finishing RG = 4 / KH of the four 8-feature
    // register groups (rg = kh RG ..), so that all the workgroup's waves
    // share the epilogue; each group loads its rows' RoPE pairs and done
    // flags before the K loop, whose time then covers their latency.  (1024
    // threads: the registers would spill; group 0 finishes everything.)
    constexpr bool SCAT = KH > 1 && !PARTIAL && 64 * WPG * KH <= 512;
    constexpr int RG = SCAT ? 4 / KH : 1;
    static_assert(!SCAT || 8 * (KH - 1) <= 2 * KH * NL, "the scatter's LDS slots fit the staging buffers");
    const bool rotate = hh < a.Hq + a.Hkv;
    float4 cs[RG][2];
    bool wr = false;
    if constexpr (SCAT) {
        const int t = min(tok0 + row32, a.M - 1);      // one row tile (TM == 1)
        wr = tok0 + row32 < a.M && row_writable(a, t, mode);
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            cs[r][0] = cs[r][1] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (rotate) {
                const float4 *rp = rope_pairs(a, t, 32 * u + 8 * (kh * RG + r) + 4 * half);
                cs[r][0] = rp[0];
                cs[r][1] = rp[1];
            }
        }
    }
    f32x16 acc[2][TM];
    if constexpr (SRC == SRC_RESID)
        gemm_core<2, TM, PW, PA, 2, NSTC, NL, NTH, true, true, 512, W8>(wp, 0, ap, kchunk, lds[kh], acc, true,
                                                                        (size_t)a.L.m_pad * a.d);
    else
        gemm_core<2, TM, PW, PA, 1, NSTC, NL, NTH, true, false, 16, W8>(wp, 0, ap, kchunk, lds[kh], acc);
    if constexpr (SCAT) {
        float4 y[2][RG];
        kparts_scatter<KH, NTH>(acc, &lds[0][0], kh, tid, y);
        if constexpr (W8) {
            // the weights' per-output-row scales of the owned register groups
            const float *sc = (hh < a.Hq ? a.sq : (hh < a.Hq + a.Hkv ? a.sk : a.sv)) + base + 32 * u;
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int r = 0; r < RG; ++r) {
                    const float4 s4 = *(const float4 *)(sc + x * (a.hd / 2) + 8 * (kh * RG + r) + 4 * half);
                    y[x][r].x *= s4.x;
                    y[x][r].y *= s4.y;
                    y[x][r].z *= s4.z;
                    y[x][r].w *= s4.w;
                }
        }
        if (!wr) return;
        const int t = tok0 + row32;
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const int jj0 = 32 * u + 8 * (kh * RG + r) + 4 * half;
            float y0[4] = {y[0][r].x, y[0][r].y, y[0][r].z, y[0][r].w};
            float y1[4] = {y[1][r].x, y[1][r].y, y[1][r].z, y[1][r].w};
            qkv_finish4_cs(rotate, y0, y1, re[0], cs[r][0], cs[r][1]);
            qkv_store4(a, t, hh, jj0, y0, y1);
        }
        return;
    }
    if constexpr (KH > 1) {
        kparts_reduce<KH, NTH>(acc, &lds[0][0], kh, tid);
        if (kh != 0) return;
    }

    if constexpr (W8) {
        // the weights' per-output-row scales (features 32 u + 8 rg + 4 half
        // + e of tile 0, the same plus hd / 2 of tile 1)
        const float *sc = (hh < a.Hq ? a.sq : (hh < a.Hq + a.Hkv ? a.sk : a.sv)) + base + 32 * u;
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const float4 s4 = *(const float4 *)(sc + x * (a.hd / 2) + 8 * rg + 4 * half);
#pragma unroll
                for (int tm = 0; tm < TM; ++tm) {
                    acc[x][tm][4 * rg] *= s4.x;
                    acc[x][tm][4 * rg + 1] *= s4.y;
                    acc[x][tm][4 * rg + 2] *= s4.z;
                    acc[x][tm][4 * rg + 3] *= s4.w;
                }
            }
    }
    if (PARTIAL) {
        const int n_all = (a.Hq + 2 * a.Hkv) * a.hd;
        float *part = (float *)(a.ws + a.L.gemm_part) + (size_t)kc * a.M * n_all;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const int t = tok0 + tm * 32 + row32;
            if (t >= a.M) continue;
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int col = hh * a.hd + 32 * u + x * (a.hd / 2) + 8 * rg + 4 * half;
                    *(float4 *)(part + (size_t)t * n_all + col) =
                        make_float4(acc[x][tm][4 * rg], acc[x][tm][4 * rg + 1], acc[x][tm][4 * rg + 2], acc[x][tm][4 * rg + 3]);
                }
        }
        // one tile column of the first chunk hands the table's row scales to
        // the finishing kernel
        if (a.L.has_escale && kc == 0 && nt == 0 && half == 0) {
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
                const int t = tok0 + tm * 32 + row32;
                if (t < a.M) ((float *)(a.ws + a.L.r_e))[t] = re[tm];
            }
        }
        return;
    }
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int t = tok0 + tm * 32 + row32;
        if (t >= a.M || !row_writable(a, t, mode)) continue;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int jj0 = 32 * u + 8 * rg + 4 * half;
            float y0[4], y1[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                y0[e] = acc[0][tm][4 * rg + e];
                y1[e] = acc[1][tm][4 * rg + e];
            }
            qkv_finish4(a, t, hh, jj0, y0, y1, re[tm]);
            qkv_store4(a, t, hh, jj0, y0, y1);
        }
    }
}

// Sum of the S partial chunks (fixed order), then row scale, RoPE, stores.
// Grid (M, heads); thread = 4 consecutive pairs of one head.
__global__ __launch_bounds__(64) void k_qkv_finish(StepArgs a, int kv_only, int mode, int S) {
    const int t = blockIdx.x;
    const int hh = blockIdx.y + (kv_only ? a.Hq : 0);
    if (!row_writable(a, t, mode)) return;
    const int hd2 = a.hd / 2;
    const int jj0 = 4 * threadIdx.x;
    if (jj0 >= hd2) return;
    const int n_all = (a.Hq + 2 * a.Hkv) * a.hd;
    const float *part = (const float *)(a.ws + a.L.gemm_part) + (size_t)t * n_all + hh * a.hd + jj0;
    float y0[4] = {0.f, 0.f, 0.f, 0.f}, y1[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s) {
        const float4 p0 = *(const float4 *)(part + (size_t)s * a.M * n_all);
        const float4 p1 = *(const float4 *)(part + (size_t)s * a.M * n_all + hd2);
        y0[0] += p0.x; y0[1] += p0.y; y0[2] += p0.z; y0[3] += p0.w;
        y1[0] += p1.x; y1[1] += p1.y; y1[2] += p1.z; y1[3] += p1.w;
    }
    qkv_finish4(a, t, hh, jj0, y0, y1, ((const float *)(a.ws + a.L.r_e))[t]);
    qkv_store4(a, t, hh, jj0, y0, y1);
}

// ---------------------------------------------------------------------------
// Output projection o Wo^T (tile of 64 features, K cut into S chunks).  The
// fp32 attention output enters as its fp16 hi and lo planes (about 22
// significant bits), multiplied with Wo converted to fp16 in LDS.  Writes
// fp32 partial sums [S][M][d]; k_oproj_finish adds the residual.
// ---------------------------------------------------------------------------
// Also the FFN's down projection: W = w_down, K = d_ff, the activation's
// planes.
// WPG waves per K part (32 WPG token rows per workgroup) and KH parts of the
// chunk inside the workgroup, reduced through LDS (kparts_reduce).  FC
// output features per workgroup (64, or 128 for many token rows: each
// workgroup reads its rows' activation planes whole, so wider tiles read
// them fewer times).
template <int TM, int PW, int PA, int NSTC, bool W8 = false, int WPG = 4, int KH = 1, int FC = 64>
__global__ __launch_bounds__(64 * WPG * KH) void k_oproj_bf16(StepArgs a, int n_mt, int S, const uint16_t *W, int K,
                                                              const uint16_t *o, const float *wsc) {
    static_assert(WPG == 4 || (WPG == 2 && TM == 1), "64-row workgroups: one row tile");
    static_assert(KH == 1 || (KH == 2 && TM == 1), "K parts: one row tile");
    static_assert(FC == 64 || (FC == 128 && KH == 1 && WPG == 4), "128-feature tiles: 128 rows, one K part");
    constexpr int NT = FC / 32;                        // MFMA tiles per wave
    constexpr int NTH = 64 * WPG;
    constexpr int NL = FC * 8 / NTH;                   // staged weight rows per thread and stage
    constexpr int ROWS = 32 * WPG * TM;
    __shared__ u32x4 lds[KH][2 * NL * NTH];
    const int kh = (KH > 1) ? (int)(threadIdx.x / NTH) : 0;
    const int n_nt = a.d / FC;
    int j;
    if (!xcd_index(S * n_nt * n_mt, j)) return;
    const int kc = j / (n_nt * n_mt);
    const int rem = j - kc * n_nt * n_mt;
    const int nt = rem / n_mt, mt = rem - (rem / n_mt) * n_mt;
    const int tid = threadIdx.x % NTH, wave = tid >> 6, lane = tid & 63, half = lane >> 5, row32 = lane & 31;
    const int tok_wg = mt * ROWS;
    if (none_active(a, tok_wg, tok_wg + ROWS)) return;
    const int kchunk = K / S / KH;
    const int k0 = kc * (K / S) + kh * kchunk;
    const uint16_t *wp[NL];
#pragma unroll
    for (int x = 0; x < NL; ++x) {
        const size_t off = (size_t)(FC * nt + (tid >> 3) + x * (NTH / 8)) * K + k0 + (tid & 7) * 8;
        wp[x] = W8 ? (const uint16_t *)((const uint8_t *)W + off) : W + off;
    }
    const void *ap[TM];
    const int tok0 = tok_wg + wave * 32 * TM;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int tb = min(tok0 / 32 + tm, a.L.m_pad / 32 - 1);
        ap[tm] = o + ((size_t)tb * (K / 16) + k0 / 16) * 512 + lane * 8;
    }
    f32x16 acc[NT][TM];
    gemm_core<NT, TM, PW, PA, 2, NSTC, NL, NTH, true, true, 512, W8>(wp, 0, ap, kchunk, lds[kh], acc, true,
                                                                     (size_t)a.L.m_pad * K);
    if constexpr (KH > 1) {
        kparts_reduce<KH, NTH>(acc, &lds[0][0], kh, tid);
        if (kh != 0) return;
    }
    if constexpr (W8) {
        // per-output-row scales of the weights (features FC nt + 32 x + 8 rg + 4 half + e)
#pragma unroll
        for (int x = 0; x < NT; ++x)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const float4 s4 = *(const float4 *)(wsc + FC * nt + 32 * x + 8 * rg + 4 * half);
#pragma unroll
                for (int tm = 0; tm < TM; ++tm) {
                    acc[x][tm][4 * rg] *= s4.x;
                    acc[x][tm][4 * rg + 1] *= s4.y;
                    acc[x][tm][4 * rg + 2] *= s4.z;
                    acc[x][tm][4 * rg + 3] *= s4.w;
                }
            }
    }

    float *part = (float *)(a.ws + a.L.gemm_part) + (size_t)kc * a.M * a.d;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int t = tok0 + tm * 32 + row32;
        if (t >= a.M) continue;
#pragma unroll
        for (int x = 0; x < NT; ++x)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int n = FC * nt + 32 * x + 8 * rg + 4 * half;
                *(float4 *)(part + (size_t)t * a.d + n) =
                    make_float4(acc[x][tm][4 * rg], acc[x][tm][4 * rg + 1], acc[x][tm][4 * rg + 2], acc[x][tm][4 * rg + 3]);
            }
    }
}

// y = residual + sum of the S partial chunks (fixed order), held in fp32,
// one workgroup per row.  The residual is E[tok] (SRC_EMBED: the first
// layer's attention) or x (SRC_RESID).  OUT_LMHEAD (the last projection of
// the last layer): y is h, with its RMS row scale r_h, the fp16 copy the
// vocabulary product consumes and the fp32 copy the sampler's exact leading
// logits read (both for positions still uncommitted, over the compact rows)
// and, on request, an fp32 row-major dump.  OUT_RESID: y is the residual
// stream x for the next projection: x in fp32 (in place), its fp16 hi and lo
// planes and its row scale r_x.
template <int SRC, int OUT>
__global__ __launch_bounds__(256) void k_resid_finish(StepArgs a, int S, float *hdump, int moe_add, int want_xr) {
    __shared__ float sh[4];
    const int t = blockIdx.x;
    const int b = t / a.C;
    if (!req_active(a, b)) return;
    const int tok = ((const int32_t *)(a.ws + a.L.inp))[t];
    const uint16_t *erow = (const uint16_t *)a.embed + (size_t)tok * a.d;
    float *xrow = (float *)(a.ws + a.L.x) + (size_t)t * a.d;
    const float *part = (const float *)(a.ws + a.L.gemm_part) + (size_t)t * a.d;
    uint16_t *hfrag = (uint16_t *)(a.ws + a.L.h);
    float *hf32 = (float *)(a.ws + a.L.hf);
    uint16_t *xp = (uint16_t *)(a.ws + a.L.xp);
    const size_t plane = (size_t)a.L.m_pad * a.d;
    int jc = -1, rc = 0;
    if (OUT == OUT_LMHEAD) {
        jc = ((const int32_t *)(a.ws + a.L.uidx))[t];
        rc = b * a.L.cp + jc;                          // compact row (jc < 0: committed, not sampled)
    }
    float ss = 0.f;
    for (int c = threadIdx.x; c < a.d / 4; c += 256) {
        const int n = 4 * c;
        float4 acc = *(const float4 *)(part + n);
        for (int s = 1; s < S; ++s) {
            const float4 p = *(const float4 *)(part + (size_t)s * a.M * a.d + n);
            acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
        }
        if (moe_add) {
            // the routed experts' gated outputs of this token, in rank order
            const float *ym = (const float *)(a.ws + a.L.moe_y) + (size_t)t * a.top_k * a.d + n;
            for (int jj = 0; jj < a.top_k; ++jj) {
                const float4 p = *(const float4 *)(ym + (size_t)jj * a.d);
                acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
            }
        }
        float r0, r1, r2, r3;
        if (SRC == SRC_RESID) {
            const float4 xv = *(const float4 *)(xrow + n);
            r0 = xv.x; r1 = xv.y; r2 = xv.z; r3 = xv.w;
        } else {
            const uint2 ev = *(const uint2 *)(erow + n);
            r0 = __uint_as_float(ev.x << 16); r1 = __uint_as_float(ev.x & 0xffff0000u);
            r2 = __uint_as_float(ev.y << 16); r3 = __uint_as_float(ev.y & 0xffff0000u);
        }
        const float h0 = r0 + acc.x, h1 = r1 + acc.y, h2 = r2 + acc.z, h3 = r3 + acc.w;
        if (OUT == OUT_LMHEAD) {
            if (jc >= 0) {
                *(uint2 *)(hfrag + frag_index(rc, n, a.d)) = make_uint2(pack_h2(h0, h1), pack_h2(h2, h3));
                *(float4 *)(hf32 + (size_t)rc * a.d + n) = make_float4(h0, h1, h2, h3);
            }
            if (hdump) *(float4 *)(hdump + (size_t)t * a.d + n) = make_float4(h0, h1, h2, h3);
        } else {
            *(float4 *)(xrow + n) = make_float4(h0, h1, h2, h3);
            const uint32_t p01 = pack_h2(h0, h1), p23 = pack_h2(h2, h3);
            const f32x2 f01 = __builtin_convertvector(__builtin_bit_cast(f16x2, p01), f32x2);
            const f32x2 f23 = __builtin_convertvector(__builtin_bit_cast(f16x2, p23), f32x2);
            const size_t fi = frag_index(t, n, a.d);
            const uint2 lo = make_uint2(pack_h2(h0 - f01.x, h1 - f01.y), pack_h2(h2 - f23.x, h3 - f23.y));
            *(uint2 *)(xp + fi) = make_uint2(p01, p23);
            *(uint2 *)(xp + plane + fi) = lo;
            if (want_xr) {                             // row-major planes: the experts gather rows
                uint16_t *xr = (uint16_t *)(a.ws + a.L.xr) + (size_t)t * a.d + n;
                *(uint2 *)xr = make_uint2(p01, p23);
                *(uint2 *)(xr + (size_t)a.M * a.d) = lo;
            }
        }
        ss += h0 * h0 + h1 * h1 + h2 * h2 + h3 * h3;
    }
    ss = block_sum_256(ss, sh);
    if (threadIdx.x == 0)
        ((float *)(a.ws + (OUT == OUT_LMHEAD ? a.L.r_h : a.L.r_x)))[t] = 1.0f / sqrtf(ss / (float)a.d + a.eps);
}

// ---------------------------------------------------------------------------
// FFN gate / up projection with the SwiGLU activation (deeper models).  Tile
// nt covers features [FW nt, FW nt + FW) of both Wg (MFMA tiles 0 .. NTF-1)
// and Wu (tiles NTF .. 2 NTF - 1), so each lane holds g and u of the same
// features of one token: act = silu(r g) * (r u), r = r_x, written as fp16 hi
// and lo planes (fragment-major [m_pad][d_ff]), the down projection's
// operand.  FW = 64 halves the reads of the activation planes per feature
// (each workgroup reads the token rows' planes whole) where the grid still
// fills the CUs.
// ---------------------------------------------------------------------------
template <int TM, int PW, int PA, int NSTC, bool W8 = false, int FW = 32>
__global__ __launch_bounds__(256) void k_ffn_up_bf16(StepArgs a, int n_mt) {
    constexpr int NTF = FW / 32;                       // 32-feature tiles of g (and of u)
    constexpr int NT = 2 * NTF;                        // MFMA tiles per wave
    constexpr int NL = NT;                             // staged weight rows per thread and stage
    __shared__ u32x4 lds[2 * NL * 256];
    const int n_nt = a.d_ff / FW;
    int j;
    if (!xcd_index(n_nt * n_mt, j)) return;
    const int nt = j / n_mt, mt = j - (j / n_mt) * n_mt;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, row32 = lane & 31;
    const int tok_wg = mt * 128 * TM;
    if (none_active(a, tok_wg, tok_wg + 128 * TM)) return;
    // staged row (tid >> 3) + 32 x: tile x, Wg for x < NTF, else Wu
    const uint16_t *wp[NL];
#pragma unroll
    for (int x = 0; x < NL; ++x) {
        const size_t off = (size_t)(FW * nt + 32 * (x % NTF) + (tid >> 3)) * a.d + (tid & 7) * 8;
        const void *W = x < NTF ? a.wg : a.wu;
        wp[x] = W8 ? (const uint16_t *)((const uint8_t *)W + off) : (const uint16_t *)W + off;
    }
    const void *ap[TM];
    const int tok0 = tok_wg + wave * 32 * TM;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int tb = min(tok0 / 32 + tm, a.L.m_pad / 32 - 1);
        ap[tm] = (const uint16_t *)(a.ws + a.L.xp) + (size_t)tb * (a.d / 16) * 512 + lane * 8;
    }
    f32x16 acc[NT][TM];
    gemm_core<NT, TM, PW, PA, 2, NSTC, NL, 256, true, true, 512, W8>(wp, 0, ap, a.d, lds, acc, true,
                                                                     (size_t)a.L.m_pad * a.d);
    if constexpr (W8) {
        // per-output-row scales of Wg (tiles 0 ..) and Wu (tiles NTF ..): features FW nt + 32 jt + 8 rg + 4 half + e
#pragma unroll
        for (int jt = 0; jt < NTF; ++jt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int f = FW * nt + 32 * jt + 8 * rg + 4 * half;
                const float4 g4 = *(const float4 *)(a.sg + f);
                const float4 u4 = *(const float4 *)(a.su + f);
#pragma unroll
                for (int tm = 0; tm < TM; ++tm) {
                    acc[jt][tm][4 * rg] *= g4.x; acc[jt][tm][4 * rg + 1] *= g4.y;
                    acc[jt][tm][4 * rg + 2] *= g4.z; acc[jt][tm][4 * rg + 3] *= g4.w;
                    acc[NTF + jt][tm][4 * rg] *= u4.x; acc[NTF + jt][tm][4 * rg + 1] *= u4.y;
                    acc[NTF + jt][tm][4 * rg + 2] *= u4.z; acc[NTF + jt][tm][4 * rg + 3] *= u4.w;
                }
            }
    }
    uint16_t *act = (uint16_t *)(a.ws + a.L.act);
    const size_t plane = (size_t)a.L.m_pad * a.d_ff;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int t = tok0 + tm * 32 + row32;
        if (t >= a.M || !req_active(a, t / a.C)) continue;
        const float r = ((const float *)(a.ws + a.L.r_x))[t];
#pragma unroll
        for (int jt = 0; jt < NTF; ++jt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float g = r * acc[jt][tm][4 * rg + e], u = r * acc[NTF + jt][tm][4 * rg + e];
                    y[e] = g / (1.0f + __expf(-g)) * u;
                }
                const uint32_t p01 = pack_h2(y[0], y[1]), p23 = pack_h2(y[2], y[3]);
                const f32x2 f01 = __builtin_convertvector(__builtin_bit_cast(f16x2, p01), f32x2);
                const f32x2 f23 = __builtin_convertvector(__builtin_bit_cast(f16x2, p23), f32x2);
                const size_t fi = frag_index(t, FW * nt + 32 * jt + 8 * rg + 4 * half, a.d_ff);
                *(uint2 *)(act + fi) = make_uint2(p01, p23);
                *(uint2 *)(act + plane + fi) =
                    make_uint2(pack_h2(y[0] - f01.x, y[1] - f01.y), pack_h2(y[2] - f23.x, y[3] - f23.y));
            }
    }
}

// ---------------------------------------------------------------------------
// Vocabulary head + fused sampler statistics over the positions still
// uncommitted (a committed position's logits are never read: its token is
// fixed).  Workgroup (slice nt, request b): 128 ids x the request's compact
// rows, 8 waves; wave w multiplies all 128 ids of the slice with compact rows
// 32w .. 32w+31 (two waves per SIMD hide each other's barrier and LDS waits;
// every activation fragment is loaded by exactly one wave).  Waves past the
// request's count only help stage the weight tiles.
// z~ = r_h[t] * (fp16(h_t) . Wlm[v]): fp16 MFMAs, the weight tile converted
// from bf16 while it is staged in LDS.  The MASK id and ids >= V are
// excluded.  Writes one (m, sum exp, m2, ids of m and m2) record per (slice,
// compact row).  These are statistics of the fp16-operand logits z~ (within
// r_h 2^-11 sum |h| |W| of the logits of the fp32 h); the sampler recomputes
// the logits of the two leading ids from the fp32 h and corrects m, m2, the
// sum and the entropy term with them (k_sample_commit).
// W8: the head is e4m3 bytes with one fp32 scale per vocabulary row:
// z~ = r_h[t] * s_v * (fp16(h_t) . e4m3(W_v)); the bytes are converted to fp16
// (exactly) while they are staged, and the scales multiply the accumulators
// before the statistics.
// ---------------------------------------------------------------------------
// One launch shape for every count of open rows: the 8 waves split the
// slice's 4 id tiles of 32 among themselves as the row tiles allow, so that
// with few open rows the MFMAs are spread over all SIMDs instead of sitting
// on one wave per row tile.  NTW id tiles per wave, G = 4 / NTW waves per row
// tile; wave w takes row tile w / G and id tiles NTW (w % G) ...; the G
// partial statistics of a row are merged through LDS in id order.
// The workgroup's row tiles: those of requests b0 .. b0 + nb - 1 in order,
// pre[k] .. pre[k + 1] - 1 being request b0 + k's (its open rows in tiles of
// 32), pre[nb] <= 8 in all; entries k >= nb hold no rows.
struct RowTiles {
    int b0, nb;
    int pre[DG_LM_GROUP_MAX + 1];
    int cnt[DG_LM_GROUP_MAX];
};

// Temperature sampling: 1 / T_s for request b at its coming step s.
__device__ __forceinline__ float inv_temperature(const StepArgs &a, int b) {
    const int s = a.step[b] + 1;
    const float T = a.N <= 1 ? a.temp0 : a.temp0 + (a.temp1 - a.temp0) * (float)(s - 1) / (float)(a.N - 1);
    return 1.0f / T;
}

template <int NTW, int PW, int PA, int NSTC, bool W8, bool SAMP>
__device__ __forceinline__ void lmhead_tiles(const StepArgs &a, float *logits, int nt,
                                             const RowTiles &rtl, const uint16_t *const (&wp)[2], u32x4 *lds,
                                             const float *wsc, VStat *mrg /* [8 waves][32 rows] */,
                                             Top2 *kmrg /* [8 waves][32 rows] */) {
    constexpr int G = 4 / NTW;
    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, row32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches below
    const int rt = wave / G, ig = wave - (wave / G) * G;
    // request of this row tile and the tile's place among that request's rows
    // (constant indices only, so that the arrays stay in registers)
    int k = 0, pk = 0, cnt = rtl.cnt[0];
#pragma unroll
    for (int q = 1; q < DG_LM_GROUP_MAX; ++q)
        if (q < rtl.nb && rt >= rtl.pre[q]) {
            k = q;
            pk = rtl.pre[q];
            cnt = rtl.cnt[q];
        }
    const int b = rtl.b0 + k;
    const bool active = rt < rtl.pre[DG_LM_GROUP_MAX];
    const int j0 = active ? (rt - pk) * 32 : 0;   // first compact row of the wave
    const int wrow0 = 32 * NTW * ig;                   // first id of the wave within the slice
    const int rbase = b * a.L.cp;
    const void *ap[1];
    ap[0] = (const uint16_t *)(a.ws + a.L.h) + (size_t)((rbase + min(j0, a.L.cp - 32)) / 32) * (a.d / 16) * 512 +
            lane * 8;
    f32x16 acc[NTW][1];
    gemm_core<NTW, 1, PW, PA, 1, NSTC, 2, 512, true, true, 512, W8>(wp, wrow0, ap, a.d, lds, acc, active);

    const int jr = j0 + row32;                         // this lane's compact row
    const bool tv = active && jr < cnt;
    const int t = tv ? b * a.C + ((const int32_t *)(a.ws + a.L.ulist))[rbase + jr] : 0;
    const float rs = tv ? ((const float *)(a.ws + a.L.r_h))[t] : 0.f;
    const int v0 = 128 * nt + wrow0;                   // first id of the wave's tiles
    auto idv = [&](int o, int r) __attribute__((always_inline)) { return v0 + 32 * o + 8 * (r >> 2) + 4 * half + (r & 3); };
    const bool ent = a.ent != 0;
    constexpr bool samp = SAMP;      // temperature sampling: a kernel of its own
    VStat st{-INFINITY, 0.f, -INFINITY, INT_MAX, 0.f, INT_MAX};
    Top2 kt{-INFINITY, -INFINITY, INT_MAX, INT_MAX};   // two largest z / T + g (temperature sampling)
    if (active) {
        if constexpr (W8) {
            // accumulator element r of tile o is id 32 o + 8 (r / 4) + 4 half + r % 4
            // of the wave's tiles
#pragma unroll
            for (int o = 0; o < NTW; ++o)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 sc = *(const float4 *)&wsc[wrow0 + 32 * o + 8 * q + 4 * half];
                    acc[o][0][4 * q + 0] *= sc.x;
                    acc[o][0][4 * q + 1] *= sc.y;
                    acc[o][0][4 * q + 2] *= sc.z;
                    acc[o][0][4 * q + 3] *= sc.w;
                }
        }
        // Statistics of this lane's logits (raw dot products: rs > 0 keeps
        // the order, the scale is applied after).  EXCL: the tiles hold MASK
        // or ids >= V, which are pushed to -inf by adding a penalty (no
        // branches).
        auto stats = [&](auto EXCL_, auto ENT_) __attribute__((always_inline)) {
            constexpr bool EXCL = decltype(EXCL_)::value;
            constexpr bool ENT = decltype(ENT_)::value;   // also t = sum (z - m) exp(z - m)
            float x[NTW][16];
#pragma unroll
            for (int o = 0; o < NTW; ++o)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    x[o][r] = acc[o][0][r];
                    if constexpr (EXCL) {
                        const int v = idv(o, r);
                        x[o][r] += (v < a.V && v != a.mask_id) ? 0.f : -INFINITY;
                    }
                }
            float mx = -INFINITY;
#pragma unroll
            for (int o = 0; o < NTW; ++o)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x[o][r]);
            // lowest id attaining the max: ids grow with (o, r), so scan backwards
            int am = INT_MAX;
#pragma unroll
            for (int o = NTW - 1; o >= 0; --o)
#pragma unroll
                for (int r = 15; r >= 0; --r) am = (x[o][r] == mx) ? idv(o, r) : am;
            // the next entry in (value desc, id asc) order: the largest value
            // other than the argmax entry, at its lowest id
            float m2 = -INFINITY;
#pragma unroll
            for (int o = 0; o < NTW; ++o)
#pragma unroll
                for (int r = 0; r < 16; ++r) m2 = fmaxf(m2, (idv(o, r) == am) ? -INFINITY : x[o][r]);
            int a2 = INT_MAX;
#pragma unroll
            for (int o = NTW - 1; o >= 0; --o)
#pragma unroll
                for (int r = 15; r >= 0; --r) a2 = (x[o][r] == m2 && idv(o, r) != am) ? idv(o, r) : a2;
            st.m = rs * mx;
            st.m2 = rs * m2;
            st.a = (mx == -INFINITY) ? INT_MAX : am;
            st.a2 = (m2 == -INFINITY) ? INT_MAX : a2;
            // sum exp(z - m) and sum (z - m) exp(z - m), in the exp2 domain:
            // u = (z - m) log2(e), p = 2^u
            float ssum = 0.f, tsum = 0.f;
            if (mx != -INFINITY) {
                constexpr float LOG2E = 1.4426950408889634f;
                const float c = rs * LOG2E, off = st.m * LOG2E;
#pragma unroll
                for (int o = 0; o < NTW; ++o)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float u = fmaf(x[o][r], c, -off);
                        const float p = __builtin_amdgcn_exp2f(u);
                        ssum += p;
                        // an excluded id has u = -inf and p = 0: the clamp keeps
                        // the product at 0 (p is already 0 below u = -150)
                        if constexpr (ENT) tsum = fmaf(fmaxf(u, -256.f), p, tsum);
                    }
            }
            st.s = ssum;
            st.t = tsum * 0.6931471805599453f;        // back to natural units
            if constexpr (samp) if (tv) {
                // Gumbel-max candidates: z / T + g for this lane's ids; the 4
                // ids of a group share one Philox call (counter v >> 2)
                const float cz = rs * inv_temperature(a, b);
                const uint64_t pos = (uint64_t)(t - b * a.C), stp = (uint64_t)(a.step[b] + 1);
#pragma unroll
                for (int o = 0; o < NTW; ++o)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int vb = idv(o, 4 * q);
                        const Philox4 ph = philox4x64_10((uint64_t)(vb >> 2), pos, stp, (uint64_t)b, a.seed, 0ull);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float key = fmaf(x[o][4 * q + e], cz, gumbel_f32(ph.w[e]));
                            top2_push(kt, (x[o][4 * q + e] == -INFINITY) ? -INFINITY : key, vb + e);
                        }
                    }
            }
        };
        const bool excl = (v0 + 32 * NTW > a.V) || (a.mask_id >= v0 && a.mask_id < v0 + 32 * NTW);
        if (ent) {
            if (excl) stats(std::true_type{}, std::true_type{});
            else stats(std::false_type{}, std::true_type{});
        } else {
            if (excl) stats(std::true_type{}, std::false_type{});
            else stats(std::false_type{}, std::false_type{});
        }
        st = vmerge(st, vshfl_xor(st, 32));
        if constexpr (samp) kt = top2_merge(kt, top2_shfl_xor(kt, 32));
    }
    if constexpr (G > 1) {
        if (active && half == 0) {
            mrg[wave * 32 + row32] = st;
            if constexpr (samp) kmrg[wave * 32 + row32] = kt;
        }
        __syncthreads();
        if (active && ig == 0) {
#pragma unroll
            for (int g = 1; g < G; ++g) {
                st = vmerge(st, mrg[(wave + g) * 32 + row32]);
                if constexpr (samp) kt = top2_merge(kt, kmrg[(wave + g) * 32 + row32]);
            }
        }
    }
    if (tv && ig == 0 && half == 0) {
        const size_t rec = (size_t)(rbase + jr) * a.L.n_slices + nt;
        ((float4 *)(a.ws + a.L.lm_part))[rec] =
            make_float4(st.m, st.s, st.m2, __uint_as_float(pack_ids(st.a, st.m, st.a2, st.m2, 128 * nt)));
        if (ent) ((float *)(a.ws + a.L.lm_tpart))[rec] = st.t;
        if constexpr (samp)
            ((float4 *)(a.ws + a.L.lm_kpart))[rec] =
                make_float4(kt.k1, kt.k2, __uint_as_float(pack_ids(kt.i1, kt.k1, kt.i2, kt.k2, 128 * nt)), 0.f);
    }
    if (logits && tv) {
#pragma unroll
        for (int o = 0; o < NTW; ++o)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int v = idv(o, r);
                if (v < a.V) logits[(size_t)t * a.V + v] = (v == a.mask_id) ? -INFINITY : rs * acc[o][0][r];
            }
    }
}

// Workgroup (slice nt, group of bp consecutive requests): the open rows of
// the group's requests, at most 8 row tiles of 32 in all (the host picks bp
// from the commit schedule's bound on open rows), share one pass over the
// slice's weights.
template <int PW, int PA, int NSTC, bool W8, bool SAMP>
__device__ __forceinline__ void lmhead_body(const StepArgs &a, float *logits, int bp) {
    constexpr int NL = 2;
    __shared__ u32x4 lds[2 * 128 * 8];
    __shared__ __align__(16) float wsc[W8 ? 128 : 1];   // the slice's row scales
    __shared__ VStat mrg[8 * 32];
    __shared__ Top2 kmrg[SAMP ? 8 * 32 : 1];
    const int n_nt = (a.V + 127) / 128;
    const int n_grp = (a.B + bp - 1) / bp;
    int j;
    if (!xcd_index(n_nt * n_grp, j)) return;
    const int nt = j / n_grp, grp = j - (j / n_grp) * n_grp;
    RowTiles rtl;
    rtl.b0 = grp * bp;
    rtl.nb = min(bp, a.B - rtl.b0);
    rtl.pre[0] = 0;
#pragma unroll
    for (int q = 0; q < DG_LM_GROUP_MAX; ++q) {   // entries past nb: no rows
        const int b = rtl.b0 + q;
        const int c = (q >= rtl.nb || a.done[b]) ? 0 : ((const int32_t *)(a.ws + a.L.ucount))[b];
        rtl.cnt[q] = c;
        rtl.pre[q + 1] = rtl.pre[q] + ((c + 31) >> 5);
    }
    const int row_tiles = rtl.pre[DG_LM_GROUP_MAX];   // uniform over the workgroup
    if (row_tiles == 0) return;
    if (row_tiles > 8) {                               // more open rows than the host's bound: flagged, not computed
        if (threadIdx.x == 0) atomicAdd((int *)(a.ws + a.L.err) + 2, 1);
        return;
    }
    const int tid = threadIdx.x;
    const uint16_t *wp[NL];
#pragma unroll
    for (int x = 0; x < NL; ++x) {
        const int v = min(128 * nt + 64 * x + (tid >> 3), a.V - 1);
        if constexpr (W8) wp[x] = (const uint16_t *)((const uint8_t *)a.lm + (size_t)v * a.d + (tid & 7) * 8);
        else wp[x] = (const uint16_t *)a.lm + (size_t)v * a.d + (tid & 7) * 8;
    }
    // published by the first barrier of the product
    if (W8 && tid < 128) wsc[tid] = a.lm_scale[min(128 * nt + tid, a.V - 1)];
    if (row_tiles > 4) lmhead_tiles<4, PW, PA, NSTC, W8, SAMP>(a, logits, nt, rtl, wp, lds, wsc, mrg, kmrg);
    else if (row_tiles > 2) lmhead_tiles<2, PW, PA, NSTC, W8, SAMP>(a, logits, nt, rtl, wp, lds, wsc, mrg, kmrg);
    else lmhead_tiles<1, PW, PA, NSTC, W8, SAMP>(a, logits, nt, rtl, wp, lds, wsc, mrg, kmrg);
}

template <int PW, int PA, int NSTC, bool SAMP = false>
__global__ __launch_bounds__(512) void k_lmhead_bf16(StepArgs a, float *logits, int bp) {
    lmhead_body<PW, PA, NSTC, false, SAMP>(a, logits, bp);
}

template <int PW, int PA, int NSTC, bool SAMP = false>
__global__ __launch_bounds__(512) void k_lmhead_fp8(StepArgs a, float *logits, int bp) {
    lmhead_body<PW, PA, NSTC, true, SAMP>(a, logits, bp);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// Instantiations by stage count: fully unrolled for the counts the
// registered shapes use (8-stage split-K chunks, d = 2048 / 2816), rolled
// otherwise.
#define DG_NST_DISPATCH(nst, LAUNCH) \
    switch (nst) {                   \
        case 8: LAUNCH(8); break;    \
        case 16: LAUNCH(16); break;  \
        case 32: LAUNCH(32); break;  \
        case 44: LAUNCH(44); break;  \
        default: LAUNCH(0); break;   \
    }

// Ring depth of a K half of NSTC stages (0: a rolled loop over an even
// stage count): 4 where 4 divides the count, else 2.
template <int NSTC>
constexpr int half_ring() { return (NSTC > 0 && NSTC % 4 == 0) ? 4 : 2; }

// In-workgroup K split of the QKV projection: KH parts of WPG waves each.
// Four parts where the part's stage count d / 256 is even (twice the loads
// in flight per CU); 64-row workgroups (WPG = 2) where 128-row ones would
// leave most CUs idle.  The residual-stream operand (two planes) with 128-row
// workgroups keeps two parts: four would leave a wave 128 registers.
static void qkv_shape(const StepArgs &a, int src, int ntn, int &kh, int &wpg) {
    wpg = ntn * ((a.M + 127) / 128) < 256 ? 2 : 4;
    kh = (a.d % 512 == 0 && (src == SRC_EMBED || wpg == 2)) ? 4 : 2;
}

hipError_t launch_qkv(const StepArgs &a, int kv_only, int mode, hipStream_t s, int src) {
    if (a.dtype != DG_BF16) return launch_qkv_f32(a, kv_only, mode, s);
    const int n_heads = kv_only ? 2 * a.Hkv : a.Hq + 2 * a.Hkv;
    const int ntn = n_heads * (a.hd / 64);
    const int TM = gemm_tm(a.M);
    const int n_mt = (a.M + 128 * TM - 1) / (128 * TM);
    if (TM == 1 && (a.d / 64) % 4 == 0) {
        // K parts inside the workgroup: no partial sums, no finishing kernel.
        // A part of NST stages: a ring of 4 stages where 4 divides the count,
        // else of 2 (d = 2816: 22 stages per half)
        int kh, wpg;
        qkv_shape(a, src, ntn, kh, wpg);
        const int rows = 32 * wpg;
        const int n_mtw = (a.M + rows - 1) / rows;
        const dim3 g(grid_pad8(ntn * n_mtw));
        const int nst = a.d / 64 / kh;
        if (nst % 2) return hipErrorInvalidValue;     // the weight ring takes pairs of stages
#define L_QKVW(N, KHV, WPGV, SRCV, W8V)                                                                    \
    hipLaunchKernelGGL((k_qkv_bf16<1, half_ring<N>(), 2, false, N, KHV, SRCV, W8V, WPGV>), g,              \
                       dim3(64 * WPGV * KHV), 0, s, a, kv_only, mode, n_mtw, 1)
#define L_QKVB(N, KHV, WPGV)                                                                               \
    do {                                                                                                   \
        if (a.proj_fp8) {                                                                                  \
            if (src == SRC_RESID) L_QKVW(N, KHV, WPGV, SRC_RESID, true);                                   \
            else L_QKVW(N, KHV, WPGV, SRC_EMBED, true);                                                    \
        } else if (src == SRC_RESID) L_QKVW(N, KHV, WPGV, SRC_RESID, false);                               \
        else L_QKVW(N, KHV, WPGV, SRC_EMBED, false);                                                       \
    } while (0)
#define L_QKV8(N, KHV)                                                                                     \
    do {                                                                                                   \
        if (src == SRC_RESID) L_QKVW(N, KHV, 4, SRC_RESID, true);                                          \
        else L_QKVW(N, KHV, 4, SRC_EMBED, true);                                                           \
    } while (0)
        if (wpg == 2) {
            if (kh == 4) {
                switch (nst) {
                    case 8: L_QKVB(8, 4, 2); break;
                    default: L_QKVB(0, 4, 2); break;
                }
            } else {
                switch (nst) {
                    case 16: L_QKVB(16, 2, 2); break;
                    default: L_QKVB(0, 2, 2); break;
                }
            }
        } else if (kh == 4) {
            // (embedding operand only)
            switch (nst) {
                case 8:
                    if (a.proj_fp8) L_QKVW(8, 4, 4, SRC_EMBED, true);
                    else L_QKVW(8, 4, 4, SRC_EMBED, false);
                    break;
                default:
                    if (a.proj_fp8) L_QKVW(0, 4, 4, SRC_EMBED, true);
                    else L_QKVW(0, 4, 4, SRC_EMBED, false);
                    break;
            }
        } else {
#define L_QKV2(N)                       \
    do {                                \
        if (a.proj_fp8) L_QKV8(N, 2);   \
        else L_QKVB(N, 2, 4);           \
    } while (0)
            switch (nst) {
                case 8: L_QKV2(8); break;
                case 16: L_QKV2(16); break;
                case 22: L_QKV2(22); break;
                case 32: L_QKV2(32); break;
                default: L_QKV2(0); break;
            }
#undef L_QKV2
        }
#undef L_QKV8
#undef L_QKVB
#undef L_QKVW
        return hipGetLastError();
    }
    const int S = gemm_splitk(ntn * n_mt, a.d);
    const int nst = a.d / 64 / S;
    const dim3 g(grid_pad8(S * ntn * n_mt));
    const bool part = S > 1;
#define L_QKVS(N, SRCV)                                                                                                 \
    do {                                                                                                                \
        if (TM == 2 && part) hipLaunchKernelGGL((k_qkv_bf16<2, 4, 2, true, N, 1, SRCV>), g, dim3(256), 0, s, a, kv_only, mode, n_mt, S);  \
        else if (TM == 2) hipLaunchKernelGGL((k_qkv_bf16<2, 4, 2, false, N, 1, SRCV>), g, dim3(256), 0, s, a, kv_only, mode, n_mt, S);  \
        else if (part) hipLaunchKernelGGL((k_qkv_bf16<1, 4, 2, true, N, 1, SRCV>), g, dim3(256), 0, s, a, kv_only, mode, n_mt, S);      \
        else hipLaunchKernelGGL((k_qkv_bf16<1, 4, 2, false, N, 1, SRCV>), g, dim3(256), 0, s, a, kv_only, mode, n_mt, S);               \
    } while (0)
#define L_QKV(N)                                         \
    do {                                                 \
        if (src == SRC_RESID) L_QKVS(N, SRC_RESID);      \
        else L_QKVS(N, SRC_EMBED);                       \
    } while (0)
    // e4m3 weights: the rolled-loop instantiations only (any stage count)
#define L_QKVS8(SRCV)                                                                                                   \
    do {                                                                                                                \
        if (TM == 2 && part) hipLaunchKernelGGL((k_qkv_bf16<2, 4, 2, true, 0, 1, SRCV, true>), g, dim3(256), 0, s, a, kv_only, mode, n_mt, S);  \
        else if (TM == 2) hipLaunchKernelGGL((k_qkv_bf16<2, 4, 2, false, 0, 1, SRCV, true>), g, dim3(256), 0, s, a, kv_only, mode, n_mt, S);  \
        else if (part) hipLaunchKernelGGL((k_qkv_bf16<1, 4, 2, true, 0, 1, SRCV, true>), g, dim3(256), 0, s, a, kv_only, mode, n_mt, S);      \
        else hipLaunchKernelGGL((k_qkv_bf16<1, 4, 2, false, 0, 1, SRCV, true>), g, dim3(256), 0, s, a, kv_only, mode, n_mt, S);               \
    } while (0)
    if (a.proj_fp8) {
        if (nst % 4) return hipErrorInvalidValue;
        if (src == SRC_RESID) L_QKVS8(SRC_RESID);
        else L_QKVS8(SRC_EMBED);
    } else {
        DG_NST_DISPATCH(nst, L_QKV)
    }
#undef L_QKV
#undef L_QKVS
#undef L_QKVS8
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !part) return e;
    hipLaunchKernelGGL(k_qkv_finish, dim3(a.M, n_heads), dim3(64), 0, s, a, kv_only, mode, S);
    return hipGetLastError();
}

// Split-K projection to d outputs (the attention output projection, or the
// FFN's down projection) and the residual finish.
static hipError_t launch_to_resid(const StepArgs &a, const uint16_t *W, const float *wsc, int K,
                                  const uint16_t *act, float *hdump, hipStream_t s, int src, int out,
                                  int moe_add, int want_xr) {
    const ProjShape p = oproj_shape(a.M, a.d, K);     // two activation planes: one row tile per wave
    // the launches below take 64-row workgroups with two K parts, or
    // 128-row workgroups with one
    if (!((p.wpg == 2 && p.kh == 2) || (p.wpg == 4 && p.kh == 1)) || K % (64 * p.S * p.kh)) return hipErrorInvalidValue;
    const int S = p.S;
    const int n_mt = (a.M + 32 * p.wpg - 1) / (32 * p.wpg);
    const int nst = K / 64 / S / p.kh;                 // stages per part
    // 128 output features per workgroup where 64 would give two or more
    // workgroups per CU
    const int fc = (p.wpg == 4 && a.d % 128 == 0 && S * (a.d / 64) * n_mt >= 512) ? 128 : 64;
    const int ntn = a.d / fc;
    const dim3 g(grid_pad8(S * ntn * n_mt));
#define L_OPROJ(N)                                                                                            \
    do {                                                                                                      \
        if (fc == 128) {                                                                                      \
            if (a.proj_fp8) hipLaunchKernelGGL((k_oproj_bf16<1, 4, 2, N, true, 4, 1, 128>), g, dim3(256), 0, s, a, n_mt, S, W, K, act, wsc); \
            else hipLaunchKernelGGL((k_oproj_bf16<1, 4, 2, N, false, 4, 1, 128>), g, dim3(256), 0, s, a, n_mt, S, W, K, act, wsc); \
        } else if (a.proj_fp8) hipLaunchKernelGGL((k_oproj_bf16<1, 4, 2, N, true>), g, dim3(256), 0, s, a, n_mt, S, W, K, act, wsc); \
        else hipLaunchKernelGGL((k_oproj_bf16<1, 4, 2, N>), g, dim3(256), 0, s, a, n_mt, S, W, K, act, wsc);  \
    } while (0)
#define L_OPROJ2(N)                                                                                           \
    do {                                                                                                      \
        if (a.proj_fp8) hipLaunchKernelGGL((k_oproj_bf16<1, half_ring<N>(), 2, N, true, 2, 2>), g, dim3(256), 0, s, a, n_mt, S, W, K, act, wsc); \
        else hipLaunchKernelGGL((k_oproj_bf16<1, half_ring<N>(), 2, N, false, 2, 2>), g, dim3(256), 0, s, a, n_mt, S, W, K, act, wsc); \
    } while (0)
    if (p.wpg == 2) {
        switch (nst) {
            case 4: L_OPROJ2(4); break;
            case 8: L_OPROJ2(8); break;
            case 16: L_OPROJ2(16); break;
            case 32: L_OPROJ2(32); break;
            default: L_OPROJ2(0); break;
        }
    } else {
        DG_NST_DISPATCH(nst, L_OPROJ)
    }
#undef L_OPROJ
#undef L_OPROJ2
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (src == SRC_RESID && out == OUT_RESID)
        hipLaunchKernelGGL((k_resid_finish<SRC_RESID, OUT_RESID>), dim3(a.M), dim3(256), 0, s, a, S, hdump, moe_add,
                           want_xr);
    else if (src == SRC_RESID)
        hipLaunchKernelGGL((k_resid_finish<SRC_RESID, OUT_LMHEAD>), dim3(a.M), dim3(256), 0, s, a, S, hdump, moe_add,
                           want_xr);
    else if (out == OUT_RESID)
        hipLaunchKernelGGL((k_resid_finish<SRC_EMBED, OUT_RESID>), dim3(a.M), dim3(256), 0, s, a, S, hdump, moe_add,
                           want_xr);
    else
        hipLaunchKernelGGL((k_resid_finish<SRC_EMBED, OUT_LMHEAD>), dim3(a.M), dim3(256), 0, s, a, S, hdump, moe_add,
                           want_xr);
    return hipGetLastError();
}

hipError_t launch_oproj(const StepArgs &a, float *hdump, hipStream_t s, int src, int out) {
    if (a.dtype != DG_BF16) return launch_oproj_f32(a, s);
    // the attention's residual finish feeds the FFN: with experts, also the
    // row-major planes of x they gather from
    return launch_to_resid(a, (const uint16_t *)a.wo, a.so, a.Hq * a.hd, (const uint16_t *)(a.ws + a.L.o), hdump, s,
                           src, out, 0, a.n_experts > 0 && out == OUT_RESID);
}

hipError_t launch_ffn(const StepArgs &a, float *hdump, hipStream_t s, int out) {
    if (a.dtype != DG_BF16 || a.d_ff <= 0) return hipErrorInvalidValue;
    const int n_mt = (a.M + 127) / 128;
    // 64-feature tiles where they still give a workgroup per CU
    const int fw = (a.d_ff % 64 == 0 && (a.d_ff / 64) * n_mt >= 256) ? 64 : 32;
    const dim3 g(grid_pad8((a.d_ff / fw) * n_mt));
#define L_UP(N)                                                                               \
    do {                                                                                      \
        if (fw == 64) {                                                                       \
            if (a.proj_fp8) hipLaunchKernelGGL((k_ffn_up_bf16<1, 4, 2, N, true, 64>), g, dim3(256), 0, s, a, n_mt); \
            else hipLaunchKernelGGL((k_ffn_up_bf16<1, 4, 2, N, false, 64>), g, dim3(256), 0, s, a, n_mt); \
        } else if (a.proj_fp8) hipLaunchKernelGGL((k_ffn_up_bf16<1, 4, 2, N, true>), g, dim3(256), 0, s, a, n_mt); \
        else hipLaunchKernelGGL((k_ffn_up_bf16<1, 4, 2, N>), g, dim3(256), 0, s, a, n_mt);    \
    } while (0)
    DG_NST_DISPATCH(a.d / 64, L_UP)
#undef L_UP
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_to_resid(a, (const uint16_t *)a.wd, a.sd, a.d_ff, (const uint16_t *)(a.ws + a.L.act), hdump, s,
                           SRC_RESID, out, a.n_experts > 0, 0);
}

template <int NSTC>
constexpr int lm8_ring() { return (NSTC > 0 && NSTC % 8 == 0) ? 8 : 4; }

hipError_t launch_lmhead(const StepArgs &a, float *logits, int bp, hipStream_t s, hipEvent_t ev0,
                         hipEvent_t ev1) {
    if (a.dtype != DG_BF16) {
        if (ev0) (void)hipEventRecord(ev0, s);
        const hipError_t e = launch_lmhead_f32(a, logits, s);
        if (ev1) (void)hipEventRecord(ev1, s);
        return e;
    }
    if (a.C > 256) return hipErrorInvalidValue;        // one workgroup covers a request's rows
    if (bp < 1 || bp > DG_LM_GROUP_MAX) return hipErrorInvalidValue;
    const bool samp = a.temp0 > 0.f;
    const dim3 g(grid_pad8(((a.V + 127) / 128) * ((a.B + bp - 1) / bp)));
    if (a.lm_fp8) {
        // a stage of e4m3 weights is half the bytes of a bf16 one: twice the
        // ring depth (where the stage count allows) keeps the same bytes in
        // flight, in the same registers
#define L_LM8(N)                                                                                              \
    do {                                                                                                      \
        constexpr int PW8 = lm8_ring<N>();                                                                    \
        if (samp) hipExtLaunchKernelGGL((k_lmhead_fp8<PW8, 2, N, true>), g, dim3(512), 0, s, ev0, ev1, 0, a, logits, bp); \
        else if (ev0) hipExtLaunchKernelGGL((k_lmhead_fp8<PW8, 2, N>), g, dim3(512), 0, s, ev0, ev1, 0, a, logits, bp); \
        else hipLaunchKernelGGL((k_lmhead_fp8<PW8, 2, N>), g, dim3(512), 0, s, a, logits, bp);        \
    } while (0)
        DG_NST_DISPATCH(a.d / 64, L_LM8)
#undef L_LM8
        return hipGetLastError();
    }
#define L_LM(N)                                                                                               \
    do {                                                                                                      \
        if (samp) hipExtLaunchKernelGGL((k_lmhead_bf16<4, 4, N, true>), g, dim3(512), 0, s, ev0, ev1, 0, a, logits, bp); \
        else if (ev0) hipExtLaunchKernelGGL((k_lmhead_bf16<4, 4, N>), g, dim3(512), 0, s, ev0, ev1, 0, a, logits, bp); \
        else hipLaunchKernelGGL((k_lmhead_bf16<4, 4, N>), g, dim3(512), 0, s, a, logits, bp);         \
    } while (0)
    DG_NST_DISPATCH(a.d / 64, L_LM)
#undef L_LM
    return hipGetLastError();
}

}  // namespace dg
