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

#include "dg_device.hpp"
#include "dg_internal.hpp"

namespace dg {

hipError_t launch_qkv_f32(const StepArgs &a, int kv_only, int mode, hipStream_t s);
hipError_t launch_oproj_f32(const StepArgs &a, hipStream_t s);
hipError_t launch_lmhead_f32(const StepArgs &a, float *logits, hipStream_t s);

// Calls f(integral_constant<int, U>) for U = 0 .. PF-1, so that register
// queues can be indexed with compile-time constants (no scratch).
template <int U, int PF>
struct Unroll {
    template <class F>
    __device__ __forceinline__ static void run(F &&f) {
        f(std::integral_constant<int, U>{});
        Unroll<U + 1, PF>::run(f);
    }
};
template <int PF>
struct Unroll<PF, PF> {
    template <class F>
    __device__ __forceinline__ static void run(F &&) {}
};

// Within one 64-wide K stage, MFMA step ks (0..3) gives lane half h the k
// values 32h + 8ks + (0..7): each lane reads the 32 contiguous token-row
// values 32h .. 32h+31 of the stage, and 16-byte chunk 4h + ks of each LDS
// weight row.
// Every row pointer is valid: rows past the end of a matrix are clamped to
// its last row by the caller and their results are discarded in the
// epilogue, so the loads need no predication.
// SPLIT: the token rows are fp32; each value x is fed as two bf16 MFMA
// operands hi = bf16(x) and lo = bf16(x - hi) (about 16 significant bits).
template <bool SPLIT>
struct ActTraits {
    static constexpr int Q = SPLIT ? 8 : 4;   // 16-byte loads per lane per stage
    __device__ static const u32x4 *at(const void *p, int k) {
        return SPLIT ? (const u32x4 *)((const float *)p + k) : (const u32x4 *)((const uint16_t *)p + k);
    }
};

__device__ __forceinline__ void split_bf16(const u32x4 &x0, const u32x4 &x1, u32x4 &hi, u32x4 &lo) {
    float f[8] = {__uint_as_float(x0[0]), __uint_as_float(x0[1]), __uint_as_float(x0[2]), __uint_as_float(x0[3]),
                  __uint_as_float(x1[0]), __uint_as_float(x1[1]), __uint_as_float(x1[2]), __uint_as_float(x1[3])};
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const __bf16 a0 = (__bf16)f[2 * i], a1 = (__bf16)f[2 * i + 1];
        const __bf16 b0 = (__bf16)(f[2 * i] - (float)a0), b1 = (__bf16)(f[2 * i + 1] - (float)a1);
        h[i] = (uint32_t)__builtin_bit_cast(uint16_t, a0) | ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
        l[i] = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
    }
    hi = u32x4{h[0], h[1], h[2], h[3]};
    lo = u32x4{l[0], l[1], l[2], l[3]};
}

template <int NT, int TM, int PF, bool SPLIT = false>
__device__ __forceinline__ void gemm_core(const uint16_t *const (&wp)[NT], const void *const (&ap)[TM],
                                          int K, u32x4 *lds /* [2][NT*256] */, f32x16 (&acc)[NT][TM]) {
    using AT = ActTraits<SPLIT>;
    constexpr int AQ = AT::Q;
    constexpr int AS = SPLIT ? 4 : 8;         // elements per 16-byte load
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int row32 = lane & 31;
    const int ck = tid & 7;
    const int nst = K >> 6;

    u32x4 wreg[PF][NT];
    u32x4 areg[PF][TM][AQ];

#pragma unroll
    for (int o = 0; o < NT; ++o)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) acc[o][tm] = zero16();

    Unroll<0, PF>::run([&](auto U) __attribute__((always_inline)) {
        constexpr int u = decltype(U)::value;
        if (u < nst) {
            const int k0 = u * 64;
#pragma unroll
            for (int x = 0; x < NT; ++x) wreg[u][x] = *(const u32x4 *)(wp[x] + k0);
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int q = 0; q < AQ; ++q) areg[u][tm][q] = *AT::at(ap[tm], k0 + AS * q);
        }
    });

    for (int base = 0; base < nst; base += PF) {
        Unroll<0, PF>::run([&](auto U) __attribute__((always_inline)) {
            constexpr int u = decltype(U)::value;
            const int st = base + u;
            if (st < nst) {
                u32x4 *buf = lds + (st & 1) * (NT * 256);
#pragma unroll
                for (int x = 0; x < NT; ++x) {
                    const int r = (tid >> 3) + 32 * x;
                    buf[r * 8 + (ck ^ (r & 7))] = wreg[u][x];
                }
                const bool more = st + PF < nst;
                const int k1 = (st + PF) * 64;
                if (more) {
#pragma unroll
                    for (int x = 0; x < NT; ++x) wreg[u][x] = *(const u32x4 *)(wp[x] + k1);
                }
                __syncthreads();
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    u32x4 af[NT];
#pragma unroll
                    for (int o = 0; o < NT; ++o) {
                        const int r = o * 32 + row32;
                        const int c = 4 * half + ks;
                        af[o] = buf[r * 8 + (c ^ (r & 7))];
                    }
                    if constexpr (SPLIT) {
#pragma unroll
                        for (int tm = 0; tm < TM; ++tm) {
                            u32x4 hi, lo;
                            split_bf16(areg[u][tm][2 * ks], areg[u][tm][2 * ks + 1], hi, lo);
#pragma unroll
                            for (int o = 0; o < NT; ++o) {
                                acc[o][tm] = mfma32(af[o], hi, acc[o][tm]);
                                acc[o][tm] = mfma32(af[o], lo, acc[o][tm]);
                            }
                        }
                    } else {
#pragma unroll
                        for (int o = 0; o < NT; ++o)
#pragma unroll
                            for (int tm = 0; tm < TM; ++tm) acc[o][tm] = mfma32(af[o], areg[u][tm][ks], acc[o][tm]);
                    }
                }
                if (more) {
#pragma unroll
                    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                        for (int q = 0; q < AQ; ++q) areg[u][tm][q] = *AT::at(ap[tm], k1 + AS * q);
                }
            }
        });
    }
}

// Tile index of this workgroup: workgroups j and j+1 (same weight tile when
// n_mt > 1) land on the same XCD.  Returns false for padding workgroups.
__device__ __forceinline__ bool xcd_tile(int total, int n_mt, int &nt, int &mt) {
    const int G = gridDim.x;               // multiple of 8
    const int i = blockIdx.x;
    const int j = (i & 7) * (G >> 3) + (i >> 3);
    if (j >= total) return false;
    nt = j / n_mt;
    mt = j - nt * n_mt;
    return true;
}

static inline int grid_pad8(int total) { return (total + 7) & ~7; }

// True when every request whose rows fall in [t0, t1) is done.
__device__ __forceinline__ bool all_done(const StepArgs &a, int t0, int t1) {
    t1 = min(t1, a.M);
    if (t0 >= t1) return true;
    for (int b = t0 / a.C; b <= (t1 - 1) / a.C; ++b)
        if (!a.done[b]) return false;
    return true;
}

// ---------------------------------------------------------------------------
// QKV projection + RoPE + scatter.  Tile nt = (head hh, pair block u) covers
// features j in [32u, 32u+32) (MFMA tile 0) and j + hd/2 (tile 1) of head hh.
// ---------------------------------------------------------------------------
template <int TM, int PF>
__global__ __launch_bounds__(256) void k_qkv_bf16(StepArgs a, int kv_only, int mode, int n_mt) {
    __shared__ u32x4 lds[2 * 2 * 256];
    const int pph = a.hd / 64;
    const int n_heads = kv_only ? 2 * a.Hkv : a.Hq + 2 * a.Hkv;
    int nt, mt;
    if (!xcd_tile(n_heads * pph * n_mt / 1, n_mt, nt, mt)) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, row32 = lane & 31;
    const int tok_wg = mt * 128 * TM;
    if (mode == WRITE_STEP && all_done(a, tok_wg, tok_wg + 128 * TM)) return;
    const int hh = nt / pph + (kv_only ? a.Hq : 0);
    const int u = nt % pph;
    const uint16_t *W;
    int base;
    if (hh < a.Hq) { W = (const uint16_t *)a.wq; base = hh * a.hd; }
    else if (hh < a.Hq + a.Hkv) { W = (const uint16_t *)a.wk; base = (hh - a.Hq) * a.hd; }
    else { W = (const uint16_t *)a.wv; base = (hh - a.Hq - a.Hkv) * a.hd; }

    const uint16_t *wp[2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
        wp[x] = W + (size_t)(base + 32 * u + x * (a.hd / 2) + (tid >> 3)) * a.d + (tid & 7) * 8;
    const int32_t *inp = (const int32_t *)(a.ws + a.L.inp);
    const void *ap[TM];
    const int tok0 = tok_wg + wave * 32 * TM;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int t = tok0 + tm * 32 + row32;
        ap[tm] = (const uint16_t *)a.embed + (size_t)inp[min(t, a.M - 1)] * a.d + 32 * half;
    }
    f32x16 acc[2][TM];
    gemm_core<2, TM, PF>(wp, ap, a.d, lds, acc);

    const float *r_e = (const float *)(a.ws + a.L.r_e);
    const float2 *rope = (const float2 *)(a.ws + a.L.rope);
    const bool rot = hh < a.Hq + a.Hkv;
    const int hd2 = a.hd / 2;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int t = tok0 + tm * 32 + row32;
        if (t >= a.M) continue;
        const int b = t / a.C;
        const int ic = t - b * a.C;
        const bool dn = (mode == WRITE_ALWAYS) ? true : (a.done[b] != 0);
        if (mode == WRITE_STEP && dn) continue;
        if (mode == WRITE_APPEND && !dn) continue;
        const float re = r_e[t];
        const int64_t pos = a.reqs.len[b] + ic;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int jj0 = 32 * u + 8 * rg + 4 * half;
            float y0[4], y1[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                y0[e] = re * acc[0][tm][4 * rg + e];
                y1[e] = re * acc[1][tm][4 * rg + e];
            }
            if (rot) {
                const float4 *rp = (const float4 *)(rope + (size_t)t * hd2 + jj0);
                const float4 cs01 = rp[0], cs23 = rp[1];
                const float c[4] = {cs01.x, cs01.z, cs23.x, cs23.z};
                const float s[4] = {cs01.y, cs01.w, cs23.y, cs23.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x1 = y0[e], x2 = y1[e];
                    y0[e] = x1 * c[e] - x2 * s[e];
                    y1[e] = x1 * s[e] + x2 * c[e];
                }
            }
            const uint2 lo = make_uint2(pack_bf2(y0[0], y0[1]), pack_bf2(y0[2], y0[3]));
            const uint2 hi = make_uint2(pack_bf2(y1[0], y1[1]), pack_bf2(y1[2], y1[3]));
            if (hh < a.Hq) {
                uint16_t *q = (uint16_t *)(a.ws + a.L.q) + ((size_t)t * a.Hq + hh) * a.hd;
                *(uint2 *)(q + jj0) = lo;
                *(uint2 *)(q + jj0 + hd2) = hi;
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
    }
}

// ---------------------------------------------------------------------------
// Output projection + residual: h = E[tok] + o Wo^T, tile of 64 features.
// o is the fp32 attention output, fed through the hi/lo bf16 split.
// ---------------------------------------------------------------------------
template <int TM, int PF>
__global__ __launch_bounds__(256) void k_oproj_bf16(StepArgs a, int n_mt) {
    __shared__ u32x4 lds[2 * 2 * 256];
    int nt, mt;
    if (!xcd_tile((a.d / 64) * n_mt, n_mt, nt, mt)) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, row32 = lane & 31;
    const int tok_wg = mt * 128 * TM;
    if (all_done(a, tok_wg, tok_wg + 128 * TM)) return;
    const int K = a.Hq * a.hd;
    const uint16_t *wp[2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
        wp[x] = (const uint16_t *)a.wo + (size_t)(64 * nt + 32 * x + (tid >> 3)) * K + (tid & 7) * 8;
    const void *ap[TM];
    const int tok0 = tok_wg + wave * 32 * TM;
    const float *o = (const float *)(a.ws + a.L.o);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int t = tok0 + tm * 32 + row32;
        ap[tm] = o + (size_t)min(t, a.M - 1) * K + 32 * half;
    }
    f32x16 acc[2][TM];
    gemm_core<2, TM, PF, true>(wp, ap, K, lds, acc);

    const int32_t *inp = (const int32_t *)(a.ws + a.L.inp);
    uint16_t *h = (uint16_t *)(a.ws + a.L.h);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int t = tok0 + tm * 32 + row32;
        if (t >= a.M) continue;
        const uint16_t *erow = (const uint16_t *)a.embed + (size_t)inp[t] * a.d;
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int n = 64 * nt + 32 * x + 8 * rg + 4 * half;
                const uint2 ev = *(const uint2 *)(erow + n);
                const float e0 = __uint_as_float(ev.x << 16), e1 = __uint_as_float(ev.x & 0xffff0000u);
                const float e2 = __uint_as_float(ev.y << 16), e3 = __uint_as_float(ev.y & 0xffff0000u);
                const uint2 hv = make_uint2(pack_bf2(e0 + acc[x][tm][4 * rg + 0], e1 + acc[x][tm][4 * rg + 1]),
                                            pack_bf2(e2 + acc[x][tm][4 * rg + 2], e3 + acc[x][tm][4 * rg + 3]));
                *(uint2 *)(h + (size_t)t * a.d + n) = hv;
            }
    }
}

// ---------------------------------------------------------------------------
// Vocabulary head + fused sampler statistics.  Tile: 128 ids (slice nt) x
// 256 tokens.  z = r_h[t] * (h_t . Wlm[v]); the MASK id and ids >= V are
// excluded.  Writes one (m, sum exp, m2, argmax) record per (slice, token).
// ---------------------------------------------------------------------------
template <int PF>
__global__ __launch_bounds__(256) void k_lmhead_bf16(StepArgs a, float *logits, int n_mt) {
    constexpr int NT = 4, TM = 2;
    __shared__ u32x4 lds[2 * NT * 256];
    const int n_nt = (a.V + 127) / 128;
    int nt, mt;
    if (!xcd_tile(n_nt * n_mt, n_mt, nt, mt)) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, row32 = lane & 31;
    const int tok_wg = mt * 256;
    if (all_done(a, tok_wg, tok_wg + 256)) return;
    const uint16_t *wp[NT];
#pragma unroll
    for (int x = 0; x < NT; ++x) {
        const int v = 128 * nt + 32 * x + (tid >> 3);
        wp[x] = (const uint16_t *)a.lm + (size_t)min(v, a.V - 1) * a.d + (tid & 7) * 8;
    }
    const uint16_t *hbuf = (const uint16_t *)(a.ws + a.L.h);
    const void *ap[TM];
    const int tok0 = tok_wg + wave * 64;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int t = tok0 + tm * 32 + row32;
        ap[tm] = hbuf + (size_t)min(t, a.M - 1) * a.d + 32 * half;
    }
    f32x16 acc[NT][TM];
    gemm_core<NT, TM, PF>(wp, ap, a.d, lds, acc);

    const float *r_h = (const float *)(a.ws + a.L.r_h);
    float4 *part = (float4 *)(a.ws + a.L.lm_part);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int t = tok0 + tm * 32 + row32;
        const bool tv = t < a.M;
        const float rs = tv ? r_h[t] : 0.f;
        VStat st{-INFINITY, 0.f, -INFINITY, INT_MAX};
        // ids visited in increasing order within the lane: ties keep the lower id
#pragma unroll
        for (int o = 0; o < NT; ++o)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int v = 128 * nt + 32 * o + 8 * (r >> 2) + 4 * half + (r & 3);
                const float zz = (v < a.V && v != a.mask_id) ? rs * acc[o][tm][r] : -INFINITY;
                acc[o][tm][r] = zz;
                if (zz > st.m) { st.m2 = st.m; st.m = zz; st.a = v; }
                else if (zz > st.m2) { st.m2 = zz; }
            }
        float s = 0.f;
        if (st.m != -INFINITY) {
#pragma unroll
            for (int o = 0; o < NT; ++o)
#pragma unroll
                for (int r = 0; r < 16; ++r) s += __expf(acc[o][tm][r] - st.m);
        }
        st.s = s;
        st = vmerge(st, vshfl_xor(st, 32));
        if (tv && half == 0) part[(size_t)nt * a.M + t] = make_float4(st.m, st.s, st.m2, __int_as_float(st.a));
        if (logits && tv) {
#pragma unroll
            for (int o = 0; o < NT; ++o)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int v = 128 * nt + 32 * o + 8 * (r >> 2) + 4 * half + (r & 3);
                    if (v < a.V) logits[(size_t)t * a.V + v] = acc[o][tm][r];
                }
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_qkv(const StepArgs &a, int kv_only, int mode, hipStream_t s) {
    if (a.dtype != DG_BF16) return launch_qkv_f32(a, kv_only, mode, s);
    const int n_heads = kv_only ? 2 * a.Hkv : a.Hq + 2 * a.Hkv;
    const int ntn = n_heads * (a.hd / 64);
    // 128 tokens per workgroup unless the grid is already large
    if (ntn * ((a.M + 127) / 128) >= 1024) {
        const int n_mt = (a.M + 255) / 256;
        hipLaunchKernelGGL((k_qkv_bf16<2, 3>), dim3(grid_pad8(ntn * n_mt)), dim3(256), 0, s, a, kv_only, mode, n_mt);
    } else {
        const int n_mt = (a.M + 127) / 128;
        hipLaunchKernelGGL((k_qkv_bf16<1, 6>), dim3(grid_pad8(ntn * n_mt)), dim3(256), 0, s, a, kv_only, mode, n_mt);
    }
    return hipGetLastError();
}

hipError_t launch_oproj(const StepArgs &a, hipStream_t s) {
    if (a.dtype != DG_BF16) return launch_oproj_f32(a, s);
    const int ntn = a.d / 64;
    if (ntn * ((a.M + 127) / 128) >= 1024) {
        const int n_mt = (a.M + 255) / 256;
        hipLaunchKernelGGL((k_oproj_bf16<2, 2>), dim3(grid_pad8(ntn * n_mt)), dim3(256), 0, s, a, n_mt);
    } else {
        const int n_mt = (a.M + 127) / 128;
        hipLaunchKernelGGL((k_oproj_bf16<1, 3>), dim3(grid_pad8(ntn * n_mt)), dim3(256), 0, s, a, n_mt);
    }
    return hipGetLastError();
}

hipError_t launch_lmhead(const StepArgs &a, float *logits, hipStream_t s) {
    if (a.dtype != DG_BF16) return launch_lmhead_f32(a, logits, s);
    const int n_mt = (a.M + 255) / 256;
    const int total = ((a.V + 127) / 128) * n_mt;
    hipLaunchKernelGGL((k_lmhead_bf16<2>), dim3(grid_pad8(total)), dim3(256), 0, s, a, logits, n_mt);
    return hipGetLastError();
}

}  // namespace dg
