// The MFMA GEMM core shared by the projection, vocabulary-head and expert
// kernels, and the workgroup-to-tile helpers they use.
#pragma once

#include <type_traits>

#include "dg_device.hpp"
#include "dg_internal.hpp"

namespace dg {

// Within one 64-wide K stage, MFMA step ks (0..3) covers k = 16ks .. 16ks+15:
// lane half h holds k = 16ks + 8h + (0..7), i.e. 16-byte chunk 2ks + h of
// each LDS weight row.  The token operand of lane (row32, half) is features
// 16ks + 8h .. + 7 of its row: ACH = 512 reads it from a fragment-major
// activation (frag_index; 1 KB contiguous per wave), ACH = 16 from a
// row-major row (the QKV projection's gathered embedding rows).
// Every row / tile pointer is valid: tiles past the end of a matrix are
// clamped to its last one by the caller and their results are discarded in
// the epilogue, so the loads need no predication.
// NPL: number of activation planes summed into the same product (the fp32
// attention output enters as an fp16 hi plane plus an fp16 lo plane); plane
// p of the token operand sits plane_elems elements after plane 0.
// F16: the weights are converted from bf16 to fp16 while they are staged in
// LDS and the activations are fp16; the MFMAs take fp16 operands.
// W8: the weights are e4m3 bytes; per stage thread tid loads the 8 bytes of
// chunk tid & 7 (k = 8 (tid & 7) .. + 7) of each of its NL rows (NL even:
// one ring register holds rows 2x and 2x + 1) and stages them as fp16 (F16)
// or bf16 chunks in the same LDS places as the 16-bit chunks, so the tile
// and its conflict-free pattern are the same.  The row pointers then address
// bytes.
#ifndef DG_NO_SCHED_FENCE
#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)
#else
#define SCHED_FENCE() ((void)0)
#endif

// Calls f(integral_constant<int, U>) for U = 0 .. N-1, so that register
// queues are indexed with compile-time constants (a ring needs no moves).
template <int U, int N>
struct Unroll {
    template <class F>
    __device__ __forceinline__ static void run(F &&f) {
        f(std::integral_constant<int, U>{});
        Unroll<U + 1, N>::run(f);
    }
};
template <int N>
struct Unroll<N, N> {
    template <class F>
    __device__ __forceinline__ static void run(F &&) {}
};

// Register rings: PW stages of weight chunks and PA stages of token-row
// chunks in flight (PA divides PW; the number of stages K/64 must be a
// multiple of PW, which the launchers guarantee).  The weight ring is the
// deep one: it covers HBM latency; token rows come from L2.  Every stage
// issues the same loads (addresses past the last stage are clamped to it and
// the surplus data is never used), so the loop has a single shape and the
// hardware wait counts stay exact.
//
// NSTC > 0 fixes the number of stages at compile time and unrolls the whole
// K loop: a rolled loop makes the compiler wait for every outstanding load at
// the loop back-edge (the ring's loads cross it), which drains the prefetch
// queue once per PW stages.
// ap[tm]: address of the first fragment block (k = 0 of the chunk) of the
// lane's token tile, plus the lane offset; consecutive k blocks are 512
// elements apart.
// LDS position of 16-byte chunk c of weight-tile row r (8 chunks per row):
// the XOR spreads the 16 rows read by a quarter-wave over all 64 banks.
__device__ __forceinline__ int wlds(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// The workgroup (NTHREADS threads) stages a weight tile of NL*NTHREADS/8 rows
// per stage (thread tid loads 16-byte chunk tid & 7 of rows tid/8 +
// x*NTHREADS/8, through wp[x]); each wave multiplies NT 32-row tiles starting
// at LDS row wrow0 with its TM token tiles.
//
// Schedule of stage st (one barrier per stage), PREFETCH = true:
//   MFMAs k-steps 0,1 of st  |  LDS reads of st's k-steps 2,3 fragments
//   write stage st+1 into the other LDS buffer, barrier
//   MFMAs k-steps 2,3 of st  |  LDS reads of st+1's k-steps 0,1 fragments
// so the fragment reads of one half-stage overlap the MFMAs of the other,
// with one stage's worth of fragment registers.
// PREFETCH = false: barrier at the start of the stage, then all of the
// stage's fragments, then its MFMAs.
// active = false (uniform per wave): the wave only helps stage the weight
// tiles and issues no MFMAs (acc stays zero).  It still issues its
// activation loads (from the clamped, valid addresses every caller passes):
// with the loads under a branch the compiler's wait counts would have to
// hold on both paths, and the path without them would cap every wait at the
// few weight loads issued since, draining the activation prefetch each
// stage.
template <int NT, int TM, int PW, int PA, int NPL = 1, int NSTC = 0, int NL = NT, int NTHREADS = 256,
          bool PREFETCH = true, bool F16 = false, int ACH = 512, bool W8 = false>
__device__ __forceinline__ void gemm_core(const uint16_t *const (&wp)[NL], int wrow0, const void *const (&ap)[TM],
                                          int K, u32x4 *lds /* [2][NL*NTHREADS] */, f32x16 (&acc)[NT][TM],
                                          bool active = true, size_t plane_elems = 0) {
    static_assert(!W8 || NL % 2 == 0, "e4m3 weights: 8-byte chunks of row pairs");
    constexpr int STAGE_CHUNKS = NL * NTHREADS;      // 16-byte LDS chunks per stage
    constexpr int NLR = W8 ? NL / 2 : NL;            // ring registers per stage
    // ring register x of the stage starting at k0 (bf16: 16 bytes of row x;
    // e4m3: 8 bytes of each of rows 2x and 2x + 1)
    auto wld = [&](int x, int k0) __attribute__((always_inline)) -> u32x4 {
        if constexpr (W8) {
            const u32x2 r0 = *(const u32x2 *)((const uint8_t *)wp[2 * x] + k0);
            const u32x2 r1 = *(const u32x2 *)((const uint8_t *)wp[2 * x + 1] + k0);
            return u32x4{r0[0], r0[1], r1[0], r1[1]};
        } else {
            return *(const u32x4 *)(wp[x] + k0);
        }
    };
    static_assert(PW % PA == 0 && PW % 2 == 0, "PA must divide PW, PW even");
    static_assert(NSTC % PW == 0, "NSTC must be a multiple of PW");
    constexpr int AQ = 4 * NPL;               // 16-byte loads per lane per stage
    auto act = [&](int tm, int st, int q) __attribute__((always_inline)) -> const u32x4 * {
        return (const u32x4 *)((const uint16_t *)ap[tm] + (size_t)(q >> 2) * plane_elems +
                               (size_t)(4 * st + (q & 3)) * ACH);
    };
    const int tid = threadIdx.x % NTHREADS;          // index within the staging group
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int row32 = lane & 31;
    const int ck = tid & 7;
    const int nst = NSTC > 0 ? NSTC : (K >> 6);
    const int klast = (nst - 1) * 64;

    u32x4 wq[PW][NLR];        // wq[i] holds the weight chunks of stage (st + i) % PW ring slot
    u32x4 aq[PA][TM][AQ];
    u32x4 af[1][4][NT];       // weight fragments: k-steps 0..3 of a stage

#pragma unroll
    for (int o = 0; o < NT; ++o)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) acc[o][tm] = zero16();

    // prologue: stages 0 .. PW-1 of weights, 0 .. PA-1 of activations
    Unroll<0, PW>::run([&](auto U) __attribute__((always_inline)) {
        constexpr int u = decltype(U)::value;
        const int k0 = min(u * 64, klast);
#pragma unroll
        for (int x = 0; x < NLR; ++x) wq[u][x] = wld(x, k0);
        if constexpr (u < PA) {
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int q = 0; q < AQ; ++q) {
                    aq[u][tm][q] = *act(tm, u, q);
                }
        }
    });
    auto stage_to_lds = [&](u32x4 *buf, const u32x4 (&w)[NLR]) __attribute__((always_inline)) {
        if constexpr (W8) {
#pragma unroll
            for (int x = 0; x < NLR; ++x) {
                const int r0 = (tid >> 3) + (NTHREADS / 8) * (2 * x), r1 = r0 + NTHREADS / 8;
                if constexpr (F16) {
                    buf[wlds(r0, ck)] = fp8x8_to_h8(w[x][0], w[x][1]);
                    buf[wlds(r1, ck)] = fp8x8_to_h8(w[x][2], w[x][3]);
                } else {
                    buf[wlds(r0, ck)] = fp8x8_to_bf8(w[x][0], w[x][1]);
                    buf[wlds(r1, ck)] = fp8x8_to_bf8(w[x][2], w[x][3]);
                }
            }
            return;
        }
#pragma unroll
        for (int x = 0; x < NL; ++x) {
            if constexpr (F16) buf[wlds((tid >> 3) + (NTHREADS / 8) * x, ck)] = bf8_to_h8(w[x]);
            else buf[wlds((tid >> 3) + (NTHREADS / 8) * x, ck)] = w[x];
        }
    };
    auto read_frags = [&](const u32x4 *buf, u32x4 (&f)[4][NT]) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int o = 0; o < NT; ++o) f[ks][o] = buf[wlds(wrow0 + o * 32 + row32, 2 * ks + half)];
    };
    auto read_half = [&](const u32x4 *buf, u32x4 (&f)[4][NT], int ks0) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = ks0; ks < ks0 + 2; ++ks)
#pragma unroll
            for (int o = 0; o < NT; ++o) f[ks][o] = buf[wlds(wrow0 + o * 32 + row32, 2 * ks + half)];
    };
    auto mfma_ks = [&](const u32x4 (&f)[4][NT], const u32x4 (&x)[TM][AQ], int ks) __attribute__((always_inline)) {
        if (!active) return;
#pragma unroll
        for (int p = 0; p < NPL; ++p)
#pragma unroll
            for (int o = 0; o < NT; ++o)
#pragma unroll
                for (int tm = 0; tm < TM; ++tm) {
                    if constexpr (F16) acc[o][tm] = mfma32_f16(f[ks][o], x[tm][4 * p + ks], acc[o][tm]);
                    else acc[o][tm] = mfma32(f[ks][o], x[tm][4 * p + ks], acc[o][tm]);
                }
    };

    if constexpr (!PREFETCH) {
#pragma unroll(NSTC > 0 ? NSTC / PW : 1)
        for (int base = 0; base < nst; base += PW) {
            Unroll<0, PW>::run([&](auto U) __attribute__((always_inline)) {
                constexpr int u = decltype(U)::value;
                constexpr int ua = u % PA;
                const int st = base + u;
                u32x4 *buf = lds + (u & 1) * STAGE_CHUNKS;
                stage_to_lds(buf, wq[u]);
                {
                    const int k1 = min((st + PW) * 64, klast);
#pragma unroll
                    for (int x = 0; x < NLR; ++x) wq[u][x] = wld(x, k1);
                }
                __syncthreads();
                read_frags(buf, af[0]);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) mfma_ks(af[0], aq[ua], ks);
                {
                    const int k1s = min(st + PA, nst - 1);
#pragma unroll
                    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                        for (int q = 0; q < AQ; ++q) {
                            aq[ua][tm][q] = *act(tm, k1s, q);
                        }
                }
            });
        }
        return;
    } else {
    // prologue: stage 0 into buffer 0 and the fragments of its k-steps 0, 1
    stage_to_lds(lds, wq[0]);
    {
        const int k1 = min(PW * 64, klast);
#pragma unroll
        for (int x = 0; x < NLR; ++x) wq[0][x] = wld(x, k1);
    }
    __syncthreads();
    read_half(lds, af[0], 0);

#pragma unroll(NSTC > 0 ? NSTC / PW : 1)
    for (int base = 0; base < nst; base += PW) {
        Unroll<0, PW>::run([&](auto U) __attribute__((always_inline)) {
            constexpr int u = decltype(U)::value;
            constexpr int ua = u % PA;
            constexpr int un = (u + 1) % PW;          // ring slot of stage st + 1
            const int st = base + u;
            u32x4 *cbuf = lds + (u & 1) * STAGE_CHUNKS;        // PW even: u & 1 == st & 1
            u32x4 *nbuf = lds + ((u & 1) ^ 1) * STAGE_CHUNKS;
            // sched_barrier(0) keeps each group where it is written: left to
            // itself the scheduler sinks the fragment reads and the ring
            // refills next to their uses, which serializes LDS and global
            // latency with the MFMAs
            SCHED_FENCE();
            mfma_ks(af[0], aq[ua], 0);
            mfma_ks(af[0], aq[ua], 1);
            read_half(cbuf, af[0], 2);                // k-steps 2, 3 of stage st
            SCHED_FENCE();
            // stage st + 1 into the other buffer
            stage_to_lds(nbuf, wq[un]);
            SCHED_FENCE();
            __syncthreads();
            mfma_ks(af[0], aq[ua], 2);
            mfma_ks(af[0], aq[ua], 3);
            read_half(nbuf, af[0], 0);                // k-steps 0, 1 of stage st + 1
            SCHED_FENCE();
            // activations of stage st + PA, then the ring slot of stage
            // st + 1 + PW: loads complete in issue order, so waiting for an
            // activation never waits for weights issued after it
            {
                const int k1s = min(st + PA, nst - 1);
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                    for (int q = 0; q < AQ; ++q) {
                        aq[ua][tm][q] = *act(tm, k1s, q);
                    }
            }
            {
                const int k1 = min((st + 1 + PW) * 64, klast);
#pragma unroll
                for (int x = 0; x < NLR; ++x) wq[un][x] = wld(x, k1);
            }
        });
    }
    }
}

// In-workgroup K split: KH groups of NTH threads each hold the partial
// accumulators acc[2][1] of their part of the K axis; afterwards group 0
// holds the sum in a fixed order ((g0 + g2) + (g1 + g3) for four parts, g0 +
// g1 for two).  The exchange goes through lds_base (the staging buffers,
// free once every wave is past its last fragment read; at least
// 8 KH / 2 NTH 16-byte slots); every thread of the workgroup calls it.
template <int KH, int NTH>
__device__ __forceinline__ void kparts_reduce(f32x16 (&acc)[2][1], void *lds_base, int kh, int tid) {
    if constexpr (KH > 1) {
        __syncthreads();
        auto fold = [&](int n) __attribute__((always_inline)) {   // groups n .. 2n-1 into 0 .. n-1
            float4 *red = (float4 *)lds_base + (size_t)((kh & (n - 1)) * 8) * NTH;   // [n][8][NTH] float4
            if (kh >= n && kh < 2 * n) {
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int r = 0; r < 16; r += 4)
                        red[(x * 4 + r / 4) * NTH + tid] =
                            make_float4(acc[x][0][r], acc[x][0][r + 1], acc[x][0][r + 2], acc[x][0][r + 3]);
            }
            __syncthreads();
            if (kh < n) {
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int r = 0; r < 16; r += 4) {
                        const float4 v = red[(x * 4 + r / 4) * NTH + tid];
                        acc[x][0][r] += v.x;
                        acc[x][0][r + 1] += v.y;
                        acc[x][0][r + 2] += v.z;
                        acc[x][0][r + 3] += v.w;
                    }
            }
        };
        if constexpr (KH == 4) {
            fold(2);
            __syncthreads();                            // group 1's reads of its slot are done
        }
        fold(1);
    }
}

// The same sum, scattered: group g ends with the KH parts of the R = 4 / KH
// register groups it owns, rg = g R .. g R + R - 1 (registers 4 rg .. 4 rg + 3
// of both tiles), added in the fixed order of kparts_reduce; y[x][r] is
// register group g R + r of tile x.  Each group writes the other groups'
// register groups to LDS (KH (KH - 1) 2 R NTH 16-byte slots) and reads its
// own from the other KH - 1 groups.  Every thread of the workgroup calls it.
template <int KH, int NTH>
__device__ __forceinline__ void kparts_scatter(const f32x16 (&acc)[2][1], void *lds_base, int kh, int tid,
                                               float4 (&y)[2][4 / KH]) {
    static_assert(KH == 2 || KH == 4, "two or four K parts");
    constexpr int R = 4 / KH;
    float4 *red = (float4 *)lds_base;                  // [destination][source != destination][2 R][NTH]
    auto slot = [&](int dst, int src) __attribute__((always_inline)) {
        return ((size_t)(dst * (KH - 1) + (src < dst ? src : src - 1)) * 2 * R) * NTH;
    };
    auto regs = [&](int x, int rg) __attribute__((always_inline)) {
        return make_float4(acc[x][0][4 * rg], acc[x][0][4 * rg + 1], acc[x][0][4 * rg + 2], acc[x][0][4 * rg + 3]);
    };
    __syncthreads();                                   // every wave is past its last fragment read
#pragma unroll
    for (int o = 0; o < KH; ++o) {
        if (o == kh) continue;
        float4 *d = red + slot(o, kh);
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int r = 0; r < R; ++r) d[(x * R + r) * NTH + tid] = regs(x, o * R + r);
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float4 v[KH];
#pragma unroll
            for (int g = 0; g < KH; ++g) {
                if (g == kh) {
                    // this group's own part: a select over the candidates, so
                    // that no register is indexed at run time
                    float4 own = regs(x, r);
#pragma unroll
                    for (int c = 1; c < KH; ++c)
                        if (c == kh) own = regs(x, c * R + r);
                    v[g] = own;
                } else {
                    v[g] = red[slot(kh, g) + (x * R + r) * NTH + tid];
                }
            }
            float4 s;
            if constexpr (KH == 4) {
                s.x = (v[0].x + v[2].x) + (v[1].x + v[3].x);
                s.y = (v[0].y + v[2].y) + (v[1].y + v[3].y);
                s.z = (v[0].z + v[2].z) + (v[1].z + v[3].z);
                s.w = (v[0].w + v[2].w) + (v[1].w + v[3].w);
            } else {
                s = make_float4(v[0].x + v[1].x, v[0].y + v[1].y, v[0].z + v[1].z, v[0].w + v[1].w);
            }
            y[x][r] = s;
        }
}

// Tile index of this workgroup: workgroups j and j+1 land on the same XCD
// (blockIdx % 8 picks the XCD), so neighbours in j share L2.  Returns false
// for padding workgroups.
__device__ __forceinline__ bool xcd_index(int total, int &j) {
    const int G = gridDim.x;               // multiple of 8
    const int i = blockIdx.x;
    j = (i & 7) * (G >> 3) + (i >> 3);
    return j < total;
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

// Request b takes part in this launch: not done (denoising step), done
// (append pass) or always (prefill).
__device__ __forceinline__ bool req_active(const StepArgs &a, int b) {
    if (a.only_req >= 0 && b != a.only_req) return false;
    return a.phase == PH_PREFILL ? true : (a.phase == PH_APPEND ? a.done[b] != 0 : a.done[b] == 0);
}

// True when no request whose rows fall in [t0, t1) takes part.
__device__ __forceinline__ bool none_active(const StepArgs &a, int t0, int t1) {
    t1 = min(t1, a.M);
    if (t0 >= t1) return true;
    for (int b = t0 / a.C; b <= (t1 - 1) / a.C; ++b)
        if (req_active(a, b)) return false;
    return true;
}

}  // namespace dg
