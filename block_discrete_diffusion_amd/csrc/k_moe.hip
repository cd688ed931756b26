// Routed experts beside a layer's FFN (which is then their shared expert):
// the mixture-of-experts layer of the DiffusionGemma Technical Report,
// part 3, section 6 (GPU time breakdown: MoE, its experts chosen per token,
// and the shared expert).  On the FFN's normed input a = r x:
//   router logits l = a Wr^T; each token's top_k experts by logit (ties to
//   the lower expert id); gates = softmax of the chosen logits;
//   x <- x + shared(a) + sum_j g_j (silu(a Wge[e_j]^T) * (a Wue[e_j]^T)) Wde[e_j]^T.
// Launches (one step, one layer):
//   k_moe_logits  split-K MFMA GEMM of the router: partial logits [S][M][E];
//   k_moe_topk    a wave per token: sums the partials (chunk order), scales by
//                 r, picks the top_k, writes the choices and gates;
//   k_moe_lists   one workgroup: per expert its token count, the start of its
//                 rows (multiples of 32) and the slots t k + j in them;
//   k_moe_dispatch  copies each chosen slot's row of x (fp16 hi / lo planes)
//                 to its place in its expert's rows, fragment-major;
//   k_moe_up      per (expert, 32 features): its rows of x against the gate
//                 and up weights, and writes the SwiGLU
//                 activation rows, fp16 hi / lo planes, fragment-major in
//                 the expert's rows;
//   k_moe_down    per (expert, 64 outputs): the gated expert outputs per slot
//                 (fp32 [M k][d]); the FFN's residual finish adds a token's
//                 k slots in rank order.
// Only the experts some token chose do work: k_moe_lists lists them, and the
// expert GEMMs' workgroups stride over (chosen expert, tile) items, so the
// weights streamed per step are those of the chosen experts.  A slot's row in an expert's list depends on arrival order
// (LDS atomics), but every MFMA row is computed on its own, so the results
// do not.
#include <algorithm>

#include "dg_device.hpp"
#include "dg_gemm.hpp"
#include "dg_internal.hpp"

namespace dg {

// Router logits, split over K: workgroup (chunk kc, 64 experts nt, 128
// tokens mt); x enters as its fp16 hi and lo planes (fragment-major, ~22
// significant bits) against the router rows converted to fp16 in LDS.
template <int NSTC>
__global__ __launch_bounds__(256) void k_moe_logits(StepArgs a, int n_mt, int S) {
    __shared__ u32x4 lds[2 * 2 * 256];
    const int E = a.n_experts;
    const int n_nt = (E + 63) / 64;
    int j;
    if (!xcd_index(S * n_nt * n_mt, j)) return;
    const int kc = j % S;
    const int rem = j / S;
    const int nt = rem / n_mt, mt = rem - (rem / n_mt) * n_mt;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, row32 = lane & 31;
    const int tok_wg = mt * 128;
    if (none_active(a, tok_wg, tok_wg + 128)) return;
    const int kchunk = a.d / S;
    const int k0 = kc * kchunk;
    const uint16_t *wp[2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
        wp[x] = (const uint16_t *)a.wr + (size_t)min(64 * nt + 32 * x + (tid >> 3), E - 1) * a.d + k0 + (tid & 7) * 8;
    const void *ap[1];
    const int tok0 = tok_wg + wave * 32;
    ap[0] = (const uint16_t *)(a.ws + a.L.xp) + ((size_t)min(tok0 / 32, a.L.m_pad / 32 - 1) * (a.d / 16) + k0 / 16) * 512 +
            lane * 8;
    f32x16 acc[2][1];
    gemm_core<2, 1, 2, 2, 2, NSTC, 2, 256, true, true>(wp, 0, ap, kchunk, lds, acc, true, (size_t)a.L.m_pad * a.d);
    const int t = tok0 + row32;
    if (t >= a.M || !req_active(a, t / a.C)) return;
    float *part = (float *)(a.ws + a.L.moe_logit) + ((size_t)kc * a.M + t) * E;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int e = 64 * nt + 32 * x + 8 * (r >> 2) + 4 * half + (r & 3);
            if (e < E) part[e] = acc[x][0][r];
        }
}

constexpr int MOE_SPLIT_MAX = 32;                     // router chunks: d / 128 <= 32

// A wave per token: the logits (chunks added in order, times r), the top_k
// in (logit desc, expert asc) order, the gates.  Lane holds experts lane,
// lane + 64, ... (E <= 256).
__global__ __launch_bounds__(256) void k_moe_topk(StepArgs a, int S) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= a.M || !req_active(a, t / a.C)) return;
    const int E = a.n_experts, k = a.top_k;
    const float r = ((const float *)(a.ws + a.L.r_x))[t];
    const float *part = (const float *)(a.ws + a.L.moe_logit) + (size_t)t * E;
    // every chunk's partial first (all loads in flight together), then the
    // sums in chunk order
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = min(lane + 64 * q, E - 1);
        float p[MOE_SPLIT_MAX];
#pragma unroll
        for (int c = 0; c < MOE_SPLIT_MAX; ++c) p[c] = c < S ? part[(size_t)c * a.M * E + e] : 0.f;
        float s = p[0];
#pragma unroll
        for (int c = 1; c < MOE_SPLIT_MAX; ++c) s += c < S ? p[c] : 0.f;
        v[q] = lane + 64 * q < E ? r * s : -INFINITY;
    }
    int32_t *sel = (int32_t *)(a.ws + a.L.moe_sel) + ((size_t)a.layer * a.M + t) * k;
    float *gate = (float *)(a.ws + a.L.moe_gate) + (size_t)t * k;
    float l0 = 0.f, den = 0.f;
    float myl = 0.f;                                   // lane jj keeps the jj-th choice
    int myi = 0;
    for (int jj = 0; jj < k; ++jj) {
        // this lane's best (value desc, id asc), then across the wave
        float bv = v[0];
        int bi = lane;
#pragma unroll
        for (int q = 1; q < 4; ++q)
            if (v[q] > bv) { bv = v[q]; bi = lane + 64 * q; }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const float ov = shfl_xor_f(bv, o);
            const int oi = shfl_xor_i(bi, o);
            if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
        }
        if ((bi & 63) == lane) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (q == (bi >> 6)) v[q] = -INFINITY;
        }
        if (lane == jj) { myl = bv; myi = bi; }
        if (jj == 0) l0 = bv;
        den += __expf(bv - l0);
    }
    if (lane < k) {
        sel[lane] = myi;
        gate[lane] = __expf(myl - l0) / den;
    }
}

// One workgroup: per expert its count of active slots, the start of its rows
// (counts rounded up to 32, in expert order) and the slots in its rows.
// The starts and the list of chosen experts are one wave's prefix sums
// (lane l holds experts 4l .. 4l + 3, E <= 256).
__global__ __launch_bounds__(1024) void k_moe_lists(StepArgs a) {
    __shared__ int cnt[256], fill[256], off[256];
    const int E = a.n_experts, k = a.top_k;
    const int tid = threadIdx.x;
    const int n = a.M * k;
    const int32_t *sel = (const int32_t *)(a.ws + a.L.moe_sel) + (size_t)a.layer * n;
    if (tid < 256) { cnt[tid] = 0; fill[tid] = 0; }
    __syncthreads();
    for (int i = tid; i < n; i += 1024)
        if (req_active(a, (i / k) / a.C)) atomicAdd(&cnt[sel[i]], 1);
    __syncthreads();
    int32_t *ids = (int32_t *)(a.ws + a.L.moe_ids);    // [0]: count of chosen experts, then their ids
    if (tid < 64) {
        int c[4], rows = 0, used = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = 4 * tid + q;
            c[q] = e < E ? cnt[e] : 0;
            rows += (c[q] + 31) & ~31;
            used += c[q] > 0 ? 1 : 0;
        }
        int rows_inc = rows, used_inc = used;         // inclusive scans over the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int r = __shfl_up(rows_inc, o, 64), u = __shfl_up(used_inc, o, 64);
            if (tid >= o) {
                rows_inc += r;
                used_inc += u;
            }
        }
        int o = rows_inc - rows, z = used_inc - used;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = 4 * tid + q;
            if (e < E) {
                off[e] = o;
                o += (c[q] + 31) & ~31;
                if (c[q] > 0) ids[1 + z++] = e;
            }
        }
        if (tid == 63) ids[0] = used_inc;
    }
    __syncthreads();
    if (tid < E) {
        ((int32_t *)(a.ws + a.L.moe_cnt))[tid] = cnt[tid];
        ((int32_t *)(a.ws + a.L.moe_off))[tid] = off[tid];
    }
    int32_t *list = (int32_t *)(a.ws + a.L.moe_list);
    // each chosen expert's padding rows hold -1 (thread: expert x / 32, row x % 32)
    for (int x = tid; x < 32 * E; x += 1024) {
        const int e = x >> 5, r = x & 31;
        const int pad = ((cnt[e] + 31) & ~31) - cnt[e];
        if (r < pad) list[off[e] + cnt[e] + r] = -1;
    }
    for (int i = tid; i < n; i += 1024)
        if (req_active(a, (i / k) / a.C)) {
            const int e = sel[i];
            list[off[e] + atomicAdd(&fill[e], 1)] = i;
        }
}

// Dispatch: the rows of x of every chosen slot, as fp16 hi and lo planes,
// fragment-major at the slot's row in its expert's rows (the operand layout
// of the expert GEMMs: coalesced 1 KB fragment loads instead of a gather of
// scattered rows in the product loop).  A wave fills one 32-row x 16-feature
// fragment block: lane l takes row 32 pt + l % 32, features 16 kb + 8 (l / 32)
// .. + 7, so its 16-byte stores are the block's contiguous 1 KB; the loads
// gather 32-byte pieces of the slots' rows of x (L2-resident).
__global__ __launch_bounds__(256) void k_moe_dispatch(StepArgs a) {
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nkb = a.d / 16;
    const int pt = w / nkb, kb = w - (w / nkb) * nkb;
    const int k = a.top_k;
    const int32_t *list = (const int32_t *)(a.ws + a.L.moe_list);
    const int32_t *cnt = (const int32_t *)(a.ws + a.L.moe_cnt);
    const int32_t *off = (const int32_t *)(a.ws + a.L.moe_off);
    const int32_t *ids = (const int32_t *)(a.ws + a.L.moe_ids);
    const int na = ids[0];
    const int rows = na > 0 ? off[ids[na]] + cnt[ids[na]] : 0;   // rows in use: up to the last chosen expert's
    const uint16_t *xr = (const uint16_t *)(a.ws + a.L.xr);
    uint16_t *xg = (uint16_t *)(a.ws + a.L.moe_xg);
    const size_t plane_in = (size_t)a.M * a.d, plane_out = (size_t)a.L.mk_pad * a.d;
    const int p = 32 * pt + (lane & 31);
    if (p >= rows) return;
    const int s = list[p];
    if (s < 0) return;                                 // a padding row of an expert
    const int kf = 16 * kb + 8 * (lane >> 5);
    const uint16_t *src = xr + (size_t)(s / k) * a.d + kf;
    const u32x4 hi = *(const u32x4 *)src, lo = *(const u32x4 *)(src + plane_in);
    const size_t fi = frag_index(p, kf, a.d);
    *(u32x4 *)(xg + fi) = hi;
    *(u32x4 *)(xg + plane_out + fi) = lo;
}

// Expert gate / up projections with the SwiGLU activation: workgroup (expert
// e, features 32 ft .. + 31 of both Wge[e] (MFMA tile 0) and Wue[e] (tile
// 1)), 512 threads: two groups of 4 waves take one half of the K axis each
// (own LDS staging buffers, same barriers), 32 of the expert's slots per
// wave per pass; the second group hands its accumulators to the first
// through LDS, which adds them (fixed order) and runs the epilogue.  The
// operand is the dispatched copy of x (fp16 hi / lo planes, fragment-major
// at the expert's rows).  act =
// silu(r g) * (r u) as fp16 hi / lo planes at the expert's rows.  KH = 1:
// one group of 256 threads over the whole K axis.
template <int NSTC, int KH>
__global__ __launch_bounds__(256 * KH) void k_moe_up(StepArgs a, int n_ft) {
    __shared__ u32x4 lds[2][2 * 2 * 256];
    const int32_t *ids = (const int32_t *)(a.ws + a.L.moe_ids);
    const int n_work = ids[0] * n_ft;
    for (int w = blockIdx.x; w < n_work; w += gridDim.x) {
    const int e = ids[1 + w / n_ft], ft = w - (w / n_ft) * n_ft;
    const int cnt = ((const int32_t *)(a.ws + a.L.moe_cnt))[e];
    const int off = ((const int32_t *)(a.ws + a.L.moe_off))[e];
    const int32_t *list = (const int32_t *)(a.ws + a.L.moe_list) + off;
    const int kh = KH == 2 ? (int)(threadIdx.x >> 8) : 0;
    const int tid = threadIdx.x & 255, wave = tid >> 6, lane = tid & 63, half = lane >> 5, row32 = lane & 31;
    const int de = a.d_e, k = a.top_k;
    const int kc = a.d / KH, k0 = kh * kc;
    const uint16_t *wp[2];
    {
        const size_t row = (size_t)e * de + 32 * ft + (tid >> 3);
        wp[0] = (const uint16_t *)a.wge + row * a.d + k0 + (tid & 7) * 8;
        wp[1] = (const uint16_t *)a.wue + row * a.d + k0 + (tid & 7) * 8;
    }
    const uint16_t *xg = (const uint16_t *)(a.ws + a.L.moe_xg);
    uint16_t *act = (uint16_t *)(a.ws + a.L.moe_act);
    const size_t plane = (size_t)a.L.mk_pad * de;
    float *red = (float *)&lds[0][0];                  // [32 values][256 threads] after the product
    for (int p0 = 0; p0 < cnt; p0 += 128) {
        const int q = p0 + wave * 32 + row32;
        const int tq = list[min(q, cnt - 1)] / k;      // rows past the count read a valid row, dropped
        // the wave's 32-row block of the expert's rows (clamped into them)
        const int row = off + min(p0 + wave * 32, (cnt - 1) & ~31);
        const void *ap[1] = {xg + ((size_t)(row / 32) * (a.d / 16) + k0 / 16) * 512 + lane * 8};
        f32x16 acc[2][1];
        gemm_core<2, 1, 4, 2, 2, NSTC, 2, 256, true, true>(wp, 0, ap, kc, lds[kh], acc, p0 + wave * 32 < cnt,
                                                           (size_t)a.L.mk_pad * a.d);
        if constexpr (KH == 2) {
            __syncthreads();                             // every wave past its last fragment read
            if (kh == 1) {
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int r = 0; r < 16; ++r) red[(x * 16 + r) * 256 + tid] = acc[x][0][r];
            }
            __syncthreads();
            if (kh == 0) {
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[x][0][r] += red[(x * 16 + r) * 256 + tid];
            }
        }
        if (kh == 0 && q < cnt) {
            const float rr = ((const float *)(a.ws + a.L.r_x))[tq];
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                float y[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const float g = rr * acc[0][0][4 * rg + x], u = rr * acc[1][0][4 * rg + x];
                    y[x] = g / (1.0f + __expf(-g)) * u;
                }
                const uint32_t p01 = pack_h2(y[0], y[1]), p23 = pack_h2(y[2], y[3]);
                const f32x2 f01 = __builtin_convertvector(__builtin_bit_cast(f16x2, p01), f32x2);
                const f32x2 f23 = __builtin_convertvector(__builtin_bit_cast(f16x2, p23), f32x2);
                const size_t fi = frag_index(off + q, 32 * ft + 8 * rg + 4 * half, de);
                *(uint2 *)(act + fi) = make_uint2(p01, p23);
                *(uint2 *)(act + plane + fi) =
                    make_uint2(pack_h2(y[0] - f01.x, y[1] - f01.y), pack_h2(y[2] - f23.x, y[3] - f23.y));
            }
        }
        __syncthreads();                                 // LDS is reused by the next pass
    }
    }
}

// Expert down projections: workgroup (expert e, outputs 64 nt .. + 63),
// 4 waves x 32 of the expert's slots per pass;
// the expert's activation rows (fragment-major, fp16 hi / lo planes) against
// Wde[e] converted to fp16 in LDS.  Writes gate * output for each slot.
template <int NSTC>
__global__ __launch_bounds__(256) void k_moe_down(StepArgs a, int n_nt) {
    __shared__ u32x4 lds[2 * 2 * 256];
    const int32_t *ids = (const int32_t *)(a.ws + a.L.moe_ids);
    const int n_work = ids[0] * n_nt;
    for (int w = blockIdx.x; w < n_work; w += gridDim.x) {
    const int e = ids[1 + w / n_nt], nt = w - (w / n_nt) * n_nt;
    const int cnt = ((const int32_t *)(a.ws + a.L.moe_cnt))[e];
    const int off = ((const int32_t *)(a.ws + a.L.moe_off))[e];
    const int32_t *list = (const int32_t *)(a.ws + a.L.moe_list) + off;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, row32 = lane & 31;
    const int de = a.d_e;
    const uint16_t *wp[2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
        wp[x] = (const uint16_t *)a.wde + ((size_t)e * a.d + 64 * nt + 32 * x + (tid >> 3)) * de + (tid & 7) * 8;
    const uint16_t *act = (const uint16_t *)(a.ws + a.L.moe_act);
    const float *gate = (const float *)(a.ws + a.L.moe_gate);
    float *y = (float *)(a.ws + a.L.moe_y);
    for (int p0 = 0; p0 < cnt; p0 += 128) {
        const void *ap[1];
        {
            const int row = off + min(p0 + wave * 32, ((cnt - 1) & ~31));   // 32-row block, in the expert's rows
            ap[0] = act + (size_t)(row / 32) * (de / 16) * 512 + lane * 8;
        }
        f32x16 acc[2][1];
        gemm_core<2, 1, 4, 2, 2, NSTC, 2, 256, true, true>(wp, 0, ap, de, lds, acc, p0 + wave * 32 < cnt,
                                                           (size_t)a.L.mk_pad * de);
#pragma unroll
        for (int tm = 0; tm < 1; ++tm) {
            const int q = p0 + wave * 32 + row32;
            if (q >= cnt) continue;
            const int s = list[q];
            const float g = gate[s];
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int n = 64 * nt + 32 * x + 8 * rg + 4 * half;
                    *(float4 *)(y + (size_t)s * a.d + n) =
                        make_float4(g * acc[x][tm][4 * rg], g * acc[x][tm][4 * rg + 1], g * acc[x][tm][4 * rg + 2],
                                    g * acc[x][tm][4 * rg + 3]);
                }
        }
        __syncthreads();
    }    }
}

hipError_t launch_moe(const StepArgs &a, hipStream_t s) {
    if (a.dtype != DG_BF16 || a.n_experts <= 0 || a.n_experts > 256 || a.top_k < 1 || a.top_k > 16 ||
        a.d_e % 256 || a.d % 128)
        return hipErrorInvalidValue;
    const int n_mt = (a.M + 127) / 128;
    const int S = a.d / 128;                           // two stages of 64 per chunk
    {
        const dim3 g(((S * ((a.n_experts + 63) / 64) * n_mt) + 7) & ~7);
        hipLaunchKernelGGL(k_moe_logits<2>, g, dim3(256), 0, s, a, n_mt, S);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_moe_topk, dim3((a.M + 3) / 4), dim3(256), 0, s, a, S);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_moe_lists, dim3(1), dim3(1024), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // a wave per 32-row x 16-feature block of every row the lists can hold
    // (those past the rows in use return at once)
    hipLaunchKernelGGL(k_moe_dispatch, dim3(((a.L.mk_pad + 31) / 32 * (a.d / 16) + 3) / 4), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
        const int n_ft = a.d_e / 32;
        const dim3 g(std::min(a.n_experts * n_ft, 256));   // one workgroup per CU, striding over the work
        // two K halves of d / 128 stages where the ring of 4 divides them
        // (d % 512 == 0), else one group over the d / 64 stages
        if ((a.d / 128) % 4 == 0) {
            switch (a.d / 128) {
                case 8: hipLaunchKernelGGL((k_moe_up<8, 2>), g, dim3(512), 0, s, a, n_ft); break;
                case 16: hipLaunchKernelGGL((k_moe_up<16, 2>), g, dim3(512), 0, s, a, n_ft); break;
                case 32: hipLaunchKernelGGL((k_moe_up<32, 2>), g, dim3(512), 0, s, a, n_ft); break;
                default: hipLaunchKernelGGL((k_moe_up<0, 2>), g, dim3(512), 0, s, a, n_ft); break;
            }
        } else {
            hipLaunchKernelGGL((k_moe_up<0, 1>), g, dim3(256), 0, s, a, n_ft);
        }
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
        const int n_nt = a.d / 64;
        const dim3 g(std::min(a.n_experts * n_nt, 512));
        switch (a.d_e / 64) {
            case 4: hipLaunchKernelGGL(k_moe_down<4>, g, dim3(256), 0, s, a, n_nt); break;
            case 8: hipLaunchKernelGGL(k_moe_down<8>, g, dim3(256), 0, s, a, n_nt); break;
            case 16: hipLaunchKernelGGL(k_moe_down<16>, g, dim3(256), 0, s, a, n_nt); break;
            default: hipLaunchKernelGGL(k_moe_down<0>, g, dim3(256), 0, s, a, n_nt); break;
        }
    }
    return hipGetLastError();
}

}  // namespace dg
