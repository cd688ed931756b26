// fp32 instantiation of the canvas step for small fp32 models: plain
// one-thread-per-output kernels with sequential fp32 dot products.  They
// follow the same definitions and workspace layout as the bf16 MFMA path
// (RMS row scale, RoPE with half-split pairs, block-bidirectional GQA
// attention over prefix || canvas keys, residual, vocabulary statistics per
// 64-id slice), and write the same per-slice statistics so the merge and
// commit kernels are shared.
#include <limits.h>

#include "dg_device.hpp"
#include "dg_internal.hpp"

namespace dg {

constexpr int F32_MAX_KEYS = 8192;   // prefix + canvas keys held in LDS per query

__global__ __launch_bounds__(128) void k_qkv_f32(StepArgs a, int kv_only, int mode) {
    const int t = blockIdx.x;
    const int hh = blockIdx.y + (kv_only ? a.Hq : 0);
    const int b = t / a.C;
    const int ic = t - b * a.C;
    const bool dn = (mode == WRITE_ALWAYS) ? true : (a.done[b] != 0);
    if (mode == WRITE_STEP && dn) return;
    if (mode == WRITE_APPEND && !dn) return;
    const int tok = ((const int32_t *)(a.ws + a.L.inp))[t];
    const float *e = (const float *)a.embed + (size_t)tok * a.d;
    const float re = ((const float *)(a.ws + a.L.r_e))[t];
    const float2 *rope = (const float2 *)(a.ws + a.L.rope) + (size_t)t * (a.hd / 2);
    const float *W;
    int base;
    if (hh < a.Hq) { W = (const float *)a.wq; base = hh * a.hd; }
    else if (hh < a.Hq + a.Hkv) { W = (const float *)a.wk; base = (hh - a.Hq) * a.hd; }
    else { W = (const float *)a.wv; base = (hh - a.Hq - a.Hkv) * a.hd; }
    const int hd2 = a.hd / 2;
    const int64_t pos = a.reqs.len[b] + ic;
    for (int j = threadIdx.x; j < hd2; j += blockDim.x) {
        const float *w0 = W + (size_t)(base + j) * a.d;
        const float *w1 = W + (size_t)(base + j + hd2) * a.d;
        float y0 = 0.f, y1 = 0.f;
        for (int k = 0; k < a.d; ++k) {
            y0 += e[k] * w0[k];
            y1 += e[k] * w1[k];
        }
        y0 *= re;
        y1 *= re;
        if (hh < a.Hq + a.Hkv) {
            const float2 cs = rope[j];
            const float x1 = y0, x2 = y1;
            y0 = x1 * cs.x - x2 * cs.y;
            y1 = x1 * cs.y + x2 * cs.x;
        }
        if (hh < a.Hq) {
            float *q = (float *)(a.ws + a.L.q) + ((size_t)t * a.Hq + hh) * a.hd;
            q[j] = y0;
            q[j + hd2] = y1;
        } else if (hh < a.Hq + a.Hkv) {
            const int g = hh - a.Hq;
            float *kr = (float *)a.reqs.k[b] + ((size_t)g * a.reqs.cap[b] + pos) * a.hd;
            kr[j] = y0;
            kr[j + hd2] = y1;
        } else {
            const int g = hh - a.Hq - a.Hkv;
            const int64_t cap = a.reqs.cap[b];
            float *vt = (float *)a.reqs.v[b] + (size_t)g * a.hd * cap + pos;
            vt[(size_t)j * cap] = y0;
            vt[(size_t)(j + hd2) * cap] = y1;
        }
    }
}

// One workgroup per (canvas position, query head, request): exact softmax
// over all prefix and canvas keys.
__global__ __launch_bounds__(256) void k_attn_f32(StepArgs a) {
    __shared__ float sc[F32_MAX_KEYS];
    __shared__ float qs[256];
    __shared__ float red[4];
    const int ic = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    if (a.done[b]) return;
    const int t = b * a.C + ic;
    const int g = h / (a.Hq / a.Hkv);
    const float *q = (const float *)(a.ws + a.L.q) + ((size_t)t * a.Hq + h) * a.hd;
    for (int e = threadIdx.x; e < a.hd; e += 256) qs[e] = q[e];
    __syncthreads();
    const int64_t cap = a.reqs.cap[b];
    const int L = (int)(a.reqs.len[b] + a.C);
    const float *Kg = (const float *)a.reqs.k[b] + (size_t)g * cap * a.hd;
    const float *Vg = (const float *)a.reqs.v[b] + (size_t)g * a.hd * cap;
    const float scale = 1.0f / sqrtf((float)a.hd);
    float mx = -INFINITY;
    for (int j = threadIdx.x; j < L; j += 256) {
        const float *kr = Kg + (size_t)j * a.hd;
        float s = 0.f;
        for (int e = 0; e < a.hd; ++e) s += qs[e] * kr[e];
        s *= scale;
        sc[j] = s;
        mx = fmaxf(mx, s);
    }
    mx = block_max_256(mx, red);
    float ls = 0.f;
    for (int j = threadIdx.x; j < L; j += 256) {
        const float p = expf(sc[j] - mx);
        sc[j] = p;
        ls += p;
    }
    const float l = block_sum_256(ls, red);   // its barriers also publish sc[]
    float *o = (float *)(a.ws + a.L.o) + ((size_t)t * a.Hq + h) * a.hd;
    for (int ch = threadIdx.x; ch < a.hd; ch += 256) {
        const float *vr = Vg + (size_t)ch * cap;
        float acc = 0.f;
        for (int j = 0; j < L; ++j) acc += sc[j] * vr[j];
        o[ch] = acc / l;
    }
}

__global__ __launch_bounds__(256) void k_oproj_f32(StepArgs a) {
    const int t = blockIdx.x;
    const int n = blockIdx.y * 256 + threadIdx.x;
    if (n >= a.d) return;
    const int K = a.Hq * a.hd;
    const int tok = ((const int32_t *)(a.ws + a.L.inp))[t];
    const float *o = (const float *)(a.ws + a.L.o) + (size_t)t * K;
    const float *w = (const float *)a.wo + (size_t)n * K;
    float acc = 0.f;
    for (int k = 0; k < K; ++k) acc += o[k] * w[k];
    const float e = ((const float *)a.embed)[(size_t)tok * a.d + n];
    ((float *)(a.ws + a.L.h))[(size_t)t * a.d + n] = e + acc;
}

// One wave per (64-id slice, compact row); lane = one id.
__global__ __launch_bounds__(64) void k_lmhead_f32(StepArgs a, float *logits) {
    const int v = blockIdx.x * 64 + threadIdx.x;
    const int r = blockIdx.y;                       // compact row: a position still uncommitted
    const int b = r / a.L.cp, j = r - (r / a.L.cp) * a.L.cp;
    if (a.done[b] || j >= ((const int32_t *)(a.ws + a.L.ucount))[b]) return;
    const int t = b * a.C + ((const int32_t *)(a.ws + a.L.ulist))[r];
    const float *h = (const float *)(a.ws + a.L.h) + (size_t)t * a.d;
    float z = -INFINITY;
    if (v < a.V && v != a.mask_id) {
        const float *w = (const float *)a.lm + (size_t)v * a.d;
        float acc = 0.f;
        for (int k = 0; k < a.d; ++k) acc += h[k] * w[k];
        z = ((const float *)(a.ws + a.L.r_h))[t] * acc;
    }
    if (logits && v < a.V) logits[(size_t)t * a.V + v] = z;
    VStat st{z, (z == -INFINITY) ? 0.f : 1.f, -INFINITY, (v < a.V) ? v : INT_MAX, 0.f, INT_MAX};
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) st = vmerge(st, vshfl_xor(st, o));
    if (threadIdx.x == 0) {
        const size_t rec = (size_t)r * a.L.n_slices + blockIdx.x;
        ((float4 *)(a.ws + a.L.lm_part))[rec] =
            make_float4(st.m, st.s, st.m2, __uint_as_float(pack_ids(st.a, st.m, st.a2, st.m2, blockIdx.x * 64)));
        ((float *)(a.ws + a.L.lm_tpart))[rec] = st.t;
    }
}

hipError_t launch_qkv_f32(const StepArgs &a, int kv_only, int mode, hipStream_t s) {
    const int n_heads = kv_only ? 2 * a.Hkv : a.Hq + 2 * a.Hkv;
    hipLaunchKernelGGL(k_qkv_f32, dim3(a.M, n_heads), dim3(128), 0, s, a, kv_only, mode);
    return hipGetLastError();
}

hipError_t launch_attention_f32(const StepArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_attn_f32, dim3(a.C, a.Hq, a.B), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_oproj_f32(const StepArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_oproj_f32, dim3(a.M, (a.d + 255) / 256), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_lmhead_f32(const StepArgs &a, float *logits, hipStream_t s) {
    hipLaunchKernelGGL(k_lmhead_f32, dim3((a.V + 63) / 64, a.L.rows_c), dim3(64), 0, s, a, logits);
    return hipGetLastError();
}

}  // namespace dg
