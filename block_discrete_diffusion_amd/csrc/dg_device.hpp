// Device-side helpers: bf16 conversion, 32x32x16 bf16 MFMA, wave shuffles and
// the merge rule of per-slice vocabulary statistics.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <limits.h>

namespace dg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
// 16 bytes as a native vector (HIP's uint4 is a struct that blocks register
// promotion of staging arrays).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// D = A * B + C for one 32x32 tile, K = 16.  Lane l holds, for A, row l%32 and
// the 8 k-slots 8*(l/32)..+7; for B, column l%32 and the same k-slots; the
// result register r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Same tile shape with fp16 operands.
__device__ __forceinline__ f32x16 mfma32_f16(const u32x4 &a, const u32x4 &b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Two floats -> two fp16 / bf16 (round to nearest even), low half first;
// one packed conversion instruction on gfx950.
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}
__device__ __forceinline__ uint32_t pack_b2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
// The two bf16 halves of a word as floats (exact).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two bf16 (one 32-bit word) -> two fp16; exact for magnitudes in
// [2^-14, 65504] since fp16 carries 3 more significand bits than bf16.
__device__ __forceinline__ uint32_t bf2_to_h2(uint32_t w) { return pack_h2(bf_lo(w), bf_hi(w)); }

// Eight fp32 values (two 16-byte words) as bf16 MFMA operands.
// split2: hi = bf16(x), lo = bf16(x - hi), about 16 significant bits.
// split3: a third term bf16(x - hi - mid); hi + mid + lo == x exactly for
// normal fp32 x (each term takes the next 8 significand bits).
__device__ __forceinline__ void split2_bf16(const u32x4 &x0, const u32x4 &x1, u32x4 &hi, u32x4 &lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float f0 = __uint_as_float(i < 2 ? x0[2 * i] : x1[2 * i - 4]);
        const float f1 = __uint_as_float(i < 2 ? x0[2 * i + 1] : x1[2 * i - 3]);
        const uint32_t h = pack_b2(f0, f1);
        hi[i] = h;
        lo[i] = pack_b2(f0 - bf_lo(h), f1 - bf_hi(h));
    }
}

__device__ __forceinline__ void split3_bf16(const u32x4 &x0, const u32x4 &x1, u32x4 &hi, u32x4 &mid, u32x4 &lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float f0 = __uint_as_float(i < 2 ? x0[2 * i] : x1[2 * i - 4]);
        const float f1 = __uint_as_float(i < 2 ? x0[2 * i + 1] : x1[2 * i - 3]);
        const uint32_t h = pack_b2(f0, f1);
        const float r0 = f0 - bf_lo(h), r1 = f1 - bf_hi(h);
        const uint32_t m = pack_b2(r0, r1);
        hi[i] = h;
        mid[i] = m;
        lo[i] = pack_b2(r0 - bf_lo(m), r1 - bf_hi(m));
    }
}

// Eight bf16 (one 16-byte word) -> eight fp16 (exact in the binary16 normal
// range; below 2^-14 rounded to the subnormal grid, spacing 2^-24).
__device__ __forceinline__ u32x4 bf8_to_h8(const u32x4 &w) {
    return u32x4{bf2_to_h2(w[0]), bf2_to_h2(w[1]), bf2_to_h2(w[2]), bf2_to_h2(w[3])};
}

// Eight OCP e4m3 bytes (one 8-byte word pair) -> eight fp16: every e4m3 value
// (normals down to 2^-6, subnormals down to 2^-9, at most 448) is a binary16
// normal, so the conversion is exact.
__device__ __forceinline__ u32x4 fp8x8_to_h8(uint32_t lo, uint32_t hi) {
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true))};
}

// The same eight e4m3 bytes as bf16 values (exact: 3 fraction bits and the
// e4m3 exponent range fit bf16).
__device__ __forceinline__ u32x4 fp8x8_to_bf8(uint32_t lo, uint32_t hi) {
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
}

// Fragment-major layout of an activation matrix X[M][K] (M padded to a
// multiple of 32, K a multiple of 16), the order in which the 32x32x16 MFMA
// consumes it as the token-side operand: 32x16 blocks, block (t/32, k/16)
// holds 512 consecutive elements, and inside a block lane l = 32*((k%16)/8)
// + t%32 owns the 8 consecutive k values of its row.  A wave then loads one
// operand fragment as a single contiguous 1 KB (bf16) read.
__device__ __forceinline__ size_t frag_index(int t, int k, int K) {
    return ((size_t)(t >> 5) * (K >> 4) + (k >> 4)) * 512 + (size_t)((((k >> 3) & 1) << 5) + (t & 31)) * 8 + (k & 7);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, 64); }

// Vocabulary statistics of a set of logits z: m = max, s = sum exp(z - m),
// a = lowest id attaining m, (m2, a2) = the next entry in the order (value
// descending, id ascending), i.e. the second largest logit (equal to m on a
// tie) and its id, t = sum (z - m) exp(z - m) (so that the entropy of
// softmax(z) is ln s - t / s).  An empty set has m = m2 = -inf and
// a = a2 = INT_MAX.
struct VStat {
    float m, s, m2;
    int a;
    float t;
    int a2;
};

// (value, id) orders before (value', id') when value is larger, or equal
// with a lower id.
__device__ __forceinline__ bool vbefore(float v, int i, float w, int j) { return v > w || (v == w && i < j); }

// Merge of two disjoint sets.  Every field is chosen by a strict order or
// built from commutative operations (floating-point + and * commute), so
// both lanes of a butterfly obtain the same bits.  Relative to the merged
// max M, a set's t becomes exp(m - M) (t + (m - M) s).
__device__ __forceinline__ VStat vmerge(const VStat &x, const VStat &y) {
    VStat r;
    r.m = fmaxf(x.m, y.m);
    const float ex = (x.m == -INFINITY) ? 0.f : __expf(x.m - r.m);
    const float ey = (y.m == -INFINITY) ? 0.f : __expf(y.m - r.m);
    r.s = x.s * ex + y.s * ey;
    const float tx = (x.m == -INFINITY) ? 0.f : (x.t + (x.m - r.m) * x.s) * ex;
    const float ty = (y.m == -INFINITY) ? 0.f : (y.t + (y.m - r.m) * y.s) * ey;
    r.t = tx + ty;
    // top two of the union: the winner's first, then the better of the
    // loser's first and the winner's second
    const bool xw = vbefore(x.m, x.a, y.m, y.a);
    r.a = xw ? x.a : y.a;
    const float lm = xw ? y.m : x.m, wm2 = xw ? x.m2 : y.m2;
    const int la = xw ? y.a : x.a, wa2 = xw ? x.a2 : y.a2;
    const bool lt = vbefore(lm, la, wm2, wa2);
    r.m2 = lt ? lm : wm2;
    r.a2 = lt ? la : wa2;
    return r;
}

__device__ __forceinline__ VStat vshfl_xor(const VStat &v, int mask) {
    VStat r;
    r.m = shfl_xor_f(v.m, mask);
    r.s = shfl_xor_f(v.s, mask);
    r.m2 = shfl_xor_f(v.m2, mask);
    r.a = shfl_xor_i(v.a, mask);
    r.t = shfl_xor_f(v.t, mask);
    r.a2 = shfl_xor_i(v.a2, mask);
    return r;
}

// Per-slice vocabulary records hold (m, s, m2, ids) as four 32-bit words;
// the ids word packs the offsets of a and a2 from the slice's first id
// (16 bits each; 0xffff: no id, i.e. an entry at -inf).
__device__ __forceinline__ uint32_t pack_ids(int a, float m, int a2, float m2, int base) {
    const uint32_t lo = (m == -INFINITY || a == INT_MAX) ? 0xffffu : (uint32_t)(a - base);
    const uint32_t hi = (m2 == -INFINITY || a2 == INT_MAX) ? 0xffffu : (uint32_t)(a2 - base);
    return lo | (hi << 16);
}
__device__ __forceinline__ int unpack_id(uint32_t w, int base) {
    return (w == 0xffffu) ? INT_MAX : base + (int)w;
}

// Deterministic block-wide sum over blockDim.x == 256 threads (fixed tree).
__device__ __forceinline__ float block_sum_256(float v, float *sh) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += shfl_xor_f(v, o);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    float t = (sh[0] + sh[1]) + (sh[2] + sh[3]);
    __syncthreads();
    return t;
}

__device__ __forceinline__ float block_max_256(float v, float *sh) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, shfl_xor_f(v, o));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    float t = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
    __syncthreads();
    return t;
}

}  // namespace dg

namespace dg {

// Counter-based random numbers for temperature sampling: Philox4x64 with 10
// rounds (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC'11).  Each round multiplies words 0 and 2 by the round
// multipliers and recombines the 128-bit products' halves with words 1, 3
// and the key; the key advances by the Weyl increments between rounds.
struct Philox4 {
    uint64_t w[4];
    // word i (runtime i in 0..3) by selects: a dynamic index would put the
    // array in scratch memory
    __device__ __forceinline__ uint64_t word(int i) const {
        const uint64_t lo = (i & 1) ? w[1] : w[0], hi = (i & 1) ? w[3] : w[2];
        return (i & 2) ? hi : lo;
    }
};

__device__ __forceinline__ Philox4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0,
                                                 uint64_t k1) {
    constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += W0;
            k1 += W1;
        }
        const uint64_t h0 = __umul64hi(M0, c0), l0 = M0 * c0;
        const uint64_t h1 = __umul64hi(M1, c2), l1 = M1 * c2;
        const uint64_t n0 = h1 ^ c1 ^ k0, n2 = h0 ^ c3 ^ k1;
        c0 = n0;
        c1 = l1;
        c2 = n2;
        c3 = l0;
    }
    return Philox4{{c0, c1, c2, c3}};
}

// Standard Gumbel noise from the top 24 bits x of a Philox word:
// u = (x + 1/2) / 2^24, g = -ln(-ln u).  -ln u is formed without
// cancellation: 24 ln 2 - ln(x + 1/2) below 2^23, else -log1p(-e) with
// e = (2^24 - x - 1/2) / 2^24 (both x + 1/2 and e exact in fp32).
__device__ __forceinline__ float gumbel_f32(uint64_t word) {
    const uint32_t x = (uint32_t)(word >> 40);
    float t;
    if (x < (1u << 23)) t = 16.635532333438687f - __logf((float)x + 0.5f);
    else t = -log1pf(-((float)((1u << 24) - x) - 0.5f) * 5.9604644775390625e-8f);
    return -__logf(t);
}

// The same in double precision (the sampler's exact draws).
__device__ __forceinline__ double gumbel_f64(uint64_t word) {
    const double u = ((double)(word >> 40) + 0.5) * 5.9604644775390625e-8;
    return -log(-log(u));
}

// Top two (value, id) entries in (value descending, id ascending) order.
struct Top2 {
    float k1, k2;
    int i1, i2;
};

__device__ __forceinline__ void top2_push(Top2 &t, float k, int i) {
    if (vbefore(k, i, t.k1, t.i1)) {
        t.k2 = t.k1; t.i2 = t.i1;
        t.k1 = k; t.i1 = i;
    } else if (vbefore(k, i, t.k2, t.i2)) {
        t.k2 = k; t.i2 = i;
    }
}

__device__ __forceinline__ Top2 top2_merge(const Top2 &x, const Top2 &y) {
    const bool xw = vbefore(x.k1, x.i1, y.k1, y.i1);
    Top2 r;
    r.k1 = xw ? x.k1 : y.k1;
    r.i1 = xw ? x.i1 : y.i1;
    const float lk = xw ? y.k1 : x.k1, wk2 = xw ? x.k2 : y.k2;
    const int li = xw ? y.i1 : x.i1, wi2 = xw ? x.i2 : y.i2;
    const bool lt = vbefore(lk, li, wk2, wi2);
    r.k2 = lt ? lk : wk2;
    r.i2 = lt ? li : wi2;
    return r;
}

__device__ __forceinline__ Top2 top2_shfl_xor(const Top2 &v, int mask) {
    return Top2{shfl_xor_f(v.k1, mask), shfl_xor_f(v.k2, mask), shfl_xor_i(v.i1, mask), shfl_xor_i(v.i2, mask)};
}

}  // namespace dg
