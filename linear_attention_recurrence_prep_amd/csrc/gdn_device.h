// Device helpers shared by the gfx950 kernels of the Gated DeltaNet library:
// bf16 <-> f32 conversion and cross-lane butterfly sums on 64-wide wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// ---------------------------------------------------------------- bf16 ----

// bf16 bits in the low / high half of a 32-bit word, widened exactly.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// f32 -> bf16 bits with the gfx950 conversion instruction (v_cvt_pk_bf16_f32:
// round to nearest, ties to even, in the default rounding mode; NaN stays NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xFFFFu; }

// 8 bf16 (one 16-byte vector) -> 8 floats.
__device__ __forceinline__ void unpack8(const uint4 w, float* f) {
    f[0] = bf16lo(w.x); f[1] = bf16hi(w.x);
    f[2] = bf16lo(w.y); f[3] = bf16hi(w.y);
    f[4] = bf16lo(w.z); f[5] = bf16hi(w.z);
    f[6] = bf16lo(w.w); f[7] = bf16hi(w.w);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}

// ------------------------------------------------------------ activations ----

// e^-|u| with subnormal results: the hardware exp2 does not return
// subnormals, so the exponent is halved (exactly) and the result squared:
// h = 2^(-|u| log2(e) / 2) stays normal for |u| < 174, and h·h rounds once,
// correctly, into the subnormal range (about 2 f32 ulp overall).
__device__ __forceinline__ float exp_neg_abs(float u) {
    const float h = __builtin_amdgcn_exp2f(fabsf(u) * -0.72134752044448170f);
    return h * h;
}

// silu(u) = u · sigmoid(u) in the form that cannot overflow, for values that
// are rounded to bf16 afterwards: with e = e^-|u| in (0, 1],
// silu(u) = (u >= 0 ? u : u·e) / (1 + e), so large negative u gives the tiny
// true value rather than u / inf.  Hardware exp2 and reciprocal, each within
// about one f32 ulp; the exp argument's rounding adds |u|·2^-24 relative, far
// below a bf16 rounding.  NaN stays NaN.
__device__ __forceinline__ float silu_fast(float u) {
    const float e = exp_neg_abs(u);
    const float s = __builtin_amdgcn_rcpf(1.0f + e);
    return (u >= 0.0f ? u : u * e) * s;
}

// ------------------------------------------------------ prologue pieces ----
// The per-element arithmetic of the prologue, shared by the prologue kernel
// and the chunk preparation that fuses it, so both produce identical bits.

// g = exp(-exp(A_log) softplus(a + dt_bias)), beta = sigmoid(b), from the
// stored bf16 a, b and the f32 A_log, dt_bias of the head.  beta uses the
// overflow-free form (e = e^-|b|: 1/(1+e), or e/(1+e) for b < 0) with the
// library exp and a true division: beta is kept in f32, so it is held to a
// few f32 ulps, not to a bf16 rounding.
__device__ __forceinline__ void gate_g_beta(uint16_t a, uint16_t b, float A_log, float dt_bias, float& g,
                                            float& beta) {
    const float x = __uint_as_float((uint32_t)a << 16) + dt_bias;
    const float sp = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
    g = expf(-expf(A_log) * sp);
    const float bb = __uint_as_float((uint32_t)b << 16);
    const float e = expf(-fabsf(bb));
    const float s = 1.f / (1.f + e);
    beta = bb >= 0.f ? s : e * s;
}

// One token of 8 channels: the depthwise conv over the K-1 window rows h and
// the new row x (weights w[j][e] for tap j, w[K-1] on the newest row), then
// SiLU (overflow-free, about 2 f32 ulp).
template <int K>
__device__ __forceinline__ void conv_silu8(const float (&w)[K][8], const float (&h)[K - 1][8], const float (&x)[8],
                                           float (&act)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float u = 0.f;
#pragma unroll
        for (int j = 0; j < K - 1; ++j) u = fmaf(w[j][e], h[j][e], u);
        u = fmaf(w[K - 1][e], x[e], u);
        act[e] = silu_fast(u);
    }
}

// ------------------------------------------------------------ cross-lane ----

// DPP controls (GCN/CDNA encoding): quad permutations, mirrors inside a
// 16-lane row and inside each 8-lane half-row.
enum : int {
    DPP_QUAD_XOR1 = 0xB1,  // quad_perm [1,0,3,2]
    DPP_QUAD_XOR2 = 0x4E,  // quad_perm [2,3,0,1]
    DPP_ROW_MIRROR = 0x140,
    DPP_ROW_HALF_MIRROR = 0x141,
};

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of W lanes (W in {4, 8, 16, 32}); every lane of a
// group receives the group's total.  Within a 16-lane row the steps are DPP
// permutations (no LDS traffic); the 32-lane step uses ds_swizzle.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(W == 4 || W == 8 || W == 16 || W == 32, "group width");
    x += dpp_mov<DPP_QUAD_XOR1>(x);
    x += dpp_mov<DPP_QUAD_XOR2>(x);
    if constexpr (W >= 8) x += dpp_mov<DPP_ROW_HALF_MIRROR>(x);
    if constexpr (W >= 16) x += dpp_mov<DPP_ROW_MIRROR>(x);
    if constexpr (W >= 32) {
        // bitmask swizzle inside 32-lane halves: lane ^ 16
        x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
    }
    return x;
}

// Two independent group sums interleaved, so their latency chains overlap.
template <int W>
__device__ __forceinline__ void group_sum2(float& x, float& y) {
    static_assert(W == 4 || W == 8 || W == 16 || W == 32, "group width");
    float a = dpp_mov<DPP_QUAD_XOR1>(x), b = dpp_mov<DPP_QUAD_XOR1>(y);
    x += a; y += b;
    a = dpp_mov<DPP_QUAD_XOR2>(x); b = dpp_mov<DPP_QUAD_XOR2>(y);
    x += a; y += b;
    if constexpr (W >= 8) {
        a = dpp_mov<DPP_ROW_HALF_MIRROR>(x); b = dpp_mov<DPP_ROW_HALF_MIRROR>(y);
        x += a; y += b;
    }
    if constexpr (W >= 16) {
        a = dpp_mov<DPP_ROW_MIRROR>(x); b = dpp_mov<DPP_ROW_MIRROR>(y);
        x += a; y += b;
    }
    if constexpr (W >= 32) {
        a = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
        b = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(y), 0x401F));
        x += a; y += b;
    }
}

// The q/k head norm of 8 channels held by each of the head's DK/8 lanes (an
// aligned lane group; every lane of it must execute this): sum of squares
// across the group, then act * scale / sqrt(mean + eps), rounded to bf16.
template <int DK>
__device__ __forceinline__ uint4 qk_norm8(const float (&act)[8], float scale, float eps) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(act[e], act[e], ss);
    ss = group_sum<DK / 8>(ss);
    const float rs = scale * __builtin_amdgcn_rsqf(ss * (1.0f / DK) + eps);
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = act[e] * rs;
    return pack8(o);
}

}  // namespace gdn
