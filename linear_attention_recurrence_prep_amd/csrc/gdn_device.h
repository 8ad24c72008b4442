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

// The depthwise conv on its operands as stored bf16 pairs.  The dot-product
// instruction (v_dot2_f32_bf16) multiplies two bf16 pairs, each product
// exact, and adds both to an f32 addend in f32.  A channel's taps (w0, w1)
// and (w2, w3) are adjacent in conv_w [C, K], so for K = 2 and 4 the weight
// pairs are the stored words; the data pair (x_s, x_{s+1}) of a channel is
// one byte permutation of two token rows, and each pair serves two tokens
// (the newer pair of one is the older pair of the token two steps on).
// Nothing is widened to f32, which halves the registers the conv holds.

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// bf16 element i (0..7) of a 16-byte vector, widened exactly
__device__ __forceinline__ float bf16_at(const uint4& v, int i) {
    const uint32_t w = word_of(v, i / 2);
    return (i & 1) ? bf16hi(w) : bf16lo(w);
}

// channel e (0..7) of two token rows as the bf16 pair (older, newer), older
// in the low half: one v_perm_b32
__device__ __forceinline__ uint32_t row_pair(const uint4& older, const uint4& newer, int e) {
    return __builtin_amdgcn_perm(word_of(newer, e / 2), word_of(older, e / 2), (e & 1) ? 0x07060302u : 0x05040100u);
}

typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

// w.lo * x.lo + w.hi * x.hi + c (bf16 pairs, f32 addend and result)
__device__ __forceinline__ float dot2_bf16(uint32_t w, uint32_t x, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, w), __builtin_bit_cast(bf16x2v_t, x), c,
                                           false);
}

// Conv weights of 8 channels: pairs (w_{2i}, w_{2i+1}) per channel and, for
// odd K, the last tap widened to f32.
template <int K>
struct ConvW {
    uint32_t p[8][K / 2];
    float last[K % 2 ? 8 : 1];
};

// From the K stored 16-byte vectors of conv_w [c0 .. c0 + 7][0 .. K - 1]
// (bf16 element e * K + j is channel c0 + e, tap j).
template <int K>
__device__ __forceinline__ ConvW<K> conv_weights(const uint4 (&wk)[K]) {
    auto bf = [&](int i) -> uint32_t {
        const uint32_t x = word_of(wk[i / 8], (i % 8) / 2);
        return (i & 1) ? x >> 16 : x & 0xFFFFu;
    };
    ConvW<K> w;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int i = 0; i < K / 2; ++i) w.p[e][i] = bf(e * K + 2 * i) | (bf(e * K + 2 * i + 1) << 16);
        if constexpr (K % 2 != 0) w.last[e] = __uint_as_float(bf(e * K + K - 1) << 16);
    }
    return w;
}

// One token of 8 channels from the K rows of the spliced input that the
// conv reads (oldest first; the last is the token's own row; w_{K-1} on it),
// then SiLU (overflow-free, about 2 f32 ulp).
template <int K>
__device__ __forceinline__ void conv_silu8(const ConvW<K>& w, const uint4 (&r)[K], float (&act)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float u = 0.f;
#pragma unroll
        for (int i = 0; i < K / 2; ++i) u = dot2_bf16(w.p[e][i], row_pair(r[2 * i], r[2 * i + 1], e), u);
        if constexpr (K % 2 != 0) u = fmaf(w.last[e], bf16_at(r[K - 1], e), u);
        act[e] = silu_fast(u);
    }
}

// ------------------------------------------------------------ cross-lane ----

// DPP controls (GCN/CDNA encoding): quad permutations, mirrors inside a
// 16-lane row and inside each 8-lane half-row.
enum : int {
    DPP_QUAD_XOR1 = 0xB1,  // quad_perm [1,0,3,2]
    DPP_QUAD_XOR2 = 0x4E,  // quad_perm [2,3,0,1]
    DPP_ROW_SHL1 = 0x101,  // lane i reads lane i + n of its 16-lane row
    DPP_ROW_SHL2 = 0x102,
    DPP_ROW_SHL4 = 0x104,
    DPP_ROW_MIRROR = 0x140,
    DPP_ROW_HALF_MIRROR = 0x141,
};

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Product over lanes k .. 7 of each aligned group of 8 lanes (k = lane & 7):
// Hillis-Steele suffix scan, three DPP row shifts.
__device__ __forceinline__ float suffix_prod8(float x) {
    const int k = threadIdx.x & 7;
    float y = dpp_mov<DPP_ROW_SHL1>(x);
    x *= k + 1 < 8 ? y : 1.f;
    y = dpp_mov<DPP_ROW_SHL2>(x);
    x *= k + 2 < 8 ? y : 1.f;
    y = dpp_mov<DPP_ROW_SHL4>(x);
    x *= k + 4 < 8 ? y : 1.f;
    return x;
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
// aligned lane group; every lane of the group executes this): sum of
// squares across the group, then act * scale / sqrt(mean + eps), rounded to
// bf16.  Lanes whose channels are v (norm = false) run the same
// instructions, as the rest of the wave does, and return act rounded to bf16
// (act * 1 is act exactly).
template <int DK>
__device__ __forceinline__ uint4 qk_norm8(const float (&act)[8], bool norm, float scale, float eps) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(act[e], act[e], ss);
    ss = group_sum<DK / 8>(ss);
    const float rs = norm ? scale * __builtin_amdgcn_rsqf(ss * (1.0f / DK) + eps) : 1.0f;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = act[e] * rs;
    return pack8(o);
}

}  // namespace gdn
