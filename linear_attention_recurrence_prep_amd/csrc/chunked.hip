// Gated delta rule in chunked form on gfx950 matrix cores.
//
// The recurrence of "mlex 0.1.2 -- src/models/gated_delta.rs"
// (GatedDeltaNet::forward loop) and "mlx-bun 0.4.0 -> 1.0.0, qwen3-delta.ts"
// (gated_delta_step), per (b, hv):
//   S_t = g_t S_{t-1} + delta_t k_t^T,   delta_t = beta_t (v_t - g_t S_{t-1} k_t),
//   y_t = S_t q_t
// is rewritten over a chunk of C steps that starts from S_0.  With
//   R[t][s] = g_{s+1} ... g_t       (decay from step s to step t, R[t][t] = 1)
//   gamma_t = g_0 ... g_t = g_0 R[t][0],   rho_s = R[C-1][s]
//   A[t][s] = beta_t R[t][s] (k_t . k_s)   for s < t   (strictly lower)
//   T       = (I + A)^-1                   (unit lower triangular)
// unrolling the recurrence inside the chunk gives, as matrices over the chunk,
//   Delta = T diag(beta) V  -  T diag(beta gamma) K S_0^T      [C x Dv]
//   Y     = diag(gamma) Q S_0^T  +  P Delta,  P[t][s] = R[t][s] (q_t . k_s), s <= t
//   S_C   = gamma_{C-1} S_0  +  (diag(rho) Delta)^T K
// (Delta's rows are the deltas of the steps, Y's rows the outputs).  This is
// the same arithmetic as the per-step loop up to rounding order: dense
// products replace the per-step dot products.
//
// Two kernels:
//  * chunk_prep_kernel, one block per (b, hv, chunk), independent of the
//    state: k k^T and q k^T on bf16 MFMA (exact products of the bf16 inputs,
//    fp32 accumulation), the decay ratios as direct products (never quotients
//    of cumulative decays, so underflow to zero is harmless), and the unit
//    lower-triangular solve by forward substitution, one column per thread,
//    for W = T diag(beta gamma) K and T.  Writes W, Tb = T diag(beta), P,
//    gamma and rho to the workspace.
//  * chunk_seq_kernel, one block per (b, hv, 16 state rows), walks the chunks
//    in order holding its 16 x Dk slice of S in MFMA accumulators; per chunk
//    it forms W S_0^T and Q S_0^T (fp32 MFMA), U = Tb V, Delta = U - W S_0^T,
//    Y = gamma Q S_0^T + P Delta and the new S, all on fp32 MFMA.
// Padding steps past T carry g = 1, beta = 0 and zero k, q: their Delta is 0
// and they leave S unchanged.
#include <algorithm>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

typedef float f4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));

constexpr int CK = 32;        // chunk length
constexpr int RB = 16;        // state rows per sequential block

__device__ __forceinline__ f4_t mfma4(float a, float b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ========================================================= chunk preparation

template <int DK>
struct PrepSmem {
    uint16_t kb[CK][DK + 8];     // bf16 rows, padded against bank conflicts
    uint16_t qb[CK][DK + 8];
    float kk[CK][CK + 1];
    float qk[CK][CK + 1];
    float a[CK][CK + 4];         // strictly lower A (row-major, 16-byte rows)
    float gs[CK], bs[CK], gm[CK];
};

template <int DK>
__global__ __launch_bounds__(256, 4) void chunk_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, float* __restrict__ W, float* __restrict__ Tb, float* __restrict__ P,
    float* __restrict__ Gm, float* __restrict__ Rho, int T, int Hk, int Hv, int NC) {
    __shared__ PrepSmem<DK> sh;
    const int unit = blockIdx.x;              // (b * Hv + hv) * NC + c
    const int c = unit % NC;
    const int n = unit / NC;
    const int b = n / Hv, hv = n % Hv;
    const int hk = hv / (Hv / Hk);
    const int t0 = c * CK;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // 1. k, q rows of the chunk (zero past T), g and beta (1 and 0 past T)
    for (int idx = tid; idx < CK * DK / 8; idx += 256) {
        const int t = idx / (DK / 8), c8 = idx % (DK / 8);
        uint4 kv = make_uint4(0, 0, 0, 0), qv = kv;
        if (t0 + t < T) {
            const int64_t off = (((int64_t)b * T + t0 + t) * Hk + hk) * DK + c8 * 8;
            kv = *reinterpret_cast<const uint4*>(k + off);
            qv = *reinterpret_cast<const uint4*>(q + off);
        }
        *reinterpret_cast<uint4*>(&sh.kb[t][c8 * 8]) = kv;
        *reinterpret_cast<uint4*>(&sh.qb[t][c8 * 8]) = qv;
    }
    if (tid < CK) {
        const int t = t0 + tid;
        const int64_t i = ((int64_t)b * T + min(t, T - 1)) * Hv + hv;
        const float gv = g[i], bv = beta[i];
        sh.gs[tid] = t < T ? gv : 1.f;
        sh.bs[tid] = t < T ? bv : 0.f;
    }
    __syncthreads();

    // 2. k k^T and q k^T, 32 x 32 each: wave w owns output tile (w / 2, w % 2)
    {
        const int mi = wave >> 1, ni = wave & 1;
        f4_t ckk = {0.f, 0.f, 0.f, 0.f}, cqk = ckk;
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
            const int col = ks * 32 + 8 * (lane >> 4);
            const uint4 ka = *reinterpret_cast<const uint4*>(&sh.kb[16 * mi + (lane & 15)][col]);
            const uint4 qa = *reinterpret_cast<const uint4*>(&sh.qb[16 * mi + (lane & 15)][col]);
            const uint4 kb = *reinterpret_cast<const uint4*>(&sh.kb[16 * ni + (lane & 15)][col]);
            ckk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8_t, ka),
                                                         __builtin_bit_cast(bf8_t, kb), ckk, 0, 0, 0);
            cqk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8_t, qa),
                                                         __builtin_bit_cast(bf8_t, kb), cqk, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sh.kk[16 * mi + 4 * (lane >> 4) + i][16 * ni + (lane & 15)] = ckk[i];
            sh.qk[16 * mi + 4 * (lane >> 4) + i][16 * ni + (lane & 15)] = cqk[i];
        }
    }
    __syncthreads();

    // 3. decay ratios R[t][s] = g_{s+1}...g_t (s <= t) for s in this thread's
    //    four columns, then A, P, gamma, rho
    {
        const int t = tid >> 3, s0 = (tid & 7) * 4;
        float r[4];
        // R[t][s0+3] = g_{s0+4}...g_t, then R[t][s] = R[t][s+1] g_{s+1} while
        // s+1 <= t; R[t][s] = 1 for s >= t (only s = t is used)
        float acc = 1.f;
        for (int u = s0 + 4; u <= t; ++u) acc *= sh.gs[u];
        r[3] = acc;
        r[2] = s0 + 3 <= t ? r[3] * sh.gs[s0 + 3] : 1.f;
        r[1] = s0 + 2 <= t ? r[2] * sh.gs[s0 + 2] : 1.f;
        r[0] = s0 + 1 <= t ? r[1] * sh.gs[s0 + 1] : 1.f;
        float av[4], pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = s0 + e;
            av[e] = s < t ? sh.bs[t] * r[e] * sh.kk[t][s] : 0.f;
            pv[e] = s <= t ? r[e] * sh.qk[t][s] : 0.f;
        }
        *reinterpret_cast<float4*>(&sh.a[t][s0]) = make_float4(av[0], av[1], av[2], av[3]);
        *reinterpret_cast<float4*>(P + ((int64_t)unit * CK + t) * CK + s0) = make_float4(pv[0], pv[1], pv[2], pv[3]);
        if (s0 == 0) {
            const float gm = sh.gs[0] * r[0];     // gamma_t = g_0 R[t][0]
            sh.gm[t] = gm;
            Gm[(int64_t)unit * CK + t] = gm;
        }
        if (t == CK - 1) *reinterpret_cast<float4*>(Rho + (int64_t)unit * CK + s0) = make_float4(r[0], r[1], r[2], r[3]);
    }
    __syncthreads();

    // 4. forward substitution (I + A) X = RHS, one column per thread:
    //    columns 0..DK-1: RHS = beta gamma k (-> W); DK..DK+CK-1: RHS = e_j (-> T).
    //    Each row is written out as soon as it is known; the scheduling
    //    barrier per row keeps the row's operands from being hoisted (the live
    //    set stays at the 32 solved values).
    if (tid < DK + CK) {
        const int j = tid;
        const bool wcol = j < DK;
        const float bj = wcol ? 0.f : sh.bs[j - DK];
        float* dst = wcol ? W + (int64_t)unit * CK * DK + j : Tb + (int64_t)unit * CK * CK + (j - DK);
        const int stride = wcol ? DK : CK;
        float x[CK];
#pragma unroll
        for (int t = 0; t < CK; ++t) {
            const float rhs = wcol ? sh.bs[t] * sh.gm[t] * bf16lo(sh.kb[t][j]) : (t == j - DK ? 1.f : 0.f);
            float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
            for (int s4 = 0; s4 < t; s4 += 4) {
                const float4 a4 = *reinterpret_cast<const float4*>(&sh.a[t][s4]);
                acc0 = fmaf(a4.x, x[s4], acc0);
                if (s4 + 1 < t) acc1 = fmaf(a4.y, x[s4 + 1], acc1);
                if (s4 + 2 < t) acc0 = fmaf(a4.z, x[s4 + 2], acc0);
                if (s4 + 3 < t) acc1 = fmaf(a4.w, x[s4 + 3], acc1);
            }
            x[t] = rhs - (acc0 + acc1);
            dst[t * stride] = wcol ? x[t] : x[t] * bj;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// ============================================================ sequential pass

template <int DK>
struct SeqBuf {
    float w[CK][DK + 4];         // W rows (f32)
    uint16_t qb[CK][DK + 8];     // q rows (bf16)
    uint16_t kb[CK][DK + 16];    // k rows (bf16); a 72-word stride keeps the
                                 // 16-bit column gathers of two rows apart
    uint16_t vt[RB][CK + 8];     // v slice transposed: vt[r][s] (bf16)
    float tb[CK][CK + 4];        // T diag(beta)
    float p[CK][CK + 4];         // P
    float gm[CK], rho[CK];
};

template <int DK>
struct SeqCfg {
    static constexpr int YSTEPS = 1024;    // y rows buffered in LDS before a flush
    static constexpr int W4 = CK * DK / 4 / 256;     // float4 of W per thread
    static constexpr int Q8 = CK * DK / 8 / 256;     // uint4 of q (and of k) per thread
    static_assert(CK * DK / 8 % 256 == 0, "whole vectors per thread");
};

template <int DK>
struct SeqSmem {
    SeqBuf<DK> buf[2];
    float s[RB][DK + 4];         // S_0 of the chunk, row-major (B operand source)
    float dt[RB][CK + 4];        // Delta^T
    float rds[CK][RB];           // diag(rho) Delta, row-major [s][r]
    uint16_t y[SeqCfg<DK>::YSTEPS][RB];
};

typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

// Global -> register staging of one chunk (native vector types, so the
// compiler keeps every element in VGPRs).
template <int DK>
struct SeqStage {
    using SC = SeqCfg<DK>;
    f4_t w[SC::W4];
    u4_t qv[SC::Q8], kv[SC::Q8];
    u4_t vv;
    f4_t tbv, pv;
    float gr;

    __device__ __forceinline__ void load(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                         const uint16_t* __restrict__ v, const float* __restrict__ W,
                                         const float* __restrict__ Tb, const float* __restrict__ P,
                                         const float* __restrict__ Gm, const float* __restrict__ Rho,
                                         int64_t unit, int b, int hk, int hv, int r0, int t0, int T, int Hk,
                                         int Hv, int Dv, int tid) {
        const f4_t* wsrc = reinterpret_cast<const f4_t*>(W + unit * CK * DK);
#pragma unroll
        for (int i = 0; i < SC::W4; ++i) w[i] = wsrc[tid + 256 * i];
#pragma unroll
        for (int i = 0; i < SC::Q8; ++i) {
            const int idx = tid + 256 * i;
            const int t = min(t0 + idx / (DK / 8), T - 1);
            const int64_t off = (((int64_t)b * T + t) * Hk + hk) * DK + (idx % (DK / 8)) * 8;
            qv[i] = *reinterpret_cast<const u4_t*>(q + off);
            kv[i] = *reinterpret_cast<const u4_t*>(k + off);
        }
        {
            // v slice: CK steps x RB rows = 64 vectors of 8 (threads 0..63)
            const int idx = tid & 63;
            const int t = min(t0 + idx / (RB / 8), T - 1);
            vv = *reinterpret_cast<const u4_t*>(v + (((int64_t)b * T + t) * Hv + hv) * Dv + r0 +
                                                 (idx % (RB / 8)) * 8);
        }
        tbv = reinterpret_cast<const f4_t*>(Tb + unit * CK * CK)[tid];
        pv = reinterpret_cast<const f4_t*>(P + unit * CK * CK)[tid];
        gr = tid < CK ? Gm[unit * CK + tid] : Rho[unit * CK + (tid & (CK - 1))];
    }

    __device__ __forceinline__ void store(SeqBuf<DK>& sb, int tid) const {
#pragma unroll
        for (int i = 0; i < SC::W4; ++i) {
            const int idx = tid + 256 * i;
            *reinterpret_cast<f4_t*>(&sb.w[idx / (DK / 4)][(idx % (DK / 4)) * 4]) = w[i];
        }
#pragma unroll
        for (int i = 0; i < SC::Q8; ++i) {
            const int idx = tid + 256 * i;
            const int t = idx / (DK / 8), c8 = idx % (DK / 8);
            *reinterpret_cast<u4_t*>(&sb.qb[t][c8 * 8]) = qv[i];
            *reinterpret_cast<u4_t*>(&sb.kb[t][c8 * 8]) = kv[i];
        }
        if (tid < 64) {
            const int t = tid / (RB / 8), r8 = (tid % (RB / 8)) * 8;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sb.vt[r8 + 2 * e][t] = (uint16_t)(vv[e] & 0xFFFFu);
                sb.vt[r8 + 2 * e + 1][t] = (uint16_t)(vv[e] >> 16);
            }
        }
        *reinterpret_cast<f4_t*>(&sb.tb[tid / (CK / 4)][(tid % (CK / 4)) * 4]) = tbv;
        *reinterpret_cast<f4_t*>(&sb.p[tid / (CK / 4)][(tid % (CK / 4)) * 4]) = pv;
        if (tid < CK) sb.gm[tid] = gr;
        else if (tid < 2 * CK) sb.rho[tid - CK] = gr;
    }
};

// 8 consecutive floats (two float4 reads)
__device__ __forceinline__ void ld8(const float* p, float* o) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// 8 consecutive bf16 -> floats
__device__ __forceinline__ void ld8h(const uint16_t* p, float* o) {
    unpack8(*reinterpret_cast<const uint4*>(p), o);
}

template <int DK>
__global__ __launch_bounds__(256) void chunk_seq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ W, const float* __restrict__ Tb, const float* __restrict__ P,
    const float* __restrict__ Gm, const float* __restrict__ Rho,
    const float* state_in, float* state_out, uint16_t* __restrict__ y,
    int T, int Hk, int Hv, int Dv, int NC, int row_blocks, int n_blocks) {
    using SC = SeqCfg<DK>;
    __shared__ SeqSmem<DK> sh;

    int lb = blockIdx.x;
    if ((n_blocks & 7) == 0) lb = (lb & 7) * (n_blocks >> 3) + (lb >> 3);
    const int n = lb / row_blocks;
    const int rblk = lb % row_blocks;
    const int b = n / Hv, hv = n % Hv;
    const int hk = hv / (Hv / Hk);
    const int r0 = rblk * RB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15;            // MFMA lane position (row / column in tile)
    const int lq = lane >> 4;            // MFMA lane quarter

    // S slice in accumulator layout: wave w owns columns [32w, 32w+32) as two
    // 16x16 tiles; tile dt, register i -> S[r = 4 lq + i][d = 16 dt + lr]
    f4_t S[2];
    const int64_t sbase = ((int64_t)n * Dv + r0) * DK;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = 32 * wave + 16 * tt + lr;
            S[tt][i] = state_in ? state_in[sbase + (4 * lq + i) * DK + d] : 0.f;
        }

    const int64_t unit0 = (int64_t)n * NC;
    SeqStage<DK> st;
    st.load(q, k, v, W, Tb, P, Gm, Rho, unit0, b, hk, hv, r0, 0, T, Hk, Hv, Dv, tid);
    st.store(sh.buf[0], tid);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sh.s[4 * lq + i][32 * wave + 16 * tt + lr] = S[tt][i];
    __syncthreads();

    int ybase = 0;
    for (int c = 0; c < NC; ++c) {
        const SeqBuf<DK>& cb = sh.buf[c & 1];
        const int t0 = c * CK;
        // next chunk (the last chunk reloads itself into the idle buffer,
        // which is never read again: no conditional load path)
        const int cn = min(c + 1, NC - 1);
        st.load(q, k, v, W, Tb, P, Gm, Rho, unit0 + cn, b, hk, hv, r0, cn * CK, T, Hk, Hv, Dv, tid);

        // ---- phase 1: wave 0/1 -> X = W S_0^T rows of m-tile w, then U, Delta
        //               wave 2/3 -> Y' = Q S_0^T rows of m-tile w-2, scaled by gamma
        const int mt = wave & 1;
        f4_t acc;
        {
            // two independent accumulation chains over the Dk blocks
            f4_t a2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                const int d0 = 32 * kb + 8 * lq;
                float bv[8], av[8];
                ld8(&sh.s[lr][d0], bv);
                if (wave < 2) ld8(&cb.w[16 * mt + lr][d0], av);
                else ld8h(&cb.qb[16 * mt + lr][d0], av);
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) a2[kb & 1] = mfma4(av[ks], bv[ks], a2[kb & 1]);
            }
            acc = a2[0] + a2[1];
        }
        if (wave < 2) {
            // U = Tb V for this m-tile: k index s = 8 lq + ks
            f4_t u = {0.f, 0.f, 0.f, 0.f};
            float av[8], bv[8];
            ld8(&cb.tb[16 * mt + lr][8 * lq], av);
            ld8h(&cb.vt[lr][8 * lq], bv);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) u = mfma4(av[ks], bv[ks], u);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * mt + 4 * lq + i;     // row of Delta (step)
                const float dlt = u[i] - acc[i];
                sh.dt[lr][t] = dlt;
                sh.rds[t][lr] = cb.rho[t] * dlt;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] *= cb.gm[16 * mt + 4 * lq + i];
        }
        __syncthreads();

        // ---- phase 2: Y = gamma Y' + P Delta (waves 2/3), S update (all)
        if (wave >= 2) {
            float av[8], bv[8];
            ld8(&cb.p[16 * mt + lr][8 * lq], av);
            ld8(&sh.dt[lr][8 * lq], bv);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) acc = mfma4(av[ks], bv[ks], acc);
            const int yoff = t0 - ybase;
#pragma unroll
            for (int i = 0; i < 4; ++i) sh.y[yoff + 16 * mt + 4 * lq + i][lr] = (uint16_t)f32_to_bf16(acc[i]);
        }
        {
            // S = gamma_C S + (diag(rho) Delta)^T K; k index s = lq + 4 ks:
            // A = rds[s][r = lr], B = k[s][d = 16 dt + lr] (16-bit gathers)
            const float gC = cb.gm[CK - 1];
            f4_t sn[2] = {S[0] * gC, S[1] * gC};
#pragma unroll
            for (int ks = 0; ks < CK / 4; ++ks) {
                const int srow = lq + 4 * ks;
                const float av = sh.rds[srow][lr];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const float bv = __uint_as_float((uint32_t)cb.kb[srow][32 * wave + 16 * tt + lr] << 16);
                    sn[tt] = mfma4(av, bv, sn[tt]);
                }
            }
            S[0] = sn[0];
            S[1] = sn[1];
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sh.s[4 * lq + i][32 * wave + 16 * tt + lr] = S[tt][i];
        st.store(sh.buf[(c + 1) & 1], tid);
        __syncthreads();

        const bool last = c + 1 == NC;
        if (last || t0 + CK - ybase == SC::YSTEPS) {
            // flush y rows [ybase, t0 + CK): RB bf16 per step, two 16-byte vectors
            const int nsteps = t0 + CK - ybase;
            for (int idx = tid; idx < nsteps * (RB / 8); idx += 256) {
                const int s = idx / (RB / 8), part = idx % (RB / 8);
                const int t = ybase + s;
                if (t < T)
                    *reinterpret_cast<uint4*>(y + (((int64_t)b * T + t) * Hv + hv) * Dv + r0 + part * 8) =
                        *reinterpret_cast<const uint4*>(&sh.y[s][part * 8]);
            }
            ybase = t0 + CK;
            // the next chunk writes sh.y only after its first barrier
        }
    }

#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            state_out[sbase + (4 * lq + i) * DK + 32 * wave + 16 * tt + lr] = S[tt][i];
}

// ================================================================== launch

bool chunked_supported(int Dk, int Dv) { return Dk == 128 && Dv % RB == 0; }

ChunkedLayout chunked_layout(int B, int T, int Hv, int Dk) {
    ChunkedLayout L;
    const int64_t NC = (T + CK - 1) / CK;
    const int64_t units = (int64_t)B * Hv * NC;
    auto a256 = [](uint64_t x) { return (x + 255) & ~uint64_t(255); };
    L.nc = (int)NC;
    L.w = 0;
    L.tb = L.w + a256(units * CK * Dk * 4);
    L.p = L.tb + a256(units * CK * CK * 4);
    L.gm = L.p + a256(units * CK * CK * 4);
    L.rho = L.gm + a256(units * CK * 4);
    L.total = L.rho + a256(units * CK * 4);
    return L;
}

int64_t chunked_blocks(int B, int T, int Hv, int Dv) {
    const int64_t NC = (T + CK - 1) / CK;
    return std::max<int64_t>((int64_t)B * Hv * NC, (int64_t)B * Hv * (Dv / RB));
}

hipError_t launch_recurrent_chunked(const RecurrentArgs& a, void* ws, hipStream_t stream) {
    if (!chunked_supported(a.Dk, a.Dv) || a.T <= 0 || a.B <= 0) return hipErrorInvalidValue;
    const ChunkedLayout L = chunked_layout(a.B, a.T, a.Hv, a.Dk);
    char* base = static_cast<char*>(ws);
    float* W = reinterpret_cast<float*>(base + L.w);
    float* Tb = reinterpret_cast<float*>(base + L.tb);
    float* P = reinterpret_cast<float*>(base + L.p);
    float* Gm = reinterpret_cast<float*>(base + L.gm);
    float* Rho = reinterpret_cast<float*>(base + L.rho);
    const int64_t units = (int64_t)a.B * a.Hv * L.nc;
    hipLaunchKernelGGL((chunk_prep_kernel<128>), dim3((unsigned)units), dim3(256), 0, stream, a.q, a.k, a.g,
                       a.beta, W, Tb, P, Gm, Rho, a.T, a.Hk, a.Hv, L.nc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int row_blocks = a.Dv / RB;
    const int64_t blocks = (int64_t)a.B * a.Hv * row_blocks;
    hipLaunchKernelGGL((chunk_seq_kernel<128>), dim3((unsigned)blocks), dim3(256), 0, stream, a.q, a.k, a.v, W,
                       Tb, P, Gm, Rho, a.state_in, a.state_out, a.y, a.T, a.Hk, a.Hv, a.Dv, L.nc, row_blocks,
                       (int)blocks);
    return hipGetLastError();
}

}  // namespace gdn
