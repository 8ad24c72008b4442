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
//   W       = T diag(beta gamma) K,  Tb = T diag(beta)
// unrolling the recurrence inside the chunk gives, as matrices over the chunk,
//   Delta = Tb V - W S_0^T                                       [C x Dv]
//   Y     = diag(gamma) Q S_0^T  +  P Delta,  P[t][s] = R[t][s] (q_t . k_s), s <= t
//   S_C   = gamma_{C-1} S_0  +  (diag(rho) Delta)^T K
// (Delta's rows are the deltas of the steps, Y's rows the outputs).  This is
// the same arithmetic as the per-step loop up to rounding order: dense
// products replace the per-step dot products.
//
// fp32 products on bf16 matrix cores.  Every f32 operand x is cut into three
// bf16 planes x = h + m + l exactly (h is x truncated to bf16, m and l the
// same on the remainders), so that a product of an f32 matrix with an exact
// bf16 matrix (q, k, v) is three bf16 MFMAs with f32 accumulation, and a
// product of two f32 matrices is the six plane products down to 2^-16 of the
// leading one (the three dropped terms are below 2^-24 relative).
//
// Operand layout.  In a 16x16x32 bf16 MFMA lane l (r = l % 16, q = l / 16)
// holds eight values of row r of A and of column r of B along the contraction
// index.  Every 32-long contraction here assigns index kperm(q, e) to
// element e of quarter q, kperm(q, e) = 4q + e (e < 4), 16 + 4q + (e - 4)
// (e >= 4).  Then the accumulators of two stacked 16x16 tiles (lane l holds
// rows 4q..4q+3 of column r of each) are, element for element, the operand of
// the next product: the state and the chunk's deltas never leave registers.
//
// Two kernels:
//  * chunk_prep_kernel, one block per (b, hv, chunk), independent of the
//    state: k k^T and q k^T on bf16 MFMA, the decay ratios as direct products
//    (never quotients of cumulative decays, so underflow to zero is
//    harmless), and the unit lower-triangular solve by forward substitution
//    for W and T.  It writes W, -Tb and -P as bf16 planes, q and k (bf16) and
//    gamma, -rho, each already in the register layout of the sequential pass.
//  * chunk_seq_kernel, one block per (b, hv, 16 state rows), walks the chunks
//    in order.  Wave w holds state columns [32w, 32w + 32) of its 16 rows in
//    MFMA accumulators.  Per chunk each wave forms its share of
//    W S_0^T - Tb V and of Q S_0^T over its columns, the four shares are summed
//    through LDS (the only exchange, one barrier per chunk), and every wave
//    then updates its state columns; two waves finish Y.
// Padding steps past T carry g = 1, beta = 0 and zero k, q: their Delta is 0
// and they leave S unchanged.
#include <algorithm>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));

constexpr int CK = 32;        // chunk length
constexpr int RB = 16;        // state rows per sequential block
constexpr int DKC = 128;      // key head size of the chunked form
constexpr int NW = DKC / 32;  // waves per sequential block (32 state columns each)

// Per-unit sizes of the workspace arrays, in 16-byte vectors (one per lane).
constexpr int kWVec = NW * 2 * 3 * 64;    // W planes       [NW][t-tile][plane][lane]
constexpr int kTVec = 2 * 3 * 64;         // -Tb, -P planes [t-tile][plane][lane]
constexpr int kQVec = NW * 2 * 64;        // q, k per k-unit [NW][tile][lane]

// ------------------------------------------------------------ bf16 planes

struct Planes {
    u4_t h, m, l;
};

// upper halves of a and b packed (a in the low half)
__device__ __forceinline__ uint32_t top16x2(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// x minus x truncated to bf16 (exact)
__device__ __forceinline__ float rest16(float x) { return x - __uint_as_float(__float_as_uint(x) & 0xFFFF0000u); }

struct Split2 {
    uint32_t h, m, l;    // bf16 pairs of each plane
};

__device__ __forceinline__ Split2 split2(float a, float b) {
    Split2 r;
    r.h = top16x2(__float_as_uint(a), __float_as_uint(b));
    const float a1 = rest16(a), b1 = rest16(b);
    r.m = top16x2(__float_as_uint(a1), __float_as_uint(b1));
    r.l = top16x2(__float_as_uint(rest16(a1)), __float_as_uint(rest16(b1)));
    return r;
}

// eight f32 (x0 then x1) -> three bf16 planes
__device__ __forceinline__ Planes split8(const f4_t x0, const f4_t x1) {
    const Split2 s0 = split2(x0[0], x0[1]), s1 = split2(x0[2], x0[3]);
    const Split2 s2 = split2(x1[0], x1[1]), s3 = split2(x1[2], x1[3]);
    Planes p;
    p.h = u4_t{s0.h, s1.h, s2.h, s3.h};
    p.m = u4_t{s0.m, s1.m, s2.m, s3.m};
    p.l = u4_t{s0.l, s1.l, s2.l, s3.l};
    return p;
}

__device__ __forceinline__ f4_t mma(u4_t a, u4_t b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8_t, a), __builtin_bit_cast(bf8_t, b), c,
                                                   0, 0, 0);
}

// f32 (planes) x exact bf16, smallest term first
__device__ __forceinline__ f4_t mma3a(const Planes& a, u4_t b, f4_t c) {
    c = mma(a.l, b, c);
    c = mma(a.m, b, c);
    return mma(a.h, b, c);
}
__device__ __forceinline__ f4_t mma3b(u4_t a, const Planes& b, f4_t c) {
    c = mma(a, b.l, c);
    c = mma(a, b.m, c);
    return mma(a, b.h, c);
}

// ========================================================= chunk preparation

struct PrepSmem {
    uint16_t kb[CK][DKC + 8];    // bf16 rows, padded against bank conflicts
    union {
        struct {
            uint16_t qb[CK][DKC + 8];
            float kk[CK][CK + 1];
            float qk[CK][CK + 1];
        } in;
        float w[CK][DKC + 4];    // solved W (the inputs above are dead by then)
    } u;
    float a[CK][CK + 4];         // strictly lower A (row-major, 16-byte rows)
    float tn[CK][CK + 4];        // -T diag(beta)
    float gs[CK], bs[CK], gm[CK];
};

struct ChunkPtrs {
    u4_t* wsw;      // W planes
    u4_t* tbn;      // -Tb planes
    u4_t* pn;       // -P planes
    float* gm;      // gamma_t
    float* rhon;    // -rho in kperm order
    u4_t* qsw;      // q rows
    u4_t* ksw;      // k columns
};

__global__ __launch_bounds__(256, 4) void chunk_prep_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const float* __restrict__ g,
                                                            const float* __restrict__ beta, ChunkPtrs o, int T,
                                                            int Hk, int Hv, int NC) {
    __shared__ PrepSmem sh;
    const int64_t unit = blockIdx.x;          // (b * Hv + hv) * NC + c
    const int c = (int)(unit % NC);
    const int n = (int)(unit / NC);
    const int b = n / Hv, hv = n % Hv;
    const int G = Hv / Hk;
    const int hk = hv / G;
    const int64_t kunit = ((int64_t)b * Hk + hk) * NC + c;
    const int t0 = c * CK;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // 1. k, q rows of the chunk (zero past T), g and beta (1 and 0 past T)
    for (int idx = tid; idx < CK * DKC / 8; idx += 256) {
        const int t = idx / (DKC / 8), c8 = idx % (DKC / 8);
        uint4 kv = make_uint4(0, 0, 0, 0), qv = kv;
        if (t0 + t < T) {
            const int64_t off = (((int64_t)b * T + t0 + t) * Hk + hk) * DKC + c8 * 8;
            kv = *reinterpret_cast<const uint4*>(k + off);
            qv = *reinterpret_cast<const uint4*>(q + off);
        }
        *reinterpret_cast<uint4*>(&sh.kb[t][c8 * 8]) = kv;
        *reinterpret_cast<uint4*>(&sh.u.in.qb[t][c8 * 8]) = qv;
    }
    if (tid < CK) {
        const int t = t0 + tid;
        const int64_t i = ((int64_t)b * T + min(t, T - 1)) * Hv + hv;
        const float gv = g[i], bv = beta[i];
        sh.gs[tid] = t < T ? gv : 1.f;
        sh.bs[tid] = t < T ? bv : 0.f;
    }
    __syncthreads();

    // 2a. q and k in operand layout, once per k-head (the first v-head of
    //     each group writes them): q rows 16j + r at columns 32w + kperm(q, e);
    //     k rows kperm(q, e) at column 32w + 16tt + r
    if (hv % G == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int slot = tid + 256 * i;
            const int w = slot >> 7, jt = (slot >> 6) & 1, l = slot & 63;
            const int r = l & 15, q4 = l >> 4;
            const u2_t lo = *reinterpret_cast<const u2_t*>(&sh.u.in.qb[16 * jt + r][32 * w + 4 * q4]);
            const u2_t hi = *reinterpret_cast<const u2_t*>(&sh.u.in.qb[16 * jt + r][32 * w + 16 + 4 * q4]);
            o.qsw[kunit * kQVec + slot] = u4_t{lo[0], lo[1], hi[0], hi[1]};
            const int d = 32 * w + 16 * jt + r;
            u4_t kv;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int s0 = p < 2 ? 4 * q4 + 2 * p : 16 + 4 * q4 + 2 * (p - 2);
                kv[p] = (uint32_t)sh.kb[s0][d] | ((uint32_t)sh.kb[s0 + 1][d] << 16);
            }
            o.ksw[kunit * kQVec + slot] = kv;
        }
    }

    // 2b. k k^T and q k^T, 32 x 32 each: wave w owns output tile (w / 2, w % 2)
    {
        const int mi = wave >> 1, ni = wave & 1;
        f4_t ckk = {0.f, 0.f, 0.f, 0.f}, cqk = ckk;
#pragma unroll
        for (int ks = 0; ks < DKC / 32; ++ks) {
            const int col = ks * 32 + 8 * (lane >> 4);
            const u4_t ka = *reinterpret_cast<const u4_t*>(&sh.kb[16 * mi + (lane & 15)][col]);
            const u4_t qa = *reinterpret_cast<const u4_t*>(&sh.u.in.qb[16 * mi + (lane & 15)][col]);
            const u4_t kb = *reinterpret_cast<const u4_t*>(&sh.kb[16 * ni + (lane & 15)][col]);
            ckk = mma(ka, kb, ckk);
            cqk = mma(qa, kb, cqk);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sh.u.in.kk[16 * mi + 4 * (lane >> 4) + i][16 * ni + (lane & 15)] = ckk[i];
            sh.u.in.qk[16 * mi + 4 * (lane >> 4) + i][16 * ni + (lane & 15)] = cqk[i];
        }
    }
    __syncthreads();

    // 3. decay ratios R[t][s] = g_{s+1}...g_t (s <= t) for s in this thread's
    //    four columns, then A, -P (planes), gamma, -rho
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
            av[e] = s < t ? sh.bs[t] * r[e] * sh.u.in.kk[t][s] : 0.f;
            pv[e] = s <= t ? -(r[e] * sh.u.in.qk[t][s]) : 0.f;
        }
        *reinterpret_cast<float4*>(&sh.a[t][s0]) = make_float4(av[0], av[1], av[2], av[3]);
        // these four columns are elements 4 half .. 4 half + 3 of quarter q4
        const int half = s0 >> 4, q4 = (s0 & 15) >> 2;
        const int l = 16 * q4 + (t & 15), jt = t >> 4;
        const Split2 p0 = split2(pv[0], pv[1]), p1 = split2(pv[2], pv[3]);
        u2_t* pdst = reinterpret_cast<u2_t*>(o.pn + unit * kTVec + (jt * 3) * 64 + l) + half;
        pdst[0] = u2_t{p0.h, p1.h};
        pdst[2 * 64] = u2_t{p0.m, p1.m};
        pdst[4 * 64] = u2_t{p0.l, p1.l};
        if (s0 == 0) {
            const float gm = sh.gs[0] * r[0];     // gamma_t = g_0 R[t][0]
            sh.gm[t] = gm;
            o.gm[unit * CK + t] = gm;
        }
        if (t == CK - 1)
            *reinterpret_cast<float4*>(o.rhon + unit * CK + 8 * q4 + 4 * half) = make_float4(-r[0], -r[1], -r[2], -r[3]);
    }
    __syncthreads();

    // 4. forward substitution (I + A) X = RHS, one column per thread:
    //    columns 0..DK-1: RHS = beta gamma k (-> W); DK..DK+CK-1: RHS = e_j (-> T).
    //    Each row goes to LDS as soon as it is known; the scheduling barrier
    //    per row keeps the row's operands from being hoisted (the live set
    //    stays at the 32 solved values).
    if (tid < DKC + CK) {
        const int j = tid;
        const bool wcol = j < DKC;
        const float nbj = wcol ? 0.f : -sh.bs[j - DKC];
        float x[CK];
#pragma unroll
        for (int t = 0; t < CK; ++t) {
            const float rhs = wcol ? sh.bs[t] * sh.gm[t] * bf16lo(sh.kb[t][j]) : (t == j - DKC ? 1.f : 0.f);
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
            if (wcol) sh.u.w[t][j] = x[t];
            else sh.tn[t][j - DKC] = x[t] * nbj;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();

    // 5. W planes (rows 16j + r, columns 32w + kperm(q, e)) and -Tb planes
    //    (rows 16j + r, columns 8q + e)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int slot = tid + 256 * i;
        const int w = slot >> 7, jt = (slot >> 6) & 1, l = slot & 63;
        const int row = 16 * jt + (l & 15), q4 = l >> 4;
        const f4_t x0 = *reinterpret_cast<const f4_t*>(&sh.u.w[row][32 * w + 4 * q4]);
        const f4_t x1 = *reinterpret_cast<const f4_t*>(&sh.u.w[row][32 * w + 16 + 4 * q4]);
        const Planes p = split8(x0, x1);
        u4_t* dst = o.wsw + unit * kWVec + ((w * 2 + jt) * 3) * 64 + l;
        dst[0] = p.h;
        dst[64] = p.m;
        dst[128] = p.l;
    }
    if (tid < 128) {
        const int jt = tid >> 6, l = tid & 63;
        const int row = 16 * jt + (l & 15), q4 = l >> 4;
        const f4_t x0 = *reinterpret_cast<const f4_t*>(&sh.tn[row][8 * q4]);
        const f4_t x1 = *reinterpret_cast<const f4_t*>(&sh.tn[row][8 * q4 + 4]);
        const Planes p = split8(x0, x1);
        u4_t* dst = o.tbn + unit * kTVec + (jt * 3) * 64 + l;
        dst[0] = p.h;
        dst[64] = p.m;
        dst[128] = p.l;
    }
}

// ============================================================ sequential pass

struct SeqIn {
    const u4_t* wsw;
    const u4_t* tbn;
    const u4_t* pn;
    const float* gm;
    const float* rhon;
    const u4_t* qsw;
    const u4_t* ksw;
    const uint16_t* v;
};

// Per-block constants of the sequential pass.  `wv` is the wave index held
// in a scalar register, so role branches and address arithmetic stay scalar.
struct SeqCtx {
    int64_t unit0, kunit0;      // first chunk of this (b, hv) and of its (b, hk)
    const uint16_t* v0;         // &v[b][0][hv][r0]
    int64_t vstride;            // Hv * Dv (one step of v and y)
    uint32_t voff;              // lane offset of V[8q][r] from a chunk's first row
    int T, wv, lane;
};

// One chunk's operands in registers (two sets alternate: one chunk ahead).
struct SeqOps {
    Planes w[2];      // W, t-tiles 0 and 1
    u4_t q[2];        // q, t-tiles 0 and 1
    u4_t k[2];        // k^T, this wave's two column tiles
    Planes tp;        // waves 0, 1: -Tb of t-tile `wave`; waves 2, 3: -P of t-tile `wave - 2`
    uint32_t vr[8];   // waves 0, 1: V[8q + e][r] (bf16 bits, packed where used)
    f4_t rho[2];      // -rho[kperm(q, e)]
    float gt;         // gamma_t, t = 16 (wave & 1) + r
    float gc;         // gamma_{C-1}

    __device__ __forceinline__ void load(const SeqIn& in, const SeqCtx& x, int c) {
        const int64_t unit = x.unit0 + c, kunit = x.kunit0 + c;
        const int wv = x.wv, lane = x.lane;
        const u4_t* ws = in.wsw + unit * kWVec + wv * 6 * 64;
        w[0].h = ws[lane];
        w[0].m = ws[64 + lane];
        w[0].l = ws[128 + lane];
        w[1].h = ws[192 + lane];
        w[1].m = ws[256 + lane];
        w[1].l = ws[320 + lane];
        const u4_t* qs = in.qsw + kunit * kQVec + wv * 2 * 64;
        const u4_t* ks = in.ksw + kunit * kQVec + wv * 2 * 64;
        q[0] = qs[lane];
        q[1] = qs[64 + lane];
        k[0] = ks[lane];
        k[1] = ks[64 + lane];
        const u4_t* ts = (wv < 2 ? in.tbn : in.pn) + unit * kTVec + (wv & 1) * 3 * 64;
        tp.h = ts[lane];
        tp.m = ts[64 + lane];
        tp.l = ts[128 + lane];
        const f4_t* rs = reinterpret_cast<const f4_t*>(in.rhon + unit * CK) + 2 * (lane >> 4);
        rho[0] = rs[0];
        rho[1] = rs[1];
        gt = in.gm[unit * CK + 16 * (wv & 1) + (lane & 15)];
        gc = in.gm[unit * CK + CK - 1];
        if (wv < 2) {
            // V[t0 + 8q + e][r]; in the last chunk steps past T read step
            // T-1 instead (their column of Tb is zero)
            const int t0 = c * CK;
            const uint16_t* vb = x.v0 + (int64_t)t0 * x.vstride;
            if (t0 + CK <= x.T) {
#pragma unroll
                for (int e = 0; e < 8; ++e) vr[e] = vb[e * x.vstride + x.voff];
            } else {
                const int lim = x.T - 1 - t0;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    vr[e] = vb[(int64_t)min(8 * (lane >> 4) + e, lim) * x.vstride + (lane & 15)];
            }
        }
    }
};

struct SeqSmem {
    f4_t x[2][NW * 2 * 64];   // per-wave shares of W S^T - Tb V, double-buffered by chunk parity
    f4_t y[2][NW * 2 * 64];   // per-wave shares of S Q^T (transposed Y')
};

__global__ __launch_bounds__(256) void chunk_seq_kernel(SeqIn in, const float* state_in, float* state_out,
                                                        uint16_t* __restrict__ y, int T, int Hk, int Hv, int Dv,
                                                        int NC, int row_blocks, int n_blocks) {
    __shared__ SeqSmem sh;

    int lb = blockIdx.x;
    if ((n_blocks & 7) == 0) lb = (lb & 7) * (n_blocks >> 3) + (lb >> 3);
    const int n = lb / row_blocks;
    const int rblk = lb % row_blocks;
    const int b = n / Hv, hv = n % Hv;
    const int hk = hv / (Hv / Hk);
    const int r0 = rblk * RB;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lq = lane >> 4;
    const f4_t zero = {0.f, 0.f, 0.f, 0.f};

    SeqCtx x;
    x.unit0 = (int64_t)n * NC;
    x.kunit0 = ((int64_t)b * Hk + hk) * NC;
    x.vstride = (int64_t)Hv * Dv;
    x.v0 = in.v + ((int64_t)b * T * Hv + hv) * Dv + r0;
    x.voff = (uint32_t)(8 * lq * x.vstride + lr);
    x.T = T;
    x.wv = wv;
    x.lane = lane;

    // state tile tt, register i: S[r0 + lr][32 wv + 16 tt + 4 lq + i]
    f4_t S[2];
    float* sp_out = state_out + ((int64_t)n * Dv + r0) * DKC + 32 * wv;
    const uint32_t soff = lr * DKC + 4 * lq;
    if (state_in) {
        const float* sp = state_in + ((int64_t)n * Dv + r0) * DKC + 32 * wv;
        S[0] = *reinterpret_cast<const f4_t*>(sp + soff);
        S[1] = *reinterpret_cast<const f4_t*>(sp + soff + 16);
    } else {
        S[0] = zero;
        S[1] = zero;
    }

    // y rows of waves 2, 3: step 16 (wv & 1) + lr of the chunk, columns r0 + 4 lq ..
    uint16_t* y0 = y + ((int64_t)b * T * Hv + hv) * Dv + r0;
    const int yt = 16 * (wv & 1) + lr;
    const uint32_t yoff = (uint32_t)(yt * x.vstride + 4 * lq);

    auto step = [&](int c, const SeqOps& o) {
        // state planes: element e of quarter lq is column kperm(lq, e)
        const Planes s = split8(S[0], S[1]);

        // this wave's share of W S^T - Tb V (rows t, columns r), two t-tiles
        f4_t x0 = zero, x1 = zero;
        if (wv < 2) {
            const u4_t v = {o.vr[0] | (o.vr[1] << 16), o.vr[2] | (o.vr[3] << 16), o.vr[4] | (o.vr[5] << 16),
                            o.vr[6] | (o.vr[7] << 16)};
            if (wv == 0) x0 = mma3a(o.tp, v, x0);
            else x1 = mma3a(o.tp, v, x1);
        }
        x0 = mma(o.w[0].l, s.h, x0);
        x1 = mma(o.w[1].l, s.h, x1);
        x0 = mma(o.w[0].h, s.l, x0);
        x1 = mma(o.w[1].h, s.l, x1);
        x0 = mma(o.w[0].m, s.m, x0);
        x1 = mma(o.w[1].m, s.m, x1);
        x0 = mma(o.w[0].m, s.h, x0);
        x1 = mma(o.w[1].m, s.h, x1);
        x0 = mma(o.w[0].h, s.m, x0);
        x1 = mma(o.w[1].h, s.m, x1);
        x0 = mma(o.w[0].h, s.h, x0);
        x1 = mma(o.w[1].h, s.h, x1);

        // this wave's share of S Q^T (rows r, columns t)
        f4_t y0v = mma(s.l, o.q[0], zero);
        f4_t y1v = mma(s.l, o.q[1], zero);
        y0v = mma(s.m, o.q[0], y0v);
        y1v = mma(s.m, o.q[1], y1v);
        y0v = mma(s.h, o.q[0], y0v);
        y1v = mma(s.h, o.q[1], y1v);

        f4_t* xb = sh.x[c & 1];
        f4_t* yb = sh.y[c & 1];
        xb[(2 * wv) * 64 + lane] = x0;
        xb[(2 * wv + 1) * 64 + lane] = x1;
        yb[(2 * wv) * 64 + lane] = y0v;
        yb[(2 * wv + 1) * 64 + lane] = y1v;
        __syncthreads();

        // D = W S^T - Tb V = -Delta, summed in wave order (identical in every wave)
        const f4_t p00 = xb[0 * 64 + lane], p10 = xb[2 * 64 + lane], p20 = xb[4 * 64 + lane], p30 = xb[6 * 64 + lane];
        const f4_t p01 = xb[1 * 64 + lane], p11 = xb[3 * 64 + lane], p21 = xb[5 * 64 + lane], p31 = xb[7 * 64 + lane];
        const f4_t d0 = ((p00 + p10) + p20) + p30;
        const f4_t d1 = ((p01 + p11) + p21) + p31;

        // S = gamma_{C-1} S + K^T (diag(rho) Delta)
        const Planes bs = split8(o.rho[0] * d0, o.rho[1] * d1);
        S[0] = S[0] * o.gc;
        S[1] = S[1] * o.gc;
        S[0] = mma3b(o.k[0], bs, S[0]);
        S[1] = mma3b(o.k[1], bs, S[1]);

        if (wv >= 2) {
            // Y^T = gamma_t (S Q^T) + D^T (-P)^T for t-tile wv - 2
            const int jt = wv & 1;
            const f4_t q0 = yb[jt * 64 + lane], q1 = yb[(2 + jt) * 64 + lane];
            const f4_t q2 = yb[(4 + jt) * 64 + lane], q3 = yb[(6 + jt) * 64 + lane];
            f4_t ys = ((q0 + q1) + q2) + q3;
            ys = ys * o.gt;
            const Planes ds = split8(d0, d1);
            ys = mma(ds.l, o.tp.h, ys);
            ys = mma(ds.h, o.tp.l, ys);
            ys = mma(ds.m, o.tp.m, ys);
            ys = mma(ds.m, o.tp.h, ys);
            ys = mma(ds.h, o.tp.m, ys);
            ys = mma(ds.h, o.tp.h, ys);
            if (c * CK + yt < T)
                *reinterpret_cast<u2_t*>(y0 + (int64_t)c * CK * x.vstride + yoff) =
                    u2_t{pack_bf16x2(ys[0], ys[1]), pack_bf16x2(ys[2], ys[3])};
        }
    };

    SeqOps oa, ob;
    oa.load(in, x, 0);
    for (int c = 0; c < NC; c += 2) {
        ob.load(in, x, min(c + 1, NC - 1));
        step(c, oa);
        if (c + 1 >= NC) break;
        oa.load(in, x, min(c + 2, NC - 1));
        step(c + 1, ob);
    }

    *reinterpret_cast<f4_t*>(sp_out + soff) = S[0];
    *reinterpret_cast<f4_t*>(sp_out + soff + 16) = S[1];
}

// ================================================================== launch

// Lane offsets of v and y rows inside a chunk are 32-bit: Hv * Dv <= 2^25.
bool chunked_supported(int Hv, int Dk, int Dv) {
    return Dk == DKC && Dv % RB == 0 && (int64_t)Hv * Dv <= (int64_t(1) << 25);
}

ChunkedLayout chunked_layout(int B, int T, int Hk, int Hv, int Dk) {
    (void)Dk;
    ChunkedLayout L;
    const int64_t NC = (T + CK - 1) / CK;
    const uint64_t units = (uint64_t)B * Hv * NC;
    const uint64_t kunits = (uint64_t)B * Hk * NC;
    auto a256 = [](uint64_t x) { return (x + 255) & ~uint64_t(255); };
    L.nc = (int)NC;
    L.wsw = 0;
    L.tbn = L.wsw + a256(units * kWVec * 16);
    L.pn = L.tbn + a256(units * kTVec * 16);
    L.gm = L.pn + a256(units * kTVec * 16);
    L.rhon = L.gm + a256(units * CK * 4);
    L.qsw = L.rhon + a256(units * CK * 4);
    L.ksw = L.qsw + a256(kunits * kQVec * 16);
    L.total = L.ksw + a256(kunits * kQVec * 16);
    return L;
}

int64_t chunked_blocks(int B, int T, int Hv, int Dv) {
    const int64_t NC = (T + CK - 1) / CK;
    return std::max<int64_t>((int64_t)B * Hv * NC, (int64_t)B * Hv * (Dv / RB));
}

hipError_t launch_recurrent_chunked(const RecurrentArgs& a, void* ws, hipStream_t stream) {
    if (!chunked_supported(a.Hv, a.Dk, a.Dv) || a.T <= 0 || a.B <= 0) return hipErrorInvalidValue;
    const ChunkedLayout L = chunked_layout(a.B, a.T, a.Hk, a.Hv, a.Dk);
    char* base = static_cast<char*>(ws);
    ChunkPtrs o;
    o.wsw = reinterpret_cast<u4_t*>(base + L.wsw);
    o.tbn = reinterpret_cast<u4_t*>(base + L.tbn);
    o.pn = reinterpret_cast<u4_t*>(base + L.pn);
    o.gm = reinterpret_cast<float*>(base + L.gm);
    o.rhon = reinterpret_cast<float*>(base + L.rhon);
    o.qsw = reinterpret_cast<u4_t*>(base + L.qsw);
    o.ksw = reinterpret_cast<u4_t*>(base + L.ksw);
    const int64_t units = (int64_t)a.B * a.Hv * L.nc;
    hipLaunchKernelGGL(chunk_prep_kernel, dim3((unsigned)units), dim3(256), 0, stream, a.q, a.k, a.g, a.beta, o,
                       a.T, a.Hk, a.Hv, L.nc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    SeqIn in;
    in.wsw = o.wsw;
    in.tbn = o.tbn;
    in.pn = o.pn;
    in.gm = o.gm;
    in.rhon = o.rhon;
    in.qsw = o.qsw;
    in.ksw = o.ksw;
    in.v = a.v;
    const int row_blocks = a.Dv / RB;
    const int64_t blocks = (int64_t)a.B * a.Hv * row_blocks;
    hipLaunchKernelGGL(chunk_seq_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, a.state_in, a.state_out,
                       a.y, a.T, a.Hk, a.Hv, a.Dv, L.nc, row_blocks, (int)blocks);
    return hipGetLastError();
}

}  // namespace gdn
