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
// fp32 products on the matrix cores.  W S^T of the sequential pass and the
// per-key preparation's cross-quarter blocks run on the f32 matrix
// instruction (16x16x4, f32 in, f32 out).  The other products run on bf16
// MFMAs: every f32 operand x is cut into three
// bf16 planes x = h + m + l exactly (h is x rounded to bf16, m the remainder
// rounded, l what is left), so that a product of an f32 matrix with an exact
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
// Three kernels:
//  * chunk_prep_kernel, one block per (b, chunk) and one v-head or the two
//    v-heads of a pair sharing a k-head, independent of the state: k k^T and
//    q k^T on bf16 MFMA, the decay ratios as direct products (never
//    quotients of cumulative decays, so underflow to zero is harmless), and
//    the unit lower-triangular solve by forward substitution for W and T.
//    It writes W and -Tb V (f32), -P (two bf16 planes), q and k (bf16) and
//    gamma, -rho, each already in the register layout of the sequential pass.
//  * chunk_seq_kernel, one block per (b, hv, 16 or 32 state rows), walks the
//    chunks in order.  Wave w holds state columns [32w, 32w + 32) of its rows
//    in MFMA accumulators.  Per chunk each wave forms its share of
//    W S_0^T - Tb V and of Q S_0^T over its columns, the four shares are
//    summed through LDS (the only exchange, one barrier per chunk), and every
//    wave then updates its state columns; two waves finish Y.
//  * chunk_seq_pairs_kernel, for grids of more than two 16-row tiles per
//    CU: two waves per tile (one per half of the Dk columns) on one SIMD,
//    the chunk operands shared by four tiles through an LDS ring, the same
//    arithmetic in the same order.
// Padding steps past T and masked steps carry g = 1, beta = 0: their Delta is
// 0 and they leave S unchanged (a masked step's y is written as zero).
//
// Per-key gate (S <- S diag(g_t), g_t a vector over the key columns): the
// same algebra with every scalar decay turned into a column scaling,
//   A[t][s] = beta_t (k_t o R(t, s)) . k_s,   P[t][s] = (q_t o R(t, s)) . k_s,
//   W = T diag(beta) (K o Gamma),   Y = (Q o Gamma) S_0^T + P Delta,
//   S_C = S_0 diag(Gamma_{C-1}) + Delta^T (K o E),
// Gamma_t = g_0 o ... o g_t, E_t = g_{t+1} o ... o g_{C-1}; chunk_prep_kernel
// <0, 1, true> forms the ratios as running products inside each quarter
// chunk and as f32 products of prefix- and suffix-scaled rows across
// quarters, and chunk_seq_kernel <1, true> takes Q o Gamma, (K o E)^T and
// Gamma_{C-1} per v-head.
#include <algorithm>
#include <cstddef>
#include <type_traits>
#include <atomic>

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
constexpr int kWVec = NW * 2 * 2 * 64;    // W in f32       [NW][t-tile][half][lane]
constexpr int kPVec = 2 * 2 * 64;         // -P planes (two) [t-tile][plane][lane]
constexpr int kQVec = NW * 2 * 64;        // q, k per k-unit [NW][tile][lane]

// ------------------------------------------------------------ bf16 planes

struct Planes {
    u4_t h, m, l;
};

typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
typedef float f2_t __attribute__((ext_vector_type(2)));

// (a, b) rounded to bf16 (nearest even), a in the low half
__device__ __forceinline__ bf2_t rne2(float a, float b) { return __builtin_convertvector(f2_t{a, b}, bf2_t); }

// The bf16 pairs (-1, 0) and (0, -1) as 32-bit words.  The first is handed
// to the dot-product instruction from a scalar register set by s_mov: as a
// compile-time constant it is encoded as the inline constant -1.0, which the
// hardware does not read as that pair.
struct NegOnes {
    bf2_t lo, hi;
};
__device__ __forceinline__ NegOnes neg_ones() {
    uint32_t lo;
    asm volatile("s_mov_b32 %0, 0xbf80" : "=s"(lo));
    return NegOnes{__builtin_bit_cast(bf2_t, lo), __builtin_bit_cast(bf2_t, 0xBF800000u)};
}

// a - h.lo and b - h.hi, each one dot-product instruction: the bf16 products
// are exact and the remainder of a rounding is exactly representable, so the
// results are exact
__device__ __forceinline__ float rem_lo(const NegOnes& n, bf2_t h, float a) {
    return __builtin_amdgcn_fdot2_f32_bf16(h, n.lo, a, false);
}
__device__ __forceinline__ float rem_hi(const NegOnes& n, bf2_t h, float b) {
    return __builtin_amdgcn_fdot2_f32_bf16(h, n.hi, b, false);
}

struct Split2 {
    uint32_t h, m, l;    // bf16 pairs of each plane
};

// x = h + m + l exactly for x = a, b: h = bf16(x), m = bf16(x - h),
// l = x - h - m (at most 8 significant bits, so a bf16 exactly)
__device__ __forceinline__ Split2 split2(const NegOnes& n, float a, float b) {
    const bf2_t h = rne2(a, b);
    const float a1 = rem_lo(n, h, a), b1 = rem_hi(n, h, b);
    const bf2_t m = rne2(a1, b1);
    const bf2_t l = rne2(rem_lo(n, m, a1), rem_hi(n, m, b1));
    return Split2{__builtin_bit_cast(uint32_t, h), __builtin_bit_cast(uint32_t, m), __builtin_bit_cast(uint32_t, l)};
}

// eight f32 (x0 then x1) -> the two leading bf16 planes (x = h + m to 2^-17)
__device__ __forceinline__ void split8hm(const NegOnes& n, const f4_t x0, const f4_t x1, u4_t& h, u4_t& m) {
    const float xs[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float a = xs[2 * p], b = xs[2 * p + 1];
        const bf2_t hp = rne2(a, b);
        h[p] = __builtin_bit_cast(uint32_t, hp);
        m[p] = __builtin_bit_cast(uint32_t, rne2(rem_lo(n, hp, a), rem_hi(n, hp, b)));
    }
}

// eight f32 (x0 then x1) -> three bf16 planes
__device__ __forceinline__ Planes split8(const NegOnes& n, const f4_t x0, const f4_t x1) {
    const Split2 s0 = split2(n, x0[0], x0[1]), s1 = split2(n, x0[2], x0[3]);
    const Split2 s2 = split2(n, x1[0], x1[1]), s3 = split2(n, x1[2], x1[3]);
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

// 16x16x4 f32 product: lane l gives A[l % 16][l / 16] and B[l / 16][l % 16]
__device__ __forceinline__ f4_t mma_f32(float a, float b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
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

// -P entries (t, s0 .. s0+3) as two bf16 planes in the operand layout of
// the sequential pass, as step 3 of the per-head form stores them: the four
// columns are elements 4 half .. 4 half + 3 of quarter q4 of lane
// 16 q4 + t % 16, t-tile t / 16
__device__ __forceinline__ void store_neg_p(u4_t* pn, int64_t unit, int t, int s0, const float (&pv)[4],
                                            const NegOnes& no) {
    const int half = s0 >> 4, q4 = (s0 & 15) >> 2;
    const int l = 16 * q4 + (t & 15), jt = t >> 4;
    const Split2 p0 = split2(no, pv[0], pv[1]), p1 = split2(no, pv[2], pv[3]);
    u2_t* pdst = reinterpret_cast<u2_t*>(pn + unit * kPVec + (jt * 2) * 64 + l) + half;
    pdst[0] = u2_t{p0.h, p1.h};
    pdst[2 * 64] = u2_t{p0.m, p1.m};
}

// f32 (planes) x f32 (planes): the six plane products down to 2^-16 of the
// leading one, smallest first
__device__ __forceinline__ f4_t mma6(const Planes& a, const Planes& b, f4_t c) {
    c = mma(a.l, b.h, c);
    c = mma(a.h, b.l, c);
    c = mma(a.m, b.m, c);
    c = mma(a.m, b.h, c);
    c = mma(a.h, b.m, c);
    return mma(a.h, b.h, c);
}

// ========================================================= chunk preparation

// Inputs of the per-key form's preparation: k and q rows in f32, the gate
// rows (then the suffix decays within each quarter chunk) and the prefix
// decays within each quarter chunk, per key column.  Nothing in the per-head
// form.
template <bool PK>
struct PkIn {
    float kf[CK][DKC + 4];
    float qf[CK][DKC + 4];
    float ge[CK][DKC + 4];
    float gam[CK][DKC + 4];
    float gq[4][DKC];          // the product of each quarter chunk's gates
};
template <>
struct PkIn<false> {};

// One block serves NH v-heads of the same k-head (NH = 2 when the GQA group
// size is even): q, k, k k^T and q k^T are shared, the rest is per head.
template <int NH, bool PK = false>
struct alignas(16) PrepSmem {
    union {
        struct {
            uint16_t kb[CK][DKC + 8];    // bf16 rows, padded against bank conflicts
            uint16_t qb[CK][DKC + 8];
            float kk[CK][CK + 1];
            float qk[CK][CK + 1];
        } in;
        PkIn<PK> pk;
        struct {                 // written once the inputs above are dead
            uint16_t tw[3][CK][CK + 8];    // planes of T diag(beta gamma)
            uint16_t tb[3][CK][CK + 8];    // planes of -T diag(beta)
        } pl[NH];
    } u;
    union {
        struct {
            float a[CK][CK + 4];     // strictly lower A (row-major, 16-byte rows)
            float tm[CK][CK + 4];    // T = (I + A)^-1
        } s[NH];
        uint16_t vs[NH][CK][128 + 8];    // a 128-column slice of the chunk's v rows
    } w;
    float gs[NH][CK], bs[NH][CK], gm[NH][CK];
};

// the decay step reads the gates four at a time
static_assert(offsetof(PrepSmem<1>, gs) % 16 == 0 && offsetof(PrepSmem<2>, gs) % 16 == 0, "16-byte gate rows");

struct ChunkPtrs {
    u4_t* wsw;      // W (f32)
    u4_t* u;        // -Tb V (f32 accumulator tiles)
    u4_t* pn;       // -P planes (two)
    float* rg;      // per unit: -rho in kperm order [32], then gamma_t [32]
                    // (per-key form: -1, 1, then Gamma_{C-1} per key column [Dk])
    u4_t* qsw;      // q rows (per-key form: Q o Gamma, two planes per v-unit)
    u4_t* ksw;      // k columns (per-key form: -(K o E)^T in f32 per v-unit)
};

// floats of the per-unit decay record (-rho, gamma; per-key form: and Gamma_{C-1})
template <bool PK>
constexpr int rg_floats() { return PK ? 2 * CK + DKC : 2 * CK; }

// KF = 0: q, k, v, g, beta are inputs.  KF = 2..4: they are computed here,
// from the mixed projection qkv, with the prologue's arithmetic (the same
// device functions as the prologue kernel, so the same bits) and a conv of
// width KF; then Dv <= 128.  NH v-heads (of one k-head) per block, four
// waves per head: wave group h (waves 4h .. 4h + 3) does head h's own steps
// exactly as a one-head block would, so the results do not depend on NH.
// A two-head block takes just under 50 KB of LDS (the k rows share space
// with the T planes), so three fit a CU where the registers allow it.
// PK: the per-key gate g [B, T, Hv, Dk] (KF = 0, NH = 1): the decay ratios
// are per key column, so A and P are formed from running products and
// decay-scaled row products instead of scaled k k^T, q k^T; K o Gamma enters
// W, and the sequential pass gets Q o Gamma, (K o E)^T and Gamma_{C-1} in
// place of q, k and gamma.
template <int KF, int NH, bool PK = false>
__global__ __launch_bounds__(256 * NH, PK ? 2 : NH == 2 ? (KF > 0 ? 6 : 3) : 4) void chunk_prep_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const float* __restrict__ g,
                                                            const float* __restrict__ beta,
                                                            const uint8_t* __restrict__ mask,
                                                            const uint16_t* __restrict__ v, PrologueIn pin,
                                                            ChunkPtrs o, int T, int Hk, int Hv, int Dv, int NC) {
    static_assert(!PK || (KF == 0 && NH == 1), "the per-key form takes prepared inputs, one v-head per block");
    __shared__ PrepSmem<NH, PK> sh;
    // head pairs fastest in the grid: the blocks in flight together read
    // whole qkv rows of a few chunks (measured 59.9 -> 57.3 us at B=1 T=4096
    // and 1738 -> 1634 us at B=4 T=32768 against chunks fastest)
    const int npairs = (int)(gridDim.x / NC);
    const int c = (int)(blockIdx.x / npairs);
    const int np = (int)(blockIdx.x % npairs);    // b * (Hv / NH) + head pair
    const int b = np / (Hv / NH);
    const int hv0 = (np % (Hv / NH)) * NH;    // the block's first v-head
    const int G = Hv / Hk;
    const int hk = hv0 / G;
    const int64_t kunit = ((int64_t)b * Hk + hk) * NC + c;
    const int t0 = c * CK;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wv >> 2, wl = wv & 3;     // this wave's head in the block, its wave in the group
    const int tl = tid & 255;                 // thread in the group
    const int hv = hv0 + grp;
    const int64_t unit = ((int64_t)b * Hv + hv) * NC + c;
    const int lr = lane & 15, lq = lane >> 4;
    const NegOnes no = neg_ones();

    // 1. k, q rows of the chunk (zero past T), g and beta
    constexpr int kVPre = CK * 128 / 8 / 256;      // 16-byte vectors per thread (first v slice)
    uint4 vpre[kVPre];
    constexpr int TPW = CK / (4 * NH);            // fused: tokens per wave
    uint4 vrow[KF > 0 ? TPW : 1];                 // fused: this lane's v rows
    if constexpr (KF > 0) {
      {
        // Wave w computes tokens t0 + TPW w .. t0 + TPW (w + 1) - 1 (every wave
        // of the block: the per-wave chain of loads, conv, SiLU and norm is
        // what bounds this phase).  Lanes 0-15 hold the q head's 8-channel
        // groups, 16-31 the k head's (aligned 16-lane groups, as in the
        // prologue kernel, for the norm's cross-lane sum), 32 .. 32 + Dv/8 - 1
        // the first v-head's and, with two heads, 48 .. 48 + Dv/8 - 1 the
        // second's.
        const int C = 2 * Hk * DKC + Hv * Dv;
        int region = 3, c0 = 0;
        if (lane < 16) { region = 0; c0 = hk * DKC + 8 * lane; }
        else if (lane < 32) { region = 1; c0 = Hk * DKC + hk * DKC + 8 * (lane - 16); }
        else if (lane < 32 + Dv / 8) { region = 2; c0 = 2 * Hk * DKC + hv0 * Dv + 8 * (lane - 32); }
        else if (NH == 2 && lane >= 48 && lane < 48 + Dv / 8) { region = 2; c0 = 2 * Hk * DKC + (hv0 + 1) * Dv + 8 * (lane - 48); }
        const bool valid = region < 3;
        // lanes without channels (v lanes past Dv/8) read a channel of the
        // first v-head instead, so that every load of the wave is taken;
        // nothing they compute is stored
        const int cr = valid ? c0 : 2 * Hk * DKC + hv0 * Dv;
        const float scale = region == 0 ? pin.q_scale : pin.k_scale;
        // the gate inputs of the group's head (one token per thread of the
        // first 32) are loaded first, so that the gate arithmetic below
        // overlaps the row loads
        uint16_t ga = 0, gb = 0;
        bool gon = false;
        if (tl < CK) {
            const int t = t0 + tl;
            const int64_t bt = (int64_t)b * T + min(t, T - 1);
            gon = t < T && (mask == nullptr || mask[bt] != 0);     // else g = 1, beta = 0
            ga = pin.a[bt * Hv + hv];
            gb = pin.b[bt * Hv + hv];
        }
        const uint16_t* xb = pin.qkv + (int64_t)b * T * C + cr;
        const uint16_t* csb = pin.conv_state_in ? pin.conv_state_in + (int64_t)b * (KF - 1) * C + cr : nullptr;
        // conv weights as stored bf16 pairs
        uint4 wk[KF];
#pragma unroll
        for (int v4 = 0; v4 < KF; ++v4) wk[v4] = reinterpret_cast<const uint4*>(pin.conv_w + (int64_t)cr * KF)[v4];
        const ConvW<KF> cw = conv_weights<KF>(wk);
        // spliced input row pr: conv state rows, then qkv rows, zero past T
        // (the same case for every lane of the wave)
        auto xpad_row = [&](int pr) -> uint4 {
            const int tr = pr - (KF - 1);
            if (tr >= T) return make_uint4(0, 0, 0, 0);
            if (tr >= 0) return *reinterpret_cast<const uint4*>(xb + (int64_t)tr * C);
            if (csb) return *reinterpret_cast<const uint4*>(csb + (int64_t)pr * C);
            return make_uint4(0, 0, 0, 0);
        };
        // the spliced input rows this wave's tokens read: tw0 .. tw0 + TPW + KF - 2
        const int tw0 = t0 + TPW * wv;
        uint4 rows[TPW + KF - 1];
#pragma unroll
        for (int i = 0; i < TPW + KF - 1; ++i) rows[i] = xpad_row(tw0 + i);
        if (tl < CK) {
            float gv, bv;
            gate_g_beta(ga, gb, pin.A_log[hv], pin.dt_bias[hv], gv, bv);
            sh.gs[grp][tl] = gon ? gv : 1.f;
            sh.bs[grp][tl] = gon ? bv : 0.f;
        }
        // the new conv state (chunk 0's blocks; q/k channels from the first
        // v-head of the group): the last KF-1 rows of the spliced input
        if (c == 0 && wv == 0 && valid && pin.conv_state_out && (region == 2 || hv0 % G == 0)) {
            // every row read before any is written (the state may be updated in place)
            uint4 tail[KF - 1];
#pragma unroll
            for (int i = 0; i < KF - 1; ++i) tail[i] = xpad_row(T + i);
            uint16_t* out = pin.conv_state_out + (int64_t)b * (KF - 1) * C + c0;
#pragma unroll
            for (int i = 0; i < KF - 1; ++i) *reinterpret_cast<uint4*>(out + (int64_t)i * C) = tail[i];
        }
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int t = tw0 + i;
            uint4 win[KF];
#pragma unroll
            for (int j = 0; j < KF; ++j) win[j] = rows[i + j];
            float act[8];
            conv_silu8<KF>(cw, win, act);
            // q/k lanes: the head norm; v lanes: act itself
            const bool live = t < T;      // rows past T are zero, as for stored inputs
            const uint4 n = qk_norm8<DKC>(act, region < 2, scale, pin.eps);
            const uint4 o = live ? n : make_uint4(0, 0, 0, 0);
            if (region == 0) *reinterpret_cast<uint4*>(&sh.u.in.qb[t - t0][8 * lane]) = o;
            else if (region == 1) *reinterpret_cast<uint4*>(&sh.u.in.kb[t - t0][8 * (lane - 16)]) = o;
            vrow[i] = o;
        }
      }
    } else {
    constexpr int kQKPer = CK * DKC / 8 / (256 * NH);     // 16-byte k (and q) vectors per thread
    uint4 kva[kQKPer], qva[kQKPer];
#pragma unroll
    for (int i = 0; i < kQKPer; ++i) {
        // rows past T are read clamped (in bounds) and zeroed below, so the
        // loads need no branch and all issue before the first LDS store
        const int idx = tid + i * 256 * NH;
        const int t = idx / (DKC / 8), c8 = idx % (DKC / 8);
        const int64_t off = (((int64_t)b * T + min(t0 + t, T - 1)) * Hk + hk) * DKC + c8 * 8;
        kva[i] = *reinterpret_cast<const uint4*>(k + off);
        qva[i] = *reinterpret_cast<const uint4*>(q + off);
    }
    // per-key form: the gate rows too, before any LDS store (steps past T
    // and masked steps decay by 1)
    constexpr int kGPer = PK ? CK * DKC / 4 / 256 : 1;
    float4 gva[kGPer];
    bool gon[kGPer];
    if constexpr (PK) {
#pragma unroll
        for (int i = 0; i < kGPer; ++i) {
            const int idx = tid + i * 256;
            const int t = idx / (DKC / 4), c4 = idx % (DKC / 4);
            const int64_t bt = (int64_t)b * T + min(t0 + t, T - 1);
            gon[i] = t0 + t < T && (mask == nullptr || mask[bt] != 0);
            gva[i] = *reinterpret_cast<const float4*>(g + (bt * Hv + hv) * DKC + 4 * c4);   // in bounds
        }
    }
#pragma unroll
    for (int i = 0; i < kQKPer; ++i) {
        const int idx = tid + i * 256 * NH;
        const int t = idx / (DKC / 8), c8 = idx % (DKC / 8);
        const bool live = t0 + t < T;
        const uint4 kv = live ? kva[i] : make_uint4(0, 0, 0, 0);
        const uint4 qv = live ? qva[i] : make_uint4(0, 0, 0, 0);
        if constexpr (PK) {
            float kf8[8], qf8[8];
            unpack8(kv, kf8);
            unpack8(qv, qf8);
            float* kd = &sh.u.pk.kf[t][c8 * 8];
            float* qd = &sh.u.pk.qf[t][c8 * 8];
            *reinterpret_cast<float4*>(kd) = make_float4(kf8[0], kf8[1], kf8[2], kf8[3]);
            *reinterpret_cast<float4*>(kd + 4) = make_float4(kf8[4], kf8[5], kf8[6], kf8[7]);
            *reinterpret_cast<float4*>(qd) = make_float4(qf8[0], qf8[1], qf8[2], qf8[3]);
            *reinterpret_cast<float4*>(qd + 4) = make_float4(qf8[4], qf8[5], qf8[6], qf8[7]);
        } else {
            *reinterpret_cast<uint4*>(&sh.u.in.kb[t][c8 * 8]) = kv;
            *reinterpret_cast<uint4*>(&sh.u.in.qb[t][c8 * 8]) = qv;
        }
    }
    if constexpr (PK) {
        // the gate rows loaded above
#pragma unroll
        for (int i = 0; i < kGPer; ++i) {
            const int idx = tid + i * 256;
            const int t = idx / (DKC / 4), c4 = idx % (DKC / 4);
            const float4 gv = gva[i];
            const bool on = gon[i];
            *reinterpret_cast<float4*>(&sh.u.pk.ge[t][4 * c4]) =
                make_float4(on ? gv.x : 1.f, on ? gv.y : 1.f, on ? gv.z : 1.f, on ? gv.w : 1.f);
        }
    }
    // the first 128-column slice of this chunk's v rows, loaded now (its
    // latency hides behind steps 2-6) and staged through LDS in step 7
    {
        const int wdt = min(128, Dv);
#pragma unroll
        for (int i = 0; i < kVPre; ++i) {
            const int idx = tl + i * 256;
            const int t = idx / (wdt / 8), c8 = idx % (wdt / 8);
            vpre[i] = make_uint4(0, 0, 0, 0);
            if (idx < CK * (wdt / 8) && t0 + t < T)
                vpre[i] = *reinterpret_cast<const uint4*>(v + (((int64_t)b * T + t0 + t) * Hv + hv) * Dv + c8 * 8);
        }
    }
    }
    if (KF == 0 && tl < CK) {
        // steps past T and masked steps: g = 1, beta = 0 (no decay, no write);
        // the fused form computed its gates above
        const int t = t0 + tl;
        const int64_t bt = (int64_t)b * T + min(t, T - 1);
        const int64_t i = bt * Hv + hv;
        const float gv = PK ? 1.f : g[i];    // (per-key gate rows are loaded above)
        const float bv = beta[i];
        const bool on = t < T && (mask == nullptr || mask[bt] != 0);
        sh.gs[grp][tl] = on ? gv : 1.f;
        sh.bs[grp][tl] = on ? bv : 0.f;
    }
    __syncthreads();

    // 2a. k^T in operand layout for this wave's columns (rows kperm(q, e),
    //     column 32w + 16tt + r); the first v-head of each group also stores
    //     it and q (rows 16j + r, columns 32w + kperm(q, e)) for the
    //     sequential pass
    u4_t kt[2];
    Planes kwp[2];        // per-key form: (K o Gamma)^T planes, formed in step 3'
    if constexpr (!PK) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int d = 32 * wl + 16 * tt + lr;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int s0 = p < 2 ? 4 * lq + 2 * p : 16 + 4 * lq + 2 * (p - 2);
                kt[tt][p] = (uint32_t)sh.u.in.kb[s0][d] | ((uint32_t)sh.u.in.kb[s0 + 1][d] << 16);
            }
        }
        if (grp == 0 && hv0 % G == 0) {
            u4_t* kd = o.ksw + kunit * kQVec + wl * 2 * 64 + lane;
            u4_t* qd = o.qsw + kunit * kQVec + wl * 2 * 64 + lane;
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                kd[jt * 64] = kt[jt];
                const u2_t lo = *reinterpret_cast<const u2_t*>(&sh.u.in.qb[16 * jt + lr][32 * wl + 4 * lq]);
                const u2_t hi = *reinterpret_cast<const u2_t*>(&sh.u.in.qb[16 * jt + lr][32 * wl + 16 + 4 * lq]);
                qd[jt * 64] = u4_t{lo[0], lo[1], hi[0], hi[1]};
            }
        }
    }

    // 2b. k k^T and q k^T, 32 x 32 each: wave w owns output tile
    //     ((w % 4) / 2, w % 2), of both products in a one-head block, of
    //     k k^T (waves 0-3) or q k^T (waves 4-7) in a two-head block
    if constexpr (!PK) {
        const int mi = wl >> 1, ni = wl & 1;
        f4_t ckk = {0.f, 0.f, 0.f, 0.f}, cqk = ckk;
#pragma unroll
        for (int ks = 0; ks < DKC / 32; ++ks) {
            const int col = ks * 32 + 8 * lq;
            const u4_t kb = *reinterpret_cast<const u4_t*>(&sh.u.in.kb[16 * ni + lr][col]);
            if (NH == 1 || grp == 0) {
                const u4_t ka = *reinterpret_cast<const u4_t*>(&sh.u.in.kb[16 * mi + lr][col]);
                ckk = mma(ka, kb, ckk);
            }
            if (NH == 1 || grp == 1) {
                const u4_t qa = *reinterpret_cast<const u4_t*>(&sh.u.in.qb[16 * mi + lr][col]);
                cqk = mma(qa, kb, cqk);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (NH == 1 || grp == 0) sh.u.in.kk[16 * mi + 4 * lq + i][16 * ni + lr] = ckk[i];
            if (NH == 1 || grp == 1) sh.u.in.qk[16 * mi + 4 * lq + i][16 * ni + lr] = cqk[i];
        }
    }
    __syncthreads();

    // 3. decay ratios R[t][s] = g_{s+1}...g_t (s <= t) for s in this thread's
    //    four columns, then A, -P (two planes), gamma, -rho
    if constexpr (!PK) {
        const int t = tl >> 3, s0 = (tl & 7) * 4;
        const float* gs = sh.gs[grp];
        // The eight threads of row t are adjacent lanes.  Thread k (s0 = 4k)
        // forms its block's gates up to step t, G_k = g_{4k} ... g_{min(4k+3, t)}
        // (1 if 4k > t); the product of the later blocks G_{k+1} ... G_7 is
        // R[t][s0+3] = g_{s0+4} ... g_t, and R[t][s] = R[t][s+1] g_{s+1} while
        // s+1 <= t; R[t][s] = 1 for s >= t (only s = t is used).
        const float4 g4 = *reinterpret_cast<const float4*>(gs + s0);
        float blk = s0 <= t ? g4.x : 1.f;
        blk *= s0 + 1 <= t ? g4.y : 1.f;
        blk *= s0 + 2 <= t ? g4.z : 1.f;
        blk *= s0 + 3 <= t ? g4.w : 1.f;
        const float later = dpp_mov<DPP_ROW_SHL1>(suffix_prod8(blk));
        float r[4];
        r[3] = (tl & 7) < 7 ? later : 1.f;
        r[2] = s0 + 3 <= t ? r[3] * g4.w : 1.f;
        r[1] = s0 + 2 <= t ? r[2] * g4.z : 1.f;
        r[0] = s0 + 1 <= t ? r[1] * g4.y : 1.f;
        float av[4], pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = s0 + e;
            av[e] = s < t ? sh.bs[grp][t] * r[e] * sh.u.in.kk[t][s] : 0.f;
            pv[e] = s <= t ? -(r[e] * sh.u.in.qk[t][s]) : 0.f;
        }
        *reinterpret_cast<float4*>(&sh.w.s[grp].a[t][s0]) = make_float4(av[0], av[1], av[2], av[3]);
        // these four columns are elements 4 half .. 4 half + 3 of quarter q4
        const int half = s0 >> 4, q4 = (s0 & 15) >> 2;
        const int l = 16 * q4 + (t & 15), jt = t >> 4;
        const Split2 p0 = split2(no, pv[0], pv[1]), p1 = split2(no, pv[2], pv[3]);
        u2_t* pdst = reinterpret_cast<u2_t*>(o.pn + unit * kPVec + (jt * 2) * 64 + l) + half;
        pdst[0] = u2_t{p0.h, p1.h};
        pdst[2 * 64] = u2_t{p0.m, p1.m};
        if (s0 == 0) {
            const float gm = gs[0] * r[0];        // gamma_t = g_0 R[t][0]
            sh.gm[grp][t] = gm;
            o.rg[unit * 2 * CK + CK + t] = gm;
        }
        if (t == CK - 1)
            *reinterpret_cast<float4*>(o.rg + unit * 2 * CK + 8 * q4 + 4 * half) = make_float4(-r[0], -r[1], -r[2], -r[3]);
    } else {
        // 3'. per-key decay ratios R_j(t, s) = g_{s+1}[j] ... g_t[j]:
        //     A[t][s] = beta_t sum_j k_t[j] k_s[j] R_j(t, s)   (s < t)
        //     P[t][s] = sum_j q_t[j] k_s[j] R_j(t, s)          (s <= t)
        //     Within each quarter chunk of eight steps (s, t in the same
        //     quarter) thread (s, jg) carries u = k_s o R(t, s) over key
        //     columns 16 jg .. 16 jg + 15 while t runs up from s to the
        //     quarter's end (a running product, never a quotient of cumulative
        //     decays); the eight column groups of a row s are adjacent lanes,
        //     summed by DPP.  Wave w holds the rows of quarter w.  Across
        //     quarters (s in an earlier one) R(t, s) splits at the boundary
        //     into factors <= 1, R(t, s) = R(t, m) o R(m, s): those blocks are
        //     f32 products on the matrix cores (below).
        auto& sw = sh.w.s[0];
        const int s = tl >> 3, jg = tl & 7;
        // a wave's eight rows s share their quarter: scalar bounds
        const int s_lo = __builtin_amdgcn_readfirstlane(s & ~7);
        const int t_hi = s_lo + 8;
        float u[16];
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const float4 x = *reinterpret_cast<const float4*>(&sh.u.pk.kf[s][16 * jg + 4 * e4]);
            u[4 * e4] = x.x;
            u[4 * e4 + 1] = x.y;
            u[4 * e4 + 2] = x.z;
            u[4 * e4 + 3] = x.w;
        }
        // the operands of step t (gate, key and query row, this thread's 16
        // columns), read one step ahead so that their LDS latency overlaps
        // the step before
        struct RowOps {
            float4 g[4], k[4], q[4];
        };
        auto row_ops = [&](int t) {
            RowOps r;
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const int j = 16 * jg + 4 * e4;
                r.g[e4] = *reinterpret_cast<const float4*>(&sh.u.pk.ge[t][j]);
                r.k[e4] = *reinterpret_cast<const float4*>(&sh.u.pk.kf[t][j]);
                r.q[e4] = *reinterpret_cast<const float4*>(&sh.u.pk.qf[t][j]);
            }
            return r;
        };
        // one step t: decay u by g_t (from the step after row s on; MASK is
        // false where every row of the wave is already behind t), the two
        // dot products, their 8-lane sums, A and P of (t, s)
        auto pk_step = [&](int t, const RowOps& r, auto mask) {
            constexpr bool MASK = decltype(mask)::value;
            // four partial sums per product (short dependent chains)
            float pa4[4], pp4[4];
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const float ga[4] = {r.g[e4].x, r.g[e4].y, r.g[e4].z, r.g[e4].w};
                const float ka[4] = {r.k[e4].x, r.k[e4].y, r.k[e4].z, r.k[e4].w};
                const float qa[4] = {r.q[e4].x, r.q[e4].y, r.q[e4].z, r.q[e4].w};
                pa4[e4] = 0.f;
                pp4[e4] = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float& ue = u[4 * e4 + i];
                    if (!MASK || t > s) ue *= ga[i];
                    pa4[e4] = fmaf(ka[i], ue, pa4[e4]);
                    pp4[e4] = fmaf(qa[i], ue, pp4[e4]);
                }
            }
            float pa = (pa4[0] + pa4[1]) + (pa4[2] + pa4[3]);
            float pp = (pp4[0] + pp4[1]) + (pp4[2] + pp4[3]);
            group_sum2<8>(pa, pp);
            if (jg == 0) {
                sw.a[t][s] = t > s ? sh.bs[0][t] * pa : 0.f;
                sw.tm[t][s] = t >= s ? pp : 0.f;       // P, kept here until its planes are cut
            }
        };
        // steps s_lo .. s_lo + 7 in pairs, the wave's own rows, where the
        // decay starts row by row
        RowOps ra = row_ops(s_lo);
        for (int t = s_lo; t < t_hi; t += 2) {
            const RowOps rb = row_ops(t + 1);
            pk_step(t, ra, std::true_type{});
            ra = row_ops(min(t + 2, t_hi - 1));
            pk_step(t + 1, rb, std::true_type{});
        }
        if (jg == 0)
            for (int t = 0; t < s_lo; ++t) {
                sw.a[t][s] = 0.f;
                sw.tm[t][s] = 0.f;
            }
        __syncthreads();
        // decays per key column within each quarter chunk: prefix products
        // (gam), suffix products (ge, over the gate rows), and the product
        // of each quarter's gates; thread (j, h) takes column j in half h
        constexpr int CQ = CK / 4, CH2 = CK / 2;
        {
            const int j = tl & (DKC - 1), h = tl / DKC;
            float gc[2 * CQ];
#pragma unroll
            for (int i = 0; i < 2 * CQ; ++i) gc[i] = sh.u.pk.ge[2 * CQ * h + i][j];
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                float gp = 1.f, ep = 1.f;
#pragma unroll
                for (int i = 0; i < CQ; ++i) {
                    const int t = CQ * (2 * h + qq) + i, r = CQ * (2 * h + qq) + CQ - 1 - i;
                    gp *= gc[CQ * qq + i];
                    sh.u.pk.gam[t][j] = gp;
                    sh.u.pk.ge[r][j] = ep;
                    ep *= gc[CQ * qq + CQ - 1 - i];
                }
                sh.u.pk.gq[2 * h + qq][j] = gp;
            }
        }
        __syncthreads();
        // Gamma_{C-1} and the blocks of A and P across quarters, each one 16 x 16
        // f32 product over the key columns on the f32 matrix instruction
        // (product e of a 32-column block takes element e of the lane's eight
        // columns, as in W S^T of the sequential pass):
        //   waves 0, 2: A, P of steps t in quarter 1 (3) against s in quarter 0
        //     (2), R(t, s) = G(t) o E(s) with G the prefix decays of t's quarter
        //     and E the suffix decays of s's (the other two 8 x 8 blocks of the
        //     tile pair unrelated steps and are dropped);
        //   waves 1, 3: A, P of t in the second half against s in the first,
        //     R(t, s) = (G(t) [o g_q2 for t in quarter 3]) o (E(s) [o g_q1 for
        //     s in quarter 0]), g_q the product of quarter q's gates.
        if (tl < DKC)
            o.rg[unit * rg_floats<PK>() + 2 * CK + tl] =
                ((sh.u.pk.gq[0][tl] * sh.u.pk.gq[1][tl]) * sh.u.pk.gq[2][tl]) * sh.u.pk.gq[3][tl];   // Gamma_{C-1}
        {
            const bool xh = (wl & 1) != 0;     // across the halves
            const bool isp = wl >= 2;          // P (q rows) instead of A (k rows)
            const int tm = xh ? CH2 + lr : (lr < CQ ? CQ + lr : CH2 + lr);     // left operand row lr: step t
            const int sn = xh ? lr : (lr < CQ ? lr : CQ + lr);                // right operand row lr: step s
            const float* xr = isp ? &sh.u.pk.qf[tm][0] : &sh.u.pk.kf[tm][0];
            const bool in3 = xh && tm >= CH2 + CQ, in0 = xh && sn < CQ;
            auto ld4 = [](const float* p) { return *reinterpret_cast<const f4_t*>(p); };
            f4_t acc2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ks = 0; ks < DKC / 32; ++ks) {
                const int c = 32 * ks + 8 * lq;
                f4_t av[2], bv[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int ch = c + 4 * h;
                    f4_t gt = ld4(&sh.u.pk.gam[tm][ch]), es = ld4(&sh.u.pk.ge[sn][ch]);
                    if (xh) {
                        const f4_t g2 = ld4(&sh.u.pk.gq[2][ch]), g1 = ld4(&sh.u.pk.gq[1][ch]);
                        const f4_t gt3 = g2 * gt, es0 = es * g1;
                        gt = in3 ? gt3 : gt;
                        es = in0 ? es0 : es;
                    }
                    av[h] = ld4(xr + ch) * gt;
                    bv[h] = ld4(&sh.u.pk.kf[sn][ch]) * es;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) acc2[ks & 1] = mma_f32(av[e >> 2][e & 3], bv[e >> 2][e & 3], acc2[ks & 1]);
            }
            const f4_t acc = acc2[0] + acc2[1];
            // output row 4 lq + i (a left row, step t), column lr (a right row, step s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * lq + i;
                const int t = xh ? CH2 + m : (m < CQ ? CQ + m : CH2 + m);
                if (xh || (m < CQ) == (lr < CQ)) {
                    if (!isp) sw.a[t][sn] = sh.bs[0][t] * acc[i];
                    else sw.tm[t][sn] = acc[i];
                }
            }
        }
        __syncthreads();
        // the chunk's decays from the quarter ones, in place: Gamma_t = g_0 ... g_t
        // is the product of the earlier quarters' gates times t's prefix in its
        // quarter, E_t = g_{t+1} ... g_{C-1} t's suffix in its quarter times the
        // later quarters' gates
        {
            const int j = tl & (DKC - 1), h = tl / DKC;
            const float g0 = sh.u.pk.gq[0][j], g1 = sh.u.pk.gq[1][j], g2 = sh.u.pk.gq[2][j], g3 = sh.u.pk.gq[3][j];
            const float g01 = g0 * g1, g23 = g2 * g3;
            const float pre[4] = {1.f, g0, g01, g01 * g2};
            const float suf[4] = {g1 * g23, g23, g3, 1.f};
#pragma unroll
            for (int i = 0; i < 2 * CQ; ++i) {
                const int t = 2 * CQ * h + i, q = t / CQ;
                if (q > 0) sh.u.pk.gam[t][j] = pre[q] * sh.u.pk.gam[t][j];
                if (q < 3) sh.u.pk.ge[t][j] = sh.u.pk.ge[t][j] * suf[q];
            }
        }
        __syncthreads();
        {
            // -P planes; gamma = 1 and -rho = -1 (the decay is in the operands)
            const int t = tl >> 3, s0 = (tl & 7) * 4;
            const float4 p4 = *reinterpret_cast<const float4*>(&sw.tm[t][s0]);
            const float pv[4] = {-p4.x, -p4.y, -p4.z, -p4.w};
            store_neg_p(o.pn, unit, t, s0, pv, no);
            if (tl < CK) sh.gm[0][tl] = 1.f;
            if (tl < 2 * CK) o.rg[unit * rg_floats<PK>() + tl] = tl < CK ? -1.f : 1.f;
        }
        auto gamma_at = [&](int t, int j) { return sh.u.pk.gam[t][j]; };
        auto e_at = [&](int t, int j) { return sh.u.pk.ge[t][j]; };
        // operands: (K o Gamma)^T planes for W (kept in registers until step
        // 6), -(K o E)^T in f32 and Q o Gamma planes for the sequential pass
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int d = 32 * wl + 16 * tt + lr;
            float xw[8], xe[8];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int s0 = p < 2 ? 4 * lq + 2 * p : 16 + 4 * lq + 2 * (p - 2);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float kv = sh.u.pk.kf[s0 + h][d];
                    xw[2 * p + h] = kv * gamma_at(s0 + h, d);
                    xe[2 * p + h] = kv * e_at(s0 + h, d);
                }
            }
            kwp[tt] = split8(no, f4_t{xw[0], xw[1], xw[2], xw[3]}, f4_t{xw[4], xw[5], xw[6], xw[7]});
            // -(K o E)^T in f32: element 4 jt + i is step 16 jt + 4 lq + i
            u4_t* kd = o.ksw + unit * 2 * kQVec + (wl * 2 + tt) * 2 * 64 + lane;
            kd[0] = __builtin_bit_cast(u4_t, f4_t{-xe[0], -xe[1], -xe[2], -xe[3]});
            kd[64] = __builtin_bit_cast(u4_t, f4_t{-xe[4], -xe[5], -xe[6], -xe[7]});
        }
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            const int t = 16 * jt + lr;
            f4_t x0, x1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c0 = 32 * wl + 4 * lq + i, c1 = c0 + 16;
                x0[i] = sh.u.pk.qf[t][c0] * gamma_at(t, c0);
                x1[i] = sh.u.pk.qf[t][c1] * gamma_at(t, c1);
            }
            u4_t qh, qm;
            split8hm(no, x0, x1, qh, qm);
            u4_t* qd = o.qsw + unit * 2 * kQVec + (wl * 2 + jt) * 64 + lane;
            qd[0] = qh;
            qd[kQVec] = qm;
        }
    }
    __syncthreads();

    // 4. T = (I + A)^-1 in 16 x 16 blocks.  A is strictly lower, so with
    //    A = [[A11, 0], [A21, A22]]:  T11 = (I + A11)^-1, T22 = (I + A22)^-1,
    //    T12 = 0 and T21 = -T22 A21 T11.
    //    4a. T11 and T22 at once by forward substitution, one column per lane
    //        (lanes 0-15: T11, lanes 16-31: T22), rows to LDS as soon as they
    //        are known; lanes 32-63 zero T12.  The scheduling barrier per row
    //        keeps the row's operands from being hoisted.
    constexpr int CH = CK / 2;
    auto& sw = sh.w.s[grp];
    if (tl < CK) {
        const int j = tl % CH, base = tl < CH ? 0 : CH;
        float x[CH];
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
            for (int s4 = 0; s4 < t; s4 += 4) {
                const float4 a4 = *reinterpret_cast<const float4*>(&sw.a[base + t][base + s4]);
                acc0 = fmaf(a4.x, x[s4], acc0);
                if (s4 + 1 < t) acc1 = fmaf(a4.y, x[s4 + 1], acc1);
                if (s4 + 2 < t) acc0 = fmaf(a4.z, x[s4 + 2], acc0);
                if (s4 + 3 < t) acc1 = fmaf(a4.w, x[s4 + 3], acc1);
            }
            x[t] = (t == j ? 1.f : 0.f) - (acc0 + acc1);
            sw.tm[base + t][base + j] = x[t];
            __builtin_amdgcn_sched_barrier(0);
        }
    } else if (tl < 2 * CK) {
        // T12 = 0: rows 0..15, columns 16..31, one row per lane pair
        const int t = (tl - CK) >> 1, h = (tl - CK) & 1;
        *reinterpret_cast<float4*>(&sw.tm[t][CH + 8 * h]) = make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(&sw.tm[t][CH + 8 * h + 4]) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    //    4b. M = A21 T11 (16 x 16, one entry per thread) into the unused upper
    //        right block of A, then T21 = -T22 M.
    {
        const int i = tl >> 4, j = tl & 15;
        float m0 = 0.f, m1 = 0.f;
#pragma unroll
        for (int k4 = 0; k4 < CH; k4 += 4) {
            const float4 a4 = *reinterpret_cast<const float4*>(&sw.a[CH + i][k4]);
            m0 = fmaf(a4.x, sw.tm[k4][j], m0);
            m1 = fmaf(a4.y, sw.tm[k4 + 1][j], m1);
            m0 = fmaf(a4.z, sw.tm[k4 + 2][j], m0);
            m1 = fmaf(a4.w, sw.tm[k4 + 3][j], m1);
        }
        sw.a[i][CH + j] = m0 + m1;
        __syncthreads();
        float u0 = 0.f, u1 = 0.f;
#pragma unroll
        for (int k4 = 0; k4 < CH; k4 += 4) {
            const float4 t4 = *reinterpret_cast<const float4*>(&sw.tm[CH + i][CH + k4]);
            u0 = fmaf(t4.x, sw.a[k4][CH + j], u0);
            u1 = fmaf(t4.y, sw.a[k4 + 1][CH + j], u1);
            u0 = fmaf(t4.z, sw.a[k4 + 2][CH + j], u0);
            u1 = fmaf(t4.w, sw.a[k4 + 3][CH + j], u1);
        }
        sw.tm[CH + i][j] = -(u0 + u1);
    }
    __syncthreads();

    // 5. planes of T diag(beta gamma) and of -T diag(beta), four entries per thread
    {
        const int t = tl >> 3, s0 = (tl & 7) * 4;
        const float4 tv = *reinterpret_cast<const float4*>(&sw.tm[t][s0]);
        const float x[4] = {tv.x, tv.y, tv.z, tv.w};
        float w4[4], b4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float bs = sh.bs[grp][s0 + e];
            w4[e] = x[e] * (bs * sh.gm[grp][s0 + e]);
            b4[e] = -(x[e] * bs);
        }
        const Split2 w0 = split2(no, w4[0], w4[1]), w1 = split2(no, w4[2], w4[3]);
        const Split2 b0 = split2(no, b4[0], b4[1]), b1 = split2(no, b4[2], b4[3]);
        *reinterpret_cast<u2_t*>(&sh.u.pl[grp].tw[0][t][s0]) = u2_t{w0.h, w1.h};
        *reinterpret_cast<u2_t*>(&sh.u.pl[grp].tw[1][t][s0]) = u2_t{w0.m, w1.m};
        *reinterpret_cast<u2_t*>(&sh.u.pl[grp].tw[2][t][s0]) = u2_t{w0.l, w1.l};
        *reinterpret_cast<u2_t*>(&sh.u.pl[grp].tb[0][t][s0]) = u2_t{b0.h, b1.h};
        *reinterpret_cast<u2_t*>(&sh.u.pl[grp].tb[1][t][s0]) = u2_t{b0.m, b1.m};
        *reinterpret_cast<u2_t*>(&sh.u.pl[grp].tb[2][t][s0]) = u2_t{b0.l, b1.l};
    }
    __syncthreads();

    // 6. W^T = K^T (T diag(beta gamma))^T on the matrix cores: wave w forms
    //    column tiles 2w, 2w+1 of W^T for both t-tiles; its accumulators are
    //    W rows 16j + r at columns 32w + kperm(q, e), the layout of the
    //    sequential pass (stored in f32; that pass cuts them into planes).
    //    Per-key form: W^T = (K o Gamma)^T (T diag(beta))^T, f32 by f32.
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
        Planes tw;
        const int row = 16 * jt + lr;
        const u2_t h0 = *reinterpret_cast<const u2_t*>(&sh.u.pl[grp].tw[0][row][4 * lq]);
        const u2_t h1 = *reinterpret_cast<const u2_t*>(&sh.u.pl[grp].tw[0][row][16 + 4 * lq]);
        const u2_t m0 = *reinterpret_cast<const u2_t*>(&sh.u.pl[grp].tw[1][row][4 * lq]);
        const u2_t m1 = *reinterpret_cast<const u2_t*>(&sh.u.pl[grp].tw[1][row][16 + 4 * lq]);
        const u2_t l0 = *reinterpret_cast<const u2_t*>(&sh.u.pl[grp].tw[2][row][4 * lq]);
        const u2_t l1 = *reinterpret_cast<const u2_t*>(&sh.u.pl[grp].tw[2][row][16 + 4 * lq]);
        tw.h = u4_t{h0[0], h0[1], h1[0], h1[1]};
        tw.m = u4_t{m0[0], m0[1], m1[0], m1[1]};
        tw.l = u4_t{l0[0], l0[1], l1[0], l1[1]};
        const f4_t zero = {0.f, 0.f, 0.f, 0.f};
        f4_t w0, w1;
        if constexpr (PK) {
            w0 = mma6(kwp[0], tw, zero);
            w1 = mma6(kwp[1], tw, zero);
        } else {
            w0 = mma3b(kt[0], tw, zero);
            w1 = mma3b(kt[1], tw, zero);
        }
        u4_t* dst = o.wsw + unit * kWVec + ((wl * 2 + jt) * 2) * 64 + lane;
        dst[0] = __builtin_bit_cast(u4_t, w0);
        dst[64] = __builtin_bit_cast(u4_t, w1);
    }

    // 7. U = -Tb V for every 16 value columns rb and t-tile j, in the
    //    accumulator layout of the sequential pass (lane holds rows
    //    16j + 4q .. 16j + 4q + 3 of column 16 rb + r); v is staged through
    //    LDS 128 columns at a time (rows past T are zero)
    Planes tb[2];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
        const int row = 16 * jt + lr;
        tb[jt].h = *reinterpret_cast<const u4_t*>(&sh.u.pl[grp].tb[0][row][8 * lq]);
        tb[jt].m = *reinterpret_cast<const u4_t*>(&sh.u.pl[grp].tb[1][row][8 * lq]);
        tb[jt].l = *reinterpret_cast<const u4_t*>(&sh.u.pl[grp].tb[2][row][8 * lq]);
    }
    for (int c0 = 0; c0 < Dv; c0 += 128) {
        const int wdt = min(128, Dv - c0);
        if (KF > 0) {
            // fused: lane 32 + j (48 + j) of wave w holds column group j of
            // tokens TPW w .. TPW (w + 1) - 1 of the first (second) v-head
            {
                const int hs = lane >= 48 ? 1 : 0;
                const int j = lane - 32 - 16 * hs;
                if (lane >= 32 && hs < NH && j < wdt / 8) {
#pragma unroll
                    for (int i = 0; i < TPW; ++i) *reinterpret_cast<uint4*>(&sh.w.vs[hs][TPW * wv + i][8 * j]) = vrow[i];
                }
            }
        } else if (c0 == 0) {
#pragma unroll
            for (int i = 0; i < kVPre; ++i) {
                const int idx = tl + i * 256;
                const int t = idx / (wdt / 8), c8 = idx % (wdt / 8);
                if (idx < CK * (wdt / 8)) *reinterpret_cast<uint4*>(&sh.w.vs[grp][t][c8 * 8]) = vpre[i];
            }
        } else {
            for (int idx = tl; idx < CK * (wdt / 8); idx += 256) {
                const int t = idx / (wdt / 8), c8 = idx % (wdt / 8);
                uint4 vv = make_uint4(0, 0, 0, 0);
                if (t0 + t < T)
                    vv = *reinterpret_cast<const uint4*>(v + (((int64_t)b * T + t0 + t) * Hv + hv) * Dv + c0 + c8 * 8);
                *reinterpret_cast<uint4*>(&sh.w.vs[grp][t][c8 * 8]) = vv;
            }
        }
        __syncthreads();
        for (int rb = wl; rb < wdt / 16; rb += 4) {
            const int col = 16 * rb + lr;
            const auto& vsh = sh.w.vs[grp];
            u4_t vb;
#pragma unroll
            for (int p = 0; p < 4; ++p)
                vb[p] = (uint32_t)vsh[8 * lq + 2 * p][col] | ((uint32_t)vsh[8 * lq + 2 * p + 1][col] << 16);
            const f4_t zero = {0.f, 0.f, 0.f, 0.f};
            u4_t* dst = o.u + (unit * (Dv / 16) + c0 / 16 + rb) * 2 * 64 + lane;
            dst[0] = __builtin_bit_cast(u4_t, mma3a(tb[0], vb, zero));
            dst[64] = __builtin_bit_cast(u4_t, mma3a(tb[1], vb, zero));
        }
        __syncthreads();
    }
}

// ============================================================ sequential pass

struct SeqIn {
    const u4_t* wsw;
    const u4_t* u;
    const u4_t* pn;
    const float* rg;
    const u4_t* qsw;
    const u4_t* ksw;
};

// Per-block constants of the sequential pass.  `wv` is the wave index held
// in a scalar register, so role branches and address arithmetic stay scalar.
struct SeqCtx {
    int64_t unit0, kunit0;      // first chunk of this (b, hv) and of its (b, hk)
    int tile0, row_tiles;       // this block's first 16-row tile, Dv / 16
    int wv, lane;
};

// A wave-uniform pointer moved to scalar registers, so that loads through it
// take the scalar-base form (the per-lane part is one fixed 32-bit offset)
// and no address registers are rewritten while earlier loads are in flight.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* uniform_ptr(const T* p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return (const __attribute__((address_space(1))) T*)(((uint64_t)hi << 32) | lo);
}

template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* uniform_ptr_w(T* p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return (__attribute__((address_space(1))) T*)(((uint64_t)hi << 32) | lo);
}

// One chunk's operands in registers (NR row tiles of 16 state rows).
template <int NR, bool PK = false>
struct SeqOps {
    f4_t wf[2][2];    // W of t-tiles 0 and 1 (f32, elements 0..3 and 4..7)
    u4_t q[2];        // q, t-tiles 0 and 1 (per-key form: Q o Gamma, leading plane)
    u4_t k[2];        // k^T, this wave's two column tiles (per-head form)
    u4_t a0[NR];      // -Tb V of t-tile (wave & 1), per row tile (f32 bits; waves 0, 1 use it)
    float rg;         // -rho[lane] (lanes 0..31), gamma[lane - 32] (lanes 32..63)
    // per-key form: Q o Gamma's second plane, -(K o E)^T in f32 (this wave's
    // column tiles tt, t-tiles jt) and Gamma_{C-1} at this lane's state
    // columns 32 w + 16 tt + 4 q .. + 3
    u4_t qm[2];
    f4_t kf[2][2];
    f4_t gd[2];

    // Loads of one chunk in four parts, so that the sequential pass can
    // spread them over the step it overlaps (part 0: W tile 0, 1: W tile 1,
    // 2: q and k, 3: the rest).  Every wave issues the same number of loads
    // (role-independent counts keep the memory waits exact).
    template <int PART>
    __device__ __forceinline__ void load(const SeqIn& in, const SeqCtx& x, int c) {
        const int64_t unit = x.unit0 + c, kunit = x.kunit0 + c;
        const int wv = x.wv, lane = x.lane;
        if constexpr (PART <= 1) {
            const auto ws = uniform_ptr(in.wsw + unit * kWVec + wv * 4 * 64 + PART * 2 * 64);
            wf[PART][0] = __builtin_bit_cast(f4_t, ws[lane]);
            wf[PART][1] = __builtin_bit_cast(f4_t, ws[64 + lane]);
        } else if constexpr (PART == 2 && PK) {
            const auto qs = uniform_ptr(in.qsw + unit * 2 * kQVec + wv * 2 * 64);
            const auto ks = uniform_ptr(in.ksw + unit * 2 * kQVec + wv * 4 * 64);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                q[t] = qs[t * 64 + lane];
                qm[t] = qs[kQVec + t * 64 + lane];
                kf[t][0] = __builtin_bit_cast(f4_t, ks[(2 * t) * 64 + lane]);
                kf[t][1] = __builtin_bit_cast(f4_t, ks[(2 * t + 1) * 64 + lane]);
            }
            const auto gs = uniform_ptr(reinterpret_cast<const f4_t*>(in.rg + unit * rg_floats<true>() + 2 * CK + 32 * wv));
            gd[0] = gs[lane >> 4];
            gd[1] = gs[4 + (lane >> 4)];
        } else if constexpr (PART == 2) {
            const auto qs = uniform_ptr(in.qsw + kunit * kQVec + wv * 2 * 64);
            const auto ks = uniform_ptr(in.ksw + kunit * kQVec + wv * 2 * 64);
            q[0] = qs[lane];
            q[1] = qs[64 + lane];
            k[0] = ks[lane];
            k[1] = ks[64 + lane];
        } else {
            // every state wave loads a -Tb V tile (waves 0, 1 add theirs; equal
            // load counts keep the memory waits exact) and rho/gamma
#pragma unroll
            for (int rt = 0; rt < NR; ++rt)
                a0[rt] = uniform_ptr(in.u + ((unit * x.row_tiles + x.tile0 + rt) * 2 + (wv & 1)) * 64)[lane];
            rg = uniform_ptr(in.rg + unit * rg_floats<PK>())[lane];
        }
    }

    __device__ __forceinline__ void load_all(const SeqIn& in, const SeqCtx& x, int c) {
        load<0>(in, x, c);
        load<1>(in, x, c);
        load<2>(in, x, c);
        load<3>(in, x, c);
    }
};

// keeps the instructions of the enclosed part where they are written
#define SEQ_PIN(stmt)                          \
    do {                                       \
        __builtin_amdgcn_sched_barrier(0);     \
        stmt;                                  \
        __builtin_amdgcn_sched_barrier(0);     \
    } while (0)

// Six waves per block: waves 0..3 hold the state (32 columns each) of NR
// tiles of 16 rows and run the chunk chain; waves 4, 5 finish y of the
// previous chunk (one t-tile each, every row tile) off that chain.  Buffers
// the output waves read one chunk late are kept three deep.  With NR = 2 a
// block serves 32 rows: the chunk's W, q, k and -P are loaded once for both
// tiles and the tiles' independent products interleave; the grid halves,
// which pays once it would exceed one block per CU (a CU runs one block of
// this kernel at a time).  Each tile's arithmetic is the same either way.
constexpr int NWY = 2;
constexpr int SEQ_THREADS = 64 * (NW + NWY);

template <int NR>
struct SeqSmem {
    f4_t x[2][NR][NW * 2 * 64];   // per-wave shares of W S^T - Tb V, by chunk parity
    f4_t y[3][NR][NW * 2 * 64];   // per-wave shares of S Q^T (transposed Y'), chunk mod 3
    float rg[3][2 * CK];          // -rho (kperm order) and gamma of the chunk, chunk mod 3
    f4_t d[2][NR][2][64];         // D of the chunk (B-operand layout), by chunk parity
};

template <int NR, bool PK = false>
__global__ __launch_bounds__(SEQ_THREADS) void chunk_seq_kernel(SeqIn in, const float* state_in,
                                                                float* state_out, uint16_t* __restrict__ y,
                                                                const uint8_t* __restrict__ mask, int T, int Hk,
                                                                int Hv, int Dv, int NC, int row_blocks,
                                                                int n_blocks) {
    __shared__ SeqSmem<NR> sh;

    int lb = blockIdx.x;
    if ((n_blocks & 7) == 0) lb = (lb & 7) * (n_blocks >> 3) + (lb >> 3);
    const int n = lb / row_blocks;
    const int rblk = lb % row_blocks;
    const int b = n / Hv, hv = n % Hv;
    const int hk = hv / (Hv / Hk);
    const int r0 = rblk * RB * NR;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lq = lane >> 4;
    const f4_t zero = {0.f, 0.f, 0.f, 0.f};
    const NegOnes no = neg_ones();
    const int64_t vstride = (int64_t)Hv * Dv;     // one step of y
    const int64_t unit0 = (int64_t)n * NC;

    if (wv >= NW) {
        // ------------------------------------------------ output waves
        // y rows of t-tile jt: Y^T = gamma_t (S Q^T) + D^T (-P)^T, with the
        // leading planes of D and P (2^-16 relative, below y's rounding)
        const int jt = wv - NW;
        const int yt = 16 * jt + lr;
        uint16_t* y0 = y + ((int64_t)b * T * Hv + hv) * Dv + r0;
        const uint32_t yoff = (uint32_t)(yt * vstride + 4 * lq);
        u4_t ch = {0, 0, 0, 0}, cm = ch;              // -P planes of the chunk finished next
        int b3 = 0;                                   // (c - 1) mod 3
        for (int c = 0; c <= NC; ++c) {
            const auto ps = uniform_ptr(in.pn + (unit0 + min(c, NC - 1)) * kPVec + jt * 2 * 64);
            const u4_t nh = ps[lane], nm = ps[64 + lane];
            __syncthreads();                          // chunk c's barrier (c == NC: the final one)
            if (c > 0) {
                const int cp = c - 1;
                const int t = cp * CK + yt;
#pragma unroll
                for (int rt = 0; rt < NR; ++rt) {
                    const f4_t* yb = sh.y[b3][rt];
                    const f4_t q0 = yb[jt * 64 + lane], q1 = yb[(2 + jt) * 64 + lane];
                    const f4_t q2 = yb[(4 + jt) * 64 + lane], q3 = yb[(6 + jt) * 64 + lane];
                    f4_t ys = (q0 + q1) + (q2 + q3);
                    ys = ys * sh.rg[b3][CK + yt];
                    u4_t dh, dm;
                    split8hm(no, sh.d[cp & 1][rt][0][lane], sh.d[cp & 1][rt][1][lane], dh, dm);
                    ys = mma(dm, ch, ys);
                    ys = mma(dh, cm, ys);
                    ys = mma(dh, ch, ys);
                    if (t < T) {
                        u2_t w = {pack_bf16x2(ys[0], ys[1]), pack_bf16x2(ys[2], ys[3])};
                        if (mask != nullptr && mask[(int64_t)b * T + t] == 0) w = u2_t{0, 0};   // masked step
                        *reinterpret_cast<__attribute__((address_space(1))) u2_t*>(
                            uniform_ptr_w(y0 + (int64_t)cp * CK * vstride + RB * rt) + yoff) = w;
                    }
                }
                b3 = b3 == 2 ? 0 : b3 + 1;
            }
            ch = nh;
            cm = nm;
        }
        return;
    }

    // ---------------------------------------------------- state waves
    // the state chain takes issue priority over the output waves sharing
    // its SIMDs (measured 114.2 -> 111.3 us at the prefill workload)
    __builtin_amdgcn_s_setprio(2);
    SeqCtx x;
    x.unit0 = unit0;
    x.kunit0 = ((int64_t)b * Hk + hk) * NC;
    x.tile0 = rblk * NR;
    x.row_tiles = Dv / RB;
    x.wv = wv;
    x.lane = lane;

    // row tile rt, state tile tt, register i: S[r0 + 16 rt + lr][32 wv + 16 tt + 4 lq + i]
    f4_t S[NR][2];
    float* sp_out = state_out + ((int64_t)n * Dv + r0) * DKC + 32 * wv;
    const uint32_t soff = lr * DKC + 4 * lq;
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) {
        if (state_in) {
            const float* sp = state_in + ((int64_t)n * Dv + r0 + RB * rt) * DKC + 32 * wv;
            S[rt][0] = *reinterpret_cast<const f4_t*>(sp + soff);
            S[rt][1] = *reinterpret_cast<const f4_t*>(sp + soff + 16);
        } else {
            S[rt][0] = zero;
            S[rt][1] = zero;
        }
    }

    // one chunk c (b3 = c mod 3) with o; the loads of chunk cn into nx are
    // spread over it (n1, the next chunk's set, is already in flight)
    auto step = [&](int c, int b3, const SeqOps<NR, PK>& o, SeqOps<NR, PK>& n1, SeqOps<NR, PK>& nx, int cn) {
        (void)n1;
        SEQ_PIN(nx.template load<0>(in, x, cn));

        // this wave's share of W S^T - Tb V (rows t, columns r), two t-tiles
        // per row tile, on the f32 matrix instruction: element e of quarter
        // lq of W's row and of S's row is column kperm(lq, e), so element e
        // of both is the operand of product e (four columns, one per quarter)
        f4_t x0[NR], x1[NR];
#pragma unroll
        for (int rt = 0; rt < NR; ++rt) {
            x0[rt] = zero;
            x1[rt] = zero;
            if (wv == 0) x0[rt] = __builtin_bit_cast(f4_t, o.a0[rt]);
            else if (wv == 1) x1[rt] = __builtin_bit_cast(f4_t, o.a0[rt]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
#pragma unroll
            for (int rt = 0; rt < NR; ++rt) {
                x0[rt] = mma_f32(o.wf[0][e >> 2][e & 3], S[rt][e >> 2][e & 3], x0[rt]);
                x1[rt] = mma_f32(o.wf[1][e >> 2][e & 3], S[rt][e >> 2][e & 3], x1[rt]);
            }
        }
        // the state's two leading bf16 planes, for S Q^T (y is rounded to
        // bf16: 2^-16 relative suffices)
        u4_t s_h[NR], s_m[NR];
#pragma unroll
        for (int rt = 0; rt < NR; ++rt) split8hm(no, S[rt][0], S[rt][1], s_h[rt], s_m[rt]);

        SEQ_PIN(nx.template load<1>(in, x, cn));

#pragma unroll
        for (int rt = 0; rt < NR; ++rt) {
            f4_t* xb = sh.x[c & 1][rt];
            xb[(2 * wv) * 64 + lane] = x0[rt];
            xb[(2 * wv + 1) * 64 + lane] = x1[rt];
        }
        float* rg = sh.rg[b3];
        if (wv == 0) rg[lane] = o.rg;
        __syncthreads();

        SEQ_PIN(nx.template load<2>(in, x, cn));
        // D = W S^T - Tb V = -Delta: the shares of waves 0, 1 and of waves 2, 3
        // summed, then the two sums (identical in every wave)
        f4_t d0[NR], d1[NR];
#pragma unroll
        for (int rt = 0; rt < NR; ++rt) {
            const f4_t* xb = sh.x[c & 1][rt];
            const f4_t p00 = xb[0 * 64 + lane], p10 = xb[2 * 64 + lane], p20 = xb[4 * 64 + lane], p30 = xb[6 * 64 + lane];
            const f4_t p01 = xb[1 * 64 + lane], p11 = xb[3 * 64 + lane], p21 = xb[5 * 64 + lane], p31 = xb[7 * 64 + lane];
            d0[rt] = (p00 + p10) + (p20 + p30);
            d1[rt] = (p01 + p11) + (p21 + p31);
        }

        if constexpr (PK) {
            // per-key: S = S diag(Gamma_{C-1}) + Delta^T (K o E), Delta = -D,
            // as the six plane products of -(K o E)^T (cut here from its f32
            // operand, off the state chain) with D: element e of both is step
            // kperm(q, e), the contraction layout of the bf16 products
#pragma unroll
            for (int rt = 0; rt < NR; ++rt) {
                const Planes dp = split8(no, d0[rt], d1[rt]);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const Planes kp = split8(no, o.kf[tt][0], o.kf[tt][1]);
                    S[rt][tt] = S[rt][tt] * o.gd[tt];
                    S[rt][tt] = mma6(kp, dp, S[rt][tt]);
                }
            }
        } else {
            // S = gamma_{C-1} S + K^T (diag(rho) Delta)
            const f4_t rh0 = *reinterpret_cast<const f4_t*>(rg + 8 * lq);
            const f4_t rh1 = *reinterpret_cast<const f4_t*>(rg + 8 * lq + 4);
            const float gc = rg[2 * CK - 1];
            Planes bs[NR];
#pragma unroll
            for (int rt = 0; rt < NR; ++rt) bs[rt] = split8(no, rh0 * d0[rt], rh1 * d1[rt]);
#pragma unroll
            for (int rt = 0; rt < NR; ++rt) {
                S[rt][0] = S[rt][0] * gc;
                S[rt][1] = S[rt][1] * gc;
                S[rt][0] = mma3b(o.k[0], bs[rt], S[rt][0]);
                S[rt][1] = mma3b(o.k[1], bs[rt], S[rt][1]);
            }
        }
        // this wave's share of S Q^T (rows r, columns t) from the planes of the
        // state before the update, issued after the update's products so
        // that they fill the matrix pipe while the update completes (the
        // output waves read it one chunk later); y is rounded to bf16, so the
        // state's two leading planes suffice (2^-16)
#pragma unroll
        for (int rt = 0; rt < NR; ++rt) {
            f4_t y0v, y1v;
            if constexpr (PK) {
                // Q o Gamma in two planes: h.h, h.m and m.h
                y0v = mma(s_m[rt], o.q[0], zero);
                y1v = mma(s_m[rt], o.q[1], zero);
                y0v = mma(s_h[rt], o.qm[0], y0v);
                y1v = mma(s_h[rt], o.qm[1], y1v);
                y0v = mma(s_h[rt], o.q[0], y0v);
                y1v = mma(s_h[rt], o.q[1], y1v);
            } else {
                y0v = mma(s_m[rt], o.q[0], zero);
                y1v = mma(s_m[rt], o.q[1], zero);
                y0v = mma(s_h[rt], o.q[0], y0v);
                y1v = mma(s_h[rt], o.q[1], y1v);
            }
            f4_t* yb = sh.y[b3][rt];
            yb[(2 * wv) * 64 + lane] = y0v;
            yb[(2 * wv + 1) * 64 + lane] = y1v;
        }

        if (wv == 0) {
#pragma unroll
            for (int rt = 0; rt < NR; ++rt) {
                sh.d[c & 1][rt][0][lane] = d0[rt];
                sh.d[c & 1][rt][1][lane] = d1[rt];
            }
        }
        SEQ_PIN(nx.template load<3>(in, x, cn));
    };

    // three operand sets: chunk c + 2 loads while chunk c runs
    SeqOps<NR, PK> o0, o1, o2;
    o0.load_all(in, x, 0);
    o1.load_all(in, x, min(1, NC - 1));
    int c = 0;
    for (; c + 3 <= NC; c += 3) {     // one exit: the sets rotate through whole rounds
        step(c, 0, o0, o1, o2, min(c + 2, NC - 1));
        step(c + 1, 1, o1, o2, o0, min(c + 3, NC - 1));
        step(c + 2, 2, o2, o0, o1, min(c + 4, NC - 1));
    }
    if (c < NC) step(c, 0, o0, o1, o2, min(c + 2, NC - 1));
    if (c + 1 < NC) step(c + 1, 1, o1, o2, o0, min(c + 3, NC - 1));
    __syncthreads();                  // the output waves' last chunk

#pragma unroll
    for (int rt = 0; rt < NR; ++rt) {
        float* so = sp_out + (int64_t)RB * rt * DKC;
        *reinterpret_cast<f4_t*>(so + soff) = S[rt][0];
        *reinterpret_cast<f4_t*>(so + soff + 16) = S[rt][1];
    }
}

// ========================================== sequential pass, row-wave pairs

// For grids of more than two row tiles per CU: two waves per 16-row state
// tile, each over one half of the Dk columns (two of the four 32-column
// slices), eight waves (64 rows of one v-head) per block, so that every SIMD
// holds two waves whose matrix products and vector work interleave.  The two
// halves of a tile exchange their shares of W S^T - Tb V and of S Q^T
// through LDS once per chunk; each half updates its own state columns and
// finishes y for one t-tile.  The chunk's W, q, k, -P and rho/gamma are
// staged by the whole block into a three-slot LDS ring two chunks ahead;
// -Tb V, read by one wave per tile, is loaded by that wave one chunk ahead.
// One barrier per chunk, between the shares and their sums: the exchange
// buffer is double-buffered, and a ring slot is refilled after the barrier
// of the step following its last read.  Slice s takes the part of
// chunk_seq_kernel's wave s and every sum is formed in that kernel's order,
// so the results are bit-identical to it.
constexpr int PWW = 8;                                        // waves per block: 4 row tiles x 2 halves
constexpr int PW_TILES = PWW / 2;
constexpr int PW_THREADS = 64 * PWW;
constexpr int PW_Q = kWVec, PW_K = PW_Q + kQVec, PW_P = PW_K + kQVec, PW_VEC = PW_P + kPVec;
static_assert(kWVec == 2 * PW_THREADS && kQVec == PW_THREADS && 2 * kPVec == PW_THREADS,
              "staging: two W vectors, one q and one k vector per thread, -P by half the threads");

struct PairSmem {
    struct Slot {
        u4_t v[PW_VEC];       // W | q | k | -P, in the workspace layout
        float rg[2 * CK];     // -rho (kperm order), gamma
    } ring[3];
    // per chunk parity and wave: its half's W S^T - Tb V share (t-tiles 0, 1)
    // and its S Q^T share of the t-tile the other half finishes
    f4_t ex[2][PWW][3][64];
};
static_assert(sizeof(PairSmem) <= 160 * 1024, "LDS of one CU");

__global__ __launch_bounds__(PW_THREADS) void chunk_seq_pairs_kernel(SeqIn in, const float* state_in,
                                                                     float* state_out, uint16_t* __restrict__ y,
                                                                     const uint8_t* __restrict__ mask, int T, int Hk,
                                                                     int Hv, int Dv, int NC, int row_blocks,
                                                                     int n_blocks) {
    __shared__ PairSmem sm;

    int lb = blockIdx.x;
    if ((n_blocks & 7) == 0) lb = (lb & 7) * (n_blocks >> 3) + (lb >> 3);
    const int n = lb / row_blocks;
    const int rblk = lb % row_blocks;
    const int b = n / Hv, hv = n % Hv;
    const int hk = hv / (Hv / Hk);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hf = wv / PW_TILES;                 // column half: slices 2 hf, 2 hf + 1
    // the later-launched half takes issue priority on the SIMD the two halves
    // share, so that it does not trail the other into each barrier
    // (measured 2506 -> 2479 us at the long prefill)
    if (hf == 1) __builtin_amdgcn_s_setprio(1);
    const int tile = rblk * PW_TILES + wv % PW_TILES;
    const int lr = lane & 15, lq = lane >> 4;
    const int r0 = tile * RB;                     // this wave's first state row
    const int row_tiles = Dv / RB;
    const int64_t unit0 = (int64_t)n * NC, kunit0 = ((int64_t)b * Hk + hk) * NC;
    const f4_t zero = {0.f, 0.f, 0.f, 0.f};
    const NegOnes no = neg_ones();
    const int64_t vstride = (int64_t)Hv * Dv;     // one step of y

    // tile tt of this half, register i: S[r0 + lr][64 hf + 16 tt + 4 lq + i]
    f4_t S[4];
    const int64_t soff = ((int64_t)n * Dv + r0 + lr) * DKC + 64 * hf + 4 * lq;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
        S[tt] = state_in ? *reinterpret_cast<const f4_t*>(state_in + soff + 16 * tt) : zero;

    // -Tb V of this tile's two t-tiles (added by half 0), one chunk ahead
    f4_t un[2] = {zero, zero};
    auto u_load = [&](int c) {
        if (hf == 0) {
            const auto su = uniform_ptr(in.u + ((unit0 + c) * row_tiles + tile) * 2 * 64);
            un[0] = __builtin_bit_cast(f4_t, su[lane]);
            un[1] = __builtin_bit_cast(f4_t, su[64 + lane]);
        }
    };
    // staging of chunk c by the whole block, coalesced: loads now, LDS stores later
    u4_t g[5], grg = {0, 0, 0, 0};
    auto stage_load = [&](int c) {
        const int64_t unit = unit0 + c, kunit = kunit0 + c;
        const auto sw = uniform_ptr(in.wsw + unit * kWVec);
        g[0] = sw[tid];
        g[1] = sw[PW_THREADS + tid];
        g[2] = uniform_ptr(in.qsw + kunit * kQVec)[tid];
        g[3] = uniform_ptr(in.ksw + kunit * kQVec)[tid];
        if (wv < PWW / 2) g[4] = uniform_ptr(in.pn + unit * kPVec)[tid];
        if (tid < 2 * CK / 4) grg = uniform_ptr(reinterpret_cast<const u4_t*>(in.rg + unit * 2 * CK))[tid];
    };
    auto stage_store = [&](int slot) {
        PairSmem::Slot& st = sm.ring[slot];
        st.v[tid] = g[0];
        st.v[PW_THREADS + tid] = g[1];
        st.v[PW_Q + tid] = g[2];
        st.v[PW_K + tid] = g[3];
        if (wv < PWW / 2) st.v[PW_P + tid] = g[4];
        if (tid < 2 * CK / 4) reinterpret_cast<u4_t*>(st.rg)[tid] = grg;
    };

    stage_load(0);
    stage_store(0);
    if (NC > 1) {
        stage_load(1);
        stage_store(1);
    }
    u_load(0);
    __syncthreads();

    uint16_t* yw = y + ((int64_t)b * T * Hv + hv) * Dv + r0 + 4 * lq;
    const int yt = 16 * hf + lr;                  // this wave finishes y of t-tile hf
    int slot = 0;
    for (int c = 0; c < NC; ++c) {
        const bool pre = c + 2 < NC;
        // the mask byte of this lane's step, loaded before the staging loads
        // so that its wait does not cover those
        bool keep = true;
        if (mask != nullptr) keep = mask[(int64_t)b * T + min(c * CK + yt, T - 1)] != 0;
        const f4_t uc0 = un[0], uc1 = un[1];
        if (c + 1 < NC) u_load(c + 1);
        if (pre) stage_load(c + 2);
        const PairSmem::Slot& o = sm.ring[slot];

        // this half's slices of W S^T - Tb V, each as the wave of chunk_seq_kernel
        // with that slice forms its share (-Tb V enters slice 0's t-tile 0 and
        // slice 1's t-tile 1)
        f4_t x[2][2];
        x[0][0] = hf == 0 ? uc0 : zero;
        x[0][1] = zero;
        x[1][0] = zero;
        x[1][1] = hf == 0 ? uc1 : zero;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int sl = 2 * hf + j;
            f4_t wf[2][2];
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                wf[jt][0] = __builtin_bit_cast(f4_t, o.v[(sl * 4 + jt * 2) * 64 + lane]);
                wf[jt][1] = __builtin_bit_cast(f4_t, o.v[(sl * 4 + jt * 2 + 1) * 64 + lane]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                x[j][0] = mma_f32(wf[0][e >> 2][e & 3], S[2 * j + (e >> 2)][e & 3], x[j][0]);
                x[j][1] = mma_f32(wf[1][e >> 2][e & 3], S[2 * j + (e >> 2)][e & 3], x[j][1]);
            }
        }
        // S Q^T shares of the two slices from the state's two leading planes
        f4_t yp[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int sl = 2 * hf + j;
            u4_t s_h, s_m;
            split8hm(no, S[2 * j], S[2 * j + 1], s_h, s_m);
            const u4_t q0 = o.v[PW_Q + (sl * 2) * 64 + lane], q1 = o.v[PW_Q + (sl * 2 + 1) * 64 + lane];
            yp[j][0] = mma(s_m, q0, zero);
            yp[j][1] = mma(s_m, q1, zero);
            yp[j][0] = mma(s_h, q0, yp[j][0]);
            yp[j][1] = mma(s_h, q1, yp[j][1]);
        }
        const f4_t xh0 = x[0][0] + x[1][0], xh1 = x[0][1] + x[1][1];
        const f4_t yh0 = yp[0][0] + yp[1][0], yh1 = yp[0][1] + yp[1][1];
        f4_t(*ex)[64] = sm.ex[c & 1][wv];
        ex[0][lane] = xh0;
        ex[1][lane] = xh1;
        ex[2][lane] = hf == 0 ? yh1 : yh0;        // for the other half's t-tile
        __syncthreads();

        // D = W S^T - Tb V = -Delta: (slices 0 + 1) + (slices 2 + 3); the
        // two halves add the same two sums (addition commutes exactly)
        const f4_t(*px)[64] = sm.ex[c & 1][wv ^ PW_TILES];
        const f4_t d0 = xh0 + px[0][lane], d1 = xh1 + px[1][lane];
        const f4_t ys = (hf == 0 ? yh0 : yh1) + px[2][lane];

        // S = gamma_{C-1} S + K^T (diag(rho) Delta) over this half's columns
        const f4_t rh0 = *reinterpret_cast<const f4_t*>(o.rg + 8 * lq);
        const f4_t rh1 = *reinterpret_cast<const f4_t*>(o.rg + 8 * lq + 4);
        const float gc = o.rg[2 * CK - 1];
        const Planes bs = split8(no, rh0 * d0, rh1 * d1);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            S[tt] = S[tt] * gc;
            S[tt] = mma3b(o.v[PW_K + (4 * hf + tt) * 64 + lane], bs, S[tt]);
        }

        // y of t-tile hf: Y^T = gamma_t (S Q^T) + D^T (-P)^T, leading planes of D and P
        u4_t dh, dm;
        split8hm(no, d0, d1, dh, dm);
        f4_t yv = ys * o.rg[CK + yt];
        const u4_t ch = o.v[PW_P + (hf * 2) * 64 + lane], cm = o.v[PW_P + (hf * 2 + 1) * 64 + lane];
        yv = mma(dm, ch, yv);
        yv = mma(dh, cm, yv);
        yv = mma(dh, ch, yv);
        const int t = c * CK + yt;
        if (t < T) {
            u2_t w = {pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3])};
            if (!keep) w = u2_t{0, 0};   // masked step
            *reinterpret_cast<u2_t*>(yw + (int64_t)t * vstride) = w;
        }

        if (pre) stage_store(slot == 0 ? 2 : slot - 1);    // slot of chunk c + 2, last read in step c - 1
        slot = slot == 2 ? 0 : slot + 1;
    }

#pragma unroll
    for (int tt = 0; tt < 4; ++tt) *reinterpret_cast<f4_t*>(state_out + soff + 16 * tt) = S[tt];
}

// ================================================================== launch

// Lane offsets of v and y rows inside a chunk are 32-bit: Hv * Dv <= 2^25.
bool chunked_supported(int Hv, int Dk, int Dv) {
    return Dk == DKC && Dv % RB == 0 && (int64_t)Hv * Dv <= (int64_t(1) << 25);
}

ChunkedLayout chunked_layout(int B, int T, int Hk, int Hv, int Dk, int Dv, bool per_key) {
    (void)Dk;
    ChunkedLayout L;
    const int64_t NC = (T + CK - 1) / CK;
    const uint64_t units = (uint64_t)B * Hv * NC;
    const uint64_t kunits = (uint64_t)B * Hk * NC;
    auto a256 = [](uint64_t x) { return (x + 255) & ~uint64_t(255); };
    L.nc = (int)NC;
    L.wsw = 0;
    L.u = L.wsw + a256(units * kWVec * 16);
    L.pn = L.u + a256(units * CK * (uint64_t)Dv * 4);
    L.rg = L.pn + a256(units * kPVec * 16);
    if (per_key) {
        // Q o Gamma (two planes) and (K o E)^T (three) per v-unit, Gamma_{C-1} in the decay record
        L.qsw = L.rg + a256(units * rg_floats<true>() * 4);
        L.ksw = L.qsw + a256(units * 2 * kQVec * 16);
        L.total = L.ksw + a256(units * 2 * kQVec * 16);
    } else {
        L.qsw = L.rg + a256(units * 2 * CK * 4);
        L.ksw = L.qsw + a256(kunits * kQVec * 16);
        L.total = L.ksw + a256(kunits * kQVec * 16);
    }
    return L;
}

int64_t chunked_blocks(int B, int T, int Hv, int Dv) {
    const int64_t NC = (T + CK - 1) / CK;
    return std::max<int64_t>((int64_t)B * Hv * NC, (int64_t)B * Hv * (Dv / RB));
}

bool layer_chunked_fusable(int Dv, int K) { return Dv <= 128 && K >= 2 && K <= 4; }

static hipError_t launch_chunked(const RecurrentArgs& a, const PrologueIn* pin, int K, void* ws,
                                 hipStream_t stream);

hipError_t launch_recurrent_chunked(const RecurrentArgs& a, void* ws, hipStream_t stream) {
    return launch_chunked(a, nullptr, 0, ws, stream);
}

// An in-place conv state is read and rewritten by the same lane of the chunk-0
// block that owns the channel; that is race-free when no other block reads
// the channel, i.e. when one preparation block serves each k-head (Hv / Hk
// of 1 or 2).  Otherwise the preparation leaves the conv state alone and a
// copy after it writes the new one (its rows are the last K - 1 tokens).
hipError_t launch_layer_chunked(const RecurrentArgs& a, const PrologueIn& p, int K, void* ws, hipStream_t stream) {
    if (!layer_chunked_fusable(a.Dv, K)) return hipErrorInvalidValue;
    const bool in_place = p.conv_state_out != nullptr && p.conv_state_out == p.conv_state_in;
    if (!in_place || a.Hv / a.Hk <= 2) return launch_chunked(a, &p, K, ws, stream);
    if (a.T < K - 1) return hipErrorInvalidValue;
    PrologueIn pn = p;
    pn.conv_state_out = nullptr;
    const hipError_t e = launch_chunked(a, &pn, K, ws, stream);
    if (e != hipSuccess) return e;
    const int C = 2 * a.Hk * a.Dk + a.Hv * a.Dv;
    return launch_conv_tail(p.qkv, p.conv_state_out, a.B, a.T, C, K, stream);
}

// The current device's CU count, looked up once per device (0 if unknown).
int device_cu_count() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 0) cus = 0;
    if (dev < kMaxDevices && cus > 0) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

static hipError_t launch_chunked(const RecurrentArgs& a, const PrologueIn* pin, int K, void* ws,
                                 hipStream_t stream) {
    if (!chunked_supported(a.Hv, a.Dk, a.Dv) || a.T <= 0 || a.B <= 0) return hipErrorInvalidValue;
    if (a.g_per_key && pin) return hipErrorInvalidValue;      // the per-key form takes prepared inputs
    const ChunkedLayout L = chunked_layout(a.B, a.T, a.Hk, a.Hv, a.Dk, a.Dv, a.g_per_key);
    char* base = static_cast<char*>(ws);
    ChunkPtrs o;
    o.wsw = reinterpret_cast<u4_t*>(base + L.wsw);
    o.u = reinterpret_cast<u4_t*>(base + L.u);
    o.pn = reinterpret_cast<u4_t*>(base + L.pn);
    o.rg = reinterpret_cast<float*>(base + L.rg);
    o.qsw = reinterpret_cast<u4_t*>(base + L.qsw);
    o.ksw = reinterpret_cast<u4_t*>(base + L.ksw);
    // two v-heads per preparation block when the GQA group size is even
    // (per-key form: one)
    const int nh = !a.g_per_key && (a.Hv / a.Hk) % 2 == 0 ? 2 : 1;
    const int64_t pblocks = (int64_t)a.B * (a.Hv / nh) * L.nc;
    const PrologueIn none{};
    const PrologueIn& pi = pin ? *pin : none;
#define GDN_PREP(KF_, NH_)                                                                                     \
    hipLaunchKernelGGL((chunk_prep_kernel<KF_, NH_>), dim3((unsigned)pblocks), dim3(256 * NH_), 0, stream, a.q, \
                       a.k, a.g, a.beta, a.mask, a.v, pi, o, a.T, a.Hk, a.Hv, a.Dv, L.nc)
    if (a.g_per_key)
        hipLaunchKernelGGL((chunk_prep_kernel<0, 1, true>), dim3((unsigned)pblocks), dim3(256), 0, stream, a.q, a.k,
                           a.g, a.beta, a.mask, a.v, pi, o, a.T, a.Hk, a.Hv, a.Dv, L.nc);
    else switch (K * 2 + nh - 1) {
        case 0: GDN_PREP(0, 1); break;
        case 1: GDN_PREP(0, 2); break;
        case 4: GDN_PREP(2, 1); break;
        case 5: GDN_PREP(2, 2); break;
        case 6: GDN_PREP(3, 1); break;
        case 7: GDN_PREP(3, 2); break;
        case 8: GDN_PREP(4, 1); break;
        case 9: GDN_PREP(4, 2); break;
        default: return hipErrorInvalidValue;
    }
#undef GDN_PREP
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    SeqIn in;
    in.wsw = o.wsw;
    in.u = o.u;
    in.pn = o.pn;
    in.rg = o.rg;
    in.qsw = o.qsw;
    in.ksw = o.ksw;
    // two row tiles per block once one tile per block would need more blocks
    // than the device has CUs (the sequential blocks run one per CU); two
    // waves per row tile, four tiles per block (chunk_seq_pairs_kernel), once
    // two tiles per block would still need more
    const int cus = device_cu_count();
    const int64_t tiles = (int64_t)a.B * a.Hv * (a.Dv / RB);
    if (!a.g_per_key && a.Dv % (PW_TILES * RB) == 0 && cus > 0 && tiles > 2 * (int64_t)cus) {
        const int rb = a.Dv / (PW_TILES * RB);
        const int64_t nb = (int64_t)a.B * a.Hv * rb;
        hipLaunchKernelGGL(chunk_seq_pairs_kernel, dim3((unsigned)nb), dim3(PW_THREADS), 0, stream, in, a.state_in,
                           a.state_out, a.y, a.mask, a.T, a.Hk, a.Hv, a.Dv, L.nc, rb, (int)nb);
        return hipGetLastError();
    }
    const bool two = !a.g_per_key && a.Dv % (2 * RB) == 0 && cus > 0 && (int64_t)a.B * a.Hv * (a.Dv / RB) > cus;
    const int row_blocks = a.Dv / (RB * (two ? 2 : 1));
    const int64_t blocks = (int64_t)a.B * a.Hv * row_blocks;
    if (a.g_per_key)
        hipLaunchKernelGGL((chunk_seq_kernel<1, true>), dim3((unsigned)blocks), dim3(SEQ_THREADS), 0, stream, in,
                           a.state_in, a.state_out, a.y, a.mask, a.T, a.Hk, a.Hv, a.Dv, L.nc, row_blocks, (int)blocks);
    else if (two)
        hipLaunchKernelGGL(chunk_seq_kernel<2>, dim3((unsigned)blocks), dim3(SEQ_THREADS), 0, stream, in,
                           a.state_in, a.state_out, a.y, a.mask, a.T, a.Hk, a.Hv, a.Dv, L.nc, row_blocks, (int)blocks);
    else
        hipLaunchKernelGGL(chunk_seq_kernel<1>, dim3((unsigned)blocks), dim3(SEQ_THREADS), 0, stream, in,
                           a.state_in, a.state_out, a.y, a.mask, a.T, a.Hk, a.Hv, a.Dv, L.nc, row_blocks, (int)blocks);
    return hipGetLastError();
}

}  // namespace gdn
