// Gated delta-rule recurrence on gfx950.
//
// Per (b, hv) the state S is fp32 [Dv, Dk]; each row S[dv, :] evolves on its
// own given the step's k, q, g, beta and v[dv]:
//   S <- g S;  kv = S k;  delta = (v - kv) beta;  S <- S + delta k^T;  y = S q
// ("mlex 0.1.2 -- src/models/gated_delta.rs", GatedDeltaNet::forward
//  recurrence loop; "mlx-bun 0.4.0 -> 1.0.0, qwen3-delta.ts",
//  gated_delta_step, which runs the same order per row).
//
// Both kernels evaluate one step in the factored form
//   a = S k,  c = S q           (old state, one pass, two interleaved sums)
//   delta = (v - g a) beta       (= (v - (gS) k) beta)
//   y     = g c + delta (k.q)    (= (gS + delta k^T) q)
//   S     = g S + delta k^T
// which is the same arithmetic up to rounding order, needs one pass over the
// row for both dot products, and lets the two cross-lane sums overlap.
//
// Mapping (CDNA4, 64-wide wavefronts): one state row per group of L = Dk/8
// lanes; lane j of a group keeps elements 4j..4j+3 and Dk/2+4j..Dk/2+4j+3
// of the row in VGPRs for the whole sequence, so a group reads a k or q row
// as two contiguous 256-byte runs (Dk = 128).  The cross-lane sums are DPP
// butterflies inside the group (plus one ds_swizzle step when L = 32).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <int DK>
struct RecCfg {
    static constexpr int NT = 256;               // threads per block (4 waves)
    static constexpr int L = DK / 8;             // lanes per state row
    static constexpr int RPW = 64 / L;           // rows per wave
    static constexpr int ROWS = 4 * RPW;         // rows per block
};

// XCD-aware block order: the hardware deals consecutive block ids out
// round-robin over the 8 XCDs; remap so consecutive logical blocks (the row
// blocks of one head, then the next head, so also the v-heads sharing a
// k-head) land on the same XCD and share its L2.
__device__ __forceinline__ int xcd_block(int n_blocks) {
    int lb = blockIdx.x;
    if ((n_blocks & 7) == 0) lb = (lb & 7) * (n_blocks >> 3) + (lb >> 3);
    return lb;
}

// ============================================================ long sequences
//
// Sequences are processed in chunks of TC steps.  While chunk c runs out of
// LDS buffer c&1, the block's threads hold chunk c+1 (k, q, v, g, beta
// loaded from HBM at the start of chunk c) in registers; after the steps they
// convert it to f32, add the per-step k.q, and write it to buffer (c+1)&1:
// one barrier per chunk.  Steps past T are padded with g = 1, beta = 0,
// which leaves every state element bit-for-bit unchanged, so the step loop
// is fully unrolled with no tail case.  y is kept in lane registers during a
// chunk (lane j of a row group holds the steps t = j mod L), then stored to
// an LDS buffer as bf16 and written to HBM only when that buffer is full or
// the sequence ends.

// Per-key gate rows of a chunk (f32, the layout of k); nothing without it.
template <int DK, int TC, bool VG>
struct GateRows {
    float4 g[TC][DK / 4];
};
template <int DK, int TC>
struct GateRows<DK, TC, false> {};

template <int DK, int TC, bool VG = false>
struct ChunkBuf : GateRows<DK, TC, VG> {
    float4 k[TC][DK / 4];
    float4 q[TC][DK / 4];
    float4 sc[TC];                           // g, beta, k.q, 0
    float4 v4[TC / 4][RecCfg<DK>::ROWS];     // v of steps 4i..4i+3, per row
};

template <int DK, int TC, int YK = 64>
struct ChunkCfg {
    using C = RecCfg<DK>;
    static constexpr int YBYTES = YK * 1024;                         // y buffer
    static constexpr int YSTEPS = YBYTES / (C::ROWS * 2) / TC * TC;  // whole chunks
    static constexpr int PAIRS = TC * DK / 8;                        // (step, 8 cols)
    static constexpr int PPT = PAIRS / C::NT;                        // per thread
    static constexpr int VVEC = TC * C::ROWS / 8;                    // uint4 of v
    static constexpr int VPT = (VVEC + C::NT - 1) / C::NT;
    static_assert(PAIRS % C::NT == 0, "chunk must give every thread whole pairs");
    static_assert(TC % 4 == 0 && 2 * TC <= C::NT, "chunk length");
};

template <int DK, int TC, bool VG = false, int YK = 64>
struct ChunkSmem {
    ChunkBuf<DK, TC, VG> buf[2];
    uint16_t y[ChunkCfg<DK, TC, YK>::YSTEPS][RecCfg<DK>::ROWS];
};

template <int DK, int TC, bool VG = false>
struct ChunkStage {
    using C = RecCfg<DK>;
    using CC = ChunkCfg<DK, TC>;
    uint4 kr[CC::PPT];
    uint4 qr[CC::PPT];
    uint4 vr[CC::VPT];
    float4 gr[VG ? 2 * CC::PPT : 1];    // per-key gate: 8 columns per (step, 8 cols) pair
    float gb;

    __device__ __forceinline__ void load(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                         const uint16_t* __restrict__ v, const float* __restrict__ g,
                                         const float* __restrict__ beta, const uint8_t* __restrict__ mask,
                                         int b, int hk, int hv, int dv0, int t0, int T, int Hk, int Hv, int Dv,
                                         int tid) {
        // indices past T / Dv are clamped; those values are never consumed
#pragma unroll
        for (int i = 0; i < CC::PPT; ++i) {
            const int p = tid + i * C::NT;
            const int t = min(t0 + p / (DK / 8), T - 1);
            const int64_t off = (((int64_t)b * T + t) * Hk + hk) * DK + (p % (DK / 8)) * 8;
            kr[i] = *reinterpret_cast<const uint4*>(k + off);
            qr[i] = *reinterpret_cast<const uint4*>(q + off);
            if constexpr (VG) {
                // padding and masked steps decay by 1 (the state is kept)
                const int ts = t0 + p / (DK / 8);
                const bool on = ts < T && (mask == nullptr || mask[(int64_t)b * T + t] != 0);
                const float4* gp = reinterpret_cast<const float4*>(
                    g + (((int64_t)b * T + t) * Hv + hv) * DK + (p % (DK / 8)) * 8);
                const float4 g0 = gp[0], g1 = gp[1];    // in bounds (t is clamped)
                gr[2 * i] = make_float4(on ? g0.x : 1.f, on ? g0.y : 1.f, on ? g0.z : 1.f, on ? g0.w : 1.f);
                gr[2 * i + 1] = make_float4(on ? g1.x : 1.f, on ? g1.y : 1.f, on ? g1.z : 1.f, on ? g1.w : 1.f);
            }
        }
#pragma unroll
        for (int i = 0; i < CC::VPT; ++i) {
            const int idx = min(tid + i * C::NT, CC::VVEC - 1);
            const int t = min(t0 + idx / (C::ROWS / 8), T - 1);
            const int row = min(dv0 + (idx % (C::ROWS / 8)) * 8, Dv - 8);
            vr[i] = *reinterpret_cast<const uint4*>(v + (((int64_t)b * T + t) * Hv + hv) * Dv + row);
        }
        {
            // padding steps past T and masked steps: g = 1, beta = 0 (the state
            // stays as it is; a masked step's y is written as zero at the flush)
            const int t = t0 + tid % TC;
            const int64_t bt = (int64_t)b * T + min(t, T - 1);
            const int64_t i = bt * Hv + hv;
            const bool is_g = (tid % (2 * TC)) < TC;
            const float x = is_g ? (VG ? 1.f : g[i]) : beta[i];    // VG: gate rows above
            const bool on = t < T && (mask == nullptr || mask[bt] != 0);
            gb = on ? x : (is_g ? 1.f : 0.f);
        }
    }

    __device__ __forceinline__ void store(ChunkBuf<DK, TC, VG>& sb, int tid) const {
#pragma unroll
        for (int i = 0; i < CC::PPT; ++i) {
            const int p = tid + i * C::NT;
            const int step = p / (DK / 8);
            const int c8 = p % (DK / 8);
            float kf[8], qf[8];
            unpack8(kr[i], kf);
            unpack8(qr[i], qf);
            sb.k[step][2 * c8] = make_float4(kf[0], kf[1], kf[2], kf[3]);
            sb.k[step][2 * c8 + 1] = make_float4(kf[4], kf[5], kf[6], kf[7]);
            sb.q[step][2 * c8] = make_float4(qf[0], qf[1], qf[2], qf[3]);
            sb.q[step][2 * c8 + 1] = make_float4(qf[4], qf[5], qf[6], qf[7]);
            if constexpr (VG) {
                sb.g[step][2 * c8] = gr[2 * i];
                sb.g[step][2 * c8 + 1] = gr[2 * i + 1];
            }
            if constexpr (!VG) {              // (the per-key step forms k.q itself)
                float kq = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) kq = fmaf(kf[e], qf[e], kq);
                kq = group_sum<DK / 8>(kq);   // the DK/8 lanes of this step
                if (c8 == 0) sb.sc[step].z = kq;
            }
        }
#pragma unroll
        for (int i = 0; i < CC::VPT; ++i) {
            const int idx = tid + i * C::NT;
            if (CC::VVEC % C::NT == 0 || idx < CC::VVEC) {
                const int step = idx / (C::ROWS / 8);
                const int part = idx % (C::ROWS / 8);
                float f[8];
                unpack8(vr[i], f);
                float* dst = reinterpret_cast<float*>(&sb.v4[step / 4][part * 8]) + (step % 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) dst[4 * e] = f[e];
            }
        }
        if (tid < TC) sb.sc[tid].x = gb;
        else if (tid < 2 * TC) sb.sc[tid - TC].y = gb;
    }
};

__device__ __forceinline__ float pick(const float4& x, int i) {
    return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w;
}

// TC steps of one chunk on this lane's 8 state elements.  With the per-key
// gate (VG) each step is the staging-free kernel's per-key step, term for
// term (k.q included), so the two forms give the same bits.
template <int DK, int TC, bool VG = false>
__device__ __forceinline__ void run_chunk(const ChunkBuf<DK, TC, VG>& sb, float (&s)[8],
                                          float (&yr)[(TC + DK / 8 - 1) / (DK / 8)], int j, int rloc) {
    constexpr int L = DK / 8;
    float4 vv;
#pragma unroll
    for (int t = 0; t < TC; ++t) {
        if (t % 4 == 0) vv = sb.v4[t / 4][rloc];
        const float4 k0 = sb.k[t][j], k1 = sb.k[t][L + j];
        const float4 q0 = sb.q[t][j], q1 = sb.q[t][L + j];
        const float4 sc = sb.sc[t];
        const float kk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
        const float qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        if constexpr (VG) {
            const float4 g0 = sb.g[t][j], g1 = sb.g[t][L + j];
            const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
            float a = 0.f, c = 0.f, kq = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float gs = gg[i] * s[i];
                a = fmaf(gs, kk[i], a);
                c = fmaf(gs, qq[i], c);
                kq = fmaf(kk[i], qq[i], kq);
                s[i] = gs;
            }
            group_sum2<L>(a, c);
            kq = group_sum<L>(kq);
            const float delta = (pick(vv, t % 4) - a) * sc.y;
            const float yo = fmaf(delta, kq, c);
#pragma unroll
            for (int i = 0; i < 8; ++i) s[i] = fmaf(delta, kk[i], s[i]);
            if (j == t % L) yr[t / L] = yo;
            continue;
        }
        float a = 0.f, c = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a = fmaf(s[i], kk[i], a);
            c = fmaf(s[i], qq[i], c);
        }
        group_sum2<L>(a, c);
        const float gt = sc.x, bt = sc.y, kq = sc.z;
        const float delta = fmaf(-gt, a, pick(vv, t % 4)) * bt;
        const float yo = fmaf(gt, c, delta * kq);
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] = fmaf(delta, kk[i], gt * s[i]);
        if (j == t % L) yr[t / L] = yo;
    }
}

template <int DK, int TC, class Smem>
__device__ __forceinline__ void flush_y(const Smem& sh, uint16_t* __restrict__ y,
                                        const uint8_t* __restrict__ mask, int b, int hv, int dv0, int tbase,
                                        int nsteps, int T, int Hv, int Dv, int tid) {
    using C = RecCfg<DK>;
    const int nvec = nsteps * (C::ROWS / 8);
    for (int idx = tid; idx < nvec; idx += C::NT) {
        const int step = idx / (C::ROWS / 8);
        const int part = idx % (C::ROWS / 8);
        const int t = tbase + step;
        const int r = dv0 + part * 8;
        if (t < T && r < Dv) {
            uint4 w = *reinterpret_cast<const uint4*>(&sh.y[step][part * 8]);
            if (mask != nullptr && mask[(int64_t)b * T + t] == 0) w = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(y + (((int64_t)b * T + t) * Hv + hv) * Dv + r) = w;
        }
    }
}

template <int DK, int TC, bool VG, int YK>
__global__ __launch_bounds__(256) void recurrent_chunk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const uint8_t* __restrict__ mask,
    const float* state_in, float* state_out, uint16_t* __restrict__ y,
    int T, int Hk, int Hv, int Dv, int row_blocks, int n_blocks) {
    using C = RecCfg<DK>;
    using CC = ChunkCfg<DK, TC, YK>;
    constexpr int L = C::L;
    constexpr int NY = (TC + L - 1) / L;
    __shared__ ChunkSmem<DK, TC, VG, YK> sh;

    const int lb = xcd_block(n_blocks);
    const int n = lb / row_blocks;          // b * Hv + hv
    const int rb = lb % row_blocks;
    const int b = n / Hv;
    const int hv = n % Hv;
    const int hk = hv / (Hv / Hk);
    const int dv0 = rb * C::ROWS;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int j = lane % L;
    const int rloc = (tid >> 6) * C::RPW + lane / L;
    const int row = dv0 + rloc;
    const bool row_ok = row < Dv;

    float s[8];
    const int64_t srow = ((int64_t)n * Dv + row) * DK;
    if (state_in != nullptr && row_ok) {
        const float4 a0 = *reinterpret_cast<const float4*>(state_in + srow + 4 * j);
        const float4 a1 = *reinterpret_cast<const float4*>(state_in + srow + DK / 2 + 4 * j);
        s[0] = a0.x; s[1] = a0.y; s[2] = a0.z; s[3] = a0.w;
        s[4] = a1.x; s[5] = a1.y; s[6] = a1.z; s[7] = a1.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] = 0.f;
    }

    const int nchunks = (T + TC - 1) / TC;   // >= 1 (this kernel runs for T > 0)
    ChunkStage<DK, TC, VG> st;
    st.load(q, k, v, g, beta, mask, b, hk, hv, dv0, 0, T, Hk, Hv, Dv, tid);
    __builtin_amdgcn_s_waitcnt(0);           // state and chunk 0 resident
    st.store(sh.buf[0], tid);
    __syncthreads();

    int ybase = 0;                           // first step held in sh.y
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * TC;
        if (c + 1 < nchunks) st.load(q, k, v, g, beta, mask, b, hk, hv, dv0, t0 + TC, T, Hk, Hv, Dv, tid);
        float yr[NY];
        run_chunk<DK, TC, VG>(sh.buf[c & 1], s, yr, j, rloc);
        // y of this chunk -> LDS (bf16); each lane holds steps t = i*L + j
        const int yoff = t0 - ybase;
#pragma unroll
        for (int i = 0; i < NY; ++i) {
            const int t = i * L + j;
            if (t < TC) sh.y[yoff + t][rloc] = (uint16_t)f32_to_bf16(yr[i]);
        }
        if (c + 1 < nchunks) st.store(sh.buf[(c + 1) & 1], tid);
        __syncthreads();
        const bool last = c + 1 == nchunks;
        if (last || yoff + TC == CC::YSTEPS) {
            flush_y<DK, TC>(sh, y, mask, b, hv, dv0, ybase, yoff + TC, T, Hv, Dv, tid);
            ybase = t0 + TC;
            if (!last) __syncthreads();      // sh.y is rewritten by the next chunk
        }
    }

    if (row_ok) {
        *reinterpret_cast<float4*>(state_out + srow + 4 * j) = make_float4(s[0], s[1], s[2], s[3]);
        *reinterpret_cast<float4*>(state_out + srow + DK / 2 + 4 * j) = make_float4(s[4], s[5], s[6], s[7]);
    }
}

// =========================================================== short sequences
//
// Decode-sized T: no staging.  Each lane loads the 8 k and q values of its
// columns straight from HBM/L2 for every step (bf16, 2 x 8 bytes each), the
// state is streamed in and out once (non-temporal: it is not reused), and y
// leaves from lane 0 of each row group.
//
// Two options (compile-time, so the plain kernel is unchanged):
//   VG    per-key decay, g [B, T, Hv, Dk]: S <- S diag(g_t).  In the factored
//         form a = S (g.k) and c = S (g.q) (elementwise products of the
//         lane's 8 columns), delta = (v - a) beta, y = c + delta (k.q),
//         S = g.S + delta k^T.
//   SNAP  after every step count listed in the snapshot list (0 = before the
//         first step), the row's state is also written to that snapshot.

// Entry i of the snapshot list (i uniform; static indexing only, so the
// by-value kernel argument is never copied to scratch).  -1 past the end.
__device__ __forceinline__ int snap_step(const SnapList& sl, int i) {
    int r = -1;
#pragma unroll
    for (int u = 0; u < kMaxSnapshots; ++u)
        if (u == i && u < sl.n) r = sl.steps[u];
    return r;
}

template <int DK>
__device__ __forceinline__ void store_row(float* dst, const float (&s)[8], int j) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    const f4v o0 = {s[0], s[1], s[2], s[3]};
    const f4v o1 = {s[4], s[5], s[6], s[7]};
    __builtin_nontemporal_store(o0, reinterpret_cast<f4v*>(dst + 4 * j));
    __builtin_nontemporal_store(o1, reinterpret_cast<f4v*>(dst + DK / 2 + 4 * j));
}

template <int DK, bool VG, bool SNAP>
__global__ __launch_bounds__(256) void recurrent_step_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const uint8_t* __restrict__ mask,
    const float* state_in, float* state_out, uint16_t* __restrict__ y,
    int T, int Hk, int Hv, int Dv, int row_blocks, int n_blocks, SnapList snap, int64_t snap_stride) {
    using C = RecCfg<DK>;
    constexpr int L = C::L;
    const int lb = xcd_block(n_blocks);
    const int n = lb / row_blocks;
    const int rb = lb % row_blocks;
    const int b = n / Hv;
    const int hv = n % Hv;
    const int hk = hv / (Hv / Hk);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int j = lane % L;
    const int row = rb * C::ROWS + (tid >> 6) * C::RPW + lane / L;
    const bool row_ok = row < Dv;
    const int rowc = min(row, Dv - 1);

    typedef float f4v __attribute__((ext_vector_type(4)));
    float s[8];
    const int64_t srow = ((int64_t)n * Dv + row) * DK;
    if (state_in != nullptr && row_ok) {
        const f4v a0 = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(state_in + srow + 4 * j));
        const f4v a1 = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(state_in + srow + DK / 2 + 4 * j));
        s[0] = a0.x; s[1] = a0.y; s[2] = a0.z; s[3] = a0.w;
        s[4] = a1.x; s[5] = a1.y; s[6] = a1.z; s[7] = a1.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] = 0.f;
    }

    int snap_i = 0, snap_next = -1;
    if constexpr (SNAP) {
        snap_next = snap_step(snap, 0);
        if (snap_next == 0) {
            if (row_ok) store_row<DK>(snap.out + srow, s, j);
            snap_i = 1;
            snap_next = snap_step(snap, 1);
        }
    }

    for (int t = 0; t < T; ++t) {
        const int64_t tok = (int64_t)b * T + t;
        if (mask != nullptr && mask[tok] == 0) {      // masked step: state kept, y = 0
            if (j == 0 && row_ok) y[(tok * Hv + hv) * Dv + row] = 0;
        } else {
        const uint16_t* kp = k + (tok * Hk + hk) * DK;
        const uint16_t* qp = q + (tok * Hk + hk) * DK;
        const uint2 kw0 = *reinterpret_cast<const uint2*>(kp + 4 * j);
        const uint2 kw1 = *reinterpret_cast<const uint2*>(kp + DK / 2 + 4 * j);
        const uint2 qw0 = *reinterpret_cast<const uint2*>(qp + 4 * j);
        const uint2 qw1 = *reinterpret_cast<const uint2*>(qp + DK / 2 + 4 * j);
        const float vt = bf16lo(v[(tok * Hv + hv) * Dv + rowc]);
        const float bt = beta[tok * Hv + hv];
        const float kk[8] = {bf16lo(kw0.x), bf16hi(kw0.x), bf16lo(kw0.y), bf16hi(kw0.y),
                             bf16lo(kw1.x), bf16hi(kw1.x), bf16lo(kw1.y), bf16hi(kw1.y)};
        const float qq[8] = {bf16lo(qw0.x), bf16hi(qw0.x), bf16lo(qw0.y), bf16hi(qw0.y),
                             bf16lo(qw1.x), bf16hi(qw1.x), bf16lo(qw1.y), bf16hi(qw1.y)};
        if constexpr (VG) {
            const float* gp = g + (tok * Hv + hv) * DK;
            const float4 g0 = *reinterpret_cast<const float4*>(gp + 4 * j);
            const float4 g1 = *reinterpret_cast<const float4*>(gp + DK / 2 + 4 * j);
            const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
            float a = 0.f, c = 0.f, kq = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float gs = gg[i] * s[i];        // the decayed state element
                a = fmaf(gs, kk[i], a);
                c = fmaf(gs, qq[i], c);
                kq = fmaf(kk[i], qq[i], kq);
                s[i] = gs;
            }
            group_sum2<L>(a, c);
            kq = group_sum<L>(kq);
            const float delta = (vt - a) * bt;
            const float yo = fmaf(delta, kq, c);
#pragma unroll
            for (int i = 0; i < 8; ++i) s[i] = fmaf(delta, kk[i], s[i]);
            if (j == 0 && row_ok) y[(tok * Hv + hv) * Dv + row] = (uint16_t)f32_to_bf16(yo);
        } else {
            const float gt = g[tok * Hv + hv];
            float a = 0.f, c = 0.f, kq = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                a = fmaf(s[i], kk[i], a);
                c = fmaf(s[i], qq[i], c);
                kq = fmaf(kk[i], qq[i], kq);
            }
            group_sum2<L>(a, c);
            kq = group_sum<L>(kq);
            const float delta = fmaf(-gt, a, vt) * bt;
            const float yo = fmaf(gt, c, delta * kq);
#pragma unroll
            for (int i = 0; i < 8; ++i) s[i] = fmaf(delta, kk[i], gt * s[i]);
            if (j == 0 && row_ok) y[(tok * Hv + hv) * Dv + row] = (uint16_t)f32_to_bf16(yo);
        }
        }
        if constexpr (SNAP) {
            if (t + 1 == snap_next) {
                if (row_ok) store_row<DK>(snap.out + snap_i * snap_stride + srow, s, j);
                ++snap_i;
                snap_next = snap_step(snap, snap_i);
            }
        }
    }

    if (row_ok) store_row<DK>(state_out + srow, s, j);
}

// ======================================================= single-token decode
//
// The layer core at T = 1 in one launch, one 512-thread block per (b,
// k-head): the block computes the prologue of its k-head's q and k channels,
// its v-heads' v channels and their gates, then advances those v-heads' state
// rows by one step.  Every channel is read, and its conv state rewritten, by
// one lane of one block, so the conv state may be updated in place.  The
// prologue uses the prologue kernel's device functions and the step is the
// staging-free kernel's arithmetic term for term (q, k, v rounded to bf16
// first), so the results are the bits of the two-launch composition.

constexpr int DEC_NT = 512;
constexpr int kDecMaxRows = 1024;   // (Hv / Hk) * Dv of one block

template <int DK, int KC>
__global__ __launch_bounds__(DEC_NT) void decode_core_kernel(PrepArgs p, const uint8_t* __restrict__ mask,
                                                             const float* state_in, float* state_out,
                                                             uint16_t* __restrict__ y) {
    __shared__ float qs[DK], ks[DK], vs[kDecMaxRows], gsh[kDecMaxRows / 8], bsh[kDecMaxRows / 8];
    constexpr int L = DK / 8;                 // lanes per state row (and per q/k head)
    const int Hk = p.Hk, Hv = p.Hv, Dv = p.Dv;
    const int b = blockIdx.x / Hk, hk = blockIdx.x % Hk;
    const int G = Hv / Hk, R = G * Dv;
    const int C = 2 * Hk * DK + Hv * Dv;
    const int tid = threadIdx.x;

    // prologue: thread i < L the q channels 8i.., L <= i < 2L the k channels,
    // 2L <= i < 2L + R/8 the v channels; threads 256.. the gates
    const int nv = R / 8;
    if (tid < 2 * L + nv) {
        const int region = tid < L ? 0 : tid < 2 * L ? 1 : 2;
        const int c0 = region == 0   ? hk * DK + 8 * tid
                       : region == 1 ? Hk * DK + hk * DK + 8 * (tid - L)
                                     : 2 * Hk * DK + hk * G * Dv + 8 * (tid - 2 * L);
        uint4 wk[KC];
#pragma unroll
        for (int v4 = 0; v4 < KC; ++v4) wk[v4] = reinterpret_cast<const uint4*>(p.conv_w + (int64_t)c0 * KC)[v4];
        const ConvW<KC> w = conv_weights<KC>(wk);
        // the conv state rows, then the token's own row
        uint4 hr[KC];
#pragma unroll
        for (int r = 0; r < KC - 1; ++r)
            hr[r] = p.conv_state_in
                        ? *reinterpret_cast<const uint4*>(p.conv_state_in + ((int64_t)b * (KC - 1) + r) * C + c0)
                        : make_uint4(0, 0, 0, 0);
        const uint4 xr = *reinterpret_cast<const uint4*>(p.qkv + (int64_t)b * C + c0);
        hr[KC - 1] = xr;
        float act[8];
        conv_silu8<KC>(w, hr, act);
        // q/k: the head norm over the head's L lanes (aligned lane groups of
        // wave 0); v lanes pass act through
        const uint4 packed = qk_norm8<DK>(act, region < 2, region == 0 ? p.q_scale : p.k_scale, p.eps);
        float o[8];
        unpack8(packed, o);
        float* dst = region == 0 ? qs + 8 * tid : region == 1 ? ks + 8 * (tid - L) : vs + 8 * (tid - 2 * L);
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e] = o[e];
        // the new conv state: rows 1.. of the old one, then the token (every
        // row read above, before this write)
        if (p.conv_state_out) {
#pragma unroll
            for (int r = 0; r < KC - 1; ++r)
                *reinterpret_cast<uint4*>(p.conv_state_out + ((int64_t)b * (KC - 1) + r) * C + c0) =
                    hr[r + 1];
        }
    }
    if (tid >= 256 && tid < 256 + G) {
        const int hl = tid - 256, hv = hk * G + hl;
        const int64_t i = (int64_t)b * Hv + hv;
        float gv, bv;
        gate_g_beta(p.a[i], p.b[i], p.A_log[hv], p.dt_bias[hv], gv, bv);
        gsh[hl] = gv;
        bsh[hl] = bv;
    }
    __syncthreads();

    // the step, RPP state rows per pass (L lanes per row, 8 elements per lane)
    constexpr int RPP = DEC_NT / L;
    const int j = tid % L, rr = tid / L;
    const bool active = mask == nullptr || mask[b] != 0;
    float kk[8], qq[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        kk[e] = ks[4 * j + e];
        kk[4 + e] = ks[DK / 2 + 4 * j + e];
        qq[e] = qs[4 * j + e];
        qq[4 + e] = qs[DK / 2 + 4 * j + e];
    }
    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) kq = fmaf(kk[i], qq[i], kq);
    kq = group_sum<L>(kq);
    typedef float f4v __attribute__((ext_vector_type(4)));
    for (int r0 = 0; r0 < R; r0 += RPP) {
        const int r = r0 + rr;
        const bool ok = r < R;
        const int rc = ok ? r : R - 1;
        const int hl = rc / Dv, dv = rc % Dv, hv = hk * G + hl;
        const int64_t srow = (((int64_t)b * Hv + hv) * Dv + dv) * DK;
        float s[8];
        if (state_in != nullptr && ok) {
            const f4v a0 = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(state_in + srow + 4 * j));
            const f4v a1 = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(state_in + srow + DK / 2 + 4 * j));
            s[0] = a0.x; s[1] = a0.y; s[2] = a0.z; s[3] = a0.w;
            s[4] = a1.x; s[5] = a1.y; s[6] = a1.z; s[7] = a1.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) s[i] = 0.f;
        }
        const int64_t yi = ((int64_t)b * Hv + hv) * Dv + dv;
        if (active) {
            const float gt = gsh[hl], bt = bsh[hl], vt = vs[rc];
            float a = 0.f, c = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                a = fmaf(s[i], kk[i], a);
                c = fmaf(s[i], qq[i], c);
            }
            group_sum2<L>(a, c);
            const float delta = fmaf(-gt, a, vt) * bt;
            const float yo = fmaf(gt, c, delta * kq);
#pragma unroll
            for (int i = 0; i < 8; ++i) s[i] = fmaf(delta, kk[i], gt * s[i]);
            if (j == 0 && ok) y[yi] = (uint16_t)f32_to_bf16(yo);
        } else if (j == 0 && ok) {
            y[yi] = 0;                        // masked step: state kept, y = 0
        }
        if (ok) store_row<DK>(state_out + srow, s, j);
    }
}

// The fused form pays while its (b, k-head) blocks fill the device in one
// round (four 512-thread blocks per CU): below that too few CUs stream the
// state, above it the blocks' serial row passes fall behind the per-step
// kernel's finer grid.  Both forms give the same bits, so the choice may
// depend on the device.
bool decode_fusable(int B, int Hk, int Hv, int Dk, int Dv, int K) {
    const int64_t cus = device_cu_count(), blocks = (int64_t)B * Hk;
    return (Dk == 32 || Dk == 64 || Dk == 128 || Dk == 256) && K >= 2 && K <= 4 &&
           (int64_t)(Hv / Hk) * Dv <= kDecMaxRows && cus > 0 && blocks >= cus && blocks <= 4 * cus;
}

template <int DK>
static hipError_t launch_decode_k(const PrepArgs& p, const uint8_t* mask, const float* si, float* so, uint16_t* y,
                                  hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.B * p.Hk));
    switch (p.K) {
        case 2: hipLaunchKernelGGL((decode_core_kernel<DK, 2>), grid, dim3(DEC_NT), 0, stream, p, mask, si, so, y); break;
        case 3: hipLaunchKernelGGL((decode_core_kernel<DK, 3>), grid, dim3(DEC_NT), 0, stream, p, mask, si, so, y); break;
        case 4: hipLaunchKernelGGL((decode_core_kernel<DK, 4>), grid, dim3(DEC_NT), 0, stream, p, mask, si, so, y); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_core(const PrepArgs& p, const uint8_t* mask, const float* state_in, float* state_out,
                              uint16_t* y, hipStream_t stream) {
    if (p.T != 1 || !decode_fusable(p.B, p.Hk, p.Hv, p.Dk, p.Dv, p.K)) return hipErrorInvalidValue;
    switch (p.Dk) {
        case 32: return launch_decode_k<32>(p, mask, state_in, state_out, y, stream);
        case 64: return launch_decode_k<64>(p, mask, state_in, state_out, y, stream);
        case 128: return launch_decode_k<128>(p, mask, state_in, state_out, y, stream);
        case 256: return launch_decode_k<256>(p, mask, state_in, state_out, y, stream);
        default: return hipErrorInvalidValue;
    }
}

// ================================================================== launch

int64_t recurrent_blocks(int B, int Hv, int Dk, int Dv) {
    const int rows = 4 * 64 / (Dk / 8);
    return (int64_t)B * Hv * ((Dv + rows - 1) / rows);
}

template <int DK, int TC, bool VG = false, int YK = 64>
static hipError_t launch_rec(const RecurrentArgs& a, hipStream_t stream, bool chunked) {
    using C = RecCfg<DK>;
    const int row_blocks = (a.Dv + C::ROWS - 1) / C::ROWS;
    const int64_t blocks = (int64_t)a.B * a.Hv * row_blocks;
    if (blocks <= 0) return hipSuccess;
    if (chunked)
        hipLaunchKernelGGL((recurrent_chunk_kernel<DK, TC, VG, YK>), dim3((unsigned)blocks), dim3(C::NT), 0, stream,
                           a.q, a.k, a.v, a.g, a.beta, a.mask, a.state_in, a.state_out, a.y, a.T, a.Hk, a.Hv,
                           a.Dv, row_blocks, (int)blocks);
    else
        hipLaunchKernelGGL((recurrent_step_kernel<DK, VG, false>), dim3((unsigned)blocks), dim3(C::NT), 0,
                           stream, a.q, a.k, a.v, a.g, a.beta, a.mask, a.state_in, a.state_out, a.y, a.T, a.Hk,
                           a.Hv, a.Dv, row_blocks, (int)blocks, SnapList{}, (int64_t)0);
    return hipGetLastError();
}

// The per-step kernel with its options: per-key decay and/or snapshots.
template <int DK, bool VG, bool SNAP>
static hipError_t launch_step_opt(const RecurrentArgs& a, hipStream_t stream) {
    using C = RecCfg<DK>;
    const int row_blocks = (a.Dv + C::ROWS - 1) / C::ROWS;
    const int64_t blocks = (int64_t)a.B * a.Hv * row_blocks;
    if (blocks <= 0) return hipSuccess;
    const SnapList sl = SNAP ? *a.snap : SnapList{};
    const int64_t stride = (int64_t)a.B * a.Hv * a.Dv * DK;
    hipLaunchKernelGGL((recurrent_step_kernel<DK, VG, SNAP>), dim3((unsigned)blocks), dim3(C::NT), 0, stream,
                       a.q, a.k, a.v, a.g, a.beta, a.mask, a.state_in, a.state_out, a.y, a.T, a.Hk, a.Hv, a.Dv,
                       row_blocks, (int)blocks, sl, stride);
    return hipGetLastError();
}

template <int DK>
static hipError_t launch_snap(const RecurrentArgs& a, hipStream_t stream) {
    return a.g_per_key ? launch_step_opt<DK, true, true>(a, stream) : launch_step_opt<DK, false, true>(a, stream);
}

// Sequences shorter than this run the staging-free kernel.
constexpr int kChunkedMinT = 8;

// The staged kernel in two configurations of the same arithmetic (so the
// same bits): long chunks and a 64 KiB y buffer, one block per CU, for a
// grid that fits the device in one round; for larger grids, or sequences
// that fill less than half a long chunk, half-length chunks and a 16 KiB y
// buffer, so that two or three blocks share a CU.
template <int DK, int TC, int TCS, bool VG>
static hipError_t launch_staged(const RecurrentArgs& a, hipStream_t stream, bool chunked) {
    if constexpr (TCS > 0) {
        using C = RecCfg<DK>;
        const int cus = device_cu_count();
        const int64_t blocks = (int64_t)a.B * a.Hv * ((a.Dv + C::ROWS - 1) / C::ROWS);
        if (chunked && (2 * a.T <= TC || (cus > 0 && blocks > cus))) return launch_rec<DK, TCS, VG, 16>(a, stream, true);
    }
    return launch_rec<DK, TC, VG>(a, stream, chunked);
}

hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t stream) {
    if (a.snap != nullptr && a.snap->n > 0) {
        switch (a.Dk) {
            case 32: return launch_snap<32>(a, stream);
            case 64: return launch_snap<64>(a, stream);
            case 128: return launch_snap<128>(a, stream);
            case 256: return launch_snap<256>(a, stream);
            default: return hipErrorInvalidValue;
        }
    }
    const bool chunked = a.T >= kChunkedMinT;
    if (a.g_per_key) {
        // the gate rows take LDS beside k and q: half-length chunks at Dk >= 128
        switch (a.Dk) {
            case 32: return launch_staged<32, 64, 0, true>(a, stream, chunked);
            case 64: return launch_staged<64, 32, 32, true>(a, stream, chunked);
            case 128: return launch_staged<128, 16, 16, true>(a, stream, chunked);
            case 256: return launch_staged<256, 8, 8, true>(a, stream, chunked);
            default: return hipErrorInvalidValue;
        }
    }
    switch (a.Dk) {
        case 32: return launch_staged<32, 64, 0, false>(a, stream, chunked);
        case 64: return launch_staged<64, 32, 32, false>(a, stream, chunked);
        case 128: return launch_staged<128, 32, 16, false>(a, stream, chunked);
        case 256: return launch_staged<256, 16, 8, false>(a, stream, chunked);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
