// Gated delta-rule recurrence on gfx950.
//
// Per (b, hv) the state S is fp32 [Dv, Dk]; each row S[dv, :] evolves on its
// own given the step's k, q, g, beta and v[dv]:
//   S <- g S;  kv = S k;  delta = (v - kv) beta;  S <- S + delta k^T;  y = S q
// ("mlex 0.1.2 -- src/models/gated_delta.rs", GatedDeltaNet::forward
//  recurrence loop; "mlx-bun 0.4.0 -> 1.0.0, qwen3-delta.ts",
//  gated_delta_step, which runs the same order per row).
//
// Mapping (CDNA4, 64-wide wavefronts):
//   * one state row per group of L = Dk/8 lanes; each lane keeps 8 floats
//     of its row in VGPRs for the whole T loop (elements 4j..4j+3 and
//     Dk/2+4j..Dk/2+4j+3 for lane j of the group, so a 16-lane group reads
//     k/q rows from LDS as contiguous 256-byte ds_read_b128 runs);
//   * a workgroup of 4 waves owns ROWS = 4*64/L consecutive rows of one
//     (b, hv); the two Dk-long dot products are DPP butterflies inside the
//     lane group (plus one ds_swizzle step when L = 32);
//   * k, q (converted to f32 once), v, g and beta for the next TC steps are
//     loaded from HBM into registers while the current TC steps run, then
//     written to LDS between two barriers; y for TC steps is buffered in LDS
//     and flushed as contiguous bf16 runs;
//   * block -> (b, hv) mapping keeps all row blocks of a head, and the
//     v-heads sharing a k-head, on the same XCD (shared L2 for k/q).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <int DK>
struct RecCfg {
    static constexpr int NT = 256;               // threads per block (4 waves)
    static constexpr int L = DK / 8;             // lanes per state row
    static constexpr int RPW = 64 / L;           // rows per wave
    static constexpr int ROWS = 4 * RPW;         // rows per block
    static constexpr int V4 = DK / 4;            // float4 per k/q row
};

template <int DK, int TC>
struct RecShared {
    float4 ks[TC][DK / 4];
    float4 qs[TC][DK / 4];
    float vs[TC][RecCfg<DK>::ROWS];
    float ys[TC][RecCfg<DK>::ROWS];
    float gs[TC];
    float bs[TC];
};

// Global -> register staging of one chunk of TC steps.  Indices past T or Dv
// are clamped to the last valid token / row: those staged values are never
// consumed (steps >= T are not run, rows >= Dv are not stored), and clamping
// keeps every load unconditional, so the compiler never has to assume a
// pending load into the staging registers.
template <int DK, int TC>
struct RecStage {
    using C = RecCfg<DK>;
    static constexpr int KQ_VEC = 2 * TC * DK / 8;            // uint4 of k and q
    static constexpr int KQ_PER_T = (KQ_VEC + C::NT - 1) / C::NT;
    static constexpr int V_VEC = TC * C::ROWS / 8;            // uint4 of v
    static constexpr int V_PER_T = (V_VEC + C::NT - 1) / C::NT;
    uint4 kq[KQ_PER_T];
    uint4 vv[V_PER_T];
    float gb;

    __device__ __forceinline__ void load(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                         const uint16_t* __restrict__ v, const float* __restrict__ g,
                                         const float* __restrict__ beta, int b, int hk, int hv, int dv0,
                                         int t0, int T, int Hk, int Hv, int Dv, int tid) {
#pragma unroll
        for (int i = 0; i < KQ_PER_T; ++i) {
            const int idx = min(tid + i * C::NT, KQ_VEC - 1);
            const int which = idx / (TC * DK / 8);
            const int rem = idx % (TC * DK / 8);
            const int t = min(t0 + rem / (DK / 8), T - 1);
            const int c8 = rem % (DK / 8);
            const uint16_t* src = which ? q : k;
            kq[i] = *reinterpret_cast<const uint4*>(src + (((int64_t)b * T + t) * Hk + hk) * DK + c8 * 8);
        }
#pragma unroll
        for (int i = 0; i < V_PER_T; ++i) {
            const int idx = min(tid + i * C::NT, V_VEC - 1);
            const int t = min(t0 + idx / (C::ROWS / 8), T - 1);
            const int row = min(dv0 + (idx % (C::ROWS / 8)) * 8, Dv - 8);
            vv[i] = *reinterpret_cast<const uint4*>(v + (((int64_t)b * T + t) * Hv + hv) * Dv + row);
        }
        {
            const int t = min(t0 + tid % TC, T - 1);
            const int64_t i = ((int64_t)b * T + t) * Hv + hv;
            gb = (tid % (2 * TC)) < TC ? g[i] : beta[i];
        }
    }

    __device__ __forceinline__ void store(RecShared<DK, TC>& sh, int tid) const {
#pragma unroll
        for (int i = 0; i < KQ_PER_T; ++i) {
            const int idx = tid + i * C::NT;
            if (KQ_VEC % C::NT == 0 || idx < KQ_VEC) {
                const int which = idx / (TC * DK / 8);
                const int rem = idx % (TC * DK / 8);
                const int step = rem / (DK / 8);
                const int c8 = rem % (DK / 8);
                float f[8];
                unpack8(kq[i], f);
                float4* dst = which ? sh.qs[step] : sh.ks[step];
                dst[2 * c8] = make_float4(f[0], f[1], f[2], f[3]);
                dst[2 * c8 + 1] = make_float4(f[4], f[5], f[6], f[7]);
            }
        }
#pragma unroll
        for (int i = 0; i < V_PER_T; ++i) {
            const int idx = tid + i * C::NT;
            if (V_VEC % C::NT == 0 || idx < V_VEC) {
                const int step = idx / (C::ROWS / 8);
                const int part = idx % (C::ROWS / 8);
                float f[8];
                unpack8(vv[i], f);
                float4* dst = reinterpret_cast<float4*>(&sh.vs[step][part * 8]);
                dst[0] = make_float4(f[0], f[1], f[2], f[3]);
                dst[1] = make_float4(f[4], f[5], f[6], f[7]);
            }
        }
        if (tid < 2 * TC) {
            if (tid < TC) sh.gs[tid] = gb;
            else sh.bs[tid - TC] = gb;
        }
    }
};

// Operands of one step, read from LDS one step ahead of their use.
template <int DK>
struct StepIn {
    float4 k0, k1, q0, q1;
    float g, beta, v;
};

template <int DK, int TC>
__device__ __forceinline__ StepIn<DK> read_step(const RecShared<DK, TC>& sh, int t, int j, int rloc) {
    using C = RecCfg<DK>;
    StepIn<DK> r;
    r.k0 = sh.ks[t][j];
    r.k1 = sh.ks[t][C::L + j];
    r.q0 = sh.qs[t][j];
    r.q1 = sh.qs[t][C::L + j];
    r.g = sh.gs[t];
    r.beta = sh.bs[t];
    r.v = sh.vs[t][rloc];
    return r;
}

// Runs `steps` (1..TC) steps of the staged chunk on this lane's 8 state
// elements; y of each step goes to sh.ys (one lane per row writes).
template <int DK, int TC>
__device__ __forceinline__ void run_chunk(RecShared<DK, TC>& sh, float (&s)[8], int steps, int j, int rloc) {
    using C = RecCfg<DK>;
    StepIn<DK> nx = read_step<DK, TC>(sh, 0, j, rloc);
    for (int t = 0; t < steps; ++t) {
        const StepIn<DK> cu = nx;
        nx = read_step<DK, TC>(sh, min(t + 1, TC - 1), j, rloc);
        const float kk[8] = {cu.k0.x, cu.k0.y, cu.k0.z, cu.k0.w, cu.k1.x, cu.k1.y, cu.k1.z, cu.k1.w};
        const float qq[8] = {cu.q0.x, cu.q0.y, cu.q0.z, cu.q0.w, cu.q1.x, cu.q1.y, cu.q1.z, cu.q1.w};
        // decay, then read-out with the decayed state
        float kv = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s[i] *= cu.g;
            kv = fmaf(s[i], kk[i], kv);
        }
        kv = group_sum<C::L>(kv);
        const float delta = (cu.v - kv) * cu.beta;
        // rank-1 update, then output with the updated state
        float yo = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s[i] = fmaf(kk[i], delta, s[i]);
            yo = fmaf(s[i], qq[i], yo);
        }
        yo = group_sum<C::L>(yo);
        if (j == 0) sh.ys[t][rloc] = yo;
    }
}

// y of one chunk: per step ROWS contiguous bf16 values of (b, t, hv, dv0..).
template <int DK, int TC>
__device__ __forceinline__ void flush_y(const RecShared<DK, TC>& sh, uint16_t* __restrict__ y, int b, int hv,
                                        int dv0, int t0, int T, int Hv, int Dv, int tid) {
    using C = RecCfg<DK>;
    constexpr int YV = TC * C::ROWS / 8;
    for (int idx = tid; idx < YV; idx += C::NT) {
        const int step = idx / (C::ROWS / 8);
        const int part = idx % (C::ROWS / 8);
        const int t = t0 + step;
        const int r = dv0 + part * 8;
        if (t < T && r < Dv) {
            const float4* src = reinterpret_cast<const float4*>(&sh.ys[step][part * 8]);
            const float4 lo = src[0], hi = src[1];
            const float f[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            *reinterpret_cast<uint4*>(y + (((int64_t)b * T + t) * Hv + hv) * Dv + r) = pack8(f);
        }
    }
}

template <int DK, int TC>
__global__ __launch_bounds__(256) void recurrent_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const float* state_in, float* state_out, uint16_t* __restrict__ y,
    int T, int Hk, int Hv, int Dv, int row_blocks, int n_blocks) {
    using C = RecCfg<DK>;
    __shared__ RecShared<DK, TC> sh;

    // XCD-aware block order: hardware dispatches consecutive block ids
    // round-robin over 8 XCDs; remap so consecutive logical blocks (row blocks
    // of one head, then the next head) share an XCD.
    int lb = blockIdx.x;
    if ((n_blocks & 7) == 0) lb = (lb & 7) * (n_blocks >> 3) + (lb >> 3);
    const int n = lb / row_blocks;          // b * Hv + hv
    const int rb = lb % row_blocks;
    const int b = n / Hv;
    const int hv = n % Hv;
    const int hk = hv / (Hv / Hk);
    const int dv0 = rb * C::ROWS;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int j = lane % C::L;              // position inside the row group
    const int rloc = wave * C::RPW + lane / C::L;   // row inside the block
    const int row = dv0 + rloc;
    const bool row_ok = row < Dv;

    // state row -> registers
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
    // the state must be resident before the step loop; waiting here keeps the
    // loop free of waits on the next chunk's in-flight prefetch
    __builtin_amdgcn_s_waitcnt(0);

    const int nchunks = (T + TC - 1) / TC;
    if (nchunks > 0) {   // uniform over the block
        RecStage<DK, TC> st;
        st.load(q, k, v, g, beta, b, hk, hv, dv0, 0, T, Hk, Hv, Dv, tid);
        st.store(sh, tid);
        __syncthreads();
        // every chunk but the last: the next chunk's HBM loads are in flight
        // while this chunk's steps run
        for (int c = 0; c + 1 < nchunks; ++c) {
            const int t0 = c * TC;
            st.load(q, k, v, g, beta, b, hk, hv, dv0, t0 + TC, T, Hk, Hv, Dv, tid);
            run_chunk<DK, TC>(sh, s, TC, j, rloc);
            __syncthreads();
            st.store(sh, tid);   // staged chunk consumed: install the next one
            flush_y<DK, TC>(sh, y, b, hv, dv0, t0, T, Hv, Dv, tid);
            __syncthreads();
        }
        const int t0 = (nchunks - 1) * TC;
        run_chunk<DK, TC>(sh, s, T - t0, j, rloc);
        __syncthreads();
        flush_y<DK, TC>(sh, y, b, hv, dv0, t0, T, Hv, Dv, tid);
    }

    if (row_ok) {
        *reinterpret_cast<float4*>(state_out + srow + 4 * j) = make_float4(s[0], s[1], s[2], s[3]);
        *reinterpret_cast<float4*>(state_out + srow + DK / 2 + 4 * j) = make_float4(s[4], s[5], s[6], s[7]);
    }
}

template <int DK, int TC>
static hipError_t launch_rec(const RecurrentArgs& a, hipStream_t stream) {
    using C = RecCfg<DK>;
    const int row_blocks = (a.Dv + C::ROWS - 1) / C::ROWS;
    const int64_t blocks = (int64_t)a.B * a.Hv * row_blocks;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((recurrent_kernel<DK, TC>), dim3((unsigned)blocks), dim3(C::NT), 0, stream,
                       a.q, a.k, a.v, a.g, a.beta, a.state_in, a.state_out, a.y,
                       a.T, a.Hk, a.Hv, a.Dv, row_blocks, (int)blocks);
    return hipGetLastError();
}

int64_t recurrent_blocks(int B, int Hv, int Dk, int Dv) {
    const int rows = 4 * 64 / (Dk / 8);
    return (int64_t)B * Hv * ((Dv + rows - 1) / rows);
}

hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t stream) {
    // short sequences (decode) use one-step chunks: no idle LDS, more blocks
    // per CU; longer ones stage TC = 4096/Dk steps (16 KiB of f32 k or q).
    const bool small = a.T <= 4;
    switch (a.Dk) {
        case 32: return small ? launch_rec<32, 1>(a, stream) : launch_rec<32, 64>(a, stream);
        case 64: return small ? launch_rec<64, 1>(a, stream) : launch_rec<64, 64>(a, stream);
        case 128: return small ? launch_rec<128, 1>(a, stream) : launch_rec<128, 32>(a, stream);
        case 256: return small ? launch_rec<256, 1>(a, stream) : launch_rec<256, 16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
