// Data-parallel prologue of the Gated DeltaNet layer on gfx950
// ("mlex 0.1.2 -- src/models/gated_delta.rs", GatedDeltaNet::forward from the
//  conv-state splice through g; "mlx-bun 0.4.0 -> 1.0.0, qwen3-delta.ts",
//  compute_g and the dtype contract in its header).
//
// Every qkv element is read from HBM once and every q/k/v element written
// once.  A thread owns 8 consecutive channels (one 16-byte vector) over TT
// consecutive tokens and slides a (K-1)-row window of the spliced input
// through registers, so the conv halo costs K-1 extra row reads per TT
// tokens (served mostly from L2).
// A 64-lane wave covers 512 channels; q/k heads (Dk channels = Dk/8 lanes)
// are aligned lane groups, so the per-head sum of squares is a DPP butterfly.
// Gates (g, beta) are computed by extra blocks of the same launch.
// q/k/v are written with non-temporal stores: each is written once and not
// read again by this kernel, and streaming them past the caches' normal
// retention measured faster both alone and followed by the recurrence.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));

// one 16-byte vector store with the non-temporal hint (a global_store ... nt)
__device__ __forceinline__ void store_stream16(uint16_t* dst, const uint4 v) {
    const u32x4_nt x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4_nt*>(dst));
}

// One wave per block (512 channels) and 4 tokens per thread: measured over a
// sweep of 2..32 tokens and 64..256 threads at the prefill workload (4
// rotating buffer sets), 4 x 64 takes 28 us against 35 us for 16 x 256; the
// short per-thread chain and the many small blocks outweigh re-reading the
// K - 1 halo rows per 4 tokens (mostly from L2).
constexpr int PREP_NT = 64;    // threads per block: 512 channels
constexpr int PREP_TT = 4;     // tokens per thread
// Only the first token chunk reads the conv state (its window starts there)
// when PREP_TT >= K - 1, which keeps an in-place conv state race-free: that
// chunk's block writes the new state after reading its own rows.
static_assert(PREP_TT >= 3, "the conv state is read by the first token chunk only (K <= 4)");

template <int DK, int K>
__global__ __launch_bounds__(PREP_NT) void prep_kernel(PrepArgs p, int c_tiles, int t_chunks,
                                                    int64_t conv_blocks) {
    const int tid = threadIdx.x;
    const int64_t bid = blockIdx.x;
    const int T = p.T, Hk = p.Hk, Hv = p.Hv, Dv = p.Dv;

    if (bid >= conv_blocks) {
        // g = exp(-exp(A_log) softplus(a + dt_bias)), beta = sigmoid(b)
        const int64_t i = (bid - conv_blocks) * PREP_NT + tid;
        if (i < (int64_t)p.B * T * Hv) {
            const int h = (int)(i % Hv);
            float g, beta;
            gate_g_beta(p.a[i], p.b[i], p.A_log[h], p.dt_bias[h], g, beta);
            p.g[i] = g;
            p.beta[i] = beta;
        }
        return;
    }

    const int HKDK = Hk * DK;
    const int C = 2 * HKDK + Hv * Dv;
    const int groups = C >> 3;
    const int ct = (int)(bid % c_tiles);
    const int64_t rest = bid / c_tiles;
    const int tc = (int)(rest % t_chunks);
    const int b = (int)(rest / t_chunks);
    const int cg = ct * PREP_NT + tid;
    const bool valid = cg < groups;
    const int c0 = cg * 8;
    const int t0 = tc * PREP_TT;
    const int t1 = min(T, t0 + PREP_TT);
    const uint16_t* xb = p.qkv + (int64_t)b * T * C + c0;
    const uint16_t* csb = p.conv_state_in ? p.conv_state_in + (int64_t)b * (K - 1) * C + c0 : nullptr;

    // conv weights of the 8 channels, as stored bf16 pairs
    uint4 wk[K];
#pragma unroll
    for (int v4 = 0; v4 < K; ++v4)
        wk[v4] = valid ? reinterpret_cast<const uint4*>(p.conv_w + (int64_t)c0 * K)[v4] : make_uint4(0, 0, 0, 0);
    const ConvW<K> w = conv_weights<K>(wk);

    // spliced input row p (0 <= p < T + K - 1): conv state rows, then qkv rows
    auto xpad_row = [&](int pr) -> uint4 {
        if (!valid) return make_uint4(0, 0, 0, 0);
        if (pr >= K - 1) return *reinterpret_cast<const uint4*>(xb + (int64_t)(pr - (K - 1)) * C);
        if (csb) return *reinterpret_cast<const uint4*>(csb + (int64_t)pr * C);
        return make_uint4(0, 0, 0, 0);
    };

    // win[0 .. K-2] = xpad rows t0 .. t0+K-2 (stored bf16), win[K-1] the token's row
    uint4 win[K];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) win[j] = xpad_row(t0 + j);

    // the new conv state: last K-1 rows of xpad (read before any write, so
    // conv_state_out may alias conv_state_in)
    if (tc == 0 && valid && p.conv_state_out) {
        uint4 tail[K - 1];
#pragma unroll
        for (int i = 0; i < K - 1; ++i) tail[i] = xpad_row(T + i);
        uint16_t* out = p.conv_state_out + (int64_t)b * (K - 1) * C + c0;
#pragma unroll
        for (int i = 0; i < K - 1; ++i) *reinterpret_cast<uint4*>(out + (int64_t)i * C) = tail[i];
    }

    uint4 rows[PREP_TT];
#pragma unroll
    for (int i = 0; i < PREP_TT; ++i)
        rows[i] = (valid && t0 + i < t1) ? *reinterpret_cast<const uint4*>(xb + (int64_t)(t0 + i) * C)
                                         : make_uint4(0, 0, 0, 0);

    // region of this lane's channels
    int region;      // 0 = q, 1 = k, 2 = v
    if (c0 < HKDK) region = 0;
    else if (c0 < 2 * HKDK) region = 1;
    else region = 2;
    const float scale = region == 0 ? p.q_scale : p.k_scale;

#pragma unroll
    for (int i = 0; i < PREP_TT; ++i) {
        if (t0 + i >= t1) break;   // uniform across the block
        const int t = t0 + i;
        win[K - 1] = rows[i];
        float act[8];
        conv_silu8<K>(w, win, act);
        // q/k heads: the norm over the head's Dk/8 lanes; v lanes pass act
        // through.  Region boundaries are multiples of Dk, so a lane group
        // never mixes regions, and most waves lie wholly inside one region
        // and skip the other branch.
        uint4 o;
        if (region < 2) o = qk_norm8<DK>(act, true, scale, p.eps);
        else o = pack8(act);
        // slide the window
#pragma unroll
        for (int j = 0; j < K - 1; ++j) win[j] = win[j + 1];

        if (!valid) continue;
        const int64_t tok = (int64_t)b * T + t;
        uint16_t* dst = region == 0   ? p.q + tok * HKDK + c0
                        : region == 1 ? p.k + tok * HKDK + (c0 - HKDK)
                                      : p.v + tok * Hv * Dv + (c0 - 2 * HKDK);
        store_stream16(dst, o);
    }
}

// The new conv state alone, for T >= K - 1: its K - 1 rows are the last
// K - 1 tokens of qkv, copied one 16-byte vector per thread.  Launched after
// every reader of the old conv state has finished (stream order), so the
// state may be updated in place.
__global__ __launch_bounds__(256) void conv_tail_kernel(const uint16_t* __restrict__ qkv, uint16_t* __restrict__ out,
                                                         int T, int C, int K, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int64_t c8n = C / 8, per_b = (int64_t)(K - 1) * c8n;
    const int64_t b = i / per_b, r = i % per_b;
    const int64_t row = r / c8n, c8 = r % c8n;
    const uint4 v = *reinterpret_cast<const uint4*>(qkv + ((b * T + T - (K - 1) + row) * C + 8 * c8));
    *reinterpret_cast<uint4*>(out + ((b * (K - 1) + row) * C + 8 * c8)) = v;
}

hipError_t launch_conv_tail(const uint16_t* qkv, uint16_t* conv_state_out, int B, int T, int C, int K,
                            hipStream_t stream) {
    if (T < K - 1 || C % 8 != 0 || K < 2) return hipErrorInvalidValue;
    const int64_t n = (int64_t)B * (K - 1) * (C / 8);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(conv_tail_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, qkv,
                       conv_state_out, T, C, K, n);
    return hipGetLastError();
}

static void prep_grid(int B, int T, int Hk, int Hv, int Dk, int Dv, int& c_tiles, int& t_chunks,
                      int64_t& conv_blocks, int64_t& gate_blocks) {
    const int64_t C = 2LL * Hk * Dk + (int64_t)Hv * Dv;
    c_tiles = (int)((C / 8 + PREP_NT - 1) / PREP_NT);
    t_chunks = T > 0 ? (T + PREP_TT - 1) / PREP_TT : 1;
    conv_blocks = (int64_t)B * t_chunks * c_tiles;
    gate_blocks = ((int64_t)B * T * Hv + PREP_NT - 1) / PREP_NT;
}

int64_t prep_blocks(int B, int T, int Hk, int Hv, int Dk, int Dv) {
    int ct, tcn;
    int64_t cb, gb;
    prep_grid(B, T, Hk, Hv, Dk, Dv, ct, tcn, cb, gb);
    return cb + gb;
}

template <int DK, int K>
static hipError_t launch_prep_t(const PrepArgs& a, hipStream_t stream) {
    int c_tiles, t_chunks;
    int64_t conv_blocks, gate_blocks;
    prep_grid(a.B, a.T, a.Hk, a.Hv, a.Dk, a.Dv, c_tiles, t_chunks, conv_blocks, gate_blocks);
    const int64_t blocks = conv_blocks + gate_blocks;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((prep_kernel<DK, K>), dim3((unsigned)blocks), dim3(PREP_NT), 0, stream,
                       a, c_tiles, t_chunks, conv_blocks);
    return hipGetLastError();
}

template <int DK>
static hipError_t launch_prep_k(const PrepArgs& a, hipStream_t stream) {
    switch (a.K) {
        case 2: return launch_prep_t<DK, 2>(a, stream);
        case 3: return launch_prep_t<DK, 3>(a, stream);
        case 4: return launch_prep_t<DK, 4>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prep(const PrepArgs& a, hipStream_t stream) {
    switch (a.Dk) {
        case 32: return launch_prep_k<32>(a, stream);
        case 64: return launch_prep_k<64>(a, stream);
        case 128: return launch_prep_k<128>(a, stream);
        case 256: return launch_prep_k<256>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
