// Output epilogue of the Gated DeltaNet layer: gated RMS normalisation of the
// recurrence output ("mlex 0.1.2 -- src/models/gated_delta.rs",
// GatedDeltaNet::forward, the step after the recurrence loop).  Per row of Dv
// values (one token of one v-head), in f32:
//
//   out = bf16( silu(z) * (y * rsqrt(mean(y^2) + eps) * w) )
//
// y and z are bf16 [rows, Dv], w is bf16 [Dv] shared by every head.
//
// The work is a pure stream (2 B read of y and of z, 2 B written per value),
// so the kernel is built for HBM bandwidth: one row per group of L lanes, each
// lane holding NV 16-byte vectors (8 values each) of its row, the sum of
// squares reduced across the group with DPP row permutations, w loaded once
// per lane.  A wave covers 64/L consecutive rows, i.e. one contiguous span of
// memory, so every load and store is a fully coalesced 16-byte access.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

// Sum over aligned groups of L lanes (L a power of two up to 64); every lane
// of a group gets the group's total (each step adds a commuted pair, so the
// lanes of a group hold identical bits).
template <int L>
__device__ __forceinline__ float lane_group_sum(float x) {
    if constexpr (L >= 2) x += dpp_mov<DPP_QUAD_XOR1>(x);
    if constexpr (L >= 4) x += dpp_mov<DPP_QUAD_XOR2>(x);
    if constexpr (L >= 8) x += dpp_mov<DPP_ROW_HALF_MIRROR>(x);
    if constexpr (L >= 16) x += dpp_mov<DPP_ROW_MIRROR>(x);
    if constexpr (L >= 32) x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
    if constexpr (L >= 64) x += __shfl_xor(x, 32);
    return x;
}

constexpr int kThreads = 256;

typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));

// One 16-byte store with the non-temporal hint (a global_store ... nt): the
// output is written once and not read again here, and streaming it past the
// caches' normal retention measured faster (plain loads stay faster for y, z).
__device__ __forceinline__ void store_stream16(uint4* dst, const uint4 v) {
    const u32x4_nt x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4_nt*>(dst));
}

// y, z, out: 16-byte vectors of the [rows, Dv] arrays (nvec = Dv / 8 per
// row).  out may be y or z itself: every lane reads all of its values before
// it writes any, and writes only the positions it read.
template <int L, int NV>
__global__ __launch_bounds__(kThreads) void gated_rmsnorm_kernel(const uint4* y, const uint4* z,
                                                                 const uint4* __restrict__ w, uint4* out,
                                                                 int64_t rows, int nvec, float inv_dv,
                                                                 float eps) {
    constexpr int kRowsPerBlock = kThreads / L;
    const int lane_in_row = threadIdx.x % L;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / L;
    // Lanes past the last row still take part in the cross-lane sum (with
    // zeros), so the DPP sources are always valid lanes.
    const bool row_ok = row < rows;

    uint4 yv[NV], zv[NV], wv[NV];
    bool on[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j = lane_in_row + i * L;
        on[i] = row_ok && j < nvec;
        const int64_t off = row * nvec + j;
        yv[i] = on[i] ? y[off] : make_uint4(0, 0, 0, 0);
        zv[i] = on[i] ? z[off] : make_uint4(0, 0, 0, 0);
        wv[i] = on[i] ? w[j] : make_uint4(0, 0, 0, 0);
    }
    float ss = 0.f;
    float yf[NV][8];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        unpack8(yv[i], yf[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(yf[i][e], yf[i][e], ss);
    }
    ss = lane_group_sum<L>(ss);
    const float r = __builtin_amdgcn_rsqf(ss * inv_dv + eps);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        if (!on[i]) continue;
        float zf[8], wf[8], o[8];
        unpack8(zv[i], zf);
        unpack8(wv[i], wf);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = silu_fast(zf[e]) * (yf[i][e] * r * wf[e]);
        store_stream16(out + row * nvec + lane_in_row + i * L, pack8(o));
    }
}

template <int L, int NV>
hipError_t launch(const GatedNormArgs& a, hipStream_t stream) {
    const int64_t blocks = (a.rows + kThreads / L - 1) / (kThreads / L);
    hipLaunchKernelGGL((gated_rmsnorm_kernel<L, NV>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint4*>(a.y), reinterpret_cast<const uint4*>(a.z),
                       reinterpret_cast<const uint4*>(a.w), reinterpret_cast<uint4*>(a.out), a.rows,
                       a.Dv / 8, 1.0f / (float)a.Dv, a.eps);
    return hipGetLastError();
}

}  // namespace

int gated_norm_lanes(int Dv) {
    const int nvec = Dv / 8;
    int L = 1;
    while (L < nvec && L < 64) L *= 2;
    return L;
}

int64_t gated_norm_blocks(int64_t rows, int Dv) {
    const int64_t per = kThreads / gated_norm_lanes(Dv);
    return (rows + per - 1) / per;
}

hipError_t launch_gated_rmsnorm(const GatedNormArgs& a, hipStream_t stream) {
    if (a.rows == 0) return hipSuccess;
    const int nvec = a.Dv / 8;
    switch (gated_norm_lanes(a.Dv)) {
        case 1: return launch<1, 1>(a, stream);
        case 2: return launch<2, 1>(a, stream);
        case 4: return launch<4, 1>(a, stream);
        case 8: return launch<8, 1>(a, stream);
        case 16: return launch<16, 1>(a, stream);
        case 32: return launch<32, 1>(a, stream);
        default:
            if (nvec <= 64) return launch<64, 1>(a, stream);
            if (nvec <= 128) return launch<64, 2>(a, stream);
            if (nvec <= 256) return launch<64, 4>(a, stream);
            return launch<64, 8>(a, stream);
    }
}

}  // namespace gdn
