// Internal launchers of the Gated DeltaNet kernels.  Arguments are validated
// by the C ABI layer (gdn_api.cpp) before these are called.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace gdn {

// States to emit after chosen step counts (the per-step kernels only).
constexpr int kMaxSnapshots = 32;
struct SnapList {
    int n = 0;                      // number of snapshots (0 = none)
    int steps[kMaxSnapshots] = {};  // strictly increasing step counts in [0, T]
    float* out = nullptr;           // [n, B, Hv, Dv, Dk]
};

struct RecurrentArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* g;
    const float* beta;
    const float* state_in;   // may be null (zeros)
    float* state_out;
    uint16_t* y;
    int B, T, Hk, Hv, Dk, Dv;
    const uint8_t* mask = nullptr;   // [B, T] step mask (0 = inactive), may be null
    bool g_per_key = false;          // g is [B, T, Hv, Dk] (per-key decay)
    const SnapList* snap = nullptr;  // states after chosen step counts, may be null
};

struct PrepArgs {
    const uint16_t* qkv;
    const uint16_t* conv_w;
    const uint16_t* conv_state_in;   // may be null (zeros)
    uint16_t* conv_state_out;        // may be null (not written)
    const uint16_t* a;
    const uint16_t* b;
    const float* A_log;
    const float* dt_bias;
    uint16_t* q;
    uint16_t* k;
    uint16_t* v;
    float* g;
    float* beta;
    int B, T, Hk, Hv, Dk, Dv, K;
    float q_scale, k_scale, eps;
};

// Number of blocks each launcher would use (for grid-size validation).
int64_t recurrent_blocks(int B, int Hv, int Dk, int Dv);
// The current device's compute-unit count, cached per device (0 if unknown).
int device_cu_count();
int64_t prep_blocks(int B, int T, int Hk, int Hv, int Dk, int Dv);

hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t stream);

// The layer core at T = 1 in one launch (prologue and step per (b, k-head)
// block; the bits of launch_prep followed by launch_recurrent).  For one to
// four (b, k-head) pairs per CU, (Hv / Hk) * Dv <= 1024, K in {2, 3, 4}; the
// conv state may be updated in place.
bool decode_fusable(int B, int Hk, int Hv, int Dk, int Dv, int K);
hipError_t launch_decode_core(const PrepArgs& p, const uint8_t* mask, const float* state_in, float* state_out,
                              uint16_t* y, hipStream_t stream);

// Chunked (matrix-core) recurrence: Dk == 128, Dv a multiple of 16,
// Hv * Dv <= 2^25.  Its workspace holds, per (b, hv, 32-step chunk), W
// [32 x Dk] and -T diag(beta) V [32 x Dv] in f32, -P
// [32 x 32] as two bf16 planes, -rho and gamma [32 each] in f32, and per
// (b, hk, chunk) q and k [32 x Dk] in bf16, all in the register layout of the
// sequential kernel (byte offsets below, each 256-byte aligned).  With the
// per-key gate (RecurrentArgs::g_per_key) q and k are replaced per (b, hv,
// chunk) by q o Gamma_t (two bf16 planes) and -(k o Gamma_{C-1} / Gamma_t)
// (f32), and the decay record also holds Gamma_{C-1} [Dk].
struct ChunkedLayout {
    int nc;                 // chunks per sequence
    uint64_t wsw, u, pn, rg, qsw, ksw, total;
};
bool chunked_supported(int Hv, int Dk, int Dv);
ChunkedLayout chunked_layout(int B, int T, int Hk, int Hv, int Dk, int Dv, bool per_key = false);
int64_t chunked_blocks(int B, int T, int Hv, int Dv);
hipError_t launch_recurrent_chunked(const RecurrentArgs& a, void* workspace, hipStream_t stream);

// The prologue's inputs, for the chunk preparation that computes q, k, v,
// g and beta itself (unused otherwise).
struct PrologueIn {
    const uint16_t* qkv;
    const uint16_t* conv_w;
    const uint16_t* conv_state_in;   // may be null (zeros)
    uint16_t* conv_state_out;        // may be null, or conv_state_in itself
    const uint16_t* a;
    const uint16_t* b;
    const float* A_log;
    const float* dt_bias;
    float q_scale, k_scale, eps;
};

// The layer core's chunked recurrence with the prologue fused into the chunk
// preparation: q, k, v, g, beta of RecurrentArgs are not read (computed from
// p), conv_state_out is written.  Needs Dv <= 128 and K in {2, 3, 4}; the
// result is bit-identical to launch_prep followed by launch_recurrent_chunked.
// An in-place conv state with Hv / Hk > 2 (several preparation blocks read a
// k-head's old conv state) is written by a separate copy after the
// preparation, which needs T >= K - 1 (always true where the layer core
// takes the chunked form).
bool layer_chunked_fusable(int Dv, int K);
hipError_t launch_layer_chunked(const RecurrentArgs& a, const PrologueIn& p, int K, void* workspace,
                                hipStream_t stream);
hipError_t launch_prep(const PrepArgs& a, hipStream_t stream);
// conv_state_out = the last K - 1 tokens of qkv (needs T >= K - 1); stream
// ordered after the launches that read conv_state_in, so in place is safe.
hipError_t launch_conv_tail(const uint16_t* qkv, uint16_t* conv_state_out, int B, int T, int C, int K,
                            hipStream_t stream);

// Output epilogue: out = bf16(silu(z) * rms_norm(y) * w) per row of Dv
// values (Dv a multiple of 8); out may alias y or z exactly.
struct GatedNormArgs {
    const uint16_t* y;
    const uint16_t* z;
    const uint16_t* w;
    uint16_t* out;
    int64_t rows;
    int Dv;
    float eps;
};
// The allocation-free layer core's workspace: a device array of kScratchBytes
// per device, held by the library until the process ends.  scratch_buffer
// returns its address on the current device (looked up on the first call on
// each device; thread-safe).  Every call on a device shares that device's
// array.
constexpr uint64_t kScratchBytes = 128ull << 20;
hipError_t scratch_buffer(void** ptr);

int gated_norm_lanes(int Dv);
int64_t gated_norm_blocks(int64_t rows, int Dv);
hipError_t launch_gated_rmsnorm(const GatedNormArgs& a, hipStream_t stream);

}  // namespace gdn
