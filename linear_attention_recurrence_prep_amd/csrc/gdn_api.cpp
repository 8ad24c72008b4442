// C ABI of the Gated DeltaNet library: argument validation, then launches on
// the caller's stream.  Every check runs before the first launch, so a failed
// call leaves all outputs untouched.
#include "../../include/gdn.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <limits>
#include <vector>

#include "gdn_launch.h"

namespace {

constexpr int kVersion = 5;
static_assert(GDN_NO_ALLOC_SCRATCH_BYTES == gdn::kScratchBytes, "the header states the scratch size");
constexpr int64_t kMaxBlocks = (1LL << 31) - 1;

thread_local char g_err[512] = "";

gdn_status fail(gdn_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

gdn_status ok() {
    g_err[0] = '\0';
    return GDN_OK;
}

struct Span {
    const char* name;
    const void* p;
    uint64_t bytes;
    bool output;
    unsigned align = 16;    // required alignment of p in bytes
};

// Element-count product with overflow detection (all factors >= 0).
bool mul_ok(uint64_t& acc, int64_t f) {
    if (f < 0) return false;
    if (f != 0 && acc > std::numeric_limits<uint64_t>::max() / 4 / (uint64_t)f) return false;
    acc *= (uint64_t)f;
    return true;
}

bool elems(uint64_t& out, std::initializer_list<int64_t> dims) {
    uint64_t acc = 1;
    for (int64_t d : dims)
        if (!mul_ok(acc, d)) return false;
    // keep every element index inside int64 with room for byte offsets
    if (acc > (1ULL << 60)) return false;
    out = acc;
    return true;
}

gdn_status check_dims(int B, int T, int Hk, int Hv, int Dk, int Dv) {
    if (B < 0 || T < 0) return fail(GDN_ERR_BAD_DIMS, "B=%d and T=%d must be >= 0", B, T);
    if (Hk < 1 || Hv < 1) return fail(GDN_ERR_BAD_DIMS, "Hk=%d and Hv=%d must be >= 1", Hk, Hv);
    if (Hv % Hk != 0) return fail(GDN_ERR_BAD_DIMS, "Hv=%d is not a multiple of Hk=%d", Hv, Hk);
    if (Dk != 32 && Dk != 64 && Dk != 128 && Dk != 256)
        return fail(GDN_ERR_UNSUPPORTED, "Dk=%d not in {32, 64, 128, 256}", Dk);
    if (Dv < 8 || Dv > 4096 || Dv % 8 != 0)
        return fail(GDN_ERR_UNSUPPORTED, "Dv=%d must be a multiple of 8 in [8, 4096]", Dv);
    return GDN_OK;
}

gdn_status check_spans(const std::vector<Span>& s, const std::vector<std::pair<int, int>>& alias_ok) {
    for (const Span& x : s) {
        if (x.p && (reinterpret_cast<uintptr_t>(x.p) & (x.align - 1u)))
            return fail(GDN_ERR_MISALIGNED, "%s is not %u-byte aligned", x.name, x.align);
    }
    for (size_t i = 0; i < s.size(); ++i) {
        for (size_t j = i + 1; j < s.size(); ++j) {
            const Span &a = s[i], &b = s[j];
            if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) continue;
            if (!a.output && !b.output) continue;
            const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
            const bool overlap = a0 < b0 + b.bytes && b0 < a0 + a.bytes;
            if (!overlap) continue;
            bool allowed = false;
            for (auto pr : alias_ok)
                if ((pr.first == (int)i && pr.second == (int)j) || (pr.first == (int)j && pr.second == (int)i))
                    allowed = a0 == b0 && a.bytes == b.bytes;
            if (!allowed) return fail(GDN_ERR_OVERLAP, "%s overlaps %s", a.name, b.name);
        }
    }
    return GDN_OK;
}

gdn_status hip_result(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

// ------------------------------------------------------------ recurrent --

gdn_status validate_recurrent(const gdn_bf16* q, const gdn_bf16* k, const gdn_bf16* v, const float* g,
                              const float* beta, const uint8_t* mask, const float* state_in, float* state_out,
                              gdn_bf16* y, int B, int T, int Hk, int Hv, int Dk, int Dv,
                              bool check_overlap = true, bool g_per_key = false,
                              const float* snapshots = nullptr, uint64_t snapshot_bytes = 0,
                              bool need_inputs = true) {
    gdn_status st = check_dims(B, T, Hk, Hv, Dk, Dv);
    if (st != GDN_OK) return st;
    uint64_t nqk, nv, ng, ns, ngate;
    if (!elems(nqk, {B, T, Hk, Dk}) || !elems(nv, {B, T, Hv, Dv}) || !elems(ng, {B, T, Hv}) ||
        !elems(ns, {B, Hv, Dv, Dk}) || !elems(ngate, {B, T, Hv, g_per_key ? Dk : 1}))
        return fail(GDN_ERR_BAD_DIMS, "tensor sizes overflow");
    if (gdn::recurrent_blocks(B, Hv, Dk, Dv) > kMaxBlocks) return fail(GDN_ERR_BAD_DIMS, "grid too large");
    if (B > 0 && !state_out) return fail(GDN_ERR_NULL_POINTER, "state_out is NULL");
    if ((int64_t)B * T > 0) {
        if (need_inputs) {
            if (!q) return fail(GDN_ERR_NULL_POINTER, "q is NULL");
            if (!k) return fail(GDN_ERR_NULL_POINTER, "k is NULL");
            if (!v) return fail(GDN_ERR_NULL_POINTER, "v is NULL");
            if (!g) return fail(GDN_ERR_NULL_POINTER, "g is NULL");
            if (!beta) return fail(GDN_ERR_NULL_POINTER, "beta is NULL");
        }
        if (!y) return fail(GDN_ERR_NULL_POINTER, "y is NULL");
    }
    if (!check_overlap) return GDN_OK;
    std::vector<Span> s = {
        {"q", q, nqk * 2, false},        {"k", k, nqk * 2, false},
        {"v", v, nv * 2, false},         {"g", g, ngate * 4, false},
        {"beta", beta, ng * 4, false},   {"state_in", state_in, ns * 4, false},
        {"state_out", state_out, ns * 4, true}, {"y", y, nv * 2, true},
        {"mask", mask, (uint64_t)B * T, false, 1},
        {"snapshots", snapshots, snapshot_bytes, true},
    };
    return check_spans(s, {{5, 6}});
}

// ------------------------------------------------------------- epilogue --

gdn_status validate_gated(const gdn_bf16* y, const gdn_bf16* z, const gdn_bf16* w, const gdn_bf16* out, int B,
                          int T, int Hv, int Dv, float eps, bool check_overlap = true) {
    if (B < 0 || T < 0) return fail(GDN_ERR_BAD_DIMS, "B=%d and T=%d must be >= 0", B, T);
    if (Hv < 1) return fail(GDN_ERR_BAD_DIMS, "Hv=%d must be >= 1", Hv);
    if (Dv < 8 || Dv > 4096 || Dv % 8 != 0)
        return fail(GDN_ERR_UNSUPPORTED, "Dv=%d must be a multiple of 8 in [8, 4096]", Dv);
    if (!std::isfinite(eps) || eps < 0.f) return fail(GDN_ERR_BAD_VALUE, "norm eps must be finite and >= 0");
    uint64_t rows, n;
    if (!elems(rows, {B, T, Hv}) || !elems(n, {B, T, Hv, Dv})) return fail(GDN_ERR_BAD_DIMS, "tensor sizes overflow");
    if (gdn::gated_norm_blocks((int64_t)rows, Dv) > kMaxBlocks) return fail(GDN_ERR_BAD_DIMS, "grid too large");
    if (rows > 0) {
        if (!y) return fail(GDN_ERR_NULL_POINTER, "y is NULL");
        if (!z) return fail(GDN_ERR_NULL_POINTER, "z is NULL");
        if (!w) return fail(GDN_ERR_NULL_POINTER, "norm_weight is NULL");
        if (!out) return fail(GDN_ERR_NULL_POINTER, "out is NULL");
    }
    if (!check_overlap) return GDN_OK;
    std::vector<Span> s = {
        {"y", y, n * 2, false}, {"z", z, n * 2, false}, {"norm_weight", w, (uint64_t)Dv * 2, false},
        {"out", out, n * 2, true},
    };
    return check_spans(s, {{0, 3}, {1, 3}});
}

// ----------------------------------------------------------------- prep --

gdn_status validate_prep(const gdn_bf16* qkv, const gdn_bf16* conv_w, const gdn_bf16* conv_state_in,
                         gdn_bf16* conv_state_out, const gdn_bf16* a, const gdn_bf16* b, const float* A_log,
                         const float* dt_bias, gdn_bf16* q, gdn_bf16* k, gdn_bf16* v, float* g, float* beta,
                         int B, int T, int Hk, int Hv, int Dk, int Dv, int K, float q_scale, float k_scale,
                         float eps, bool check_overlap = true, bool need_outputs = true) {
    gdn_status st = check_dims(B, T, Hk, Hv, Dk, Dv);
    if (st != GDN_OK) return st;
    if (K < 2 || K > 4) return fail(GDN_ERR_UNSUPPORTED, "K=%d not in {2, 3, 4}", K);
    if (!std::isfinite(q_scale) || !std::isfinite(k_scale))
        return fail(GDN_ERR_BAD_VALUE, "q_scale and k_scale must be finite");
    if (!std::isfinite(eps) || eps < 0.f) return fail(GDN_ERR_BAD_VALUE, "eps must be finite and >= 0");
    const int64_t C = 2LL * Hk * Dk + (int64_t)Hv * Dv;
    if (C > (1LL << 30)) return fail(GDN_ERR_BAD_DIMS, "too many channels");
    uint64_t nx, nw, ncs, ng, nqk, nv;
    if (!elems(nx, {B, T, C}) || !elems(nw, {C, K}) || !elems(ncs, {B, K - 1, C}) || !elems(ng, {B, T, Hv}) ||
        !elems(nqk, {B, T, Hk, Dk}) || !elems(nv, {B, T, Hv, Dv}))
        return fail(GDN_ERR_BAD_DIMS, "tensor sizes overflow");
    if (gdn::prep_blocks(B, T, Hk, Hv, Dk, Dv) > kMaxBlocks) return fail(GDN_ERR_BAD_DIMS, "grid too large");
    if (B > 0 && !conv_w) return fail(GDN_ERR_NULL_POINTER, "conv_w is NULL");
    if ((int64_t)B * T > 0) {
        if (!qkv) return fail(GDN_ERR_NULL_POINTER, "qkv is NULL");
        if (!a) return fail(GDN_ERR_NULL_POINTER, "a is NULL");
        if (!b) return fail(GDN_ERR_NULL_POINTER, "b is NULL");
        if (!A_log) return fail(GDN_ERR_NULL_POINTER, "A_log is NULL");
        if (!dt_bias) return fail(GDN_ERR_NULL_POINTER, "dt_bias is NULL");
    }
    if ((int64_t)B * T > 0 && need_outputs) {
        if (!q) return fail(GDN_ERR_NULL_POINTER, "q is NULL");
        if (!k) return fail(GDN_ERR_NULL_POINTER, "k is NULL");
        if (!v) return fail(GDN_ERR_NULL_POINTER, "v is NULL");
        if (!g) return fail(GDN_ERR_NULL_POINTER, "g is NULL");
        if (!beta) return fail(GDN_ERR_NULL_POINTER, "beta is NULL");
    }
    if (!check_overlap) return GDN_OK;
    std::vector<Span> s = {
        {"qkv", qkv, nx * 2, false},
        {"conv_w", conv_w, nw * 2, false},
        {"conv_state_in", conv_state_in, ncs * 2, false},
        {"conv_state_out", conv_state_out, ncs * 2, true},
        {"a", a, ng * 2, false},
        {"b", b, ng * 2, false},
        {"A_log", A_log, (uint64_t)Hv * 4, false},
        {"dt_bias", dt_bias, (uint64_t)Hv * 4, false},
        {"q", q, nqk * 2, true},
        {"k", k, nqk * 2, true},
        {"v", v, nv * 2, true},
        {"g", g, ng * 4, true},
        {"beta", beta, ng * 4, true},
    };
    return check_spans(s, {{2, 3}});
}

// -------------------------------------------------------------- workspace --

struct Workspace {
    uint64_t q, k, v, g, beta, chunked, total;
    bool use_chunked;
    bool fused;      // chunked with the prologue inside its preparation: no q/k/v/g/beta region
};

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// The layer core takes the chunked recurrence for sequences of 64 steps and
// more, and for shorter ones once the batch is large: measured on MI355X at
// Hv = 32, Dk = Dv = 128, the per-step form (whose cost grows with the rounds
// of state-row blocks the device runs) stays ahead up to T = 16 at every
// batch, up to T = 32 with 2048 state tiles of 16 rows and up to T = 48 with
// fewer.  A fixed rule (no device query), so the composition is the same on
// every device.
bool layer_uses_chunked(int B, int T, int Hv, int Dk, int Dv) {
    if (!gdn::chunked_supported(Hv, Dk, Dv)) return false;
    const int64_t tiles = (int64_t)B * Hv * (Dv / 16);
    return T >= 64 || (T > 32 && tiles >= 2048) || (T > 16 && tiles >= 4096);
}

// The layer core's workspace: the prologue's q, k, v (bf16) and g, beta (f32)
// when they pass through memory, then the chunked recurrence's part when that
// form is used.  With the chunked form and Dv <= 128 the prologue runs inside
// the chunk preparation for every aliasing of the conv state, so the first
// part is absent.
bool workspace_layout(int B, int T, int Hk, int Hv, int Dk, int Dv, Workspace& w) {
    uint64_t nqk, nv, ng;
    if (!elems(nqk, {B, T, Hk, Dk}) || !elems(nv, {B, T, Hv, Dv}) || !elems(ng, {B, T, Hv})) return false;
    w.use_chunked = B > 0 && layer_uses_chunked(B, T, Hv, Dk, Dv);
    w.fused = w.use_chunked && gdn::layer_chunked_fusable(Dv, 4);
    if (w.fused) nqk = nv = ng = 0;
    w.q = 0;
    w.k = w.q + align256(nqk * 2);
    w.v = w.k + align256(nqk * 2);
    w.g = w.v + align256(nv * 2);
    w.beta = w.g + align256(ng * 4);
    w.chunked = w.beta + align256(ng * 4);
    w.total = w.chunked + (w.use_chunked ? gdn::chunked_layout(B, T, Hk, Hv, Dk, Dv).total : 0);
    if ((int64_t)B * T == 0) w.total = 0;
    return true;
}

uint64_t chunked_bytes(int B, int T, int Hk, int Hv, int Dk, int Dv, bool per_key = false) {
    if ((int64_t)B * T == 0 || !gdn::chunked_supported(Hv, Dk, Dv)) return 0;
    return gdn::chunked_layout(B, T, Hk, Hv, Dk, Dv, per_key).total;
}

}  // namespace

extern "C" {

int gdn_version(void) { return kVersion; }

const char* gdn_status_string(int status) {
    switch (status) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_NULL_POINTER: return "GDN_ERR_NULL_POINTER";
        case GDN_ERR_BAD_DIMS: return "GDN_ERR_BAD_DIMS";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
        case GDN_ERR_MISALIGNED: return "GDN_ERR_MISALIGNED";
        case GDN_ERR_OVERLAP: return "GDN_ERR_OVERLAP";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
        case GDN_ERR_BAD_VALUE: return "GDN_ERR_BAD_VALUE";
        case GDN_ERR_HIP: return "GDN_ERR_HIP";
        default: return "GDN_ERR_UNKNOWN";
    }
}

const char* gdn_last_error(void) { return g_err; }

gdn_status gdn_recurrent_masked(const gdn_bf16* q, const gdn_bf16* k, const gdn_bf16* v, const float* g,
                                const float* beta, const uint8_t* mask, const float* state_in, float* state_out,
                                gdn_bf16* y, int B, int T, int Hk, int Hv, int Dk, int Dv, void* stream) {
    gdn_status st = validate_recurrent(q, k, v, g, beta, mask, state_in, state_out, y, B, T, Hk, Hv, Dk, Dv);
    if (st != GDN_OK) return st;
    if (B == 0) return ok();
    gdn::RecurrentArgs a{q, k, v, g, beta, state_in, state_out, y, B, T, Hk, Hv, Dk, Dv, mask};
    return hip_result(gdn::launch_recurrent(a, static_cast<hipStream_t>(stream)), "recurrent");
}

gdn_status gdn_recurrent_snapshots(const gdn_bf16* q, const gdn_bf16* k, const gdn_bf16* v, const float* g,
                                   int g_per_key, const float* beta, const uint8_t* mask, const float* state_in,
                                   float* state_out, gdn_bf16* y, const int32_t* snap_steps, int n_snap,
                                   float* snapshots, int B, int T, int Hk, int Hv, int Dk, int Dv, void* stream) {
    if (n_snap < 0 || n_snap > gdn::kMaxSnapshots)
        return fail(GDN_ERR_BAD_VALUE, "n_snap=%d not in [0, %d]", n_snap, gdn::kMaxSnapshots);
    gdn::SnapList sl;
    sl.n = n_snap;
    if (n_snap > 0) {
        if (!snap_steps) return fail(GDN_ERR_NULL_POINTER, "snap_steps is NULL");
        for (int i = 0; i < n_snap; ++i) {
            const int32_t t = snap_steps[i];
            if (t < 0 || t > T) return fail(GDN_ERR_BAD_VALUE, "snap_steps[%d]=%d not in [0, T=%d]", i, t, T);
            if (i > 0 && t <= snap_steps[i - 1])
                return fail(GDN_ERR_BAD_VALUE, "snap_steps must be strictly increasing (entry %d)", i);
            sl.steps[i] = t;
        }
    }
    gdn_status st = check_dims(B, T, Hk, Hv, Dk, Dv);
    if (st != GDN_OK) return st;
    uint64_t ns;
    if (!elems(ns, {n_snap, B, Hv, Dv, Dk})) return fail(GDN_ERR_BAD_DIMS, "snapshot size overflows");
    if (n_snap > 0 && B > 0 && !snapshots) return fail(GDN_ERR_NULL_POINTER, "snapshots is NULL");
    st = validate_recurrent(q, k, v, g, beta, mask, state_in, state_out, y, B, T, Hk, Hv, Dk, Dv, true,
                            g_per_key != 0, n_snap > 0 ? snapshots : nullptr, ns * 4);
    if (st != GDN_OK) return st;
    if (B == 0) return ok();
    sl.out = snapshots;
    gdn::RecurrentArgs a{q, k, v, g, beta, state_in, state_out, y, B, T, Hk, Hv, Dk, Dv, mask};
    a.g_per_key = g_per_key != 0;
    a.snap = n_snap > 0 ? &sl : nullptr;
    return hip_result(gdn::launch_recurrent(a, static_cast<hipStream_t>(stream)), "recurrent");
}

gdn_status gdn_recurrent_per_key(const gdn_bf16* q, const gdn_bf16* k, const gdn_bf16* v, const float* g,
                                 const float* beta, const uint8_t* mask, const float* state_in, float* state_out,
                                 gdn_bf16* y, int B, int T, int Hk, int Hv, int Dk, int Dv, void* stream) {
    return gdn_recurrent_snapshots(q, k, v, g, 1, beta, mask, state_in, state_out, y, nullptr, 0, nullptr, B, T,
                                   Hk, Hv, Dk, Dv, stream);
}

gdn_status gdn_recurrent(const gdn_bf16* q, const gdn_bf16* k, const gdn_bf16* v, const float* g,
                         const float* beta, const float* state_in, float* state_out, gdn_bf16* y, int B,
                         int T, int Hk, int Hv, int Dk, int Dv, void* stream) {
    return gdn_recurrent_masked(q, k, v, g, beta, nullptr, state_in, state_out, y, B, T, Hk, Hv, Dk, Dv, stream);
}

size_t gdn_recurrent_chunked_workspace_bytes(int B, int T, int Hk, int Hv, int Dk, int Dv) {
    if (check_dims(B, T, Hk, Hv, Dk, Dv) != GDN_OK) return 0;
    uint64_t n;
    if (!elems(n, {B, T, Hv, Dk})) return 0;
    return (size_t)chunked_bytes(B, T, Hk, Hv, Dk, Dv);
}

// The chunked recurrence, per-head gate g [B,T,Hv] or per-key gate g [B,T,Hv,Dk].
static gdn_status recurrent_chunked_impl(const gdn_bf16* q, const gdn_bf16* k, const gdn_bf16* v, const float* g,
                                         bool per_key, const float* beta, const uint8_t* mask,
                                         const float* state_in, float* state_out, gdn_bf16* y, void* workspace,
                                         size_t workspace_bytes, int B, int T, int Hk, int Hv, int Dk, int Dv,
                                         void* stream) {
    gdn_status st = validate_recurrent(q, k, v, g, beta, mask, state_in, state_out, y, B, T, Hk, Hv, Dk, Dv, true,
                                       per_key);
    if (st != GDN_OK) return st;
    if (!gdn::chunked_supported(Hv, Dk, Dv))
        return fail(GDN_ERR_UNSUPPORTED,
                    "chunked recurrence needs Dk == 128, Dv %% 16 == 0 and Hv * Dv <= 2^25 (Dk=%d, Dv=%d, Hv=%d)", Dk,
                    Dv, Hv);
    if (gdn::chunked_blocks(B, T, Hv, Dv) > kMaxBlocks) return fail(GDN_ERR_BAD_DIMS, "grid too large");
    const uint64_t need = chunked_bytes(B, T, Hk, Hv, Dk, Dv, per_key);
    if (need > 0) {
        if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL but %llu bytes are needed",
                                    (unsigned long long)need);
        if (workspace_bytes < need)
            return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, %llu needed", workspace_bytes,
                        (unsigned long long)need);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(GDN_ERR_MISALIGNED, "workspace is not 256-byte aligned");
        uint64_t nqk, nv, ng, ns, ngate;
        elems(nqk, {B, T, Hk, Dk});
        elems(nv, {B, T, Hv, Dv});
        elems(ng, {B, T, Hv});
        elems(ns, {B, Hv, Dv, Dk});
        elems(ngate, {B, T, Hv, per_key ? Dk : 1});
        std::vector<Span> s = {
            {"q", q, nqk * 2, false},      {"k", k, nqk * 2, false},
            {"v", v, nv * 2, false},       {"g", g, ngate * 4, false},
            {"beta", beta, ng * 4, false}, {"state_in", state_in, ns * 4, false},
            {"state_out", state_out, ns * 4, true}, {"y", y, nv * 2, true},
            {"workspace", workspace, need, true}, {"mask", mask, (uint64_t)B * T, false, 1},
        };
        st = check_spans(s, {{5, 6}});
        if (st != GDN_OK) return st;
    }
    if (B == 0) return ok();
    gdn::RecurrentArgs a{q, k, v, g, beta, state_in, state_out, y, B, T, Hk, Hv, Dk, Dv, mask};
    a.g_per_key = per_key;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) return hip_result(gdn::launch_recurrent(a, s), "recurrent");
    return hip_result(gdn::launch_recurrent_chunked(a, workspace, s), "chunked recurrent");
}

gdn_status gdn_recurrent_chunked_masked(const gdn_bf16* q, const gdn_bf16* k, const gdn_bf16* v,
                                        const float* g, const float* beta, const uint8_t* mask,
                                        const float* state_in, float* state_out, gdn_bf16* y, void* workspace,
                                        size_t workspace_bytes, int B, int T, int Hk, int Hv, int Dk, int Dv,
                                        void* stream) {
    return recurrent_chunked_impl(q, k, v, g, false, beta, mask, state_in, state_out, y, workspace,
                                  workspace_bytes, B, T, Hk, Hv, Dk, Dv, stream);
}

gdn_status gdn_recurrent_chunked_per_key(const gdn_bf16* q, const gdn_bf16* k, const gdn_bf16* v, const float* g,
                                         const float* beta, const uint8_t* mask, const float* state_in,
                                         float* state_out, gdn_bf16* y, void* workspace, size_t workspace_bytes,
                                         int B, int T, int Hk, int Hv, int Dk, int Dv, void* stream) {
    return recurrent_chunked_impl(q, k, v, g, true, beta, mask, state_in, state_out, y, workspace,
                                  workspace_bytes, B, T, Hk, Hv, Dk, Dv, stream);
}

size_t gdn_recurrent_chunked_per_key_workspace_bytes(int B, int T, int Hk, int Hv, int Dk, int Dv) {
    if (check_dims(B, T, Hk, Hv, Dk, Dv) != GDN_OK) return 0;
    uint64_t n;
    if (!elems(n, {B, T, Hv, Dk})) return 0;
    return (size_t)chunked_bytes(B, T, Hk, Hv, Dk, Dv, true);
}

gdn_status gdn_recurrent_chunked(const gdn_bf16* q, const gdn_bf16* k, const gdn_bf16* v, const float* g,
                                 const float* beta, const float* state_in, float* state_out, gdn_bf16* y,
                                 void* workspace, size_t workspace_bytes, int B, int T, int Hk, int Hv, int Dk,
                                 int Dv, void* stream) {
    return gdn_recurrent_chunked_masked(q, k, v, g, beta, nullptr, state_in, state_out, y, workspace,
                                        workspace_bytes, B, T, Hk, Hv, Dk, Dv, stream);
}

gdn_status gdn_prep(const gdn_bf16* qkv, const gdn_bf16* conv_w, const gdn_bf16* conv_state_in,
                    gdn_bf16* conv_state_out, const gdn_bf16* a, const gdn_bf16* b, const float* A_log,
                    const float* dt_bias, gdn_bf16* q, gdn_bf16* k, gdn_bf16* v, float* g, float* beta, int B,
                    int T, int Hk, int Hv, int Dk, int Dv, int K, float q_scale, float k_scale, float eps,
                    void* stream) {
    gdn_status st = validate_prep(qkv, conv_w, conv_state_in, conv_state_out, a, b, A_log, dt_bias, q, k, v, g,
                                  beta, B, T, Hk, Hv, Dk, Dv, K, q_scale, k_scale, eps);
    if (st != GDN_OK) return st;
    if (B == 0) return ok();
    if (T == 0 && !conv_state_out) return ok();
    gdn::PrepArgs p{qkv, conv_w, conv_state_in, conv_state_out, a, b, A_log, dt_bias, q, k, v, g, beta,
                    B, T, Hk, Hv, Dk, Dv, K, q_scale, k_scale, eps};
    return hip_result(gdn::launch_prep(p, static_cast<hipStream_t>(stream)), "prep");
}

size_t gdn_layer_core_workspace_bytes(int B, int T, int Hk, int Hv, int Dk, int Dv) {
    if (check_dims(B, T, Hk, Hv, Dk, Dv) != GDN_OK) return 0;
    Workspace w;
    if (!workspace_layout(B, T, Hk, Hv, Dk, Dv, w)) return 0;
    return (size_t)w.total;
}

// The layer core, optionally followed by the output epilogue (gated: z and
// norm_weight given), which then runs in place on y.
static gdn_status layer_core_impl(const gdn_bf16* qkv, const gdn_bf16* conv_w, const gdn_bf16* conv_state_in,
                                  gdn_bf16* conv_state_out, const gdn_bf16* a, const gdn_bf16* b,
                                  const float* A_log, const float* dt_bias, const uint8_t* mask,
                                  const float* state_in, float* state_out, gdn_bf16* y, void* workspace,
                                  size_t workspace_bytes, int B, int T, int Hk, int Hv, int Dk, int Dv, int K,
                                  float q_scale, float k_scale, float eps, bool gated, const gdn_bf16* z,
                                  const gdn_bf16* norm_weight, float norm_eps, void* stream) {
    gdn_status st = check_dims(B, T, Hk, Hv, Dk, Dv);
    if (st != GDN_OK) return st;
    Workspace w;
    if (!workspace_layout(B, T, Hk, Hv, Dk, Dv, w)) return fail(GDN_ERR_BAD_DIMS, "tensor sizes overflow");
    if (w.total > 0) {
        if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL but %llu bytes are needed",
                                    (unsigned long long)w.total);
        if (workspace_bytes < w.total)
            return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, %llu needed", workspace_bytes,
                        (unsigned long long)w.total);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(GDN_ERR_MISALIGNED, "workspace is not 256-byte aligned");
    }
    char* ws = static_cast<char*>(workspace);
    const bool staged = w.total && !w.fused;     // prologue outputs pass through the workspace
    gdn_bf16* wq = staged ? reinterpret_cast<gdn_bf16*>(ws + w.q) : nullptr;
    gdn_bf16* wk = staged ? reinterpret_cast<gdn_bf16*>(ws + w.k) : nullptr;
    gdn_bf16* wv = staged ? reinterpret_cast<gdn_bf16*>(ws + w.v) : nullptr;
    float* wg = staged ? reinterpret_cast<float*>(ws + w.g) : nullptr;
    float* wb = staged ? reinterpret_cast<float*>(ws + w.beta) : nullptr;

    // the prologue half (its outputs are the workspace, or registers and LDS
    // when fused; overlap of the user buffers is checked below across both
    // halves)
    st = validate_prep(qkv, conv_w, conv_state_in, conv_state_out, a, b, A_log, dt_bias, wq, wk, wv, wg, wb, B, T,
                       Hk, Hv, Dk, Dv, K, q_scale, k_scale, eps, false, !w.fused);
    if (st != GDN_OK) return st;
    st = validate_recurrent(wq, wk, wv, wg, wb, mask, state_in, state_out, y, B, T, Hk, Hv, Dk, Dv, false, false,
                            nullptr, 0, !w.fused);
    if (st != GDN_OK) return st;
    if (gated) {
        st = validate_gated(y, z, norm_weight, y, B, T, Hv, Dv, norm_eps, false);
        if (st != GDN_OK) return st;
    }
    if (w.use_chunked && gdn::chunked_blocks(B, T, Hv, Dv) > kMaxBlocks) return fail(GDN_ERR_BAD_DIMS, "grid too large");
    {
        const int64_t C = 2LL * Hk * Dk + (int64_t)Hv * Dv;
        uint64_t nx, nw, ncs, ng, nv, ns;
        elems(nx, {B, T, C});
        elems(nw, {C, K});
        elems(ncs, {B, K - 1, C});
        elems(ng, {B, T, Hv});
        elems(nv, {B, T, Hv, Dv});
        elems(ns, {B, Hv, Dv, Dk});
        std::vector<Span> s = {
            {"qkv", qkv, nx * 2, false},
            {"conv_w", conv_w, nw * 2, false},
            {"conv_state_in", conv_state_in, ncs * 2, false},
            {"conv_state_out", conv_state_out, ncs * 2, true},
            {"a", a, ng * 2, false},
            {"b", b, ng * 2, false},
            {"A_log", A_log, (uint64_t)Hv * 4, false},
            {"dt_bias", dt_bias, (uint64_t)Hv * 4, false},
            {"state_in", state_in, ns * 4, false},
            {"state_out", state_out, ns * 4, true},
            {"y", y, nv * 2, true},
            {"workspace", workspace, w.total, true},
            {"mask", mask, (uint64_t)B * T, false, 1},
            {"z", gated ? z : nullptr, nv * 2, false},
            {"norm_weight", gated ? norm_weight : nullptr, (uint64_t)Dv * 2, false},
        };
        st = check_spans(s, {{2, 3}, {8, 9}});
        if (st != GDN_OK) return st;
    }
    if (B == 0) return ok();
    hipStream_t s = static_cast<hipStream_t>(stream);
    gdn::RecurrentArgs r{wq, wk, wv, wg, wb, state_in, state_out, y, B, T, Hk, Hv, Dk, Dv, mask};
    if (w.fused) {
        // the prologue runs inside the chunk preparation (same arithmetic, same bits)
        const gdn::PrologueIn p{qkv, conv_w, conv_state_in, conv_state_out, a, b, A_log, dt_bias,
                                q_scale, k_scale, eps};
        st = hip_result(gdn::launch_layer_chunked(r, p, K, ws + w.chunked, s), "chunked layer core");
    } else if (T == 1 && gdn::decode_fusable(B, Hk, Hv, Dk, Dv, K)) {
        // single-token decode of a large batch: prologue and step in one launch (same bits)
        gdn::PrepArgs p{qkv, conv_w, conv_state_in, conv_state_out, a, b, A_log, dt_bias, wq, wk, wv, wg, wb,
                        B, T, Hk, Hv, Dk, Dv, K, q_scale, k_scale, eps};
        st = hip_result(gdn::launch_decode_core(p, mask, state_in, state_out, y, s), "decode layer core");
    } else {
        if (T > 0 || conv_state_out) {
            gdn::PrepArgs p{qkv, conv_w, conv_state_in, conv_state_out, a, b, A_log, dt_bias, wq, wk, wv, wg, wb,
                            B, T, Hk, Hv, Dk, Dv, K, q_scale, k_scale, eps};
            st = hip_result(gdn::launch_prep(p, s), "prep");
            if (st != GDN_OK) return st;
        }
        st = w.use_chunked ? hip_result(gdn::launch_recurrent_chunked(r, ws + w.chunked, s), "chunked recurrent")
                           : hip_result(gdn::launch_recurrent(r, s), "recurrent");
    }
    if (st != GDN_OK || !gated) return st;
    gdn::GatedNormArgs e{y, z, norm_weight, y, (int64_t)B * T * Hv, Dv, norm_eps};
    return hip_result(gdn::launch_gated_rmsnorm(e, s), "gated rmsnorm");
}

gdn_status gdn_layer_core_masked(const gdn_bf16* qkv, const gdn_bf16* conv_w, const gdn_bf16* conv_state_in,
                                 gdn_bf16* conv_state_out, const gdn_bf16* a, const gdn_bf16* b,
                                 const float* A_log, const float* dt_bias, const uint8_t* mask,
                                 const float* state_in, float* state_out, gdn_bf16* y, void* workspace,
                                 size_t workspace_bytes, int B, int T, int Hk, int Hv, int Dk, int Dv, int K,
                                 float q_scale, float k_scale, float eps, void* stream) {
    return layer_core_impl(qkv, conv_w, conv_state_in, conv_state_out, a, b, A_log, dt_bias, mask, state_in,
                           state_out, y, workspace, workspace_bytes, B, T, Hk, Hv, Dk, Dv, K, q_scale, k_scale,
                           eps, false, nullptr, nullptr, 0.f, stream);
}

gdn_status gdn_layer_core_no_alloc(const gdn_bf16* qkv, const gdn_bf16* conv_w, const gdn_bf16* conv_state_in,
                                   gdn_bf16* conv_state_out, const gdn_bf16* a, const gdn_bf16* b,
                                   const float* A_log, const float* dt_bias, const uint8_t* mask,
                                   const float* state_in, float* state_out, gdn_bf16* y, int B, int T, int Hk,
                                   int Hv, int Dk, int Dv, int K, float q_scale, float k_scale, float eps,
                                   void* stream) {
    gdn_status st = check_dims(B, T, Hk, Hv, Dk, Dv);
    if (st != GDN_OK) return st;
    Workspace w;
    if (!workspace_layout(B, T, Hk, Hv, Dk, Dv, w)) return fail(GDN_ERR_BAD_DIMS, "tensor sizes overflow");
    if (w.total > gdn::kScratchBytes)
        return fail(GDN_ERR_WORKSPACE,
                    "these sizes need %llu bytes of workspace, more than the %llu bytes of library scratch; "
                    "call gdn_layer_core_masked with a caller workspace instead",
                    (unsigned long long)w.total, (unsigned long long)gdn::kScratchBytes);
    void* scratch = nullptr;
    const hipError_t e = gdn::scratch_buffer(&scratch);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "library scratch set-up failed: %s", hipGetErrorString(e));
    return layer_core_impl(qkv, conv_w, conv_state_in, conv_state_out, a, b, A_log, dt_bias, mask, state_in,
                           state_out, y, scratch, (size_t)gdn::kScratchBytes, B, T, Hk, Hv, Dk, Dv, K, q_scale,
                           k_scale, eps, false, nullptr, nullptr, 0.f, stream);
}

gdn_status gdn_layer_core_gated(const gdn_bf16* qkv, const gdn_bf16* conv_w, const gdn_bf16* conv_state_in,
                                gdn_bf16* conv_state_out, const gdn_bf16* a, const gdn_bf16* b,
                                const float* A_log, const float* dt_bias, const gdn_bf16* z,
                                const gdn_bf16* norm_weight, const uint8_t* mask, const float* state_in,
                                float* state_out, gdn_bf16* out, void* workspace, size_t workspace_bytes, int B,
                                int T, int Hk, int Hv, int Dk, int Dv, int K, float q_scale, float k_scale,
                                float eps, float norm_eps, void* stream) {
    return layer_core_impl(qkv, conv_w, conv_state_in, conv_state_out, a, b, A_log, dt_bias, mask, state_in,
                           state_out, out, workspace, workspace_bytes, B, T, Hk, Hv, Dk, Dv, K, q_scale, k_scale,
                           eps, true, z, norm_weight, norm_eps, stream);
}

gdn_status gdn_gated_rmsnorm(const gdn_bf16* y, const gdn_bf16* z, const gdn_bf16* norm_weight, gdn_bf16* out,
                             int B, int T, int Hv, int Dv, float eps, void* stream) {
    gdn_status st = validate_gated(y, z, norm_weight, out, B, T, Hv, Dv, eps);
    if (st != GDN_OK) return st;
    const int64_t rows = (int64_t)B * T * Hv;
    if (rows == 0) return ok();
    gdn::GatedNormArgs e{y, z, norm_weight, out, rows, Dv, eps};
    return hip_result(gdn::launch_gated_rmsnorm(e, static_cast<hipStream_t>(stream)), "gated rmsnorm");
}

gdn_status gdn_layer_core(const gdn_bf16* qkv, const gdn_bf16* conv_w, const gdn_bf16* conv_state_in,
                          gdn_bf16* conv_state_out, const gdn_bf16* a, const gdn_bf16* b, const float* A_log,
                          const float* dt_bias, const float* state_in, float* state_out, gdn_bf16* y,
                          void* workspace, size_t workspace_bytes, int B, int T, int Hk, int Hv, int Dk,
                          int Dv, int K, float q_scale, float k_scale, float eps, void* stream) {
    return gdn_layer_core_masked(qkv, conv_w, conv_state_in, conv_state_out, a, b, A_log, dt_bias, nullptr,
                                 state_in, state_out, y, workspace, workspace_bytes, B, T, Hk, Hv, Dk, Dv, K,
                                 q_scale, k_scale, eps, stream);
}

}  // extern "C"
