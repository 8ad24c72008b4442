/*
 * gdn.h -- C ABI of the Gated DeltaNet layer-core library for MI355X (gfx950).
 *
 * The library computes the data-parallel prologue and the per-timestep gated
 * delta-rule recurrence of the Gated DeltaNet linear-attention layer, as
 * defined by "mlex 0.1.2 -- src/models/gated_delta.rs" (GatedDeltaNet::forward)
 * and "mlx-bun 0.4.0 -> 1.0.0, package/src/model/qwen3-delta.ts" (the
 * layout/dtype contract in its file header, compute_g and gated_delta_step).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers (HIP device memory of the current device),
 *   row-major and contiguous.  bf16 tensors are raw bfloat16 bit patterns
 *   (gdn_bf16).  Every tensor pointer must be 16-byte aligned.
 * - Ownership: the caller owns every buffer.  The library never allocates or
 *   frees device memory and keeps no caller pointer after returning; the
 *   only device memory it holds is the scratch array of
 *   gdn_layer_core_no_alloc (reserved by the code object, see there).
 * - Execution: every call only enqueues kernels on `stream` (a hipStream_t
 *   passed as void*; NULL is the null stream) and returns without
 *   synchronising.  Outputs are valid once the stream reaches that point.
 * - Errors: all argument validation happens before any launch; on a non-zero
 *   status no kernel was enqueued and no output was touched.  The status is
 *   one of gdn_status; gdn_last_error() returns a thread-local description of
 *   the most recent failure on the calling thread.  A GDN_ERR_HIP status means
 *   a launch failed; the stream may then hold partial work.
 * - Aliasing: outputs must not overlap any other argument, with two
 *   exceptions: state_out may equal state_in exactly (in-place state update),
 *   and conv_state_out may equal conv_state_in exactly.
 * - Dimensions: B >= 0 and T >= 0 (zero is allowed, see each call);
 *   Hk >= 1, Hv >= 1, Hv % Hk == 0 (GQA: v-head hv reads k-head
 *   hk = hv / (Hv / Hk), the repeat order of the pages); Dk in
 *   {32, 64, 128, 256}; Dv a multiple of 8 in [8, 4096]; conv kernel size K
 *   in {2, 3, 4}.
 * - Concurrency: calls on different streams or threads are independent,
 *   except gdn_layer_core_no_alloc calls on one device, which share that
 *   device's scratch array.  The library's other global state is the
 *   thread-local error and a per-device cache of the compute-unit count
 *   (read once; it picks between kernels whose results are bit-identical).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t gdn_bf16; /* raw bfloat16 bits */

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_NULL_POINTER = -1, /* a required pointer is NULL */
    GDN_ERR_BAD_DIMS = -2,     /* negative/zero size, Hv % Hk != 0, overflow */
    GDN_ERR_UNSUPPORTED = -3,  /* Dk, Dv or K outside the supported set */
    GDN_ERR_MISALIGNED = -4,   /* a tensor pointer is not 16-byte aligned */
    GDN_ERR_OVERLAP = -5,      /* an output overlaps another argument */
    GDN_ERR_WORKSPACE = -6,    /* workspace missing or too small */
    GDN_ERR_BAD_VALUE = -7,    /* non-finite or negative scale / eps */
    GDN_ERR_HIP = -8           /* a kernel launch failed */
} gdn_status;

/* Library ABI version (incremented when entry points are added or changed). */
int gdn_version(void);

/* Static name of a status code. */
const char *gdn_status_string(int status);

/* Thread-local text of the last failure on this thread ("" if none). */
const char *gdn_last_error(void);

/*
 * gdn_recurrent -- the gated delta rule over T steps.
 * ("mlex ... gated_delta.rs", recurrence loop of GatedDeltaNet::forward;
 *  "mlx-bun ... qwen3-delta.ts", gated_delta_step and gatedDeltaUpdate.)
 *
 * For each batch row b, v-head hv (k-head hk = hv / (Hv/Hk)) and t = 0..T-1:
 *   S <- g_t S;  kv = S k_t;  delta = (v_t - kv) beta_t;
 *   S <- S + delta k_t^T;  y_t = S q_t (rounded to bf16, nearest even).
 * S is fp32 [Dv, Dk] per (b, hv), held on chip across the T loop.
 *
 *   q, k      [B,T,Hk,Dk] bf16   (already normalised and scaled)
 *   v         [B,T,Hv,Dv] bf16
 *   g, beta   [B,T,Hv]    f32
 *   state_in  [B,Hv,Dv,Dk] f32, or NULL for a zero initial state
 *   state_out [B,Hv,Dv,Dk] f32, may equal state_in
 *   y         [B,T,Hv,Dv] bf16
 * T == 0 copies state_in (or zeros) to state_out; B == 0 does nothing.
 * q, k, v, g, beta and y may be NULL only when B*T == 0.
 */
gdn_status gdn_recurrent(const gdn_bf16 *q, const gdn_bf16 *k, const gdn_bf16 *v,
                         const float *g, const float *beta,
                         const float *state_in, float *state_out, gdn_bf16 *y,
                         int B, int T, int Hk, int Hv, int Dk, int Dv, void *stream);

/*
 * gdn_recurrent_masked -- gdn_recurrent with a step mask.
 * ("mlx-bun ... qwen3-delta.ts", the masked variant of the step kernel that
 *  padded prefill selects: the whole step runs only where the mask is set.)
 *
 *   mask  [B,T] uint8, nonzero = active step; NULL = every step active
 *         (then identical to gdn_recurrent).  Any alignment; read only.
 * An inactive step leaves the state untouched (no decay, no update) and
 * writes y_t = 0 (+0.0 in bf16).  Masking steps out equals dropping them from
 * the sequence, row by row.  Other arguments as gdn_recurrent.
 */
gdn_status gdn_recurrent_masked(const gdn_bf16 *q, const gdn_bf16 *k, const gdn_bf16 *v,
                                const float *g, const float *beta, const uint8_t *mask,
                                const float *state_in, float *state_out, gdn_bf16 *y,
                                int B, int T, int Hk, int Hv, int Dk, int Dv, void *stream);

/*
 * gdn_recurrent_chunked -- the same recurrence as gdn_recurrent, evaluated in
 * chunks of 32 steps on the matrix cores: within a chunk the deltas of all
 * steps solve one unit lower-triangular system built from k_t . k_s, beta
 * and the decay ratios, and the state advances by one dense product per
 * chunk.  Precision: the state path is fp32 -- W S^T runs on the f32 matrix
 * instruction; in the other products every f32 operand is cut exactly into
 * three bf16 planes and the plane products are kept down to 2^-16 of the
 * leading one (the dropped terms are below 2^-24 relative), with f32
 * accumulation; y is formed from the two leading planes (2^-16 relative) and
 * then rounded to bf16 (nearest even).  Results differ
 * from gdn_recurrent by rounding only: the same tolerances hold against the
 * exact recurrence, not bit equality.
 * Arguments as gdn_recurrent plus a caller-owned device workspace of at least
 * gdn_recurrent_chunked_workspace_bytes(...) bytes (256-byte aligned; not
 * read before written; may be NULL when that size is 0).
 * Supported sizes: Dk == 128, Dv a multiple of 16 and Hv * Dv <= 2^25 (else
 * GDN_ERR_UNSUPPORTED).  Splitting a sequence at a multiple of 32 steps and
 * carrying the state gives bit-identical results.
 */
gdn_status gdn_recurrent_chunked(const gdn_bf16 *q, const gdn_bf16 *k, const gdn_bf16 *v,
                                 const float *g, const float *beta,
                                 const float *state_in, float *state_out, gdn_bf16 *y,
                                 void *workspace, size_t workspace_bytes,
                                 int B, int T, int Hk, int Hv, int Dk, int Dv, void *stream);

/* gdn_recurrent_chunked with a step mask (semantics of gdn_recurrent_masked;
 * NULL = every step active). */
gdn_status gdn_recurrent_chunked_masked(const gdn_bf16 *q, const gdn_bf16 *k, const gdn_bf16 *v,
                                        const float *g, const float *beta, const uint8_t *mask,
                                        const float *state_in, float *state_out, gdn_bf16 *y,
                                        void *workspace, size_t workspace_bytes,
                                        int B, int T, int Hk, int Hv, int Dk, int Dv, void *stream);

/* Workspace bytes of gdn_recurrent_chunked (0 for unsupported sizes or
 * B*T == 0). */
size_t gdn_recurrent_chunked_workspace_bytes(int B, int T, int Hk, int Hv, int Dk, int Dv);

/*
 * gdn_prep -- the data-parallel prologue.
 * ("mlex ... gated_delta.rs", GatedDeltaNet::forward from the conv-state
 *  splice through g; "mlx-bun ... qwen3-delta.ts", compute_g.)
 *
 *   xpad = [conv_state_in (zeros if NULL) ; qkv[b]] along T      (T+K-1 rows)
 *   u[t,c] = sum_j conv_w[c,j] xpad[t+j,c]   (cross-correlation, no bias)
 *   x = u sigmoid(u)                                              (SiLU)
 *   q = x[:, 0:Hk*Dk], k = x[:, Hk*Dk:2*Hk*Dk], v = x[:, 2*Hk*Dk:]
 *   q_hat = q / sqrt(mean_Dk(q^2) + eps) * q_scale (per head), k_hat likewise
 *   with k_scale; q_hat, k_hat, v rounded once to bf16 (nearest even).
 *   g = exp(-exp(A_log[hv]) softplus(a + dt_bias[hv])), beta = sigmoid(b), f32.
 *   conv_state_out = the last K-1 rows of xpad.
 *
 *   qkv            [B,T,C] bf16, C = 2*Hk*Dk + Hv*Dv
 *   conv_w         [C,K] bf16
 *   conv_state_in  [B,K-1,C] bf16 or NULL (zeros)
 *   conv_state_out [B,K-1,C] bf16 or NULL (not written); may equal
 *                  conv_state_in
 *   a, b           [B,T,Hv] bf16
 *   A_log, dt_bias [Hv] f32
 *   q, k           [B,T,Hk,Dk] bf16 out;  v [B,T,Hv,Dv] bf16 out
 *   g, beta        [B,T,Hv] f32 out
 *   q_scale, k_scale finite; eps finite and >= 0.
 * T == 0 only writes conv_state_out (a copy of conv_state_in, or zeros).
 */
gdn_status gdn_prep(const gdn_bf16 *qkv, const gdn_bf16 *conv_w,
                    const gdn_bf16 *conv_state_in, gdn_bf16 *conv_state_out,
                    const gdn_bf16 *a, const gdn_bf16 *b,
                    const float *A_log, const float *dt_bias,
                    gdn_bf16 *q, gdn_bf16 *k, gdn_bf16 *v, float *g, float *beta,
                    int B, int T, int Hk, int Hv, int Dk, int Dv, int K,
                    float q_scale, float k_scale, float eps, void *stream);

/*
 * Bytes of device workspace gdn_layer_core needs for these sizes, sized to
 * the path the call takes (see gdn_layer_core):
 *   - chunked form with Dv <= 128: the chunked recurrence's workspace only
 *     (the prologue runs inside the chunk preparation; its q, k, v, g, beta
 *     never reach memory);
 *   - chunked form with Dv > 128: the bf16 q, k, v and f32 g, beta of the
 *     prologue, then the chunked recurrence's workspace;
 *   - per-step form: the prologue's q, k, v, g, beta only.
 * Each part is 256-byte aligned.  Returns 0 for invalid sizes (and when
 * B*T == 0).  The same for every conv kernel size K and every aliasing of
 * the conv state.
 */
size_t gdn_layer_core_workspace_bytes(int B, int T, int Hk, int Hv, int Dk, int Dv);

/*
 * gdn_layer_core -- gdn_prep followed by the recurrence, on one stream:
 * gdn_recurrent_chunked when it supports the sizes and T >= 64, or T > 32
 * with B * Hv * Dv / 16 >= 2048, or T > 16 with B * Hv * Dv / 16 >= 4096;
 * else gdn_recurrent.  Results are bit-identical to making those two calls
 * (which the library may fuse: the prologue runs inside the chunk preparation,
 * and single-token decode of a large batch is one launch).
 * ("mlex ... gated_delta.rs", GatedDeltaNet::forward between the input
 *  projections and the output normalisation.)
 *
 * Arguments as gdn_prep (inputs) and gdn_recurrent (state_in, state_out, y).
 * workspace: device buffer of at least gdn_layer_core_workspace_bytes(...)
 * bytes, 256-byte aligned, owned by the caller, not read before it is
 * written; it may be NULL when that size is 0.
 */
gdn_status gdn_layer_core(const gdn_bf16 *qkv, const gdn_bf16 *conv_w,
                          const gdn_bf16 *conv_state_in, gdn_bf16 *conv_state_out,
                          const gdn_bf16 *a, const gdn_bf16 *b,
                          const float *A_log, const float *dt_bias,
                          const float *state_in, float *state_out, gdn_bf16 *y,
                          void *workspace, size_t workspace_bytes,
                          int B, int T, int Hk, int Hv, int Dk, int Dv, int K,
                          float q_scale, float k_scale, float eps, void *stream);

/*
 * gdn_layer_core_masked -- gdn_layer_core with a step mask on the recurrence
 * (semantics of gdn_recurrent_masked; NULL = every step active).  As on the
 * pages, the mask applies to the recurrence only: the prologue (conv, norms,
 * gates, conv_state_out) runs over every token.  Bit-identical to gdn_prep
 * followed by gdn_recurrent_chunked_masked / gdn_recurrent_masked under the
 * same rule as gdn_layer_core.
 */
gdn_status gdn_layer_core_masked(const gdn_bf16 *qkv, const gdn_bf16 *conv_w,
                                 const gdn_bf16 *conv_state_in, gdn_bf16 *conv_state_out,
                                 const gdn_bf16 *a, const gdn_bf16 *b,
                                 const float *A_log, const float *dt_bias, const uint8_t *mask,
                                 const float *state_in, float *state_out, gdn_bf16 *y,
                                 void *workspace, size_t workspace_bytes,
                                 int B, int T, int Hk, int Hv, int Dk, int Dv, int K,
                                 float q_scale, float k_scale, float eps, void *stream);

/*
 * gdn_recurrent_snapshots -- the recurrence (per-step form) that also emits
 * the state after chosen numbers of steps, so that a speculative-verify
 * rollback to the first `keep` tokens of a window needs a copy, not a replay
 * ("mlx-bun 0.4.0 -> 1.0.0, qwen3-delta.ts", the recurrent cache's verify
 * round: it restores the pre-round state and replays the first `keep` window
 * tokens, relying on the state after `keep` steps being the same arithmetic
 * prefix whether or not the rest was processed).
 *
 *   snap_steps  HOST array of n_snap step counts, strictly increasing, each
 *               in [0, T]; n_snap in [0, 32].  Count n means "after the first
 *               n steps" (0 = state_in, T = state_out); masked steps count.
 *   snapshots   device f32 [n_snap, B, Hv, Dv, Dk], written (NULL allowed
 *               when n_snap == 0 or B == 0); must not overlap anything else.
 *   g_per_key   0: g is [B, T, Hv] (per-head decay, as gdn_recurrent_masked);
 *               1: g is [B, T, Hv, Dk], the per-key ("vectorized") decay that
 *               the same page names beside the per-head gate it ports:
 *               S[i][j] <- g_t[j] * S[i][j] at the decay step, all else as
 *               gdn_recurrent.
 *
 * The other arguments and rules are those of gdn_recurrent_masked.  The
 * state (state_out and every snapshot) is bit-identical to the state_out of
 * gdn_recurrent_masked run over the same prefix (per-head gate); y agrees
 * within the recurrence tolerance (y may differ in the last bit for T >= 8,
 * where gdn_recurrent stages the steps through a different kernel).
 */
gdn_status gdn_recurrent_snapshots(const gdn_bf16 *q, const gdn_bf16 *k, const gdn_bf16 *v,
                                   const float *g, int g_per_key, const float *beta,
                                   const uint8_t *mask, const float *state_in, float *state_out,
                                   gdn_bf16 *y, const int32_t *snap_steps, int n_snap,
                                   float *snapshots, int B, int T, int Hk, int Hv, int Dk, int Dv,
                                   void *stream);

/*
 * gdn_recurrent_per_key -- the recurrence with the per-key decay gate g
 * [B, T, Hv, Dk] f32 (gdn_recurrent_snapshots with g_per_key = 1 and no
 * snapshots).  Per-step form for every T (for T >= 8 with k, q and the gate
 * rows staged through LDS; the same bits as the snapshot entry point).
 */
gdn_status gdn_recurrent_per_key(const gdn_bf16 *q, const gdn_bf16 *k, const gdn_bf16 *v,
                                 const float *g, const float *beta, const uint8_t *mask,
                                 const float *state_in, float *state_out, gdn_bf16 *y,
                                 int B, int T, int Hk, int Hv, int Dk, int Dv, void *stream);

/*
 * gdn_recurrent_chunked_per_key -- the recurrence with the per-key decay gate
 * of gdn_recurrent_per_key, in the chunked matrix-core form of
 * gdn_recurrent_chunked (the same precision: fp32 state path, y from two
 * bf16 planes before its bf16 rounding).
 * Within a chunk the decay from step s to step t is per key column,
 * g_{s+1}[j] ... g_t[j]; it is formed as running products inside each
 * quarter of the chunk and as a product of two such factors across quarters,
 * never as a quotient of cumulative decays, so any gate values in [0, 1] are
 * safe.
 * Arguments as gdn_recurrent_per_key (mask: 0 = inactive step, y written +0,
 * state untouched; NULL = every step active) plus a caller-owned device
 * workspace of at least gdn_recurrent_chunked_per_key_workspace_bytes(...)
 * bytes (256-byte aligned; not read before written; NULL allowed when that
 * size is 0).  Supported sizes and errors as gdn_recurrent_chunked.
 */
gdn_status gdn_recurrent_chunked_per_key(const gdn_bf16 *q, const gdn_bf16 *k, const gdn_bf16 *v,
                                         const float *g, const float *beta, const uint8_t *mask,
                                         const float *state_in, float *state_out, gdn_bf16 *y,
                                         void *workspace, size_t workspace_bytes,
                                         int B, int T, int Hk, int Hv, int Dk, int Dv, void *stream);

/* Workspace bytes of gdn_recurrent_chunked_per_key (0 for unsupported sizes
 * or B*T == 0). */
size_t gdn_recurrent_chunked_per_key_workspace_bytes(int B, int T, int Hk, int Hv, int Dk, int Dv);

/*
 * gdn_gated_rmsnorm -- output epilogue of the layer: gated RMS normalisation
 * of the recurrence output ("mlex 0.1.2 -- src/models/gated_delta.rs",
 * GatedDeltaNet::forward, the step after the recurrence loop).  Per row of Dv
 * values (one token b, t of one v-head hv), computed in f32:
 *
 *   out[b,t,hv,:] = bf16( silu(z) * y / sqrt(mean(y^2) + eps) * norm_weight )
 *
 * silu(u) = u / (1 + e^-u); the result is rounded to nearest even.
 *
 *   y            [B, T, Hv, Dv] bf16  the recurrence output as stored
 *   z            [B, T, Hv, Dv] bf16  the gate (the layer's z projection)
 *   norm_weight  [Dv] bf16            per-channel weight, shared by all heads
 *   out          [B, T, Hv, Dv] bf16  (= [B, T, Hv*Dv], the layer's output
 *                                      before its output projection)
 *   eps          finite, >= 0 (with eps = 0 an all-zero row gives NaN, as the
 *                formula does; the arithmetic is f32, as on the page, so with
 *                eps = 0 a row whose mean square lies below the f32 normal
 *                range, 2^-126, is outside the stated accuracy)
 *
 * Dv is a multiple of 8 in [8, 4096].  Device pointers, caller-owned, each
 * 16-byte aligned; norm_weight may be NULL only when B*T == 0.  out may be
 * exactly y or exactly z (in place); any other overlap of out with an input is
 * an error.  Only enqueues on `stream`; every check runs before the launch.
 */
gdn_status gdn_gated_rmsnorm(const gdn_bf16 *y, const gdn_bf16 *z, const gdn_bf16 *norm_weight,
                             gdn_bf16 *out, int B, int T, int Hv, int Dv, float eps, void *stream);

/*
 * gdn_layer_core_gated -- gdn_layer_core_masked followed by the output
 * epilogue: the recurrence writes y into `out`, then gdn_gated_rmsnorm turns
 * it, in place, into silu(z)·rms_norm(y)·norm_weight (bit-identical to those
 * two calls).  z and norm_weight are as in gdn_gated_rmsnorm and must not
 * overlap any output (out, state_out, conv_state_out, workspace); norm_eps is
 * the epilogue's eps, eps the prologue's.  Workspace: as gdn_layer_core
 * (gdn_layer_core_workspace_bytes).
 */
gdn_status gdn_layer_core_gated(const gdn_bf16 *qkv, const gdn_bf16 *conv_w,
                                const gdn_bf16 *conv_state_in, gdn_bf16 *conv_state_out,
                                const gdn_bf16 *a, const gdn_bf16 *b,
                                const float *A_log, const float *dt_bias,
                                const gdn_bf16 *z, const gdn_bf16 *norm_weight, const uint8_t *mask,
                                const float *state_in, float *state_out, gdn_bf16 *out,
                                void *workspace, size_t workspace_bytes,
                                int B, int T, int Hk, int Hv, int Dk, int Dv, int K,
                                float q_scale, float k_scale, float eps, float norm_eps,
                                void *stream);

/*
 * gdn_layer_core_no_alloc -- gdn_layer_core_masked with no workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * allocates nothing and frees nothing; its workspace is a device array of
 * GDN_NO_ALLOC_SCRATCH_BYTES that the library holds on each device where it
 * runs, until the process ends.
 *
 * Arguments, results and rules are those of gdn_layer_core_masked (mask may
 * be NULL); the results are bit-identical to that call with a caller
 * workspace.  The caller still owns every input and output.
 *   - Sizes whose workspace (gdn_layer_core_workspace_bytes) exceeds
 *     GDN_NO_ALLOC_SCRATCH_BYTES return GDN_ERR_WORKSPACE before anything
 *     else happens.  At Hk = 16, Hv = 32, Dk = Dv = 128 that is B*T above
 *     about 2900 tokens on the chunked path.
 *   - The first call on a device looks up that device's array (no launch,
 *     no allocation by this library); a call with B == 0 does only that, so
 *     it can be made once before a graph capture starts.
 *   - Every call on a device shares that device's array and leaves its last
 *     contents there (nothing in it needs to start at zero: each call writes
 *     before it reads).  Calls that can overlap in time on one device -- on
 *     different streams without ordering, or from several threads -- race
 *     on the array and give undefined results; serialise them.
 */
#define GDN_NO_ALLOC_SCRATCH_BYTES ((size_t)128 << 20)

gdn_status gdn_layer_core_no_alloc(const gdn_bf16 *qkv, const gdn_bf16 *conv_w,
                                   const gdn_bf16 *conv_state_in, gdn_bf16 *conv_state_out,
                                   const gdn_bf16 *a, const gdn_bf16 *b,
                                   const float *A_log, const float *dt_bias, const uint8_t *mask,
                                   const float *state_in, float *state_out, gdn_bf16 *y,
                                   int B, int T, int Hk, int Hv, int Dk, int Dv, int K,
                                   float q_scale, float k_scale, float eps, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
