/*
 * Gated DeltaNet layer core -- CPU ORACLE (test infrastructure only).
 *
 * This file is the plain, slow, single-threaded fp64 definition that the HIP
 * library is checked against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header, table
 * or helper with the HIP library, and the library never calls it.
 *
 * Sources (the two pages that define the method):
 *   [mlex]  "mlex 0.1.2 -- src/models/gated_delta.rs", GatedDeltaNet::forward
 *           (the op-by-op layer: conv-state splice, depthwise conv1d + SiLU,
 *           q/k/v split, q/k RMS normalisation, GQA repeat, beta, g, and the
 *           per-timestep recurrence loop).
 *   [bun]   "mlx-bun 0.4.0 -> 1.0.0, package/src/model/qwen3-delta.ts"
 *           (the dtype/layout contract in the file header, compute_g, and the
 *           gated_delta_step kernel source, which performs the same per-step
 *           operations in the same order).
 *
 * Everything is computed in double precision from the exact stored input
 * values (bf16 and f32 inputs widen exactly).  No blocking, fusion or
 * reordering beyond the definition: loops follow the pages' order.
 *
 * Readings where the pages leave a step open (each also listed in the design
 * notes of the repository):
 *   - conv weight is [C,K], applied as a cross-correlation (no flip, no bias):
 *     w[c,K-1] multiplies the newest token ([mlex] conv1d call with stride 1,
 *     padding 0, groups = conv_dim over the spliced input).
 *   - RMS normalisation is x / sqrt(mean(x^2) + eps) over the head dimension,
 *     with no weight; q and k are then multiplied by runtime scales q_scale and
 *     k_scale ([mlex] scales q by inv_scale^2 and k by inv_scale; [bun]'s
 *     header describes both as inv_scale * rms_norm, hence runtime scales).
 *   - softplus(x) = log(1 + e^x) evaluated as max(x,0) + log1p(exp(-|x|))
 *     ([bun] compute_g uses logaddexp(x, 0), the same function).
 *   - beta is kept at f32 ([mlex] computes sigmoid in f32).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- formats */

/* Exact widening of a bfloat16 bit pattern (the upper half of an IEEE
 * binary32) to double. */
static double bf16_bits_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bfloat16 value, ties to even, directly from
 * double (no intermediate binary32 rounding).  bfloat16 has the binary32
 * exponent range and 8 significant bits, so the spacing of representable
 * values at magnitude |x| in [2^e, 2^(e+1)) is 2^(e-7), with e clamped to
 * -126 below the normal range (subnormals).  [bun] header: y is stored in the
 * input dtype (bf16). */
uint16_t oracle_f64_to_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    double ax = fabs(x);
    if (isinf(ax))
        return (uint16_t)(sign | 0x7F80u);
    if (ax == 0.0)
        return sign;
    int e2;
    frexp(ax, &e2);          /* ax = m * 2^e2, m in [0.5, 1) */
    int e = e2 - 1;          /* floor(log2(ax)) */
    if (e < -126)
        e = -126;
    double spacing = ldexp(1.0, e - 7);
    /* ax / spacing is exact (power-of-two scaling); nearbyint rounds to the
     * nearest integer with ties to even in the default rounding mode. */
    double r = nearbyint(ax / spacing) * spacing;
    if (r >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)r;      /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFFu));
}

void oracle_round_bf16_array(const double *x, uint16_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = oracle_f64_to_bf16(x[i]);
}

void oracle_bf16_to_f64_array(const uint16_t *h, double *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = bf16_bits_to_f64(h[i]);
}

/* ---------------------------------------------------------- scalar pieces */

/* SiLU: u * sigmoid(u).  [mlex] applies silu to the conv output. */
static double silu(double u)
{
    return u / (1.0 + exp(-u));
}

/* softplus(x) = log(1 + exp(x)) = logaddexp(x, 0).  [bun] compute_g. */
static double softplus(double x)
{
    return fmax(x, 0.0) + log1p(exp(-fabs(x)));
}

/* sigmoid(x) = 1 / (1 + exp(-x)).  [mlex] beta = sigmoid(b). */
static double sigmoid(double x)
{
    return 1.0 / (1.0 + exp(-x));
}

/* --------------------------------------------------- prologue components */

/*
 * RMS normalisation with a scale, per row of D values:
 *   out = x / sqrt(mean(x^2) + eps) * scale
 * [mlex] normalises q and k over the head dimension with no weight and then
 * scales them.
 */
void oracle_rms_scale(const double *x, double *out, long rows, int D,
                      double scale, double eps)
{
    for (long r = 0; r < rows; ++r) {
        const double *xr = x + r * D;
        double ss = 0.0;
        for (long d = 0; d < D; ++d)
            ss += xr[d] * xr[d];
        double rinv = 1.0 / sqrt(ss / (double)D + eps);
        for (long d = 0; d < D; ++d)
            out[r * D + d] = xr[d] * rinv * scale;
    }
}

/*
 * Gate and write strength per (token, v-head) ([mlex] beta and g; [bun]
 * compute_g):
 *   g    = exp(-exp(A_log[h]) * softplus(a + dt_bias[h]))
 *   beta = sigmoid(b)
 * a, b: [BT, Hv] bf16 bits; A_log, dt_bias: [Hv] f32; g, beta: [BT, Hv].
 */
void oracle_gates(const uint16_t *a, const uint16_t *b, const float *A_log,
                  const float *dt_bias, double *g, double *beta, long BT, int Hv)
{
    for (long r = 0; r < BT; ++r) {
        for (long h = 0; h < Hv; ++h) {
            long i = r * Hv + h;
            double x = bf16_bits_to_f64(a[i]) + (double)dt_bias[h];
            g[i] = exp(-exp((double)A_log[h]) * softplus(x));
            beta[i] = sigmoid(bf16_bits_to_f64(b[i]));
        }
    }
}

/* ------------------------------------------------------------------ prep */

/*
 * Prologue of the layer core ([mlex] GatedDeltaNet::forward, from the conv
 * state splice through g; [bun] compute_g).
 *
 * Inputs (row-major, exact stored values):
 *   qkv           [B,T,C] bf16 bits, C = 2*Hk*Dk + Hv*Dv (mixed q|k|v)
 *   conv_w        [C,K]   bf16 bits
 *   conv_state_in [B,K-1,C] bf16 bits, or NULL for zeros
 *   a, b          [B,T,Hv] bf16 bits
 *   A_log, dt_bias [Hv] f32
 * Outputs (double, unrounded):
 *   q_out, k_out  [B,T,Hk,Dk]     v_out [B,T,Hv,Dv]
 *   g_out, beta_out [B,T,Hv]
 *   conv_state_out [B,K-1,C] bf16 bits (exact copies of the last K-1 rows of
 *                  the spliced input), or NULL to skip.
 * Returns 0, or -1 on bad sizes / allocation failure.
 */
int oracle_prep(const uint16_t *qkv, const uint16_t *conv_w,
                const uint16_t *conv_state_in, uint16_t *conv_state_out,
                const uint16_t *a, const uint16_t *b,
                const float *A_log, const float *dt_bias,
                double *q_out, double *k_out, double *v_out,
                double *g_out, double *beta_out,
                int B, int T, int Hk, int Hv, int Dk, int Dv, int K,
                double q_scale, double k_scale, double eps)
{
    if (B < 0 || T < 0 || Hk < 1 || Hv < 1 || Dk < 1 || Dv < 1 || K < 1)
        return -1;
    const long C = 2L * Hk * Dk + (long)Hv * Dv;
    const long P = (long)T + K - 1; /* rows of the spliced input */
    double *xpad = (double *)malloc(sizeof(double) * (size_t)(P > 0 ? P : 1) * (size_t)C);
    double *act = (double *)malloc(sizeof(double) * (size_t)C);
    if (!xpad || !act) {
        free(xpad);
        free(act);
        return -1;
    }

    for (int bb = 0; bb < B; ++bb) {
        /* conv-state splice: xpad = [conv_state_in (or zeros) ; qkv[b]] along T */
        for (long p = 0; p < P; ++p) {
            for (long c = 0; c < C; ++c) {
                double x;
                if (p < K - 1)
                    x = conv_state_in
                            ? bf16_bits_to_f64(conv_state_in[((long)bb * (K - 1) + p) * C + c])
                            : 0.0;
                else
                    x = bf16_bits_to_f64(qkv[((long)bb * T + (p - (K - 1))) * C + c]);
                xpad[p * C + c] = x;
            }
        }
        /* the new conv state is the last K-1 rows of the spliced input */
        if (conv_state_out) {
            for (long i = 0; i < K - 1; ++i)
                for (long c = 0; c < C; ++c)
                    conv_state_out[((long)bb * (K - 1) + i) * C + c] =
                        oracle_f64_to_bf16(xpad[((long)T + i) * C + c]);
        }

        for (long t = 0; t < T; ++t) {
            /* depthwise causal conv1d (cross-correlation) followed by SiLU */
            for (long c = 0; c < C; ++c) {
                double u = 0.0;
                for (long j = 0; j < K; ++j)
                    u += bf16_bits_to_f64(conv_w[c * K + j]) * xpad[(t + j) * C + c];
                act[c] = silu(u);
            }
            /* split: q = [0, Hk*Dk), k = [Hk*Dk, 2*Hk*Dk), v = rest; q and k
             * are RMS-normalised per head and scaled, v passes through */
            oracle_rms_scale(act, q_out + ((long)bb * T + t) * Hk * Dk, Hk, Dk, q_scale, eps);
            oracle_rms_scale(act + (long)Hk * Dk, k_out + ((long)bb * T + t) * Hk * Dk,
                             Hk, Dk, k_scale, eps);
            for (long c = 0; c < (long)Hv * Dv; ++c)
                v_out[((long)bb * T + t) * Hv * Dv + c] = act[2L * Hk * Dk + c];
        }
    }
    /* write strength and gate, per (token, v-head) */
    oracle_gates(a, b, A_log, dt_bias, g_out, beta_out, (long)B * T, Hv);
    free(xpad);
    free(act);
    return 0;
}

/* ------------------------------------------------------------ recurrence */

/*
 * Gated delta rule ([mlex] GatedDeltaNet::forward recurrence loop; [bun]
 * gated_delta_step performs the same operations in the same order).
 *
 * For every batch row b and v-head hv (k-head hk = hv / (Hv/Hk), the repeat
 * order of the pages' GQA mapping) and every t = 0..T-1:
 *   S <- g_t * S                       (decay)
 *   kv_i = sum_j S[i,j] k_t[j]          (read-out with the decayed state)
 *   delta_i = (v_t[i] - kv_i) * beta_t
 *   S[i,j] <- S[i,j] + delta_i k_t[j]   (rank-1 update)
 *   y_t[i] = sum_j S[i,j] q_t[j]         (output with the updated state)
 *
 * Masked steps ([bun] qwen3-delta.ts, the masked variant of the step
 * kernel, selected for padded prefill): mask [B,T] (NULL = every step
 * active); a step whose mask byte is 0 leaves S untouched (no decay, no
 * update) and writes y_t = 0.
 *
 * Per-key decay (the "vectorized" gate, g of shape [B,T,Hv,Dk], that
 * [bun] names beside the per-head gate it ports): the decay step scales each
 * state column by its own factor, S[i,j] <- g_t[j] * S[i,j]; every other
 * step is unchanged.  g_per_key selects this form.
 *
 * Layouts: q,k [B,T,Hk,Dk]; v,y [B,T,Hv,Dv]; g,beta [B,T,Hv] (g [B,T,Hv,Dk]
 * with g_per_key); state_in/state_out [B,Hv,Dv,Dk] (state_in NULL = zeros;
 * may alias out).  All double.  Returns 0, or -1 on bad sizes / allocation
 * failure.
 */
static int recurrence(const double *q, const double *k, const double *v,
                      const double *g, int g_per_key, const double *beta,
                      const unsigned char *mask, const double *state_in, double *state_out,
                      double *y, int B, int T, int Hk, int Hv, int Dk, int Dv)
{
    if (B < 0 || T < 0 || Hk < 1 || Hv < 1 || Dk < 1 || Dv < 1 || Hv % Hk != 0)
        return -1;
    const int rep = Hv / Hk;
    double *S = (double *)malloc(sizeof(double) * (size_t)Dv * (size_t)Dk);
    double *kv = (double *)malloc(sizeof(double) * (size_t)Dv);
    double *delta = (double *)malloc(sizeof(double) * (size_t)Dv);
    if (!S || !kv || !delta) {
        free(S);
        free(kv);
        free(delta);
        return -1;
    }
    for (long bb = 0; bb < B; ++bb) {
        for (long hv = 0; hv < Hv; ++hv) {
            const long hk = hv / rep;
            const long base = (bb * Hv + hv) * (long)Dv * Dk;
            for (long i = 0; i < (long)Dv * Dk; ++i)
                S[i] = state_in ? state_in[base + i] : 0.0;
            for (long t = 0; t < T; ++t) {
                const double *kt = k + ((bb * T + t) * Hk + hk) * Dk;
                const double *qt = q + ((bb * T + t) * Hk + hk) * Dk;
                const double *vt = v + ((bb * T + t) * Hv + hv) * Dv;
                const double *gt = g_per_key ? g + ((bb * T + t) * Hv + hv) * Dk
                                             : g + (bb * T + t) * Hv + hv;
                const double bt = beta[(bb * T + t) * Hv + hv];
                double *yt = y + ((bb * T + t) * Hv + hv) * Dv;
                if (mask && !mask[bb * T + t]) {
                    for (long i = 0; i < Dv; ++i)
                        yt[i] = 0.0;
                    continue;
                }
                for (long i = 0; i < Dv; ++i)
                    for (long j = 0; j < Dk; ++j)
                        S[i * Dk + j] = S[i * Dk + j] * (g_per_key ? gt[j] : gt[0]);
                for (long i = 0; i < Dv; ++i) {
                    double acc = 0.0;
                    for (long j = 0; j < Dk; ++j)
                        acc += S[i * Dk + j] * kt[j];
                    kv[i] = acc;
                }
                for (long i = 0; i < Dv; ++i)
                    delta[i] = (vt[i] - kv[i]) * bt;
                for (long i = 0; i < Dv; ++i)
                    for (long j = 0; j < Dk; ++j)
                        S[i * Dk + j] = S[i * Dk + j] + delta[i] * kt[j];
                for (long i = 0; i < Dv; ++i) {
                    double acc = 0.0;
                    for (long j = 0; j < Dk; ++j)
                        acc += S[i * Dk + j] * qt[j];
                    yt[i] = acc;
                }
            }
            for (long i = 0; i < (long)Dv * Dk; ++i)
                state_out[base + i] = S[i];
        }
    }
    free(S);
    free(kv);
    free(delta);
    return 0;
}

/* The recurrence with the per-head gate g [B,T,Hv]. */
int oracle_recurrent(const double *q, const double *k, const double *v,
                     const double *g, const double *beta, const unsigned char *mask,
                     const double *state_in, double *state_out, double *y,
                     int B, int T, int Hk, int Hv, int Dk, int Dv)
{
    return recurrence(q, k, v, g, 0, beta, mask, state_in, state_out, y, B, T, Hk, Hv, Dk, Dv);
}

/* The recurrence with the per-key gate g [B,T,Hv,Dk]. */
int oracle_recurrent_per_key(const double *q, const double *k, const double *v,
                             const double *g, const double *beta, const unsigned char *mask,
                             const double *state_in, double *state_out, double *y,
                             int B, int T, int Hk, int Hv, int Dk, int Dv)
{
    return recurrence(q, k, v, g, 1, beta, mask, state_in, state_out, y, B, T, Hk, Hv, Dk, Dv);
}

/* ------------------------------------------------------------ layer core */

/*
 * Prologue then recurrence, with the stored-dtype roundings of the pages'
 * contract in between ([bun] header: q, k, v are bf16 and g is f32 when they
 * reach the recurrence; beta kept at f32 as [mlex] computes it):
 *   q, k, v  -> bf16 (round to nearest, ties to even)
 *   g, beta  -> f32  (C conversion, round to nearest even)
 * y_out is the recurrence output in double (callers round to bf16 for
 * storage); state_out is double.  mask [B,T] (NULL = all active) masks
 * recurrence steps only, as in the pages (the conv runs over every token).
 */
int oracle_layer_core(const uint16_t *qkv, const uint16_t *conv_w,
                      const uint16_t *conv_state_in, uint16_t *conv_state_out,
                      const uint16_t *a, const uint16_t *b,
                      const float *A_log, const float *dt_bias, const unsigned char *mask,
                      const double *state_in, double *state_out, double *y_out,
                      int B, int T, int Hk, int Hv, int Dk, int Dv, int K,
                      double q_scale, double k_scale, double eps)
{
    if (B < 0 || T < 0 || Hk < 1 || Hv < 1 || Dk < 1 || Dv < 1 || K < 1 || Hv % Hk != 0)
        return -1;
    const size_t nq = (size_t)B * T * Hk * Dk, nv = (size_t)B * T * Hv * Dv;
    const size_t ng = (size_t)B * T * Hv;
    double *q = (double *)malloc(sizeof(double) * (nq ? nq : 1));
    double *k = (double *)malloc(sizeof(double) * (nq ? nq : 1));
    double *v = (double *)malloc(sizeof(double) * (nv ? nv : 1));
    double *g = (double *)malloc(sizeof(double) * (ng ? ng : 1));
    double *be = (double *)malloc(sizeof(double) * (ng ? ng : 1));
    int rc = -1;
    if (!q || !k || !v || !g || !be)
        goto done;
    if (oracle_prep(qkv, conv_w, conv_state_in, conv_state_out, a, b, A_log, dt_bias,
                    q, k, v, g, be, B, T, Hk, Hv, Dk, Dv, K, q_scale, k_scale, eps) != 0)
        goto done;
    for (size_t i = 0; i < nq; ++i) {
        q[i] = bf16_bits_to_f64(oracle_f64_to_bf16(q[i]));
        k[i] = bf16_bits_to_f64(oracle_f64_to_bf16(k[i]));
    }
    for (size_t i = 0; i < nv; ++i)
        v[i] = bf16_bits_to_f64(oracle_f64_to_bf16(v[i]));
    for (size_t i = 0; i < ng; ++i) {
        g[i] = (double)(float)g[i];
        be[i] = (double)(float)be[i];
    }
    rc = oracle_recurrent(q, k, v, g, be, mask, state_in, state_out, y_out, B, T, Hk, Hv, Dk, Dv);
done:
    free(q);
    free(k);
    free(v);
    free(g);
    free(be);
    return rc;
}

/* ------------------------------------------------------- output epilogue */

/*
 * Gated RMS normalisation of the recurrence output ([mlex]
 * GatedDeltaNet::forward, the step after the recurrence loop): the stored
 * bf16 y is widened, each row of Dv values (one token of one v-head) is
 * normalised with no weight inside the norm, scaled by the per-channel
 * norm_weight (shared by all heads), and gated by silu(z):
 *   out[r][d] = silu(z[r][d]) * (y[r][d] / sqrt(mean_d y[r][d]^2 + eps) * w[d])
 * y, z are [rows, Dv] bf16, w is [Dv] bf16; out is double (callers round to
 * bf16 for storage, as the page casts the f32 result to the input dtype).
 */
int oracle_gated_rmsnorm(const uint16_t *y, const uint16_t *z, const uint16_t *w,
                         double *out, long rows, int Dv, double eps)
{
    if (rows < 0 || Dv < 1)
        return -1;
    for (long r = 0; r < rows; ++r) {
        const uint16_t *yr = y + r * Dv, *zr = z + r * Dv;
        double ss = 0.0;
        for (int d = 0; d < Dv; ++d) {
            double u = bf16_bits_to_f64(yr[d]);
            ss += u * u;
        }
        double rinv = 1.0 / sqrt(ss / (double)Dv + eps);
        for (int d = 0; d < Dv; ++d) {
            double normed = bf16_bits_to_f64(yr[d]) * rinv * bf16_bits_to_f64(w[d]);
            out[r * Dv + d] = silu(bf16_bits_to_f64(zr[d])) * normed;
        }
    }
    return 0;
}
