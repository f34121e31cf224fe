/*
 * attn_oracle.c -- plain fp64 CPU oracle of the learned-relative grouped-query
 * attention forward with per-query sinks.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (pages cited by title and API entry):
 *
 *  - "nemo_automodel.components.models.inkling2.flex_attention", class
 *    Inkling2FlexAttention: the logit scale is head_dim^-0.5; forward combines
 *    content attention with a learned relative term and a sink; relative
 *    profiles are laid out [batch, heads, sequence, relative_extent] and no
 *    sequence-by-sequence bias is ever formed; the result is FP32
 *    [batch, sequence, heads, head_dim].  Parameter list of forward: q
 *    [B,S,Hq,D], k/v [B,Sk,Hkv,D], profiles [B,Hq,S,E], sink [B,S,Hq], valid
 *    [B,S], key_valid [B,Sk], positions [B,S] (logical, restarting at every
 *    document), key_positions [B,Sk], query_offset (global column of the first
 *    local query).
 *  - "nemo_automodel.components.models.inkling2.attention" (v0.4),
 *    Inkling2Attention.forward: the sink carries no value (a virtual sink whose
 *    value is zero); Inkling2Attention._eager: a quadratic reference exists and
 *    leaves its inputs untouched.
 *  - "nemo_automodel.components.attention.flex_attention", sliding-window
 *    mask mod and forward's sliding_window / enable_gqa parameters.
 *
 * Readings taken where the pages leave a step open (each is stated again in
 * the repository's design notes):
 *  - document membership: query i (global column gi = query_offset + i) and
 *    key j are in the same document iff gi - positions[i] == j - key_positions[j]
 *    (both sides name the column where the document starts);
 *  - causal order on global columns: j <= gi;
 *  - window W > 0 keeps keys whose logical distance r = positions[i] -
 *    key_positions[j] satisfies r < W (W keys including the query itself);
 *    W <= 0 means no window;
 *  - relative bias = profiles[b,h,i,r] for 0 <= r < E, and 0 otherwise;
 *  - the bias is added unscaled: z = scale * <q,k> + bias;
 *  - GQA: query head h reads key/value head h / (Hq/Hkv);
 *  - the sink sigma = sink[b,i,h] is one more logit in the softmax
 *    denominator, with a zero value vector;
 *  - lse = ln(exp(sigma) + sum_j exp(z_j)) (natural log, sink included);
 *  - a row with no allowed key: out = 0 and lse = sigma.
 *
 * Precision: every input element is converted exactly to double (bf16 by
 * placing its 16 bits in the top half of an IEEE single; fp32 by promotion),
 * and every sum, exponential and logarithm is taken in double in plain
 * sequential order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact conversion of a bf16 bit pattern to double. */
static double bf16_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* profiles_dtype: 0 fp32, 1 bf16, 2 fp64 (profiles formed by attn_oracle_relproj_profiles) */
static double profile_at(const void* profiles, int profiles_dtype, size_t idx)
{
    if (profiles_dtype == 1)
        return bf16_to_double(((const uint16_t*)profiles)[idx]);
    if (profiles_dtype == 2)
        return ((const double*)profiles)[idx];
    return (double)((const float*)profiles)[idx];
}

/*
 * Is key j visible from query i of batch row b?  Plain statement of the mask:
 * both tokens real, key not after the query, same document, inside the window.
 */
static int allowed(const uint8_t* valid, const uint8_t* key_valid,
                   const int32_t* positions, const int32_t* key_positions,
                   int64_t window, int64_t query_offset,
                   int Sq, int Sk, int b, int i, int j)
{
    int64_t gi = query_offset + i;
    int64_t p_i = positions[(size_t)b * Sq + i];
    int64_t k_j = key_positions[(size_t)b * Sk + j];
    if (!valid[(size_t)b * Sq + i]) return 0;
    if (!key_valid[(size_t)b * Sk + j]) return 0;
    if ((int64_t)j > gi) return 0;                       /* causal */
    if (gi - p_i != (int64_t)j - k_j) return 0;         /* same document */
    if (window > 0 && !(p_i - k_j < window)) return 0;  /* sliding window */
    return 1;
}

/*
 * Forward for the query rows listed in `rows` (flattened b*Sq + i); all rows
 * when rows == NULL (then n_rows must be B*Sq).  Outputs are compact over the
 * listed rows: out[n_rows, Hq, D], lse[n_rows, Hq], n_allowed[n_rows].
 *
 * q, k, v: bf16 bit patterns.  profiles: fp32, bf16 or fp64 (profiles_is_bf16 = 0, 1, 2).
 * Every pointer is a host pointer; nothing is allocated beyond one logit buffer
 * of Sk doubles per thread.  Returns 0, or -1 on bad arguments / no memory.
 */
int attn_oracle_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const void* profiles, int profiles_is_bf16,
                    const float* sink, const uint8_t* valid, const uint8_t* key_valid,
                    const int32_t* positions, const int32_t* key_positions,
                    int64_t window, int64_t query_offset,
                    int B, int Sq, int Sk, int Hq, int Hkv, int D, int E,
                    const int64_t* rows, int64_t n_rows,
                    double* out, double* lse, int32_t* n_allowed, int n_threads)
{
    if (!q || !k || !v || !profiles || !sink || !valid || !key_valid || !positions ||
        !key_positions || !out || !lse || !n_allowed)
        return -1;
    if (B < 0 || Sq < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || E <= 0 || Hq % Hkv)
        return -1;
    if (!rows && n_rows != (int64_t)B * Sq) return -1;
    const int G = Hq / Hkv;
    const double scale = 1.0 / sqrt((double)D);
    int failed = 0;

#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif

#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        uint8_t* ok = (uint8_t*)malloc((size_t)(Sk > 0 ? Sk : 1));
        if (!z || !ok) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n_rows; ++t) {
            if (!z || !ok) continue;
            int64_t row = rows ? rows[t] : t;
            int b = (int)(row / Sq), i = (int)(row % Sq);
            int count = 0;
            for (int j = 0; j < Sk; ++j) {
                ok[j] = (uint8_t)allowed(valid, key_valid, positions, key_positions,
                                         window, query_offset, Sq, Sk, b, i, j);
                count += ok[j];
            }
            n_allowed[t] = count;
            for (int h = 0; h < Hq; ++h) {
                int g = h / G;
                double sigma = (double)sink[((size_t)b * Sq + i) * Hq + h];
                double* o = out + ((size_t)t * Hq + h) * D;
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                if (count == 0) {
                    lse[(size_t)t * Hq + h] = sigma;
                    continue;
                }
                const uint16_t* qrow = q + (((size_t)b * Sq + i) * Hq + h) * D;
                int64_t p_i = positions[(size_t)b * Sq + i];
                /* pass 1: logits of the allowed keys and their maximum */
                double M = sigma;
                for (int j = 0; j < Sk; ++j) {
                    if (!ok[j]) continue;
                    const uint16_t* krow = k + (((size_t)b * Sk + j) * Hkv + g) * D;
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += bf16_to_double(qrow[d]) * bf16_to_double(krow[d]);
                    int64_t r = p_i - (int64_t)key_positions[(size_t)b * Sk + j];
                    double bias = 0.0;
                    if (r >= 0 && r < E)
                        bias = profile_at(profiles, profiles_is_bf16,
                                          (((size_t)b * Hq + h) * Sq + i) * (size_t)E + (size_t)r);
                    z[j] = scale * dot + bias;
                    if (z[j] > M) M = z[j];
                }
                /* pass 2: normaliser (sink included) and value accumulation */
                double L = exp(sigma - M);
                for (int j = 0; j < Sk; ++j) {
                    if (!ok[j]) continue;
                    double p = exp(z[j] - M);
                    L += p;
                    const uint16_t* vrow = v + (((size_t)b * Sk + j) * Hkv + g) * D;
                    for (int d = 0; d < D; ++d) o[d] += p * bf16_to_double(vrow[d]);
                }
                for (int d = 0; d < D; ++d) o[d] /= L;
                lse[(size_t)t * Hq + h] = M + log(L);
            }
        }
        free(z);
        free(ok);
    }
    return failed ? -1 : 0;
}

/*
 * Generic flex-attention forward without the relative term (page
 * "nemo_automodel.components.attention.flex_attention": FlexAttention and its
 * forward).  Layouts are head-major as on that page: q [B,Hq,Sq,D], k / v
 * [B,Hkv,Sk,D] (bf16 bit patterns), sink_weights [Hq] (or NULL), tokens
 * [B,Sq] (or NULL).  Readings (stated in the repository's design notes):
 *  - "causal": key j visible from query i iff j <= i;
 *  - "block_causal": additionally i and j in the same block, where a block
 *    ends with (and includes) a token equal to eos_id: block(t) = number of
 *    eos tokens strictly before t;
 *  - fixed_block_size F > 0: additionally i / F == j / F;
 *  - sliding_window W > 0: additionally i - j < W (W tokens including i);
 *  - the given scale (> 0) applies only when there are no sink weights;
 *    otherwise the scale is head_dim^-0.5;
 *  - sink_weights[h]: one more logit in the softmax denominator, zero value.
 * Outputs for the listed rows (flattened b*Sq + i, all when rows == NULL):
 * out[n_rows, Hq, D], lse[n_rows, Hq] (-inf for an empty row without sink),
 * n_allowed[n_rows].
 */
static int64_t eos_block(const int32_t* tokens, int32_t eos_id, int Sq, int b, int t)
{
    int64_t n = 0;
    for (int u = 0; u < t; ++u)
        if (tokens[(size_t)b * Sq + u] == eos_id) ++n;
    return n;
}

int flex_oracle_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const float* sink_weights, const int32_t* tokens, int32_t eos_id,
                    int64_t fixed_block_size, int64_t window, double scale_arg,
                    int B, int Sq, int Sk, int Hq, int Hkv, int D,
                    const int64_t* rows, int64_t n_rows,
                    double* out, double* lse, int32_t* n_allowed, int n_threads)
{
    if (!q || !k || !v || !out || !lse || !n_allowed) return -1;
    if (B < 0 || Sq < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv) return -1;
    if ((tokens || fixed_block_size > 0) && Sq != Sk) return -1;
    if (!rows && n_rows != (int64_t)B * Sq) return -1;
    const int G = Hq / Hkv;
    const double scale = (!sink_weights && scale_arg > 0.0) ? scale_arg : 1.0 / sqrt((double)D);
    int failed = 0;

#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif

#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        uint8_t* ok = (uint8_t*)malloc((size_t)(Sk > 0 ? Sk : 1));
        if (!z || !ok) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n_rows; ++t) {
            if (!z || !ok) continue;
            int64_t row = rows ? rows[t] : t;
            int b = (int)(row / Sq), i = (int)(row % Sq);
            int64_t blk_i = tokens ? eos_block(tokens, eos_id, Sq, b, i) : 0;
            int count = 0;
            for (int j = 0; j < Sk; ++j) {
                int visible = j <= i;
                if (visible && tokens) visible = eos_block(tokens, eos_id, Sq, b, j) == blk_i;
                if (visible && fixed_block_size > 0) visible = (i / fixed_block_size) == (j / fixed_block_size);
                if (visible && window > 0) visible = (int64_t)i - j < window;
                ok[j] = (uint8_t)visible;
                count += visible;
            }
            n_allowed[t] = count;
            for (int h = 0; h < Hq; ++h) {
                int g = h / G;
                double sigma = sink_weights ? (double)sink_weights[h] : -INFINITY;
                double* o = out + ((size_t)t * Hq + h) * D;
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                if (count == 0) {
                    lse[(size_t)t * Hq + h] = sigma;
                    continue;
                }
                const uint16_t* qrow = q + (((size_t)b * Hq + h) * Sq + i) * D;
                double M = sigma;
                for (int j = 0; j < Sk; ++j) {
                    if (!ok[j]) continue;
                    const uint16_t* krow = k + (((size_t)b * Hkv + g) * Sk + j) * D;
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += bf16_to_double(qrow[d]) * bf16_to_double(krow[d]);
                    z[j] = scale * dot;
                    if (z[j] > M) M = z[j];
                }
                double L = sink_weights ? exp(sigma - M) : 0.0;
                for (int j = 0; j < Sk; ++j) {
                    if (!ok[j]) continue;
                    double p = exp(z[j] - M);
                    L += p;
                    const uint16_t* vrow = v + (((size_t)b * Hkv + g) * Sk + j) * D;
                    for (int d = 0; d < D; ++d) o[d] += p * bf16_to_double(vrow[d]);
                }
                for (int d = 0; d < D; ++d) o[d] /= L;
                lse[(size_t)t * Hq + h] = M + log(L);
            }
        }
        free(z);
        free(ok);
    }
    return failed ? -1 : 0;
}

/*
 * Gradients of the forward above.  The page "nemo_automodel.components.models.
 * inkling2.flex_attention" (module summary and class Inkling2FlexAttention)
 * makes the per-query sinks differentiable and lets gradients reach the
 * profiles and flow in through the returned log-sum-exp; q, k and v are the
 * ordinary attention inputs.  The gradients are the plain derivatives of the
 * forward's definition (chain rule through the sink-augmented softmax).  For a loss with
 * dL/dout = dout [B,Sq,Hq,D] and dL/dlse = dlse [B,Sq,Hq] (dlse may be NULL:
 * zero), per row (b, i, h) with P_j = e^{z_j - lse}, p_s = e^{sigma - lse}:
 *   Delta  = <dout, out>
 *   dz_j   = P_j (<dout, v_j> - Delta + dlse)          (allowed j)
 *   dq     = scale * sum_j dz_j k_j;   dk_j += scale * dz_j q;   dv_j += P_j dout
 *   dprofiles[b,h,i,r] = dz_j for the allowed j at distance r in [0, E), else 0
 *   dsink  = p_s (dlse - Delta)
 * out / lse are recomputed here in fp64.  Outputs: dq [B,Sq,Hq,D],
 * dk / dv [B,Sk,Hkv,D], dprofiles [B,Hq,Sq,E], dsink [B,Sq,Hq], all fp64.
 *
 * Only the query rows row_lo <= i < row_hi take part (row_hi <= 0 or above
 * Sq means Sq); the others' outputs stay 0.  dq / dprofiles / dsink of the
 * rows taken are those of the whole computation, and dk / dv are exact for
 * the keys that no row outside the range can see (under the causal order
 * with row_hi = Sq: keys j >= query_offset + row_lo; with a window w as well:
 * keys j with j + w - 1 < query_offset + row_hi, when row_hi < Sq).
 *
 * The work is spread over threads by (batch row, K/V head): each thread owns
 * the dk / dv rows of its head group, and every output element sums its
 * terms in the same order (rows ascending, then the group's heads) whatever
 * the thread count.  n_threads <= 0 leaves OpenMP's default.
 *
 * magnitudes != 0 returns, in the same arrays, each output's sum of absolute
 * contributions instead (every product and difference above taken in
 * absolute value: |dout . v| -> sum |dout_d v_d|, Delta -> sum |dout_d out_d|,
 * dlse -> |dlse|).  Tests scale their rounding tolerance by it.
 */
int attn_oracle_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const void* profiles, int profiles_is_bf16,
                    const float* sink, const uint8_t* valid, const uint8_t* key_valid,
                    const int32_t* positions, const int32_t* key_positions,
                    int64_t window, int64_t query_offset,
                    int B, int Sq, int Sk, int Hq, int Hkv, int D, int E,
                    const double* dout, const double* dlse, int row_lo, int row_hi, int magnitudes,
                    double* dq, double* dk, double* dv, double* dprofiles, double* dsink, int n_threads)
{
    if (!q || !k || !v || !profiles || !sink || !valid || !key_valid || !positions || !key_positions ||
        !dout || !dq || !dk || !dv || !dprofiles || !dsink)
        return -1;
    if (B < 0 || Sq < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || E <= 0 || Hq % Hkv) return -1;
    const int G = Hq / Hkv;
    const double scale = 1.0 / sqrt((double)D);
    memset(dq, 0, sizeof(double) * (size_t)B * Sq * Hq * D);
    memset(dk, 0, sizeof(double) * (size_t)B * Sk * Hkv * D);
    memset(dv, 0, sizeof(double) * (size_t)B * Sk * Hkv * D);
    memset(dprofiles, 0, sizeof(double) * (size_t)B * Hq * Sq * E);
    memset(dsink, 0, sizeof(double) * (size_t)B * Sq * Hq);
    const int i_lo = row_lo > 0 ? row_lo : 0;
    const int i_hi = (row_hi <= 0 || row_hi > Sq) ? Sq : row_hi;
    int failed = 0;

#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif

#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        double* o = (double*)malloc(sizeof(double) * (size_t)D);
        uint8_t* ok = (uint8_t*)malloc((size_t)(Sk > 0 ? Sk : 1));
        if (!z || !o || !ok) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int bg = 0; bg < B * Hkv; ++bg) {
            if (!z || !o || !ok) continue;
            const int b = bg / Hkv, g = bg % Hkv;
            for (int i = i_lo; i < i_hi; ++i) {
                int count = 0;
                for (int j = 0; j < Sk; ++j) {
                    ok[j] = (uint8_t)allowed(valid, key_valid, positions, key_positions, window, query_offset,
                                             Sq, Sk, b, i, j);
                    count += ok[j];
                }
                int64_t p_i = positions[(size_t)b * Sq + i];
                for (int h = g * G; h < (g + 1) * G; ++h) {
                    size_t row = ((size_t)b * Sq + i) * Hq + h;
                    double sigma = (double)sink[row];
                    double dl = dlse ? dlse[row] : 0.0;
                    const double* dov = dout + row * D;
                    if (count == 0) {                  /* lse = sigma, out = 0: only the sink moves lse */
                        dsink[row] = isinf(sigma) && sigma < 0 ? 0.0 : (magnitudes ? fabs(dl) : dl);
                        continue;
                    }
                    const uint16_t* qrow = q + row * D;
                    double M = sigma;
                    for (int j = 0; j < Sk; ++j) {
                        if (!ok[j]) continue;
                        const uint16_t* krow = k + (((size_t)b * Sk + j) * Hkv + g) * D;
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d) dot += bf16_to_double(qrow[d]) * bf16_to_double(krow[d]);
                        int64_t r = p_i - (int64_t)key_positions[(size_t)b * Sk + j];
                        double bias = 0.0;
                        if (r >= 0 && r < E)
                            bias = profile_at(profiles, profiles_is_bf16, (((size_t)b * Hq + h) * Sq + i) * (size_t)E + r);
                        z[j] = scale * dot + bias;
                        if (z[j] > M) M = z[j];
                    }
                    double L = exp(sigma - M);
                    for (int d = 0; d < D; ++d) o[d] = 0.0;
                    for (int j = 0; j < Sk; ++j) {
                        if (!ok[j]) continue;
                        double pj = exp(z[j] - M);
                        L += pj;
                        const uint16_t* vrow = v + (((size_t)b * Sk + j) * Hkv + g) * D;
                        for (int d = 0; d < D; ++d) o[d] += pj * bf16_to_double(vrow[d]);
                    }
                    double lse = M + log(L);
                    double delta = 0.0;
                    for (int d = 0; d < D; ++d)
                        delta += magnitudes ? fabs(dov[d] * (o[d] / L)) : dov[d] * (o[d] / L);
                    dsink[row] = magnitudes ? exp(sigma - lse) * (fabs(dl) + delta) : exp(sigma - lse) * (dl - delta);
                    for (int j = 0; j < Sk; ++j) {
                        if (!ok[j]) continue;
                        double pj = exp(z[j] - lse);
                        const uint16_t* krow = k + (((size_t)b * Sk + j) * Hkv + g) * D;
                        const uint16_t* vrow = v + (((size_t)b * Sk + j) * Hkv + g) * D;
                        double dp = 0.0;
                        for (int d = 0; d < D; ++d)
                            dp += magnitudes ? fabs(dov[d] * bf16_to_double(vrow[d])) : dov[d] * bf16_to_double(vrow[d]);
                        double dz = magnitudes ? pj * (dp + delta + fabs(dl)) : pj * (dp - delta + dl);
                        double* dkr = dk + (((size_t)b * Sk + j) * Hkv + g) * D;
                        double* dvr = dv + (((size_t)b * Sk + j) * Hkv + g) * D;
                        double* dqr = dq + row * D;
                        for (int d = 0; d < D; ++d) {
                            double kd = bf16_to_double(krow[d]), qd = bf16_to_double(qrow[d]), od = dov[d];
                            if (magnitudes) {
                                kd = fabs(kd);
                                qd = fabs(qd);
                                od = fabs(od);
                            }
                            dqr[d] += scale * dz * kd;
                            dkr[d] += scale * dz * qd;
                            dvr[d] += pj * od;
                        }
                        int64_t r = p_i - (int64_t)key_positions[(size_t)b * Sk + j];
                        if (r >= 0 && r < E) dprofiles[(((size_t)b * Hq + h) * Sq + i) * (size_t)E + r] = dz;
                    }
                }
            }
        }
        free(z); free(o); free(ok);
    }
    return failed ? -1 : 0;
}

/*
 * Relative logits from relative features (reading of the page
 * "nemo_automodel.components.models.inkling2.attention", v0.4: class
 * Inkling2Attention, attributes qkvr (the fused projection that also yields
 * relative features), d_rel (their width), relative_table and rel_extent;
 * and of the page "nemo_automodel.components.models.inkling2.flex_attention",
 * forward parameter profiles: relative logits of shape [batch, heads,
 * sequence, relative_extent] that keep the projection's rounding boundary).
 * The pages give no formula; the reading taken:
 *
 *   profiles[b,h,i,r] = sum_c rfeat[b,i,h,c] * table[t,r,c],  0 <= r < E,
 *
 * rfeat [B,Sq,Hq,d_rel] and table [T,E,d_rel] bf16 bit patterns, t = h when the
 * table has one slice per head (T = Hq), t = 0 when it is shared (T = 1).
 * Every product of two bf16 values is exact in double; the d_rel products
 * are summed in plain sequential order in double and the result is written
 * unrounded: profiles [B,Hq,Sq,E] fp64.  Returns 0, or -1 on bad arguments.
 */
int attn_oracle_relproj_profiles(const uint16_t* rfeat, const uint16_t* table, int table_heads,
                                 int B, int Sq, int Hq, int d_rel, int E, double* profiles)
{
    if (!rfeat || !table || !profiles || B < 0 || Sq < 0 || Hq <= 0 || d_rel <= 0 || E <= 0) return -1;
    if (table_heads != 1 && table_heads != Hq) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t bhi = 0; bhi < (int64_t)B * Hq * Sq; ++bhi) {
        int i = (int)(bhi % Sq);
        int h = (int)((bhi / Sq) % Hq);
        int b = (int)(bhi / ((int64_t)Sq * Hq));
        const uint16_t* f = rfeat + (((size_t)b * Sq + i) * Hq + h) * (size_t)d_rel;
        const uint16_t* t = table + (size_t)(table_heads == 1 ? 0 : h) * E * (size_t)d_rel;
        double* out = profiles + (size_t)bhi * E;
        for (int r = 0; r < E; ++r) {
            double sum = 0.0;
            for (int c = 0; c < d_rel; ++c)
                sum += bf16_to_double(f[c]) * bf16_to_double(t[(size_t)r * d_rel + c]);
            out[r] = sum;
        }
    }
    return 0;
}

/* Threads the OpenMP runtime will use for a parallel region (reported by callers). */
int attn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Mask only: n_allowed[B*Sq] for every query row, and, when `mask` is not
 * NULL, the whole visibility matrix mask[B, Sq, Sk] (1 = allowed).  Uses the
 * same `allowed` statement as attn_oracle_fwd.  Returns 0, or -1 on bad
 * arguments.
 */
int attn_oracle_mask(const uint8_t* valid, const uint8_t* key_valid,
                     const int32_t* positions, const int32_t* key_positions,
                     int64_t window, int64_t query_offset, int B, int Sq, int Sk,
                     int32_t* n_allowed, uint8_t* mask, int n_threads)
{
    if (!valid || !key_valid || !positions || !key_positions || !n_allowed) return -1;
    if (B < 0 || Sq < 0 || Sk < 0) return -1;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t row = 0; row < (int64_t)B * Sq; ++row) {
        int b = (int)(row / Sq), i = (int)(row % Sq);
        int count = 0;
        for (int j = 0; j < Sk; ++j) {
            int a = allowed(valid, key_valid, positions, key_positions, window, query_offset,
                            Sq, Sk, b, i, j);
            count += a;
            if (mask) mask[(size_t)row * Sk + j] = (uint8_t)a;
        }
        n_allowed[row] = count;
    }
    return 0;
}
