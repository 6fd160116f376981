/*
 * DMS ORACLE -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU statement of what DMS decode / prefill attention computes.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * this file.  It shares no code, header, table or helper with the GPU library;
 * it never looks at a compact store: it keeps the full, uncompressed K/V of
 * every token and decides per (query, key) whether the key is visible.
 *
 * Sources (the method is described in prose only):
 *  [MV] "NVIDIA veroeffentlicht Qwen3-8B-DMS-8x mit innovativer
 *       Speicherkompression fuer verbesserte Inferenzzeiten" (mindverse news
 *       page), section "Dynamic Memory Sparsification (DMS): Eine innovative
 *       Loesung": eviction is learned per head; the policy spans the range from
 *       a sliding window over the most recent 512 tokens to full attention; a
 *       token marked for eviction is kept for a while after it is marked
 *       (delayed eviction).
 *  [ST] "Nvidia DMS: szhatie pamyati LLM v 8 raz" (stiva.ai blog), sections
 *       "Dynamic Memory Sparsification: ..." (one keep/evict signal per token)
 *       and "Klyuchevoe izobretenie: delayed eviction" (a marked token stays
 *       readable for some hundreds of further steps, then is removed).
 *  [FD] "FastDMS: vLLM BF16/FP8 ... 6.4x KV cache" (molayo1419.me), quality
 *       method paragraph: the eviction-disabled reference is the same engine
 *       with a 1M-token window, i.e. the whole KV cache is kept.
 *
 * Readings taken where the pages leave a step open:
 *  - a token's keep/evict decision is taken from its own logit when it is
 *    appended; it is marked iff logit > 0 (a logit of exactly 0 is not marked);
 *  - the delay window w counts query steps: a marked token at position s is
 *    visible to the queries t = s, s+1, ..., s+w-1 and to no later one
 *    (t < s + w); an unmarked token is visible to every t >= s;
 *  - a query always sees its own token (the causal diagonal);
 *  - scores are scale * <q, k> with scale = 1/sqrt(head_dim) unless given;
 *  - grouped-query attention maps q head hq to kv head hq / (Hq / Hkv).
 *
 * Arithmetic: inputs are bf16 bit patterns; every product, sum, exp and divide
 * is done in double.  Softmax subtracts the maximum visible score before exp.
 *
 * FP8 K/V (a compact store holding K and V as 8-bit floats; the FastDMS page
 * [FD] lists FP8 KV caches beside BF16 ones): each (token, kv head) row of K,
 * and of V, is stored as OCP FP8 E4M3 codes with one fp32 scale:
 *   amax  = max_d |x_d|                       (x: the row's bf16 values)
 *   scale = amax / 448 in fp32 (448 is the largest finite E4M3 value), or 1 for
 *           an all-zero row
 *   c_d   = the finite E4M3 value nearest to x_d / scale (fp32 quotient), ties
 *           to the code with an even last bit; beyond +-448 that is +-448
 *   x^_d  = value(c_d) * scale
 * and attention reads x^ in place of x.
 *
 * Eviction logits from a K channel ([MV] "Technische Details und
 * Implementierung": a single neuron of the attention makes the eviction
 * decisions; [ST] the first section: existing neurons of the attention layers
 * are given the keep/evict signal): the logit of (token s, kv head h) is the
 * value of channel c of the token's K row for h, k[s][h][c]; that channel keeps
 * its value in attention.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Eviction marks: m = (logit > 0), one byte per logit ([ST] keep/evict signal). */
void dms_oracle_marks(const float* logits, int64_t n, uint8_t* marks) {
    for (int64_t i = 0; i < n; ++i) marks[i] = logits[i] > 0.0f ? 1 : 0;
}

/* Eviction logits read from channel c of K ([MV] "Technische Details und
 * Implementierung"; [ST]): k is bf16 [n_rows][n_kv_heads][d], out fp32
 * [n_rows][n_kv_heads] = the value of k[r][h][c]. */
void dms_oracle_k_channel_logits(const uint16_t* k, int64_t n_rows, int32_t n_kv_heads, int32_t d, int32_t c,
                                 float* out) {
    for (int64_t r = 0; r < n_rows; ++r)
        for (int32_t h = 0; h < n_kv_heads; ++h)
            out[r * n_kv_heads + h] = (float)bf16_bits_to_double(k[(r * n_kv_heads + h) * d + c]);
}

/* The visibility rule ([MV], [ST]): key position s is visible to query position
 * t iff s <= t and (s is not marked, or t < s + w). */
static int visible(int64_t t, int64_t s, int marked, int64_t window) {
    if (s > t) return 0;
    if (!marked) return 1;
    return t < s + window;
}

/* Live set of one head at query position t: every s <= t visible to t, in
 * ascending order.  marks are read as marks[s * stride].  Writes the positions
 * to out (when out is not NULL) and returns how many there are. */
int64_t dms_oracle_live_positions(int64_t t, int64_t window, const uint8_t* marks,
                                  int64_t stride, int32_t* out) {
    int64_t n = 0;
    for (int64_t s = 0; s <= t; ++s) {
        if (visible(t, s, marks[s * stride], window)) {
            if (out) out[n] = (int32_t)s;
            ++n;
        }
    }
    return n;
}

/* Bytes of one stored K (or V) row of head_dim values: bf16 values take 2
 * bytes each; an FP8 row takes one byte per E4M3 code plus its fp32 scale. */
int64_t dms_oracle_row_bytes(int32_t head_dim, int32_t fp8) {
    return fp8 ? (int64_t)head_dim * 1 + 4 : (int64_t)head_dim * 2;
}

/* What a compact KV store holds for one (sequence, layer) once the token at
 * query position t is in.  The FastDMS announcement (molayo1419.me) reports KV
 * memory as real allocator memory (its memory table), for a store that drops
 * evicted tokens and reclaims their slots (its release paragraph and the
 * "What's the catch?" table); the bytes therefore follow the live sets:
 *   marks [n_kv_heads columns, row s = position s], rows 0 .. t read
 *   out[0] live      = sum over kv heads h of |V_h(t)| * 2 * row_bytes
 *                      (one K and one V row per live token)
 *   out[1] allocated = sum over kv heads h of ceil(|V_h(t)| / page_slots)
 *                      * page_slots * 2 * row_bytes  (whole pages; the live
 *                      tokens of a head fill its slots densely because a freed
 *                      slot is taken by the next token)
 *   out[2] dense     = (t + 1) * n_kv_heads * 2 * head_dim * 2
 *                      (every token kept, bf16: the eviction-disabled store)
 * |V_h(t)| is counted with the visibility rule, token by token. */
void dms_oracle_kv_bytes(int64_t t, int64_t window, const uint8_t* marks, int32_t n_kv_heads,
                         int32_t head_dim, int32_t fp8, int64_t page_slots, int64_t* out) {
    const int64_t row = dms_oracle_row_bytes(head_dim, fp8);
    out[0] = out[1] = 0;
    for (int32_t h = 0; h < n_kv_heads; ++h) {
        int64_t n = 0;
        for (int64_t s = 0; s <= t; ++s) n += visible(t, s, marks[s * n_kv_heads + h], window);
        out[0] += n * 2 * row;
        out[1] += (n + page_slots - 1) / page_slots * page_slots * 2 * row;
    }
    out[2] = (t + 1) * n_kv_heads * 2 * (int64_t)head_dim * 2;
}

/* Masked attention over the full K/V of one (sequence, layer).
 *
 *   q     [n_queries][n_q_heads][head_dim]   bf16 bits, row i is the query at
 *                                            position query_pos[i]
 *   k, v  [n_keys][n_kv_heads][head_dim]     bf16 bits, row s = position s
 *   marks [n_keys][n_kv_heads]               0/1
 *   out   [n_queries][n_q_heads][head_dim]   double
 *
 * For each query t and q head hq (kv head h = hq / group):
 *   z_s = scale * sum_d q[t,hq,d] * k[s,h,d]           for visible s
 *   out = sum_s exp(z_s - max z) v[s,h,:] / sum_s exp(z_s - max z)
 * Returns 0, or -1 when a query position is outside [0, n_keys). */
int dms_oracle_attend(int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                      int64_t window, double scale, int64_t n_queries,
                      const int64_t* query_pos, const uint16_t* q, int64_t n_keys,
                      const uint16_t* k, const uint16_t* v, const uint8_t* marks,
                      double* out) {
    const int32_t group = n_q_heads / n_kv_heads;
    for (int64_t i = 0; i < n_queries; ++i)
        if (query_pos[i] < 0 || query_pos[i] >= n_keys) return -1;
    if (scale == 0.0) scale = 1.0 / sqrt((double)head_dim);

#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)n_keys);
        double* qd = (double*)malloc(sizeof(double) * (size_t)head_dim);
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int64_t i = 0; i < n_queries; ++i) {
            for (int32_t hq = 0; hq < n_q_heads; ++hq) {
                const int64_t t = query_pos[i];
                const int32_t h = hq / group;
                const uint16_t* qrow = q + (i * n_q_heads + hq) * (int64_t)head_dim;
                for (int32_t d = 0; d < head_dim; ++d) qd[d] = bf16_bits_to_double(qrow[d]);

                double zmax = -INFINITY;
                for (int64_t s = 0; s <= t; ++s) {
                    if (!visible(t, s, marks[s * n_kv_heads + h], window)) continue;
                    const uint16_t* krow = k + (s * n_kv_heads + h) * (int64_t)head_dim;
                    double dot = 0.0;
                    for (int32_t d = 0; d < head_dim; ++d) dot += qd[d] * bf16_bits_to_double(krow[d]);
                    z[s] = scale * dot;
                    if (z[s] > zmax) zmax = z[s];
                }

                double* o = out + (i * n_q_heads + hq) * (int64_t)head_dim;
                for (int32_t d = 0; d < head_dim; ++d) o[d] = 0.0;
                double denom = 0.0;
                for (int64_t s = 0; s <= t; ++s) {
                    if (!visible(t, s, marks[s * n_kv_heads + h], window)) continue;
                    const double wgt = exp(z[s] - zmax);
                    const uint16_t* vrow = v + (s * n_kv_heads + h) * (int64_t)head_dim;
                    denom += wgt;
                    for (int32_t d = 0; d < head_dim; ++d) o[d] += wgt * bf16_bits_to_double(vrow[d]);
                }
                for (int32_t d = 0; d < head_dim; ++d) o[d] /= denom;
            }
        }
        free(qd);
        free(z);
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * OCP FP8 E4M3: sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 *   exponent field 0:     (-1)^s * 2^-6 * m / 8            (zero and subnormals)
 *   exponent field 1..15: (-1)^s * 2^(e-7) * (1 + m / 8)
 *   S.1111.111 is NaN; there is no infinity; the largest finite value is
 *   S.1111.110 = 1.75 * 2^8 = 448.
 * ------------------------------------------------------------------------- */
double dms_oracle_e4m3_value(uint8_t code) {
    const int sgn = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sgn ? -mag : mag;
}

/* The finite E4M3 code nearest to x (ties: the code with an even last bit);
 * the sign of x is kept, so x in (-2^-10, 0] gives -0 (0x80) or +0.  NaN gives
 * 0x7f.  Codes 0x00..0x7e are the non-negative finite values in increasing
 * order, so the nearest one is found by walking them. */
uint8_t dms_oracle_e4m3_encode(float x) {
    if (isnan(x)) return 0x7f;
    const uint8_t sgn = signbit(x) ? 0x80 : 0x00;
    const double a = fabs((double)x);
    uint8_t best = 0;
    double best_d = a;  /* distance to code 0 (value 0) */
    for (int c = 1; c <= 0x7e; ++c) {
        const double d = fabs(dms_oracle_e4m3_value((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = (uint8_t)c;
            best_d = d;
        }
    }
    return (uint8_t)(sgn | best);
}

/* Quantise n_rows rows of d bf16 values each to E4M3 codes and one scale per row
 * (see the header): codes[r*d + i], scales[r]. */
void dms_oracle_quantize_rows(const uint16_t* x, int64_t n_rows, int32_t d, uint8_t* codes, float* scales) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) {
        const uint16_t* row = x + r * d;
        float amax = 0.0f;
        for (int32_t i = 0; i < d; ++i) {
            const float v = fabsf((float)bf16_bits_to_double(row[i]));
            if (v > amax) amax = v;
        }
        const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
        scales[r] = scale;
        for (int32_t i = 0; i < d; ++i) codes[r * d + i] = dms_oracle_e4m3_encode((float)bf16_bits_to_double(row[i]) / scale);
    }
}

/* Masked attention as dms_oracle_attend, with K and V given as E4M3 codes and
 * one scale per (key, kv head) row:
 *   k8, v8 [n_keys][n_kv_heads][head_dim] codes, ks, vs [n_keys][n_kv_heads] scales;
 * key values value(k8) * ks, value values value(v8) * vs (double). */
int dms_oracle_attend_fp8(int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                          int64_t window, double scale, int64_t n_queries,
                          const int64_t* query_pos, const uint16_t* q, int64_t n_keys,
                          const uint8_t* k8, const float* ks, const uint8_t* v8, const float* vs,
                          const uint8_t* marks, double* out) {
    const int32_t group = n_q_heads / n_kv_heads;
    for (int64_t i = 0; i < n_queries; ++i)
        if (query_pos[i] < 0 || query_pos[i] >= n_keys) return -1;
    if (scale == 0.0) scale = 1.0 / sqrt((double)head_dim);
    double table[256];
    for (int c = 0; c < 256; ++c) table[c] = dms_oracle_e4m3_value((uint8_t)c);

#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)n_keys);
        double* qd = (double*)malloc(sizeof(double) * (size_t)head_dim);
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int64_t i = 0; i < n_queries; ++i) {
            for (int32_t hq = 0; hq < n_q_heads; ++hq) {
                const int64_t t = query_pos[i];
                const int32_t h = hq / group;
                const uint16_t* qrow = q + (i * n_q_heads + hq) * (int64_t)head_dim;
                for (int32_t d = 0; d < head_dim; ++d) qd[d] = bf16_bits_to_double(qrow[d]);

                double zmax = -INFINITY;
                for (int64_t s = 0; s <= t; ++s) {
                    if (!visible(t, s, marks[s * n_kv_heads + h], window)) continue;
                    const uint8_t* krow = k8 + (s * n_kv_heads + h) * (int64_t)head_dim;
                    const double kscale = (double)ks[s * n_kv_heads + h];
                    double dot = 0.0;
                    for (int32_t d = 0; d < head_dim; ++d) dot += qd[d] * (table[krow[d]] * kscale);
                    z[s] = scale * dot;
                    if (z[s] > zmax) zmax = z[s];
                }

                double* o = out + (i * n_q_heads + hq) * (int64_t)head_dim;
                for (int32_t d = 0; d < head_dim; ++d) o[d] = 0.0;
                double denom = 0.0;
                for (int64_t s = 0; s <= t; ++s) {
                    if (!visible(t, s, marks[s * n_kv_heads + h], window)) continue;
                    const double wgt = exp(z[s] - zmax);
                    const uint8_t* vrow = v8 + (s * n_kv_heads + h) * (int64_t)head_dim;
                    const double vscale = (double)vs[s * n_kv_heads + h];
                    denom += wgt;
                    for (int32_t d = 0; d < head_dim; ++d) o[d] += wgt * (table[vrow[d]] * vscale);
                }
                for (int32_t d = 0; d < head_dim; ++d) o[d] /= denom;
            }
        }
        free(qd);
        free(z);
    }
    return 0;
}

