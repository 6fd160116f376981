/* Runs every entry point of the oracle once or more on small inputs, edge cases
 * included, for a build with AddressSanitizer and UndefinedBehaviorSanitizer:
 * any out-of-bounds access, use of freed memory or undefined operation aborts
 * the run.  The values are checked only against closed forms that need no
 * other code (the thorough pins live in the Python tests). */
#include "../../oracle/dms_oracle.c"

#include <stdio.h>

static int fails = 0;
#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++fails;                                                     \
        }                                                                \
    } while (0)

static uint16_t bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

int main(void) {
    enum { T = 70, HKV = 2, HQ = 4, D = 16 };
    /* marks: every float class */
    const float lg[] = {-1.f, 0.f, -0.f, 1e-30f, INFINITY, -INFINITY, NAN, 1.4e-45f};
    uint8_t mk8[8];
    dms_oracle_marks(lg, 8, mk8);
    CHECK(mk8[0] == 0 && mk8[1] == 0 && mk8[3] == 1 && mk8[4] == 1 && mk8[5] == 0 && mk8[6] == 0);

    uint8_t* marks = malloc(T * HKV);
    for (int i = 0; i < T * HKV; ++i) marks[i] = (uint8_t)((i * 7) % 3 == 0);
    int32_t pos[T];
    for (int64_t w = 1; w <= T + 1; w += 3)
        for (int64_t t = 0; t < T; ++t) {
            const int64_t n = dms_oracle_live_positions(t, w, marks, HKV, pos);
            CHECK(n >= (t + 1 < w ? t + 1 : w) && n <= t + 1);
            CHECK(n == dms_oracle_live_positions(t, w, marks, HKV, NULL));
        }

    uint16_t *q = malloc(sizeof(uint16_t) * T * HQ * D), *k = malloc(sizeof(uint16_t) * T * HKV * D),
             *v = malloc(sizeof(uint16_t) * T * HKV * D);
    for (int i = 0; i < T * HQ * D; ++i) q[i] = bf16((float)((i * 37) % 11) / 5.f - 1.f);
    for (int i = 0; i < T * HKV * D; ++i) {
        k[i] = bf16((float)((i * 13) % 7) / 3.f - 1.f);
        v[i] = bf16((float)((i * 5) % 9) / 4.f - 1.f);
    }
    int64_t qp[T];
    for (int i = 0; i < T; ++i) qp[i] = i;
    double* out = malloc(sizeof(double) * T * HQ * D);
    CHECK(dms_oracle_attend(HQ, HKV, D, 5, 0.0, T, qp, q, T, k, v, marks, out) == 0);
    for (int i = 0; i < T * HQ * D; ++i) CHECK(isfinite(out[i]));
    /* w = 1, all marked: o_t = v_t */
    uint8_t* all = malloc(T * HKV);
    memset(all, 1, T * HKV);
    CHECK(dms_oracle_attend(HQ, HKV, D, 1, 0.3, T, qp, q, T, k, v, all, out) == 0);
    for (int t = 0; t < T; ++t)
        for (int hq = 0; hq < HQ; ++hq)
            for (int d = 0; d < D; ++d)
                CHECK(out[((int64_t)t * HQ + hq) * D + d] == bf16_bits_to_double(v[((int64_t)t * HKV + hq / 2) * D + d]));
    const int64_t bad = T;
    CHECK(dms_oracle_attend(HQ, HKV, D, 5, 0.0, 1, &bad, q, T, k, v, marks, out) == -1);

    float* kl = malloc(sizeof(float) * T * HKV);
    dms_oracle_k_channel_logits(k, T, HKV, D, D - 1, kl);
    CHECK(kl[0] == (float)bf16_bits_to_double(k[D - 1]));

    /* FP8: every code, every float class */
    for (int c = 0; c < 256; ++c) {
        const double x = dms_oracle_e4m3_value((uint8_t)c);
        if (!isnan(x)) CHECK(dms_oracle_e4m3_value(dms_oracle_e4m3_encode((float)x)) == x);
    }
    CHECK(dms_oracle_e4m3_encode(NAN) == 0x7f);
    CHECK(dms_oracle_e4m3_encode(INFINITY) == 0x7e && dms_oracle_e4m3_encode(-INFINITY) == 0xfe);
    CHECK(dms_oracle_e4m3_encode(1e-30f) == 0x00 && dms_oracle_e4m3_encode(-1e-30f) == 0x80);
    uint8_t *k8 = malloc(T * HKV * D), *v8 = malloc(T * HKV * D);
    float *ks = malloc(sizeof(float) * T * HKV), *vs = malloc(sizeof(float) * T * HKV);
    memset(v, 0, sizeof(uint16_t) * D); /* an all-zero row: scale 1 */
    dms_oracle_quantize_rows(k, T * HKV, D, k8, ks);
    dms_oracle_quantize_rows(v, T * HKV, D, v8, vs);
    CHECK(vs[0] == 1.0f);
    CHECK(dms_oracle_attend_fp8(HQ, HKV, D, 7, 0.0, T, qp, q, T, k8, ks, v8, vs, marks, out) == 0);
    for (int i = 0; i < T * HQ * D; ++i) CHECK(isfinite(out[i]));

    /* bytes */
    int64_t b[3];
    dms_oracle_kv_bytes(T - 1, 1 << 20, marks, HKV, D, 0, 64, b);
    CHECK(b[0] == b[2] && b[1] == HKV * 128 * 2 * (2 * D)); /* 70 tokens: two pages per head */
    dms_oracle_kv_bytes(0, 1, all, HKV, D, 1, 64, b);
    CHECK(b[0] == HKV * 2 * (D + 4));
    CHECK(dms_oracle_row_bytes(128, 0) == 256 && dms_oracle_row_bytes(128, 1) == 132);

    free(marks); free(q); free(k); free(v); free(out); free(all); free(kl);
    free(k8); free(v8); free(ks); free(vs);
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("oracle driver ok\n");
    return 0;
}
