/* Oracle stress for host sanitizer builds (AddressSanitizer, UBSan): random
 * small problems in every storage format, with and without a row subset, key
 * ranges and sliding windows, plus rejected inputs (a block-table entry past
 * the pool, a length past the table row) and the element decoders over every
 * code.  Test infrastructure: plain C. */
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_attention(int P, int W, int Hq, int Hkv, int D, int num_pages, int bt_stride,
                     int causal, int kv_fmt, double scale, const uint16_t *q,
                     const void *k_pool, const void *v_pool, const void *k_scale,
                     const void *v_scale, const int32_t *block_table,
                     const int32_t *seq_lens, const int32_t *rows, int n_rows,
                     int key_lo, int key_hi, int window_left, double *out, double *lse);
void oracle_decode_bf16(const uint16_t *src, double *dst, int64_t n);
void oracle_decode_e4m3(const uint8_t *src, double *dst, int64_t n);
void oracle_decode_e2m1(const uint8_t *src, double *dst, int64_t n);
void oracle_decode_e8m0(const uint8_t *src, double *dst, int64_t n);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (uint32_t)(state >> 16);
}

static uint16_t bf16_of(float x)
{
    union { float f; uint32_t u; } v = {x};
    return (uint16_t)(v.u >> 16);
}

static void *fill(size_t bytes)
{
    uint8_t *b = malloc(bytes ? bytes : 1);
    for (size_t i = 0; i < bytes; ++i)
        b[i] = (uint8_t)rnd();
    return b;
}

int main(int argc, char **argv)
{
    int iters = argc > 1 ? atoi(argv[1]) : 200;
    int bad = 0;
    for (int it = 0; it < iters; ++it) {
        int P = 1 + rnd() % 3, W = 1 + rnd() % 4, Hkv = 1 + rnd() % 2, G = 1 + rnd() % 3;
        int Hq = Hkv * G, fmt = rnd() % 4;   /* 3: bf16, token-major V pages */
        int D = fmt == 2 ? 32 * (1 + rnd() % 2) : (rnd() % 2 ? 8 : 64);
        int bt_stride = 1 + rnd() % 4, num_pages = P * bt_stride + rnd() % 3;
        int causal = rnd() % 2, cap = 16 * bt_stride;
        int32_t *seq = malloc(sizeof(int32_t) * P), *bt = malloc(sizeof(int32_t) * P * bt_stride);
        for (int p = 0; p < P; ++p) {
            int L = rnd() % (cap + 1);
            if (causal && L > 0 && L < W)
                L = W <= cap ? W : 0;
            seq[p] = L;
        }
        for (int i = 0; i < P * bt_stride; ++i)
            bt[i] = rnd() % num_pages;
        size_t elems = (size_t)num_pages * Hkv * 16 * D;
        size_t pool_bytes = fmt == 0 || fmt == 3 ? 2 * elems : fmt == 1 ? elems : elems / 2;
        void *kp = fill(pool_bytes), *vp = fill(pool_bytes), *ks = NULL, *vs = NULL;
        if (fmt == 0 || fmt == 3) {   /* finite bf16 values */
            uint16_t *k16 = kp, *v16 = vp;
            for (size_t i = 0; i < elems; ++i) {
                k16[i] = bf16_of((float)((int)(rnd() % 2001) - 1000) / 400.f);
                v16[i] = bf16_of((float)((int)(rnd() % 2001) - 1000) / 400.f);
            }
        } else if (fmt == 1) {
            float *kf = malloc(sizeof(float) * num_pages * Hkv * 16);
            float *vf = malloc(sizeof(float) * num_pages * Hkv * 16);
            for (int i = 0; i < num_pages * Hkv * 16; ++i) {
                kf[i] = 0.01f * (1 + rnd() % 100);
                vf[i] = 0.01f * (1 + rnd() % 100);
            }
            ks = kf, vs = vf;
        } else {
            ks = fill((size_t)num_pages * Hkv * 16 * (D / 32));
            vs = fill((size_t)num_pages * Hkv * 16 * (D / 32));
        }
        size_t qn = (size_t)P * W * Hq * D;
        uint16_t *q = malloc(sizeof(uint16_t) * qn);
        for (size_t i = 0; i < qn; ++i)
            q[i] = bf16_of((float)((int)(rnd() % 2001) - 1000) / 500.f);
        int n_rows = 0, *rows = NULL;
        if (rnd() % 2) {
            n_rows = 1 + rnd() % 5;
            rows = malloc(sizeof(int) * 3 * n_rows);
            for (int r = 0; r < n_rows; ++r) {
                rows[3 * r] = rnd() % P;
                rows[3 * r + 1] = rnd() % W;
                rows[3 * r + 2] = rnd() % Hq;
            }
        }
        int key_lo = 0, key_hi = INT_MAX;
        if (rnd() % 3 == 0) {
            key_lo = rnd() % (cap + 1);
            key_hi = key_lo + rnd() % (cap + 1);
        }
        int window_left = rnd() % 3 == 0 ? (int)(1 + rnd() % (cap + 1)) : 0;
        int n = rows ? n_rows : P * W * Hq;
        double *out = malloc(sizeof(double) * (size_t)n * D), *lse = malloc(sizeof(double) * n);
        int rc = oracle_attention(P, W, Hq, Hkv, D, num_pages, bt_stride, causal, fmt, 0.125, q,
                                  kp, vp, ks, vs, bt, seq, rows, n_rows, key_lo, key_hi,
                                  window_left, out, lse);
        if (rc != 0) {
            fprintf(stderr, "oracle_stress: valid input rejected (iteration %d)\n", it);
            bad = 1;
        }
        /* rejected inputs: a table entry past the pool, a length past the row */
        int p0 = 0;
        if (seq[p0] > 0) {
            int32_t keep = bt[0];
            bt[0] = num_pages;
            if (oracle_attention(P, W, Hq, Hkv, D, num_pages, bt_stride, causal, fmt, 0.125, q,
                                 kp, vp, ks, vs, bt, seq, rows, n_rows, key_lo, key_hi,
                                 window_left, out, lse) == 0) {
                fprintf(stderr, "oracle_stress: bad table entry accepted (iteration %d)\n", it);
                bad = 1;
            }
            bt[0] = keep;
        }
        int32_t keep_L = seq[p0];
        seq[p0] = cap + 1;
        if (oracle_attention(P, W, Hq, Hkv, D, num_pages, bt_stride, causal, fmt, 0.125, q, kp,
                             vp, ks, vs, bt, seq, rows, n_rows, key_lo, key_hi, window_left,
                             out, lse) == 0) {
            fprintf(stderr, "oracle_stress: overlong length accepted (iteration %d)\n", it);
            bad = 1;
        }
        seq[p0] = keep_L;
        free(out), free(lse), free(rows), free(q), free(kp), free(vp), free(ks), free(vs);
        free(seq), free(bt);
    }
    uint16_t codes16[65536];
    uint8_t codes8[256];
    double *dst = malloc(sizeof(double) * 65536);
    for (int i = 0; i < 65536; ++i)
        codes16[i] = (uint16_t)i;
    for (int i = 0; i < 256; ++i)
        codes8[i] = (uint8_t)i;
    oracle_decode_bf16(codes16, dst, 65536);
    oracle_decode_e4m3(codes8, dst, 256);
    oracle_decode_e2m1(codes8, dst, 256);
    oracle_decode_e8m0(codes8, dst, 256);
    free(dst);
    printf("oracle_stress: %d problems, %s\n", iters, bad ? "FAILED" : "ok");
    return bad;
}
