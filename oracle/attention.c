/*
 * Oracle -- TEST INFRASTRUCTURE ONLY.  Plain, slow, fp64 CPU attention over a
 * paged KV cache.  Only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark may load this code; the library never does.  It shares no
 * source, header or constant with the HIP path.
 *
 * What it computes (passages it follows):
 *  - "ChunkedSmallT re-streams full KV per query chunk", section Finding: every
 *    one of the W window rows attends the request's visible key range.
 *  - "DFlash2 leaves the paged graph fast path ...", section The route change and
 *    section Scope: attention is computed for the P x (1+k) block rows only,
 *    against each request's own paged context, addressed through one shared
 *    pool, a batched block table and per-request sequence lengths.
 *  - same page, section The cost: a non-causal row attends its request's
 *    entire span.
 *  - "perf(dflash): widen the verify window ...", section What changed: only
 *    the first seq_len entries of a request are read (stale rows beyond it are
 *    never looked at); section Exactness: rows are independent.
 *  - causal verify alignment: window row i sits at absolute position
 *    L - W + i and sees keys at positions <= L - W + i (bottom-right mask).
 *  - "DFlash2 leaves the paged graph fast path ...", section The cost, notes
 *    that the draft path does not apply a window and defers it to a separate
 *    issue.  The sliding window read here: with window_left = N > 0 a row
 *    whose last visible key is at position h sees only keys h - N + 1 .. h.
 *  - "ChunkedSmallT re-streams full KV per query chunk", section Measurement,
 *    times a 4-bit KV cache ("nvfp4") without defining it.  The 4-bit format
 *    read here is OCP MXFP4: E2M1 elements in blocks of 32 consecutive head-dim
 *    elements of one token, each block with one E8M0 power-of-two scale.
 *
 * Steps, in order: gather the request's visible pages into contiguous K and V
 * (decoded exactly to fp64), then for each row the textbook softmax attention
 *   s_j = scale * <q, k_j>,  m = max s_j,  l = sum exp(s_j - m),
 *   o = sum exp(s_j - m) v_j / l,  lse = m + ln l   (natural log).
 * An empty visible set gives o = 0 and lse = -inf.
 *
 * Storage it reads (the library's documented layout):
 *   q        uint16 bf16 bits  [P][W][Hq][D]
 *   k_pool   [num_pages][Hkv][16][D]   bf16 bits or e4m3fn bytes
 *   v_pool   [num_pages][Hkv][D][16]   (each page-head stored transposed), or
 *            [num_pages][Hkv][16][D] like K for bf16 with token-major values
 *   k_scale, v_scale  fp32 [num_pages][Hkv][16]  (fp8 only)
 *   MXFP4 (two E2M1 codes per byte, the even element in the low nibble):
 *   k_pool   [num_pages][Hkv][16][D/2]  byte (t, i): elements 2i, 2i+1 of token t
 *   v_pool   [num_pages][Hkv][D][8]     byte (d, i): element d of tokens 2i, 2i+1
 *   k_scale  E8M0 bytes [num_pages][Hkv][16][D/32]: block b of token t covers
 *            elements 32b .. 32b+31 of its row
 *   v_scale  E8M0 bytes [num_pages][Hkv][D/32][16]: the same blocks, stored
 *            block-major like the transposed value page
 *   block_table int32 [P][bt_stride], seq_lens int32 [P]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_PAGE 16

/* bf16 is the upper half of an IEEE binary32: widen by 16 zero bits. */
double oracle_bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit floating point, E4M3 ("FN": no infinities, S.1111.111 is NaN),
 * exponent bias 7:  normal   (-1)^s * 2^(e-7) * (1 + m/8),  e in 1..15
 *                   subnormal (-1)^s * 2^(-6) * (m/8),       e == 0      */
double oracle_e4m3_to_double(uint8_t code)
{
    int s = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* OCP MX E2M1 (4-bit: sign, 2 exponent bits with bias 1, 1 mantissa bit):
 *   normal    (-1)^s * 2^(e-1) * (1 + m/2),  e in 1..3
 *   subnormal (-1)^s * (m/2),                e == 0
 * No infinities or NaN. */
double oracle_e2m1_to_double(uint8_t nibble)
{
    int s = (nibble >> 3) & 1;
    int e = (nibble >> 1) & 3;
    int m = nibble & 1;
    double mag = e == 0 ? m / 2.0 : ldexp(1.0 + m / 2.0, e - 1);
    return s ? -mag : mag;
}

/* OCP MX E8M0 scale: 2^(e-127); 0xFF is NaN. */
double oracle_e8m0_to_double(uint8_t e)
{
    return e == 0xFF ? NAN : ldexp(1.0, (int)e - 127);
}

/* ORACLE_KV_BF16_VTOK: bf16 pools whose value pages are token-major like K */
enum { ORACLE_KV_BF16 = 0, ORACLE_KV_E4M3 = 1, ORACLE_KV_MXFP4 = 2, ORACLE_KV_BF16_VTOK = 3 };

typedef struct {
    int P, W, Hq, Hkv, D, num_pages, bt_stride, causal, kv_fmt;
    double scale;
    const uint16_t *q;
    const void *k_pool, *v_pool;
    const void *k_scale, *v_scale;
    const int32_t *block_table, *seq_lens;
} oracle_in;

/* nibble k (0 = low) of byte b */
static uint8_t nibble(uint8_t b, int k)
{
    return k ? (uint8_t)(b >> 4) : (uint8_t)(b & 15);
}

/* MX block scale of element d of token slot in a page-head: K scales are
 * token-major [16][D/32], V scales block-major [D/32][16] */
static double mx_scale(const void *scales, const oracle_in *in, int64_t page, int kvh, int slot,
                       int d, int block_major)
{
    int64_t head = (page * in->Hkv + kvh) * ORACLE_PAGE * (in->D / 32);
    int64_t idx = block_major ? head + (int64_t)(d / 32) * ORACLE_PAGE + slot
                              : head + (int64_t)slot * (in->D / 32) + d / 32;
    return oracle_e8m0_to_double(((const uint8_t *)scales)[idx]);
}

static double k_elem(const oracle_in *in, int64_t page, int kvh, int slot, int d)
{
    if (in->kv_fmt == ORACLE_KV_MXFP4) {
        int64_t byte = ((page * in->Hkv + kvh) * ORACLE_PAGE + slot) * (in->D / 2) + d / 2;
        uint8_t code = nibble(((const uint8_t *)in->k_pool)[byte], d & 1);
        return oracle_e2m1_to_double(code) * mx_scale(in->k_scale, in, page, kvh, slot, d, 0);
    }
    int64_t idx = ((page * in->Hkv + kvh) * ORACLE_PAGE + slot) * in->D + d;
    if (in->kv_fmt == ORACLE_KV_E4M3) {
        double sc = (double)((const float *)in->k_scale)[(page * in->Hkv + kvh) * ORACLE_PAGE + slot];
        return oracle_e4m3_to_double(((const uint8_t *)in->k_pool)[idx]) * sc;
    }
    return oracle_bf16_to_double(((const uint16_t *)in->k_pool)[idx]);
}

static double v_elem(const oracle_in *in, int64_t page, int kvh, int slot, int d)
{
    if (in->kv_fmt == ORACLE_KV_MXFP4) {
        int64_t byte = ((page * in->Hkv + kvh) * in->D + d) * (ORACLE_PAGE / 2) + slot / 2;
        uint8_t code = nibble(((const uint8_t *)in->v_pool)[byte], slot & 1);
        return oracle_e2m1_to_double(code) * mx_scale(in->v_scale, in, page, kvh, slot, d, 1);
    }
    if (in->kv_fmt == ORACLE_KV_BF16_VTOK)
        return oracle_bf16_to_double(
            ((const uint16_t *)in->v_pool)[((page * in->Hkv + kvh) * ORACLE_PAGE + slot) * in->D + d]);
    int64_t idx = ((page * in->Hkv + kvh) * in->D + d) * ORACLE_PAGE + slot;
    if (in->kv_fmt == ORACLE_KV_E4M3) {
        double sc = (double)((const float *)in->v_scale)[(page * in->Hkv + kvh) * ORACLE_PAGE + slot];
        return oracle_e4m3_to_double(((const uint8_t *)in->v_pool)[idx]) * sc;
    }
    return oracle_bf16_to_double(((const uint16_t *)in->v_pool)[idx]);
}

/* Gather the first L tokens of request p, KV head kvh, into dense [L][D]. */
static void gather(const oracle_in *in, int p, int kvh, int L, double *K, double *V)
{
    for (int t = 0; t < L; ++t) {
        int64_t page = in->block_table[(int64_t)p * in->bt_stride + t / ORACLE_PAGE];
        int slot = t % ORACLE_PAGE;
        for (int d = 0; d < in->D; ++d) {
            K[(int64_t)t * in->D + d] = k_elem(in, page, kvh, slot, d);
            V[(int64_t)t * in->D + d] = v_elem(in, page, kvh, slot, d);
        }
    }
}

/* One query row against keys j in [lo, hi) of the gathered K/V. */
static void attend_row(const oracle_in *in, const double *qrow, const double *K,
                       const double *V, int lo, int hi, double *s, double *o, double *lse)
{
    int D = in->D;
    for (int d = 0; d < D; ++d)
        o[d] = 0.0;
    if (hi <= lo) {
        *lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (int j = lo; j < hi; ++j) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += qrow[d] * K[(int64_t)j * D + d];
        s[j - lo] = in->scale * acc;
        if (s[j - lo] > m)
            m = s[j - lo];
    }
    double l = 0.0;
    for (int j = lo; j < hi; ++j) {
        double e = exp(s[j - lo] - m);
        l += e;
        for (int d = 0; d < D; ++d)
            o[d] += e * V[(int64_t)j * D + d];
    }
    for (int d = 0; d < D; ++d)
        o[d] /= l;
    *lse = m + log(l);
}

/*
 * Full or sampled attention.
 *   rows == NULL: every (p, i, h); out is [P][W][Hq][D], lse is [P][W][Hq].
 *   rows != NULL: n_rows triples (p, i, h); out is [n_rows][D], lse [n_rows].
 * Keys are further restricted to absolute positions [key_lo, key_hi) (pass
 * 0 and INT32_MAX for plain attention) so a test can form split partials, and
 * to the row's last window_left keys when window_left > 0.
 * Returns 0, or -1 on an argument the library would also reject.
 */
int oracle_attention(int P, int W, int Hq, int Hkv, int D, int num_pages, int bt_stride,
                     int causal, int kv_fmt, double scale, const uint16_t *q,
                     const void *k_pool, const void *v_pool, const void *k_scale,
                     const void *v_scale, const int32_t *block_table,
                     const int32_t *seq_lens, const int32_t *rows, int n_rows,
                     int key_lo, int key_hi, int window_left, double *out, double *lse)
{
    if (P < 1 || W < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || bt_stride < 1)
        return -1;
    if (kv_fmt < ORACLE_KV_BF16 || kv_fmt > ORACLE_KV_BF16_VTOK)
        return -1;
    if ((kv_fmt == ORACLE_KV_E4M3 || kv_fmt == ORACLE_KV_MXFP4) && (!k_scale || !v_scale))
        return -1;
    if (kv_fmt == ORACLE_KV_MXFP4 && D % 32)
        return -1;
    for (int p = 0; p < P; ++p) {
        int L = seq_lens[p];
        if (L < 0 || L > bt_stride * ORACLE_PAGE)
            return -1;
        if (causal && L > 0 && L < W)
            return -1;
        for (int t = 0; t < L; t += ORACLE_PAGE) {
            int32_t pg = block_table[(int64_t)p * bt_stride + t / ORACLE_PAGE];
            if (pg < 0 || pg >= num_pages)
                return -1;
        }
    }
    oracle_in in = {P, W, Hq, Hkv, D, num_pages, bt_stride, causal, kv_fmt, scale,
                    q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens};
    int G = Hq / Hkv;
    int total = rows ? n_rows : P * W * Hq;

    for (int p = 0; p < P; ++p) {
        int L = seq_lens[p];
        for (int kvh = 0; kvh < Hkv; ++kvh) {
            /* does this (p, kvh) own any requested row? */
            int wanted = 0;
            for (int r = 0; r < total && !wanted; ++r) {
                int rp = rows ? rows[3 * r] : r / (W * Hq);
                int rh = rows ? rows[3 * r + 2] : r % Hq;
                wanted = (rp == p && rh / G == kvh);
            }
            if (!wanted)
                continue;
            int Lg = L > 0 ? L : 1;
            double *K = malloc(sizeof(double) * (size_t)Lg * D);
            double *V = malloc(sizeof(double) * (size_t)Lg * D);
            if (!K || !V) {
                free(K);
                free(V);
                return -2;
            }
            gather(&in, p, kvh, L, K, V);
#pragma omp parallel
            {
                double *s = malloc(sizeof(double) * (size_t)Lg);
                double *qrow = malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
                for (int r = 0; r < total; ++r) {
                    int rp = rows ? rows[3 * r] : r / (W * Hq);
                    int ri = rows ? rows[3 * r + 1] : (r / Hq) % W;
                    int rh = rows ? rows[3 * r + 2] : r % Hq;
                    if (rp != p || rh / G != kvh)
                        continue;
                    int n_vis = causal ? L - W + ri + 1 : L;
                    if (n_vis < 0)
                        n_vis = 0;
                    int lo = key_lo > 0 ? key_lo : 0;
                    int hi = key_hi < n_vis ? key_hi : n_vis;
                    if (window_left > 0 && n_vis - window_left > lo)
                        lo = n_vis - window_left;    /* sliding window */
                    const uint16_t *qsrc = q + (((int64_t)rp * W + ri) * Hq + rh) * D;
                    for (int d = 0; d < D; ++d)
                        qrow[d] = oracle_bf16_to_double(qsrc[d]);
                    double *orow = out + (int64_t)r * D;
                    attend_row(&in, qrow, K, V, lo, hi, s, orow, &lse[r]);
                }
                free(s);
                free(qrow);
            }
            free(K);
            free(V);
        }
    }
    return 0;
}

/* Decode helpers exposed for the format pins. */
void oracle_decode_bf16(const uint16_t *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = oracle_bf16_to_double(src[i]);
}

void oracle_decode_e4m3(const uint8_t *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = oracle_e4m3_to_double(src[i]);
}

/* src holds one E2M1 code per byte (low nibble) */
void oracle_decode_e2m1(const uint8_t *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = oracle_e2m1_to_double(src[i] & 15);
}

void oracle_decode_e8m0(const uint8_t *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = oracle_e8m0_to_double(src[i]);
}

#ifdef _OPENMP
#include <omp.h>
#endif
/* Threads the parallel loops above run with. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
