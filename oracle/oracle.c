/*
 * oracle.c -- plain CPU reference for paged attention decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library.  It shares no
 * code with the HIP library: it has its own number formats, its own pool
 * addressing and its own quantizer, all written out from the definitions
 * below.  It is slow on purpose: fp64, no blocking, no fusion.
 *
 * What it computes
 * ----------------
 * decode:   for every sequence s and query head h, with kv head kvh = h / G
 *           (G = num_heads / num_kv_heads, contiguous head groups):
 *             gather the contiguous K, V of tokens 0 .. L-1 of s through the
 *             block table (logical block t / BS -> physical block, slot t % BS),
 *             x_t = scale * sum_d q[s][h][d] * K[t][d]
 *             out[s][h][:] = sum_t softmax(x)_t * V[t][:]
 *           i.e. the scaled dot-product attention softmax(q K^T / sqrt(d_k)) V
 *           of "KVcache-learning" (fairy2021.github.io), chapter s01 (the
 *           self-attention formula) and chapter s05 (PagedAttention: the same
 *           math over K/V kept in non-contiguous physical blocks reached via a
 *           block table).  Paging changes only where K/V are stored, not the
 *           result ("vLLM PagedAttention deep dive", jsqmd.com, section 9).
 *           The block-table indexing follows the kernel entry shown in
 *           "KV Cache and PagedAttention (vllm-musa)", 7yue.com, section 5.
 *           L = 0 gives zeros (no page covers it; a padded batch needs it).
 *
 * write:    token i with slot = slot_mapping[i] >= 0 goes to physical block
 *           slot / BS, position slot % BS ("append the new token's K/V to the
 *           cache", KVcache-learning s02).  int8 / fp8-e4m3 caches store one
 *           fp16 scale per (token, kv head), separately for K and V
 *           (KVcache-learning s09 recommends a KV-cache scaling factor; the
 *           per-token-and-head granularity is this library's reading):
 *             a   = max_d |x_d|                         (fp32)
 *             s32 = a / 127  (int8)  or  a / 448 (e4m3)  (fp32 IEEE division)
 *             s16 = binary16(s32) rounded to nearest even; s = value of s16
 *             s == 0: every code is 0
 *             int8: code = clamp(round_half_even(x_d / s), -127, 127)
 *             e4m3: code = E4M3 encode of x_d / s, round to nearest even,
 *                   saturating at +-448 (OCP 8-bit floating point spec, E4M3)
 *           The dequantized value is code * s.
 *
 * copy:     copy-on-write block copy (KVcache-learning s05, copy-on-write):
 *           every byte of the K tile, V tile and scales of block src is
 *           copied into block dst, for all kv heads.
 *
 * Pool layout (the library's documented ABI layout, re-derived here from its
 * description, not shared):
 *   the slice (b, kvh) of K or V starts at byte ((b * Hkv + kvh) * BS * D * eb),
 *   eb = bytes per element.  A slice is a run of tiles of TB = min(BS, 16)
 *   tokens (one tile for BS <= 16, two for BS = 32), each TB * D * eb bytes.
 *   Token t is position u = t % TB of tile t / TB; inside its tile, byte j of
 *   its D-vector (j = d * eb + byte-in-element) lives at
 *     K: ((j / 16) * TB + u) * 16 + j % 16     (16-byte columns, token-minor)
 *     V, eb 2 or 4: ((j / 4) * TB + u) * 4 + j % 4   (4-byte columns, token-minor)
 *     V, eb 1 (int8 / E4M3): ((d / 4) * (TB / 4) + u / 4) * 16 + (d % 4) * 4 + u % 4
 *        (16-byte groups of 4 elements x 4 tokens, token-minor inside)
 *   scales: fp16 [num_blocks][Hkv][BS].
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_I8 = 2, ORC_E4M3 = 3 };

static int orc_elem_bytes(int kind) { return kind == ORC_F32 ? 4 : kind == ORC_F16 ? 2 : 1; }

/* ---- IEEE 754 binary16 ------------------------------------------------- */

double orc_f16_to_f64(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp(1.0 + m / 1024.0, e - 15);
    return sign ? -v : v;
}

/* Round a float to binary16, nearest-even; overflow gives infinity. */
uint16_t orc_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (isnan(x)) return sign | 0x7E00;
    if (a >= 65520.0) return sign | 0x7C00;   /* halfway above 65504 and beyond */
    if (a < ldexp(1.0, -14)) {                  /* subnormal range, step 2^-24 */
        double q = nearbyint(ldexp(a, 24));     /* exact scaling, RNE to integer */
        return sign | (uint16_t)q;              /* q == 1024 is the smallest normal */
    }
    int e;
    double f = frexp(a, &e);                    /* a = f * 2^e, f in [0.5, 1) */
    f *= 2.0; e -= 1;                           /* f in [1, 2) */
    double mant = nearbyint((f - 1.0) * 1024.0);
    if (mant == 1024.0) { mant = 0.0; e += 1; }
    if (e + 15 >= 31) return sign | 0x7C00;
    return sign | (uint16_t)((e + 15) << 10) | (uint16_t)mant;
}

/* ---- OCP OFP8 E4M3: bias 7, no infinities, S.1111.111 is NaN ----------- */

double orc_e4m3_to_f64(uint8_t c)
{
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Nearest-even encode, saturating to +-448; NaN maps to 0x7F. */
uint8_t orc_f32_to_e4m3(float y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0;
    double a = fabs((double)y);
    if (isnan(y)) return 0x7F;
    if (a >= 448.0) return sign | 0x7E;          /* 1.75 * 2^8 */
    if (a < ldexp(1.0, -6)) {                    /* subnormals, step 2^-9 */
        double q = nearbyint(ldexp(a, 9));
        return sign | (uint8_t)q;                /* q == 8 is the smallest normal */
    }
    int e;
    double f = frexp(a, &e);
    f *= 2.0; e -= 1;
    double mant = nearbyint((f - 1.0) * 8.0);
    if (mant == 8.0) { mant = 0.0; e += 1; }
    return sign | (uint8_t)((e + 7) << 3) | (uint8_t)mant;
}

int8_t orc_f32_to_i8(float y)
{
    double q = nearbyint((double)y);
    if (q > 127.0) q = 127.0;
    if (q < -127.0) q = -127.0;
    return (int8_t)q;
}

/* Quantize one D-vector: codes[n] and its fp16 scale. */
void orc_quantize_row(const float *x, int n, int kind, uint8_t *codes, uint16_t *scale_out)
{
    float a = 0.0f;
    for (int d = 0; d < n; d++) {
        float v = fabsf(x[d]);
        if (v > a) a = v;
    }
    float qmax = (kind == ORC_I8) ? 127.0f : 448.0f;
    float s32 = a / qmax;
    uint16_t s16 = orc_f32_to_f16(s32);
    float s = (float)orc_f16_to_f64(s16);
    *scale_out = s16;
    for (int d = 0; d < n; d++) {
        if (s == 0.0f) { codes[d] = 0; continue; }
        float y = x[d] / s;
        codes[d] = (kind == ORC_I8) ? (uint8_t)orc_f32_to_i8(y) : orc_f32_to_e4m3(y);
    }
}

/* ---- pool addressing ---------------------------------------------------- */

static size_t orc_tile_base(int64_t b, int kvh, int Hkv, int BS, int D, int eb)
{
    return ((size_t)b * Hkv + kvh) * (size_t)BS * D * eb;
}

static int orc_tile_rows(int BS) { return BS < 16 ? BS : 16; }

static size_t orc_k_byte(int t, int j, int BS, int D, int eb)
{
    int TB = orc_tile_rows(BS), u = t % TB;
    return (size_t)(t / TB) * TB * D * eb + ((size_t)(j / 16) * TB + u) * 16 + j % 16;
}

static size_t orc_v_byte(int t, int j, int BS, int D, int eb)
{
    int TB = orc_tile_rows(BS), u = t % TB;
    size_t tile = (size_t)(t / TB) * TB * D * eb;
    if (eb == 1)
        return tile + ((size_t)(j / 4) * (TB / 4) + u / 4) * 16 + (j % 4) * 4 + u % 4;
    return tile + ((size_t)(j / 4) * TB + u) * 4 + j % 4;
}

/* Value of element d of token slot t in tile (b, kvh); is_v selects the V layout. */
static double orc_load(const uint8_t *pool, const uint16_t *scales, int kind, int is_v,
                       int64_t b, int kvh, int t, int d, int Hkv, int BS, int D)
{
    int eb = orc_elem_bytes(kind);
    size_t base = orc_tile_base(b, kvh, Hkv, BS, D, eb);
    unsigned char raw[4];
    for (int k = 0; k < eb; k++) {
        int j = d * eb + k;
        raw[k] = pool[base + (is_v ? orc_v_byte(t, j, BS, D, eb) : orc_k_byte(t, j, BS, D, eb))];
    }
    switch (kind) {
    case ORC_F32: { float f; memcpy(&f, raw, 4); return (double)f; }
    case ORC_F16: { uint16_t h; memcpy(&h, raw, 2); return orc_f16_to_f64(h); }
    default: {
        double s = orc_f16_to_f64(scales[((size_t)b * Hkv + kvh) * BS + t]);
        double c = (kind == ORC_I8) ? (double)(int8_t)raw[0] : orc_e4m3_to_f64(raw[0]);
        return c * s;
    }
    }
}

static void orc_store_raw(uint8_t *pool, int is_v, size_t base, int t, int d, int eb,
                          const unsigned char *raw, int BS, int D)
{
    for (int k = 0; k < eb; k++) {
        int j = d * eb + k;
        pool[base + (is_v ? orc_v_byte(t, j, BS, D, eb) : orc_k_byte(t, j, BS, D, eb))] = raw[k];
    }
}

/* ---- write -------------------------------------------------------------- */

/* src values are float (fp16 sources are widened exactly by the caller).
 * Returns the number of tokens written. */
int orc_write(const float *key, const float *value, const int64_t *slot_mapping, int T,
              uint8_t *k_pool, uint8_t *v_pool, uint16_t *k_scale, uint16_t *v_scale,
              int cache_kind, int num_blocks, int Hkv, int D, int BS)
{
    int eb = orc_elem_bytes(cache_kind), written = 0;
    uint8_t *codes = (uint8_t *)malloc((size_t)D);
    for (int i = 0; i < T; i++) {
        int64_t slot = slot_mapping[i];
        if (slot < 0 || slot >= (int64_t)num_blocks * BS) continue;
        int64_t b = slot / BS;
        int t = (int)(slot % BS);
        for (int kvh = 0; kvh < Hkv; kvh++) {
            for (int which = 0; which < 2; which++) {
                const float *x = (which ? value : key) + ((size_t)i * Hkv + kvh) * D;
                uint8_t *pool = which ? v_pool : k_pool;
                size_t base = orc_tile_base(b, kvh, Hkv, BS, D, eb);
                if (cache_kind == ORC_F32 || cache_kind == ORC_F16) {
                    for (int d = 0; d < D; d++) {
                        unsigned char raw[4];
                        if (cache_kind == ORC_F32) memcpy(raw, &x[d], 4);
                        else { uint16_t h = orc_f32_to_f16(x[d]); memcpy(raw, &h, 2); }
                        orc_store_raw(pool, which, base, t, d, eb, raw, BS, D);
                    }
                } else {
                    uint16_t s16;
                    orc_quantize_row(x, D, cache_kind, codes, &s16);
                    for (int d = 0; d < D; d++) orc_store_raw(pool, which, base, t, d, 1, &codes[d], BS, D);
                    (which ? v_scale : k_scale)[((size_t)b * Hkv + kvh) * BS + t] = s16;
                }
            }
        }
        written++;
    }
    free(codes);
    return written;
}

/* ---- copy-on-write block copy ------------------------------------------ */

int orc_copy_blocks(uint8_t *k_pool, uint8_t *v_pool, uint16_t *k_scale, uint16_t *v_scale,
                    int cache_kind, const int32_t *pairs, int n_pairs, int num_blocks,
                    int Hkv, int D, int BS)
{
    size_t blk = (size_t)Hkv * BS * D * orc_elem_bytes(cache_kind);
    size_t sblk = (size_t)Hkv * BS;
    int done = 0;
    for (int p = 0; p < n_pairs; p++) {
        int32_t src = pairs[2 * p], dst = pairs[2 * p + 1];
        if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks) continue;
        memmove(k_pool + (size_t)dst * blk, k_pool + (size_t)src * blk, blk);
        memmove(v_pool + (size_t)dst * blk, v_pool + (size_t)src * blk, blk);
        if (cache_kind == ORC_I8 || cache_kind == ORC_E4M3) {
            memmove(k_scale + (size_t)dst * sblk, k_scale + (size_t)src * sblk, sblk * 2);
            memmove(v_scale + (size_t)dst * sblk, v_scale + (size_t)src * sblk, sblk * 2);
        }
        done++;
    }
    return done;
}

/* ---- decode ------------------------------------------------------------- */

/* q: double [S][H][D]; out: double [S][H][D].  Returns the thread count used. */
int orc_decode(double *out, const double *q, const uint8_t *k_pool, const uint8_t *v_pool,
               const uint16_t *k_scale, const uint16_t *v_scale, int cache_kind,
               const int32_t *block_tables, int max_blocks, const int32_t *seq_lens,
               int S, int H, int Hkv, int D, int BS, double scale, int num_threads)
{
    if (S < 0 || H <= 0 || Hkv <= 0 || H % Hkv || D <= 0 || BS <= 0) return -1;
    int G = H / Hkv;
    int used = 1;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
#pragma omp for schedule(dynamic, 1)
        for (int unit = 0; unit < S * Hkv; unit++) {
            int s = unit / Hkv, kvh = unit % Hkv;
            int L = seq_lens[s] < 0 ? 0 : seq_lens[s];
            double *K = (double *)malloc(sizeof(double) * ((size_t)L * D + 1));
            double *V = (double *)malloc(sizeof(double) * ((size_t)L * D + 1));
            double *x = (double *)malloc(sizeof(double) * ((size_t)L + 1));
            /* 1. reassemble contiguous K, V of this (seq, kv head) */
            for (int t = 0; t < L; t++) {
                int64_t b = block_tables[(size_t)s * max_blocks + t / BS];
                for (int d = 0; d < D; d++) {
                    K[(size_t)t * D + d] = orc_load(k_pool, k_scale, cache_kind, 0, b, kvh, t % BS, d, Hkv, BS, D);
                    V[(size_t)t * D + d] = orc_load(v_pool, v_scale, cache_kind, 1, b, kvh, t % BS, d, Hkv, BS, D);
                }
            }
            /* 2. textbook softmax(q K^T * scale) V per query head of the group */
            for (int g = 0; g < G; g++) {
                int h = kvh * G + g;
                const double *qv = q + ((size_t)s * H + h) * D;
                double *o = out + ((size_t)s * H + h) * D;
                for (int d = 0; d < D; d++) o[d] = 0.0;
                if (L == 0) continue;
                double m = -INFINITY;
                for (int t = 0; t < L; t++) {
                    double dot = 0.0;
                    for (int d = 0; d < D; d++) dot += qv[d] * K[(size_t)t * D + d];
                    x[t] = scale * dot;
                    if (x[t] > m) m = x[t];
                }
                double Z = 0.0;
                for (int t = 0; t < L; t++) {
                    x[t] = exp(x[t] - m);
                    Z += x[t];
                }
                for (int t = 0; t < L; t++)
                    for (int d = 0; d < D; d++) o[d] += x[t] * V[(size_t)t * D + d];
                for (int d = 0; d < D; d++) o[d] /= Z;
            }
            free(K); free(V); free(x);
        }
    }
    return used;
}

/* Array helpers for the Python wrapper (element-wise over n values). */
void orc_f16_to_f64_n(const uint16_t *h, double *out, int64_t n)
{ for (int64_t i = 0; i < n; i++) out[i] = orc_f16_to_f64(h[i]); }
void orc_f32_to_f16_n(const float *x, uint16_t *out, int64_t n)
{ for (int64_t i = 0; i < n; i++) out[i] = orc_f32_to_f16(x[i]); }
void orc_e4m3_to_f64_n(const uint8_t *c, double *out, int64_t n)
{ for (int64_t i = 0; i < n; i++) out[i] = orc_e4m3_to_f64(c[i]); }
void orc_f32_to_e4m3_n(const float *y, uint8_t *out, int64_t n)
{ for (int64_t i = 0; i < n; i++) out[i] = orc_f32_to_e4m3(y[i]); }
void orc_f32_to_i8_n(const float *y, int8_t *out, int64_t n)
{ for (int64_t i = 0; i < n; i++) out[i] = orc_f32_to_i8(y[i]); }
void orc_quantize_rows(const float *x, int64_t rows, int n, int kind, uint8_t *codes, uint16_t *scales)
{ for (int64_t r = 0; r < rows; r++) orc_quantize_row(x + r * n, n, kind, codes + r * n, scales + r); }
