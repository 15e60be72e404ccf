/*
 * kvrq_oracle.c -- plain CPU oracle for the rotated INT4 paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes, links
 * or calls this file; only the tests, the smoke check and the benchmark's
 * CPU baseline do.  It shares no code with the HIP path.
 *
 * What it computes (SAW-INT4, "System-Aware 4-Bit KV-Cache Quantization for
 * Real-World LLM Serving"):
 *
 *   write   K~ = quant(K H_blk), V~ = quant(V H_blk)
 *           (wispaper.ai blog, section 3 "method", the core formula; the
 *           backslash of \tilde is lost there, read as K-tilde / V-tilde).
 *           H_blk is block diagonal: the head dimension is cut into
 *           independent blocks of 16..128 channels, each rotated by a
 *           Hadamard matrix (same blog, section 2 "core intuition", the
 *           block-diagonal design bullet).  Quantisation is token-wise INT4
 *           (fugumt.com abstract; nervesearch.ai TL;DR), one group per
 *           (token, head, tensor), asymmetric, fp16 scale and fp16 zero.
 *
 *   decode  softmax attention of the query over the de-quantised cache.
 *           The query is rotated with the same H_blk so the rotated-space
 *           dot product equals the original one (wispaper.ai blog,
 *           section 3, third numbered consequence of the fusion).  V is
 *           stored rotated, so the attention output is rotated back once
 *           (H is symmetric and orthonormal, hence its own inverse).
 *
 * The write is an encoding, so it follows the steps one by one in fp32, in
 * a fixed order (the pages fix no order; this order is the reading used by
 * both sides):
 *   1. slot < 0: skip; page = slot / P, off = slot % P
 *   2. x_d = fp32(bf16 x_d)                                  (exact)
 *   3. per block of b channels: Walsh-Hadamard butterflies, stage width
 *      h = 1, 2, 4, ..., b/2, pair (i, i+h) -> (u+w, u-w); then y *= r_b,
 *      r_b = (float)(1 / sqrt((double)b)).  b = 0: no rotation.
 *   4. mn = min y, mx = max y; both + 0.0f so that -0 is stored as +0
 *   5. scale32 = (mx - mn) / 15.0f; s16 = fp16_rne(scale32); z16 = fp16_rne(mn)
 *   6. s16 == 0: all codes 0; else inv = 1.0f / s16,
 *      v = (y - z16) * inv, q = min(max(rint_even(v), 0), 15)
 *   7. byte i = q[2i] | q[2i+1] << 4
 *   8. codes at [page][Hkv][P][D/2], (s16, z16) at [page][Hkv][P][2]
 *
 * The 2-bit variant (an open question on the pages: wispaper.ai blog, section
 * 5, limitations) takes the same steps with 3 levels for 15 (scale32 =
 * (mx - mn) / 3.0f, q clamped to [0, 3]), four codes per byte (channel d at
 * bit 2 (d % 4) of byte d / 4) and D/4-byte rows.
 *
 * The decode has a plain definition and is computed in fp64 from it.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 * Floating point is IEEE binary32/binary64 with SSE (no x87 excess
 * precision on x86-64); contraction is disabled so that every operation
 * rounds on its own.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ---------------------------------------------------------------------- */
/* number formats, written from the IEEE 754 definitions                   */
/* ---------------------------------------------------------------------- */

ORACLE_API float kvrq_oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* binary16 bits -> binary32, exact. */
ORACLE_API float kvrq_oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1Fu;
    uint32_t m = h & 0x3FFu;
    uint32_t bits;
    if (e == 0) {
        /* zero or subnormal: m * 2^-24, exact in binary32 */
        float v = (float)m * 5.9604644775390625e-08f;
        memcpy(&bits, &v, 4);
        bits |= sign;
    } else if (e == 31) {
        bits = sign | 0x7F800000u | (m << 13);
    } else {
        bits = sign | ((e - 15u + 127u) << 23) | (m << 13);
    }
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* binary32 -> binary16 bits, round to nearest, ties to even; subnormal
 * results are kept, overflow goes to infinity. */
ORACLE_API uint16_t kvrq_oracle_f32_to_f16(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t exp = (x >> 23) & 0xFFu;
    uint32_t man = x & 0x7FFFFFu;
    if (exp == 0xFF)
        return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));
    int e = (int)exp - 127 + 15; /* biased binary16 exponent */
    if (e >= 31)
        return (uint16_t)(sign | 0x7C00u);
    uint32_t q, rem, half;
    if (e <= 0) {
        /* subnormal (or zero) result: value = m * 2^-24 with m = sig * 2^(e-14) */
        if (exp == 0)
            return (uint16_t)sign; /* binary32 subnormal: far below 2^-25 */
        uint32_t sig = man | 0x800000u;
        int shift = 14 - e; /* >= 14 */
        if (shift > 24)
            return (uint16_t)sign; /* < 2^-25: rounds to zero */
        q = sig >> shift;
        rem = sig & ((1u << shift) - 1u);
        half = 1u << (shift - 1);
    } else {
        q = ((uint32_t)e << 10) | (man >> 13);
        rem = man & 0x1FFFu;
        half = 0x1000u;
    }
    if (rem > half || (rem == half && (q & 1u)))
        q += 1u; /* a carry may move into the exponent, up to infinity */
    return (uint16_t)(sign | q);
}

/* r_b: the binary32 value of 1/sqrt(b) taken through binary64. */
ORACLE_API float kvrq_oracle_rb(int b)
{
    return (float)(1.0 / sqrt((double)b));
}

/* ---------------------------------------------------------------------- */
/* rotation                                                               */
/* ---------------------------------------------------------------------- */

/* In-place block-diagonal Walsh-Hadamard transform of n fp32 values with
 * block b, in the canonical stage order, then multiplied by r_b.  b = 0 (or
 * b = 1) leaves y unchanged.  n must be a multiple of b. */
ORACLE_API void kvrq_oracle_fwht_f32(float *y, int n, int b)
{
    if (b <= 1)
        return;
    const float r = kvrq_oracle_rb(b);
    for (int base = 0; base < n; base += b) {
        float *blk = y + base;
        for (int h = 1; h < b; h <<= 1) {
            for (int i = 0; i < b; ++i) {
                if (i & h)
                    continue;
                float u = blk[i];
                float w = blk[i + h];
                blk[i] = u + w;
                blk[i + h] = u - w;
            }
        }
        for (int i = 0; i < b; ++i)
            blk[i] = blk[i] * r;
    }
}

/* Exact rotation by its plain definition, in fp64:
 *   y_i = sum_k H[i][k] x_k,  H[i][k] = (-1)^popcount(i & k) / sqrt(b)
 * inside each block (Sylvester order).  b = 0 copies. */
ORACLE_API void kvrq_oracle_rotate_f64(const double *x, double *y, int n, int b)
{
    if (b <= 1) {
        for (int i = 0; i < n; ++i)
            y[i] = x[i];
        return;
    }
    const double r = 1.0 / sqrt((double)b);
    for (int base = 0; base < n; base += b) {
        for (int i = 0; i < b; ++i) {
            double acc = 0.0;
            for (int k = 0; k < b; ++k) {
                double s = (__builtin_popcount((unsigned)(i & k)) & 1) ? -1.0 : 1.0;
                acc += s * x[base + k];
            }
            y[base + i] = acc * r;
        }
    }
}

/* ---------------------------------------------------------------------- */
/* write                                                                   */
/* ---------------------------------------------------------------------- */

/* Steps 6 and 7 of the write for given parameters: the codes of the D rotated fp32 values
 * y under the binary16 scale s16 and zero z16 (s16 == +-0: all codes 0), packed as below.
 * quant_row calls it with the parameters it derives; a checker calls it with another
 * encoder's parameters to re-derive the codes those parameters imply.
 *   codes   D*bits/8 bytes; vpre optional, D fp32 pre-round values (0 when s16 == 0) */
ORACLE_API int kvrq_oracle_codes_from_params(const float *y, int D, int bits, uint16_t s16,
                                             uint16_t z16, uint8_t *codes, float *vpre)
{
    if (D > 1024 || D % 8 || (bits != 4 && bits != 2))
        return 1;
    const float levels = (float)((1 << bits) - 1);
    uint8_t q[1024];
    if ((s16 & 0x7FFFu) == 0) {
        for (int d = 0; d < D; ++d) {
            q[d] = 0;
            if (vpre)
                vpre[d] = 0.0f;
        }
    } else {
        const float sf = kvrq_oracle_f16_to_f32(s16);
        const float zf = kvrq_oracle_f16_to_f32(z16);
        const float inv = 1.0f / sf;
        for (int d = 0; d < D; ++d) {
            float t = y[d] - zf;
            float v = t * inv;
            float r = rintf(v);
            if (r < 0.0f)
                r = 0.0f;
            if (r > levels)
                r = levels;
            q[d] = (uint8_t)r;
            if (vpre)
                vpre[d] = v;
        }
    }
    for (int i = 0; i < D * bits / 8; ++i)
        codes[i] = 0;
    for (int d = 0; d < D; ++d)
        codes[d * bits / 8] |= (uint8_t)(q[d] << ((d * bits) % 8));
    return 0;
}

/* Quantise one row of D bf16 values with rotation block b to `bits` bits (4, or 2 for
 * the 2-bit variant the pages leave open: wispaper.ai blog, section 5, limitations).
 *   codes   D*bits/8 bytes; channel d sits at bit (d*bits) % 8 of byte d*bits/8
 *           (4 bits: the even channel in the low nibble)
 *   params  [0] = s16 bits, [1] = z16 bits
 *   vpre    optional, D fp32 pre-round values v (0 when s16 == 0)
 *   y_out   optional, D fp32 rotated values y
 * The steps are those of 4 bits with 2^bits - 1 levels in place of 15.
 * Returns 0, or 1 for a bad shape. */
ORACLE_API int kvrq_oracle_quant_row(const uint16_t *x, int D, int b, int bits, uint8_t *codes,
                                     uint16_t *params, float *vpre, float *y_out)
{
    float y[1024];
    if (D > 1024 || D % 8 || (b > 1 && D % b) || (bits != 4 && bits != 2))
        return 1;
    const float levels = (float)((1 << bits) - 1);
    for (int d = 0; d < D; ++d)
        y[d] = kvrq_oracle_bf16_to_f32(x[d]);
    kvrq_oracle_fwht_f32(y, D, b);

    float mn = y[0], mx = y[0];
    for (int d = 1; d < D; ++d) {
        if (y[d] < mn)
            mn = y[d];
        if (y[d] > mx)
            mx = y[d];
    }
    mn = mn + 0.0f;
    mx = mx + 0.0f;
    const float scale32 = (mx - mn) / levels;
    const uint16_t s16 = kvrq_oracle_f32_to_f16(scale32);
    const uint16_t z16 = kvrq_oracle_f32_to_f16(mn);
    params[0] = s16;
    params[1] = z16;
    kvrq_oracle_codes_from_params(y, D, bits, s16, z16, codes, vpre);
    if (y_out)
        for (int d = 0; d < D; ++d)
            y_out[d] = y[d];
    return 0;
}

/* Write T tokens of K and V into the paged cache.
 *   k, v          bf16 bits, token t head h at  k[t*k_stride + h*D]
 *   slots         [T], slot = page*P + off, < 0 = skip
 *   *_codes       uint8 [num_pages][Hkv][P][D*bits/8], bits = k_bits or v_bits (4 or 2)
 *   *_params      uint16 [num_pages][Hkv][P][2]
 *   k_vpre/v_vpre optional fp32 [T][Hkv][D] pre-round values
 * Returns 0, 1 for bad bit widths, or 2 for a slot outside the pool. */
ORACLE_API int kvrq_oracle_write(int T, int Hkv, int D, int P, int num_pages, int k_block,
                                 int v_block, int k_bits, int v_bits, const uint16_t *k,
                                 const uint16_t *v,
                                 int64_t k_stride, int64_t v_stride, const int32_t *slots,
                                 uint8_t *k_codes, uint8_t *v_codes, uint16_t *k_params,
                                 uint16_t *v_params, float *k_vpre, float *v_vpre)
{
    int bad = 0;
    if ((k_bits != 4 && k_bits != 2) || (v_bits != 4 && v_bits != 2))
        return 1;
    const int64_t rows = (int64_t)T * Hkv;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r) {
        const int t = (int)(r / Hkv);
        const int h = (int)(r % Hkv);
        const int32_t slot = slots[t];
        if (slot < 0)
            continue;
        const int64_t page = slot / P;
        const int64_t off = slot % P;
        if (page >= num_pages) {
            bad = 1;
            continue;
        }
        const int64_t cell = (page * Hkv + h) * P + off;
        for (int tensor = 0; tensor < 2; ++tensor) {
            const uint16_t *src = tensor == 0 ? k + (int64_t)t * k_stride + (int64_t)h * D
                                              : v + (int64_t)t * v_stride + (int64_t)h * D;
            const int bits = tensor == 0 ? k_bits : v_bits;
            uint8_t *dst_c = (tensor == 0 ? k_codes : v_codes) + cell * (D * bits / 8);
            uint16_t *dst_p = (tensor == 0 ? k_params : v_params) + cell * 2;
            float *vp = tensor == 0 ? k_vpre : v_vpre;
            if (vp)
                vp += ((int64_t)t * Hkv + h) * D;
            kvrq_oracle_quant_row(src, D, tensor == 0 ? k_block : v_block, bits, dst_c, dst_p, vp,
                                  NULL);
        }
    }
    return bad ? 2 : 0;
}

/* ---------------------------------------------------------------------- */
/* decode (fp64, plain definition)                                          */
/* ---------------------------------------------------------------------- */

/* Code of channel d in a row of `bits`-bit codes (the write's packing). */
static int code_at(const uint8_t *row, int d, int bits)
{
    return (row[d * bits / 8] >> ((d * bits) % 8)) & ((1 << bits) - 1);
}

/* Softmax attention of one query row over tokens 0..L-1 of KV head h of one
 * sequence, written from its definition (wispaper.ai blog, section 3: the query is
 * rotated by the K block matrix; V is stored rotated and the output is rotated back):
 *   q' = H_K q;  k_t = c_t s_t + z_t, v_t likewise (read from the stored codes and
 *   fp16 parameters at page_row[t / P], offset t % P);
 *   p_t = exp(sm_scale q'.k_t - max);  o = H_V (sum_t p_t v_t / sum_t p_t).
 * qrow: bf16 bits [D]; o: fp64 [D]; L <= 0 gives zeros.  Returns 1 when a page id is
 * outside the pool (those tokens are left out). */
static int attend_row(const uint16_t *qrow, int L, const int32_t *page_row, int h, int Hkv,
                      int D, int P, int num_pages, int k_block, int v_block, int k_bits,
                      int v_bits, double sm_scale,
                      const uint8_t *k_codes, const uint8_t *v_codes,
                      const uint16_t *k_params, const uint16_t *v_params, double *o)
{
    double qx[1024], qr[1024], acc[1024], kh[1024];
    int bad = 0;
    for (int d = 0; d < D; ++d)
        acc[d] = 0.0;
    if (L <= 0) {
        for (int d = 0; d < D; ++d)
            o[d] = 0.0;
        return 0;
    }
    for (int d = 0; d < D; ++d)
        qx[d] = (double)kvrq_oracle_bf16_to_f32(qrow[d]);
    kvrq_oracle_rotate_f64(qx, qr, D, k_block);

    double *score = (double *)malloc(sizeof(double) * (size_t)L);
    double m = -INFINITY;
    for (int t = 0; t < L; ++t) {
        const int32_t page = page_row[t / P];
        if (page < 0 || page >= num_pages) {
            bad = 1;
            score[t] = -INFINITY;
            continue;
        }
        const int64_t cell = ((int64_t)page * Hkv + h) * P + t % P;
        const double sc = kvrq_oracle_f16_to_f32(k_params[cell * 2 + 0]);
        const double zr = kvrq_oracle_f16_to_f32(k_params[cell * 2 + 1]);
        const uint8_t *c = k_codes + cell * (D * k_bits / 8);
        for (int d = 0; d < D; ++d) {
            const int code = code_at(c, d, k_bits);
            kh[d] = code * sc + zr;
        }
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += qr[d] * kh[d];
        score[t] = sm_scale * dot;
        if (score[t] > m)
            m = score[t];
    }
    double l = 0.0;
    for (int t = 0; t < L; ++t) {
        const double p = exp(score[t] - m);
        l += p;
        const int32_t page = page_row[t / P];
        if (page < 0 || page >= num_pages)
            continue;
        const int64_t cell = ((int64_t)page * Hkv + h) * P + t % P;
        const double sc = kvrq_oracle_f16_to_f32(v_params[cell * 2 + 0]);
        const double zr = kvrq_oracle_f16_to_f32(v_params[cell * 2 + 1]);
        const uint8_t *c = v_codes + cell * (D * v_bits / 8);
        for (int d = 0; d < D; ++d) {
            const int code = code_at(c, d, v_bits);
            acc[d] += p * (code * sc + zr);
        }
    }
    free(score);
    for (int d = 0; d < D; ++d)
        acc[d] /= l;
    kvrq_oracle_rotate_f64(acc, o, D, v_block);
    return bad;
}

/* Attention of S sequences x Hq query heads over the de-quantised cache.
 *   q           bf16 bits [S][Hq][D]
 *   page_table  int32 [S][max_pages]
 *   seq_lens    int32 [S]; tokens 0..L-1 are attended
 *   sm_scale    softmax scale (<= 0: 1/sqrt(D))
 *   k_bits, v_bits  code widths of the two pools (4, or 2)
 *   out         fp64 [S][Hq][D]; an empty sequence yields zeros
 * Query head g reads KV head g / (Hq/Hkv).  Returns 0, 1 for bad shapes,
 * 2 for a page id outside the pool. */
ORACLE_API int kvrq_oracle_decode(int S, int Hq, int Hkv, int D, int P, int num_pages,
                                  int k_block, int v_block, int k_bits, int v_bits,
                                  const uint16_t *q,
                                  const int32_t *page_table, int max_pages,
                                  const int32_t *seq_lens, double sm_scale,
                                  const uint8_t *k_codes, const uint8_t *v_codes,
                                  const uint16_t *k_params, const uint16_t *v_params,
                                  double *out)
{
    if (Hkv <= 0 || Hq % Hkv || D > 1024 || (k_bits != 4 && k_bits != 2) ||
        (v_bits != 4 && v_bits != 2))
        return 1;
    const int G = Hq / Hkv;
    if (sm_scale <= 0.0)
        sm_scale = 1.0 / sqrt((double)D);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t sg = 0; sg < (int64_t)S * Hq; ++sg) {
        const int s = (int)(sg / Hq);
        const int g = (int)(sg % Hq);
        bad |= attend_row(q + sg * D, seq_lens[s], page_table + (int64_t)s * max_pages, g / G,
                          Hkv, D, P, num_pages, k_block, v_block, k_bits, v_bits, sm_scale,
                          k_codes, v_codes, k_params, v_params, out + sg * D);
    }
    return bad ? 2 : 0;
}

/* Extend (chunked prefill) attention over the paged cache: sequence s holds seq_lens[s]
 * tokens, the last n_s = qo_start[s + 1] - qo_start[s] of which are the new chunk with
 * one query row each.  Row i of the chunk sits at position p = seq_lens[s] - n_s + i and
 * attends causally over tokens 0..p, i.e. it is the decode of a sequence of p + 1
 * tokens.
 *   q           bf16 bits [total_q][Hq][D], total_q = qo_start[S]
 *   qo_start    int32 [S + 1], non-decreasing, qo_start[0] = 0
 *   out         fp64 [total_q][Hq][D]
 * Returns 0, 1 for bad shapes (including n_s > seq_lens[s]), 2 for a page id outside
 * the pool. */
ORACLE_API int kvrq_oracle_extend(int S, int Hq, int Hkv, int D, int P, int num_pages,
                                  int k_block, int v_block, int k_bits, int v_bits,
                                  const uint16_t *q,
                                  const int32_t *qo_start, const int32_t *page_table,
                                  int max_pages, const int32_t *seq_lens, double sm_scale,
                                  const uint8_t *k_codes, const uint8_t *v_codes,
                                  const uint16_t *k_params, const uint16_t *v_params,
                                  double *out)
{
    if (Hkv <= 0 || Hq % Hkv || D > 1024 || qo_start[0] != 0 || (k_bits != 4 && k_bits != 2) ||
        (v_bits != 4 && v_bits != 2))
        return 1;
    for (int s = 0; s < S; ++s) {
        const int n = qo_start[s + 1] - qo_start[s];
        if (n < 0 || n > seq_lens[s])
            return 1;
    }
    const int G = Hq / Hkv;
    if (sm_scale <= 0.0)
        sm_scale = 1.0 / sqrt((double)D);
    const int64_t total_q = qo_start[S];
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t rg = 0; rg < total_q * Hq; ++rg) {
        const int64_t r = rg / Hq;
        const int g = (int)(rg % Hq);
        int s = 0;
        while (qo_start[s + 1] <= r)
            ++s;
        const int n = qo_start[s + 1] - qo_start[s];
        const int len = seq_lens[s] - n + (int)(r - qo_start[s]) + 1;
        bad |= attend_row(q + rg * D, len, page_table + (int64_t)s * max_pages, g / G, Hkv, D, P,
                          num_pages, k_block, v_block, k_bits, v_bits, sm_scale, k_codes,
                          v_codes, k_params, v_params, out + rg * D);
    }
    return bad ? 2 : 0;
}
