/*
 * kvq_oracle.c -- reference CPU implementation of the 2-bit mixed-precision
 * KV cache: quantize, pack, unpack, dequantize and decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this library; the product library never does, and
 * this file shares no code, header or table with it.
 *
 * Everything here is written as plain loops that follow the definitions, with
 * no blocking, fusion or reordering.  Where a floating-point step decides an
 * integer (a quantized code) it is done in IEEE single precision, one
 * round-to-nearest-even operation at a time (build with -ffp-contract=off, no
 * fast-math).  Attention is computed in double precision.
 *
 * What is computed, and where the pages state it:
 *  - KIVI explainer (aibr.jp, "KIVI: tuning-free asymmetric 2-bit KV cache
 *    quantization"), section 3 (core technical elements): Keys are quantized
 *    per channel, Values per token, with asymmetric (zero-point) quantization
 *    and a full-precision residual part; new tokens are appended in a
 *    streaming fashion.
 *  - MiniKV summary (f-binder), "proposed method": Keys are quantized in small
 *    groups with a range per channel, because Keys have channel outliers;
 *    Values per token.  "Problem setting": keep the attention output close to
 *    the unquantized one.
 *  - Kitty abstract (fugumt, arXiv 2511.18643): Key channels are ranked and a
 *    small fraction is kept at higher (4-bit) precision, per page and at run
 *    time; each mixed-precision Key page is split into two tensors of uniform
 *    2-bit precision; the layout is page-centric.
 *  - notes.yuuk.io "KV cache quantization", open questions: the channel
 *    selection is a magnitude heuristic; boost ratios are 12.5 % and 25 %;
 *    one Key head is shared by several query heads (GQA).
 *
 * Readings of points the pages leave open:
 *  R1  page = 128 consecutive tokens of one (sequence, KV head); Key groups
 *      are tokens [32g, 32g+32) of a page; Value groups are channels
 *      [32h, 32h+32) of one token; the residual window holds 128 tokens.
 *  R2  quantizer Q(x; L): m = min, M = max; z = m (a zero minimum stored as
 *      +0); s = dtype_rne(fp32((M - m) / L)); if s == 0 all codes are 0, else
 *      code = clamp(rint_even((x - z) * fp32(1 / s)), 0, L).
 *  R3  channel score = max |K| over the page's tokens, compared through the
 *      sign-cleared bit pattern; ties go to the lower channel index; the k
 *      highest scores are boosted; their list is stored in ascending order.
 *  R4  boosted channels use L = 15 over the same 32-token groups; the 4-bit
 *      code is split into a lo plane (code & 3, all channels, natural
 *      position) and a hi plane (code >> 2, boosted channels only, column j =
 *      j-th boosted channel); code = 4 * hi + lo.
 *  R5  scale and zero are stored in the KV dtype.
 *  R6  byte layout: see the page-layout section below.
 *  R7  the residual window keeps K and V bit-exact; append flushes a full
 *      window into a page before inserting (flush-before-insert).
 *  R8  attention: softmax(scale * q . k) over every page token (dequantized)
 *      and every residual token (exact), no mask, scale = 1/sqrt(128) unless
 *      given; query head hq reads KV head hq / (Hq / Hkv).
 *  R18 query-aware channel ranking (MixKVQ abstract, fugumt, arXiv
 *      2512.19206: a Key channel needs high precision according to its
 *      intrinsic quantization difficulty and its relevance to the query).
 *      Difficulty of channel c on a page = the sum of its four Key-group
 *      ranges, (r0 + r1) + (r2 + r3) with r_g = fp32(max - min) over the
 *      group's 32 tokens; relevance rel_c >= 0 is supplied per (sequence, KV
 *      head); score = |fp32(difficulty * rel)|; ties go to the lower channel.
 *      The relevance of a query is the sum over the query heads that share
 *      the KV head of |q_c|, in fp32, heads in ascending order.
 *  R20 prefill attention (MiniKV summary, "proposed method": the prefill
 *      processes the whole input; a two-stage selective flash-attention
 *      yields the attention output and the cumulative attention scores in
 *      linear memory) is causal: query position i attends to key positions
 *      j <= i; query head hq reads KV head hq / (Hq / Hkv); scale as R8.
 *  R21 cumulative score of key position j for KV head h: the sum, over the
 *      query heads of h and over the query positions i >= j, of the softmax
 *      probability P[i][j] (the accumulated attention the heavy-hitter
 *      selection ranks by).
 *  R22 token selection (same section: heavy hitters and a recent window are
 *      kept, 25 % of the budget each by default): the last `recent`
 *      positions are kept; of the others, the `heavy` positions of largest
 *      score, ties to the lower position; the kept list is ascending.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define D 128 /* head dimension */
#define P 128 /* tokens per page */
#define GK 32 /* tokens per Key group */
#define GV 32 /* channels per Value group */
#define R 128 /* residual window length */

enum { DT_F16 = 0, DT_BF16 = 1 };

/* ORA_PLANT = n > 0 builds a copy with mistake n planted, so the tests can
   show that their pins catch it.  The oracle proper is built with 0. */
#ifndef ORA_PLANT
#define ORA_PLANT 0
#endif

/* ------------------------------------------------------------------------
 * Storage dtypes.  IEEE 754 binary16 (10 mantissa bits, 5 exponent bits) and
 * bfloat16 (7 mantissa bits, 8 exponent bits), decoded exactly and encoded
 * with one round-to-nearest-even step, written from the format definitions.
 * ---------------------------------------------------------------------- */
static int mant_bits(int dt) { return dt == DT_F16 ? 10 : 7; }
static int exp_bits(int dt) { return dt == DT_F16 ? 5 : 8; }

double ora_decode(int dt, uint16_t h) {
    int mb = mant_bits(dt), eb = exp_bits(dt);
    int bias = (1 << (eb - 1)) - 1;
    int ef = (h >> mb) & ((1 << eb) - 1);
    int mant = h & ((1 << mb) - 1);
    double v;
    if (ef == 0)
        v = ldexp((double)mant, 1 - bias - mb); /* zero or subnormal */
    else if (ef == (1 << eb) - 1)
        v = mant ? NAN : INFINITY;
    else
        v = ldexp((double)((1 << mb) + mant), ef - bias - mb);
    return (h & 0x8000) ? -v : v;
}

uint16_t ora_encode(int dt, double x) {
    int mb = mant_bits(dt), eb = exp_bits(dt);
    int bias = (1 << (eb - 1)) - 1, emin = 1 - bias;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    uint16_t inf = (uint16_t)(((1 << eb) - 1) << mb);
    double a = fabs(x);
    if (isnan(x)) return sign | inf | (uint16_t)(1 << (mb - 1));
    if (isinf(x)) return sign | inf;
    if (a < ldexp(1.0, emin)) {
        /* subnormal range: a multiple of 2^(emin - mb); rounding up to
           2^mb units gives exactly the smallest normal's bit pattern */
        double m = nearbyint(ldexp(a, mb - emin));
        return sign | (uint16_t)m;
    }
    int ex;
    double fr = frexp(a, &ex); /* a = fr * 2^ex, fr in [0.5, 1) */
    int e = ex - 1;            /* a = (2 fr) * 2^e, 2 fr in [1, 2) */
    double m = nearbyint((2.0 * fr - 1.0) * (double)(1 << mb));
    if (m == (double)(1 << mb)) {
        m = 0.0;
        e += 1;
    }
    if (e > bias) return sign | inf; /* overflow rounds to infinity */
    return sign | (uint16_t)(((e + bias) << mb) | (int)m);
}

/* Decode a stored value to single precision (exact: both formats are subsets
   of binary32). */
static float dec32(int dt, uint16_t h) { return (float)ora_decode(dt, h); }

/* ------------------------------------------------------------------------
 * R2: one asymmetric min/max group (KIVI explainer, section 3).
 * x[i * stride], i < n, are the group's stored values; codes go to
 * code[i * code_stride].
 * ---------------------------------------------------------------------- */
void ora_quantize_group(int dt, const uint16_t *x, int n, int stride, int L,
                        uint16_t *s_out, uint16_t *z_out, uint8_t *code,
                        int code_stride) {
    float lo = dec32(dt, x[0]), hi = lo;
    for (int i = 1; i < n; i++) {
        float v = dec32(dt, x[(size_t)i * stride]);
        if (v < lo) lo = v;
        if (v > hi) hi = v;
    }
    lo = lo + 0.0f; /* a zero minimum is stored as +0 */
    float range = hi - lo;
    float s32 = range / (float)(ORA_PLANT == 13 ? L + 1 : L);
    uint16_t s = ora_encode(dt, s32);
    uint16_t z = ora_encode(dt, lo); /* exact: lo is a stored value */
    float sf = dec32(dt, s), zf = dec32(dt, z);
    *s_out = s;
    *z_out = z;
    if (sf == 0.0f) {
        for (int i = 0; i < n; i++) code[(size_t)i * code_stride] = 0;
        return;
    }
    float inv = 1.0f / sf;
    for (int i = 0; i < n; i++) {
        float v = dec32(dt, x[(size_t)i * stride]);
        float d = v - zf;
        float t = d * inv;
        float r = ORA_PLANT == 5 ? floorf(t) : rintf(t); /* round half to even */
        if (r < 0.0f) r = 0.0f;
        if (r > (float)L) r = (float)L;
        code[(size_t)i * code_stride] = (uint8_t)r;
    }
}

/* n independent groups of glen contiguous values each (group i at
   x[i * glen]), quantized one after another with the quantizer above: scale
   and zero of group i in s_out[i], z_out[i], its codes at code[i * glen]. */
void ora_quantize_groups(int dt, const uint16_t *x, int n, int glen, int L,
                         uint16_t *s_out, uint16_t *z_out, uint8_t *code) {
    for (int i = 0; i < n; i++)
        ora_quantize_group(dt, x + (size_t)i * glen, glen, 1, ORA_PLANT == 22 ? 3 : L, s_out + i,
                           z_out + i, code + (size_t)i * glen, 1); /* plant: L ignored */
}

/* ------------------------------------------------------------------------
 * R3: magnitude-ranked channel selection (Kitty abstract; notes.yuuk.io open
 * questions).  K is [ntok][nch] stored values.  boosted[c] = 1 for the k
 * chosen channels; idx[0..k) lists them in ascending order.
 * ---------------------------------------------------------------------- */
void ora_select_channels(const uint16_t *K, int ntok, int nch, int k,
                         uint8_t *boosted, uint8_t *idx) {
    uint32_t *key = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)nch);
    for (int c = 0; c < nch; c++) {
        uint32_t m = 0;
        for (int t = 0; t < ntok; t++) {
            uint32_t a = K[(size_t)t * nch + c] & 0x7FFFu; /* |K| as bits */
            if (ORA_PLANT == 10 ? (t == 0 || a < m) : a > m) m = a;
        }
        key[c] = (m << 8) | (uint32_t)(ORA_PLANT == 2 ? c : 255 - c); /* lower channel wins ties */
    }
    int j = 0;
    for (int c = 0; c < nch; c++) {
        int rank = 0; /* number of channels with a strictly larger key */
        for (int c2 = 0; c2 < nch; c2++)
            if (key[c2] > key[c]) rank++;
        boosted[c] = (uint8_t)(rank < k);
    }
    for (int c = 0; c < nch; c++)
        if (boosted[c]) idx[j++] = (uint8_t)c;
    free(key);
}

/* ------------------------------------------------------------------------
 * R18: query-aware channel selection.  K is one page [P][D] of stored values
 * of dtype dt; rel[D] the channel relevance.  Outputs as ora_select_channels.
 * ---------------------------------------------------------------------- */
void ora_select_channels_rel(int dt, const uint16_t *K, const float *rel, int k,
                             uint8_t *boosted, uint8_t *idx) {
    uint64_t key[D];
    for (int c = 0; c < D; c++) {
        float r[P / GK];
        for (int g = 0; g < P / GK; g++) {
            float lo = dec32(dt, K[(size_t)g * GK * D + c]), hi = lo;
            for (int t = 1; t < GK; t++) {
                float v = dec32(dt, K[(size_t)(g * GK + t) * D + c]);
                if (v < lo) lo = v;
                if (v > hi) hi = v;
            }
            r[g] = hi - lo;
        }
        float diff = ORA_PLANT == 15 ? fmaxf(fmaxf(r[0], r[1]), fmaxf(r[2], r[3]))
                                     : (r[0] + r[1]) + (r[2] + r[3]);
        float score = fabsf(ORA_PLANT == 14 ? diff : diff * rel[c]);
        uint32_t bits;
        memcpy(&bits, &score, sizeof bits);
        key[c] = ((uint64_t)bits << 8) | (uint64_t)(255 - c); /* lower channel wins ties */
    }
    int j = 0;
    for (int c = 0; c < D; c++) {
        int rank = 0;
        for (int c2 = 0; c2 < D; c2++)
            if (key[c2] > key[c]) rank++;
        boosted[c] = (uint8_t)(rank < k);
    }
    for (int c = 0; c < D; c++)
        if (boosted[c]) idx[j++] = (uint8_t)c;
}

/* R18: relevance of a query batch, rel[b][h][c] = sum over the g = Hq / Hkv
   query heads h g + j (j ascending) of |q[b][h g + j][c]|, in fp32. */
void ora_query_relevance(int dt, int B, int Hq, int Hkv, const uint16_t *q, float *rel) {
    int g = Hq / Hkv;
    for (int b = 0; b < B; b++)
        for (int h = 0; h < Hkv; h++)
            for (int c = 0; c < D; c++) {
                float acc = 0.0f;
                for (int j = 0; j < g; j++) {
                    float a = fabsf(dec32(dt, q[((size_t)b * Hq + h * g + j) * D + c]));
                    acc = ORA_PLANT == 16 ? fmaxf(acc, a) : acc + a;
                }
                rel[((size_t)b * Hkv + h) * D + c] = acc;
            }
}

/* ------------------------------------------------------------------------
 * R6: page layout.  One page (128 tokens of one sequence and KV head) is one
 * contiguous blob of segments, in this order, each starting on 16 bytes:
 *   K_lo    [P][D/4]   2-bit lo plane of every Key channel, token-major
 *   K_hi    [P][k/4]   2-bit hi plane of the k boosted channels, token-major
 *   K_scale [P/GK][D]  dtype
 *   K_zero  [P/GK][D]  dtype
 *   K_idx   k bytes    boosted channel ids, ascending, zero-padded to 16 B
 *   V_codes            2-bit Value codes, 1024 B per 32-token step, see below
 *   V_scale [D/GV][P]  dtype, group-major
 *   V_zero  [D/GV][P]  dtype
 * 2-bit fields are little-endian: bit b of a segment is bit (b % 8) of byte
 * (b / 8).  K_lo: element (t, c) at bit 2 (t D + c).  K_hi: (t, j) at bit
 * 2 (t k + j).  V_codes: token t, channel c at
 *   step s = t / 32, u = t % 32, r = u % 16, G = r / 4,
 *   word w = 2 (u / 16) + (r % 4) / 2, half = (r % 4) % 2,
 *   byte = 1024 s + 16 (16 G + c % 16) + 4 w, bit = 8 byte + 16 half + 2 (c / 16)
 * i.e. every 16-byte block holds the codes of one channel column (c % 16)
 * for eight tokens and all eight 16-channel tiles, two tokens per 32-bit word.
 * ---------------------------------------------------------------------- */
typedef struct {
    size_t klo, khi, ks, kz, kidx, vc, vs, vz, total;
} layout_t;

static size_t round16(size_t x) { return (x + 15) / 16 * 16; }

static layout_t layout_of(int k) {
    layout_t L;
    size_t o = 0;
    L.klo = o; o += round16((size_t)P * D / 4);
    L.khi = o; o += round16((size_t)P * k / 4);
    L.ks = o;  o += round16((size_t)(P / GK) * D * 2);
    L.kz = o;  o += round16((size_t)(P / GK) * D * 2);
    L.kidx = o; o += round16((size_t)k);
    L.vc = o;  o += round16((size_t)P * D / 4);
    L.vs = o;  o += round16((size_t)(D / GV) * P * 2);
    L.vz = o;  o += round16((size_t)(D / GV) * P * 2);
    L.total = o;
    return L;
}

size_t ora_page_bytes(int k) { return layout_of(k).total; }

/* segment offsets, for tests: klo khi ks kz kidx vc vs vz total */
void ora_page_layout(int k, int64_t *out9) {
    layout_t L = layout_of(k);
    size_t v[9] = {L.klo, L.khi, L.ks, L.kz, L.kidx, L.vc, L.vs, L.vz, L.total};
    for (int i = 0; i < 9; i++) out9[i] = (int64_t)v[i];
}

static size_t klo_bit(int t, int c) { return 2 * ((size_t)t * D + c); }
static size_t khi_bit(int k, int t, int j) { return 2 * ((size_t)t * k + j); }
size_t ora_vcode_bit(int t, int c) {
    int s = t / 32, u = t % 32, r = u % 16, G = r / 4;
    int w = 2 * (u / 16) + (r % 4) / 2, half = (r % 4) % 2;
    size_t byte = (size_t)1024 * s + 16 * (size_t)(16 * G + c % 16) + 4 * (size_t)w;
    return 8 * byte + 16 * (size_t)half + 2 * (size_t)(c / 16);
}
size_t ora_klo_bit(int t, int c) { return klo_bit(t, c); }
size_t ora_khi_bit(int k, int t, int j) { return khi_bit(k, t, j); }

static void put2(uint8_t *seg, size_t bit, unsigned v) {
    seg[bit / 8] |= (uint8_t)((v & 3u) << (bit % 8));
}
static unsigned get2(const uint8_t *seg, size_t bit) {
    return (seg[bit / 8] >> (bit % 8)) & 3u;
}
static void put16(uint8_t *seg, size_t i, uint16_t v) {
    seg[2 * i] = (uint8_t)(v & 0xFF);
    seg[2 * i + 1] = (uint8_t)(v >> 8);
}
static uint16_t get16(const uint8_t *seg, size_t i) {
    return (uint16_t)(seg[2 * i] | (seg[2 * i + 1] << 8));
}

/* ------------------------------------------------------------------------
 * Quantize one page (R1-R6).  Kp, Vp: [P][D] stored values of one sequence
 * and KV head.  page: ora_page_bytes(k) bytes.  Optional outputs (may be
 * NULL): kcode[P][D] (4-bit code for boosted channels, 2-bit otherwise) and
 * vcode[P][D], taken before packing.
 * ---------------------------------------------------------------------- */
static int quantize_page_sel(int dt, int k, const uint16_t *Kp, const uint16_t *Vp,
                             const float *rel, uint8_t *page, uint8_t *kcode_out,
                             uint8_t *vcode_out) {
    if (k < 0 || k > D || k % 4) return -1;
    layout_t L = layout_of(k);
    memset(page, 0, L.total);
    uint8_t boosted[D], idx[D];
    if (rel)
        ora_select_channels_rel(dt, Kp, rel, k, boosted, idx);
    else
        ora_select_channels(Kp, P, D, k, boosted, idx);

    uint8_t kcode[P * D], vcode[P * D];
    /* Keys: per channel, per 32-token group (R2, R4) */
    for (int g = 0; g < P / GK; g++)
        for (int c = 0; c < D; c++) {
            uint16_t s, z;
            ora_quantize_group(dt, Kp + (size_t)g * GK * D + c, GK, D,
                               boosted[c] && ORA_PLANT != 1 ? 15 : 3, &s, &z,
                               kcode + (size_t)g * GK * D + c, D);
            put16(page + L.ks, (size_t)g * D + c, s);
            put16(page + L.kz, (size_t)g * D + c, z);
        }
    /* Values: per token, per 32-channel group (R1, R2) */
    for (int t = 0; t < P; t++)
        for (int h = 0; h < D / GV; h++) {
            uint16_t s, z;
            if (ORA_PLANT == 11 && t < GV) /* Value groups along tokens */
                ora_quantize_group(dt, Vp + (size_t)t * D + h * GV, GV, D, 3, &s, &z,
                                   vcode + (size_t)t * D + h * GV, D);
            else
                ora_quantize_group(dt, Vp + (size_t)t * D + h * GV, GV, 1, 3, &s, &z,
                                   vcode + (size_t)t * D + h * GV, 1);
            put16(page + L.vs, (size_t)h * P + t, s);
            put16(page + L.vz, (size_t)h * P + t, z);
        }
    /* Two uniform 2-bit Key planes (R4) */
    for (int t = 0; t < P; t++) {
        int j = 0;
        for (int c = 0; c < D; c++) {
            unsigned code = kcode[(size_t)t * D + c];
            put2(page + L.klo, klo_bit(t, c), ORA_PLANT == 3 && boosted[c] ? code >> 2 : code & 3u);
            if (boosted[c]) {
                put2(page + L.khi, khi_bit(k, t, j), ORA_PLANT == 3 ? code & 3u : code >> 2);
                j++;
            }
        }
    }
    for (int j = 0; j < k; j++) page[L.kidx + j] = idx[j];
    for (int t = 0; t < P; t++)
        for (int c = 0; c < D; c++)
            put2(page + L.vc, ora_vcode_bit(t, c), vcode[(size_t)t * D + c]);
    if (kcode_out) memcpy(kcode_out, kcode, sizeof kcode);
    if (vcode_out) memcpy(vcode_out, vcode, sizeof vcode);
    return 0;
}

int ora_quantize_page(int dt, int k, const uint16_t *Kp, const uint16_t *Vp,
                      uint8_t *page, uint8_t *kcode_out, uint8_t *vcode_out) {
    return quantize_page_sel(dt, k, Kp, Vp, NULL, page, kcode_out, vcode_out);
}

/* The same page with the query-aware selection (R18); rel: [D] relevance. */
int ora_quantize_page_rel(int dt, int k, const uint16_t *Kp, const uint16_t *Vp,
                          const float *rel, uint8_t *page, uint8_t *kcode_out,
                          uint8_t *vcode_out) {
    return quantize_page_sel(dt, k, Kp, Vp, rel, page, kcode_out, vcode_out);
}

/* ------------------------------------------------------------------------
 * Read a page back: codes (4-bit Key code = 4 hi + lo), metadata, index.
 * Any output may be NULL.  ks, kz: [P/GK][D] stored bits; vs, vz: [D/GV][P].
 * ---------------------------------------------------------------------- */
int ora_unpack_page(int dt, int k, const uint8_t *page, uint8_t *kcode,
                    uint8_t *klo, uint8_t *khi, uint8_t *vcode, uint16_t *ks,
                    uint16_t *kz, uint16_t *vs, uint16_t *vz, uint8_t *idx) {
    (void)dt;
    if (k < 0 || k > D || k % 4) return -1;
    layout_t L = layout_of(k);
    int col[D]; /* hi-plane column of each channel, -1 if not boosted */
    for (int c = 0; c < D; c++) col[c] = -1;
    for (int j = 0; j < k; j++) {
        int c = page[L.kidx + j];
        col[c] = j;
        if (idx) idx[j] = (uint8_t)c;
    }
    for (int t = 0; t < P; t++)
        for (int c = 0; c < D; c++) {
            unsigned lo = get2(page + L.klo, klo_bit(t, c));
            unsigned hi = col[c] >= 0 ? get2(page + L.khi, khi_bit(k, t, col[c])) : 0;
            if (klo) klo[(size_t)t * D + c] = (uint8_t)lo;
            if (kcode) kcode[(size_t)t * D + c] = (uint8_t)(4 * hi + lo);
            if (vcode) vcode[(size_t)t * D + c] = (uint8_t)get2(page + L.vc, ora_vcode_bit(t, c));
        }
    if (khi)
        for (int t = 0; t < P; t++)
            for (int j = 0; j < k; j++)
                khi[(size_t)t * k + j] = (uint8_t)get2(page + L.khi, khi_bit(k, t, j));
    for (size_t i = 0; i < (size_t)(P / GK) * D; i++) {
        if (ks) ks[i] = get16(page + L.ks, i);
        if (kz) kz[i] = get16(page + L.kz, i);
    }
    for (size_t i = 0; i < (size_t)(D / GV) * P; i++) {
        if (vs) vs[i] = get16(page + L.vs, i);
        if (vz) vz[i] = get16(page + L.vz, i);
    }
    return 0;
}

/* Dequantize one page to double: xhat = code * s + z (R2).  Kh, Vh: [P][D]. */
int ora_dequantize_page(int dt, int k, const uint8_t *page, double *Kh, double *Vh) {
    uint8_t kcode[P * D], vcode[P * D];
    uint16_t ks[(P / GK) * D], kz[(P / GK) * D], vs[(D / GV) * P], vz[(D / GV) * P];
    if (ora_unpack_page(dt, k, page, kcode, NULL, NULL, vcode, ks, kz, vs, vz, NULL))
        return -1;
    for (int t = 0; t < P; t++)
        for (int c = 0; c < D; c++) {
            size_t km = (size_t)((ORA_PLANT == 6 ? (t + 1) % P : t) / GK) * D + c;
            size_t vm = (size_t)(c / GV) * P + t;
            Kh[(size_t)t * D + c] = kcode[(size_t)t * D + c] * ora_decode(dt, ks[km]) + ora_decode(dt, kz[km]);
            Vh[(size_t)t * D + c] = vcode[(size_t)t * D + c] * ora_decode(dt, vs[vm]) +
                                    (ORA_PLANT == 4 ? 0.0 : ora_decode(dt, vz[vm]));
        }
    return 0;
}

/* ------------------------------------------------------------------------
 * R8: decode attention in double precision over one cache.
 * pages: byte (((b Hkv + h) max_pages + p) page_bytes); kres, vres:
 * [B][Hkv][R][D] stored values (the first n_res rows are live); q:
 * [B][Hq][D] stored values; out: [B][Hq][D] doubles.  Only (b, h) units
 * u = b Hkv + h with u0 <= u < u1 are computed.
 * ---------------------------------------------------------------------- */
int ora_attention(int dt, int k, int B, int Hq, int Hkv, int max_pages,
                  int n_pages, int n_res, const uint8_t *pages,
                  const uint16_t *kres, const uint16_t *vres, const uint16_t *q,
                  double scale, double *out, int u0, int u1) {
    if (Hkv <= 0 || Hq % Hkv || n_pages < 0 || n_pages > max_pages || n_res < 0 ||
        n_res > R || n_pages * P + n_res == 0)
        return -1;
    int g = Hq / Hkv;
    size_t pb = ora_page_bytes(k);
    size_t T = (size_t)n_pages * P + (size_t)n_res;
    if (u0 < 0) u0 = 0;
    if (u1 > B * Hkv) u1 = B * Hkv;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = u0; u < u1; u++) {
        int b = u / Hkv, h = u % Hkv;
        double *Kh = (double *)malloc(sizeof(double) * T * D);
        double *Vh = (double *)malloc(sizeof(double) * T * D);
        double *sc = (double *)malloc(sizeof(double) * T);
        if (!Kh || !Vh || !sc) {
            err = -2;
            free(Kh); free(Vh); free(sc);
            continue;
        }
        for (int p = 0; p < n_pages; p++) {
            const uint8_t *pg = pages + ((size_t)u * max_pages + p) * pb;
            ora_dequantize_page(dt, k, pg, Kh + (size_t)p * P * D, Vh + (size_t)p * P * D);
        }
        for (int t = 0; t < n_res; t++)
            for (int c = 0; c < D; c++) {
                if (ORA_PLANT == 9 && t == n_res - 1) { /* newest token dropped */
                    Kh[((size_t)n_pages * P + t) * D + c] = -1e300;
                    Vh[((size_t)n_pages * P + t) * D + c] = 0.0;
                    continue;
                }
                size_t src = (((size_t)u * R) + t) * D + c;
                size_t dst = ((size_t)n_pages * P + t) * D + c;
                Kh[dst] = ora_decode(dt, kres[src]);
                Vh[dst] = ora_decode(dt, vres[src]);
            }
        for (int j = 0; j < g; j++) {
            int hq = h * g + j;
            int hsrc = ORA_PLANT == 7 ? (j * Hkv + h) % Hq : hq; /* strided head map */
            const uint16_t *qv = q + ((size_t)b * Hq + hsrc) * D;
            double qd[D];
            for (int c = 0; c < D; c++) qd[c] = ora_decode(dt, qv[c]);
            double m = -INFINITY;
            for (size_t t = 0; t < T; t++) {
                double s = 0.0;
                for (int c = 0; c < D; c++) s += qd[c] * Kh[t * D + c];
                sc[t] = (ORA_PLANT == 8 ? 1.0 : scale) * s;
                if (sc[t] > m) m = sc[t];
            }
            double l = 0.0, o[D];
            for (int c = 0; c < D; c++) o[c] = 0.0;
            for (size_t t = 0; t < T; t++) {
                double w = exp(sc[t] - m);
                l += w;
                for (int c = 0; c < D; c++) o[c] += w * Vh[t * D + c];
            }
            for (int c = 0; c < D; c++) out[((size_t)b * Hq + hq) * D + c] = o[c] / l;
        }
        free(Kh);
        free(Vh);
        free(sc);
    }
    return err;
}

int ora_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------
 * R20, R21: causal prefill attention of one sequence, in double precision.
 * q: [Hq][T][D], k, v: [Hkv][T][D] stored values; out: [Hq][T][D] doubles;
 * score: [Hkv][T] doubles (cumulative attention per key position).
 * ---------------------------------------------------------------------- */
int ora_prefill_attention(int dt, int T, int Hq, int Hkv, const uint16_t *q,
                          const uint16_t *k, const uint16_t *v, double scale,
                          double *out, double *score) {
    if (T <= 0 || Hkv <= 0 || Hq % Hkv) return -1;
    int g = Hq / Hkv;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < Hkv; h++) {
        double *Kh = (double *)malloc(sizeof(double) * (size_t)T * D);
        double *Vh = (double *)malloc(sizeof(double) * (size_t)T * D);
        double *w = (double *)malloc(sizeof(double) * (size_t)T);
        if (!Kh || !Vh || !w) {
            err = -2;
            free(Kh); free(Vh); free(w);
            continue;
        }
        for (size_t x = 0; x < (size_t)T * D; x++) {
            Kh[x] = ora_decode(dt, k[(size_t)h * T * D + x]);
            Vh[x] = ora_decode(dt, v[(size_t)h * T * D + x]);
        }
        for (int j = 0; j < T; j++) score[(size_t)h * T + j] = 0.0;
        for (int a = 0; a < g; a++) {
            int hq = h * g + a;
            for (int i = 0; i < T; i++) {
                const uint16_t *qi = q + ((size_t)hq * T + i) * D;
                double qd[D];
                for (int c = 0; c < D; c++) qd[c] = ora_decode(dt, qi[c]);
                int last = ORA_PLANT == 17 ? T - 1 : i; /* causal mask dropped */
                double m = -INFINITY;
                for (int j = 0; j <= last; j++) {
                    double d = 0.0;
                    for (int c = 0; c < D; c++) d += qd[c] * Kh[(size_t)j * D + c];
                    w[j] = scale * d;
                    if (w[j] > m) m = w[j];
                }
                double l = 0.0;
                for (int j = 0; j <= last; j++) {
                    w[j] = exp(w[j] - m);
                    l += w[j];
                }
                double o[D];
                for (int c = 0; c < D; c++) o[c] = 0.0;
                for (int j = 0; j <= last; j++) {
                    double pr = w[j] / l;
                    score[(size_t)h * T + j] += ORA_PLANT == 18 ? w[j] : pr; /* unnormalized */
                    for (int c = 0; c < D; c++) o[c] += pr * Vh[(size_t)j * D + c];
                }
                for (int c = 0; c < D; c++) out[((size_t)hq * T + i) * D + c] = o[c];
            }
        }
        free(Kh);
        free(Vh);
        free(w);
    }
    return err;
}

/* R20: the causal attention output of chosen query positions only, in
   double precision, for checks of long sequences where the full run costs
   O(T^2).  rows[0..nrows) are query positions (any order, each < T); out:
   [Hq][nrows][D] doubles, out[hq][r] = sum over j <= rows[r] of
   softmax_j(scale q_{hq,rows[r]} . k_j) v_j with the KV head of hq (R12).
   Each (query head, row) is computed on its own, as one row of the full
   prefill above. */
int ora_prefill_rows(int dt, int T, int Hq, int Hkv, const uint16_t *q,
                     const uint16_t *k, const uint16_t *v, double scale, int nrows,
                     const int32_t *rows, double *out) {
    if (T <= 0 || Hkv <= 0 || Hq % Hkv || nrows < 0) return -1;
    for (int r = 0; r < nrows; r++)
        if (rows[r] < 0 || rows[r] >= T) return -1;
    int g = Hq / Hkv;
    size_t n = (size_t)Hkv * T * D;
    double *Kd = (double *)malloc(sizeof(double) * n);
    double *Vd = (double *)malloc(sizeof(double) * n);
    if (!Kd || !Vd) {
        free(Kd);
        free(Vd);
        return -2;
    }
#pragma omp parallel for schedule(static)
    for (long x = 0; x < (long)n; x++) {
        Kd[x] = ora_decode(dt, k[x]);
        Vd[x] = ora_decode(dt, v[x]);
    }
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (long job = 0; job < (long)Hq * nrows; job++) {
        int hq = (int)(job / nrows), r = (int)(job % nrows);
        int h = hq / g, i = rows[r];
        double *w = (double *)malloc(sizeof(double) * (size_t)(i + 1));
        if (!w) {
            err = -2;
            continue;
        }
        const uint16_t *qi = q + ((size_t)hq * T + i) * D;
        const double *Kh = Kd + (size_t)h * T * D, *Vh = Vd + (size_t)h * T * D;
        double qd[D];
        for (int c = 0; c < D; c++) qd[c] = ora_decode(dt, qi[c]);
        int last = ORA_PLANT == 21 ? i - 1 : i; /* plant: the diagonal key left out */
        double m = -INFINITY;
        for (int j = 0; j <= last; j++) {
            double d = 0.0;
            for (int c = 0; c < D; c++) d += qd[c] * Kh[(size_t)j * D + c];
            w[j] = scale * d;
            if (w[j] > m) m = w[j];
        }
        double l = 0.0;
        for (int j = 0; j <= last; j++) {
            w[j] = exp(w[j] - m);
            l += w[j];
        }
        double o[D];
        for (int c = 0; c < D; c++) o[c] = 0.0;
        for (int j = 0; j <= last; j++) {
            double pr = w[j] / l;
            for (int c = 0; c < D; c++) o[c] += pr * Vh[(size_t)j * D + c];
        }
        for (int c = 0; c < D; c++) out[((size_t)hq * nrows + r) * D + c] = o[c];
        free(w);
    }
    free(Kd);
    free(Vd);
    return err;
}

/* R22: heavy hitters + recent window.  Sorting (a library step) orders the
   candidate positions by score, higher first, the lower position first among
   equal scores. */
static const double *sel_score;
static int sel_cmp(const void *a, const void *b) {
    int i = *(const int *)a, j = *(const int *)b;
    if (sel_score[i] != sel_score[j]) return sel_score[i] > sel_score[j] ? -1 : 1;
    return ORA_PLANT == 19 ? (i < j ? 1 : -1) : (i < j ? -1 : 1); /* ties to the lower */
}

int ora_select_tokens(int T, const double *score, int heavy, int recent, int32_t *keep) {
    if (T < 0 || heavy < 0 || recent < 0) return -1;
    if (recent > T) recent = T;
    int n_old = T - recent;
    if (heavy > n_old) heavy = n_old;
    int *idx = (int *)malloc(sizeof(int) * (size_t)(n_old > 0 ? n_old : 1));
    char *kept = (char *)calloc((size_t)(T > 0 ? T : 1), 1);
    if (!idx || !kept) {
        free(idx); free(kept);
        return -2;
    }
    for (int j = 0; j < n_old; j++) idx[j] = j;
    sel_score = score;
    qsort(idx, (size_t)n_old, sizeof(int), sel_cmp);
    for (int r = 0; r < heavy; r++) kept[idx[r]] = 1;
    for (int j = n_old + (ORA_PLANT == 20 ? 1 : 0); j < T; j++) kept[j] = 1; /* recent window */
    int n = 0;
    for (int j = 0; j < T; j++)
        if (kept[j]) keep[n++] = j;
    free(idx);
    free(kept);
    return n;
}
