/*
 * kvq_oracle.c -- plain, slow CPU oracle for packed KV-cache quantization,
 * the Equivalent Right Shift (ERS) bit-width shrink and decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no source, header, table or helper with the HIP library;
 * everything here is written from the pages' formulas and from the layout text
 * of the library's public header, one step at a time, single-threaded.
 *
 * Sources (cited by page title and section):
 *   [PMKVQ]   "PM-KVQ: Progressive Mixed-Precision KV Cache Quantization for
 *              Long-CoT LLMs" (papernotes.org summary).
 *   [CHANMIX] "Channel-Aware Mixed-Precision Quantization for Efficient
 *              Long-Context Inference" (papernotes.org summary).
 *
 * Floating point: the quantizer decides integer codes, so it runs in IEEE
 * binary32 with one rounding per operation (no contraction; build with
 * -ffp-contract=off, no fast-math), exactly as the GPU kernel does.  Parameter
 * narrowing is written from the format definitions.  Dequantization and
 * attention run in binary64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* parameter dtypes: same numbering as the public header's enum */
#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2
#define ORC_E4M3 3

/* ------------------------------------------------------------------------ */
/* O1. Number formats.                                                       */
/*                                                                           */
/* A finite binary floating-point format with p significand bits (implicit  */
/* bit included) and minimum normal exponent emin represents, in the binade  */
/* [2^e, 2^(e+1)) with e >= emin, exactly the multiples of 2^(e-p+1); below  */
/* 2^emin it represents the multiples of 2^(emin-p+1) (subnormals).  Round-  */
/* to-nearest-even picks the nearest multiple, ties to the even multiple.    */
/* The helper below does exactly that in binary64, where every binary32     */
/* input and every candidate is exact.                                       */
/* ------------------------------------------------------------------------ */

/* Round |x| (finite, exact in double) to the format (p, emin); returns the
 * rounded magnitude as a double (may be 2^(emax+1) or more: caller handles
 * overflow). */
static double round_to_format(double ax, int p, int emin)
{
    if (ax == 0.0) return 0.0;
    int e;
    (void)frexp(ax, &e);          /* ax = f * 2^e, f in [0.5, 1) */
    e -= 1;                       /* ax in [2^e, 2^(e+1)) */
    if (e < emin) e = emin;
    double quantum = ldexp(1.0, e - p + 1);
    double r = ax / quantum;      /* exact: power-of-two division */
    double n = nearbyint(r);      /* default rounding mode: ties to even */
    return n * quantum;           /* exact */
}

/* IEEE 754 binary16: p = 11, emin = -14, emax = 15, max finite 65504. */
uint16_t orc_f32_to_f16(float x)
{
    uint32_t bits;
    memcpy(&bits, &x, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if (isnan(x)) return (uint16_t)(sign | 0x7E00u);
    double ax = fabs((double)x);
    if (isinf(x)) return (uint16_t)(sign | 0x7C00u);
    double r = round_to_format(ax, 11, -14);
    if (r > 65504.0) return (uint16_t)(sign | 0x7C00u);   /* overflow -> inf */
    if (r == 0.0) return sign;
    int e;
    double f = frexp(r, &e);      /* r = f * 2^e, f in [0.5,1) */
    e -= 1;                       /* r in [2^e, 2^(e+1)) */
    if (e < -14) {                /* subnormal: r = m * 2^-24 */
        uint16_t m = (uint16_t)ldexp(r, 24);
        return (uint16_t)(sign | m);
    }
    uint16_t m = (uint16_t)(ldexp(f * 2.0, 10) - 1024.0);  /* fraction bits */
    uint16_t ex = (uint16_t)(e + 15);
    return (uint16_t)(sign | (ex << 10) | m);
}

double orc_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = (m == 0) ? INFINITY : NAN;
    else v = ldexp(1024.0 + m, e - 25);
    return s ? -v : v;
}

/* bfloat16: p = 8, emin = -126, emax = 127. */
uint16_t orc_f32_to_bf16(float x)
{
    uint32_t bits;
    memcpy(&bits, &x, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
    if (isinf(x)) return (uint16_t)(sign | 0x7F80u);
    double r = round_to_format(fabs((double)x), 8, -126);
    double maxf = ldexp(255.0, 127 - 7);               /* (2 - 2^-7) * 2^127 */
    if (r > maxf) return (uint16_t)(sign | 0x7F80u);
    float rf = (float)r;                                 /* exact: r is a bf16 value */
    uint32_t rb;
    memcpy(&rb, &rf, 4);
    return (uint16_t)(sign | (uint16_t)(rb >> 16));
}

double orc_bf16_to_f64(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 fraction bits;
 * p = 4, emin = -6; no infinities, S.1111.111 is NaN, so the largest finite
 * magnitude is 1.75 * 2^8 = 448.  Narrowing rounds to nearest even and then
 * saturates finite overflow to +-448. */
uint8_t orc_f32_to_e4m3(float x)
{
    uint8_t sign = (uint8_t)(signbit(x) ? 0x80u : 0u);
    if (isnan(x)) return (uint8_t)(sign | 0x7Fu);
    double r = isinf(x) ? 1e300 : round_to_format(fabs((double)x), 4, -6);
    if (r > 448.0) r = 448.0;
    if (r == 0.0) return sign;
    int e;
    double f = frexp(r, &e);
    e -= 1;
    if (e < -6) {                 /* subnormal: r = m * 2^-9, m in 1..7 */
        uint8_t m = (uint8_t)ldexp(r, 9);
        return (uint8_t)(sign | m);
    }
    uint8_t m = (uint8_t)(ldexp(f * 2.0, 3) - 8.0);
    uint8_t ex = (uint8_t)(e + 7);
    return (uint8_t)(sign | (ex << 3) | m);
}

double orc_e4m3_to_f64(uint8_t c)
{
    int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) v = NAN;
    else if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(8.0 + m, e - 10);
    return s ? -v : v;
}

/* parameter storage: raw bits, pb bytes each */
static int param_bytes(int pdt)
{
    switch (pdt) {
    case ORC_F32: return 4;
    case ORC_F16: return 2;
    case ORC_BF16: return 2;
    case ORC_E4M3: return 1;
    default: return 0;
    }
}

/* narrow a binary32 value to the parameter dtype and store its raw bits */
static void param_store(void *arr, int64_t i, int pdt, float x)
{
    switch (pdt) {
    case ORC_F32: ((float *)arr)[i] = x; break;
    case ORC_F16: ((uint16_t *)arr)[i] = orc_f32_to_f16(x); break;
    case ORC_BF16: ((uint16_t *)arr)[i] = orc_f32_to_bf16(x); break;
    case ORC_E4M3: ((uint8_t *)arr)[i] = orc_f32_to_e4m3(x); break;
    }
}

/* exact value of a stored parameter */
static double param_load(const void *arr, int64_t i, int pdt)
{
    switch (pdt) {
    case ORC_F32: return (double)((const float *)arr)[i];
    case ORC_F16: return orc_f16_to_f64(((const uint16_t *)arr)[i]);
    case ORC_BF16: return orc_bf16_to_f64(((const uint16_t *)arr)[i]);
    case ORC_E4M3: return orc_e4m3_to_f64(((const uint8_t *)arr)[i]);
    }
    return NAN;
}

/* exported for tests */
double orc_param_value(const void *arr, int64_t i, int pdt) { return param_load(arr, i, pdt); }
void orc_param_narrow(void *arr, int64_t i, int pdt, float x) { param_store(arr, i, pdt, x); }

/* ------------------------------------------------------------------------ */
/* O2. Asymmetric uniform quantizer of one group.                            */
/*                                                                           */
/* [CHANMIX] Key design 1: S = (C_max - C_min) / (2^b - 1); the zero point   */
/* is the group minimum and the maximum error of x^ = S*q + Z is S/2.        */
/* [PMKVQ] Training strategy: asymmetric groups of 128.                      */
/* Reading: S and Z are first narrowed to the stored parameter dtype (round  */
/* to nearest even), and the codes are computed from the stored S', Z':      */
/*    q = clamp(rne((x - Z') / S'), 0, 2^b - 1), all in binary32;            */
/* S' == 0 (constant group or underflow) gives q = 0 for every element.     */
/* ------------------------------------------------------------------------ */
void orc_quantize_group(const float *x, int64_t stride, int n, int bits, int pdt,
                        uint16_t *codes, int64_t code_stride,
                        void *s_arr, void *z_arr, int64_t pidx)
{
    float mn = x[0], mx = x[0];
    for (int i = 1; i < n; i++) {
        float v = x[(int64_t)i * stride];
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    /* the extremes are real numbers: -0 and +0 are the same value, kept as +0 */
    mn = mn + 0.0f;
    mx = mx + 0.0f;
    float levels = (float)((1u << bits) - 1u);
    float s = (mx - mn) / levels;                 /* two binary32 roundings */
    param_store(s_arr, pidx, pdt, s);
    param_store(z_arr, pidx, pdt, mn);
    float sp = (float)param_load(s_arr, pidx, pdt);  /* exact in binary32 */
    float zp = (float)param_load(z_arr, pidx, pdt);
    for (int i = 0; i < n; i++) {
        float v = x[(int64_t)i * stride];
        uint16_t q = 0;
        if (sp != 0.0f) {
            float d = v - zp;
            float r = d / sp;
            float rr = nearbyintf(r);             /* ties to even */
            if (!(rr > 0.0f)) rr = 0.0f;
            if (rr > levels) rr = levels;
            q = (uint16_t)rr;
        }
        codes[(int64_t)i * code_stride] = q;
    }
}

/* ------------------------------------------------------------------------ */
/* O5. Packing (layout text of the public header).                          */
/*                                                                           */
/* A packed row is a little-endian bit string: bit i of the row is bit      */
/* (i mod 8) of byte (i div 8).  Element e of a b-bit row occupies bits      */
/* [e*b, (e+1)*b), least significant code bit first.                         */
/*   K tile, uniform b: 128 rows = tokens of the tile, elements = channels.  */
/*   V tile, uniform b: 128 rows = channels, elements = tokens of the tile.  */
/* ------------------------------------------------------------------------ */
static void put_bits(uint8_t *row, int64_t bitpos, int width, uint32_t value)
{
    for (int k = 0; k < width; k++) {
        int64_t b = bitpos + k;
        uint8_t mask = (uint8_t)(1u << (b & 7));
        if ((value >> k) & 1u) row[b >> 3] |= mask;
        else row[b >> 3] &= (uint8_t)~mask;
    }
}

static uint32_t get_bits(const uint8_t *row, int64_t bitpos, int width)
{
    uint32_t v = 0;
    for (int k = 0; k < width; k++) {
        int64_t b = bitpos + k;
        v |= (uint32_t)((row[b >> 3] >> (b & 7)) & 1u) << k;
    }
    return v;
}

/* codes[r][e] (row-major 128x128 uint16) -> packed tile of 128 rows of 16*b bytes */
void orc_pack_rows(const uint16_t *codes, int bits, uint8_t *tile)
{
    int row_bytes = 16 * bits;
    for (int r = 0; r < 128; r++)
        for (int e = 0; e < 128; e++)
            put_bits(tile + (int64_t)r * row_bytes, (int64_t)e * bits, bits, codes[r * 128 + e]);
}

void orc_unpack_rows(const uint8_t *tile, int bits, uint16_t *codes)
{
    int row_bytes = 16 * bits;
    for (int r = 0; r < 128; r++)
        for (int e = 0; e < 128; e++)
            codes[r * 128 + e] = (uint16_t)get_bits(tile + (int64_t)r * row_bytes, (int64_t)e * bits, bits);
}

/* Value tile (header layout text): 32-bit little-endian words W[w][c][a],
 * w < b, c < 128, a < 4; word W[w][c][a] holds the codes of channel c for
 * tokens 32a + w*(32/b) + i, i < 32/b, code i at bits [i*b, i*b + b).  With
 * c = 64h + 16q + n (h < 2, q < 4, n < 16) it sits at word index
 * w*512 + ((h*16 + n)*4 + a)*4 + q.  Bit position of the code of (channel c,
 * token t): */
static int64_t vtile_bitpos(int c, int t, int bits)
{
    int per_word = 32 / bits;
    int a = t / 32, w = (t % 32) / per_word, i = t % per_word;
    int h = c / 64, q = (c / 16) % 4, n = c % 16;
    int64_t word = (int64_t)w * 512 + ((h * 16 + n) * 4 + a) * 4 + q;
    return word * 32 + (int64_t)i * bits;
}

/* codes[c][t] (128x128, channel-major) -> 2048*bits-byte value tile */
void orc_pack_vtile(const uint16_t *codes, int bits, uint8_t *tile)
{
    for (int c = 0; c < 128; c++)
        for (int t = 0; t < 128; t++)
            put_bits(tile, vtile_bitpos(c, t, bits), bits, codes[c * 128 + t]);
}

void orc_unpack_vtile(const uint8_t *tile, int bits, uint16_t *codes)
{
    for (int c = 0; c < 128; c++)
        for (int t = 0; t < 128; t++)
            codes[c * 128 + t] = (uint16_t)get_bits(tile, vtile_bitpos(c, t, bits), bits);
}

/* Mixed-bit key tile ([CHANMIX] Key design 3: retrieval 4 / outlier 3 /
 * normal 2 / sub-normal 1 bit, as many 1-bit as 3-bit channels, channels
 * reordered so every byte holds exactly 8 code bits).
 * Slot widths (header layout text): slots 0..7 are 4-bit; slots 8..23
 * alternate 3-bit (even slot) and 1-bit (odd slot); slots 24..127 are 2-bit.
 * A token's 34-byte logical row is the little-endian bit string of its 128
 * slot codes in slot order.  The tile stores those rows as five column planes
 * (header layout text): plane g < 4 sits at tile offset 1024*g with 8 bytes
 * per token, holding logical bytes g, 4+g, 8+6g .. 13+6g in that order (one
 * 4-bit pair, one (3,1,3,1) group, six 2-bit quads); plane 4 sits at offset
 * 4096 with 2 bytes per token, holding logical bytes 32 and 33; tokens are in
 * order inside every plane.  Tile size 4352. */
int orc_mixed_slot_bits(int j)
{
    if (j < 8) return 4;
    if (j < 24) return (j % 2 == 0) ? 3 : 1;
    return 2;
}

static int mixed_slot_bitpos(int j)
{
    int pos = 0;
    for (int i = 0; i < j; i++) pos += orc_mixed_slot_bits(i);
    return pos;
}

static int64_t mixed_byte_addr(int t, int rb)  /* token t, logical row byte rb */
{
    int plane, at;
    if (rb >= 32) return 4096 + 2 * t + (rb - 32);
    if (rb < 4) { plane = rb; at = 0; }                 /* 4-bit pair */
    else if (rb < 8) { plane = rb - 4; at = 1; }        /* (3,1,3,1) group */
    else { plane = (rb - 8) / 6; at = 2 + (rb - 8) % 6; }   /* 2-bit quads */
    return 1024 * plane + 8 * t + at;
}

/* codes[t][j] (128x128, token-major, slot order) -> 4352-byte tile */
void orc_pack_mixed(const uint16_t *codes, uint8_t *tile)
{
    for (int t = 0; t < 128; t++) {
        uint8_t row[34];
        memset(row, 0, sizeof row);
        for (int j = 0; j < 128; j++)
            put_bits(row, mixed_slot_bitpos(j), orc_mixed_slot_bits(j), codes[t * 128 + j]);
        for (int rb = 0; rb < 34; rb++) tile[mixed_byte_addr(t, rb)] = row[rb];
    }
}

void orc_unpack_mixed(const uint8_t *tile, uint16_t *codes)
{
    for (int t = 0; t < 128; t++) {
        uint8_t row[34];
        for (int rb = 0; rb < 34; rb++) row[rb] = tile[mixed_byte_addr(t, rb)];
        for (int j = 0; j < 128; j++)
            codes[t * 128 + j] = (uint16_t)get_bits(row, mixed_slot_bitpos(j), orc_mixed_slot_bits(j));
    }
}

/* Mixed-width value tile (header layout text; value channel classes as in
 * [CHANMIX] Key design 3, read for values with per-class token groups):
 * value slot j holds channel v_slot_chan[j]; slots 0..15 are 4-bit, 16..31
 * 3-bit, 32..47 1-bit, 48..127 2-bit.  Each (token, class) is one group with
 * its own S', Z' (params [class][token] per stream, class order 4, 3, 1, 2
 * bits).  The tile
 * holds eight blocks of 16 slots (block b = slots 16b .. 16b+15) in order;
 * block b stores its codes in fields of cw = 4 bits (b < 2; the 3-bit codes
 * of block 1 in the low 3 bits) or cw = 2 bits (b >= 2; the 1-bit codes of
 * block 2 in the low bit).  Block b starts at word 64 * (4b) for b < 2 and
 * 64 * (8 + 2(b - 2)) after; inside it, word (w * 16 + n) * 4 + a (w < cw,
 * n < 16, a < 4) holds slot 16b + n for the 32/cw tokens
 * 32a + w * (32/cw) + i, code i at bits [i*cw, i*cw + cw).  Tile size 5120. */
int orc_vmixed_slot_bits(int j)
{
    return j < 16 ? 4 : (j < 32 ? 3 : (j < 48 ? 1 : 2));
}

static int vmixed_class(int j) { return j < 16 ? 0 : (j < 32 ? 1 : (j < 48 ? 2 : 3)); }

static int vmixed_field(int j) { return j < 32 ? 4 : 2; }     /* stored field width */

static int64_t vmixed_bitpos(int j, int t)
{
    int b = j / 16, n = j % 16, cw = vmixed_field(j), per = 32 / cw;
    int64_t base = 64 * (int64_t)(b < 2 ? 4 * b : 8 + 2 * (b - 2));
    int a = t / 32, w = (t % 32) / per, i = t % per;
    int64_t word = base + ((int64_t)w * 16 + n) * 4 + a;
    return word * 32 + (int64_t)i * cw;
}

/* codes[j][t] (128 slots x 128 tokens) -> 5120-byte tile */
void orc_pack_vmixed(const uint16_t *codes, uint8_t *tile)
{
    for (int j = 0; j < 128; j++)
        for (int t = 0; t < 128; t++)
            put_bits(tile, vmixed_bitpos(j, t), vmixed_field(j), codes[j * 128 + t]);
}

void orc_unpack_vmixed(const uint8_t *tile, uint16_t *codes)
{
    for (int j = 0; j < 128; j++)
        for (int t = 0; t < 128; t++)
            codes[j * 128 + t] = (uint16_t)get_bits(tile, vmixed_bitpos(j, t), vmixed_field(j));
}

/* ------------------------------------------------------------------------ */
/* O3/O4. Quantize one (batch, kv-head) stream of n_tok tokens (multiple of  */
/* 128), token t0 at element 0.                                              */
/* [CHANMIX] Background and Overall framework; [PMKVQ] related work on KIVI: */
/* keys are grouped channel-wise (one group = one channel over a 128-token   */
/* tile), values token-wise (one group = one token's 128 channels).          */
/* Outputs: tile i of the stream is written at codes + i * tile_stride.      */
/* Key params: [n_tiles][128] (per slot); value params: [n_tok].             */
/* ------------------------------------------------------------------------ */
void orc_quantize_k(const float *k, int64_t t_stride, int n_tok, int bits, int pdt,
                    uint8_t *codes, int64_t tile_stride, void *s, void *z)
{
    uint16_t *c = (uint16_t *)malloc(128 * 128 * sizeof(uint16_t));
    for (int g = 0; g < n_tok / 128; g++) {
        const float *base = k + (int64_t)g * 128 * t_stride;
        for (int ch = 0; ch < 128; ch++)
            orc_quantize_group(base + ch, t_stride, 128, bits, pdt,
                               c + ch, 128, s, z, (int64_t)g * 128 + ch);
        orc_pack_rows(c, bits, codes + (int64_t)g * tile_stride);
    }
    free(c);
}

/* slot_chan[j] = channel stored in slot j (a permutation of 0..127) */
void orc_quantize_k_mixed(const float *k, int64_t t_stride, int n_tok, int pdt,
                          const int16_t *slot_chan, uint8_t *codes, int64_t tile_stride,
                          void *s, void *z)
{
    uint16_t *c = (uint16_t *)malloc(128 * 128 * sizeof(uint16_t));
    for (int g = 0; g < n_tok / 128; g++) {
        const float *base = k + (int64_t)g * 128 * t_stride;
        for (int j = 0; j < 128; j++)
            orc_quantize_group(base + slot_chan[j], t_stride, 128, orc_mixed_slot_bits(j), pdt,
                               c + j, 128, s, z, (int64_t)g * 128 + j);
        orc_pack_mixed(c, codes + (int64_t)g * tile_stride);
    }
    free(c);
}

void orc_quantize_v(const float *v, int64_t t_stride, int n_tok, int bits, int pdt,
                    uint8_t *codes, int64_t tile_stride, void *s, void *z)
{
    uint16_t *tc = (uint16_t *)malloc(128 * 128 * sizeof(uint16_t)); /* [t][c] */
    uint16_t *ct = (uint16_t *)malloc(128 * 128 * sizeof(uint16_t)); /* [c][t] */
    for (int g = 0; g < n_tok / 128; g++) {
        for (int t = 0; t < 128; t++) {
            int64_t tok = (int64_t)g * 128 + t;
            orc_quantize_group(v + tok * t_stride, 1, 128, bits, pdt, tc + t * 128, 1, s, z, tok);
        }
        for (int t = 0; t < 128; t++)
            for (int ch = 0; ch < 128; ch++) ct[ch * 128 + t] = tc[t * 128 + ch];
        orc_pack_vtile(ct, bits, codes + (int64_t)g * tile_stride);
    }
    free(tc);
    free(ct);
}

/* Values with mixed channel widths: for every token, the slots of each class
 * form one group (the class's channels of that token) quantized at the
 * class width; params s[class * n_tok + tok], z[...]. */
void orc_quantize_v_mixed(const float *v, int64_t t_stride, int n_tok, int pdt,
                          const int16_t *slot_chan, uint8_t *codes, int64_t tile_stride,
                          void *s, void *z)
{
    uint16_t *jt = (uint16_t *)malloc(128 * 128 * sizeof(uint16_t));   /* [slot][t] */
    static const int first[5] = {0, 16, 32, 48, 128};
    for (int g = 0; g < n_tok / 128; g++) {
        for (int t = 0; t < 128; t++) {
            int64_t tok = (int64_t)g * 128 + t;
            for (int k = 0; k < 4; k++) {
                float x[128];
                uint16_t q[128];
                int n = first[k + 1] - first[k];
                for (int i = 0; i < n; i++) x[i] = v[tok * t_stride + slot_chan[first[k] + i]];
                orc_quantize_group(x, 1, n, orc_vmixed_slot_bits(first[k]), pdt, q, 1, s, z,
                                   (int64_t)k * n_tok + tok);
                for (int i = 0; i < n; i++) jt[(first[k] + i) * 128 + t] = q[i];
            }
        }
        orc_pack_vmixed(jt, codes + (int64_t)g * tile_stride);
    }
    free(jt);
}

/* ------------------------------------------------------------------------ */
/* O6. Equivalent Right Shift ([PMKVQ] Key design 1, ERS equation):          */
/*   X_b = ((2^(2b) - 2^b + 1) * (X_2b + 2^(b-1))) >> 3b,                    */
/*   Z_b = Z_2b,  S_b = (2^b + 1) * S_2b.                                    */
/* The rounding bracket around the product encloses an integer, so it does  */
/* nothing; ">> 3b" is floor division by 2^(3b).  The product reaches about */
/* 4.29e9 at b = 8, so it is formed in unsigned 64-bit here (the library    */
/* uses unsigned 32-bit, which the product never exceeds).                  */
/* ------------------------------------------------------------------------ */
uint32_t orc_ers(uint32_t x2b, int b)
{
    uint64_t c = (1ull << (2 * b)) - (1ull << b) + 1ull;
    uint64_t n = (uint64_t)x2b + (1ull << (b - 1));
    return (uint32_t)((c * n) >> (3 * b));
}

/* The halving rules of [PMKVQ]'s ablation (Key design 1 and the ablation
 * table), method 0/1/2:
 *   0 Equivalent Right Shift, as above;
 *   1 direct right shift -- keep the high b bits of the 2b-bit code, i.e.
 *     floor(X / 2^b);
 *   2 modified right shift -- not defined on the page; read as the shift with
 *     rounding, floor((X + 2^(b-1)) / 2^b), clamped to 2^b - 1.
 * Zero points stay; the scale becomes (2^b + 1) S for ERS and 2^b S for the
 * two shifts (one step of the new code spans 2^b old steps). */
uint32_t orc_shift(uint32_t x2b, int b, int method)
{
    uint32_t top = (1u << b) - 1u;
    if (method == 1) return x2b / (1u << b);
    if (method == 2) {
        uint32_t r = (x2b + (1u << (b - 1))) / (1u << b);
        return r < top ? r : top;
    }
    return orc_ers(x2b, b);
}

/* Shrink one packed uniform-width key tile in place: 16384 codes of 2b bits
 * -> b bits, code order unchanged. */
void orc_shrink_tile_m(uint8_t *tile, int to_bits, int method)
{
    int from = 2 * to_bits;
    uint16_t *c = (uint16_t *)malloc(128 * 128 * sizeof(uint16_t));
    orc_unpack_rows(tile, from, c);
    for (int i = 0; i < 128 * 128; i++) c[i] = (uint16_t)orc_shift(c[i], to_bits, method);
    memset(tile, 0, (size_t)16 * from * 128);
    orc_pack_rows(c, to_bits, tile);
    free(c);
}
void orc_shrink_tile(uint8_t *tile, int to_bits) { orc_shrink_tile_m(tile, to_bits, 0); }

/* Shrink one value tile in place: every code goes from its position in the
 * 2b-bit word planes to its position in the b-bit word planes. */
void orc_shrink_vtile_m(uint8_t *tile, int to_bits, int method)
{
    int from = 2 * to_bits;
    uint16_t *c = (uint16_t *)malloc(128 * 128 * sizeof(uint16_t));
    orc_unpack_vtile(tile, from, c);
    for (int i = 0; i < 128 * 128; i++) c[i] = (uint16_t)orc_shift(c[i], to_bits, method);
    memset(tile, 0, (size_t)16 * from * 128);
    orc_pack_vtile(c, to_bits, tile);
    free(c);
}
void orc_shrink_vtile(uint8_t *tile, int to_bits) { orc_shrink_vtile_m(tile, to_bits, 0); }

/* S_b = narrow(binary32(f * S_2b)), f = 2^b + 1 (ERS) or 2^b (the shifts);
 * exact before narrowing for binary16, bfloat16 and e4m3 scales (at most
 * 11 + 9 significant bits). */
void orc_shrink_scales_m(void *s, int64_t n, int to_bits, int pdt, int method)
{
    float f = method == 0 ? (float)((1u << to_bits) + 1u) : (float)(1u << to_bits);
    for (int64_t i = 0; i < n; i++) {
        float sv = (float)param_load(s, i, pdt);
        param_store(s, i, pdt, f * sv);
    }
}
void orc_shrink_scales(void *s, int64_t n, int to_bits, int pdt) { orc_shrink_scales_m(s, n, to_bits, pdt, 0); }

/* ------------------------------------------------------------------------ */
/* O7/O8. Decode attention over one (batch, kv-head) stream, binary64.       */
/* [CHANMIX] Overall framework / Key design 3: the decode step reads the     */
/* packed cache, dequantizes it to full precision (x^ = S'*q + Z') and runs */
/* ordinary attention.  For each of the G query heads of this kv head:      */
/*   s_t = sigma * sum_c q_c K^[t][c];  p = softmax(s);  o = sum_t p_t V^[t] */
/* Two-pass softmax, no tiling.  q is bfloat16 (raw bits); sigma is the     */
/* binary32 softmax scale.  k_bits == 0 selects the mixed-bit key layout;   */
/* then slot_chan maps slots to channels.  out: [G][128].                    */
/* ------------------------------------------------------------------------ */
int orc_decode_attn(const uint8_t *kc, int64_t k_tile_stride, const void *ks, const void *kz, int k_bits,
                    const int16_t *slot_chan,
                    const uint8_t *vc, int64_t v_tile_stride, const void *vs, const void *vz, int v_bits,
                    const int16_t *v_slot_chan,
                    int pdt, int n_tok, const uint16_t *q, int G, float scale, double *out)
{
    if (n_tok <= 0 || n_tok % 128) return 1;
    double *K = (double *)malloc((size_t)n_tok * 128 * sizeof(double));
    double *V = (double *)malloc((size_t)n_tok * 128 * sizeof(double));
    double *sc = (double *)malloc((size_t)n_tok * sizeof(double));
    uint16_t *codes = (uint16_t *)malloc(128 * 128 * sizeof(uint16_t));
    if (!K || !V || !sc || !codes) { free(K); free(V); free(sc); free(codes); return 2; }

    for (int g = 0; g < n_tok / 128; g++) {
        /* keys: codes[t][slot] */
        if (k_bits == 0) orc_unpack_mixed(kc + (int64_t)g * k_tile_stride, codes);
        else orc_unpack_rows(kc + (int64_t)g * k_tile_stride, k_bits, codes);
        for (int t = 0; t < 128; t++)
            for (int j = 0; j < 128; j++) {
                int ch = (k_bits == 0) ? slot_chan[j] : j;
                double S = param_load(ks, (int64_t)g * 128 + j, pdt);
                double Z = param_load(kz, (int64_t)g * 128 + j, pdt);
                K[((int64_t)g * 128 + t) * 128 + ch] = S * codes[t * 128 + j] + Z;
            }
        /* values: codes[c][t] (mixed widths: codes[slot][t]) */
        if (v_bits == 0) {
            orc_unpack_vmixed(vc + (int64_t)g * v_tile_stride, codes);
            for (int t = 0; t < 128; t++) {
                int64_t tok = (int64_t)g * 128 + t;
                for (int j = 0; j < 128; j++) {
                    double S = param_load(vs, (int64_t)vmixed_class(j) * n_tok + tok, pdt);
                    double Z = param_load(vz, (int64_t)vmixed_class(j) * n_tok + tok, pdt);
                    V[tok * 128 + v_slot_chan[j]] = S * codes[j * 128 + t] + Z;
                }
            }
        } else {
            orc_unpack_vtile(vc + (int64_t)g * v_tile_stride, v_bits, codes);
            for (int t = 0; t < 128; t++) {
                int64_t tok = (int64_t)g * 128 + t;
                double S = param_load(vs, tok, pdt);
                double Z = param_load(vz, tok, pdt);
                for (int ch = 0; ch < 128; ch++) V[tok * 128 + ch] = S * codes[ch * 128 + t] + Z;
            }
        }
    }

    double sigma = (double)scale;
    for (int h = 0; h < G; h++) {
        double qd[128];
        for (int ch = 0; ch < 128; ch++) qd[ch] = orc_bf16_to_f64(q[h * 128 + ch]);
        double m = -INFINITY;
        for (int t = 0; t < n_tok; t++) {
            double acc = 0.0;
            for (int ch = 0; ch < 128; ch++) acc += qd[ch] * K[(int64_t)t * 128 + ch];
            sc[t] = sigma * acc;
            if (sc[t] > m) m = sc[t];
        }
        double l = 0.0;
        for (int t = 0; t < n_tok; t++) { sc[t] = exp(sc[t] - m); l += sc[t]; }
        for (int ch = 0; ch < 128; ch++) {
            double o = 0.0;
            for (int t = 0; t < n_tok; t++) o += sc[t] * V[(int64_t)t * 128 + ch];
            out[h * 128 + ch] = o / l;
        }
    }
    free(K); free(V); free(sc); free(codes);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O9. Progressive schedule accounting ([PMKVQ] Overall framework and Key   */
/* design 1: every block starts at 16 bits; when its memory budget is full  */
/* the whole cache drops one level 16 -> 8 -> 4 -> 2, down to the block's   */
/* target width).  Bytes of a block = key codes + value codes + all stored  */
/* scales and zero points.  Before appending a group of 128 tokens, while   */
/* the block with the group added at the current width would exceed the    */
/* budget, halve the width.  Fails (returns -1) if even the floor width     */
/* does not fit.                                                             */
/* ------------------------------------------------------------------------ */
int64_t orc_block_bytes(int B, int H, int64_t n_tok, int k_bits, int v_bits, int pdt)
{
    int64_t groups = n_tok / 128;
    int pb = param_bytes(pdt);
    int64_t per_group = (int64_t)16 * k_bits * 128 + (int64_t)16 * v_bits * 128   /* codes */
                        + (int64_t)2 * 128 * pb                                    /* key S,Z per channel */
                        + (int64_t)2 * 128 * pb;                                   /* value S,Z per token */
    return (int64_t)B * H * groups * per_group;
}

/* Replays appends of 128-token groups from 0 to n_total tokens, starting at
 * start_bits; writes (token count before the append, new width) for every
 * halving into events (pairs), returns the number of halvings or -1. */
int orc_schedule(int B, int H, int64_t n_total, int start_bits, int floor_bits, int pdt,
                 int64_t budget, int64_t *events, int max_events)
{
    int bits = start_bits, n = 0;
    for (int64_t t = 0; t < n_total; t += 128) {
        while (orc_block_bytes(B, H, t + 128, bits, bits, pdt) > budget) {
            if (bits / 2 < floor_bits || bits == 1) return -1;
            bits /= 2;
            if (n < max_events) { events[2 * n] = t; events[2 * n + 1] = bits; }
            n++;
        }
    }
    return n;
}

/* ------------------------------------------------------------------------ */
/* Array forms of the format conversions, for the tests' exhaustive sweeps. */
/* ------------------------------------------------------------------------ */
void orc_narrow_array(const float *x, int64_t n, int pdt, void *out)
{
    for (int64_t i = 0; i < n; i++) param_store(out, i, pdt, x[i]);
}

void orc_decode_array(const void *in, int64_t n, int pdt, double *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = param_load(in, i, pdt);
}

void orc_shift_array(const uint32_t *x, int64_t n, int b, int method, uint32_t *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_shift(x[i], b, method);
}

void orc_ers_array(const uint32_t *x, int64_t n, int b, uint32_t *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_ers(x[i], b);
}
