/*
 * oracle.c -- plain, slow, single-threaded CPU reference for entropy-coded
 * weight decoding.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline of the benchmark may load this file's library. The product's
 * decode path never calls it, and the two share no code, header, table or
 * constant generator.
 *
 * What the method computes, and where it is described:
 *
 *  - Weights are kept as 8-bit codes of a full-range base format (Int8 or
 *    Float8 e4m3), flattened into one symbol stream and compressed without
 *    loss by an ANS coder; what is stored is that bitstream plus per-channel
 *    scales plus metadata, and the decoder runs on the device, filling a
 *    buffer just before a transformer block needs its weights.
 *    [EntQuant summary "Float8@2bits: Entropy Coding Enables Data-Free Model
 *    Compression", technical part §2 "Concepto Central", "Codificación de
 *    Pesos", "Decodificación en Tiempo de Inferencia".]
 *  - BF16 weights are split into the 8-bit exponent, which is entropy coded,
 *    and a sign+mantissa byte kept raw; decoding rebuilds the original bit
 *    pattern exactly. [DFloat11 write-up, sections "Margen de compresión
 *    restante en el exponente de BFloat16" and "Formato DFloat11".]
 *  - Decoding is split into independent segments so that many of them can be
 *    decoded at once. [EntroLLM summary, "Metodología" item 3.]
 *
 * The pages name ANS (and rANS, in the discussion under the DFloat11
 * write-up) but print no coder. The coder written out here is range ANS as
 * published by Duda ("Asymmetric numeral systems", 2013) with interleaved
 * states as published by Giesen ("Interleaved entropy coders", 2014), with
 * this library's format parameters:
 *     probability scale   M = 2^12 (frequencies sum to 4096)
 *     state               32 bits, kept in [L, 2^32) with L = 2^16
 *     renormalisation     16-bit words
 *     interleaving        K lane states per chunk; symbol i of a chunk
 *                         belongs to lane i mod K (K = 64 in the container)
 *
 * Every step below follows the plain definition, in the order of the method;
 * there is no blocking, fusion or reordering. All state arithmetic is done
 * in uint64_t so that no intermediate can wrap.
 *
 * Build: gcc -O2 -fPIC -shared -ffp-contract=off -o liboracle.so oracle.c -lm
 * (-ffp-contract=off: the dequantisation product must be one IEEE single
 *  multiply, never fused with anything.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_PROB_BITS 12u
#define ORC_M (1u << ORC_PROB_BITS)        /* 4096 */
#define ORC_L (1ull << 16)                 /* lower end of the state interval */
#define ORC_WORD_BITS 16u
#define ORC_CONTAINER_LANES 64u

/* Status codes of a chunk decode. */
#define ORC_OK 0
#define ORC_BAD_STATE 1 /* a lane did not return to L */
#define ORC_BAD_WORDS 2 /* the word stream ran out, or was not used up */

/* ------------------------------------------------------------------------ */
/* 1. Number formats                                                         */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* The default NaN: the pattern an invalid operation (0 * inf) produces. */
#define ORC_DEFAULT_NAN 0xFFC00000u

static int is_nan_bits(uint32_t u)
{
    return ((u & 0x7F800000u) == 0x7F800000u) && ((u & 0x007FFFFFu) != 0);
}

/* fp32 -> bf16, round to nearest, ties to even.
 * bf16 keeps the upper 16 bits of the fp32 pattern. The dropped half r is
 * compared with the half-way point 0x8000: above rounds up, below truncates,
 * equal rounds to the even result. A carry out of the mantissa moves into the
 * exponent, so the largest finite values round to infinity, as RNE requires.
 * A NaN stays a NaN: it is truncated and its quiet bit (bit 6) is set. */
uint16_t orc_bf16_from_f32_bits(uint32_t u)
{
    if (is_nan_bits(u))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t hi = u >> 16;
    uint32_t r = u & 0xFFFFu;
    if (r > 0x8000u || (r == 0x8000u && (hi & 1u)))
        hi += 1u;
    return (uint16_t)hi;
}

/* OCP Float8 E4M3 ("E4M3FN"): 1 sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits, no infinities, NaN only at S.1111.111.
 *   E = 0        : subnormal, value = m * 2^-9
 *   otherwise    : value = (1 + m/8) * 2^(E-7)
 * A NaN code is widened as IEEE 754-2008 §6.2.3 widens a NaN into a wider
 * format: it stays a NaN with its sign, and its trailing significand (the
 * 3 mantissa bits, all ones, the first of them the quiet bit) becomes the
 * leading bits of the fp32 trailing significand:
 *   S.1111.111 -> S << 31 | 0x7F800000 | 7 << 20  (0x7FF00000 / 0xFFF00000). */
uint32_t orc_e4m3_to_f32_bits(uint8_t c)
{
    uint32_t sign = c >> 7;
    uint32_t E = (c >> 3) & 15u;
    uint32_t m = c & 7u;
    if (E == 15u && m == 7u)
        return (sign << 31) | 0x7F800000u | (m << 20);
    double v;
    if (E == 0u)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + (double)m / 8.0, (int)E - 7);
    if (sign)
        v = -v;
    return f32_bits((float)v); /* exact: every e4m3 value is an fp32 value */
}

/* Int8 code: the byte is the two's-complement integer. */
uint32_t orc_int8_to_f32_bits(uint8_t c)
{
    return f32_bits((float)(int8_t)c);
}

/* Symbol kinds of a tensor. */
#define ORC_KIND_INT8 0
#define ORC_KIND_E4M3 1
#define ORC_KIND_BF16EXP 2

/* IEEE single-precision product v * s, rounded to nearest even, with the
 * NaN rules of IEEE 754-2008 §6.2.3 made explicit: a NaN operand is
 * returned quieted with its payload (the code's value is looked at first,
 * then the scale), and an invalid product (0 * inf) is the default NaN. */
uint32_t orc_mul_f32_bits(uint32_t vb, uint32_t sb)
{
    if (is_nan_bits(vb))
        return vb | 0x00400000u;
    if (is_nan_bits(sb))
        return sb | 0x00400000u;
    float p = bits_f32(vb) * bits_f32(sb);
    uint32_t pb = f32_bits(p);
    return is_nan_bits(pb) ? ORC_DEFAULT_NAN : pb;
}

/* Dequantisation of one code: bf16 = RNE16(fl32(value(code) * scale)).
 * [Codes of a full-range base format times per-channel scales: EntQuant
 *  summary technical part §2 "Codificación de Pesos"; the product is fixed
 *  as one fp32 multiply rounded to bf16, the library's reading of a decode
 *  "to usable weights".]
 * One IEEE single-precision multiply, rounded to nearest even, then the
 * fp32 -> bf16 rounding above. */
uint16_t orc_dequant_bf16(uint8_t code, int kind, float scale)
{
    uint32_t vb = (kind == ORC_KIND_E4M3) ? orc_e4m3_to_f32_bits(code)
                                          : orc_int8_to_f32_bits(code);
    return orc_bf16_from_f32_bits(orc_mul_f32_bits(vb, f32_bits(scale)));
}

/* BF16 = sign(1) | exponent(8) | mantissa(7). The exponent byte is the coded
 * symbol; the sign+mantissa byte is sign<<7 | mantissa. */
void orc_bf16_split(uint16_t w, uint8_t *exp_byte, uint8_t *sm_byte)
{
    *exp_byte = (uint8_t)((w >> 7) & 0xFFu);
    *sm_byte = (uint8_t)(((w >> 15) << 7) | (w & 0x7Fu));
}

uint16_t orc_bf16_merge(uint8_t exp_byte, uint8_t sm_byte)
{
    uint16_t sign = (uint16_t)(sm_byte >> 7);
    uint16_t mant = (uint16_t)(sm_byte & 0x7Fu);
    return (uint16_t)((sign << 15) | ((uint16_t)exp_byte << 7) | mant);
}

/* ------------------------------------------------------------------------ */
/* 2. Frequency table                                                        */
/* ------------------------------------------------------------------------ */

/* Quantise symbol counts to frequencies that sum to M = 4096.
 * [The pages fix no rule: the EntQuant summary, technical part §2
 *  "Codificación de Pesos", says only that the symbol stream is entropy
 *  coded. This rule is the library's reading; any table that sums to M and
 *  gives every present symbol f >= 1 decodes exactly.]
 *   present symbol s : f[s] = max(1, round(c[s] * M / N))  (half rounds up)
 *   absent symbol    : f[s] = 0
 *   while the sum exceeds M: take 1 from the largest f (smallest symbol on a
 *     tie) among those above 1;
 *   while the sum is below M: add 1 to the symbol with the largest count
 *     (smallest symbol on a tie);
 *   a single present symbol gets f = M.
 * Returns the number of present symbols (0 for an empty tensor, in which case
 * every f is 0). */
int orc_quantize_freqs(const uint64_t counts[256], uint16_t freq[256])
{
    uint64_t N = 0;
    int present = 0;
    for (int s = 0; s < 256; s++) {
        N += counts[s];
        if (counts[s])
            present++;
        freq[s] = 0;
    }
    if (present == 0)
        return 0;
    if (present == 1) {
        for (int s = 0; s < 256; s++)
            if (counts[s])
                freq[s] = (uint16_t)ORC_M;
        return 1;
    }
    uint64_t sum = 0;
    for (int s = 0; s < 256; s++) {
        if (!counts[s])
            continue;
        /* round(c*M/N) with halves rounded up = floor((2*c*M + N) / (2*N)) */
        uint64_t q = (2u * counts[s] * (uint64_t)ORC_M + N) / (2u * N);
        if (q < 1)
            q = 1;
        freq[s] = (uint16_t)q;
        sum += q;
    }
    while (sum > ORC_M) {
        int best = -1;
        for (int s = 0; s < 256; s++)
            if (freq[s] > 1 && (best < 0 || freq[s] > freq[best]))
                best = s;
        freq[best]--;
        sum--;
    }
    while (sum < ORC_M) {
        int best = -1;
        for (int s = 0; s < 256; s++)
            if (counts[s] && (best < 0 || counts[s] > counts[best]))
                best = s;
        freq[best]++;
        sum++;
    }
    return present;
}

/* cum[s] = sum of f[t] for t < s, in ascending byte order; cum[256] = sum. */
void orc_cumulative(const uint16_t freq[256], uint32_t cum[257])
{
    cum[0] = 0;
    for (int s = 0; s < 256; s++)
        cum[s + 1] = cum[s] + freq[s];
}

/* Slot table: slots cum[s] .. cum[s]+f[s]-1 belong to symbol s. */
static void slot_table(const uint16_t freq[256], uint8_t slot_sym[ORC_M])
{
    uint32_t cum[257];
    orc_cumulative(freq, cum);
    for (int s = 0; s < 256; s++)
        for (uint32_t k = cum[s]; k < cum[s + 1]; k++)
            slot_sym[k] = (uint8_t)s;
}

/* Returns 1 when the table is usable by the coder: sum is exactly M. */
int orc_table_valid(const uint16_t freq[256])
{
    uint32_t sum = 0;
    for (int s = 0; s < 256; s++)
        sum += freq[s];
    return sum == ORC_M;
}

/* ------------------------------------------------------------------------ */
/* 3. Interleaved rANS on one chunk                                          */
/* ------------------------------------------------------------------------ */

/* Encode n symbols with K interleaved lanes.
 * [Range ANS encode step: Duda, "Asymmetric numeral systems" (2013);
 *  interleaved states: Giesen, "Interleaved entropy coders" (2014). The pages
 *  name the coder only: EntQuant summary technical part §2, and rANS in the
 *  discussion under the DFloat11 write-up.]
 *
 * The decoder reads symbols front to back, so the encoder walks them back to
 * front. Every lane starts at x = L. For symbol i (lane j = i mod K, symbol s
 * with frequency f and cumulative c):
 *   1. renormalise: if x_j >= 2^20 * f (that is ((L >> 12) << 16) * f), put
 *      the low 16 bits of x_j on the emission list and shift x_j right by 16;
 *   2. code:        x_j = floor(x_j / f) * M + (x_j mod f) + c.
 * After the last (i.e. first) symbol, the K states are the chunk's initial
 * decoder states and the emission list, reversed, is the word stream the
 * decoder consumes front to back.
 *
 * Returns the number of words written to words[] (at most n), or -1 if a
 * symbol has frequency 0, or -2 if K is 0 or the table does not sum to M. */
int64_t orc_encode_chunk(const uint8_t *sym, uint32_t n, uint32_t K,
                         const uint16_t freq[256], uint32_t *states,
                         uint16_t *words)
{
    if (K == 0 || !orc_table_valid(freq))
        return -2;
    uint32_t cum[257];
    orc_cumulative(freq, cum);
    uint64_t *x = (uint64_t *)malloc(sizeof(uint64_t) * K);
    uint16_t *emitted = (uint16_t *)malloc(sizeof(uint16_t) * (n ? n : 1));
    for (uint32_t j = 0; j < K; j++)
        x[j] = ORC_L;
    uint64_t n_emitted = 0;
    for (uint32_t i = n; i-- > 0;) {
        uint32_t j = i % K;
        uint32_t s = sym[i];
        uint64_t f = freq[s];
        if (f == 0) {
            free(x);
            free(emitted);
            return -1;
        }
        uint64_t x_max = ((ORC_L >> ORC_PROB_BITS) << ORC_WORD_BITS) * f;
        if (x[j] >= x_max) {
            emitted[n_emitted++] = (uint16_t)(x[j] & 0xFFFFu);
            x[j] >>= ORC_WORD_BITS;
        }
        x[j] = (x[j] / f) * ORC_M + (x[j] % f) + cum[s];
    }
    for (uint32_t j = 0; j < K; j++)
        states[j] = (uint32_t)x[j];
    for (uint64_t k = 0; k < n_emitted; k++)
        words[k] = emitted[n_emitted - 1 - k];
    free(x);
    free(emitted);
    return (int64_t)n_emitted;
}

/* [Range ANS decode step (Duda 2013) with interleaved lanes (Giesen 2014);
 *  the device decodes during inference: EntQuant summary technical part §2
 *  "Decodificación en Tiempo de Inferencia".]
 * Decode n symbols with K interleaved lanes, front to back.
 * States x_j start at states[j]; the word pointer p starts at 0. For symbol
 * i = 0, 1, ..., n-1 (lane j = i mod K; so within a step of K symbols the
 * lanes go in ascending order):
 *   1. slot = x_j mod M; s = the symbol owning that slot;
 *      x_j = f[s] * floor(x_j / M) + slot - cum[s]; output s;
 *   2. if x_j < L: x_j = x_j * 2^16 + words[p]; p = p + 1.
 * A read past n_words is not made (the state is left as it is) and marks the
 * chunk ORC_BAD_WORDS. At the end every lane must be back at L and p must
 * equal n_words: otherwise ORC_BAD_WORDS if the word count is wrong, else
 * ORC_BAD_STATE. Returns the status, or -2 if K is 0 or the table is
 * invalid. */
int orc_decode_chunk(const uint32_t *states, const uint16_t *words,
                     uint32_t n_words, uint32_t n, uint32_t K,
                     const uint16_t freq[256], uint8_t *out)
{
    if (K == 0 || !orc_table_valid(freq))
        return -2;
    uint32_t cum[257];
    uint8_t slot_sym[ORC_M];
    orc_cumulative(freq, cum);
    slot_table(freq, slot_sym);
    uint64_t *x = (uint64_t *)malloc(sizeof(uint64_t) * K);
    for (uint32_t j = 0; j < K; j++)
        x[j] = states[j];
    uint64_t p = 0;
    int overrun = 0;
    for (uint32_t i = 0; i < n; i++) {
        uint32_t j = i % K;
        uint64_t slot = x[j] & (ORC_M - 1u);
        uint32_t s = slot_sym[slot];
        x[j] = (uint64_t)freq[s] * (x[j] >> ORC_PROB_BITS) + slot - cum[s];
        out[i] = (uint8_t)s;
        if (x[j] < ORC_L) {
            if (p < n_words) {
                x[j] = (x[j] << ORC_WORD_BITS) | words[p];
                p++;
            } else {
                overrun = 1;
            }
        }
    }
    int status = ORC_OK;
    if (overrun || p != n_words)
        status = ORC_BAD_WORDS;
    else
        for (uint32_t j = 0; j < K; j++)
            if (x[j] != ORC_L)
                status = ORC_BAD_STATE;
    free(x);
    return status;
}

/* ------------------------------------------------------------------------ */
/* 4. Container: one tensor as a run of chunk regions                        */
/* ------------------------------------------------------------------------ */

/* [Independent segments decoded at once: EntroLLM summary, "Metodología"
 *  item 3; weights decoded on the device before a block runs: EntQuant
 *  summary technical part §2 "Decodificación en Tiempo de Inferencia".]
 * A tensor of n symbols is cut into chunks of C symbols (the last one may be
 * shorter): chunk k holds symbols [kC, min((k+1)C, n)). Each chunk region is
 *     uint32 states[64]   little-endian, state of lane j at index j
 *     uint16 words[n_w]   little-endian, in decoder order
 *     zero bytes up to the next multiple of 16
 * and the regions follow each other in chunk order. For every chunk the
 * descriptor row holds {n_symbols, n_words, byte_offset, elem_offset}, the
 * byte offset being relative to the start of this tensor's regions.
 * Host byte order is little-endian on every machine this runs on; the
 * layout is written byte by byte anyway. */

static uint64_t region_bytes(uint64_t n_words)
{
    uint64_t b = 4u * ORC_CONTAINER_LANES + 2u * n_words;
    return (b + 15u) / 16u * 16u;
}

static void put_u32(uint8_t *p, uint32_t v)
{
    p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); p[2] = (uint8_t)(v >> 16); p[3] = (uint8_t)(v >> 24);
}
static void put_u16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static uint32_t get_u32(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
static uint16_t get_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Number of chunks of a tensor of n symbols, chunk size C. */
uint64_t orc_n_chunks(uint64_t n, uint32_t C) { return C ? (n + C - 1) / C : 0; }

/* Upper bound of the bytes one tensor can take (at most one word per symbol). */
uint64_t orc_tensor_bound(uint64_t n, uint32_t C)
{
    uint64_t k = orc_n_chunks(n, C);
    return k * (4u * ORC_CONTAINER_LANES + 16u) + 2u * n;
}

/* Encode a tensor. desc receives 4 uint64 per chunk. Returns the number of
 * bytes written, or a negative error (-1 symbol with f = 0, -2 bad table or
 * C, -3 out of space). */
int64_t orc_encode_tensor(const uint8_t *sym, uint64_t n, uint32_t C,
                          const uint16_t freq[256], uint8_t *out,
                          uint64_t out_cap, uint64_t *desc)
{
    if (C == 0 || C % ORC_CONTAINER_LANES != 0)
        return -2;
    uint64_t k_chunks = orc_n_chunks(n, C);
    uint32_t states[ORC_CONTAINER_LANES];
    uint16_t *words = (uint16_t *)malloc(sizeof(uint16_t) * C);
    uint64_t off = 0;
    for (uint64_t k = 0; k < k_chunks; k++) {
        uint64_t e0 = k * C;
        uint32_t cn = (uint32_t)((n - e0 < C) ? (n - e0) : C);
        int64_t nw = orc_encode_chunk(sym + e0, cn, ORC_CONTAINER_LANES, freq, states, words);
        if (nw < 0) {
            free(words);
            return nw;
        }
        uint64_t rb = region_bytes((uint64_t)nw);
        if (off + rb > out_cap) {
            free(words);
            return -3;
        }
        memset(out + off, 0, rb);
        for (uint32_t j = 0; j < ORC_CONTAINER_LANES; j++)
            put_u32(out + off + 4u * j, states[j]);
        for (int64_t w = 0; w < nw; w++)
            put_u16(out + off + 4u * ORC_CONTAINER_LANES + 2u * (uint64_t)w, words[w]);
        desc[4 * k + 0] = cn;
        desc[4 * k + 1] = (uint64_t)nw;
        desc[4 * k + 2] = off;
        desc[4 * k + 3] = e0;
        off += rb;
    }
    free(words);
    return (int64_t)off;
}

/* Decode the chunks described by desc (4 uint64 per chunk, byte offsets
 * relative to blob) into sym_out[elem_offset ...]. status_out (one per chunk)
 * receives each chunk's status. Returns the number of chunks whose status is
 * not ORC_OK, or -2 on an invalid table. */
int64_t orc_decode_tensor(const uint8_t *blob, const uint64_t *desc,
                          uint64_t n_chunks, const uint16_t freq[256],
                          uint8_t *sym_out, int32_t *status_out)
{
    if (!orc_table_valid(freq))
        return -2;
    uint32_t states[ORC_CONTAINER_LANES];
    int64_t bad = 0;
    uint16_t *words = NULL;
    uint64_t cap = 0;
    for (uint64_t k = 0; k < n_chunks; k++) {
        uint32_t cn = (uint32_t)desc[4 * k + 0];
        uint32_t nw = (uint32_t)desc[4 * k + 1];
        const uint8_t *r = blob + desc[4 * k + 2];
        if (nw > cap) {
            free(words);
            cap = nw;
            words = (uint16_t *)malloc(sizeof(uint16_t) * cap);
        }
        for (uint32_t j = 0; j < ORC_CONTAINER_LANES; j++)
            states[j] = get_u32(r + 4u * j);
        for (uint32_t w = 0; w < nw; w++)
            words[w] = get_u16(r + 4u * ORC_CONTAINER_LANES + 2u * w);
        int st = orc_decode_chunk(states, words, nw, cn, ORC_CONTAINER_LANES, freq,
                                  sym_out + desc[4 * k + 3]);
        if (status_out)
            status_out[k] = st;
        if (st != ORC_OK)
            bad++;
    }
    free(words);
    return bad;
}

/* ------------------------------------------------------------------------ */
/* 5. Whole-array helpers (plain loops over the scalar definitions above)    */
/* ------------------------------------------------------------------------ */

void orc_count_symbols(const uint8_t *sym, uint64_t n, uint64_t counts[256])
{
    for (int s = 0; s < 256; s++)
        counts[s] = 0;
    for (uint64_t i = 0; i < n; i++)
        counts[sym[i]]++;
}

/* bf16 output of a tensor of rows x cols codes, row-major: element i is in
 * row floor(i / cols) and uses scales[row]. */
void orc_dequant_tensor(const uint8_t *codes, uint64_t rows, uint64_t cols,
                        int kind, const float *scales, uint16_t *out)
{
    for (uint64_t r = 0; r < rows; r++)
        for (uint64_t c = 0; c < cols; c++)
            out[r * cols + c] = orc_dequant_bf16(codes[r * cols + c], kind, scales[r]);
}

void orc_bf16_split_array(const uint16_t *w, uint64_t n, uint8_t *exp_out, uint8_t *sm_out)
{
    for (uint64_t i = 0; i < n; i++)
        orc_bf16_split(w[i], &exp_out[i], &sm_out[i]);
}

void orc_bf16_merge_array(const uint8_t *e, const uint8_t *sm, uint64_t n, uint16_t *out)
{
    for (uint64_t i = 0; i < n; i++)
        out[i] = orc_bf16_merge(e[i], sm[i]);
}

void orc_bf16_from_f32_array(const uint32_t *u, uint64_t n, uint16_t *out)
{
    for (uint64_t i = 0; i < n; i++)
        out[i] = orc_bf16_from_f32_bits(u[i]);
}

void orc_e4m3_table(uint32_t out[256])
{
    for (int c = 0; c < 256; c++)
        out[c] = orc_e4m3_to_f32_bits((uint8_t)c);
}
