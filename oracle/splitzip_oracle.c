/*
 * splitzip_oracle.c -- plain, slow, single-threaded CPU oracle of the SplitZip
 * lossless BF16 codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load, link or call
 * this file; only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no header, helper, table or constant with the
 * HIP library: every layout rule below is re-derived here from the pages.
 *
 * Source of every step: the page "splitzip_codec.py -- SplitZip codec adapter
 * for diffusers-dynamic-offloader" (page 1: module docstring "Method" and
 * "Payload layout", functions calibrate_codebook, assemble_payload,
 * encode_torch, decode_torch), and the page "SplitZip in DDO -- VMM routes"
 * (page 2: "Invariants common to both routes", item 1, the fixed wire format).
 *
 * Readings where the pages are silent or ambiguous (each one is listed in the
 * design notes of the repository as well):
 *   R1  top-16 ties: page 1 sorts counts with an unstable descending argsort,
 *       so equal counts have no fixed order there.  Here: count descending,
 *       then exponent value ascending.
 *   R2  fewer than 16 distinct exponents: only that many codes are assigned;
 *       unused dec_lut slots stay 0.
 *   R3  the 4-bit code written for an escaped element is (16 & 0xF) = 0.
 *   R4  the even-indexed element occupies the HIGH nibble of its pk byte;
 *       for odd n the last low nibble is a zero pad that decode ignores.
 *   R5  padding bytes between sections are zero; there is no trailing pad.
 *   R6  n = 0 is valid: empty payload, no codes, coverage reported as 1.
 *   R7  escapes are stored in ascending element order.  Decode validation
 *       (optional) rejects lpos >= chunk, idx >= n, negative chunk ids and
 *       non-increasing idx.
 * All arithmetic is integer; no float conversion touches the data.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_ECAPACITY 2
#define ORC_ECORRUPT 3
#define ORC_ENOMEM 4

/* Page 1, helper _align4: round a byte offset up to a multiple of 4. */
static uint64_t round_up4(uint64_t v) { return (v + 3u) & ~(uint64_t)3u; }

/* Page 1 docstring "Method": the exponent byte is bits 7..14 of the 16-bit
 * view of a BF16 value. */
static unsigned exponent_of(uint16_t bits) { return (unsigned)((bits >> 7) & 0xFFu); }

/* Page 1 docstring "Method" / encode_torch: the stored byte keeps the sign
 * (bit 15) in its bit 7 and the seven low mantissa bits verbatim. */
static unsigned signmant_of(uint16_t bits) {
    return (unsigned)(((bits >> 8) & 0x80u) | (bits & 0x7Fu));
}

/* Page 1 docstring "Method" / decode_torch: reconstruction puts the sign back
 * at bit 15, the exponent at bits 7..14 and the low mantissa at bits 0..6. */
static uint16_t rebuild(unsigned sm, unsigned ex) {
    return (uint16_t)(((sm & 0x80u) << 8) | ((ex & 0xFFu) << 7) | (sm & 0x7Fu));
}

/* ---------------------------------------------------------------------------
 * Calibration (page 1, calibrate_codebook)
 * ------------------------------------------------------------------------- */

/* Step 1: count how often each exponent byte occurs. */
void orc_histogram(const uint16_t *x, uint64_t n, uint64_t counts[256]) {
    for (int v = 0; v < 256; ++v) counts[v] = 0;
    for (uint64_t i = 0; i < n; ++i) counts[exponent_of(x[i])] += 1;
}

typedef struct {
    uint64_t count;
    unsigned value;
} orc_bin;

/* Reading R1: order by count descending, then by exponent value ascending. */
static int orc_bin_order(const void *pa, const void *pb) {
    const orc_bin *a = (const orc_bin *)pa, *b = (const orc_bin *)pb;
    if (a->count != b->count) return a->count > b->count ? -1 : 1;
    if (a->value != b->value) return a->value < b->value ? -1 : 1;
    return 0;
}

/* Steps 2-4: keep the exponents that occur, sort them by frequency, give the
 * first min(16, #distinct) of them the codes 0, 1, 2, ... in that order and
 * fill the four lookup tables:
 *   enc[v]      code of v, 0 when v has no code
 *   marked[v]   code of v, 16 when v has no code (escape marker)
 *   dec[c]      exponent carried by code c (0 for unused codes, reading R2)
 *   common[v]   1 when v has a code
 * covered is the number of elements whose exponent received a code; the
 * coverage of page 1 is covered / n. */
void orc_select(const uint64_t counts[256], uint8_t enc[256], uint8_t marked[256],
                uint8_t dec[16], uint8_t common[256], uint32_t *n_codes,
                uint64_t *covered) {
    orc_bin bins[256];
    int distinct = 0;
    for (int v = 0; v < 256; ++v) {
        if (counts[v] > 0) {
            bins[distinct].count = counts[v];
            bins[distinct].value = (unsigned)v;
            ++distinct;
        }
    }
    qsort(bins, (size_t)distinct, sizeof(orc_bin), orc_bin_order);
    int top = distinct < 16 ? distinct : 16;

    memset(enc, 0, 256);
    memset(marked, 16, 256);
    memset(dec, 0, 16);
    memset(common, 0, 256);
    uint64_t cov = 0;
    for (int code = 0; code < top; ++code) {
        unsigned v = bins[code].value;
        enc[v] = (uint8_t)code;
        marked[v] = (uint8_t)code;
        dec[code] = (uint8_t)v;
        common[v] = 1;
        cov += bins[code].count;
    }
    *n_codes = (uint32_t)top;
    *covered = cov;
}

void orc_calibrate(const uint16_t *x, uint64_t n, uint64_t counts[256], uint8_t enc[256],
                   uint8_t marked[256], uint8_t dec[16], uint8_t common[256],
                   uint32_t *n_codes, uint64_t *covered) {
    orc_histogram(x, n, counts);
    orc_select(counts, enc, marked, dec, common, n_codes, covered);
}

/* ---------------------------------------------------------------------------
 * Wire layout (page 1, assemble_payload; page 2, invariant 1)
 *   pk        n_pairs = ceil(n/2) bytes          at off[0] = 0
 *   sm        n bytes                            at off[1] = align4(n_pairs)
 *   chunk_id  n_esc int32, little-endian         at off[2] = align4(off[1] + n)
 *   local_pos n_esc uint16, little-endian        at off[3] = off[2] + 4 n_esc
 *   esc_val   n_esc bytes                        at off[4] = align4(off[3] + 2 n_esc)
 *   total     off[4] + n_esc
 * ------------------------------------------------------------------------- */
void orc_layout(uint64_t n, uint64_t n_esc, uint64_t off[5], uint64_t *total) {
    uint64_t n_pairs = (n + 1) / 2;
    off[0] = 0;
    off[1] = round_up4(off[0] + n_pairs);
    off[2] = round_up4(off[1] + n);
    off[3] = off[2] + 4 * n_esc;
    off[4] = round_up4(off[3] + 2 * n_esc);
    *total = off[4] + n_esc;
}

static void put_le32(uint8_t *p, uint32_t v) {
    p[0] = (uint8_t)(v & 0xFFu);
    p[1] = (uint8_t)((v >> 8) & 0xFFu);
    p[2] = (uint8_t)((v >> 16) & 0xFFu);
    p[3] = (uint8_t)((v >> 24) & 0xFFu);
}
static void put_le16(uint8_t *p, uint32_t v) {
    p[0] = (uint8_t)(v & 0xFFu);
    p[1] = (uint8_t)((v >> 8) & 0xFFu);
}
static uint32_t get_le32(const uint8_t *p) {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
           ((uint32_t)p[3] << 24);
}
static uint32_t get_le16(const uint8_t *p) { return (uint32_t)p[0] | ((uint32_t)p[1] << 8); }

/* ---------------------------------------------------------------------------
 * Encode (page 1, encode_torch then assemble_payload)
 *
 * marked = the escape-marked table of a codebook (any codebook: it need not
 * have been calibrated on x).  On success buf[0 .. *total) holds the payload;
 * when cap < *total nothing is written and ORC_ECAPACITY is returned with
 * *n_esc_out, off and *total still describing the payload that would result.
 * ------------------------------------------------------------------------- */
int orc_encode(const uint16_t *x, uint64_t n, const uint8_t marked[256], uint32_t chunk,
               uint8_t *buf, uint64_t cap, uint64_t *n_esc_out, uint64_t off[5],
               uint64_t *total) {
    if (chunk == 0 || chunk > 65536u) return ORC_EINVAL;
    uint64_t n_pairs = (n + 1) / 2;

    /* Per-element split, code lookup and escape list, in element order. */
    uint8_t *pk = (uint8_t *)calloc(n_pairs ? n_pairs : 1, 1);
    uint8_t *sm = (uint8_t *)malloc(n ? n : 1);
    uint64_t *esc_idx = (uint64_t *)malloc(sizeof(uint64_t) * (n ? n : 1));
    if (!pk || !sm || !esc_idx) {
        free(pk); free(sm); free(esc_idx);
        return ORC_ENOMEM;
    }
    uint64_t n_esc = 0;
    for (uint64_t i = 0; i < n; ++i) {
        unsigned ex = exponent_of(x[i]);
        unsigned m = marked[ex];
        unsigned nibble = m & 0xFu; /* reading R3: an escape writes code 0 */
        if (i % 2 == 0)
            pk[i / 2] = (uint8_t)(nibble << 4); /* reading R4: even -> high */
        else
            pk[i / 2] = (uint8_t)(pk[i / 2] | nibble);
        sm[i] = (uint8_t)signmant_of(x[i]);
        if (m > 15) esc_idx[n_esc++] = i; /* loop order: ascending index */
    }

    orc_layout(n, n_esc, off, total);
    *n_esc_out = n_esc;
    if (*total > cap) {
        free(pk); free(sm); free(esc_idx);
        return ORC_ECAPACITY;
    }

    /* Assembly into a zero-filled buffer (reading R5). */
    memset(buf, 0, *total);
    memcpy(buf + off[0], pk, n_pairs);
    memcpy(buf + off[1], sm, n);
    for (uint64_t r = 0; r < n_esc; ++r) {
        uint64_t i = esc_idx[r];
        put_le32(buf + off[2] + 4 * r, (uint32_t)(i / chunk));
        put_le16(buf + off[3] + 2 * r, (uint32_t)(i % chunk));
        buf[off[4] + r] = (uint8_t)exponent_of(x[i]);
    }
    free(pk); free(sm); free(esc_idx);
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Decode (page 1, decode_torch)
 *
 * Reads the sections at the offsets the caller hands in (as page 1 reads them
 * from the payload metadata).  Out-of-bounds sections and escape positions
 * are always rejected with ORC_ECORRUPT (the oracle never writes outside
 * out[0..n)); with validate != 0 the escape stream must moreover be strictly
 * increasing, chunk-local positions must be < chunk and the offsets must equal
 * the layout rule.
 * ------------------------------------------------------------------------- */
/* count items of width bytes starting at byte off lie inside buf[0, buf_len)
 * (written so that no sum or product can wrap around) */
static int section_fits(uint64_t off, uint64_t count, uint64_t width, uint64_t buf_len) {
    return off <= buf_len && count <= (buf_len - off) / width;
}

int orc_decode(const uint8_t *buf, uint64_t buf_len, uint64_t n, uint64_t n_esc,
               uint32_t chunk, const uint64_t off[5], const uint8_t dec[16], uint16_t *out,
               int validate) {
    if (chunk == 0 || chunk > 65536u) return ORC_EINVAL;
    uint64_t n_pairs = (n + 1) / 2;
    if (!section_fits(off[0], n_pairs, 1, buf_len) || !section_fits(off[1], n, 1, buf_len) ||
        !section_fits(off[2], n_esc, 4, buf_len) || !section_fits(off[3], n_esc, 2, buf_len) ||
        !section_fits(off[4], n_esc, 1, buf_len))
        return ORC_ECORRUPT;
    if (validate) {
        uint64_t want[5], total;
        orc_layout(n, n_esc, want, &total);
        for (int s = 0; s < 5; ++s)
            if (want[s] != off[s]) return ORC_ECORRUPT;
    }
    const uint8_t *pk = buf + off[0];
    const uint8_t *sm = buf + off[1];

    /* Dense part: every element through the 16-entry table. */
    for (uint64_t i = 0; i < n; ++i) {
        unsigned code = (i % 2 == 0) ? (unsigned)(pk[i / 2] >> 4) : (unsigned)(pk[i / 2] & 0xFu);
        out[i] = rebuild(sm[i], dec[code]);
    }

    /* Escape patch: each escape carries its raw exponent and its position. */
    uint64_t prev = 0;
    for (uint64_t r = 0; r < n_esc; ++r) {
        uint32_t cid_bits = get_le32(buf + off[2] + 4 * r);
        int32_t cid = (int32_t)cid_bits;
        uint32_t pos = get_le16(buf + off[3] + 2 * r);
        unsigned ex = buf[off[4] + r];
        if (cid < 0) return ORC_ECORRUPT;
        uint64_t idx = (uint64_t)cid * chunk + pos;
        if (idx >= n) return ORC_ECORRUPT;
        if (validate) {
            if (pos >= chunk) return ORC_ECORRUPT;
            if (r > 0 && idx <= prev) return ORC_ECORRUPT;
        }
        prev = idx;
        out[idx] = rebuild(sm[idx], ex);
    }
    return ORC_OK;
}
