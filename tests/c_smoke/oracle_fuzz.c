/*
 * oracle_fuzz.c -- drives the CPU oracle (oracle/splitzip_oracle.c) under the
 * address and undefined-behaviour sanitizers: seeded random round trips with
 * own and foreign codebooks and every chunk size class, then decodes of
 * damaged payloads and metadata (flipped bytes, truncation, absurd escape
 * counts and offsets), which must end in a status code, never in an access
 * outside the buffers.  Exit status 0 when every round trip was exact.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_calibrate(const uint16_t *x, uint64_t n, uint64_t counts[256], uint8_t enc[256],
                   uint8_t marked[256], uint8_t dec[16], uint8_t common[256], uint32_t *n_codes,
                   uint64_t *covered);
void orc_layout(uint64_t n, uint64_t n_esc, uint64_t off[5], uint64_t *total);
int orc_encode(const uint16_t *x, uint64_t n, const uint8_t marked[256], uint32_t chunk,
               uint8_t *buf, uint64_t cap, uint64_t *n_esc_out, uint64_t off[5], uint64_t *total);
int orc_decode(const uint8_t *buf, uint64_t buf_len, uint64_t n, uint64_t n_esc, uint32_t chunk,
               const uint64_t off[5], const uint8_t dec[16], uint16_t *out, int validate);

/* SplitMix64 (Steele, Lea & Flood 2014) */
static uint64_t state = 0x5eed;
static uint64_t next(void) {
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int main(int argc, char **argv) {
    const int iters = argc > 1 ? atoi(argv[1]) : 300;
    int bad = 0;
    for (int it = 0; it < iters; ++it) {
        const uint64_t n = next() % 5000;
        uint16_t *x = malloc(n * 2 + 2);
        uint16_t *out = malloc(n * 2 + 2);
        const unsigned spread = 1 + (unsigned)(next() % 40);    /* distinct exponents */
        for (uint64_t i = 0; i < n; ++i) {
            const unsigned e = 100 + (unsigned)(next() % spread);
            x[i] = (uint16_t)(((next() & 1) << 15) | ((e & 0xFF) << 7) | (next() & 0x7F));
        }
        uint64_t counts[256], covered;
        uint8_t enc[256], marked[256], dec[16], common[256];
        uint32_t n_codes;
        orc_calibrate(x, n, counts, enc, marked, dec, common, &n_codes, &covered);
        if (next() % 5 == 0) {  /* foreign codebook: up to 16 random exponents */
            memset(marked, 16, 256);
            const unsigned k = (unsigned)(next() % 17);
            for (unsigned c = 0; c < k; ++c) {
                unsigned v = (unsigned)(next() % 256);
                while (marked[v] != 16) v = (v + 1) % 256;
                marked[v] = (uint8_t)c;
            }
        }
        const uint32_t chunks[] = {1, 3, 1000, 1024, 4096, 65536};
        const uint32_t chunk = chunks[next() % 6];
        uint64_t off[5], total, n_esc;
        orc_layout(n, n, off, &total);
        uint8_t *buf = malloc(total + 1);
        if (orc_encode(x, n, marked, chunk, buf, total, &n_esc, off, &total) != 0) {
            fprintf(stderr, "encode failed at iteration %d\n", it);
            return 1;
        }
        /* a foreign codebook's dec table is the one that decodes it */
        uint8_t fdec[16];
        memset(fdec, 0, 16);
        for (int v = 0; v < 256; ++v)
            if (marked[v] < 16) fdec[marked[v]] = (uint8_t)v;
        if (orc_decode(buf, total, n, n_esc, chunk, off, fdec, out, 1) != 0 ||
            memcmp(out, x, n * 2) != 0) {
            fprintf(stderr, "round trip failed at iteration %d (n=%llu)\n", it,
                    (unsigned long long)n);
            ++bad;
        }
        /* damaged payloads and metadata: any status, no stray access */
        for (int k = 0; k < 8; ++k) {
            uint8_t *b2 = malloc(total + 1);
            memcpy(b2, buf, total);
            uint64_t len = total, o2[5], e2 = n_esc;
            memcpy(o2, off, sizeof o2);
            switch (next() % 7) {
            case 0: if (total) b2[next() % total] ^= (uint8_t)(1 + next() % 255); break;
            case 1: len = total ? next() % total : 0; break;
            case 2: e2 = next() >> (next() % 64); break;
            case 3: o2[next() % 5] = next() >> (next() % 64); break;
            case 4: e2 = UINT64_MAX - next() % 8; break;              /* wraps 4e, 2e, e */
            case 5: o2[next() % 5] = UINT64_MAX - next() % 64; break; /* wraps off + len */
            default: e2 = n_esc + 1 + next() % 8; break;
            }
            (void)orc_decode(b2, len, n, e2, chunk, o2, fdec, out, (int)(next() & 1));
            free(b2);
        }
        free(buf);
        free(x);
        free(out);
    }
    printf("%d iterations, %d round-trip failures\n", iters, bad);
    return bad ? 1 : 0;
}
