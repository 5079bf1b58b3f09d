/*
 * abi_host_check.c -- exercises the host-side parts of the C ABI (sizes,
 * status strings, argument checks) without a GPU, for a build of the library
 * with the host sanitizers.  Every call here must return before any device
 * work.  Exit status 0 when all answers are as the header states.
 */
#include <stdint.h>
#include <stdio.h>

#include "splitzip.h"

static int failures = 0;
#define EXPECT(cond)                                                          \
    do {                                                                      \
        if (!(cond)) {                                                        \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond);        \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

int main(void) {
    EXPECT(splitzip_abi_version() == SPLITZIP_ABI_VERSION);
    size_t cb = 0, meta = 0;
    splitzip_struct_sizes(&cb, &meta);
    EXPECT(cb == sizeof(splitzip_codebook) && meta == sizeof(splitzip_meta));
    for (int s = -2; s < 10; ++s) EXPECT(splitzip_status_string(s) != NULL);
    /* layout sizes: closed form P + n + 7e + (-P mod 4) + (-n mod 4) + 2 (e mod 2) */
    for (uint64_t n = 0; n < 300; ++n)
        for (uint64_t e = 0; e <= n; e += 7) {
            const uint64_t P = (n + 1) / 2;
            const uint64_t want = P + n + 7 * e + ((4 - P % 4) % 4) + ((4 - n % 4) % 4) + 2 * (e % 2);
            EXPECT(splitzip_payload_size(n, e) == want);
        }
    EXPECT(splitzip_payload_size(SPLITZIP_MAX_N, SPLITZIP_MAX_N) > SPLITZIP_MAX_N);
    size_t prev = 0;
    for (uint64_t n = 0; n < (1ull << 36); n = n * 3 + 1) {
        const size_t w = splitzip_workspace_size(n);
        /* a count per 8192-element tile, at most 512 staged escapes per tile */
        EXPECT(w >= prev && w >= n / 4 && w <= splitzip_workspace_size(0) + n / 2 + 4096);
        prev = w;
    }
    const uint64_t ns[3] = {0, 1000, 33554432};
    EXPECT(splitzip_workspace_size_batch(ns, 3) >= splitzip_workspace_size(33554432));
    EXPECT(splitzip_workspace_size_batch(NULL, 0) > 0);
    /* argument errors: nothing reaches the device */
    uint16_t *x = (uint16_t *)0x1000;
    splitzip_codebook *c = (splitzip_codebook *)0x2000;
    splitzip_meta *m = (splitzip_meta *)0x3000;
    uint8_t *p = (uint8_t *)0x4000;
    void *ws = (void *)0x5000;
    EXPECT(splitzip_workspace_init(NULL, 1 << 20, NULL) == SPLITZIP_ERR_INVALID);
    EXPECT(splitzip_calibrate(NULL, 5, c, ws, 1 << 20, NULL) == SPLITZIP_ERR_INVALID);
    EXPECT(splitzip_calibrate((uint16_t *)0x1002, 5, c, ws, 1 << 20, NULL) == SPLITZIP_ERR_INVALID);
    EXPECT(splitzip_calibrate(x, SPLITZIP_MAX_N + 1, c, ws, 1 << 20, NULL) == SPLITZIP_ERR_INVALID);
    EXPECT(splitzip_calibrate(x, 5, c, ws, 10, NULL) == SPLITZIP_ERR_WORKSPACE);
    EXPECT(splitzip_encode(x, 100, c, p, 10, m, ws, 1 << 30, NULL) == SPLITZIP_ERR_CAPACITY);
    EXPECT(splitzip_encode(x, 100, c, p, 1 << 20, m, ws, 10, NULL) == SPLITZIP_ERR_WORKSPACE);
    EXPECT(splitzip_encode_chunked(x, 100, c, 0, p, 1 << 20, m, ws, 1 << 30, NULL) ==
           SPLITZIP_ERR_INVALID);
    EXPECT(splitzip_encode_chunked(x, 100, c, 65537, p, 1 << 20, m, ws, 1 << 30, NULL) ==
           SPLITZIP_ERR_INVALID);
    EXPECT(splitzip_decode(p, 10, m, p, (uint16_t *)0x6000, 100, NULL, NULL) ==
           SPLITZIP_ERR_INVALID);
    EXPECT(splitzip_decode(p, 1 << 20, m, p, (uint16_t *)0x6004, 100, NULL, NULL) ==
           SPLITZIP_ERR_INVALID);
    EXPECT(splitzip_decode(p, 1 << 20, m, p, (uint16_t *)0x6000, 100, (int32_t *)0x7002, NULL) ==
           SPLITZIP_ERR_INVALID);
    EXPECT(splitzip_decode_slot(p, 100, m, p, 100, (uint8_t *)0x8000, 1 << 20, NULL, NULL) ==
           SPLITZIP_ERR_INVALID);
    EXPECT(splitzip_decode_slot(p, 1 << 20, m, p, 100, p + 64, 1 << 20, NULL, NULL) ==
           SPLITZIP_ERR_INVALID);
    splitzip_item items[2] = {{x, 100, c, p, 10, m, (uint16_t *)0x6000},
                              {x, 100, c, p, 1 << 20, m, (uint16_t *)0x6000}};
    EXPECT(splitzip_encode_batch(items, 2, ws, 1 << 30, NULL) == SPLITZIP_ERR_CAPACITY);
    EXPECT(splitzip_calibrate_batch(NULL, 1, ws, 1 << 30, NULL) == SPLITZIP_ERR_INVALID);
    EXPECT(splitzip_decode_batch(NULL, 2, NULL, NULL) == SPLITZIP_ERR_INVALID);
    splitzip_slot_item slots[1] = {{p, 100, m, p, 100, (uint8_t *)0x8000, 1 << 20}};
    EXPECT(splitzip_decode_slot_batch(slots, 1, NULL, NULL) == SPLITZIP_ERR_INVALID);
    /* in-place decode schedule: argument errors, then for many sizes and
       pass counts the ranges the header promises (lo[2] = 0, hi[2] = t_min,
       nested ranges, t_min = the first tile whose output starts at or past
       the dense sections' end) */
    {
        uint64_t t_min = 0, lo[9], hi[9];
        EXPECT(splitzip_slot_schedule(100, 1, &t_min, lo, hi) == 0);
        EXPECT(splitzip_slot_schedule(100, 9, &t_min, lo, hi) == 0);
        EXPECT(splitzip_slot_schedule(SPLITZIP_MAX_N + 1, 4, &t_min, lo, hi) == 0);
        EXPECT(splitzip_slot_schedule(100, 4, NULL, lo, hi) == 0);
        EXPECT(splitzip_slot_schedule(100, 4, &t_min, NULL, hi) == 0);
        for (uint64_t n = 1; n <= SPLITZIP_MAX_N; n = n * 5 / 2 + 3) {
            for (uint32_t passes = 2; passes <= 8; ++passes) {
                for (int k = 0; k < 9; ++k) lo[k] = hi[k] = 0xdead;
                const uint32_t used = splitzip_slot_schedule(n, passes, &t_min, lo, hi);
                EXPECT(used == 2 || used == passes);
                const uint64_t tiles = (n + 8191) / 8192;
                const uint64_t dense = splitzip_payload_size(n, 0);
                /* dense sections end at off_cid, the first 4-aligned offset past P' + n */
                const uint64_t P = (n + 1) / 2, off_cid = ((((P + 3) & ~3ull) + n) + 3) & ~3ull;
                uint64_t want = (off_cid + 16383) / 16384;
                if (want > tiles) want = tiles;
                EXPECT(dense == off_cid && t_min == want);
                EXPECT(lo[0] == 0 && hi[0] == 0 && lo[1] == 0 && hi[1] == 0);
                EXPECT(lo[2] == 0 && hi[2] == t_min);
                for (uint32_t k = 2; k < used; ++k)
                    EXPECT(lo[k] <= lo[k + 1] && lo[k + 1] <= hi[k + 1] && hi[k + 1] <= hi[k]);
                if (used == passes && passes > 2) EXPECT(lo[passes] < hi[passes]);   /* last pass holds a tile */
                for (uint32_t k = used + 1; k <= passes; ++k) EXPECT(lo[k] == 0 && hi[k] == 0);
            }
        }
    }
    printf("%d failures\n", failures);
    return failures ? 1 : 0;
}
