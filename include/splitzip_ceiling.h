/*
 * Reference memory streams for measuring the SplitZip kernels
 * (libsplitzip_ceiling.so; not part of the codec).
 *
 * Each call moves the same bytes with the same access pattern as one codec
 * kernel of libsplitzip.so -- load and store widths, cache hints, workgroup
 * shape and the map from workgroups to data -- but replaces the coding with
 * a few XORs.  Its rate is therefore the ceiling of that access pattern on
 * the GPU it runs on, which is what a codec kernel can at best approach:
 *
 *   splitzip_ceiling_read           the calibrate histogram pass (reads 2n B)
 *   splitzip_ceiling_encode_shape   the dense encode (reads 2n B, writes
 *                                   n/2 B of nibbles and n B of bytes)
 *   splitzip_ceiling_decode_shape   the dense decode (reads n/2 + n B,
 *                                   writes 2n B)
 *
 * and probes of the part's costs that the codec's design rests on:
 *
 *   splitzip_ceiling_order          the same patterns in another order of
 *                                   tiles over the XCDs
 *   splitzip_ceiling_encode_wide / _decode_wide   the same patterns with
 *                                   thread-contiguous 32-element units
 *   splitzip_ceiling_encode_arrive  the encode pattern with a fused arrival
 *   splitzip_ceiling_encode_fenced  the encode pattern with a fence per
 *                                   workgroup
 *   splitzip_ceiling_atomics        device-scope atomics: latency, and cost
 *                                   on one address against spread ones
 *   splitzip_ceiling_launch         ordinary against cooperative launches
 *
 * Every tile-per-workgroup stream takes its tiles in the codec's order: in a
 * launch of at least 32,768 tiles each XCD (workgroup b runs on XCD b % 8)
 * takes 64 consecutive tiles in turn, and the last (tiles mod 512)
 * workgroups, like every smaller launch, take tile b.
 *
 * Conventions: every pointer is a device (or pinned host) address the
 * caller owns and keeps alive until the stream has run the call; calls are
 * asynchronous on `stream` (0 = the null stream); the output bytes are
 * meaningless, only the traffic matters.  Return values are the SPLITZIP_OK
 * / SPLITZIP_ERR_INVALID / SPLITZIP_ERR_HIP codes of splitzip.h.
 */
#ifndef SPLITZIP_CEILING_H
#define SPLITZIP_CEILING_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes at d_x (16-byte aligned, bytes a multiple of 16) as
 * 1024-thread workgroups, each streaming one contiguous range with 4 16-byte
 * non-temporal loads in flight per thread.  `grid` workgroups (0: two per
 * compute unit).  d_sink: 4 device bytes that receive a value only in the
 * unlikely case that the XOR of a workgroup's data hits a fixed constant (it
 * keeps the loads alive).  INVALID for a bad pointer, alignment or size. */
int splitzip_ceiling_read(const void *d_x, uint64_t bytes, uint32_t grid, uint32_t *d_sink,
                          hipStream_t stream);

/* The encode pattern over n elements (n a positive multiple of 8192): one
 * 8192-element tile per 256-thread workgroup; per 8 elements a 16-byte
 * non-temporal load of d_x, a 4-byte non-temporal store to d_pk + i/2 and an
 * 8-byte non-temporal store to d_sm + i.  d_x, d_pk, d_sm 16-byte aligned;
 * d_pk holds n/2 bytes, d_sm n bytes.  INVALID otherwise. */
int splitzip_ceiling_encode_shape(const uint16_t *d_x, uint64_t n, uint8_t *d_pk, uint8_t *d_sm,
                                  hipStream_t stream);

/* The decode pattern over n elements (n a positive multiple of 8192): one
 * 8192-element tile per 256-thread workgroup; per 8 elements a 4-byte
 * non-temporal load of d_pk + i/2, an 8-byte non-temporal load of d_sm + i
 * and a 16-byte non-temporal store to d_out + i.  Pointers 16-byte aligned; d_pk
 * holds n/2 bytes, d_sm n bytes, d_out 2n bytes.  INVALID otherwise. */
int splitzip_ceiling_decode_shape(const uint8_t *d_pk, const uint8_t *d_sm, uint16_t *d_out,
                                  uint64_t n, hipStream_t stream);

/* The encode (decode = 0: d_x -> d_pk, d_sm) or decode (decode = 1: d_pk,
 * d_sm -> d_out) pattern of the shapes above with `run` consecutive tiles per
 * XCD in turn (run a power of two up to 65536; 0: tile b for workgroup b),
 * at any launch size; the last (tiles mod 8 * run) workgroups take tile b.
 * The unused pointer may be NULL.  Sizes, alignment and errors as for the
 * shapes above. */
int splitzip_ceiling_order(uint32_t decode, uint32_t run, const uint16_t *d_x, uint8_t *d_pk,
                           uint8_t *d_sm, uint16_t *d_out, uint64_t n, hipStream_t stream);

/* The encode / decode patterns with thread-contiguous 32-element units: per
 * 32 elements four 16-byte loads of d_x, one 16-byte store to d_pk + i/2 and
 * two to d_sm + i (encode); one 16-byte load of d_pk + i/2, two of d_sm + i
 * and four 16-byte stores to d_out + i (decode).  Sizes, alignment and
 * errors as for the shapes above. */
int splitzip_ceiling_encode_wide(const uint16_t *d_x, uint64_t n, uint8_t *d_pk, uint8_t *d_sm,
                                 hipStream_t stream);
int splitzip_ceiling_decode_wide(const uint8_t *d_pk, const uint8_t *d_sm, uint16_t *d_out,
                                 uint64_t n, hipStream_t stream);

/* The encode pattern, then what a placement fused into the encode kernel
 * would add: each workgroup stores a 4-byte count to d_counts[tile] (n/8192
 * of them), waits for its stores to complete and arrives on a two-level
 * counter (groups of 16 workgroups) in d_ctrs (8 * (1 + ceil(tiles / 16))
 * uint64 words, counters 64 bytes apart, tagged with `epoch` in their high
 * half: a counter with another tag is claimed for it, so d_ctrs needs no
 * clearing as long as every call passes a new nonzero epoch); the last
 * arrival writes `epoch` to *d_ready.  All pointers 16-byte aligned. */
int splitzip_ceiling_encode_arrive(const uint16_t *d_x, uint64_t n, uint8_t *d_pk, uint8_t *d_sm,
                                   uint32_t *d_counts, uint64_t *d_ctrs, uint32_t *d_ready,
                                   uint32_t epoch, hipStream_t stream);

/* The encode pattern with an agent-scope fence (__threadfence) at the end of
 * every workgroup.  As splitzip_ceiling_encode_shape otherwise. */
int splitzip_ceiling_encode_fenced(const uint16_t *d_x, uint64_t n, uint8_t *d_pk, uint8_t *d_sm,
                                   hipStream_t stream);

/* `grid` workgroups of 64 threads; lane 0 of workgroup b adds 1 to
 * d_ctrs[(b % spread) * 8] (device scope) `rounds` times, each add waiting
 * for the previous one's result.  d_ctrs: 8 * spread uint64 words, 16-byte
 * aligned; spread in [1, 4096], rounds in [1, 2^20]. */
int splitzip_ceiling_atomics(uint64_t *d_ctrs, uint32_t grid, uint32_t spread, uint32_t rounds,
                             hipStream_t stream);

/* An almost empty kernel (`grid` <= 1024 workgroups of 64 threads; one
 * thread adds 1 to *d_sink), launched ordinarily or, with cooperative != 0,
 * with hipLaunchCooperativeKernel. */
int splitzip_ceiling_launch(uint32_t cooperative, uint32_t grid, uint32_t *d_sink,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPLITZIP_CEILING_H */
