/*
 * splitzip.h -- C ABI of the MI355X (gfx950) SplitZip lossless BF16 codec.
 *
 * The method (page "splitzip_codec.py -- SplitZip codec adapter for
 * diffusers-dynamic-offloader", module docstring "Method"): view every BF16
 * value as 16 bits; keep its sign and 7 low mantissa bits as one byte (sm);
 * code its 8-bit exponent through a per-tensor table of the 16 most frequent
 * exponents as a 4-bit code, two codes per byte (pk); send every exponent
 * outside that table to a sparse escape stream of (int32 chunk id, uint16
 * position inside a 1024-element chunk, uint8 raw exponent).  Decoding is
 * bit-exact.
 *
 * Wire format (same page, "Payload layout" and function assemble_payload;
 * page "SplitZip in DDO -- VMM routes", "Invariants common to both routes"
 * item 1), with A(v) = v rounded up to a multiple of 4, P = ceil(n/2),
 * e = number of escapes:
 *   pk        uint8[P]           at off[0] = 0             (even element = high nibble)
 *   sm        uint8[n]           at off[1] = A(P)
 *   chunk_id  int32 LE [e]       at off[2] = A(off[1] + n)
 *   local_pos uint16 LE [e]      at off[3] = off[2] + 4e
 *   esc_val   uint8[e]           at off[4] = A(off[3] + 2e)
 *   total size                   comp_bytes = off[4] + e
 * Padding bytes are zero.  Escapes are in ascending element order.
 *
 * Conventions for every entry point:
 *   - All device work is enqueued asynchronously on `stream` (a hipStream_t,
 *     NULL = the default stream); no entry point synchronises, allocates or
 *     frees memory.  Every buffer is owned by the caller.
 *   - The return value reports argument errors and launch failures only
 *     (SPLITZIP_OK or an error code, nothing is enqueued on error).  Errors
 *     found by the device (capacity overflow, corrupt escape stream) are
 *     written to the status field / word named by the function.
 *   - Device pointers ("d_") may also be pinned host memory mapped into the
 *     device address space (hipHostMalloc): a decode then reads its payload,
 *     or an encode writes it, over the host link with no separate copy.
 *     Never pageable host memory: a kernel access to it faults.
 *   - Tensor and payload buffers must be 16-byte aligned.
 *   - n is limited to SPLITZIP_MAX_N elements.
 */
#ifndef SPLITZIP_H
#define SPLITZIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPLITZIP_ABI_VERSION 2
#define SPLITZIP_CHUNK 1024u
#define SPLITZIP_MAX_N (1ull << 36)

enum splitzip_status {
    SPLITZIP_OK = 0,
    SPLITZIP_ERR_INVALID = 1,   /* null/misaligned pointer, n out of range, bad size */
    SPLITZIP_ERR_CAPACITY = 2,  /* payload buffer smaller than the payload */
    SPLITZIP_ERR_CORRUPT = 3,   /* inconsistent payload / metadata */
    SPLITZIP_ERR_HIP = 4,       /* a HIP runtime call or launch failed */
    SPLITZIP_ERR_WORKSPACE = 5, /* workspace too small for n */
    SPLITZIP_ERR_INTERNAL = 6   /* device-side progress guard tripped (must not happen) */
};

/* Per-tensor codebook (page 1, SplitZipCodebook and calibrate_codebook).
 * Code c (0..n_codes-1) is the c-th most frequent exponent; equal counts are
 * ordered by exponent value ascending.  Unused dec_lut slots are 0. */
typedef struct splitzip_codebook {
    uint8_t enc_lut[256];        /* exponent -> code, 0 when it has none      */
    uint8_t enc_lut_marked[256]; /* exponent -> code, 16 when it escapes      */
    uint8_t dec_lut[16];         /* code -> exponent                          */
    uint8_t common_lut[256];     /* 1 when the exponent has a code            */
    uint32_t n_codes;            /* min(16, number of distinct exponents)     */
    uint32_t reserved;
    uint64_t covered;            /* elements whose exponent has a code        */
    uint64_t total;              /* n; coverage = covered / total (1 if n=0)  */
    uint64_t counts[256];        /* exponent histogram                        */
} splitzip_codebook;

/* Payload metadata (page 1, PayloadMeta); written by splitzip_encode. */
typedef struct splitzip_meta {
    uint64_t n;          /* elements                                          */
    uint64_t n_pairs;    /* ceil(n/2) = bytes of pk                           */
    uint64_t chunk_size; /* elements per chunk: 1024, or as given to
                            splitzip_encode_chunked                           */
    uint64_t n_esc;      /* escapes                                           */
    uint64_t comp_bytes; /* payload size; when status is CAPACITY, the size
                            that would have been needed                       */
    uint64_t offsets[5]; /* pk, sm, chunk_id, local_pos, esc_val              */
    uint64_t covered;    /* copied from the codebook used                     */
    uint64_t total;
    int32_t status;      /* SPLITZIP_OK or SPLITZIP_ERR_CAPACITY / _INTERNAL  */
    uint32_t flags;      /* SPLITZIP_META_* bits                              */
} splitzip_meta;

/* splitzip_meta.flags: the escape stream is in strictly ascending element
 * order.  splitzip_encode sets it (its escapes always are); metadata from
 * elsewhere (page 1, PayloadMeta: no such field) leaves it clear, and then
 * every decode applies the escapes in an order-independent pass of its own,
 * as page 1, decode_torch does. */
#define SPLITZIP_META_ASCENDING 1u

/* One tensor of a batched call.  The array of items lives in host memory;
 * the pointers in it are device pointers.  Each batched call reads only the
 * fields it needs:
 *   calibrate  x, n -> cb
 *   encode     x, n, cb, payload, capacity -> payload, meta
 *   decode     payload, capacity (readable bytes), meta, cb (its dec_lut), n -> out */
typedef struct splitzip_item {
    const uint16_t *x;     /* n BF16 values as uint16 bit patterns (16-byte aligned) */
    uint64_t n;            /* elements                                               */
    splitzip_codebook *cb; /* codebook of this tensor                                */
    uint8_t *payload;      /* payload buffer (16-byte aligned)                       */
    uint64_t capacity;     /* bytes of the payload buffer                            */
    splitzip_meta *meta;   /* metadata of the payload                                */
    uint16_t *out;         /* decoded output (16-byte aligned)                       */
} splitzip_item;

/* One payload of a batched in-place decode (splitzip_decode_slot_batch);
 * the array lives in host memory, the pointers are device pointers with the
 * meaning they have for splitzip_decode_slot. */
typedef struct splitzip_slot_item {
    uint8_t *slot;               /* payload at its head; receives the n values   */
    uint64_t slot_bytes;
    const splitzip_meta *meta;
    const uint8_t *dec_lut;      /* the codebook's 16-entry dec_lut              */
    uint64_t n;
    uint8_t *stash;              /* scratch of stash_bytes >= comp_bytes         */
    uint64_t stash_bytes;
} splitzip_slot_item;

/* ABI version of the loaded library (SPLITZIP_ABI_VERSION). */
int splitzip_abi_version(void);

/* sizeof(splitzip_codebook) and sizeof(splitzip_meta) as compiled into the
 * library, for bindings that mirror the structs. */
void splitzip_struct_sizes(size_t *codebook_bytes, size_t *meta_bytes);

/* Human-readable name of a status code (static string, never NULL). */
const char *splitzip_status_string(int status);

/* Exact payload size for n elements with n_esc escapes (host function; the
 * layout rule above).  splitzip_payload_size(n, n) bounds every payload. */
uint64_t splitzip_payload_size(uint64_t n, uint64_t n_esc);

/* Pass schedule of the in-place decode of n elements (splitzip_decode_slot;
 * host only, no GPU work), for inspection and tests.  The slot holds the
 * payload (layout rule above) and receives 2n output bytes; 8192-element
 * tile t writes bytes [16384 t, 16384 t + 2 len_t).  *t_min receives the
 * first tile whose output starts at or past the dense sections' end.  Tiles
 * whose output starts at or past comp_bytes run in pass 1; the tiles from
 * *t_min up to those run in the last pass; a tile w below *t_min runs in
 * pass p(w), where p(w) >= k exactly when lo[k] <= w < hi[k] (k = 2 ..
 * used passes; lo[2] = 0, hi[2] = *t_min).  lo and hi are host arrays of
 * passes + 1 entries; the entries of levels above the passes used, and [0]
 * and [1], are set to 0.  Returns the number of passes used (`passes`, or 2
 * should the schedule not apply), or 0 for passes outside [2, 8], n above
 * SPLITZIP_MAX_N or a NULL pointer. */
uint32_t splitzip_slot_schedule(uint64_t n, uint32_t passes, uint64_t *t_min, uint64_t *lo,
                                uint64_t *hi);

/* Bytes of device workspace needed by calibrate and encode for tensors of up
 * to n elements (host function): about n/4 bytes plus a fixed ~1.2 MB.  Encode
 * keeps one escape count per 8192-element tile and stages up to 512 escapes
 * per tile until their final ranks are known; a tile with more has them
 * derived from the input again.  A workspace of S bytes serves every n with
 * splitzip_workspace_size(n) <= S. */
size_t splitzip_workspace_size(uint64_t n);

/* Bytes of workspace needed by the batched calls on `count` tensors of the
 * given element counts (host array); also enough for any single call on one
 * of them. */
size_t splitzip_workspace_size_batch(const uint64_t *n, uint32_t count);

/* Zero-fill the calibrate area of a workspace (enqueues a fill kernel).
 * Optional: no call needs the workspace to hold any particular value
 * beforehand (its arrival counters carry a tag per call, so a value left
 * by an interrupted call, by another process or by a stray write is simply
 * replaced).  One workspace must not be used by two calls that can run at
 * the same time.
 * Errors: INVALID (null or unaligned d_ws, ws_bytes below the minimum), HIP. */
int splitzip_workspace_init(void *d_ws, size_t ws_bytes, void *stream);

/* Calibrate the top-16 exponent codebook of one tensor (page 1,
 * calibrate_codebook): 256-bin exponent histogram, then the 16 most frequent
 * exponents (count descending, exponent ascending on ties) receive codes
 * 0..15.
 *   d_x   n BF16 values as uint16 bit patterns (16-byte aligned, device)
 *   d_cb  output codebook (device)
 *   d_ws  initialised workspace of ws_bytes >= splitzip_workspace_size(n)
 * Errors: INVALID, WORKSPACE, HIP. */
int splitzip_calibrate(const uint16_t *d_x, uint64_t n, splitzip_codebook *d_cb, void *d_ws,
                       size_t ws_bytes, void *stream);

/* Encode one tensor with a codebook (page 1, encode_torch and
 * assemble_payload).  The codebook may come from another tensor: every
 * exponent without a code becomes an escape.
 *   d_payload  output buffer of `capacity` bytes (16-byte aligned, device);
 *              bytes [0, comp_bytes) receive the payload, bytes beyond are
 *              not touched.
 *   d_meta     output metadata (device); meta->status = SPLITZIP_ERR_CAPACITY
 *              when capacity < comp_bytes (then only the dense sections and
 *              the escapes that fit are written, and comp_bytes holds the
 *              size needed).
 * Synchronous errors: INVALID, CAPACITY (capacity below
 * splitzip_payload_size(n, 0)), WORKSPACE, HIP. */
int splitzip_encode(const uint16_t *d_x, uint64_t n, const splitzip_codebook *d_cb,
                    uint8_t *d_payload, uint64_t capacity, splitzip_meta *d_meta, void *d_ws,
                    size_t ws_bytes, void *stream);

/* splitzip_encode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid it): the same
 * computation and output, with no workspace argument.  Its scratch is a
 * SPLITZIP_NOALLOC_SCRATCH_BYTES array in device memory the library owns
 * (each device that runs the call holds its own copy until the process
 * ends); no call allocates or frees memory.  Every call on one device shares
 * that device's array: calls that may run at the same time on one device
 * (on different streams, or a graph replay overlapping a call) race and
 * must not be issued; calls ordered on one stream are fine, as nothing in
 * the array needs any value before a call.
 * Synchronous errors: as splitzip_encode, and WORKSPACE when n exceeds
 * SPLITZIP_NOALLOC_MAX_N (16,312 encode tiles of 8192 elements). */
#define SPLITZIP_NOALLOC_SCRATCH_BYTES (32ull << 20)
#define SPLITZIP_NOALLOC_MAX_N 133627904ull
int splitzip_encode_noalloc(const uint16_t *d_x, uint64_t n, const splitzip_codebook *d_cb,
                            uint8_t *d_payload, uint64_t capacity, splitzip_meta *d_meta,
                            void *stream);

/* Encode with another escape-stream chunk size (page 1, encode, parameter
 * chunk_size): chunk id = element / chunk_size, local position = element %
 * chunk_size.  Only the escape sections and meta->chunk_size differ from
 * splitzip_encode, which is this call with chunk_size = 1024.
 * Synchronous errors as for splitzip_encode, and INVALID unless
 * 1 <= chunk_size <= 65536 (positions are uint16) and ceil(n / chunk_size)
 * <= 2^31 (chunk ids are int32). */
int splitzip_encode_chunked(const uint16_t *d_x, uint64_t n, const splitzip_codebook *d_cb,
                            uint32_t chunk_size, uint8_t *d_payload, uint64_t capacity,
                            splitzip_meta *d_meta, void *d_ws, size_t ws_bytes, void *stream);

/* Decode a payload back to BF16 bit patterns (page 1, decode_torch): dense
 * 16-entry table lookup plus the escape patch.  Escapes are applied in any
 * order: a stream marked SPLITZIP_META_ASCENDING (every payload of
 * splitzip_encode) is patched tile by tile in the dense pass; any other
 * stream by a second pass that applies each escape at its index.
 *   d_payload  payload laid out as d_meta describes (device, 16-byte aligned),
 *              payload_bytes readable bytes; a buffer shorter than the dense
 *              sections of n elements (splitzip_payload_size(n, 0)) is an
 *              argument error
 *   d_meta     metadata of the payload (device); meta->n must equal n, the
 *              offsets must follow the layout rule for (n, meta->n_esc) and
 *              comp_bytes must not exceed payload_bytes, else nothing is
 *              decoded and status bit 1 is set
 *   d_dec_lut  the codebook's 16-entry dec_lut (device)
 *   d_out      n uint16 outputs (device, 16-byte aligned, must not overlap
 *              the payload)
 *   d_status   optional (may be NULL) device int32 that the caller has set to
 *              0; decode ORs in 1 for inconsistent metadata (see d_meta),
 *              2 when an escape points outside the tensor,
 *              4 when a chunk-local position is >= chunk_size, 8 when escapes
 *              are not strictly increasing.  Decode never writes outside
 *              d_out[0..n).  Any chunk_size in [1, 65536] whose chunk ids fit
 *              int32 is accepted.
 * Synchronous errors: INVALID, HIP. */
int splitzip_decode(const uint8_t *d_payload, uint64_t payload_bytes, const splitzip_meta *d_meta,
                    const uint8_t *d_dec_lut, uint16_t *d_out, uint64_t n, int32_t *d_status,
                    void *stream);

/* In-place decode of a payload that occupies the head of its own output
 * buffer (page "splitzip_codec.py -- SplitZip codec adapter for
 * diffusers-dynamic-offloader", GpuSplitZipDecoder.decode_slot_into; page
 * "SplitZip in DDO -- VMM routes", the CUDA route: the transfer lands the
 * compressed bytes in the weight's own slot and the slot is expanded in place
 * on the upload stream).
 *   d_slot      buffer of slot_bytes >= max(2n, splitzip_payload_size(n, 0))
 *               bytes (device, 16-byte aligned); on entry bytes
 *               [0, comp_bytes) hold the payload, on completion bytes [0, 2n)
 *               hold the n decoded BF16 bit patterns
 *   d_meta      metadata of the payload (device), checked as for
 *               splitzip_decode; comp_bytes must not exceed slot_bytes nor
 *               stash_bytes, else the slot is left untouched and status bit 1
 *               is set
 *   d_dec_lut   the codebook's 16-entry dec_lut (device)
 *   d_stash     caller-owned device scratch of stash_bytes >= comp_bytes
 *               (splitzip_payload_size(n, n_esc)) bytes, 16-byte aligned, not
 *               overlapping the slot; it receives what a later step reads
 *               after the slot head has been overwritten (see below)
 *   d_status    optional, as for splitzip_decode (escapes are re-applied from
 *               the decoded sign and mantissa)
 * Two to six kernels on `stream` (and, with d_status, a validation
 * kernel), in passes over 8192-element tiles (splitzip_slot_schedule): the
 * first decodes the tiles whose output lies past the payload and copies to
 * the stash the escape sections, the packed nibbles of every other tile and
 * the sign/mantissa bytes of the tiles the last pass decodes; each later
 * pass decodes the tiles whose output covers only bytes that no tile of the
 * same or a later pass still reads from the slot, the last pass the rest
 * from the stash.  Calls that share a stash must be ordered on one stream.
 * The kernels' workgroups depend on no other workgroup, so the decode
 * shares the GPU with concurrent work as any kernel does (on a GPU the
 * decode has to itself, splitzip_decode_slot_batch_resident is faster for
 * single slots and slower for groups).  The environment variable SPLITZIP_SLOT_LAUNCH selects a form for
 * every slot decode of the process: "two" (this one), "one" (the resident
 * form) or "coop" (the resident form, its first kernel launched
 * cooperatively); SPLITZIP_SLOT_PASSES (2..8) fixes this form's number of
 * passes (2: every overlapping tile's inputs stashed, one pass decoding them
 * all), which is otherwise chosen per launch (up to 6, fewer when the last
 * pass would not fill the GPU); SPLITZIP_SLOT_WAIT_US sets the resident form's
 * bounded wait in microseconds (0: nearly every barrier gives up).
 * Synchronous errors: INVALID (also for overlapping slot and stash), HIP. */
int splitzip_decode_slot(uint8_t *d_slot, uint64_t slot_bytes, const splitzip_meta *d_meta,
                         const uint8_t *d_dec_lut, uint64_t n, uint8_t *d_stash,
                         uint64_t stash_bytes, int32_t *d_status, void *stream);

/* In-place decode of a group of slots (page "SplitZip in DDO -- VMM routes",
 * "Route B (fallback)": the staging route expands the slots of an execution
 * group after their upload, on the upload stream): the
 * same result as splitzip_decode_slot on every item in order, up to 32
 * items sharing each launch of its kernels.  Each item needs its own
 * stash; no slot or stash may overlap another item's buffers.  d_status
 * (optional) collects the status bits of all items.
 * Synchronous errors: INVALID (any item; nothing is enqueued), HIP. */
int splitzip_decode_slot_batch(const splitzip_slot_item *items, uint32_t count, int32_t *d_status,
                               void *stream);

/* In-place decode of a group of slots (page "SplitZip in DDO -- VMM routes",
 * as splitzip_decode_slot_batch): the same result, in a form that needs the
 * whole grid resident at once and pays off for single slots on a GPU that the
 * decode has to itself (e.g. a bulk restore between compute phases).  Two kernels per 32
 * items on `stream`.  The first is an ordinary launch of as many workgroups
 * as the GPU keeps resident at once: each decodes its tiles whose output
 * lies past the payload, loads the inputs of up to three whole tiles whose
 * output overlaps the payload into registers, waits on a grid barrier (every
 * load of the payload done) and then writes them, one barrier per item (one
 * item's stores overlap the next one's loads); overlapping tiles beyond that
 * reach, a partial last one, and the escape sections when a later step needs
 * them go through the stash.  The barrier's wait is bounded: when concurrent
 * work keeps part of the grid from being placed (checked after about 20 us)
 * or the wait passes 200 us, the launch gives up, stashes its held tiles
 * instead and leaves them, and every later item of the launch, to the
 * second kernel -- the same result, later (then slower than
 * splitzip_decode_slot_batch, which shares the GPU without waiting).  The
 * second kernel also decodes an item whose escape stream is not marked
 * ascending (its escapes applied by index); otherwise it reads one word and
 * ends.  The barrier's counters live in the library, 64 blocks per device,
 * one per stream that used one last: calls may run at the same time on at
 * most 64 streams of a device.  Arguments, stash rules and errors as for
 * splitzip_decode_slot_batch. */
int splitzip_decode_slot_batch_resident(const splitzip_slot_item *items, uint32_t count,
                                        int32_t *d_status, void *stream);

/* Batched forms of calibrate / encode / decode for many tensors with one
 * codebook each (the per-tensor granularity of page 1, SplitZipCodebook):
 * the same computation as calling the single-tensor function on every item
 * in order, with the tensors of up to 32 consecutive items sharing each
 * kernel launch (encode uses chunk_size 1024).  `items` is a host array of `count` entries, read before the
 * call returns.  Error codes as for the single-tensor calls; on an argument
 * error nothing is enqueued.  Encode needs a workspace of at least
 * splitzip_workspace_size_batch(n, count) bytes.  For decode, d_status (may
 * be NULL) collects the status bits of all items. */
int splitzip_calibrate_batch(const splitzip_item *items, uint32_t count, void *d_ws,
                             size_t ws_bytes, void *stream);
int splitzip_encode_batch(const splitzip_item *items, uint32_t count, void *d_ws,
                          size_t ws_bytes, void *stream);
int splitzip_decode_batch(const splitzip_item *items, uint32_t count, int32_t *d_status,
                          void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPLITZIP_H */
