// splitzip.hip -- SplitZip lossless BF16 codec for MI355X (gfx950): HIP
// kernels and the C ABI declared in include/splitzip.h.
//
// Method and wire format: page "splitzip_codec.py -- SplitZip codec adapter
// for diffusers-dynamic-offloader" (module docstring "Method" and "Payload
// layout"; functions calibrate_codebook, assemble_payload, encode_torch,
// decode_torch) and page "SplitZip in DDO -- VMM routes" ("Invariants common
// to both routes", item 1).  Ties among equally frequent exponents are broken
// by ascending exponent value.
//
// All work is integer and streams through HBM; nothing is a contraction, so
// no matrix cores.  Two measured properties of this part shape the kernels:
// device-scope atomics on one address serialise (about 12 ns each), and an
// agent-scope fence (L2 write-back + invalidate) issued by every workgroup
// costs tens of microseconds.  So no kernel takes a global ticket, keeps a
// per-workgroup counter on one address or issues a device fence.
//
// Every kernel works on a batch of up to kMaxBatch tensors whose descriptors
// travel by value in the kernel arguments; a single-tensor call is a batch of
// one.  Workgroups find their tensor by a binary search over the batch's
// prefix of workgroups (or tiles) per tensor.
//   k_calibrate   exponent histogram in LDS (64 lane-private copies, so equal
//                 exponents in a wave never hit one bank), merged with device
//                 atomics into 16 spread copies per tensor; the last arriver
//                 of each group of 16 workgroups reports to the tensor's top
//                 counter and the tensor's last group folds the copies and
//                 runs the top-16 select.
//   k_encode      one 8192-element tile per workgroup: 16-byte loads, code
//                 table in LDS, nibble packing, sign/mantissa bytes, wave
//                 ballots to rank the tile's escapes; the escape count goes
//                 to the workspace, and so do the escapes themselves when
//                 there are at most 512.  Tiles never talk to each other.
//   k_encode_sums (large launches only) escapes per block of tiles and per
//                 256-tile superblock, so escape placement needs few loads.
//   k_encode_tail every workgroup takes a block of 1-64 tiles, finds the rank
//                 of its first escape and the tensor's escape count, and
//                 writes chunk id, chunk-local position and raw exponent of
//                 each of its escapes at its final rank (staged ones copied,
//                 the others derived from the input again); the tensor's
//                 first workgroup writes the padding and the metadata.
//   k_decode      one 8192-element tile per workgroup:
//                 pk + sm -> bf16 through a 256-entry pair table in LDS and
//                 16-byte stores; meanwhile one wave finds the tile's escapes
//                 by a search of the sorted chunk ids, and after a workgroup
//                 barrier they are patched over the dense output (only for
//                 streams the metadata marks ascending).
//   k_decode_check  after every decode: applies the escapes of streams not
//                 marked ascending by scatter, in any order; with a status
//                 word it validates every escape and re-applies it.
//   k_decode_slot_stage / k_decode_slot_level  in-place decode of payloads
//                 that sit at the head of their own output buffers, in
//                 passes: the first decodes the tiles past the payload and
//                 stashes what later passes read after the slot head has been
//                 overwritten; each later pass decodes the tiles whose output
//                 no tile of that or a later pass still reads.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "splitzip.h"

namespace {

// Build-time tuning knobs; the defaults are the measured best on MI355X.
#ifndef SPLITZIP_ENC_UNITS
#define SPLITZIP_ENC_UNITS 4        // encode: 8-element units per thread per tile
#endif
#ifndef SPLITZIP_TAIL_MIN_TILES
#define SPLITZIP_TAIL_MIN_TILES 1   // escape placement: fewest tiles per workgroup
#endif
#ifndef SPLITZIP_TAIL_TARGET_WGS
#define SPLITZIP_TAIL_TARGET_WGS 1024   // ... and the workgroup count it aims at
#endif
#ifndef SPLITZIP_TAIL_DIRECT
#define SPLITZIP_TAIL_DIRECT (1u << 22)   // tile counts the tail launch may read without sums
#endif
#ifndef SPLITZIP_TAIL_THREADS
#define SPLITZIP_TAIL_THREADS 256   // escape placement workgroup size
#endif

constexpr uint32_t kChunk = SPLITZIP_CHUNK;
constexpr int kMaxBatch = 32;                 // tensors per launch
constexpr int kThreads = 256;                 // encode / decode workgroup
constexpr int kUnit = 8;                      // elements per 16-byte load
constexpr int kEncUnits = SPLITZIP_ENC_UNITS; // units per thread per tile
constexpr int kEncTile = kThreads * kUnit * kEncUnits;   // 8192 elements
constexpr int kCalThreads = 1024;
constexpr int kCalMaxGrid = 512;              // workgroups per tensor, at most
constexpr int kCalTarget = 2;                 // resident 1024-thread workgroups per CU
constexpr uint64_t kCalLongLoop = 32;         // ... one instead when each still loops this often
constexpr int kCalGroup = 16;                 // arrivals per first-level counter
constexpr int kCalSingle = 32;                // one counter when a tensor has at most this many workgroups
constexpr int kCalCopies = 16;                // global histogram copies per tensor
constexpr int kBinCountBits = 37;             // a copy's bin: tag << 37 | count (counts < 2^37)
constexpr uint64_t kBinCountMask = (1ull << kBinCountBits) - 1;
// Encode tiles placed per tail workgroup: chosen per launch, a power of two
// from kTailMinTiles (enough workgroups to spread dense escape streams over
// the GPU) to kTailMaxTiles (fewer workgroups when the launch has many tiles).
constexpr int kTailMinTiles = SPLITZIP_TAIL_MIN_TILES;
constexpr int kTailMaxTiles = 64;
constexpr uint64_t kTailTargetWgs = SPLITZIP_TAIL_TARGET_WGS;
constexpr int kTailThreads = SPLITZIP_TAIL_THREADS;
constexpr int kSuperTiles = 256;              // tiles per second-level count sum
constexpr uint64_t kTailDirect = SPLITZIP_TAIL_DIRECT;
constexpr uint32_t kMaxChunk = 65536;         // chunk-local positions are uint16
#ifndef SPLITZIP_DEC_THREADS
#define SPLITZIP_DEC_THREADS 256    // decode workgroup
#endif
#ifndef SPLITZIP_DEC_UNITS
#define SPLITZIP_DEC_UNITS 4        // decode: 8-element units per thread per tile
#endif
constexpr int kDecThreads = SPLITZIP_DEC_THREADS;
constexpr int kDecUnits = SPLITZIP_DEC_UNITS;
constexpr int kDecStaged = 512;               // decode: escapes per tile above which sm goes to LDS
// Encode: a tile stages at most kStageCap escapes in the workspace; the
// placement kernel derives the escapes of a tile with more from the input
// again (16 KB read instead of 8 bytes staged and read back per escape).
constexpr uint32_t kStageCap = 512;

// Workspace layout (bytes).  The calibrate area: per tensor of a launch a
// slot with its arrival counters (64 bytes apart) and its global histogram
// copies, all tagged per call (see tagged_arrive and k_calibrate), so that
// nothing needs clearing between calls; then the encode tile counts, the
// count sums per tail block and per superblock, and the escape staging area,
// whose sizes depend only on the workspace size.  Nothing in the workspace
// needs to hold any particular value before a call.
constexpr size_t kCalCounters = 1 + kCalMaxGrid / kCalGroup;             // top + groups
// generation word, counters, uint64 copies[16][256]
constexpr size_t kCalSlot = 64 + 64 * kCalCounters + 8 * 256 * kCalCopies;
constexpr size_t kWsTiles = (kCalSlot * kMaxBatch + 255) & ~size_t(255);
static_assert(kCalSlot % 64 == 0, "copies start on a cache line");
constexpr size_t kWsSlack = 64;
static_assert(kWsTiles % 256 == 0, "alignment");
static_assert(kCalThreads >= 256 && ((uint64_t)SPLITZIP_MAX_N >> kBinCountBits) == 0,
              "calibrate: a thread per bin, counts fit a copy's bin");
static_assert(kSuperTiles == kThreads && kTailMaxTiles <= 64 && kTailMaxTiles <= kTailThreads &&
                  kTailThreads % 64 == 0 && (kTailMinTiles & (kTailMinTiles - 1)) == 0 &&
                  kTailMinTiles <= kTailMaxTiles && kSuperTiles / kTailMinTiles <= kTailThreads,
              "count sums: one tile per thread, whole tail blocks per superblock");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef u32x2 u32x2_a4 __attribute__((aligned(4)));

__host__ __device__ constexpr uint64_t align4(uint64_t v) { return (v + 3u) & ~uint64_t(3); }
__host__ __device__ constexpr uint64_t align16(uint64_t v) { return (v + 15u) & ~uint64_t(15); }

struct Layout {
    uint64_t n_pairs, off_sm, off_cid, off_lpos, off_ev, total;
};

// Page 1, assemble_payload: section offsets for n elements and e escapes.
__host__ __device__ inline Layout layout_of(uint64_t n, uint64_t e) {
    Layout L;
    L.n_pairs = (n + 1) / 2;
    L.off_sm = align4(L.n_pairs);
    L.off_cid = align4(L.off_sm + n);
    L.off_lpos = L.off_cid + 4 * e;
    L.off_ev = align4(L.off_lpos + 2 * e);
    L.total = L.off_ev + e;
    return L;
}

// Tile capacity and staging area of a workspace of ws_bytes.
struct WsPlan {
    uint64_t t_max;       // encode tiles the workspace holds
    uint64_t off_count;   // uint32[t_max] escapes per tile
    uint64_t off_bsum;    // uint32[t_max / kTailMinTiles + 64] escapes per tail workgroup
    uint64_t off_ssum;    // uint32[t_max / kSuperTiles + 64] escapes per kSuperTiles tiles
    uint64_t off_stage;   // uint32[t_max * kStageCap] staged escapes
};

// per tile: its count, its share of the block and superblock sums, its stage
constexpr uint64_t kWsPerTile =
    4 + 4 / kTailMinTiles + 1 + 4 * (uint64_t)kStageCap;
constexpr uint64_t kWsFixed = kWsTiles + kWsSlack + 4 * 128;
static_assert(kTailMinTiles <= 4, "block sums fit the per-tile budget");

// head: bytes before the encode area (the calibrate area of a workspace;
// none in an encode-only buffer)
__host__ constexpr WsPlan ws_plan(size_t ws_bytes, size_t head = kWsTiles) {
    WsPlan P{0, 0, 0, 0, 0};
    if (ws_bytes < head + kWsSlack + 4 * 128) return P;
    P.t_max = (ws_bytes - head - kWsSlack - 4 * 128) / kWsPerTile;
    P.off_count = head;
    P.off_bsum = align16(P.off_count + 4 * P.t_max);
    P.off_ssum = align16(P.off_bsum + 4 * (P.t_max / kTailMinTiles + 64));
    P.off_stage = align16(P.off_ssum + 4 * (P.t_max / kSuperTiles + 64));
    return P;
}
static_assert(kWsFixed == kWsTiles + kWsSlack + 4 * 128, "workspace plan");

// Chunk id and chunk-local position of element i (shift and mask when the
// chunk size is a power of two).
__host__ __device__ inline void chunk_split(uint64_t i, uint32_t chunk, uint64_t &cid,
                                            uint32_t &pos) {
    if ((chunk & (chunk - 1)) == 0) {
        const int sh = __builtin_ctz(chunk);
        cid = i >> sh;
        pos = (uint32_t)(i & (chunk - 1));
    } else {
        cid = i / chunk;
        pos = (uint32_t)(i - cid * chunk);
    }
}

// A chunk size the wire format can carry for n elements: positions fit
// uint16 and chunk ids int32.
__host__ __device__ inline bool chunk_ok(uint64_t n, uint64_t chunk) {
    return chunk >= 1 && chunk <= kMaxChunk && (n + chunk - 1) / chunk <= (1ull << 31);
}

// popcount of the bits of m held by lanes below this one
__device__ inline uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ inline uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) v += __shfl_xor(v, s, 64);
    return v;
}

// Wait until every vector memory operation this wave issued has completed
// (for atomics: performed at the device coherence point).
__device__ inline void wait_vector_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Tagged arrival counters: a 64-bit word (tag << 32 | arrivals), `total`
// arrivals per call.  Every arriver (or, in a tree, a member that the
// arriver's own arrival depends on) claims the word for the call's tag
// before it arrives: a word with another tag (junk, an interrupted call,
// the last call) is replaced by (tag << 32); a claim that finds the tag
// leaves the word alone.  The last arrival puts (tag << 32) back, so that a
// replay of a captured graph (the same tag again) also starts from zero.
// `cur` is a value of *c read earlier in this call (or the word's value now).
__device__ inline void tagged_claim(uint64_t *c, uint64_t cur, uint64_t want, uint64_t tag_mask) {
    // a failed exchange leaves the current value in cur: normally another
    // arrival's claim, so the loop ends; bounded regardless
    for (int k = 0; k < 64 && (cur & tag_mask) != want; ++k)
        if (__hip_atomic_compare_exchange_strong(c, &cur, want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
            break;
}
__device__ inline uint64_t ld_agent(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void counter_claim(uint64_t *c, uint64_t cur, uint32_t tag) {
    tagged_claim(c, cur, (uint64_t)tag << 32, ~0ull << 32);
}
// Returns true for the last of `total` arrivals of the call, which leaves
// (reset_tag << 32) behind: the same tag for a replay of the same
// arguments, or the next call's tag when it is known.
__device__ inline bool tagged_arrive(uint64_t *c, uint64_t total, uint32_t reset_tag) {
    const uint64_t prev = __hip_atomic_fetch_add(c, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = (uint32_t)prev + 1ull == total;
    if (last)
        __hip_atomic_store(c, (uint64_t)reset_tag << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return last;
}

// Last k in [0, count) with start[k] <= g, for start[0] = 0 <= g < start[count].
template <typename T>
__device__ inline uint32_t find_item(const T *start, uint32_t count, uint64_t g) {
    uint32_t lo = 0, hi = count;
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if ((uint64_t)start[mid] <= g) lo = mid; else hi = mid;
    }
    return lo;
}

// Page 1, docstring "Method": the exponent is bits 7..14 of the 16-bit view;
// the stored byte keeps bit 15 (sign) as its bit 7 and the 7 low mantissa bits.
__device__ inline uint32_t exp_lo(uint32_t w) { return (w >> 7) & 0xFFu; }
__device__ inline uint32_t exp_hi(uint32_t w) { return (w >> 23) & 0xFFu; }
__device__ inline uint32_t sm_of16(uint32_t b) { return ((b >> 8) & 0x80u) | (b & 0x7Fu); }
// Reconstruction: sign back to bit 15, exponent to bits 7..14.
__device__ inline uint32_t join16(uint32_t sm, uint32_t ex) {
    return ((sm & 0x80u) << 8) | (ex << 7) | (sm & 0x7Fu);
}

// Word k of a 4-word vector without dynamic register indexing.
__device__ inline uint32_t word_of(const u32x4 q, int k) {
    return k == 0 ? q.x : (k == 1 ? q.y : (k == 2 ? q.z : q.w));
}

// ---------------------------------------------------------------------------
// Calibrate (page 1, calibrate_codebook)
// ---------------------------------------------------------------------------

struct CalItem {
    const uint16_t *x;
    uint64_t n;
    splitzip_codebook *cb;
};

struct CalArgs {
    uint32_t count;
    uint32_t wg_start[kMaxBatch + 1];   // first workgroup of each tensor
    CalItem it[kMaxBatch];
    uint8_t *ws;                        // calibrate slots
    uint64_t ticket;                    // counter tags: ticket + tensor + 1
};

// (8 waves per SIMD: two 1024-thread workgroups per compute unit fit)
__global__ __launch_bounds__(kCalThreads, 8) void k_calibrate(CalArgs a) {
    __shared__ uint32_t hist[256 * 64];   // [exponent][lane]
    __shared__ uint32_t part[4 * 256];
    __shared__ __attribute__((aligned(16))) uint64_t key[256];
    __shared__ __attribute__((aligned(16))) uint64_t cand[64];
    __shared__ uint64_t wcov[4];
    __shared__ uint32_t wdist[4];
    __shared__ uint32_t proceed;

    const uint32_t item = find_item(a.wg_start, a.count, blockIdx.x);
    const CalItem I = a.it[item];
    const uint32_t wg = blockIdx.x - a.wg_start[item];
    const uint32_t nwg = a.wg_start[item + 1] - a.wg_start[item];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // The tensor's slot: generation word, arrival counters, global copies.
    // The call's tag is the generation the last call left behind, which
    // already tags every counter and bin; a word that is not a generation
    // (its low half is not the complement of its high half: junk, a fresh
    // workspace) gives way to a tag from the host's ticket, and counters
    // and bins with another tag are claimed for it (tagged_claim).  The
    // values this workgroup needs are read now and used after the
    // histogram, so in the common case nothing waits for them.
    uint64_t *genp = reinterpret_cast<uint64_t *>(a.ws + (size_t)item * kCalSlot);
    uint64_t *ctrs = genp + 8;
    uint64_t *copies = ctrs + 8 * kCalCounters;
    uint64_t *mine = copies + (wg % kCalCopies) * 256;
    const bool single = nwg <= (uint32_t)kCalSingle;
    uint64_t gw = 0, seen = 0, seen_top = 0, seen_grp = 0;
    if (tid <= 256) gw = ld_agent(genp);
    if (tid < 256) seen = ld_agent(mine + tid);
    if (tid == 256) {
        seen_top = ld_agent(ctrs);
        if (!single) seen_grp = ld_agent(ctrs + 8 * (1 + wg / kCalGroup));
    }
    uint32_t *hl = hist + lane;
    const uint64_t nvec = I.n >> 3;
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(I.x);
    // One contiguous range of 16-byte loads per workgroup, 4 loads in flight
    // per thread (measured 6.4-6.7 TB/s against 5.8-6.0 for loads interleaved
    // over the whole grid).  The first round goes out before the LDS
    // histogram is cleared.
    const uint64_t per = (nvec + nwg - 1) / nwg;
    const uint64_t vlo = (uint64_t)wg * per;
    const uint64_t nv = vlo + per < nvec ? vlo + per : nvec;
    constexpr uint64_t stride = kCalThreads;
    uint64_t v = vlo + tid;
    u32x4 q[4];
    if (v + 3 * stride < nv) {
#pragma unroll
        for (int k = 0; k < 4; ++k) q[k] = __builtin_nontemporal_load(xv + v + k * stride);
    }
    for (int i = tid; i < 256 * 64; i += kCalThreads) hist[i] = 0;
    __syncthreads();

    while (v + 3 * stride < nv) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                atomicAdd(hl + exp_lo(q[k][w]) * 64, 1u);
                atomicAdd(hl + exp_hi(q[k][w]) * 64, 1u);
            }
        }
        v += 4 * stride;
        if (v + 3 * stride < nv) {
#pragma unroll
            for (int k = 0; k < 4; ++k) q[k] = __builtin_nontemporal_load(xv + v + k * stride);
        }
    }
    for (; v < nv; v += stride) {
        u32x4 q = __builtin_nontemporal_load(xv + v);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            atomicAdd(hl + exp_lo(q[w]) * 64, 1u);
            atomicAdd(hl + exp_hi(q[w]) * 64, 1u);
        }
    }
    if (wg == 0 && (uint64_t)tid < (I.n & 7)) {
        uint32_t b = I.x[(nvec << 3) + tid];
        atomicAdd(hl + exp_lo(b) * 64, 1u);
    }
    __syncthreads();

    {   // fold the 64 lane copies: 4 threads per bin, staggered over banks
        const int bin = tid & 255, quarter = tid >> 8;
        uint32_t s = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) s += hist[bin * 64 + ((quarter * 16 + k + bin) & 63)];
        part[tid] = s;
    }
    __syncthreads();
    // Merge into one of kCalCopies global copies (few workgroups per
    // address, so the device atomics do not queue up behind each other).  A
    // bin holds tag << 37 | count: the first workgroup of a call to reach a
    // bin with another tag (junk, an interrupted call, the last call)
    // replaces it by the tag with count 0; adds leave the tag alone.
    const bool gen_ok = (uint32_t)gw == ~(uint32_t)(gw >> 32);
    const uint32_t tag = gen_ok ? (uint32_t)(gw >> 32) : (uint32_t)(a.ticket + item) + 1u;
    const uint32_t next = tag + 1u;
    const uint64_t btag = (uint64_t)tag << kBinCountBits;    // the tag's low 27 bits
    if (tid < 256) {
        tagged_claim(mine + tid, seen, btag, ~kBinCountMask);
        const uint32_t s = part[tid] + part[256 + tid] + part[512 + tid] + part[768 + tid];
        if (s) __hip_atomic_fetch_add(mine + tid, (uint64_t)s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_vector_memory();
    __syncthreads();

    // Arrival: with few workgroups one counter; else the last arriver of
    // each group of kCalGroup reports to the tensor's top counter (claimed
    // by the first workgroup of each group, whose arrival precedes the
    // group's report).  The last arriver of all sums the copies' bins that
    // carry this call's tag, then tags counters, bins and the generation
    // word for the next call.
    if (tid == 256) {
        bool go;
        if (single) {
            counter_claim(ctrs, seen_top, tag);
            go = tagged_arrive(ctrs, nwg, next);
        } else {
            const uint32_t g = wg / kCalGroup;
            const uint32_t gsize = min((uint32_t)kCalGroup, nwg - g * kCalGroup);
            if (wg % kCalGroup == 0) counter_claim(ctrs, seen_top, tag);
            counter_claim(ctrs + 8 * (1 + g), seen_grp, tag);
            go = tagged_arrive(ctrs + 8 * (1 + g), gsize, next) &&
                 tagged_arrive(ctrs, (nwg + kCalGroup - 1) / kCalGroup, next);
        }
        proceed = go;
    }
    __syncthreads();
    if (!proceed) return;
    uint64_t c = 0;
    if (tid < 256) {
        uint64_t copy[kCalCopies];
#pragma unroll
        for (int k = 0; k < kCalCopies; ++k) copy[k] = ld_agent(copies + k * 256 + tid);
        const uint64_t nbtag = (uint64_t)next << kBinCountBits;
#pragma unroll
        for (int k = 0; k < kCalCopies; ++k) {
            c += (copy[k] & ~kBinCountMask) == btag ? (copy[k] & kBinCountMask) : 0;
            __hip_atomic_store(copies + k * 256 + tid, nbtag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (tid == 0)
        __hip_atomic_store(genp, ((uint64_t)next << 32) | (uint64_t)~next, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    if (tid < 256) {
        // unique sort key: count first, then the smaller exponent value
        key[tid] = c ? ((c << 8) | (uint64_t)(255 - tid)) : 0;
    }
    __syncthreads();
    // Rank = number of larger keys, needed exactly only below 16.  First
    // each key's rank inside its group of 64 (4 threads per key, 16 keys
    // each): a key with 16 larger ones in its group has a rank of 16 or more,
    // so the candidates are the nonzero keys that rank below 16 in their
    // group (at most 64).  Every key larger than a key of global rank below
    // 16 is a candidate, and every key that is not one has at least the 16
    // candidates of its group above it, so a key's rank among the candidates
    // is its rank when that is below 16, and 16 or more otherwise.
    {
        const int bin = tid & 255, quarter = tid >> 8;
        const uint64_t own = key[bin];
        const u64x2 *kv = reinterpret_cast<const u64x2 *>(key + (bin & ~63) + quarter * 16);
        u64x2 kk[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) kk[j] = kv[j];
        uint32_t r = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) r += (kk[j].x > own ? 1u : 0u) + (kk[j].y > own ? 1u : 0u);
        part[tid] = r;
    }
    __syncthreads();
    if (tid < 256) {
        const uint32_t group_rank = part[tid] + part[256 + tid] + part[512 + tid] + part[768 + tid];
        const uint64_t own = key[tid];
        const bool keep = own != 0 && group_rank < 16;
        const uint64_t m = __ballot(keep);
        uint64_t *slots = cand + (tid >> 6) * 16;
        if (keep) slots[lanes_below(m)] = own;
        if (lane < 16 && (uint32_t)lane >= (uint32_t)__popcll(m)) slots[lane] = 0;
    }
    __syncthreads();
    {
        const int bin = tid & 255, quarter = tid >> 8;
        const uint64_t own = key[bin];
        const u64x2 *kv = reinterpret_cast<const u64x2 *>(cand + quarter * 16);
        u64x2 kk[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) kk[j] = kv[j];
        uint32_t r = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) r += (kk[j].x > own ? 1u : 0u) + (kk[j].y > own ? 1u : 0u);
        part[tid] = r;
    }
    __syncthreads();
    // codes; per wave the covered count and the distinct exponents, so that
    // one barrier gives the totals before the codebook is written
    uint32_t code = 16;
    if (tid < 256) {
        const uint32_t rank = part[tid] + part[256 + tid] + part[512 + tid] + part[768 + tid];
        code = (c > 0 && rank < 16) ? rank : 16u;
        uint64_t cov = code < 16 ? c : 0;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) cov += __shfl_xor(cov, off, 64);
        const uint32_t dist = (uint32_t)__popcll(__ballot(c > 0));
        if (lane == 0) {
            wcov[tid >> 6] = cov;
            wdist[tid >> 6] = dist;
        }
    }
    __syncthreads();
    if (tid < 256) {
        const uint32_t distinct = wdist[0] + wdist[1] + wdist[2] + wdist[3];
        const uint32_t n_codes = distinct < 16 ? distinct : 16u;
        splitzip_codebook *cb = I.cb;
        cb->enc_lut[tid] = (uint8_t)(code < 16 ? code : 0);
        cb->enc_lut_marked[tid] = (uint8_t)code;
        cb->common_lut[tid] = (uint8_t)(code < 16 ? 1 : 0);
        cb->counts[tid] = c;
        if (code < 16) cb->dec_lut[code] = (uint8_t)tid;
        if (tid < 16 && (uint32_t)tid >= n_codes) cb->dec_lut[tid] = 0;   // (other slots)
        if (tid == 0) {
            cb->n_codes = n_codes;
            cb->reserved = 0;
            cb->covered = wcov[0] + wcov[1] + wcov[2] + wcov[3];
            cb->total = I.n;
        }
    }
}

// ---------------------------------------------------------------------------
// Encode (page 1, encode_torch + assemble_payload)
// ---------------------------------------------------------------------------

struct EncItem {
    const uint16_t *x;
    uint64_t n;
    const splitzip_codebook *cb;
    uint8_t *payload;
    uint64_t capacity;
    splitzip_meta *meta;
    uint32_t chunk;                       // elements per chunk of the escape stream
};

struct EncArgs {
    uint32_t count;
    uint32_t blk_start[kMaxBatch + 1];    // first tail workgroup of each tensor
    uint32_t sup_start[kMaxBatch + 1];    // first superblock (kSuperTiles tiles) of each tensor
    uint64_t tile_start[kMaxBatch + 1];   // first tile of each tensor
    EncItem it[kMaxBatch];
    uint32_t *tile_count;                 // escapes per tile
    uint32_t *blk_sum;                    // escapes per tail workgroup, or null
    uint32_t *sup_sum;                    // escapes per superblock, or null
    uint32_t tail_tiles;                  // tiles per tail workgroup (power of two)
    uint32_t *stage;                      // per tile, up to kStageCap: (position << 8) | raw exponent
};

// One 8-element unit: codes -> 4 pk bytes, sign/mantissa -> 8 sm bytes,
// escape mask (bit j = element j escapes).
__device__ inline void encode_unit(const u32x4 q, const uint8_t *lut, uint32_t &pk,
                                   uint32_t &sm0, uint32_t &sm1, uint32_t &flags) {
    pk = 0;
    flags = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t w = q[k];
        const uint32_t m_even = lut[exp_lo(w)];
        const uint32_t m_odd = lut[exp_hi(w)];
        // table entry: nibble | (escape << 4), at most 31 (normalised when the
        // table is loaded); the even element takes the high nibble
        const uint32_t byte = ((m_even & 15u) << 4) | (m_odd & 15u);
        pk |= byte << (8 * k);
        flags |= ((m_even >> 4) | ((m_odd >> 4) << 1)) << (2 * k);
    }
    sm0 = sm_of16(q[0]) | (sm_of16(q[0] >> 16) << 8) | (sm_of16(q[1]) << 16) |
          (sm_of16(q[1] >> 16) << 24);
    sm1 = sm_of16(q[2]) | (sm_of16(q[2] >> 16) << 8) | (sm_of16(q[3]) << 16) |
          (sm_of16(q[3] >> 16) << 24);
}

// Marked-code table of a codebook in LDS (one entry per thread of the first
// 256).  Page 1, encode_torch: an exponent escapes when its marked code is
// above 15, and its nibble is the marked code's low 4 bits, whatever byte the
// caller's table holds.  Stored as nibble | (escape << 4), so that m >> 4 is
// exactly one flag bit.
__device__ inline void load_marked_table(const splitzip_codebook *cb, uint8_t *lut) {
    const int tid = threadIdx.x;
    if (tid < 256) {
        const uint32_t v = cb->enc_lut_marked[tid];
        lut[tid] = (uint8_t)((v & 15u) | (v > 15u ? 16u : 0u));
    }
}

// Escape mask of one 8-element unit (bit j: element j escapes).
__device__ inline uint32_t unit_flags(const u32x4 q, const uint8_t *lut) {
    uint32_t f = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        f |= ((uint32_t)(lut[exp_lo(q[k])] >> 4) | ((uint32_t)(lut[exp_hi(q[k])] >> 4) << 1)) << (2 * k);
    return f;
}

// Ranks of a tile's escapes in element order (unit, thread, element of the
// unit), from every thread's per-unit escape masks: first[u] is the rank of
// this thread's first escape in unit u; returns the tile's escape count.
// One workgroup barrier (after the per-wave totals are in `wtot`); the caller
// orders a later reuse of `wtot` behind another barrier.
__device__ inline uint32_t tile_ranks(const uint32_t *flags, uint32_t (*wtot)[4], uint32_t *first) {
    static_assert(kThreads == 256 && kTailThreads == 256, "four waves per tile workgroup");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t pre[kEncUnits];
#pragma unroll
    for (int u = 0; u < kEncUnits; ++u) {
        const uint32_t c = __builtin_popcount(flags[u]);   // 0..8: four bits
        const uint64_t any = __ballot(c != 0);
        uint32_t p = 0, tot = 0;
        if (any) {
#pragma unroll
            for (int bit = 0; bit < 4; ++bit) {
                const uint64_t m = __ballot((c >> bit) & 1u);
                p += lanes_below(m) << bit;
                tot += (uint32_t)__popcll(m) << bit;
            }
        }
        pre[u] = p;
        if (lane == 0) wtot[u][wave] = tot;
    }
    __syncthreads();
    uint32_t total = 0;
#pragma unroll
    for (int u = 0; u < kEncUnits; ++u) {
        uint32_t b = total;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            b += (w < wave) ? wtot[u][w] : 0u;
            total += wtot[u][w];
        }
        first[u] = b + pre[u];
    }
    return total;
}

// Dense sections of one tile, its escape count, and (up to kStageCap) its
// escapes staged in element order; no communication between tiles.
// Tile of workgroup b in a launch of G one-tile workgroups.  Workgroups go
// to the 8 XCDs in turn (b % 8), so with the plain order the XCDs work on
// interleaved tiles; a large launch instead gives each XCD 64 consecutive
// tiles in turn, which streams faster there (the encode's access pattern
// 6.25 against 5.89 TB/s over 2^30 elements, the decode's 6.11 against 5.96;
// no gain, or a loss, below 2^28 elements).  The last G mod 512 workgroups
// keep the plain order.
constexpr uint64_t kXcdRun = 64;
constexpr uint64_t kXcdBlockedMin = 32768;   // tiles per launch
__device__ inline uint64_t launch_tile(uint64_t b, uint64_t G) {
    constexpr uint64_t B = 8 * kXcdRun;
    if (G < kXcdBlockedMin || b >= G / B * B) return b;
    const uint64_t x = b % 8, j = b / 8;   // the j-th workgroup of XCD x
    return (j / kXcdRun) * B + x * kXcdRun + j % kXcdRun;
}

__global__ __launch_bounds__(kThreads) void k_encode(EncArgs a) {
    __shared__ uint8_t lut[256];
    __shared__ uint32_t wtot[kEncUnits][4];

    const uint64_t gt = launch_tile(blockIdx.x, gridDim.x);
    const uint32_t item = find_item(a.tile_start, a.count, gt);
    const EncItem I = a.it[item];
    const uint64_t t = gt - a.tile_start[item];
    const uint64_t ntiles = a.tile_start[item + 1] - a.tile_start[item];
    const Layout L0 = layout_of(I.n, 0);

    const int tid = threadIdx.x;
    const uint64_t base = t * kEncTile;
    const bool full = base + kEncTile <= I.n;

    u32x4 q[kEncUnits];
    if (full) {
#pragma unroll
        for (int u = 0; u < kEncUnits; ++u) {
            const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
            q[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(I.x + i0));
        }
    }
    load_marked_table(I.cb, lut);
    __syncthreads();

    uint32_t flags[kEncUnits];
    if (full) {
#pragma unroll
        for (int u = 0; u < kEncUnits; ++u) {
            const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
            uint32_t pk, sm0, sm1;
            encode_unit(q[u], lut, pk, sm0, sm1, flags[u]);
            __builtin_nontemporal_store(pk, reinterpret_cast<uint32_t *>(I.payload + i0 / 2));
            u32x2 smv = {sm0, sm1};
            __builtin_nontemporal_store(smv,
                                        reinterpret_cast<u32x2_a4 *>(I.payload + L0.off_sm + i0));
        }
    } else {
        // last, partial tile: element-wise with bounds checks
#pragma unroll
        for (int u = 0; u < kEncUnits; ++u) {
            const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
            uint32_t codes[kUnit];
            uint32_t f = 0;
            uint32_t wv[4] = {0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < kUnit; ++j) {
                const uint64_t i = i0 + j;
                uint32_t b = 0;
                codes[j] = 0;
                if (i < I.n) {
                    b = I.x[i];
                    const uint32_t m = lut[exp_lo(b)];
                    codes[j] = m & 15u;
                    f |= (m >> 4) << j;
                    I.payload[L0.off_sm + i] = (uint8_t)sm_of16(b);
                }
                wv[j >> 1] |= b << (16 * (j & 1));
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint64_t i = i0 + 2 * k;
                if (i < I.n) {
                    const uint32_t lo = (i + 1 < I.n) ? codes[2 * k + 1] : 0u;
                    I.payload[i / 2] = (uint8_t)((codes[2 * k] << 4) | lo);
                }
            }
            q[u] = u32x4{wv[0], wv[1], wv[2], wv[3]};
            flags[u] = f;
        }
    }
    if (t == ntiles - 1 && tid == 0) {
        // zero padding between the dense sections (page 1: the payload is
        // assembled in a zero-filled buffer)
        for (uint64_t b = L0.n_pairs; b < L0.off_sm; ++b) I.payload[b] = 0;
        for (uint64_t b = L0.off_sm + I.n; b < L0.off_cid; ++b) I.payload[b] = 0;
    }

    uint32_t first[kEncUnits];
    const uint32_t tile_total = tile_ranks(flags, wtot, first);
    if (tid == 0) a.tile_count[gt] = tile_total;
    if (tile_total > kStageCap) return;   // placement derives them from the input again
    // every thread writes its own escapes at their ranks
    uint32_t *stage = a.stage + gt * kStageCap;
#pragma unroll
    for (int u = 0; u < kEncUnits; ++u) {
        uint32_t f = flags[u];
        uint32_t r = first[u];
        const uint32_t l0 = (uint32_t)u * (kThreads * kUnit) + tid * kUnit;
        while (f) {
            const int j = __builtin_ctz(f);
            f &= f - 1;
            const uint32_t w = word_of(q[u], j >> 1);
            const uint32_t ex = (j & 1) ? exp_hi(w) : exp_lo(w);
            stage[r++] = ((l0 + j) << 8) | ex;
        }
    }
}

// Inclusive scan of one value per thread across the workgroup (a multiple of
// 64 threads; lds_waves holds one word per wave).
__device__ inline uint32_t block_scan_incl(uint32_t v, uint32_t *lds_waves) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(v, off, 64);
        if (lane >= off) v += y;
    }
    if (lane == 63) lds_waves[wave] = v;
    __syncthreads();
    for (int w = 0; w < wave; ++w) v += lds_waves[w];
    return v;
}

// Count sums for large tensors: one workgroup per superblock of kSuperTiles
// tiles writes the escapes of each of its tail blocks (tail_tiles tiles) and
// of the whole superblock, so that a tail workgroup needs only a few dozen
// loads for its prefix.
__global__ __launch_bounds__(kThreads) void k_encode_sums(EncArgs a) {
    __shared__ uint32_t part[kThreads / 64];
    const uint32_t item = find_item(a.sup_start, a.count, blockIdx.x);
    const uint32_t sup = blockIdx.x - a.sup_start[item];
    const uint64_t tfirst = a.tile_start[item];
    const uint64_t ntiles = a.tile_start[item + 1] - tfirst;
    const int tid = threadIdx.x;
    const uint64_t t = (uint64_t)sup * kSuperTiles + tid;
    uint32_t v = t < ntiles ? a.tile_count[tfirst + t] : 0u;
    const uint64_t w = wave_sum_u64(v);
    if ((tid & 63) == 0) part[tid >> 6] = (uint32_t)w;
    // sums over aligned groups of tail_tiles (<= 64) lanes
    const uint32_t tt = a.tail_tiles;
    uint32_t g = v;
    for (uint32_t off = 1; off < tt; off <<= 1) g += __shfl_xor(g, (int)off, 64);
    __syncthreads();
    const uint64_t blk = (uint64_t)sup * (kSuperTiles / tt) + tid / tt;
    const uint64_t nblk = a.blk_start[item + 1] - a.blk_start[item];
    if (tid % tt == 0 && blk < nblk) a.blk_sum[a.blk_start[item] + blk] = g;
    if (tid == 0) {
        uint32_t sum = 0;
#pragma unroll
        for (int k = 0; k < kThreads / 64; ++k) sum += part[k];
        a.sup_sum[blockIdx.x] = sum;
    }
}

// Sum of src[0, n) and of src[0, split) for this thread's share, with
// 16-byte loads (four counts each, four in flight per thread: a single round
// trip up to 4096 entries, the tile counts of a 2^25-element tensor); the
// counts before the first 16-byte boundary and after the last whole load one
// by one.  Every placement workgroup reads all of its tensor's counts, so
// this read is most of a single tensor's placement: 16-byte loads took it
// from 3.96 to 2.80 us per workgroup against 4-byte ones (timestamped copy
// of the kernel, 2^25 elements, 1,024 workgroups).
__device__ inline void sum_prefix(const uint32_t *src, uint64_t n, uint64_t split,
                                  uint64_t &before, uint64_t &all) {
    const int tid = threadIdx.x;
    const uint64_t h0 = ((16u - ((uintptr_t)src & 15u)) & 15u) / 4;   // src is 4-byte aligned
    const uint64_t h = h0 < n ? h0 : n;
    if ((uint64_t)tid < h) {
        all += src[tid];
        before += (uint64_t)tid < split ? src[tid] : 0u;
    }
    const u32x4 *v = reinterpret_cast<const u32x4 *>(src + h);
    const uint64_t nv = (n - h) / 4;
    constexpr int kIn = 4;
    for (uint64_t q0 = 0; q0 < nv; q0 += kIn * kTailThreads) {
        u32x4 c[kIn];
#pragma unroll
        for (int j = 0; j < kIn; ++j) {
            const uint64_t q = q0 + j * kTailThreads + tid;
            c[j] = q < nv ? v[q] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < kIn; ++j) {
            const uint64_t k = h + 4 * (q0 + j * kTailThreads + tid);   // index of c[j].x
            all += (uint64_t)c[j].x + c[j].y + c[j].z + c[j].w;
            before += (k < split ? c[j].x : 0u) + (k + 1 < split ? c[j].y : 0u) +
                      (k + 2 < split ? c[j].z : 0u) + (k + 3 < split ? c[j].w : 0u);
        }
    }
    for (uint64_t k = h + 4 * nv + tid; k < n; k += kTailThreads) {
        all += src[k];
        before += k < split ? src[k] : 0u;
    }
}

// Escape of rank r, staged as (position in tile << 8) | raw exponent for the
// tile starting at element tile_base: chunk id, chunk-local position and raw
// exponent at their offsets (the chunk ids that fit are written even when
// the payload does not fit, as the capacity error reports).
__device__ inline void place_escape(const EncItem &I, const Layout &L, bool fits,
                                    uint64_t tile_base, uint32_t word, uint64_t r) {
    const uint64_t i = tile_base + (word >> 8);
    uint64_t cid;
    uint32_t pos;
    chunk_split(i, I.chunk, cid, pos);
    if (L.off_cid + 4 * r + 4 <= I.capacity)
        *reinterpret_cast<uint32_t *>(I.payload + L.off_cid + 4 * r) = (uint32_t)cid;
    if (fits) {
        *reinterpret_cast<uint16_t *>(I.payload + L.off_lpos + 2 * r) = (uint16_t)pos;
        I.payload[L.off_ev + r] = (uint8_t)(word & 0xFFu);
    }
}

// One 8-element unit of bf16 bits at element i0 (zeros past n): a 16-byte
// load when the whole tile is in range, else element by element.
__device__ inline u32x4 load_unit(const uint16_t *x, uint64_t n, uint64_t i0, bool full) {
    if (full) return *reinterpret_cast<const u32x4 *>(x + i0);
    // last tile only: one element at a time keeps the register count down
    uint32_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
#pragma unroll 1
    for (int j = 0; j < kUnit; ++j) {
        const uint32_t v = (i0 + j < n ? (uint32_t)x[i0 + j] : 0u) << (16 * (j & 1));
        const int k = j >> 1;
        w0 |= k == 0 ? v : 0u;
        w1 |= k == 1 ? v : 0u;
        w2 |= k == 2 ? v : 0u;
        w3 |= k == 3 ? v : 0u;
    }
    return u32x4{w0, w1, w2, w3};
}

// The kEncUnits units of this thread in the tile at element tb.
__device__ inline void load_tile(const EncItem &I, uint64_t tb, u32x4 *qt) {
    const bool full = tb + kEncTile <= I.n;
#pragma unroll
    for (int u = 0; u < kEncUnits; ++u)
        qt[u] = load_unit(I.x, I.n, tb + (uint64_t)u * (kThreads * kUnit) + threadIdx.x * kUnit, full);
}

// Escapes of one encode tile whose count exceeded the staging cap, derived
// from the input again (its values qt, loaded by the caller; the same table
// and the same ranks as k_encode) and written at ranks rank0 + r.  Every
// thread puts the position in tile and the raw exponent of each of its
// escapes into LDS by rank, shifted so that 16-byte blocks of LDS line up
// with 16-byte blocks of the position and exponent sections; the workgroup
// then writes the three sections 16 bytes per lane (4 chunk ids, 8
// positions, 16 exponents), the few ranks outside whole blocks one by one.
__device__ void rederive_tile(const EncItem &I, const Layout &L, bool fits, const uint8_t *lut,
                              uint32_t (*wtot)[4], uint16_t *rpos, uint8_t *rex, uint64_t tb,
                              uint64_t rank0, const u32x4 *qt) {
    const uint32_t tid = threadIdx.x;
    uint32_t flags[kEncUnits];
#pragma unroll
    for (int u = 0; u < kEncUnits; ++u) {
        const uint64_t i0 = tb + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
        const uint32_t valid = i0 + kUnit <= I.n ? 0xFFu : (i0 < I.n ? (1u << (I.n - i0)) - 1u : 0u);
        flags[u] = unit_flags(qt[u], lut) & valid;
        // one unit's table reads at a time: hoisting all of them costs occupancy
        __builtin_amdgcn_sched_barrier(0);
    }
    uint32_t first[kEncUnits];
    const uint32_t total = tile_ranks(flags, wtot, first);
    // byte addresses of rank 0 in the three sections and their offsets in a
    // 16-byte block (positions: in units of 2 bytes)
    uint8_t *dc = I.payload + L.off_cid + 4 * rank0;
    uint8_t *dl = I.payload + L.off_lpos + 2 * rank0;
    uint8_t *de = I.payload + L.off_ev + rank0;
    const uint32_t al = (uint32_t)((uintptr_t)dl & 15u) >> 1;
    const uint32_t ae = (uint32_t)((uintptr_t)de & 15u);
#pragma unroll
    for (int u = 0; u < kEncUnits; ++u) {
        uint32_t f = flags[u];
        uint32_t r = first[u];
        const uint32_t l0 = (uint32_t)u * (kThreads * kUnit) + tid * kUnit;
        while (f) {
            const int j = __builtin_ctz(f);
            f &= f - 1;
            const uint32_t w = word_of(qt[u], j >> 1);
            rpos[al + r] = (uint16_t)(l0 + j);
            rex[ae + r] = (uint8_t)((j & 1) ? exp_hi(w) : exp_lo(w));
            ++r;
        }
    }
    __syncthreads();
    // Chunk ids in 32-bit arithmetic when the chunk size is a power of two
    // that divides the tile (then the tile starts a chunk).
    const uint32_t chunk = I.chunk;
    const bool pow2 = (chunk & (chunk - 1)) == 0 && chunk <= (uint32_t)kEncTile;
    if (fits && pow2) {
        const int sh = __builtin_ctz(chunk);
        const uint32_t cbase = (uint32_t)(tb >> sh), msk = chunk - 1u;
        const uint32_t nth = kTailThreads;
        {   // chunk ids: 4 ranks per 16-byte block
            uint32_t *d32 = reinterpret_cast<uint32_t *>(dc);
            uint32_t h = ((16u - (uint32_t)((uintptr_t)dc & 15u)) & 15u) >> 2;
            h = h < total ? h : total;
            const uint32_t nb = (total - h) >> 2;
            u32x4 *dv = reinterpret_cast<u32x4 *>(d32 + h);
            for (uint32_t c = tid; c < nb; c += nth) {
                const uint16_t *p = rpos + al + h + 4 * c;
                dv[c] = u32x4{cbase + ((uint32_t)p[0] >> sh), cbase + ((uint32_t)p[1] >> sh),
                              cbase + ((uint32_t)p[2] >> sh), cbase + ((uint32_t)p[3] >> sh)};
            }
            // fewer than 4 ranks before the blocks and after them
            const uint32_t k = tid < h ? tid : h + 4 * nb + (tid - h);
            if (tid < h + 4 && k < total) d32[k] = cbase + ((uint32_t)rpos[al + k] >> sh);
        }
        {   // positions: 8 ranks per block, LDS blocks aligned with them
            uint16_t *d16 = reinterpret_cast<uint16_t *>(dl);
            uint32_t h = (8u - al) & 7u;
            h = h < total ? h : total;
            const uint32_t nb = (total - h) >> 3;
            const u32x4 *src = reinterpret_cast<const u32x4 *>(rpos + al + h);
            u32x4 *dv = reinterpret_cast<u32x4 *>(d16 + h);
            const uint32_t m2 = msk | (msk << 16);
            for (uint32_t c = tid; c < nb; c += nth) {
                const u32x4 v = src[c];
                dv[c] = u32x4{v.x & m2, v.y & m2, v.z & m2, v.w & m2};
            }
            const uint32_t k = tid < h ? tid : h + 8 * nb + (tid - h);
            if (tid < h + 8 && k < total) d16[k] = (uint16_t)((uint32_t)rpos[al + k] & msk);
        }
        {   // raw exponents: 16 ranks per block, LDS blocks aligned with them
            uint32_t h = (16u - ae) & 15u;
            h = h < total ? h : total;
            const uint32_t nb = (total - h) >> 4;
            const u32x4 *src = reinterpret_cast<const u32x4 *>(rex + ae + h);
            u32x4 *dv = reinterpret_cast<u32x4 *>(de + h);
            for (uint32_t c = tid; c < nb; c += nth) dv[c] = src[c];
            const uint32_t k = tid < h ? tid : h + 16 * nb + (tid - h);
            if (tid < h + 16 && k < total) de[k] = rex[ae + k];
        }
    } else {
#pragma unroll 1
        for (uint32_t k = tid; k < total; k += kTailThreads)
            place_escape(I, L, fits, tb, ((uint32_t)rpos[al + k] << 8) | rex[ae + k], rank0 + k);
    }
    __syncthreads();   // before the next tile reuses rpos and rex
}

// Escape placement: every workgroup takes tail_tiles tiles of one tensor,
// finds the rank of its first escape and the tensor's escape count (from the
// tile counts, or for large tensors from the superblock and block sums),
// then writes each tile's escapes at their final ranks as chunk id,
// chunk-local position and raw exponent: copied from the staging area, or
// for a tile above the staging cap derived from the input again.  The
// tensor's first tail workgroup writes the padding and the metadata.
// (at most 128 VGPRs: four waves per SIMD, so a single tensor's 1,024
// workgroups are all resident at once)
__global__ __launch_bounds__(kTailThreads, 4) void k_encode_tail(EncArgs a) {
    __shared__ uint64_t red[2][kTailThreads / 64];
    __shared__ uint32_t waves[kTailThreads / 64];
    __shared__ uint32_t scan[kTailMaxTiles + 1];
    __shared__ uint8_t lut[256];
    __shared__ uint32_t wtot[kEncUnits][4];
    // a re-derived tile's escapes by rank: position in tile, raw exponent
    __shared__ __attribute__((aligned(16))) uint16_t rpos[kEncTile + 8];
    __shared__ __attribute__((aligned(16))) uint8_t rex[kEncTile + 16];
    const uint32_t item = find_item(a.blk_start, a.count, blockIdx.x);
    const EncItem I = a.it[item];
    const uint32_t blk = blockIdx.x - a.blk_start[item];
    const uint64_t tfirst = a.tile_start[item], tend = a.tile_start[item + 1];
    const uint64_t ntiles = tend - tfirst;
    const uint32_t *counts = a.tile_count + tfirst;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t tt = a.tail_tiles;
    const uint64_t t0 = (uint64_t)blk * tt;
    const uint64_t t1 = t0 + tt < ntiles ? t0 + tt : ntiles;

    // this block's own tile counts (issued first, used after the sweep), and
    // with them the first S = kTailThreads / tt staged escapes of each of its
    // tiles, one per thread: a sparse tensor's tiles stage at most that many,
    // so the escapes are at hand when the ranks are known (no second round
    // trip); entries past a tile's count are read but not used
    const uint64_t mine_t = t0 + tid;
    const uint32_t mine_c = ((uint32_t)tid < tt && mine_t < t1) ? counts[mine_t] : 0u;
    const uint32_t spt = kTailThreads / tt;   // tt: a power of two up to kTailMaxTiles
    const uint32_t sj = (uint32_t)tid / spt, si = (uint32_t)tid % spt;
    const uint32_t spec = t0 + sj < t1 ? a.stage[(tfirst + t0 + sj) * kStageCap + si] : 0u;
    // the codebook's coverage for the metadata, loaded now (by the whole
    // workgroup that writes the metadata: a uniform load, kept in scalar
    // registers)
    uint64_t cb_cov = 0, cb_tot = 0;
    if (blk == 0) {
        cb_cov = I.cb->covered;
        cb_tot = I.cb->total;
    }
    uint64_t before = 0, all = 0;
    if (a.sup_sum) {
        // superblocks before this one and in total, then the blocks of this
        // superblock before this block
        const uint64_t sup = t0 / kSuperTiles;
        sum_prefix(a.sup_sum + a.sup_start[item], a.sup_start[item + 1] - a.sup_start[item], sup,
                   before, all);
        const uint64_t b0 = sup * (kSuperTiles / tt);
        if (b0 + tid < blk) before += a.blk_sum[a.blk_start[item] + b0 + tid];
    } else {
        sum_prefix(counts, ntiles, t0, before, all);
    }
    before = wave_sum_u64(before);
    all = wave_sum_u64(all);
    if (lane == 0) {
        red[0][wave] = before;
        red[1][wave] = all;
    }
    // exclusive scan of this block's tile counts
    const uint32_t incl = block_scan_incl(mine_c, waves);
    if ((uint32_t)tid < tt) scan[tid + 1] = incl;
    if (tid == 0) scan[0] = 0;
    // a tile above the staging cap has to be derived from the input again
    const bool beyond = __syncthreads_or(mine_c > spt) != 0;   // some tile stages more than S
    const bool rederive = beyond && __syncthreads_or(mine_c > kStageCap) != 0;
    uint64_t P = 0, e = 0;
#pragma unroll
    for (int w = 0; w < kTailThreads / 64; ++w) {
        P += red[0][w];
        e += red[1][w];
    }
    const Layout L = layout_of(I.n, e);
    const bool fits = L.total <= I.capacity;

    const uint32_t nt = (uint32_t)(t1 - t0);
    const uint32_t total = scan[nt];
    if (!beyond) {
        // every tile's escapes came with the counts
        if (sj < nt && si < scan[sj + 1] - scan[sj])
            place_escape(I, L, fits, (t0 + sj) * kEncTile, spec, P + scan[sj] + si);
    } else if (!rederive && total <= 8 * kTailThreads) {
        // few escapes: one pass over all of them, the tile of escape k found
        // in the block's scan, 8 staged loads in flight
        uint32_t w8[8], j8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t k = q * kTailThreads + tid;
            uint32_t lo = 0;
            w8[q] = 0;
            if (k < total) {
                uint32_t hi = nt;   // last j with scan[j] <= k
                while (hi - lo > 1) {
                    const uint32_t mid = (lo + hi) >> 1;
                    if (scan[mid] <= k) lo = mid; else hi = mid;
                }
                w8[q] = a.stage[(tfirst + t0 + lo) * kStageCap + (k - scan[lo])];
            }
            j8[q] = lo;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t k = q * kTailThreads + tid;
            if (k >= total) break;
            place_escape(I, L, fits, (t0 + j8[q]) * kEncTile, w8[q], P + k);
        }
    } else {
        // first tile above the cap (nt when none); the values of the next
        // one are loaded while a tile is worked on
        uint32_t jd = 0;
        while (jd < nt && scan[jd + 1] - scan[jd] <= kStageCap) ++jd;
        u32x4 qt[kEncUnits];
        if (rederive) {
            load_tile(I, (t0 + jd) * kEncTile, qt);
            load_marked_table(I.cb, lut);
            __syncthreads();
        }
        // tile by tile: staged escapes with every kTailThreads-th one per
        // thread, 8 staged loads in flight; tiles above the cap re-derived
        for (uint32_t j = 0; j < nt; ++j) {
            const uint32_t k_first = scan[j], c = scan[j + 1] - k_first;
            const uint64_t tb = (t0 + j) * kEncTile;
            if (c > kStageCap) {
                uint32_t jn = j + 1;
                while (jn < nt && scan[jn + 1] - scan[jn] <= kStageCap) ++jn;
                u32x4 qn[kEncUnits];
                if (jn < nt) load_tile(I, (t0 + jn) * kEncTile, qn);
                rederive_tile(I, L, fits, lut, wtot, rpos, rex, tb, P + k_first, qt);
#pragma unroll
                for (int u = 0; u < kEncUnits; ++u) qt[u] = qn[u];
                continue;
            }
            const uint32_t *st = a.stage + (tfirst + t0 + j) * kStageCap;
            for (uint32_t k0 = 0; k0 < c; k0 += 8 * kTailThreads) {
                uint32_t w8[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const uint32_t k = k0 + q * kTailThreads + tid;
                    w8[q] = k < c ? st[k] : 0u;
                }
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const uint32_t k = k0 + q * kTailThreads + tid;
                    if (k >= c) break;
                    place_escape(I, L, fits, tb, w8[q], P + k_first + k);
                }
            }
        }
    }
    if (blk == 0 && tid == 0) {
        if (fits)
            for (uint64_t b = L.off_lpos + 2 * e; b < L.off_ev; ++b) I.payload[b] = 0;
        splitzip_meta *m = I.meta;
        m->n = I.n;
        m->n_pairs = L.n_pairs;
        m->chunk_size = I.chunk;
        m->n_esc = e;
        m->comp_bytes = L.total;
        m->offsets[0] = 0;
        m->offsets[1] = L.off_sm;
        m->offsets[2] = L.off_cid;
        m->offsets[3] = L.off_lpos;
        m->offsets[4] = L.off_ev;
        m->covered = cb_cov;
        m->total = cb_tot;
        m->status = fits ? SPLITZIP_OK : SPLITZIP_ERR_CAPACITY;
        m->flags = SPLITZIP_META_ASCENDING;   // ranks follow element order
    }
}

// ---------------------------------------------------------------------------
// Decode (page 1, decode_torch)
// ---------------------------------------------------------------------------

struct DecItem {
    const uint8_t *payload;
    uint64_t payload_bytes;
    const splitzip_meta *meta;
    const uint8_t *dec_lut;
    uint16_t *out;
    uint64_t n;
    // In-place (slot) decode: the payload sits at the head of the output
    // buffer.  Pass 1 copies into `stash` (same offsets as in the payload)
    // what later passes read after the slot head has been overwritten, and
    // decodes the tiles whose output lies past the payload; the later passes
    // decode the rest (see the schedule above k_decode_slot_stage).
    uint8_t *stash;         // pass 1 only
    uint64_t other_bytes;   // size of the buffer the pass does not read from
};

// One tensor's share of a pass of the multi-pass in-place decode (tile
// indices; see the schedule above k_decode_slot_stage).  Pass 1: the tiles
// [a0, a1) also copy their sm bytes to the stash.  Later passes: the
// launch's workgroups for this tensor decode the tiles [a0, a1) then
// [b0, b1).  In the tensor's last pass (last != 0) they read their sm bytes
// from the stash, and `extra` workgroups come before them, one for each tile
// from t_min on whose output may overlap the payload (the host bounds the
// payload by the slot and the stash); every workgroup of the last pass then
// applies an escape stream not marked ascending.
struct SlotPass {
    uint32_t t_min;   // first tile whose output starts at or past the dense sections' end
    uint32_t a0, a1, b0, b1;
    uint32_t last, extra;
};

struct DecArgs {
    uint32_t count;
    uint64_t tile_start[kMaxBatch + 1];   // first decode tile (slot passes: workgroup) of each tensor
    DecItem it[kMaxBatch];
    SlotPass pass[kMaxBatch];             // multi-pass in-place decode only
    int32_t *status;
    uint64_t *order_sync;                 // this device's arrival counters (below)
    uint64_t order_ticket;                // this call's first counter, and its tag
    uint64_t *hold_block;                 // resident in-place decode: the call's barrier block,
    uint32_t hold_tag;                    // its tag,
    uint32_t wait_ticks;                  // and the barrier's bounded wait (10 ns ticks)
};
static_assert(sizeof(DecArgs) <= 4096, "kernel arguments");

// Arrival counters of the order-independent escape pass (streams not marked
// ascending): tensor k of a call uses counter (ticket + k) mod kOrderSlots,
// tagged (ticket + k + 1) in its high half (see tagged_arrive), so a
// counter needs no clearing and a stale or foreign value is simply replaced.  Library
// state on every device that runs a decode, kept until the process ends;
// calls that run at the same time use different counters unless 65,536
// tensors' decodes are issued while one of them waits to run.
constexpr uint32_t kOrderSlots = 65536;
__device__ __align__(256) uint64_t g_order_sync[kOrderSlots];

// Metadata must describe exactly the layout of (n, n_esc) and fit the buffer.
__device__ inline bool meta_ok(const DecItem &I, const splitzip_meta &m, Layout &L) {
    if (m.n != I.n || !chunk_ok(I.n, m.chunk_size) || m.n_esc > I.n) return false;
    L = layout_of(I.n, m.n_esc);
    return m.n_pairs == L.n_pairs && m.offsets[0] == 0 && m.offsets[1] == L.off_sm &&
           m.offsets[2] == L.off_cid && m.offsets[3] == L.off_lpos && m.offsets[4] == L.off_ev &&
           m.comp_bytes == L.total && L.total <= I.payload_bytes;
}
__device__ inline bool meta_ok(const DecItem &I, Layout &L) { return meta_ok(I, *I.meta, L); }

enum DecMode { kPlain = 0, kSlotStage = 1, kSlotLevel = 2 };

// Slot decode: first tile whose output lies wholly beyond the payload.
__device__ inline uint64_t slot_split(uint64_t comp_bytes, uint64_t tiles, uint64_t tile) {
    const uint64_t t = (comp_bytes + 2 * tile - 1) / (2 * tile);
    return t < tiles ? t : tiles;
}

// First r in [lo, hi) with cid[r] >= key (hi when none), for chunk ids sorted
// on [lo, hi); one wave.  A 64-entry window at the interpolated guess settles
// most searches with one load; otherwise a 64-ary search narrows the range.
__device__ inline uint64_t lower_bound_wave(const int32_t *cid, uint64_t lo, uint64_t hi,
                                            int64_t key, uint64_t guess, int lane) {
    if (hi > lo + 64) {
        uint64_t wlo = guess > 32 ? guess - 32 : 0;
        if (wlo < lo) wlo = lo;
        if (wlo > hi - 64) wlo = hi - 64;
        const int64_t v = cid[wlo + lane];
        const uint64_t below = __ballot(v < key);
        const uint32_t k = __popcll(below);
        const bool left_ok = (wlo == lo) || (below & 1ull);
        if (left_ok && k < 64) return wlo + k;
        if (!left_ok) hi = wlo;              // answer in [lo, wlo]
        else lo = wlo + 64;                  // whole window below the key
    }
    // Then 64 samples 64 apart around the guess (dense streams, where the
    // guess is off by more than the window): brackets the answer within 64.
    if (hi > lo + 64 * 64) {
        uint64_t blo = guess > 32 * 64 ? guess - 32 * 64 : 0;
        if (blo < lo) blo = lo;
        if (blo > hi - 64 * 64) blo = hi - 64 * 64;
        const uint64_t sx = blo + (uint64_t)lane * 64;
        const int64_t v = cid[sx];
        const uint32_t k = __popcll(__ballot(v < key));
        const uint64_t s_lo = __shfl(sx, k > 0 ? (int)k - 1 : 0, 64);
        const uint64_t s_hi = __shfl(sx, k < 64 ? (int)k : 63, 64);
        if (k == 0) hi = blo;                // answer in [lo, blo]
        else if (k == 64) lo = s_lo + 1;     // every sample below the key
        else {
            lo = s_lo + 1;                   // answer in (s_lo, s_hi]
            hi = s_hi;
        }
    }
    while (hi > lo + 63) {
        const uint64_t span = hi - lo;
        const uint64_t s = lo + (span * (uint64_t)(lane + 1)) / 65;
        const int64_t v = cid[s];
        const uint32_t k = __popcll(__ballot(v < key));
        const uint64_t s_lo = __shfl(s, k > 0 ? (int)k - 1 : 0, 64);
        const uint64_t s_hi = __shfl(s, k < 64 ? (int)k : 63, 64);
        const uint64_t nlo = k > 0 ? s_lo + 1 : lo;
        const uint64_t nhi = k < 64 ? s_hi : hi;
        lo = nlo;
        hi = nhi;
    }
    const uint64_t p = lo + lane;
    const int64_t v = p < hi ? (int64_t)cid[p] : INT64_MAX;
    return lo + __popcll(__ballot(v < key));
}

// Order-independent escape pass (page 1, decode_torch applies the escapes
// by index, in any order) for a tensor whose stream is not marked ascending:
// every workgroup of the tensor releases its dense stores and arrives; the
// last to arrive applies all escapes.  The sign and mantissa come from the
// payload, or after an in-place decode from the decoded value.
template <bool kFromOut>
__device__ void order_pass(const DecArgs &a, const DecItem &I, uint32_t item, const Layout &L,
                           uint32_t *last) {
    __threadfence();   // this wave's dense stores before the arrival
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint64_t t = a.order_ticket + item;
        const uint64_t ntiles = a.tile_start[item + 1] - a.tile_start[item];
        uint64_t *c = a.order_sync + (t & (kOrderSlots - 1));
        counter_claim(c, ld_agent(c), (uint32_t)t + 1u);   // a rare path: not hidden
        *last = tagged_arrive(c, ntiles, (uint32_t)t + 1u);
    }
    __syncthreads();
    if (!*last) return;
    __threadfence();   // every other workgroup's dense stores before the patches
    const uint64_t e = I.meta->n_esc;
    const uint64_t chunk = I.meta->chunk_size;
    const uint8_t *sm = I.payload + L.off_sm;
    const int32_t *cid = reinterpret_cast<const int32_t *>(I.payload + L.off_cid);
    const uint16_t *lpos = reinterpret_cast<const uint16_t *>(I.payload + L.off_lpos);
    const uint8_t *ev = I.payload + L.off_ev;
    for (uint64_t r = threadIdx.x; r < e; r += blockDim.x) {
        const int32_t c = cid[r];
        if (c < 0) continue;
        const uint64_t idx = (uint64_t)c * chunk + lpos[r];
        if (idx >= I.n) continue;
        const uint32_t keep = kFromOut ? sm_of16(I.out[idx]) : sm[idx];
        I.out[idx] = (uint16_t)join16(keep, ev[r]);
    }
}

// Workgroup barrier that orders LDS only: the waves' global loads and stores
// stay in flight across it (a full __syncthreads waits for all of them).
__device__ inline void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Dense decode and escape patch of one tile.  A full tile's pk and sm words
// are in registers; pk and sm point at the sections that a partial tile and
// the patch read, the escape sections are at I.payload, and the pair table
// is in LDS.
template <int kTh, int kUnits>
__device__ __forceinline__ void decode_body(const DecItem &I, const splitzip_meta &M, const Layout &L,
                                            uint64_t base, bool full, const uint8_t *pk,
                                            const uint8_t *sm, const uint32_t (&pkw)[kUnits],
                                            const u32x2 (&smw)[kUnits], const uint32_t *pair_lut,
                                            uint64_t *range, uint32_t *tile_buf) {
    constexpr int kDecTile = kTh * kUnit * kUnits;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const uint64_t e = M.n_esc;
    const int32_t *cid = reinterpret_cast<const int32_t *>(I.payload + L.off_cid);
    const uint16_t *lpos = reinterpret_cast<const uint16_t *>(I.payload + L.off_lpos);
    const uint8_t *ev = I.payload + L.off_ev;

    // A tensor whose escapes average more than 512 per tile is decoded tile
    // by tile in LDS (dense values, the patch, then one coalesced store):
    // scattering thousands of 2-byte stores per tile to memory costs more
    // than writing the tile twice.
    const bool ascending = (M.flags & SPLITZIP_META_ASCENDING) != 0;
    const bool in_lds = ascending && full && e * (uint64_t)kDecTile > 512 * I.n;
    const uint32_t chunk = (uint32_t)M.chunk_size;

    // Dense part first: every element through the pair table, 16-byte stores.
    if (full) {
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const int l0 = u * (kTh * kUnit) + tid * kUnit;
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t ee = pair_lut[(pkw[u] >> (8 * k)) & 0xFFu];
                const uint32_t s = smw[u][k >> 1] >> (16 * (k & 1));
                o[k] = join16(s & 0xFFu, ee & 0xFFu) | (join16((s >> 8) & 0xFFu, ee >> 16) << 16);
            }
            if (in_lds)
                *reinterpret_cast<u32x4 *>(tile_buf + l0 / 2) = o;
            else   // non-temporal: 5 % faster than plain stores for this stream
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(I.out + base + l0));
        }
    } else {
        for (uint64_t i = base + tid; i < I.n; i += kTh) {
            const uint32_t byte = pk[i / 2];
            const uint32_t code = (i & 1) ? (byte & 15u) : (byte >> 4);
            I.out[i] = (uint16_t)join16(sm[i], pair_lut[code << 4] & 0xFFu);
        }
    }
    // An escape stream not known to be ascending cannot be searched per
    // tile: it is applied by index after the dense part of every tile.
    if (e == 0 || !ascending) return;

    // Escape patch: the tile's escapes are among those with chunk ids in
    // [c0, c1) of the sorted stream (exactly those when tiles and chunks
    // align), found by one wave while the dense stores drain; they are
    // applied after the workgroup barrier, which orders them after the dense
    // stores of every wave of the workgroup.
    if (tid < 64) {
        // chunks that hold the tile's elements: [c0, c1)
        uint64_t c0, c1, nchunks;
        uint32_t p0, p1, pn;
        chunk_split(base, chunk, c0, p0);
        chunk_split(base + kDecTile - 1, chunk, c1, p1);
        chunk_split(I.n - 1, chunk, nchunks, pn);
        ++c1;
        ++nchunks;
        if (c1 > nchunks) c1 = nchunks;
        // interpolated guesses (hints only: the search is exact for any guess)
        const double per_chunk = (double)e / (double)nchunks;
        const uint64_t r0 =
            lower_bound_wave(cid, 0, e, (int64_t)c0, (uint64_t)(per_chunk * (double)c0), lane);
        const uint64_t r1 = lower_bound_wave(cid, r0, e, (int64_t)c1,
                                             r0 + (uint64_t)(per_chunk * (double)(c1 - c0)), lane);
        if (lane == 0) {
            range[0] = r0;
            range[1] = r1;
        }
    }
    __syncthreads();
    const uint64_t r0 = range[0], r1 = range[1];
    if (in_lds) {
        // the decoded value already holds the sign and mantissa
        uint16_t *t16 = reinterpret_cast<uint16_t *>(tile_buf);
        for (uint64_t rb = r0; rb < r1; rb += 8 * kTh) {
            int32_t l8[8];
            uint32_t e8[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint64_t r = rb + q * kTh + tid;
                l8[q] = -1;
                e8[q] = 0;
                if (r < r1) {
                    const int64_t v = (int64_t)cid[r] * chunk + lpos[r] - (int64_t)base;
                    e8[q] = ev[r];
                    if (v >= 0 && v < kDecTile) l8[q] = (int32_t)v;
                }
            }
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (l8[q] >= 0)
                    t16[l8[q]] = (uint16_t)((t16[l8[q]] & 0x807Fu) | (e8[q] << 7));
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const int l0 = u * (kTh * kUnit) + tid * kUnit;
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(tile_buf + l0 / 2),
                                        reinterpret_cast<u32x4 *>(I.out + base + l0));
        }
        return;
    }
    // A tile with many escapes in a sparse tensor keeps its sm bytes (still
    // in registers) in LDS for the patch, instead of reading each one back
    // from memory.
    const bool staged = full && r1 - r0 > kDecStaged;
    if (staged) {
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const int o = u * (kTh * kUnit) + tid * kUnit;
            tile_buf[o / 4] = smw[u].x;
            tile_buf[o / 4 + 1] = smw[u].y;
        }
        __syncthreads();
    }
    const uint8_t *sm_lds = reinterpret_cast<const uint8_t *>(tile_buf);
#ifndef SPLITZIP_DEC_PATCH
#define SPLITZIP_DEC_PATCH 4
#endif
    constexpr int kPatch = SPLITZIP_DEC_PATCH;
    // kPatch escapes per thread in flight: their stream entries, then their
    // sm bytes, then the stores
    for (uint64_t rb = r0; rb < r1; rb += kPatch * kTh) {
        int64_t idx[kPatch];
        uint32_t evv[kPatch], smv[kPatch];
#pragma unroll
        for (int q = 0; q < kPatch; ++q) {
            const uint64_t r = rb + q * kTh + tid;
            idx[q] = -1;
            evv[q] = 0;
            if (r < r1) {
                const int64_t v = (int64_t)cid[r] * chunk + lpos[r];
                evv[q] = ev[r];
                if (v >= (int64_t)base && v < (int64_t)(base + kDecTile) && v < (int64_t)I.n)
                    idx[q] = v;
            }
        }
#pragma unroll
        for (int q = 0; q < kPatch; ++q)
            smv[q] = idx[q] < 0 ? 0u : (staged ? sm_lds[idx[q] - (int64_t)base] : sm[idx[q]]);
#pragma unroll
        for (int q = 0; q < kPatch; ++q)
            if (idx[q] >= 0) I.out[idx[q]] = (uint16_t)join16(smv[q], evv[q]);
    }
}

template <int kTh, int kUnits, int kMode>
__device__ __forceinline__ void decode_tile(const DecArgs &a) {
    constexpr int kDecTile = kTh * kUnit * kUnits;
    static_assert(kTh >= 256, "one pair-table entry per thread");
    __shared__ uint32_t pair_lut[256];      // pk byte -> (even exponent, odd exponent << 16)
    __shared__ uint64_t range[2];
    __shared__ uint32_t last_arrival;
    // Output tile of a tensor with dense escapes, or the sm bytes of a tile
    // with many escapes in an otherwise sparse tensor.
    __shared__ uint32_t tile_buf[kDecTile / 2];
    const uint64_t gt = launch_tile(blockIdx.x, gridDim.x);
    const uint32_t item = find_item(a.tile_start, a.count, gt);
    const DecItem I = a.it[item];
    const int tid = threadIdx.x;
    const Layout L0 = layout_of(I.n, 0);
    uint64_t tile = gt - a.tile_start[item];
    // Slot passes: the tile this workgroup decodes, and where its sm bytes
    // are (the slot in passes before the tensor's last one, else the stash).
    const uint8_t *sm_src = I.payload;
    bool sm_copy = false;   // pass 1: this tile's sm bytes go to the stash
    bool has_tile = true;   // last pass: false for the workgroups placed before the others
    if (kMode == kSlotLevel) {
        const SlotPass Q = a.pass[item];
        uint64_t j = tile;
        if (Q.last) {
            has_tile = j >= Q.extra;
            j = has_tile ? j - Q.extra : 0;
        }
        const uint64_t la = Q.a1 - Q.a0;
        tile = j < la ? Q.a0 + j : Q.b0 + (j - la);
        if (!Q.last) sm_src = reinterpret_cast<const uint8_t *>(I.out);
    } else if (kMode == kSlotStage) {
        const SlotPass Q = a.pass[item];
        sm_copy = tile >= Q.t_min || (tile >= Q.a0 && tile < Q.a1);
    }
    const uint64_t base = tile * kDecTile;
    const bool full = has_tile && base + kDecTile <= I.n;
    // The dense sections depend on n alone (the host checked that the buffers
    // hold them), so their loads go out before the metadata arrives; in pass
    // 1 the sm bytes only of the tiles that need them.
    const uint8_t *pk = I.payload;
    const uint8_t *sm = sm_src + L0.off_sm;
    uint32_t pkw[kUnits];
    u32x2 smw[kUnits];
    if (full) {
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const uint64_t i0 = base + (uint64_t)u * (kTh * kUnit) + tid * kUnit;
            pkw[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(pk + i0 / 2));
            if (kMode != kSlotStage || sm_copy)
                smw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2_a4 *>(sm + i0));
        }
    }
    // Then the metadata, as one copy: the compiler reads it with scalar
    // loads, whose wait leaves the stream loads in flight (reading fields
    // through the pointer took vector loads, and vector loads complete in
    // order, so their wait was a wait for the whole tile), and the table's two
    // bytes, loaded by every lane (no branch around the loads) and combined
    // where the table is written.
    const splitzip_meta M = *I.meta;
    const uint32_t lut_lo = I.dec_lut[(tid >> 4) & 15];
    const uint32_t lut_hi = I.dec_lut[tid & 15];
    Layout L;
    if (!meta_ok(I, M, L) || (kMode != kPlain && L.total > I.other_bytes)) {
        // nothing is written for inconsistent metadata
        if (kMode != kSlotLevel && gt == a.tile_start[item] && tid == 0 && a.status)
            atomicOr(a.status, 1);
        return;
    }
    const uint64_t tiles = (I.n + kDecTile - 1) / kDecTile;
    const uint64_t t_split = kMode == kPlain ? tiles : slot_split(L.total, tiles, kDecTile);
    if (kMode == kSlotStage) {
        // Every workgroup of the tensor copies its share of the escape
        // sections.
        const uint64_t esc_bytes = L.total - L.off_cid;
        const uint32_t *src = reinterpret_cast<const uint32_t *>(I.payload + L.off_cid);
        uint32_t *dst = reinterpret_cast<uint32_t *>(I.stash + L.off_cid);
        const uint64_t stride = tiles * kTh;
        for (uint64_t w = tile * kTh + tid; w < esc_bytes / 4; w += stride) dst[w] = src[w];
        if (tile == 0 && tid < (int)(esc_bytes & 3)) {
            const uint64_t b = L.off_cid + (esc_bytes & ~uint64_t(3)) + tid;
            I.stash[b] = I.payload[b];
        }
        if (tile < t_split) {   // output overlaps the payload: copy the inputs a later pass reads
            if (full) {
#pragma unroll
                for (int u = 0; u < kUnits; ++u) {
                    const uint64_t i0 = base + (uint64_t)u * (kTh * kUnit) + tid * kUnit;
                    *reinterpret_cast<uint32_t *>(I.stash + i0 / 2) = pkw[u];
                    if (sm_copy) *reinterpret_cast<u32x2_a4 *>(I.stash + L0.off_sm + i0) = smw[u];
                }
            } else {
                for (uint64_t b = base / 2 + tid; b < L0.n_pairs; b += kTh) I.stash[b] = pk[b];
                if (sm_copy)
                    for (uint64_t i = base + tid; i < I.n; i += kTh) I.stash[L0.off_sm + i] = sm[i];
            }
            return;
        }
    }
    if (tid < 256) pair_lut[tid] = lut_lo | (lut_hi << 16);
    lds_barrier();   // the pair table; the stream loads may still be in flight
    const bool ordered = M.n_esc && !(M.flags & SPLITZIP_META_ASCENDING);
    if (kMode != kSlotLevel) {
        decode_body<kTh, kUnits>(I, M, L, base, full, pk, sm, pkw, smw, pair_lut, range, tile_buf);
        if (kMode == kPlain && ordered) order_pass<false>(a, I, item, L, &last_arrival);
        return;
    }
    // Slot pass: one tile per workgroup (a second tile's code in the same
    // kernel, as a loop or a second copy, doubled its registers and cost the
    // pass occupancy).  In the tensor's last pass workgroup m < extra takes
    // tile t_min + m, whose output overlaps the payload past the dense
    // sections (it covers the escape sections), every input from the stash;
    // nothing when that tile's output lies past the payload.
    const SlotPass Q = a.pass[item];
    if (has_tile)
        decode_body<kTh, kUnits>(I, M, L, base, full, pk, sm, pkw, smw, pair_lut, range, tile_buf);
    else if (Q.t_min + (gt - a.tile_start[item]) < t_split) {
        const uint64_t bt = (Q.t_min + (gt - a.tile_start[item])) * kDecTile;
        const bool ft = bt + kDecTile <= I.n;
        const uint8_t *sms = I.payload + L0.off_sm;
        if (ft) {
#pragma unroll
            for (int u = 0; u < kUnits; ++u) {
                const uint64_t i0 = bt + (uint64_t)u * (kTh * kUnit) + tid * kUnit;
                pkw[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(pk + i0 / 2));
                smw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2_a4 *>(sms + i0));
            }
        }
        decode_body<kTh, kUnits>(I, M, L, bt, ft, pk, sms, pkw, smw, pair_lut, range, tile_buf);
    }
    if (Q.last && ordered) order_pass<true>(a, I, item, L, &last_arrival);
}

template <int kUnits>
__global__ __launch_bounds__(kDecThreads) void k_decode(DecArgs a) {
    decode_tile<kDecThreads, kUnits, kPlain>(a);
}

// ---------------------------------------------------------------------------
// In-place decode, multi-pass form (page 1, decode_slot_into; page "SplitZip
// in DDO -- VMM routes", the CUDA route's expansion in place)
// ---------------------------------------------------------------------------
//
// Tile t (T = 8192 elements, len_t of them) reads pk bytes [tT/2, ...), sm
// bytes [S + tT, S + tT + len_t) (S = the sm section's offset) and the
// escape sections, and writes slot bytes [2tT, 2tT + 2len_t).  Pass 1
// (k_decode_slot_stage) decodes the tiles whose output starts at or past
// comp_bytes (t >= t_split) and copies to the stash the escape sections, the
// pk bytes of every other tile, and the sm bytes of the tiles named below.
// From pass 2 on (k_decode_slot_level) every tile reads its pk bytes and
// the escapes from the stash, so the one hazard left is a tile w whose
// output covers the sm bytes of another tile t that reads them from the
// slot: t must run in an earlier pass than w.  For the tiles below t_min
// (output starting before the dense sections' end), with readers(w) the
// tiles below t_min whose sm bytes meet w's output:
//   depth(w) = 0 without readers, 1 + max depth(readers) otherwise, and
//              unbounded when w is among its own readers;
//   pass(w)  = min(K, 2 + depth(w)).
// Tiles at pass K, and the tiles from t_min to t_split (their outputs cover
// the escape sections), read their sm bytes from the stash as well; pass K
// decodes both.  A tile's readers lie all below it or all above it (a range
// around 2w - S/T), depth grows toward the tile(s) that overlap their own
// sm bytes, so each pass's tiles form one range on each side of those and
// the host finds the ranges by bisection.  With K passes the stash carries
// the pk bytes (a quarter of the tensor's raw bytes) plus the sm bytes of
// the pass-K tiles (about 3/2^(K+1) of the tiles) instead of every
// overlapping tile's inputs, so the slot decode moves about 1.32x its
// algorithmic bytes at K = 4 against 1.65x at K = 2 (every overlapping tile
// stashed, pass 2 decoding them all).
__global__ __launch_bounds__(kDecThreads) void k_decode_slot_stage(DecArgs a) {
    decode_tile<kDecThreads, kDecUnits, kSlotStage>(a);
}

__global__ __launch_bounds__(kDecThreads) void k_decode_slot_level(DecArgs a) {
    decode_tile<kDecThreads, kDecUnits, kSlotLevel>(a);
}

// ---------------------------------------------------------------------------
// In-place decode, resident form (page 1, decode_slot_into; page "SplitZip in
// DDO -- VMM routes", the CUDA route's expansion in place)
// ---------------------------------------------------------------------------
//
// Tile t writes slot bytes [2tT, 2(t+1)T) (T = 8192 elements); the tiles from
// t_split = ceil(comp / 2T) on write only past the payload.  One ordinary
// launch with as many workgroups as the GPU keeps resident at once: every
// workgroup first decodes its tiles from t_split on, then loads the pk/sm
// inputs of its tiles wg + jG below t_split (j < kHold) into registers,
// their escape entries having gone to LDS; after a grid barrier it writes
// the held tiles straight from the registers, then their escapes.  After the
// barrier a workgroup reads no slot byte and only the stash bytes it wrote
// itself, so the barrier needs no cache flush: it only has to order the held
// tiles' stores after every load of the first phase.  Overlapping tiles
// beyond the registers' reach (more than kHold * G of them), and a partial
// last one, go through the stash as in the multi-pass form.  A group of
// slots takes one barrier per slot, the stores of one slot overlapping the
// loads of the next.
//
// An ordinary launch does not promise that the whole grid is resident (other
// work may hold part of the GPU), so the barrier's wait is bounded: a
// workgroup that has waited kStartWaitTicks while part of the grid has not
// started, or wait_ticks (10 ns each) in any case, marks the round aborted
// unless its last arrival has already come, and that arrival's atomic on the
// top counter decides: go unless a mark came first.  An abort is sticky for
// the rest of the launch (the grid stayed partly absent).  (The same kernels
// may also be launched cooperatively; then the runtime places the grid
// whole and no barrier gives up.)  On an abort every
// workgroup stashes its held tiles' inputs (and its share of the escape
// sections) and leaves the slot to k_decode_slot_defer, launched after this
// kernel, which decodes the stashed tiles as the multi-pass form's last
// pass does.  A stream not marked ascending is always left to it (its
// escapes are applied by index once every tile is decoded).  Neither outcome
// depends on which workgroups were resident.
constexpr int kHold = 3;                   // held tiles per workgroup and tensor
constexpr uint32_t kHoldEsc = 512;         // escape entries per held tile in LDS
constexpr int kCoopTile = kDecThreads * kUnit * kDecUnits;   // 8192 elements
constexpr int kCoopUnits = kCoopTile / kUnit;                // 8-element units per tile
static_assert(kHold <= kDecThreads / 64, "one wave finds each held tile's escapes");

struct CoopLds {
    uint32_t pair_lut[256];
    uint32_t tile[kCoopTile / 2];          // one decoded tile
    uint32_t esc[kHold][kHoldEsc];         // (position << 16) | (sign, mantissa << 8) | exponent, or ~0
    uint64_t hr0[kHold], hr1[kHold];       // escape ranks of the held tiles
    uint64_t dr0, dr1;                     // escape ranks of a direct tile
};

// Grid barrier of the resident in-place decode.  Same-address atomics
// serialise at the memory side, so the grid arrives in two levels:
// workgroups on the counter of their group of kCoopGroup, the last of each
// group on the top counter, whose arrival tells it whether the round is
// complete.  Whoever knows a round's outcome writes it to every group's
// flag, and each group polls only its own flag.  The group and top counters
// are tagged ((tag << 32) | value, see tagged_claim) and claimed by the
// launch that increments them.  Besides them each group has a start word
// and a leave word, and the launch a leave word and a pending word; the last
// workgroup to leave puts all of them back to (tag << 32), so that the next
// launch on the block, or a replay of the same arguments, starts from zero.
constexpr uint32_t kCoopGroup = 16;                        // workgroups per group counter
constexpr uint32_t kCoopMaxGrid = 2048;
constexpr uint32_t kCoopGroups = kCoopMaxGrid / kCoopGroup;
constexpr uint32_t kCoopLine = 16;                         // words per counter (128 bytes)
constexpr uint32_t kCoopWords = (2 * kCoopGroups + 2) * kCoopLine;
constexpr uint32_t kCoopBlocks = 64;                       // streams with blocks of their own
constexpr uint64_t kGo = 1, kAbort = 2;
constexpr uint64_t kHoldWaitUs = 200;   // barrier wait before a workgroup gives up
constexpr uint32_t kStartWaitTicks = 2000;   // 20 us: the wait while part of the grid has not started
__device__ __align__(256) uint64_t g_coop_sync[kCoopBlocks * kCoopWords];

struct CoopBar {
    uint64_t *blk;        // the launch's block of counters and flags
    uint32_t tag, passed;
};

__device__ inline uint32_t coop_ngroups() { return (gridDim.x + kCoopGroup - 1) / kCoopGroup; }
__device__ inline uint32_t coop_gsize(uint32_t g) { return min(kCoopGroup, gridDim.x - g * kCoopGroup); }

__device__ inline uint64_t *coop_grp(const CoopBar &b, uint32_t g) { return b.blk + g * kCoopLine; }
__device__ inline uint64_t *coop_flag(const CoopBar &b, uint32_t g) {
    return b.blk + (kCoopGroups + g) * kCoopLine;
}
// the number of the group's workgroups that have started, and that have left
__device__ inline uint64_t *coop_started(const CoopBar &b, uint32_t g) { return coop_flag(b, g) + 1; }
__device__ inline uint64_t *coop_left(const CoopBar &b, uint32_t g) { return coop_flag(b, g) + 2; }
__device__ inline uint64_t *coop_top(const CoopBar &b) { return b.blk + 2 * kCoopGroups * kCoopLine; }
__device__ inline uint64_t *coop_top_left(const CoopBar &b) { return coop_top(b) + 1; }
// (tag << 32) | (first aborted round << 8) | 1 when some slot of the launch
// was left to the second kernel
__device__ inline uint64_t *coop_pending(const CoopBar &b) {
    return b.blk + (2 * kCoopGroups + 1) * kCoopLine;
}
__device__ inline void coop_set_pending(const CoopBar &b) {
    __hip_atomic_store(coop_pending(b), ((uint64_t)b.tag << 32) | 1u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Claims this workgroup's group counter (and, for the first workgroup of a
// group, the top counter: every arrival on it follows the arrival of some
// group's first workgroup, which claimed it before arriving), and counts
// the workgroup on its group's start word (an atomic whose result it does
// not wait for; start and leave words are not tagged, see coop_leave).
__device__ inline void coop_bar_init(CoopBar &b, uint64_t *blk, uint32_t tag) {
    b.blk = blk;
    b.tag = tag;
    b.passed = 0;
    if (threadIdx.x == 0) {
        const uint32_t g = blockIdx.x / kCoopGroup;
        __hip_atomic_fetch_add(coop_started(b, g), 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint64_t *c = coop_grp(b, g);
        counter_claim(c, ld_agent(c), tag);
        if (g * kCoopGroup == blockIdx.x) counter_claim(coop_top(b), ld_agent(coop_top(b)), tag);
    }
}

// The top counter's low word: the arrivals of the launch's groups in its
// low 24 bits, and in the high 8 bits the first round that a workgroup gave
// up waiting on (0: none).  An abort is sticky: that round and every later
// one of the launch abort, so the first aborted round decides every verdict.
constexpr uint32_t kCountMask = (1u << 24) - 1;
__device__ inline uint32_t top_count(uint64_t v) { return (uint32_t)v & kCountMask; }
__device__ inline uint32_t top_abort_round(uint64_t v) { return (uint32_t)v >> 24 & 0xFFu; }
__device__ inline uint64_t round_verdict(uint32_t abort_round, uint32_t round) {
    return abort_round != 0 && abort_round <= round ? kAbort : kGo;
}
static_assert(kMaxBatch < 0xFF, "rounds fit the top counter's abort field");
static_assert(kMaxBatch * kCoopGroups <= kCountMask, "arrivals fit the top counter");

// Arrival of this workgroup for round `round` (thread 0); true for the last
// arrival of the round over the whole grid, which also learns the first
// aborted round so far.  Until a round aborts, no workgroup arrives for a
// round before every one has arrived for the previous one, so the counts
// identify each round's last arrival.  After an abort, workgroups that gave
// up go on while others have yet to arrive, the counters mix rounds, and a
// "last arrival" may be misplaced or missing -- but it then sees the abort
// (set before any workgroup went on), so every verdict stays an abort, and
// a workgroup that finds no flag gives up by itself.
__device__ inline bool coop_arrive(const CoopBar &b, uint32_t round, uint32_t &abort_round) {
    const uint32_t group = blockIdx.x / kCoopGroup;
    abort_round = 0;
    const uint64_t p = __hip_atomic_fetch_add(coop_grp(b, group), 1ull, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)p + 1u != coop_gsize(group) * round) return false;
    const uint64_t q = __hip_atomic_fetch_add(coop_top(b), 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    abort_round = top_abort_round(q);
    return top_count(q) + 1u == coop_ngroups() * round;
}

// Whether every workgroup of the grid has started (thread 0; read only by a
// workgroup that has waited a while).  A workgroup that has started runs to
// its end on its compute unit, so once every one has started every barrier
// of the launch completes; while some have not, other work holds the
// compute units they need.
__device__ inline bool coop_all_started(const CoopBar &b) {
    const uint32_t ng = coop_ngroups();
    bool ok = true;
    for (uint32_t g0 = 0; g0 < ng && ok; g0 += 8) {
        uint64_t v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = g0 + j < ng ? ld_agent(coop_started(b, g0 + j)) : 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (g0 + j < ng) ok = ok && (uint32_t)v[j] >= coop_gsize(g0 + j);
    }
    return ok;
}

// A workgroup that has waited too long on round `round` marks it aborted
// unless the round is already complete (its count reached) or an earlier
// round aborted.  0: the round completed first (its last arrival then
// decides it from the abort field it saw); 1: the round aborts, marked by
// another workgroup (which publishes it); 2: marked by this one.
__device__ inline int coop_poison(const CoopBar &b, uint32_t round) {
    uint64_t *top = coop_top(b);
    uint64_t cur = ld_agent(top);
    counter_claim(top, cur, b.tag);   // (its group's first workgroup may not have run)
    if ((uint32_t)(cur >> 32) != b.tag) cur = ld_agent(top);
    for (int k = 0; k < 4096; ++k) {
        if ((uint32_t)(cur >> 32) != b.tag) return 2;   // (not a state this launch produces)
        const uint32_t ar = top_abort_round(cur);
        if (ar != 0) return ar <= round ? 1 : 0;
        if (top_count(cur) >= coop_ngroups() * round) return 0;
        if (__hip_atomic_compare_exchange_strong(top, &cur, cur | (uint64_t)round << 24, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            return 2;
    }
    return 2;
}

// One round; true when the grid goes on (every workgroup arrived before any
// gave up, in this round or an earlier one).  A waiting workgroup gives up
// after kStartWaitTicks (staggered by 1 us over the workgroups of a group,
// so that one of them usually decides for all) if the grid has not all
// started by then, else after wait_ticks.  Whoever decides the verdict
// publishes (round << 2) | verdict to every group's flag: the round's last
// arrival, or the workgroup that marked the launch aborted.  A flag may be overwritten by an older round's late
// publication; a waiter reads its round's verdict from any flag of this
// round or later, or of an earlier aborted round (aborts are sticky), and
// otherwise keeps waiting.  `st` is a word of LDS.
__device__ inline bool coop_barrier(CoopBar &b, uint32_t wait_ticks, bool fence, uint32_t *st) {
    if (fence) __threadfence();   // (stash bytes other workgroups read after a go)
    wait_vector_memory();
    __syncthreads();
    ++b.passed;
    const uint32_t r = b.passed;
    if (threadIdx.x < 64) {
        uint64_t verdict = 0;
        int publish = 0;
        if (threadIdx.x == 0) {
            uint32_t ar;
            if (coop_arrive(b, r, ar)) {
                verdict = round_verdict(ar, r);
                publish = 1;
            } else {
                const uint64_t *f = coop_flag(b, blockIdx.x / kCoopGroup);
                const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
                const uint32_t start_ticks =
                    min(wait_ticks, kStartWaitTicks + blockIdx.x % kCoopGroup * 100u);
                bool waited = false, started = false;
                for (uint32_t k = 1;; ++k) {
                    const uint64_t v = ld_agent(f);
                    if ((uint32_t)(v >> 32) == b.tag) {
                        const uint32_t fr = (uint32_t)v >> 2;
                        if ((v & 3u) == kAbort && fr <= r) {   // this round or an earlier one aborted
                            verdict = kAbort;
                            break;
                        }
                        if ((v & 3u) == kAbort && fr > r) {    // a later round aborted: the first decides
                            verdict = round_verdict(top_abort_round(ld_agent(coop_top(b))), r);
                            break;
                        }
                        if ((v & 3u) == kGo && fr >= r) {
                            verdict = kGo;
                            break;
                        }
                    }
                    if (!waited && (k & 7) == 0) {
                        const uint64_t dt = __builtin_amdgcn_s_memrealtime() - t0;
                        bool give_up = dt > wait_ticks;
                        if (!give_up && !started && dt > start_ticks) {
                            started = coop_all_started(b);
                            give_up = !started;
                        }
                        if (give_up) {
                            waited = true;   // once: afterwards the round is decided either way
                            const int pz = coop_poison(b, r);
                            if (pz) {
                                verdict = kAbort;
                                publish = pz == 2;
                                break;
                            }
                        }
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            if (verdict != kGo) coop_set_pending(b);
            *st = (uint32_t)verdict;
        }
        if (__shfl(publish, 0, 64)) {
            const uint64_t w = ((uint64_t)b.tag << 32) | ((uint64_t)r << 2) | __shfl(verdict, 0, 64);
            for (uint32_t g = threadIdx.x; g < coop_ngroups(); g += 64)
                __hip_atomic_store(coop_flag(b, g), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    if (fence) __threadfence();
    return *st == kGo;
}

// Every workgroup leaves once, on leave words of its own (two levels, as the
// rounds), so the last to leave is known even when aborted rounds mixed the
// round counters.  It puts the block back to (tag << 32); with `record` (the
// first kernel) it records the first aborted round in the pending word for
// the second kernel and keeps a pending mark, else it clears the word.  Its
// reads follow every workgroup's stores, which precede their leaving.
__device__ inline void coop_leave(CoopBar &b, bool record) {
    wait_vector_memory();
    __syncthreads();
    if (threadIdx.x != 0) return;
    const uint32_t g = blockIdx.x / kCoopGroup;
    const uint64_t p = __hip_atomic_fetch_add(coop_left(b, g), 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)p + 1u != coop_gsize(g)) return;
    const uint64_t q = __hip_atomic_fetch_add(coop_top_left(b), 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)q + 1u != coop_ngroups()) return;
    const uint64_t z = (uint64_t)b.tag << 32;
    const uint32_t ar = top_abort_round(ld_agent(coop_top(b)));
    for (uint32_t k = 0; k < coop_ngroups(); ++k) {
        __hip_atomic_store(coop_grp(b, k), z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(coop_flag(b, k), z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(coop_started(b, k), z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(coop_left(b, k), z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __hip_atomic_store(coop_top(b), z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(coop_top_left(b), z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t pend = z;
    if (record && (ar != 0 || ld_agent(coop_pending(b)) == (z | 1u))) pend = z | (uint64_t)ar << 8 | 1u;
    __hip_atomic_store(coop_pending(b), pend, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Dense values of the first cnt < T elements of a tile into the LDS tile,
// element by element (pk bytes from pkb, sm bytes from smb).
__device__ inline void decode_partial_lds(const uint8_t *pkb, const uint8_t *smb, uint32_t cnt,
                                          const uint32_t *pair_lut, uint32_t *tile, uint32_t tid) {
    uint16_t *t16 = reinterpret_cast<uint16_t *>(tile);
    for (uint32_t i = tid; i < cnt; i += kDecThreads) {
        const uint32_t ee = pair_lut[pkb[i / 2]];
        t16[i] = (uint16_t)join16(smb[i], (i & 1) ? ee >> 16 : ee & 0xFFu);
    }
}

// Dense values of one unit (pair table in LDS): its 8 BF16 bit patterns.
__device__ __forceinline__ u32x4 decode_unit(const uint32_t *pair_lut, uint32_t p, u32x2 m) {
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t ee = pair_lut[(p >> (8 * k)) & 0xFFu];
        const uint32_t s = m[k >> 1] >> (16 * (k & 1));
        o[k] = join16(s & 0xFFu, ee & 0xFFu) | (join16((s >> 8) & 0xFFu, ee >> 16) << 16);
    }
    return o;
}

// ... into the LDS tile at element l0.
__device__ __forceinline__ void decode_unit_lds(const uint32_t *pair_lut, uint32_t p, u32x2 m,
                                                uint32_t *tile, uint32_t l0) {
    *reinterpret_cast<u32x4 *>(tile + l0 / 2) = decode_unit(pair_lut, p, m);
}

// The dense values of a whole tile, from registers straight to out[0, T).
__device__ __forceinline__ void store_units(const uint32_t *pair_lut, const uint32_t (&p)[kDecUnits],
                                            const u32x2 (&m)[kDecUnits], uint16_t *out, uint32_t tid) {
#pragma unroll
    for (int u = 0; u < kDecUnits; ++u)
        __builtin_nontemporal_store(decode_unit(pair_lut, p[u], m[u]),
                                    reinterpret_cast<u32x4 *>(out + (u * kDecThreads + tid) * kUnit));
}

// The LDS tile to out[0, cnt).
__device__ __forceinline__ void store_tile(const uint32_t *tile, uint16_t *out, uint32_t cnt,
                                           uint32_t tid) {
    if (cnt == kCoopTile) {
#pragma unroll
        for (int u = 0; u < kDecUnits; ++u) {
            const uint32_t l0 = (u * kDecThreads + tid) * kUnit;
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(tile + l0 / 2),
                                        reinterpret_cast<u32x4 *>(out + l0));
        }
    } else {
        const uint16_t *t16 = reinterpret_cast<const uint16_t *>(tile);
        for (uint32_t i = tid; i < cnt; i += kDecThreads) out[i] = t16[i];
    }
}

// Escape ranks [r0, r1) of the chunks that hold the tile at element base
// (one wave; the stream ascending).
__device__ inline void tile_escape_range(const int32_t *cid, uint64_t e, uint64_t n, uint32_t chunk,
                                         uint64_t base, uint64_t &r0, uint64_t &r1) {
    const int lane = threadIdx.x & 63;
    uint64_t c0, c1, nchunks;
    uint32_t p0, p1, pn;
    chunk_split(base, chunk, c0, p0);
    chunk_split(base + kCoopTile - 1, chunk, c1, p1);
    chunk_split(n - 1, chunk, nchunks, pn);
    ++c1;
    ++nchunks;
    if (c1 > nchunks) c1 = nchunks;
    const double per_chunk = (double)e / (double)nchunks;
    r0 = lower_bound_wave(cid, 0, e, (int64_t)c0, (uint64_t)(per_chunk * (double)c0), lane);
    r1 = lower_bound_wave(cid, r0, e, (int64_t)c1, r0 + (uint64_t)(per_chunk * (double)(c1 - c0)), lane);
}

// Applies the escapes of ranks [r0, r1) that fall in the LDS tile at element base.
__device__ inline void patch_tile_lds(uint32_t *tile, const int32_t *cid, const uint16_t *lpos,
                                      const uint8_t *ev, uint64_t r0, uint64_t r1, uint32_t chunk,
                                      uint64_t base, uint32_t tid) {
    uint16_t *t16 = reinterpret_cast<uint16_t *>(tile);
    for (uint64_t r = r0 + tid; r < r1; r += kDecThreads) {
        const int64_t v = (int64_t)cid[r] * chunk + lpos[r] - (int64_t)base;
        if (v >= 0 && v < kCoopTile) t16[v] = (uint16_t)((t16[v] & 0x807Fu) | ((uint32_t)ev[r] << 7));
    }
}

// Escapes of the LDS tile at element base (ranks found by wave 0 in the
// ascending stream cid/lpos/ev), then the tile to out[base, base + cnt).
__device__ inline void finish_tile(CoopLds &sh, bool patch, const int32_t *cid, const uint16_t *lpos,
                                   const uint8_t *ev, uint64_t e, uint64_t n, uint32_t chunk,
                                   uint64_t base, uint32_t cnt, uint16_t *out, uint32_t tid) {
    if (patch && tid < 64) {
        uint64_t r0, r1;
        tile_escape_range(cid, e, n, chunk, base, r0, r1);
        if (tid == 0) {
            sh.dr0 = r0;
            sh.dr1 = r1;
        }
    }
    __syncthreads();
    if (patch) {
        patch_tile_lds(sh.tile, cid, lpos, ev, sh.dr0, sh.dr1, chunk, base, tid);
        __syncthreads();
    }
    store_tile(sh.tile, out + base, cnt, tid);
    __syncthreads();
}

// (5 workgroups per compute unit: at most 96 VGPRs, 1,280 resident workgroups)
__global__ __launch_bounds__(kDecThreads, 5) void k_decode_slot_hold(DecArgs a) {
    __shared__ CoopLds sh;
    __shared__ uint32_t verdict;
    CoopBar bar;
    coop_bar_init(bar, a.hold_block, a.hold_tag);

#pragma unroll 1
    for (uint32_t item = 0; item < a.count; ++item) {
        // Fresh copies of the ids for every tensor keep the compiler from
        // hoisting the addresses of every held unit out of the loop (they
        // would take the registers the held tiles need).
        uint32_t tid = threadIdx.x, wg = blockIdx.x, G = gridDim.x;
        asm volatile("" : "+v"(tid), "+s"(wg), "+s"(G));
        const DecItem I = a.it[item];
        if (I.n == 0) continue;
        Layout L;
        if (!meta_ok(I, L) || L.total > I.other_bytes) {   // payload fits slot and stash
            if (wg == 0 && tid == 0 && a.status) atomicOr(a.status, 1);
            continue;
        }
        const uint64_t e = I.meta->n_esc;
        const uint32_t chunk = (uint32_t)I.meta->chunk_size;
        const bool ascending = (I.meta->flags & SPLITZIP_META_ASCENDING) != 0;
        const bool patch = e && ascending;   // escapes applied tile by tile
        // an unmarked stream with escapes is left to k_decode_slot_defer whole
        const bool deferred = e && !ascending;
        // A tensor whose escapes average more than 512 per tile is patched
        // tile by tile in LDS; a sparser one has its dense values stored
        // straight from registers and its escapes stored after them.
        const bool in_lds = patch && e * (uint64_t)kCoopTile > (uint64_t)kHoldEsc * I.n;
        const Layout L0 = layout_of(I.n, 0);
        const uint32_t *pk = reinterpret_cast<const uint32_t *>(I.payload);
        const u32x2 *sm = reinterpret_cast<const u32x2 *>(I.payload + L0.off_sm);
        const uint8_t *sm8 = I.payload + L0.off_sm;
        const int32_t *cid = reinterpret_cast<const int32_t *>(I.payload + L.off_cid);
        const uint16_t *lpos = reinterpret_cast<const uint16_t *>(I.payload + L.off_lpos);
        const uint8_t *ev = I.payload + L.off_ev;
        const int32_t *scid = reinterpret_cast<const int32_t *>(I.stash + L.off_cid);
        const uint16_t *slpos = reinterpret_cast<const uint16_t *>(I.stash + L.off_lpos);
        const uint8_t *sev = I.stash + L.off_ev;
        const uint64_t tiles = (I.n + kCoopTile - 1) / kCoopTile;
        const uint64_t t_split = slot_split(L.total, tiles, kCoopTile);
        // Tiles below t_split: tile wg + jG is held in registers for j <
        // kHold when it is whole; the others (beyond the registers' reach,
        // or the partial last tile) go through the stash, copied and read
        // back by the same workgroup.
        const uint32_t last_cnt = (uint32_t)(I.n - (tiles - 1) * kCoopTile);
        const bool part_held = last_cnt < kCoopTile && tiles - 1 < t_split;
        const uint64_t t_whole = part_held ? tiles - 1 : t_split;   // whole tiles below t_split
        const uint64_t reach = deferred ? 0 : (uint64_t)kHold * G;
        const bool mine_part = part_held && (tiles - 1) % G == wg;
        // Stashed tiles search and patch their escapes after the barrier,
        // from the stash: then the escape sections go there first, and the
        // barrier makes every workgroup's copy visible.
        const bool stashed = part_held || t_whole > reach;
        const bool esc_to_stash = a.status || (e && (!ascending || stashed));

        // ---- phase 1: the stashed tiles' inputs, the held tiles' escape
        // entries, the escape sections when a later pass reads them, the
        // direct tiles, then the held tiles' inputs
        for (uint64_t t = wg + reach; t < t_whole; t += G) {
            const uint64_t k0 = t * kCoopUnits;
            uint32_t *spk = reinterpret_cast<uint32_t *>(I.stash);
            u32x2 *ssm = reinterpret_cast<u32x2 *>(I.stash + L0.off_sm);
#pragma unroll
            for (int u = 0; u < kDecUnits; ++u) {
                const uint64_t k = k0 + u * kDecThreads + tid;
                spk[k] = __builtin_nontemporal_load(pk + k);
                ssm[k] = __builtin_nontemporal_load(sm + k);
            }
        }
        if (mine_part) {   // the partial tile's inputs, at their payload offsets
            const uint64_t base = (tiles - 1) * kCoopTile;
            for (uint32_t i = tid; i < last_cnt; i += kDecThreads) {
                I.stash[L0.off_sm + base + i] = I.payload[L0.off_sm + base + i];
                if (!(i & 1)) I.stash[(base + i) / 2] = I.payload[(base + i) / 2];
            }
        }
        __syncthreads();   // the previous tensor's last reads of LDS
        if (tid < 256)
            sh.pair_lut[tid] = (uint32_t)I.dec_lut[(tid >> 4) & 15] | ((uint32_t)I.dec_lut[tid & 15] << 16);
        if (patch && (tid >> 6) < kHold) {   // wave j: the escapes of held tile j
            const uint32_t wave = tid >> 6, lane = tid & 63;
            const uint64_t t = wg + (uint64_t)wave * G;
            const uint64_t base = t * kCoopTile;
            uint64_t r0 = 0, r1 = 0;
            if (t < t_whole) tile_escape_range(cid, e, I.n, chunk, base, r0, r1);
            if (lane == 0) {
                sh.hr0[wave] = r0;
                sh.hr1[wave] = r1;
            }
            // (position << 16) | (sign and mantissa << 8) | exponent
            if (r1 - r0 <= kHoldEsc)
                for (uint64_t r = r0 + lane; r < r1; r += 64) {
                    const int64_t v = (int64_t)cid[r] * chunk + lpos[r] - (int64_t)base;
                    sh.esc[wave][r - r0] = (v >= 0 && v < kCoopTile)
                                               ? ((uint32_t)v << 16) | ((uint32_t)sm8[base + v] << 8) | ev[r]
                                               : ~0u;
                }
        }
        __syncthreads();
        if (esc_to_stash) {
            // the escape sections, for the stashed tiles, the validation
            // pass or the order-independent pass
            const uint64_t bytes = L.total - L.off_cid;
            const uint32_t *src = reinterpret_cast<const uint32_t *>(I.payload + L.off_cid);
            uint32_t *dst = reinterpret_cast<uint32_t *>(I.stash + L.off_cid);
            for (uint64_t w = (uint64_t)wg * kDecThreads + tid; w < bytes / 4; w += (uint64_t)G * kDecThreads)
                dst[w] = src[w];
            if (wg == 0 && tid < (uint32_t)(bytes & 3)) {
                const uint64_t b = L.off_cid + (bytes & ~uint64_t(3)) + tid;
                I.stash[b] = I.payload[b];
            }
        }
        if (patch) {
            // held tiles with many escapes: their entries to the stash, read
            // back after the barrier by this workgroup
            for (int j = 0; j < kHold; ++j) {
                const uint64_t r0 = sh.hr0[j], r1 = sh.hr1[j];
                if (r1 - r0 <= kHoldEsc) continue;
                for (uint64_t r = r0 + tid; r < r1; r += kDecThreads) {
                    reinterpret_cast<int32_t *>(I.stash + L.off_cid)[r] = cid[r];
                    reinterpret_cast<uint16_t *>(I.stash + L.off_lpos)[r] = lpos[r];
                    I.stash[L.off_ev + r] = ev[r];
                }
            }
        }
        // direct tiles: their output lies past the payload.  Whole tiles of
        // a sparse tensor: dense values straight to memory, then the escapes.
        const uint64_t t_dl = in_lds ? t_split : (last_cnt < kCoopTile ? tiles - 1 : tiles);
        for (uint64_t t = t_split + wg; t < t_dl; t += G) {
            const uint64_t base = t * kCoopTile;
            const uint32_t *pkt = pk + t * kCoopUnits;
            const u32x2 *smt = sm + t * kCoopUnits;
            uint32_t p[kDecUnits];
            u32x2 m[kDecUnits];
#pragma unroll
            for (int u = 0; u < kDecUnits; ++u) {
                p[u] = __builtin_nontemporal_load(pkt + u * kDecThreads + tid);
                m[u] = __builtin_nontemporal_load(smt + u * kDecThreads + tid);
            }
            store_units(sh.pair_lut, p, m, I.out + base, tid);
            if (patch) {
                if (tid < 64) {
                    uint64_t r0, r1;
                    tile_escape_range(cid, e, I.n, chunk, base, r0, r1);
                    if (tid == 0) {
                        sh.dr0 = r0;
                        sh.dr1 = r1;
                    }
                }
                __syncthreads();   // (also orders the dense stores before the patches)
                for (uint64_t r = sh.dr0 + tid; r < sh.dr1; r += kDecThreads) {
                    const int64_t v = (int64_t)cid[r] * chunk + lpos[r] - (int64_t)base;
                    if (v >= 0 && v < kCoopTile) I.out[base + v] = (uint16_t)join16(sm8[base + v], ev[r]);
                }
                __syncthreads();
            }
        }
        // the rest (a dense tensor's tiles, the partial last tile) through LDS
        for (uint64_t t = t_split + wg; t < tiles; t += G) {
            if (t < t_dl) continue;
            const uint64_t base = t * kCoopTile;
            const uint32_t cnt = t == tiles - 1 ? last_cnt : kCoopTile;
            if (cnt == kCoopTile) {
                const uint32_t *pkt = pk + t * kCoopUnits;
                const u32x2 *smt = sm + t * kCoopUnits;
#pragma unroll
                for (int u = 0; u < kDecUnits; ++u)
                    decode_unit_lds(sh.pair_lut, __builtin_nontemporal_load(pkt + u * kDecThreads + tid),
                                    __builtin_nontemporal_load(smt + u * kDecThreads + tid), sh.tile,
                                    (u * kDecThreads + tid) * kUnit);
            } else {
                decode_partial_lds(I.payload + base / 2, sm8 + base, cnt, sh.pair_lut, sh.tile, tid);
            }
            finish_tile(sh, patch, cid, lpos, ev, e, I.n, chunk, base, cnt, I.out, tid);
        }
        // the held tiles' inputs last: their registers are live only across
        // the barrier
        uint32_t hpk[kHold][kDecUnits];
        u32x2 hsm[kHold][kDecUnits];
#pragma unroll
        for (int j = 0; j < kHold; ++j) {
            const uint64_t t = wg + (uint64_t)j * G;
            // (defined on both paths, so that no register stays live
            // across the loop over tensors)
#pragma unroll
            for (int u = 0; u < kDecUnits; ++u) {
                hpk[j][u] = 0;
                hsm[j][u] = u32x2{0u, 0u};
            }
            if (t < t_whole && !deferred) {
                const uint32_t *pkt = pk + t * kCoopUnits;
                const u32x2 *smt = sm + t * kCoopUnits;
#pragma unroll
                for (int u = 0; u < kDecUnits; ++u) {
                    hpk[j][u] = __builtin_nontemporal_load(pkt + u * kDecThreads + tid);
                    hsm[j][u] = __builtin_nontemporal_load(smt + u * kDecThreads + tid);
                }
            }
        }
        if (deferred) {
            if (wg == 0 && tid == 0) coop_set_pending(bar);
            continue;
        }
        if (!coop_barrier(bar, a.wait_ticks, patch && stashed, &verdict)) {
            // aborted: the held tiles' inputs and this workgroup's share of
            // the escape sections to the stash, for k_decode_slot_defer
#pragma unroll
            for (int j = 0; j < kHold; ++j) {
                const uint64_t t = wg + (uint64_t)j * G;
                if (t >= t_whole) break;
                uint32_t *spk = reinterpret_cast<uint32_t *>(I.stash) + t * kCoopUnits;
                u32x2 *ssm = reinterpret_cast<u32x2 *>(I.stash + L0.off_sm) + t * kCoopUnits;
#pragma unroll
                for (int u = 0; u < kDecUnits; ++u) {
                    spk[u * kDecThreads + tid] = hpk[j][u];
                    ssm[u * kDecThreads + tid] = hsm[j][u];
                }
            }
            if (e && !esc_to_stash) {
                const uint64_t bytes = L.total - L.off_cid;
                const uint32_t *src = reinterpret_cast<const uint32_t *>(I.payload + L.off_cid);
                uint32_t *dst = reinterpret_cast<uint32_t *>(I.stash + L.off_cid);
                for (uint64_t w = (uint64_t)wg * kDecThreads + tid; w < bytes / 4;
                     w += (uint64_t)G * kDecThreads)
                    dst[w] = src[w];
                if (wg == 0 && tid < (uint32_t)(bytes & 3)) {
                    const uint64_t b = L.off_cid + (bytes & ~uint64_t(3)) + tid;
                    I.stash[b] = I.payload[b];
                }
            }
            continue;
        }

        // ---- phase 2: the held tiles (dense values straight from the
        // registers, or through LDS for a tile with many escapes), their
        // escapes, then the stashed tiles
#pragma unroll
        for (int j = 0; j < kHold; ++j) {
            const uint64_t t = wg + (uint64_t)j * G;
            if (t >= t_whole) break;
            const uint64_t base = t * kCoopTile;
            if (!patch || sh.hr1[j] - sh.hr0[j] <= kHoldEsc) {
                store_units(sh.pair_lut, hpk[j], hsm[j], I.out + base, tid);
                continue;
            }
#pragma unroll
            for (int u = 0; u < kDecUnits; ++u)
                decode_unit_lds(sh.pair_lut, hpk[j][u], hsm[j][u], sh.tile, (u * kDecThreads + tid) * kUnit);
            __syncthreads();
            // entries this workgroup copied to the stash
            patch_tile_lds(sh.tile, scid, slpos, sev, sh.hr0[j], sh.hr1[j], chunk, base, tid);
            __syncthreads();
            store_tile(sh.tile, I.out + base, kCoopTile, tid);
            __syncthreads();
        }
        if (patch) {
            __syncthreads();   // the dense stores before the escapes' stores
            for (int j = 0; j < kHold; ++j) {
                const uint64_t t = wg + (uint64_t)j * G;
                const uint64_t c = sh.hr1[j] - sh.hr0[j];
                if (t >= t_whole || c > kHoldEsc) continue;
                uint16_t *o = I.out + t * kCoopTile;
                for (uint32_t k = tid; k < (uint32_t)c; k += kDecThreads) {
                    const uint32_t w = sh.esc[j][k];
                    if (w != ~0u) o[w >> 16] = (uint16_t)join16((w >> 8) & 0xFFu, w & 0xFFu);
                }
            }
        }
        if (stashed) {
            for (uint64_t t = wg + reach; t < t_whole; t += G) {
                const uint32_t *spk = reinterpret_cast<const uint32_t *>(I.stash) + t * kCoopUnits;
                const u32x2 *ssm = reinterpret_cast<const u32x2 *>(I.stash + L0.off_sm) + t * kCoopUnits;
                uint32_t p[kDecUnits];
                u32x2 m[kDecUnits];
#pragma unroll
                for (int u = 0; u < kDecUnits; ++u) {
                    p[u] = __builtin_nontemporal_load(spk + u * kDecThreads + tid);
                    m[u] = __builtin_nontemporal_load(ssm + u * kDecThreads + tid);
                }
                __syncthreads();   // LDS tile free
#pragma unroll
                for (int u = 0; u < kDecUnits; ++u)
                    decode_unit_lds(sh.pair_lut, p[u], m[u], sh.tile, (u * kDecThreads + tid) * kUnit);
                finish_tile(sh, patch, scid, slpos, sev, e, I.n, chunk, t * kCoopTile, kCoopTile, I.out,
                            tid);
            }
            if (mine_part) {
                const uint64_t base = (tiles - 1) * kCoopTile;
                __syncthreads();
                decode_partial_lds(I.stash + base / 2, I.stash + L0.off_sm + base, last_cnt, sh.pair_lut,
                                   sh.tile, tid);
                finish_tile(sh, patch, scid, slpos, sev, e, I.n, chunk, base, last_cnt, I.out, tid);
            }
        }
    }
    coop_leave(bar, true);
}

// The slots k_decode_slot_hold left: those whose barrier aborted and those
// with an unmarked escape stream.  Their tiles below t_split are decoded
// from the stash (the inputs and escape sections the first kernel put
// there) as the multi-pass form's last pass does; an unmarked stream's
// escapes are then applied at their indices by the last workgroup to finish
// the tensor.  The last workgroup of the grid puts the barrier block back.
__global__ __launch_bounds__(kDecThreads) void k_decode_slot_defer(DecArgs a) {
    __shared__ CoopLds sh;
    __shared__ uint32_t last;
    // the first kernel's last workgroup put the counters back to (tag << 32)
    CoopBar bar;
    bar.blk = a.hold_block;
    bar.tag = a.hold_tag;
    bar.passed = 0;
    if (threadIdx.x == 0) {
        const uint64_t pend = ld_agent(coop_pending(bar));
        last = (uint32_t)(pend >> 32) == bar.tag && (pend & 1u) ? 1u | ((uint32_t)pend & 0xFF00u) : 0u;
    }
    __syncthreads();
    if (!last) return;   // nothing was left (the common case)
    const uint32_t abort_round = last >> 8;
    uint32_t round = 0;

#pragma unroll 1
    for (uint32_t item = 0; item < a.count; ++item) {
        const uint32_t tid = threadIdx.x, wg = blockIdx.x, G = gridDim.x;
        const DecItem I = a.it[item];
        if (I.n == 0) continue;
        Layout L;
        if (!meta_ok(I, L) || L.total > I.other_bytes) continue;   // reported by the first kernel
        const uint64_t e = I.meta->n_esc;
        const uint32_t chunk = (uint32_t)I.meta->chunk_size;
        const bool ascending = (I.meta->flags & SPLITZIP_META_ASCENDING) != 0;
        const bool deferred = e && !ascending;
        if (!deferred) {
            ++round;
            if (round_verdict(abort_round, round) == kGo) continue;
        }
        const bool patch = e && ascending;
        const Layout L0 = layout_of(I.n, 0);
        const int32_t *scid = reinterpret_cast<const int32_t *>(I.stash + L.off_cid);
        const uint16_t *slpos = reinterpret_cast<const uint16_t *>(I.stash + L.off_lpos);
        const uint8_t *sev = I.stash + L.off_ev;
        const uint64_t tiles = (I.n + kCoopTile - 1) / kCoopTile;
        const uint64_t t_split = slot_split(L.total, tiles, kCoopTile);
        const uint32_t last_cnt = (uint32_t)(I.n - (tiles - 1) * kCoopTile);
        __syncthreads();   // the previous tensor's last reads of LDS
        if (tid < 256)
            sh.pair_lut[tid] = (uint32_t)I.dec_lut[(tid >> 4) & 15] | ((uint32_t)I.dec_lut[tid & 15] << 16);
        __syncthreads();
        for (uint64_t t = wg; t < t_split; t += G) {
            const uint64_t base = t * kCoopTile;
            const uint32_t cnt = t == tiles - 1 ? last_cnt : kCoopTile;
            if (cnt == kCoopTile) {
                const uint32_t *spk = reinterpret_cast<const uint32_t *>(I.stash) + t * kCoopUnits;
                const u32x2 *ssm = reinterpret_cast<const u32x2 *>(I.stash + L0.off_sm) + t * kCoopUnits;
#pragma unroll
                for (int u = 0; u < kDecUnits; ++u)
                    decode_unit_lds(sh.pair_lut, __builtin_nontemporal_load(spk + u * kDecThreads + tid),
                                    __builtin_nontemporal_load(ssm + u * kDecThreads + tid), sh.tile,
                                    (u * kDecThreads + tid) * kUnit);
            } else {
                decode_partial_lds(I.stash + base / 2, I.stash + L0.off_sm + base, cnt, sh.pair_lut,
                                   sh.tile, tid);
            }
            finish_tile(sh, patch, scid, slpos, sev, e, I.n, chunk, base, cnt, I.out, tid);
        }
        if (deferred) {
            // every workgroup releases its stores and arrives; the last one
            // applies every escape at its index (sign and mantissa from the
            // decoded value)
            __threadfence();
            wait_vector_memory();
            __syncthreads();
            if (tid == 0) {
                const uint64_t t = a.order_ticket + item;
                uint64_t *c = a.order_sync + (t & (kOrderSlots - 1));
                counter_claim(c, ld_agent(c), (uint32_t)t + 1u);
                last = tagged_arrive(c, G, (uint32_t)t + 1u);
            }
            __syncthreads();
            if (last) {
                __threadfence();
                for (uint64_t r = tid; r < e; r += kDecThreads) {
                    const int32_t c = scid[r];
                    if (c < 0) continue;
                    const uint64_t idx = (uint64_t)c * chunk + slpos[r];
                    if (idx >= I.n) continue;
                    I.out[idx] = (uint16_t)join16(sm_of16(I.out[idx]), sev[r]);
                }
            }
        }
    }
    coop_leave(bar, false);
}

// Validation (and order-independent re-application) of every escape, only
// when a status word is requested.  The sign and mantissa come from the
// payload, or, after a slot decode (whose stash holds only part of the sm
// section), from the decoded output itself.
template <bool kFromOut>
__global__ __launch_bounds__(kThreads) void k_decode_check(DecArgs a) {
    const uint64_t gs = (uint64_t)gridDim.x * kThreads;
    int32_t bad = 0;
    for (uint32_t item = 0; item < a.count; ++item) {
        const DecItem I = a.it[item];
        if (I.n == 0) continue;
        Layout L;
        if (!meta_ok(I, L) || (kFromOut && L.total > I.other_bytes))
            continue;   // reported by k_decode
        const uint64_t e = I.meta->n_esc;
        const uint64_t chunk = I.meta->chunk_size;
        const uint8_t *sm = I.payload + L.off_sm;
        const int32_t *cid = reinterpret_cast<const int32_t *>(I.payload + L.off_cid);
        const uint16_t *lpos = reinterpret_cast<const uint16_t *>(I.payload + L.off_lpos);
        const uint8_t *ev = I.payload + L.off_ev;
        for (uint64_t r = (uint64_t)blockIdx.x * kThreads + threadIdx.x; r < e; r += gs) {
            const int32_t c = cid[r];
            const uint32_t pos = lpos[r];
            if (c < 0) { bad |= 2; continue; }
            if (pos >= chunk) bad |= 4;
            const uint64_t idx = (uint64_t)c * chunk + pos;
            if (idx >= I.n) { bad |= 2; continue; }
            if (r > 0) {
                const int32_t pc = cid[r - 1];
                const uint64_t prev = (uint64_t)(uint32_t)pc * chunk + lpos[r - 1];
                if (pc < 0 || prev >= idx) bad |= 8;
            }
            const uint32_t keep = kFromOut ? sm_of16(I.out[idx]) : sm[idx];
            I.out[idx] = (uint16_t)join16(keep, ev[r]);
        }
    }
    if (bad && a.status) atomicOr(a.status, bad);
}

__global__ void k_fill_zero(uint32_t *p, uint64_t words) {
    for (uint64_t k = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; k < words;
         k += (uint64_t)gridDim.x * blockDim.x)
        p[k] = 0;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// Compute units of the current device, cached per device (host threads may
// race to fill an entry; they all store the same value).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

bool cu_count(int &cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
    int c = dev < kMaxDevices ? g_cu_count[dev].load(std::memory_order_relaxed) : 0;
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return false;
        if (c <= 0) c = 1;
        if (dev < kMaxDevices) g_cu_count[dev].store(c, std::memory_order_relaxed);
    }
    cus = c;
    return true;
}

// Workgroups of the resident slot decode that the current device keeps
// resident at once (0: none), and whether it has cooperative launches,
// cached per device (-1: not known yet).
std::atomic<int> g_coop_grid[kMaxDevices];
std::atomic<int> g_coop_ok[kMaxDevices];

bool coop_grid(uint32_t &grid, bool &coop) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
    int g = dev < kMaxDevices ? g_coop_grid[dev].load(std::memory_order_relaxed) : 0;
    int c = dev < kMaxDevices ? g_coop_ok[dev].load(std::memory_order_relaxed) : -1;
    if (g == 0 || c < 0) {
        int per_cu = 0, cus = 0;
        if (!cu_count(cus) ||
            hipDeviceGetAttribute(&c, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_decode_slot_hold, kDecThreads, 0) !=
                hipSuccess)
            return false;
        g = per_cu > 0 ? per_cu * cus : -1;
        if (g > (int)kCoopMaxGrid) g = (int)kCoopMaxGrid;
        c = c ? 1 : 0;
        if (dev < kMaxDevices) {
            g_coop_grid[dev].store(g, std::memory_order_relaxed);
            g_coop_ok[dev].store(c, std::memory_order_relaxed);
        }
    }
    grid = g > 0 ? (uint32_t)g : 0u;
    coop = c == 1;
    return true;
}

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// The current device's address of g_order_sync (each device holds its own
// copy), cached per device.
std::atomic<uint64_t *> g_order_pool[kMaxDevices];
// Workspace of splitzip_encode_noalloc, for callers that cannot allocate:
// an encode-only area (tile counts, count sums, staging) of fixed size in
// device memory the library owns.  Each device holds its own copy until the
// process ends; host code reaches it only through its per-device address.
constexpr size_t kScratchBytes = SPLITZIP_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr WsPlan kScratchPlan = ws_plan(kScratchBytes, 0);
static_assert(kScratchPlan.t_max * kEncTile == SPLITZIP_NOALLOC_MAX_N,
              "the header's limit is the scratch plan's");
std::atomic<uint8_t *> g_scratch[kMaxDevices];

// Address of `scratch` on the current device, looked up on the first call
// on that device.
bool scratch_of_device(uint8_t *&p) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
    p = dev < kMaxDevices ? g_scratch[dev].load(std::memory_order_relaxed) : nullptr;
    if (p) return true;
    void *q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return false;
    p = static_cast<uint8_t *>(q);
    if (dev < kMaxDevices) g_scratch[dev].store(p, std::memory_order_relaxed);
    return true;
}

// Tags of the tagged arrival counters: each call takes as many as it has
// tensors (shared by calibrate and decode; only uniqueness matters).
std::atomic<uint64_t> g_ticket{0};

bool order_counters(DecArgs &a, uint32_t count) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
    uint64_t *p = dev < kMaxDevices ? g_order_pool[dev].load(std::memory_order_relaxed) : nullptr;
    if (!p) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(g_order_sync)) != hipSuccess || !q) return false;
        p = static_cast<uint64_t *>(q);
        if (dev < kMaxDevices) g_order_pool[dev].store(p, std::memory_order_relaxed);
    }
    a.order_sync = p;
    a.order_ticket = g_ticket.fetch_add(count, std::memory_order_relaxed);
    return true;
}

// The barrier block of a resident slot decode.  Calls on one stream run
// one after another and share a block (each claims it with its own tag);
// each stream keeps its block while it is among the kCoopBlocks streams of
// the device that used one last, so two calls that run at the same time
// share a block only when more than kCoopBlocks streams decode slots at once.
std::atomic<uint64_t *> g_coop_pool[kMaxDevices];
struct CoopOwner {
    hipStream_t stream;
    uint64_t used;   // 0: never
};
CoopOwner g_coop_owner[kMaxDevices][kCoopBlocks];
uint64_t g_coop_clock = 0;
std::mutex g_coop_mutex;

bool coop_block(DecArgs &a, hipStream_t s) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
    uint64_t *p = dev < kMaxDevices ? g_coop_pool[dev].load(std::memory_order_relaxed) : nullptr;
    if (!p) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(g_coop_sync)) != hipSuccess || !q) return false;
        p = static_cast<uint64_t *>(q);
        if (dev < kMaxDevices) g_coop_pool[dev].store(p, std::memory_order_relaxed);
    }
    uint32_t blk = 0;
    {
        std::lock_guard<std::mutex> lock(g_coop_mutex);
        CoopOwner *own = g_coop_owner[dev < kMaxDevices ? dev : 0];
        for (uint32_t k = 0; k < kCoopBlocks; ++k) {
            if (own[k].used && own[k].stream == s) {
                blk = k;
                break;
            }
            if (own[k].used < own[blk].used) blk = k;   // else the least recently used
        }
        own[blk].stream = s;
        own[blk].used = ++g_coop_clock;
    }
    const uint64_t ticket = g_ticket.fetch_add(1, std::memory_order_relaxed);
    a.hold_block = p + (uint64_t)blk * kCoopWords;
    a.hold_tag = (uint32_t)ticket + 1u;
    return true;
}

inline uint64_t enc_tiles(uint64_t n) { return (n + kEncTile - 1) / kEncTile; }

inline uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

// Device address of a codebook's dec_lut (address arithmetic only).
inline const uint8_t *dec_lut_of(const splitzip_codebook *cb) {
    return reinterpret_cast<const uint8_t *>(cb) + offsetof(splitzip_codebook, dec_lut);
}

int launched() {
    return hipGetLastError() == hipSuccess ? SPLITZIP_OK : SPLITZIP_ERR_HIP;
}

// Argument checks shared by the single and batched entry points.
int check_calibrate_item(const uint16_t *x, uint64_t n, const splitzip_codebook *cb) {
    if (n > SPLITZIP_MAX_N || (n && (!x || !aligned(x, 16))) || !cb || !aligned(cb, 8))
        return SPLITZIP_ERR_INVALID;
    return SPLITZIP_OK;
}

int check_encode_item(const uint16_t *x, uint64_t n, const splitzip_codebook *cb,
                      const uint8_t *payload, uint64_t capacity, const splitzip_meta *meta) {
    if (check_calibrate_item(x, n, cb) || !meta || !aligned(meta, 8) || (!payload && capacity) ||
        !aligned(payload, 16))
        return SPLITZIP_ERR_INVALID;
    if (capacity < layout_of(n, 0).total) return SPLITZIP_ERR_CAPACITY;
    return SPLITZIP_OK;
}

int check_decode_item(const uint8_t *payload, uint64_t payload_bytes, const splitzip_meta *meta,
                      const uint8_t *dec_lut, const uint16_t *out, uint64_t n) {
    if (n > SPLITZIP_MAX_N || !meta || !aligned(meta, 8) || !dec_lut ||
        (n && (!payload || !aligned(payload, 16) || !out || !aligned(out, 16))))
        return SPLITZIP_ERR_INVALID;
    // no payload of n elements is shorter than its dense sections
    if (n && payload_bytes < layout_of(n, 0).total) return SPLITZIP_ERR_INVALID;
    return SPLITZIP_OK;
}

// Calibrate launch for up to kMaxBatch tensors: the GPU's worth of resident
// workgroups is shared out in proportion to size (at least one per tensor,
// at most one per 4096 16-byte loads and kCalMaxGrid per tensor).
int launch_calibrate(const CalItem *items, uint32_t count, uint8_t *ws, hipStream_t s) {
    int cus = 0;
    if (!cu_count(cus)) return SPLITZIP_ERR_HIP;
    CalArgs a{};
    a.count = count;
    a.ws = ws;
    uint64_t total = 0;
    for (uint32_t k = 0; k < count; ++k) total += items[k].n;
    // Two resident workgroups per compute unit hide the latency of short
    // ranges; a launch large enough that one per compute unit still runs
    // kCalLongLoop rounds of loads is faster with one (longer contiguous
    // ranges, half the merges: 2 % on 32 tensors of 32M elements).
    const uint64_t long_enough = kCalLongLoop * 4 * (uint64_t)kCalThreads * (uint64_t)cus;
    const uint64_t target = (uint64_t)((total >> 3) >= long_enough ? 1 : kCalTarget) * cus;
    uint32_t wg = 0;
    for (uint32_t k = 0; k < count; ++k) {
        a.it[k] = items[k];
        uint64_t g = total ? ceil_div(target * items[k].n, total) : 1;
        const uint64_t by_size = ceil_div(items[k].n >> 3, 4 * (uint64_t)kCalThreads);
        if (g > by_size) g = by_size;
        if (g > kCalMaxGrid) g = kCalMaxGrid;
        if (g == 0) g = 1;
        a.wg_start[k] = wg;
        wg += (uint32_t)g;
    }
    a.wg_start[count] = wg;
    a.ticket = g_ticket.fetch_add(count, std::memory_order_relaxed);
    k_calibrate<<<wg, kCalThreads, 0, s>>>(a);
    return launched();
}

// Encode launch (main + tail) for up to kMaxBatch tensors whose tiles fit the
// workspace plan.
int launch_encode(const EncItem *items, uint32_t count, const WsPlan &P, uint8_t *ws,
                  hipStream_t s) {
    EncArgs a{};
    a.count = count;
    a.tile_count = reinterpret_cast<uint32_t *>(ws + P.off_count);
    a.stage = reinterpret_cast<uint32_t *>(ws + P.off_stage);
    uint64_t tiles = 0;
    for (uint32_t k = 0; k < count; ++k) tiles += enc_tiles(items[k].n);
    uint32_t tt = kTailMinTiles;
    while (tt < (uint32_t)kTailMaxTiles && tiles / (2 * tt) >= kTailTargetWgs) tt *= 2;
    a.tail_tiles = tt;
    tiles = 0;
    uint32_t blks = 0, sups = 0;
    uint64_t direct_loads = 0;   // tile counts read by the tail launch without sums
    for (uint32_t k = 0; k < count; ++k) {
        a.it[k] = items[k];
        a.tile_start[k] = tiles;
        a.blk_start[k] = blks;
        a.sup_start[k] = sups;
        const uint64_t t = enc_tiles(items[k].n);
        tiles += t;
        const uint64_t b = ceil_div(t, tt);
        blks += (uint32_t)(b ? b : 1);   // an empty tensor still gets its metadata
        sups += (uint32_t)ceil_div(t, kSuperTiles);
        direct_loads += t * b;
    }
    a.tile_start[count] = tiles;
    a.blk_start[count] = blks;
    a.sup_start[count] = sups;
    if (tiles > P.t_max) return SPLITZIP_ERR_WORKSPACE;
    if (tiles) {
        k_encode<<<(unsigned)tiles, kThreads, 0, s>>>(a);
        if (hipGetLastError() != hipSuccess) return SPLITZIP_ERR_HIP;
    }
    // When every tail workgroup reading all of its tensor's tile counts adds
    // up to more than kTailDirect loads (16 MB at the default, about the cost
    // of a launch), one more launch first sums the counts per tail block and
    // per superblock.  A single call on a 64 MiB tensor stays below it
    // (measured: 3 us less on the GPU and one launch fewer per call); a batch
    // of 32 such tensors is above it (2.5 us less with the sums).
    if (direct_loads > kTailDirect) {
        a.blk_sum = reinterpret_cast<uint32_t *>(ws + P.off_bsum);
        a.sup_sum = reinterpret_cast<uint32_t *>(ws + P.off_ssum);
        k_encode_sums<<<sups, kThreads, 0, s>>>(a);
        if (hipGetLastError() != hipSuccess) return SPLITZIP_ERR_HIP;
    }
    k_encode_tail<<<blks, kTailThreads, 0, s>>>(a);
    return launched();
}

// Decode launch for up to kMaxBatch tensors.  8192-element tiles: measured
// against 16K and 32K tiles (and 4K), they stream fastest once the dense
// stores no longer wait for the escape search.
int launch_decode(const DecItem *items, uint32_t count, int32_t *status, hipStream_t s) {
    DecArgs a{};
    a.count = count;
    a.status = status;
    if (!order_counters(a, count)) return SPLITZIP_ERR_HIP;
    uint64_t tiles = 0;
    for (uint32_t k = 0; k < count; ++k) {
        a.it[k] = items[k];
        a.tile_start[k] = tiles;
        tiles += ceil_div(items[k].n, (uint64_t)kDecUnits * kDecThreads * kUnit);
    }
    a.tile_start[count] = tiles;
    if (tiles) {
        k_decode<kDecUnits><<<(unsigned)tiles, kDecThreads, 0, s>>>(a);
        if (hipGetLastError() != hipSuccess) return SPLITZIP_ERR_HIP;
    }
    if (status) {
        uint64_t n = 0;
        for (uint32_t k = 0; k < count; ++k) n += items[k].n;
        uint64_t cgrid = ceil_div(n, 16 * kThreads);
        if (cgrid > 1024) cgrid = 1024;
        if (cgrid == 0) cgrid = 1;
        k_decode_check<false><<<(unsigned)cgrid, kThreads, 0, s>>>(a);
    }
    return launched();
}

// Multi-pass in-place decode schedule (see the comment above
// k_decode_slot_stage): tile w < t_min runs in pass p(w) in [2, passes];
// p(w) >= k exactly when lo[k] <= w < hi[k] (k >= 2; lo[2] = 0, hi[2] =
// t_min).
constexpr uint32_t kSlotMaxPasses = 8;
// Passes chosen per launch: the most, up to kSlotAutoPasses, whose last pass
// still has kSlotMinFinal workgroups over the launch's tensors.  Measured on
// 64 KV tensors of 2^25 elements (4,096 tiles each): groups of 32 slots take
// 2.02 / 1.73 / 1.59 ms for 2 / 3 / 6 passes (6,144 workgroups in the last of
// six); one slot per call 2.60 / 2.73 ms for 2 / 3 passes (1,536 workgroups
// in the last of three), a launch that does not fill the GPU costing more
// than the stash bytes it saves.
constexpr uint32_t kSlotAutoPasses = 6;
constexpr uint64_t kSlotMinFinal = 4096;
struct SlotPlan {
    uint32_t passes;
    uint64_t t_min;
    uint64_t lo[kSlotMaxPasses + 1], hi[kSlotMaxPasses + 1];
};

struct SlotGeom {
    uint64_t n, tiles, t_min, s0;
};

// Tiles below t_min whose sm bytes meet tile w's output: [ta, tb]; false when none.
bool slot_readers(const SlotGeom &G, uint64_t w, uint64_t &ta, uint64_t &tb) {
    constexpr uint64_t T = kCoopTile;
    const uint64_t len = G.n - w * T < T ? G.n - w * T : T;
    const uint64_t o0 = 2 * w * T, o1 = o0 + 2 * len;
    if (o1 <= G.s0 || o0 >= G.s0 + G.n) return false;
    ta = o0 > G.s0 ? (o0 - G.s0) / T : 0;
    tb = (o1 - 1 - G.s0) / T;
    if (tb > G.t_min - 1) tb = G.t_min - 1;
    return ta <= tb;
}

// min(passes, 2 + depth(w)), following the reader nearest the
// self-overlapping tiles (the deepest one).
uint32_t slot_pass_of(const SlotGeom &G, uint64_t w, uint32_t passes) {
    uint32_t d = 2;
    while (d < passes) {
        uint64_t ta, tb;
        if (!slot_readers(G, w, ta, tb)) return d;
        if (ta <= w && w <= tb) return passes;
        w = tb < w ? tb : ta;
        ++d;
    }
    return d;
}

SlotPlan slot_plan(uint64_t n, uint32_t passes) {
    constexpr uint64_t T = kCoopTile;
    SlotPlan P{};
    const Layout L0 = layout_of(n, 0);
    const uint64_t tiles = (n + T - 1) / T;
    uint64_t t_min = (L0.off_cid + 2 * T - 1) / (2 * T);
    if (t_min > tiles) t_min = tiles;
    P.t_min = t_min;
    P.passes = 2;
    P.lo[2] = 0;
    P.hi[2] = t_min;
    if (t_min == 0 || passes <= 2) return P;
    const SlotGeom G{n, tiles, t_min, L0.off_sm};
    // a tile that overlaps its own sm bytes: the one holding the section's first byte
    uint64_t wz = L0.off_sm / T;
    if (wz > t_min - 1) wz = t_min - 1;
    if (slot_pass_of(G, wz, passes) != passes) return P;   // not expected; two passes are always valid
    for (uint32_t k = 3; k <= passes; ++k) {
        // pass is nondecreasing on [0, wz] and nonincreasing on [wz, t_min)
        uint64_t lo = 0, hi = wz;   // first w in [0, wz] with pass >= k
        while (lo < hi) {
            const uint64_t mid = lo + (hi - lo) / 2;
            if (slot_pass_of(G, mid, passes) >= k) hi = mid; else lo = mid + 1;
        }
        P.lo[k] = lo;
        lo = wz + 1;
        hi = t_min;   // first w in (wz, t_min) with pass < k, else t_min
        while (lo < hi) {
            const uint64_t mid = lo + (hi - lo) / 2;
            if (slot_pass_of(G, mid, passes) < k) hi = mid; else lo = mid + 1;
        }
        P.hi[k] = lo;
    }
    P.passes = passes;
    return P;
}

// Number of passes for a launch of `count` slots (SPLITZIP_SLOT_PASSES, 2..8,
// fixes it for every launch).
uint32_t slot_passes(const splitzip_slot_item *items, uint32_t count) {
    if (const char *v = getenv("SPLITZIP_SLOT_PASSES")) {
        const unsigned long k = strtoul(v, nullptr, 10);
        return k < 2 ? 2u : (k > kSlotMaxPasses ? kSlotMaxPasses : (uint32_t)k);
    }
    for (uint32_t k = kSlotAutoPasses; k > 2; --k) {
        uint64_t last = 0;
        for (uint32_t i = 0; i < count; ++i) {
            const SlotPlan P = slot_plan(items[i].n, k);
            if (P.passes == k) last += P.hi[k] - P.lo[k];
        }
        if (last >= kSlotMinFinal) return k;
    }
    return 2;
}

// In-place decode of up to kMaxBatch payloads, each at the head of its own
// output buffer (a slot): the resident form, or the multi-pass form (pass 1
// copies to the stash what later passes read after the slot head has been
// overwritten and decodes the tiles past the payload, later passes decode
// the rest).
int launch_decode_slot(const splitzip_slot_item *items, uint32_t count, int32_t *status, bool resident,
                       hipStream_t s) {
    constexpr uint64_t kTile = (uint64_t)kDecUnits * kDecThreads * kUnit;
    DecArgs a{};
    a.count = count;
    a.status = status;
    uint64_t tiles = 0, n_all = 0;
    for (uint32_t k = 0; k < count; ++k) {
        const splitzip_slot_item &I = items[k];
        a.it[k] = DecItem{I.slot, I.slot_bytes, I.meta, I.dec_lut,
                          reinterpret_cast<uint16_t *>(I.slot), I.n, I.stash, I.stash_bytes};
        a.tile_start[k] = tiles;
        tiles += ceil_div(I.n, kTile);
        n_all += I.n;
    }
    a.tile_start[count] = tiles;
    if (tiles == 0) return SPLITZIP_OK;
    // The resident form (k_decode_slot_hold, then k_decode_slot_defer for
    // what it left) in an ordinary launch, or the multi-pass form
    // (k_decode_slot_stage, then k_decode_slot_level once per later pass).
    // The environment variable SPLITZIP_SLOT_LAUNCH selects a form for every
    // call: "one" (resident), "coop" (resident, the first kernel launched
    // cooperatively) or "two" (multi-pass);
    // SPLITZIP_SLOT_WAIT_US sets the resident form's bounded barrier wait
    // (default kHoldWaitUs; 0 makes nearly every barrier give up, which
    // exercises the path taken when the grid is not resident).
    const char *form = getenv("SPLITZIP_SLOT_LAUNCH");
    const bool want_two = form && strcmp(form, "two") == 0;
    const bool want_one = form && strcmp(form, "one") == 0;
    const bool want_coop = form && strcmp(form, "coop") == 0;
    const bool one_kernel = want_one || want_coop || (resident && !want_two);
    uint32_t grid = 0;
    bool coop_ok = false;
    if (one_kernel && !coop_grid(grid, coop_ok)) return SPLITZIP_ERR_HIP;
    const bool coop = grid && coop_ok && want_coop;
    int cus = 0;
    if (!cu_count(cus)) return SPLITZIP_ERR_HIP;
    if (!order_counters(a, count)) return SPLITZIP_ERR_HIP;
    if (grid) {
        if (!coop_block(a, s)) return SPLITZIP_ERR_HIP;
        const char *w = getenv("SPLITZIP_SLOT_WAIT_US");
        const uint64_t us = w ? strtoull(w, nullptr, 10) : kHoldWaitUs;
        a.wait_ticks = (uint32_t)(us < 40000000ull ? us * 100 : 4000000000ull);
        if (coop) {
            void *args[] = {&a};
            if (hipLaunchCooperativeKernel(reinterpret_cast<const void *>(k_decode_slot_hold), dim3(grid),
                                           dim3(kDecThreads), args, 0, s) != hipSuccess)
                return SPLITZIP_ERR_HIP;
        } else {
            k_decode_slot_hold<<<grid, kDecThreads, 0, s>>>(a);
        }
        if (hipGetLastError() != hipSuccess) return SPLITZIP_ERR_HIP;
        k_decode_slot_defer<<<(unsigned)(cus < (int)kCoopMaxGrid ? cus : (int)kCoopMaxGrid), kDecThreads,
                              0, s>>>(a);
        if (hipGetLastError() != hipSuccess) return SPLITZIP_ERR_HIP;
    }
    SlotPlan plan[kMaxBatch];
    uint32_t most = 2;
    if (!grid) {
        const uint32_t passes = slot_passes(items, count);
        for (uint32_t k = 0; k < count; ++k) {
            plan[k] = slot_plan(items[k].n, passes);
            const SlotPlan &P = plan[k];
            a.pass[k] = SlotPass{(uint32_t)P.t_min, (uint32_t)P.lo[P.passes], (uint32_t)P.hi[P.passes],
                                 0, 0, 0, 0};
            if (P.passes > most) most = P.passes;
        }
        k_decode_slot_stage<<<(unsigned)tiles, kDecThreads, 0, s>>>(a);
        if (hipGetLastError() != hipSuccess) return SPLITZIP_ERR_HIP;
    }
    for (uint32_t k = 0; k < count; ++k) {
        a.it[k].payload = items[k].stash;
        a.it[k].payload_bytes = items[k].stash_bytes;
        a.it[k].stash = nullptr;
        a.it[k].other_bytes = items[k].slot_bytes;
    }
    for (uint32_t p = 2; !grid && p <= most; ++p) {
        // pass p: per tensor the tiles [lo[p], lo[p+1]) and [hi[p+1], hi[p]),
        // or in its last pass [lo[p], hi[p])
        uint64_t wgs = 0;
        for (uint32_t k = 0; k < count; ++k) {
            const SlotPlan &P = plan[k];
            SlotPass Q{(uint32_t)P.t_min, 0, 0, 0, 0, 0, 0};
            if (items[k].n && p < P.passes) {
                Q.a0 = (uint32_t)P.lo[p];
                Q.a1 = (uint32_t)P.lo[p + 1];
                Q.b0 = (uint32_t)P.hi[p + 1];
                Q.b1 = (uint32_t)P.hi[p];
            } else if (items[k].n && p == P.passes) {
                Q.a0 = (uint32_t)P.lo[p];
                Q.a1 = (uint32_t)P.hi[p];
                Q.last = 1;
                // one workgroup per tile from t_min on whose output may
                // overlap the payload: it fits both the slot and the stash
                const uint64_t room = items[k].slot_bytes < items[k].stash_bytes
                                          ? items[k].slot_bytes : items[k].stash_bytes;
                uint64_t reach = ceil_div(room, 2 * kTile);
                const uint64_t tiles_k = ceil_div(items[k].n, kTile);
                if (reach > tiles_k) reach = tiles_k;
                Q.extra = (uint32_t)(reach > P.t_min ? reach - P.t_min : 0);
            }
            a.pass[k] = Q;
            a.tile_start[k] = wgs;
            wgs += (uint64_t)(Q.a1 - Q.a0) + (Q.b1 - Q.b0) + Q.extra;
        }
        a.tile_start[count] = wgs;
        if (wgs == 0) continue;
        k_decode_slot_level<<<(unsigned)wgs, kDecThreads, 0, s>>>(a);
        if (hipGetLastError() != hipSuccess) return SPLITZIP_ERR_HIP;
    }
    if (status) {
        uint64_t cgrid = ceil_div(n_all, 16 * kThreads);
        if (cgrid > 1024) cgrid = 1024;
        k_decode_check<true><<<(unsigned)cgrid, kThreads, 0, s>>>(a);
    }
    return launched();
}

int check_slot_item(const splitzip_slot_item &I) {
    if (I.n > SPLITZIP_MAX_N || !I.meta || !aligned(I.meta, 8) || !I.dec_lut)
        return SPLITZIP_ERR_INVALID;
    if (I.n == 0) return SPLITZIP_OK;
    const uint64_t dense = layout_of(I.n, 0).total;
    const uint64_t need = dense > 2 * I.n ? dense : 2 * I.n;
    if (!I.slot || !aligned(I.slot, 16) || I.slot_bytes < need || !I.stash ||
        !aligned(I.stash, 16) || I.stash_bytes < dense)
        return SPLITZIP_ERR_INVALID;
    const uintptr_t a0 = (uintptr_t)I.slot, b0 = (uintptr_t)I.stash;
    if (a0 < b0 + I.stash_bytes && b0 < a0 + I.slot_bytes) return SPLITZIP_ERR_INVALID;
    return SPLITZIP_OK;
}

}  // namespace

extern "C" {

int splitzip_abi_version(void) { return SPLITZIP_ABI_VERSION; }

void splitzip_struct_sizes(size_t *codebook_bytes, size_t *meta_bytes) {
    if (codebook_bytes) *codebook_bytes = sizeof(splitzip_codebook);
    if (meta_bytes) *meta_bytes = sizeof(splitzip_meta);
}

const char *splitzip_status_string(int status) {
    switch (status) {
        case SPLITZIP_OK: return "ok";
        case SPLITZIP_ERR_INVALID: return "invalid argument";
        case SPLITZIP_ERR_CAPACITY: return "payload buffer too small";
        case SPLITZIP_ERR_CORRUPT: return "corrupt payload or metadata";
        case SPLITZIP_ERR_HIP: return "HIP runtime error";
        case SPLITZIP_ERR_WORKSPACE: return "workspace too small";
        case SPLITZIP_ERR_INTERNAL: return "internal error";
        default: return "unknown status";
    }
}

uint64_t splitzip_payload_size(uint64_t n, uint64_t n_esc) { return layout_of(n, n_esc).total; }

uint32_t splitzip_slot_schedule(uint64_t n, uint32_t passes, uint64_t *t_min, uint64_t *lo,
                                uint64_t *hi) {
    if (n > SPLITZIP_MAX_N || passes < 2 || passes > kSlotMaxPasses || !t_min || !lo || !hi) return 0;
    const SlotPlan P = slot_plan(n, passes);
    *t_min = P.t_min;
    for (uint32_t k = 0; k <= passes; ++k) {
        lo[k] = k >= 2 && k <= P.passes ? P.lo[k] : 0;
        hi[k] = k >= 2 && k <= P.passes ? P.hi[k] : 0;
    }
    return P.passes;
}

size_t splitzip_workspace_size(uint64_t n) {
    uint64_t t = enc_tiles(n);
    if (t == 0) t = 1;
    // smallest size whose plan holds t tiles
    return (size_t)(kWsFixed + t * kWsPerTile);
}

size_t splitzip_workspace_size_batch(const uint64_t *n, uint32_t count) {
    // tiles of the largest launch: consecutive groups of kMaxBatch tensors
    uint64_t most = 0;
    for (uint32_t k0 = 0; n && k0 < count; k0 += kMaxBatch) {
        uint64_t t = 0;
        for (uint32_t k = k0; k < count && k < k0 + kMaxBatch; ++k) t += enc_tiles(n[k]);
        if (t > most) most = t;
    }
    if (most == 0) most = 1;
    return (size_t)(kWsFixed + most * kWsPerTile);
}

int splitzip_workspace_init(void *d_ws, size_t ws_bytes, void *stream) {
    if (!d_ws || !aligned(d_ws, 16) || ws_bytes < splitzip_workspace_size(0))
        return SPLITZIP_ERR_INVALID;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    k_fill_zero<<<256, 256, 0, s>>>(reinterpret_cast<uint32_t *>(d_ws), kWsTiles / 4);
    return launched();
}

int splitzip_calibrate(const uint16_t *d_x, uint64_t n, splitzip_codebook *d_cb, void *d_ws,
                       size_t ws_bytes, void *stream) {
    if (check_calibrate_item(d_x, n, d_cb) || !d_ws || !aligned(d_ws, 16))
        return SPLITZIP_ERR_INVALID;
    if (ws_bytes < splitzip_workspace_size(0)) return SPLITZIP_ERR_WORKSPACE;
    const CalItem it{d_x, n, d_cb};
    return launch_calibrate(&it, 1, reinterpret_cast<uint8_t *>(d_ws),
                            reinterpret_cast<hipStream_t>(stream));
}

int splitzip_encode_chunked(const uint16_t *d_x, uint64_t n, const splitzip_codebook *d_cb,
                            uint32_t chunk_size, uint8_t *d_payload, uint64_t capacity,
                            splitzip_meta *d_meta, void *d_ws, size_t ws_bytes, void *stream) {
    const int rc = check_encode_item(d_x, n, d_cb, d_payload, capacity, d_meta);
    if (rc) return rc;
    if (!d_ws || !aligned(d_ws, 16) || !chunk_ok(n, chunk_size)) return SPLITZIP_ERR_INVALID;
    const WsPlan P = ws_plan(ws_bytes);
    if (ws_bytes < splitzip_workspace_size(n) || P.t_max < enc_tiles(n))
        return SPLITZIP_ERR_WORKSPACE;
    const EncItem it{d_x, n, d_cb, d_payload, capacity, d_meta, chunk_size};
    return launch_encode(&it, 1, P, reinterpret_cast<uint8_t *>(d_ws),
                         reinterpret_cast<hipStream_t>(stream));
}

int splitzip_encode(const uint16_t *d_x, uint64_t n, const splitzip_codebook *d_cb,
                    uint8_t *d_payload, uint64_t capacity, splitzip_meta *d_meta, void *d_ws,
                    size_t ws_bytes, void *stream) {
    return splitzip_encode_chunked(d_x, n, d_cb, kChunk, d_payload, capacity, d_meta, d_ws,
                                   ws_bytes, stream);
}

int splitzip_encode_noalloc(const uint16_t *d_x, uint64_t n, const splitzip_codebook *d_cb,
                            uint8_t *d_payload, uint64_t capacity, splitzip_meta *d_meta,
                            void *stream) {
    const int rc = check_encode_item(d_x, n, d_cb, d_payload, capacity, d_meta);
    if (rc) return rc;
    if (enc_tiles(n) > kScratchPlan.t_max) return SPLITZIP_ERR_WORKSPACE;   // n > SPLITZIP_NOALLOC_MAX_N
    uint8_t *ws = nullptr;
    if (!scratch_of_device(ws)) return SPLITZIP_ERR_HIP;
    const EncItem it{d_x, n, d_cb, d_payload, capacity, d_meta, kChunk};
    return launch_encode(&it, 1, kScratchPlan, ws, reinterpret_cast<hipStream_t>(stream));
}

int splitzip_decode(const uint8_t *d_payload, uint64_t payload_bytes, const splitzip_meta *d_meta,
                    const uint8_t *d_dec_lut, uint16_t *d_out, uint64_t n, int32_t *d_status,
                    void *stream) {
    if (check_decode_item(d_payload, payload_bytes, d_meta, d_dec_lut, d_out, n) ||
        (d_status && !aligned(d_status, 4)))
        return SPLITZIP_ERR_INVALID;
    if (n == 0) return SPLITZIP_OK;
    const DecItem it{d_payload, payload_bytes, d_meta, d_dec_lut, d_out, n, nullptr, 0};
    return launch_decode(&it, 1, d_status, reinterpret_cast<hipStream_t>(stream));
}

int splitzip_decode_slot(uint8_t *d_slot, uint64_t slot_bytes, const splitzip_meta *d_meta,
                         const uint8_t *d_dec_lut, uint64_t n, uint8_t *d_stash,
                         uint64_t stash_bytes, int32_t *d_status, void *stream) {
    const splitzip_slot_item it{d_slot, slot_bytes, d_meta, d_dec_lut, n, d_stash, stash_bytes};
    return splitzip_decode_slot_batch(&it, 1, d_status, stream);
}

static int decode_slot_batch(const splitzip_slot_item *items, uint32_t count, int32_t *d_status,
                             bool resident, void *stream) {
    if ((count && !items) || (d_status && !aligned(d_status, 4))) return SPLITZIP_ERR_INVALID;
    for (uint32_t k = 0; k < count; ++k)
        if (check_slot_item(items[k])) return SPLITZIP_ERR_INVALID;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (uint32_t k0 = 0; k0 < count; k0 += kMaxBatch) {
        const uint32_t m = count - k0 < (uint32_t)kMaxBatch ? count - k0 : (uint32_t)kMaxBatch;
        const int rc = launch_decode_slot(items + k0, m, d_status, resident, s);
        if (rc) return rc;
    }
    return SPLITZIP_OK;
}

int splitzip_decode_slot_batch(const splitzip_slot_item *items, uint32_t count, int32_t *d_status,
                               void *stream) {
    return decode_slot_batch(items, count, d_status, false, stream);
}

int splitzip_decode_slot_batch_resident(const splitzip_slot_item *items, uint32_t count,
                                        int32_t *d_status, void *stream) {
    return decode_slot_batch(items, count, d_status, true, stream);
}

int splitzip_calibrate_batch(const splitzip_item *items, uint32_t count, void *d_ws,
                             size_t ws_bytes, void *stream) {
    if ((count && !items) || !d_ws || !aligned(d_ws, 16)) return SPLITZIP_ERR_INVALID;
    for (uint32_t k = 0; k < count; ++k)
        if (check_calibrate_item(items[k].x, items[k].n, items[k].cb)) return SPLITZIP_ERR_INVALID;
    if (ws_bytes < splitzip_workspace_size(0)) return SPLITZIP_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    CalItem chunk[kMaxBatch];
    for (uint32_t k0 = 0; k0 < count; k0 += kMaxBatch) {
        const uint32_t m = count - k0 < (uint32_t)kMaxBatch ? count - k0 : (uint32_t)kMaxBatch;
        for (uint32_t k = 0; k < m; ++k)
            chunk[k] = CalItem{items[k0 + k].x, items[k0 + k].n, items[k0 + k].cb};
        const int rc = launch_calibrate(chunk, m, reinterpret_cast<uint8_t *>(d_ws), s);
        if (rc) return rc;
    }
    return SPLITZIP_OK;
}

int splitzip_encode_batch(const splitzip_item *items, uint32_t count, void *d_ws,
                          size_t ws_bytes, void *stream) {
    if ((count && !items) || !d_ws || !aligned(d_ws, 16)) return SPLITZIP_ERR_INVALID;
    for (uint32_t k = 0; k < count; ++k) {
        const splitzip_item &I = items[k];
        const int rc = check_encode_item(I.x, I.n, I.cb, I.payload, I.capacity, I.meta);
        if (rc) return rc;
    }
    const WsPlan P = ws_plan(ws_bytes);
    for (uint32_t k0 = 0; k0 < count; k0 += kMaxBatch) {
        uint64_t tiles = 0;
        for (uint32_t k = k0; k < count && k < k0 + kMaxBatch; ++k) tiles += enc_tiles(items[k].n);
        if (tiles > P.t_max) return SPLITZIP_ERR_WORKSPACE;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    EncItem chunk[kMaxBatch];
    for (uint32_t k0 = 0; k0 < count; k0 += kMaxBatch) {
        const uint32_t m = count - k0 < (uint32_t)kMaxBatch ? count - k0 : (uint32_t)kMaxBatch;
        for (uint32_t k = 0; k < m; ++k) {
            const splitzip_item &I = items[k0 + k];
            chunk[k] = EncItem{I.x, I.n, I.cb, I.payload, I.capacity, I.meta, kChunk};
        }
        const int rc = launch_encode(chunk, m, P, reinterpret_cast<uint8_t *>(d_ws), s);
        if (rc) return rc;
    }
    return SPLITZIP_OK;
}

int splitzip_decode_batch(const splitzip_item *items, uint32_t count, int32_t *d_status,
                          void *stream) {
    if ((count && !items) || (d_status && !aligned(d_status, 4))) return SPLITZIP_ERR_INVALID;
    for (uint32_t k = 0; k < count; ++k) {
        const splitzip_item &I = items[k];
        if (!I.cb || check_decode_item(I.payload, I.capacity, I.meta, dec_lut_of(I.cb), I.out, I.n))
            return SPLITZIP_ERR_INVALID;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    DecItem chunk[kMaxBatch];
    for (uint32_t k0 = 0; k0 < count; k0 += kMaxBatch) {
        const uint32_t m = count - k0 < (uint32_t)kMaxBatch ? count - k0 : (uint32_t)kMaxBatch;
        for (uint32_t k = 0; k < m; ++k) {
            const splitzip_item &I = items[k0 + k];
            chunk[k] = DecItem{I.payload, I.capacity, I.meta, dec_lut_of(I.cb), I.out, I.n, nullptr, 0};
        }
        const int rc = launch_decode(chunk, m, d_status, s);
        if (rc) return rc;
    }
    return SPLITZIP_OK;
}

}  // extern "C"
