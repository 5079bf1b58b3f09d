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
// Kernels (all integer work, HBM-bandwidth bound, no matrix cores):
//   k_calibrate      exponent histogram in LDS (one private copy per lane of
//                    a wave, so equal exponents never collide on a bank), one
//                    device atomic per non-empty bin per workgroup, and a
//                    top-16 select by the last workgroup to finish.
//   k_encode         persistent tile loop: 16-byte loads, LDS code table,
//                    nibble packing, sign+mantissa bytes, wave ballots to
//                    rank escapes, decoupled look-back across tiles (tickets
//                    handed out in start order, so every awaited tile is
//                    running or done) giving each escape its global rank in
//                    ascending element order.
//   k_encode_tail    moves the staged positions / raw exponents behind the
//                    chunk ids once the escape count is known, writes the
//                    metadata and leaves the workspace clean for the next call.
//   k_decode_dense   pk + sm -> bf16 through a 256-entry pair table in LDS.
//   k_decode_patch   one lane per escape: rebuild the element from its raw
//                    exponent and its own sign/mantissa byte.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "splitzip.h"

namespace {

constexpr uint32_t kChunk = SPLITZIP_CHUNK;
constexpr int kThreads = 256;                 // encode / decode workgroup
constexpr int kUnit = 8;                      // elements per 16-byte load
constexpr int kEncUnits = 2;                  // units per thread per tile
constexpr int kEncTile = kThreads * kUnit * kEncUnits;   // 4096 elements
constexpr int kDecUnits = 4;
constexpr int kDecTile = kThreads * kUnit * kDecUnits;   // 8192 elements
constexpr int kCalThreads = 1024;

// Workspace layout (bytes).  The tile-status region and the staging areas
// depend only on the workspace size, so one workspace serves any n that fits.
constexpr size_t kWsTicket = 0;      // uint32 encode tile ticket
constexpr size_t kWsCalDone = 4;     // uint32 calibrate workgroups finished
constexpr size_t kWsGuard = 8;       // uint32 progress guard tripped
constexpr size_t kWsTotalEsc = 16;   // uint64 escape count of the last encode
constexpr size_t kWsHist = 256;      // uint64[256] global histogram
constexpr size_t kWsStatus = 256 + 2048;  // uint64[t_max] look-back words
constexpr size_t kWsSlack = 64;

constexpr uint64_t kFlagAgg = 1ull << 62;
constexpr uint64_t kFlagPrefix = 2ull << 62;
constexpr uint64_t kValueMask = (1ull << 62) - 1;
constexpr uint32_t kSpinLimit = 1u << 20;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef u32x2 u32x2_a4 __attribute__((aligned(4)));

__host__ __device__ inline uint64_t align4(uint64_t v) { return (v + 3u) & ~uint64_t(3); }
__host__ __device__ inline uint64_t align16(uint64_t v) { return (v + 15u) & ~uint64_t(15); }

struct Layout {
    uint64_t n_pairs, off_sm, off_cid, off_lpos, off_ev, total;
};

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

// Staging areas and look-back capacity of a workspace of ws_bytes.
struct WsPlan {
    uint64_t t_max;       // tiles the status region holds
    uint64_t off_lpos;    // uint16[t_max * kEncTile]
    uint64_t off_ev;      // uint8[t_max * kEncTile]
};

__host__ inline WsPlan ws_plan(size_t ws_bytes) {
    WsPlan P{0, 0, 0};
    if (ws_bytes < kWsStatus + kWsSlack) return P;
    P.t_max = (ws_bytes - kWsStatus - kWsSlack) / (8 + 3 * (uint64_t)kEncTile);
    P.off_lpos = align16(kWsStatus + 8 * P.t_max);
    P.off_ev = align16(P.off_lpos + 2 * P.t_max * kEncTile);
    return P;
}

__device__ inline uint64_t ld_agent(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_agent(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Page 1, docstring "Method": the exponent is bits 7..14 of the 16-bit view;
// the stored byte keeps bit 15 (sign) as its bit 7 and the 7 low mantissa bits.
__device__ inline uint32_t exp_lo(uint32_t w) { return (w >> 7) & 0xFFu; }
__device__ inline uint32_t exp_hi(uint32_t w) { return (w >> 23) & 0xFFu; }
__device__ inline uint32_t sm_of16(uint32_t b) { return ((b >> 8) & 0x80u) | (b & 0x7Fu); }
// Reconstruction: sign back to bit 15, exponent to bits 7..14.
__device__ inline uint32_t join16(uint32_t sm, uint32_t ex) {
    return ((sm & 0x80u) << 8) | (ex << 7) | (sm & 0x7Fu);
}

// ---------------------------------------------------------------------------
// Calibrate (page 1, calibrate_codebook)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kCalThreads) void k_calibrate(const uint16_t *__restrict__ x,
                                                           uint64_t n,
                                                           splitzip_codebook *__restrict__ cb,
                                                           uint8_t *__restrict__ ws) {
    __shared__ uint32_t hist[256 * 64];   // [exponent][lane]
    __shared__ uint32_t part[4 * 256];
    __shared__ uint64_t cnt[256];
    __shared__ uint64_t covered;
    __shared__ uint32_t is_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    for (int i = tid; i < 256 * 64; i += kCalThreads) hist[i] = 0;
    __syncthreads();

    uint32_t *hl = hist + lane;
    const uint64_t nvec = n >> 3;
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x);
    const uint64_t stride = (uint64_t)gridDim.x * kCalThreads;
    uint64_t v = (uint64_t)blockIdx.x * kCalThreads + tid;
    for (; v + 3 * stride < nvec; v += 4 * stride) {
        u32x4 q[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) q[k] = __builtin_nontemporal_load(xv + v + k * stride);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                atomicAdd(hl + exp_lo(q[k][w]) * 64, 1u);
                atomicAdd(hl + exp_hi(q[k][w]) * 64, 1u);
            }
        }
    }
    for (; v < nvec; v += stride) {
        u32x4 q = __builtin_nontemporal_load(xv + v);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            atomicAdd(hl + exp_lo(q[w]) * 64, 1u);
            atomicAdd(hl + exp_hi(q[w]) * 64, 1u);
        }
    }
    if (blockIdx.x == 0 && (uint64_t)tid < (n & 7)) {
        uint32_t b = x[(nvec << 3) + tid];
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
    if (tid < 256) {
        uint32_t s = part[tid] + part[256 + tid] + part[512 + tid] + part[768 + tid];
        if (s) atomicAdd(reinterpret_cast<unsigned long long *>(ws + kWsHist) + tid,
                         (unsigned long long)s);
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        uint32_t prev = __hip_atomic_fetch_add(reinterpret_cast<uint32_t *>(ws + kWsCalDone), 1u,
                                               __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        is_last = (prev == gridDim.x - 1) ? 1u : 0u;
        covered = 0;
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();

    // Last workgroup: every histogram atomic of this call is visible.  Rank of
    // exponent v = number of exponents with a larger count, or an equal count
    // and a smaller value; ranks 0..15 of occurring exponents become codes.
    uint64_t *ghist = reinterpret_cast<uint64_t *>(ws + kWsHist);
    if (tid < 256) cnt[tid] = ld_agent(ghist + tid);
    __syncthreads();
    uint32_t code = 16;
    uint64_t c = 0;
    if (tid < 256) {
        c = cnt[tid];
        uint32_t rank = 0;
        for (int u = 0; u < 256; ++u) {
            uint64_t cu = cnt[u];
            rank += (cu > c || (cu == c && u < tid)) ? 1u : 0u;
        }
        code = (c > 0 && rank < 16) ? rank : 16u;
        cb->enc_lut[tid] = (uint8_t)(code < 16 ? code : 0);
        cb->enc_lut_marked[tid] = (uint8_t)code;
        cb->common_lut[tid] = (uint8_t)(code < 16 ? 1 : 0);
        cb->counts[tid] = c;
        if (code < 16) {
            cb->dec_lut[code] = (uint8_t)tid;
            atomicAdd(reinterpret_cast<unsigned long long *>(&covered), (unsigned long long)c);
        }
        st_agent(ghist + tid, 0);   // leave the histogram clean for the next call
    }
    const int distinct = __syncthreads_count(tid < 256 && c > 0);
    const uint32_t n_codes = distinct < 16 ? (uint32_t)distinct : 16u;
    if (tid < 16 && (uint32_t)tid >= n_codes) cb->dec_lut[tid] = 0;
    if (tid == 0) {
        cb->n_codes = n_codes;
        cb->reserved = 0;
        cb->covered = covered;
        cb->total = n;
        *reinterpret_cast<uint32_t *>(ws + kWsCalDone) = 0;
    }
}

// ---------------------------------------------------------------------------
// Encode (page 1, encode_torch + assemble_payload)
// ---------------------------------------------------------------------------

struct EncArgs {
    const uint16_t *x;
    uint64_t n;
    uint64_t ntiles;
    const splitzip_codebook *cb;
    uint8_t *payload;
    uint64_t capacity;
    uint64_t n_pairs, off_sm, off_cid;
    uint8_t *ws;
    uint16_t *stage_lpos;
    uint8_t *stage_ev;
};

// Word k of a 4-word vector without dynamic register indexing.
__device__ inline uint32_t word_of(const u32x4 q, int k) {
    return k == 0 ? q.x : (k == 1 ? q.y : (k == 2 ? q.z : q.w));
}

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
        // marked code: 0..15, or 16 for an escape, whose nibble is 16 & 15 = 0
        const uint32_t byte = ((m_even & 15u) << 4) | (m_odd & 15u);
        pk |= byte << (8 * k);
        flags |= ((m_even >> 4) | ((m_odd >> 4) << 1)) << (2 * k);
    }
    sm0 = sm_of16(q[0]) | (sm_of16(q[0] >> 16) << 8) | (sm_of16(q[1]) << 16) |
          (sm_of16(q[1] >> 16) << 24);
    sm1 = sm_of16(q[2]) | (sm_of16(q[2] >> 16) << 8) | (sm_of16(q[3]) << 16) |
          (sm_of16(q[3] >> 16) << 24);
}

__global__ __launch_bounds__(kThreads) void k_encode(EncArgs a) {
    __shared__ uint8_t lut[256];
    __shared__ uint32_t wtot[kEncUnits][4];
    __shared__ uint32_t tile_slot[2];
    __shared__ uint64_t excl_slot;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    uint32_t *ticket = reinterpret_cast<uint32_t *>(a.ws + kWsTicket);
    uint64_t *status = reinterpret_cast<uint64_t *>(a.ws + kWsStatus);

    lut[tid] = a.cb->enc_lut_marked[tid];
    if (tid == 0) tile_slot[0] = atomicAdd(ticket, 1u);
    __syncthreads();

    uint32_t it = 0;
    uint64_t t = tile_slot[0];
    while (t < a.ntiles) {
        if (tid == 0) tile_slot[(it + 1) & 1] = atomicAdd(ticket, 1u);
        const uint64_t base = t * kEncTile;
        const bool full = base + kEncTile <= a.n;

        u32x4 q[kEncUnits];
        uint32_t flags[kEncUnits];
        if (full) {
#pragma unroll
            for (int u = 0; u < kEncUnits; ++u) {
                const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
                q[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.x + i0));
            }
#pragma unroll
            for (int u = 0; u < kEncUnits; ++u) {
                const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
                uint32_t pk, sm0, sm1;
                encode_unit(q[u], lut, pk, sm0, sm1, flags[u]);
                *reinterpret_cast<uint32_t *>(a.payload + i0 / 2) = pk;
                u32x2 smv = {sm0, sm1};
                *reinterpret_cast<u32x2_a4 *>(a.payload + a.off_sm + i0) = smv;
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
                    if (i < a.n) {
                        b = a.x[i];
                        const uint32_t m = lut[exp_lo(b)];
                        codes[j] = m & 15u;
                        f |= (m >> 4) << j;
                        a.payload[a.off_sm + i] = (uint8_t)sm_of16(b);
                    }
                    wv[j >> 1] |= b << (16 * (j & 1));
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint64_t i = i0 + 2 * k;
                    if (i < a.n) {
                        const uint32_t lo = (i + 1 < a.n) ? codes[2 * k + 1] : 0u;
                        a.payload[i / 2] = (uint8_t)((codes[2 * k] << 4) | lo);
                    }
                }
                q[u] = u32x4{wv[0], wv[1], wv[2], wv[3]};
                flags[u] = f;
            }
        }
        if (t == a.ntiles - 1 && tid == 0) {
            // zero padding between the dense sections (page 1: the payload is
            // assembled in a zero-filled buffer)
            for (uint64_t b = a.n_pairs; b < a.off_sm; ++b) a.payload[b] = 0;
            for (uint64_t b = a.off_sm + a.n; b < a.off_cid; ++b) a.payload[b] = 0;
        }

        // Escape ranks inside the tile, in element order (unit, thread, j).
        uint32_t pre[kEncUnits];
#pragma unroll
        for (int u = 0; u < kEncUnits; ++u) {
            const uint32_t c = __builtin_popcount(flags[u]);
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

        uint32_t tile_total = 0;
        uint32_t ubase[kEncUnits];
#pragma unroll
        for (int u = 0; u < kEncUnits; ++u) {
            ubase[u] = tile_total;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                ubase[u] += (w < wave) ? wtot[u][w] : 0u;
                tile_total += wtot[u][w];
            }
        }

        // Decoupled look-back (wave 0): publish this tile's count, then add
        // the counts of earlier tiles until one with a published prefix.
        if (wave == 0) {
            uint64_t excl = 0;
            if (t == 0) {
                if (lane == 0) st_agent(status, kFlagPrefix | tile_total);
            } else {
                if (lane == 0) st_agent(status + t, kFlagAgg | tile_total);
                int64_t j = (int64_t)t - 1;
                uint32_t spins = 0;
                while (true) {
                    const int64_t idx = j - lane;
                    const uint64_t v = idx >= 0 ? ld_agent(status + idx) : kFlagPrefix;
                    const uint32_t flag = (uint32_t)(v >> 62);
                    const uint64_t pm = __ballot(flag == 2);
                    const uint64_t im = __ballot(flag == 0);
                    const int fp = pm ? (__ffsll((unsigned long long)pm) - 1) : 64;
                    const uint64_t before = fp == 64 ? ~0ull : ((1ull << fp) - 1);
                    if (im & before) {
                        if (++spins > kSpinLimit) {
                            if (lane == 0)
                                atomicOr(reinterpret_cast<uint32_t *>(a.ws + kWsGuard), 1u);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                        continue;
                    }
                    excl += wave_sum_u64(lane <= fp ? (v & kValueMask) : 0);
                    if (fp < 64) break;
                    j -= 64;
                }
                if (lane == 0) st_agent(status + t, kFlagPrefix | (excl + tile_total));
            }
            if (lane == 0) {
                excl_slot = excl;
                if (t == a.ntiles - 1)
                    st_agent(reinterpret_cast<uint64_t *>(a.ws + kWsTotalEsc), excl + tile_total);
            }
        }
        __syncthreads();

        if (tile_total) {
            const uint64_t excl = excl_slot;
#pragma unroll
            for (int u = 0; u < kEncUnits; ++u) {
                uint32_t f = flags[u];
                uint64_t r = excl + ubase[u] + pre[u];
                const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
                while (f) {
                    const int j = __builtin_ctz(f);
                    f &= f - 1;
                    const uint64_t i = i0 + j;
                    const uint32_t w = word_of(q[u], j >> 1);
                    const uint32_t ex = (j & 1) ? exp_hi(w) : exp_lo(w);
                    const uint64_t at = a.off_cid + 4 * r;
                    if (at + 4 <= a.capacity)
                        *reinterpret_cast<uint32_t *>(a.payload + at) = (uint32_t)(i / kChunk);
                    a.stage_lpos[r] = (uint16_t)(i % kChunk);
                    a.stage_ev[r] = (uint8_t)ex;
                    ++r;
                }
            }
        }
        ++it;
        t = tile_slot[it & 1];
    }
}

struct TailArgs {
    uint64_t n;
    uint64_t ntiles;
    const splitzip_codebook *cb;
    uint8_t *payload;
    uint64_t capacity;
    splitzip_meta *meta;
    uint8_t *ws;
    const uint16_t *stage_lpos;
    const uint8_t *stage_ev;
};

__global__ __launch_bounds__(kThreads) void k_encode_tail(TailArgs a) {
    const uint64_t e =
        a.ntiles ? ld_agent(reinterpret_cast<const uint64_t *>(a.ws + kWsTotalEsc)) : 0;
    const Layout L = layout_of(a.n, e);
    const bool fits = L.total <= a.capacity;
    const uint64_t g = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    const uint64_t gs = (uint64_t)gridDim.x * kThreads;
    if (fits && e) {
        // local_pos: e uint16 from the staging area to off_lpos (4-aligned)
        uint32_t *lp_dst = reinterpret_cast<uint32_t *>(a.payload + L.off_lpos);
        const uint32_t *lp_src = reinterpret_cast<const uint32_t *>(a.stage_lpos);
        for (uint64_t k = g; k < e / 2; k += gs) lp_dst[k] = lp_src[k];
        uint32_t *ev_dst = reinterpret_cast<uint32_t *>(a.payload + L.off_ev);
        const uint32_t *ev_src = reinterpret_cast<const uint32_t *>(a.stage_ev);
        for (uint64_t k = g; k < e / 4; k += gs) ev_dst[k] = ev_src[k];
        if (g == 0) {
            if (e & 1) {
                *reinterpret_cast<uint16_t *>(a.payload + L.off_lpos + 2 * (e - 1)) =
                    a.stage_lpos[e - 1];
                a.payload[L.off_lpos + 2 * e] = 0;       // alignment padding
                a.payload[L.off_lpos + 2 * e + 1] = 0;
            }
            for (uint64_t k = e & ~uint64_t(3); k < e; ++k) a.payload[L.off_ev + k] = a.stage_ev[k];
        }
    }
    // leave the look-back words clear for the next call
    uint64_t *status = reinterpret_cast<uint64_t *>(a.ws + kWsStatus);
    for (uint64_t k = g; k < a.ntiles; k += gs) status[k] = 0;
    if (g == 0) {
        uint32_t *guard = reinterpret_cast<uint32_t *>(a.ws + kWsGuard);
        splitzip_meta *m = a.meta;
        m->n = a.n;
        m->n_pairs = L.n_pairs;
        m->chunk_size = kChunk;
        m->n_esc = e;
        m->comp_bytes = L.total;
        m->offsets[0] = 0;
        m->offsets[1] = L.off_sm;
        m->offsets[2] = L.off_cid;
        m->offsets[3] = L.off_lpos;
        m->offsets[4] = L.off_ev;
        m->covered = a.cb->covered;
        m->total = a.cb->total;
        m->status = *guard ? SPLITZIP_ERR_INTERNAL : (fits ? SPLITZIP_OK : SPLITZIP_ERR_CAPACITY);
        m->reserved = 0;
        *guard = 0;
        *reinterpret_cast<uint32_t *>(a.ws + kWsTicket) = 0;
        *reinterpret_cast<uint64_t *>(a.ws + kWsTotalEsc) = 0;
    }
}

// ---------------------------------------------------------------------------
// Decode (page 1, decode_torch)
// ---------------------------------------------------------------------------

struct DecArgs {
    const uint8_t *payload;
    uint64_t payload_bytes;
    const splitzip_meta *meta;
    const uint8_t *dec_lut;
    uint16_t *out;
    uint64_t n;
    int32_t *status;
};

// Metadata must describe exactly the layout of (n, n_esc) and fit the buffer.
__device__ inline bool meta_ok(const DecArgs &a, Layout &L) {
    const splitzip_meta *m = a.meta;
    if (m->n != a.n || m->chunk_size != kChunk || m->n_esc > a.n) return false;
    L = layout_of(a.n, m->n_esc);
    return m->n_pairs == L.n_pairs && m->offsets[0] == 0 && m->offsets[1] == L.off_sm &&
           m->offsets[2] == L.off_cid && m->offsets[3] == L.off_lpos &&
           m->offsets[4] == L.off_ev && m->comp_bytes == L.total && L.total <= a.payload_bytes;
}

__global__ __launch_bounds__(kThreads) void k_decode_dense(DecArgs a) {
    __shared__ uint32_t pair_lut[256];   // pk byte -> (even exponent, odd exponent)
    Layout L;
    if (!meta_ok(a, L)) {
        if (blockIdx.x == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
        return;
    }
    const int tid = threadIdx.x;
    pair_lut[tid] = (uint32_t)a.dec_lut[tid >> 4] | ((uint32_t)a.dec_lut[tid & 15] << 16);
    __syncthreads();

    const uint64_t base = (uint64_t)blockIdx.x * kDecTile;
    const uint8_t *pk = a.payload;
    const uint8_t *sm = a.payload + L.off_sm;
    if (base + kDecTile <= a.n) {
        uint32_t pkw[kDecUnits];
        u32x2 smw[kDecUnits];
#pragma unroll
        for (int u = 0; u < kDecUnits; ++u) {
            const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
            pkw[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(pk + i0 / 2));
            smw[u] = *reinterpret_cast<const u32x2_a4 *>(sm + i0);
        }
#pragma unroll
        for (int u = 0; u < kDecUnits; ++u) {
            const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t ee = pair_lut[(pkw[u] >> (8 * k)) & 0xFFu];
                const uint32_t s = smw[u][k >> 1] >> (16 * (k & 1));
                o[k] = join16(s & 0xFFu, ee & 0xFFu) | (join16((s >> 8) & 0xFFu, ee >> 16) << 16);
            }
            __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(a.out + i0));
        }
    } else {
        for (uint64_t i = base + tid; i < a.n && i < base + kDecTile; i += kThreads) {
            const uint32_t byte = pk[i / 2];
            const uint32_t code = (i & 1) ? (byte & 15u) : (byte >> 4);
            a.out[i] = (uint16_t)join16(sm[i], a.dec_lut[code]);
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_decode_patch(DecArgs a) {
    Layout L;
    if (!meta_ok(a, L)) return;   // reported by k_decode_dense
    const uint64_t e = a.meta->n_esc;
    const uint8_t *sm = a.payload + L.off_sm;
    const uint8_t *cid_b = a.payload + L.off_cid;
    const uint16_t *lpos = reinterpret_cast<const uint16_t *>(a.payload + L.off_lpos);
    const uint8_t *ev = a.payload + L.off_ev;
    const uint64_t gs = (uint64_t)gridDim.x * kThreads;
    int32_t bad = 0;
    for (uint64_t r = (uint64_t)blockIdx.x * kThreads + threadIdx.x; r < e; r += gs) {
        const int32_t cid = *reinterpret_cast<const int32_t *>(cid_b + 4 * r);
        const uint32_t pos = lpos[r];
        if (cid < 0) { bad |= 2; continue; }
        if (pos >= kChunk) bad |= 4;
        const uint64_t idx = (uint64_t)cid * kChunk + pos;
        if (idx >= a.n) { bad |= 2; continue; }
        if (r > 0) {
            const int32_t pc = *reinterpret_cast<const int32_t *>(cid_b + 4 * (r - 1));
            const uint64_t prev = (uint64_t)(uint32_t)pc * kChunk + lpos[r - 1];
            if (pc < 0 || prev >= idx) bad |= 8;
        }
        a.out[idx] = (uint16_t)join16(sm[idx], ev[r]);
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

constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];
int g_enc_blocks_per_cu[kMaxDevices];

bool device_info(int &cus, int &enc_occ) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
    if (g_cu_count[dev] == 0) {
        int c = 0, occ = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return false;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_encode, kThreads, 0) !=
            hipSuccess)
            return false;
        g_enc_blocks_per_cu[dev] = occ > 0 ? occ : 1;
        g_cu_count[dev] = c > 0 ? c : 1;
    }
    cus = g_cu_count[dev];
    enc_occ = g_enc_blocks_per_cu[dev];
    return true;
}

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline uint64_t enc_tiles(uint64_t n) { return (n + kEncTile - 1) / kEncTile; }

int launched() {
    return hipGetLastError() == hipSuccess ? SPLITZIP_OK : SPLITZIP_ERR_HIP;
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
        case SPLITZIP_ERR_INTERNAL: return "device progress guard tripped";
        default: return "unknown status";
    }
}

uint64_t splitzip_payload_size(uint64_t n, uint64_t n_esc) { return layout_of(n, n_esc).total; }

size_t splitzip_workspace_size(uint64_t n) {
    uint64_t t = enc_tiles(n);
    if (t == 0) t = 1;
    // smallest size whose plan holds t tiles
    return (size_t)(kWsStatus + kWsSlack + t * (8 + 3 * (uint64_t)kEncTile));
}

int splitzip_workspace_init(void *d_ws, size_t ws_bytes, void *stream) {
    if (!d_ws || !aligned(d_ws, 16) || ws_bytes < splitzip_workspace_size(0))
        return SPLITZIP_ERR_INVALID;
    const WsPlan P = ws_plan(ws_bytes);
    const uint64_t words = (kWsStatus + 8 * P.t_max) / 4;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    k_fill_zero<<<256, 256, 0, s>>>(reinterpret_cast<uint32_t *>(d_ws), words);
    return launched();
}

int splitzip_calibrate(const uint16_t *d_x, uint64_t n, splitzip_codebook *d_cb, void *d_ws,
                       size_t ws_bytes, void *stream) {
    if (n > SPLITZIP_MAX_N || (n && (!d_x || !aligned(d_x, 16))) || !d_cb || !aligned(d_cb, 8) ||
        !d_ws || !aligned(d_ws, 16))
        return SPLITZIP_ERR_INVALID;
    if (ws_bytes < splitzip_workspace_size(0)) return SPLITZIP_ERR_WORKSPACE;
    int cus = 0, occ = 0;
    if (!device_info(cus, occ)) return SPLITZIP_ERR_HIP;
    const uint64_t nvec = n >> 3;
    uint64_t grid = (nvec + 4 * kCalThreads - 1) / (4 * kCalThreads);
    const uint64_t cap = 2 * (uint64_t)cus;
    if (grid > cap) grid = cap;
    if (grid == 0) grid = 1;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    k_calibrate<<<(unsigned)grid, kCalThreads, 0, s>>>(d_x, n, d_cb,
                                                      reinterpret_cast<uint8_t *>(d_ws));
    return launched();
}

int splitzip_encode(const uint16_t *d_x, uint64_t n, const splitzip_codebook *d_cb,
                    uint8_t *d_payload, uint64_t capacity, splitzip_meta *d_meta, void *d_ws,
                    size_t ws_bytes, void *stream) {
    if (n > SPLITZIP_MAX_N || (n && (!d_x || !aligned(d_x, 16))) || !d_cb || !aligned(d_cb, 8) ||
        !d_meta || !aligned(d_meta, 8) || !d_ws || !aligned(d_ws, 16) ||
        (!d_payload && capacity) || !aligned(d_payload, 16))
        return SPLITZIP_ERR_INVALID;
    const Layout L0 = layout_of(n, 0);
    if (capacity < L0.total) return SPLITZIP_ERR_CAPACITY;
    const uint64_t ntiles = enc_tiles(n);
    const WsPlan P = ws_plan(ws_bytes);
    if (ws_bytes < splitzip_workspace_size(n) || P.t_max < ntiles) return SPLITZIP_ERR_WORKSPACE;
    int cus = 0, occ = 0;
    if (!device_info(cus, occ)) return SPLITZIP_ERR_HIP;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint8_t *ws = reinterpret_cast<uint8_t *>(d_ws);
    uint16_t *stage_lpos = reinterpret_cast<uint16_t *>(ws + P.off_lpos);
    uint8_t *stage_ev = ws + P.off_ev;
    if (ntiles) {
        EncArgs a{d_x,      n,        ntiles,    d_cb, d_payload, capacity, L0.n_pairs,
                  L0.off_sm, L0.off_cid, ws,      stage_lpos, stage_ev};
        uint64_t grid = (uint64_t)cus * occ;
        if (grid > ntiles) grid = ntiles;
        k_encode<<<(unsigned)grid, kThreads, 0, s>>>(a);
        if (hipGetLastError() != hipSuccess) return SPLITZIP_ERR_HIP;
    }
    TailArgs t{n, ntiles, d_cb, d_payload, capacity, d_meta, ws, stage_lpos, stage_ev};
    uint64_t tgrid = (ntiles + 7) / 8;
    if (tgrid > 512) tgrid = 512;
    if (tgrid == 0) tgrid = 1;
    k_encode_tail<<<(unsigned)tgrid, kThreads, 0, s>>>(t);
    return launched();
}

int splitzip_decode(const uint8_t *d_payload, uint64_t payload_bytes, const splitzip_meta *d_meta,
                    const uint8_t *d_dec_lut, uint16_t *d_out, uint64_t n, int32_t *d_status,
                    void *stream) {
    if (n > SPLITZIP_MAX_N || !d_meta || !aligned(d_meta, 8) || !d_dec_lut ||
        (n && (!d_payload || !aligned(d_payload, 16) || !d_out || !aligned(d_out, 16))) ||
        (d_status && !aligned(d_status, 4)))
        return SPLITZIP_ERR_INVALID;
    if (n == 0) return SPLITZIP_OK;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    DecArgs a{d_payload, payload_bytes, d_meta, d_dec_lut, d_out, n, d_status};
    const uint64_t grid = (n + kDecTile - 1) / kDecTile;
    k_decode_dense<<<(unsigned)grid, kThreads, 0, s>>>(a);
    if (hipGetLastError() != hipSuccess) return SPLITZIP_ERR_HIP;
    uint64_t pgrid = (n + 16 * kThreads - 1) / (16 * kThreads);
    if (pgrid > 1024) pgrid = 1024;
    k_decode_patch<<<(unsigned)pgrid, kThreads, 0, s>>>(a);
    return launched();
}

}  // extern "C"
