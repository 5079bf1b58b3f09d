// Reference memory streams: the access patterns of the codec kernels with the
// coding replaced by XORs, so that their rates are the ceilings the codec
// kernels are measured against.  Interface and conventions in
// include/splitzip_ceiling.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "splitzip.h"
#include "splitzip_ceiling.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef u32x2 u32x2_a4 __attribute__((aligned(4)));

constexpr int kReadThreads = 1024;   // calibrate's workgroup
constexpr int kReadInFlight = 4;     // 16-byte loads in flight per thread
constexpr int kThreads = 256;        // encode / decode workgroup
constexpr int kUnit = 8;             // elements per thread and unit
constexpr int kUnits = 4;            // units per thread and tile
constexpr uint64_t kTile = (uint64_t)kThreads * kUnit * kUnits;
constexpr uint32_t kSinkMagic = 0x9E3779B9u;

// The codec's map from workgroups to tiles (one tile per workgroup): in a
// launch of at least 32,768 tiles each XCD (workgroup b runs on XCD b % 8)
// takes 64 consecutive tiles in turn, the last G mod 512 workgroups keeping
// the plain order; smaller launches take the plain order.
__device__ inline uint64_t launch_tile(uint64_t b, uint64_t G) {
    constexpr uint64_t kRun = 64, B = 8 * kRun;
    if (G < 32768 || b >= G / B * B) return b;
    const uint64_t x = b % 8, j = b / 8;
    return (j / kRun) * B + x * kRun + j % kRun;
}

__global__ __launch_bounds__(kReadThreads) void k_read_shape(const u32x4 *x, uint64_t nvec,
                                                             uint32_t *sink) {
    const uint64_t per = (nvec + gridDim.x - 1) / gridDim.x;
    const uint64_t lo = (uint64_t)blockIdx.x * per;
    const uint64_t hi = lo + per < nvec ? lo + per : nvec;
    constexpr uint64_t stride = kReadThreads;
    uint32_t acc = 0;
    uint64_t v = lo + threadIdx.x;
    for (; v + (kReadInFlight - 1) * stride < hi; v += kReadInFlight * stride) {
        u32x4 q[kReadInFlight];
#pragma unroll
        for (int k = 0; k < kReadInFlight; ++k) q[k] = __builtin_nontemporal_load(x + v + k * stride);
#pragma unroll
        for (int k = 0; k < kReadInFlight; ++k) acc ^= q[k].x ^ q[k].y ^ q[k].z ^ q[k].w;
    }
    for (; v < hi; v += stride) {
        const u32x4 q = __builtin_nontemporal_load(x + v);
        acc ^= q.x ^ q.y ^ q.z ^ q.w;
    }
    if (acc == kSinkMagic) sink[0] = acc;
}

__global__ __launch_bounds__(kThreads) void k_encode_shape(const uint16_t *x, uint8_t *pk,
                                                           uint8_t *sm) {
    const uint64_t base = launch_tile(blockIdx.x, gridDim.x) * kTile;
    const int tid = threadIdx.x;
    u32x4 q[kUnits];
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
        const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
        q[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x + i0));
    }
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
        const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
        const uint32_t p = q[u].x ^ q[u].y ^ q[u].z ^ q[u].w;
        const u32x2 s = {q[u].x ^ q[u].z, q[u].y ^ q[u].w};
        __builtin_nontemporal_store(p, reinterpret_cast<uint32_t *>(pk + i0 / 2));
        __builtin_nontemporal_store(s, reinterpret_cast<u32x2_a4 *>(sm + i0));
    }
}

__global__ __launch_bounds__(kThreads) void k_decode_shape(const uint8_t *pk, const uint8_t *sm,
                                                           uint16_t *out) {
    const uint64_t base = launch_tile(blockIdx.x, gridDim.x) * kTile;
    const int tid = threadIdx.x;
    uint32_t p[kUnits];
    u32x2 s[kUnits];
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
        const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
        p[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(pk + i0 / 2));
        s[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2_a4 *>(sm + i0));
    }
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
        const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
        const u32x4 o = {p[u] ^ s[u].x, p[u] ^ s[u].y, s[u].x ^ 0x5A5A5A5Au, s[u].y ^ 0xA5A5A5A5u};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(out + i0));
    }
}

// ---- probes behind the design's choices (see include/splitzip_ceiling.h) ----

// The encode pattern with thread-contiguous 32-element units.
__global__ __launch_bounds__(kThreads) void k_encode_wide(const uint16_t *x, uint8_t *pk, uint8_t *sm) {
    const uint64_t i0 = launch_tile(blockIdx.x, gridDim.x) * kTile + (uint64_t)threadIdx.x * 32;
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x + i0);
    u32x4 q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = __builtin_nontemporal_load(xv + k);
    const u32x4 p = {q[0].x ^ q[0].y, q[1].x ^ q[1].y, q[2].x ^ q[2].y, q[3].x ^ q[3].y};
    const u32x4 s0 = {q[0].x ^ q[0].z, q[0].y ^ q[0].w, q[1].x ^ q[1].z, q[1].y ^ q[1].w};
    const u32x4 s1 = {q[2].x ^ q[2].z, q[2].y ^ q[2].w, q[3].x ^ q[3].z, q[3].y ^ q[3].w};
    __builtin_nontemporal_store(p, reinterpret_cast<u32x4 *>(pk + i0 / 2));
    __builtin_nontemporal_store(s0, reinterpret_cast<u32x4 *>(sm + i0));
    __builtin_nontemporal_store(s1, reinterpret_cast<u32x4 *>(sm + i0 + 16));
}

// The decode pattern with thread-contiguous 32-element units.
__global__ __launch_bounds__(kThreads) void k_decode_wide(const uint8_t *pk, const uint8_t *sm,
                                                          uint16_t *out) {
    const uint64_t i0 = launch_tile(blockIdx.x, gridDim.x) * kTile + (uint64_t)threadIdx.x * 32;
    const u32x4 p = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(pk + i0 / 2));
    const u32x4 s0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(sm + i0));
    const u32x4 s1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(sm + i0 + 16));
    u32x4 *o = reinterpret_cast<u32x4 *>(out + i0);
    __builtin_nontemporal_store(u32x4{p.x ^ s0.x, p.y ^ s0.y, p.z ^ s0.z, p.w ^ s0.w}, o);
    __builtin_nontemporal_store(u32x4{p.x ^ s1.x, p.y ^ s1.y, p.z ^ s1.z, p.w ^ s1.w}, o + 1);
    __builtin_nontemporal_store(u32x4{s0.x, s0.y ^ p.x, s1.z, s1.w ^ p.y}, o + 2);
    __builtin_nontemporal_store(u32x4{s1.x ^ p.z, s0.z, s0.w ^ p.w, s1.y}, o + 3);
}

__device__ inline uint64_t ld_agent(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Replaces a counter whose high half is not `epoch` by (epoch << 32).
__device__ inline void claim(uint64_t *c, uint32_t epoch) {
    uint64_t cur = ld_agent(c);
    for (int k = 0; k < 64 && (uint32_t)(cur >> 32) != epoch; ++k)
        if (__hip_atomic_compare_exchange_strong(c, &cur, (uint64_t)epoch << 32, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            break;
}

// The encode pattern, then a fused arrival as a placement in the same kernel
// would need it: the tile's count is stored, the workgroup waits for its
// stores to complete (s_waitcnt) and arrives on a two-level counter (groups
// of 16 workgroups, each counter on its own 64-byte line, tagged with the
// call's epoch); the last arrival writes the epoch to *ready.
__global__ __launch_bounds__(kThreads) void k_encode_arrive(const uint16_t *x, uint8_t *pk, uint8_t *sm,
                                                            uint32_t *counts, uint64_t *ctrs,
                                                            uint32_t *ready, uint32_t epoch) {
    constexpr uint32_t kGroup = 16;
    const uint32_t t = blockIdx.x, tiles = gridDim.x;
    const uint32_t ngroups = (tiles + kGroup - 1) / kGroup, g = t / kGroup;
    uint64_t *top = ctrs, *grp = ctrs + 8 * (1 + g);
    const uint64_t dt = launch_tile(t, tiles);   // the tile this workgroup codes
    const uint64_t base = dt * kTile;
    const int tid = threadIdx.x;
    u32x4 q[kUnits];
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
        const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
        q[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x + i0));
    }
    if (tid == 0) {
        claim(grp, epoch);
        if (t % kGroup == 0) claim(top, epoch);
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
        const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
        const uint32_t p = q[u].x ^ q[u].y ^ q[u].z ^ q[u].w;
        const u32x2 s = {q[u].x ^ q[u].z, q[u].y ^ q[u].w};
        acc ^= p;
        __builtin_nontemporal_store(p, reinterpret_cast<uint32_t *>(pk + i0 / 2));
        __builtin_nontemporal_store(s, reinterpret_cast<u32x2_a4 *>(sm + i0));
    }
    if (tid == 0) __hip_atomic_store(counts + dt, acc & 0xFFu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t gsize = g * kGroup + kGroup <= tiles ? kGroup : tiles - g * kGroup;
        const uint64_t prev = __hip_atomic_fetch_add(grp, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)prev + 1u == gsize) {
            const uint64_t p2 = __hip_atomic_fetch_add(top, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((uint32_t)p2 + 1u == ngroups)
                __hip_atomic_store(ready, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// The encode / decode patterns with `run` consecutive tiles per XCD in turn
// (0: the plain order, every launch size; the last G mod 8*run workgroups
// keep it too).
__device__ inline uint64_t run_tile(uint64_t b, uint64_t G, uint32_t run) {
    if (run == 0) return b;
    const uint64_t B = 8ull * run;
    if (b >= G / B * B) return b;
    const uint64_t x = b % 8, j = b / 8;
    return (j / run) * B + x * run + j % run;
}

__global__ __launch_bounds__(kThreads) void k_encode_order(const uint16_t *x, uint8_t *pk, uint8_t *sm,
                                                           uint32_t run) {
    const uint64_t base = run_tile(blockIdx.x, gridDim.x, run) * kTile;
    const int tid = threadIdx.x;
    u32x4 q[kUnits];
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
        const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
        q[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x + i0));
    }
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
        const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
        const uint32_t p = q[u].x ^ q[u].y ^ q[u].z ^ q[u].w;
        const u32x2 s = {q[u].x ^ q[u].z, q[u].y ^ q[u].w};
        __builtin_nontemporal_store(p, reinterpret_cast<uint32_t *>(pk + i0 / 2));
        __builtin_nontemporal_store(s, reinterpret_cast<u32x2_a4 *>(sm + i0));
    }
}

__global__ __launch_bounds__(kThreads) void k_decode_order(const uint8_t *pk, const uint8_t *sm,
                                                           uint16_t *out, uint32_t run) {
    const uint64_t base = run_tile(blockIdx.x, gridDim.x, run) * kTile;
    const int tid = threadIdx.x;
    uint32_t p[kUnits];
    u32x2 s[kUnits];
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
        const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
        p[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(pk + i0 / 2));
        s[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2_a4 *>(sm + i0));
    }
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
        const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
        const u32x4 o = {p[u] ^ s[u].x, p[u] ^ s[u].y, s[u].x ^ 0x5A5A5A5Au, s[u].y ^ 0xA5A5A5A5u};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(out + i0));
    }
}

// The encode pattern with an agent-scope fence (__threadfence: write-back of
// the L2 and invalidation) at the end of every workgroup.
__global__ __launch_bounds__(kThreads) void k_encode_fenced(const uint16_t *x, uint8_t *pk, uint8_t *sm) {
    const uint64_t base = launch_tile(blockIdx.x, gridDim.x) * kTile;
    const int tid = threadIdx.x;
    u32x4 q[kUnits];
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
        const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
        q[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x + i0));
    }
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
        const uint64_t i0 = base + (uint64_t)u * (kThreads * kUnit) + tid * kUnit;
        const uint32_t p = q[u].x ^ q[u].y ^ q[u].z ^ q[u].w;
        const u32x2 s = {q[u].x ^ q[u].z, q[u].y ^ q[u].w};
        __builtin_nontemporal_store(p, reinterpret_cast<uint32_t *>(pk + i0 / 2));
        __builtin_nontemporal_store(s, reinterpret_cast<u32x2_a4 *>(sm + i0));
    }
    __threadfence();
}

// Device-scope atomic adds: lane 0 of every 64-thread workgroup adds 1 to
// ctrs[(blockIdx % spread) * 8] `rounds` times, each add waiting for the
// previous one's result.
__global__ __launch_bounds__(64) void k_atomics(uint64_t *ctrs, uint32_t spread, uint32_t rounds) {
    if (threadIdx.x) return;
    uint64_t *c = ctrs + (uint64_t)(blockIdx.x % spread) * 8;
    uint64_t v = 0;
    for (uint32_t r = 0; r < rounds; ++r)   // (v >> 63 is 0, but makes each add wait for the last)
        v += __hip_atomic_fetch_add(c, 1ull + (v >> 63), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v == 0x9E3779B97F4A7C15ull) ctrs[1] = v;
}

// An almost empty kernel, for launch costs.
__global__ __launch_bounds__(64) void k_touch(uint32_t *sink) {
    if (threadIdx.x == 0 && blockIdx.x == 0) sink[0] += 1u;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int launched() { return hipGetLastError() == hipSuccess ? SPLITZIP_OK : SPLITZIP_ERR_HIP; }

// tile counts fit a one-dimensional grid
bool tiles_ok(uint64_t n) { return n && n % kTile == 0 && n / kTile <= 0x7FFFFFFFu; }

}  // namespace

extern "C" int splitzip_ceiling_read(const void *d_x, uint64_t bytes, uint32_t grid,
                                     uint32_t *d_sink, hipStream_t stream) {
    if (!d_x || !aligned16(d_x) || bytes == 0 || bytes % 16 || !d_sink ||
        ((uintptr_t)d_sink & 3u))
        return SPLITZIP_ERR_INVALID;
    if (grid == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return SPLITZIP_ERR_HIP;
        grid = 2u * (uint32_t)(cus > 0 ? cus : 1);
    }
    k_read_shape<<<grid, kReadThreads, 0, stream>>>(static_cast<const u32x4 *>(d_x), bytes / 16,
                                                   d_sink);
    return launched();
}

extern "C" int splitzip_ceiling_encode_shape(const uint16_t *d_x, uint64_t n, uint8_t *d_pk,
                                             uint8_t *d_sm, hipStream_t stream) {
    if (!tiles_ok(n) || !d_x || !d_pk || !d_sm || !aligned16(d_x) || !aligned16(d_pk) ||
        !aligned16(d_sm))
        return SPLITZIP_ERR_INVALID;
    k_encode_shape<<<(uint32_t)(n / kTile), kThreads, 0, stream>>>(d_x, d_pk, d_sm);
    return launched();
}

extern "C" int splitzip_ceiling_decode_shape(const uint8_t *d_pk, const uint8_t *d_sm,
                                             uint16_t *d_out, uint64_t n, hipStream_t stream) {
    if (!tiles_ok(n) || !d_pk || !d_sm || !d_out || !aligned16(d_pk) || !aligned16(d_sm) ||
        !aligned16(d_out))
        return SPLITZIP_ERR_INVALID;
    k_decode_shape<<<(uint32_t)(n / kTile), kThreads, 0, stream>>>(d_pk, d_sm, d_out);
    return launched();
}

extern "C" int splitzip_ceiling_order(uint32_t decode, uint32_t run, const uint16_t *d_x,
                                      uint8_t *d_pk, uint8_t *d_sm, uint16_t *d_out, uint64_t n,
                                      hipStream_t stream) {
    if (!tiles_ok(n) || !d_pk || !d_sm || !aligned16(d_pk) || !aligned16(d_sm) ||
        (run & (run - 1)) || run > 65536 || decode > 1)
        return SPLITZIP_ERR_INVALID;
    if (decode ? (!d_out || !aligned16(d_out)) : (!d_x || !aligned16(d_x))) return SPLITZIP_ERR_INVALID;
    if (decode)
        k_decode_order<<<(uint32_t)(n / kTile), kThreads, 0, stream>>>(d_pk, d_sm, d_out, run);
    else
        k_encode_order<<<(uint32_t)(n / kTile), kThreads, 0, stream>>>(d_x, d_pk, d_sm, run);
    return launched();
}

extern "C" int splitzip_ceiling_encode_wide(const uint16_t *d_x, uint64_t n, uint8_t *d_pk,
                                            uint8_t *d_sm, hipStream_t stream) {
    if (!tiles_ok(n) || !d_x || !d_pk || !d_sm || !aligned16(d_x) || !aligned16(d_pk) ||
        !aligned16(d_sm))
        return SPLITZIP_ERR_INVALID;
    k_encode_wide<<<(uint32_t)(n / kTile), kThreads, 0, stream>>>(d_x, d_pk, d_sm);
    return launched();
}

extern "C" int splitzip_ceiling_decode_wide(const uint8_t *d_pk, const uint8_t *d_sm,
                                            uint16_t *d_out, uint64_t n, hipStream_t stream) {
    if (!tiles_ok(n) || !d_pk || !d_sm || !d_out || !aligned16(d_pk) || !aligned16(d_sm) ||
        !aligned16(d_out))
        return SPLITZIP_ERR_INVALID;
    k_decode_wide<<<(uint32_t)(n / kTile), kThreads, 0, stream>>>(d_pk, d_sm, d_out);
    return launched();
}

extern "C" int splitzip_ceiling_encode_arrive(const uint16_t *d_x, uint64_t n, uint8_t *d_pk,
                                              uint8_t *d_sm, uint32_t *d_counts, uint64_t *d_ctrs,
                                              uint32_t *d_ready, uint32_t epoch, hipStream_t stream) {
    if (!tiles_ok(n) || !d_x || !d_pk || !d_sm || !d_counts || !d_ctrs || !d_ready ||
        !aligned16(d_x) || !aligned16(d_pk) || !aligned16(d_sm) || !aligned16(d_counts) ||
        !aligned16(d_ctrs) || !aligned16(d_ready) || epoch == 0)
        return SPLITZIP_ERR_INVALID;
    k_encode_arrive<<<(uint32_t)(n / kTile), kThreads, 0, stream>>>(d_x, d_pk, d_sm, d_counts, d_ctrs,
                                                                  d_ready, epoch);
    return launched();
}

extern "C" int splitzip_ceiling_encode_fenced(const uint16_t *d_x, uint64_t n, uint8_t *d_pk,
                                              uint8_t *d_sm, hipStream_t stream) {
    if (!tiles_ok(n) || !d_x || !d_pk || !d_sm || !aligned16(d_x) || !aligned16(d_pk) ||
        !aligned16(d_sm))
        return SPLITZIP_ERR_INVALID;
    k_encode_fenced<<<(uint32_t)(n / kTile), kThreads, 0, stream>>>(d_x, d_pk, d_sm);
    return launched();
}

extern "C" int splitzip_ceiling_atomics(uint64_t *d_ctrs, uint32_t grid, uint32_t spread,
                                        uint32_t rounds, hipStream_t stream) {
    if (!d_ctrs || !aligned16(d_ctrs) || grid == 0 || spread == 0 || spread > 4096 || rounds == 0 ||
        rounds > (1u << 20))
        return SPLITZIP_ERR_INVALID;
    k_atomics<<<grid, 64, 0, stream>>>(d_ctrs, spread, rounds);
    return launched();
}

extern "C" int splitzip_ceiling_launch(uint32_t cooperative, uint32_t grid, uint32_t *d_sink,
                                       hipStream_t stream) {
    if (!d_sink || ((uintptr_t)d_sink & 3u) || grid == 0 || grid > 1024) return SPLITZIP_ERR_INVALID;
    if (cooperative) {
        void *args[] = {&d_sink};
        if (hipLaunchCooperativeKernel(reinterpret_cast<const void *>(k_touch), dim3(grid), dim3(64),
                                       args, 0, stream) != hipSuccess)
            return SPLITZIP_ERR_HIP;
        return SPLITZIP_OK;
    }
    k_touch<<<grid, 64, 0, stream>>>(d_sink);
    return launched();
}
