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
    const uint64_t base = (uint64_t)blockIdx.x * kTile;
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
    const uint64_t base = (uint64_t)blockIdx.x * kTile;
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
