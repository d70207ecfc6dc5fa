// HBM bandwidth probes for the benchmark's ceiling measurement: the plainest
// streaming read and streaming copy this hardware runs, with the same access
// shape the library's kernels use (16-byte buffer loads, whole contiguous
// kilobytes per wave instruction, non-temporal cache policy, several loads
// in flight per lane).  Not part of the method; kept in a source of its own.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/svla.h"

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;                 // 16-byte loads in flight per lane

__device__ __forceinline__ __amdgpu_buffer_rsrc_t probe_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Each workgroup streams its own contiguous range of `per_wg` bytes (a
// multiple of 16 KiB); the read probe folds the words into one value per lane
// so the loads cannot be dropped, and writes it to sink[blockIdx.x] only when it
// equals a value the data never holds (never, in practice).
__global__ void __launch_bounds__(kProbeThreads)
svla_probe_read(const void *src, uint32_t per_wg, unsigned int *sink)
{
    const auto r = probe_rsrc((const char *)src + (size_t)blockIdx.x * per_wg, per_wg);
    unsigned int acc = 0u;
    for (uint32_t off = threadIdx.x * 16u; off < per_wg; off += kProbeThreads * 16u * kProbeUnroll) {
        u32x4_t v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + u * kProbeThreads * 16u), 0, 2);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

__global__ void __launch_bounds__(kProbeThreads)
svla_probe_copy(const void *src, void *dst, uint32_t per_wg)
{
    const auto rs = probe_rsrc((const char *)src + (size_t)blockIdx.x * per_wg, per_wg);
    const auto rd = probe_rsrc((char *)dst + (size_t)blockIdx.x * per_wg, per_wg);
    for (uint32_t off = threadIdx.x * 16u; off < per_wg; off += kProbeThreads * 16u * kProbeUnroll) {
        u32x4_t v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off + u * kProbeThreads * 16u), 0, 2);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, (int)(off + u * kProbeThreads * 16u), 0, 2);
    }
}

}  // namespace

extern "C" svla_status svla_hbm_probe(int mode, const void *src, void *dst, size_t bytes,
                                      unsigned int *sink, int workgroups, svla_stream stream)
{
    const size_t chunk = (size_t)kProbeThreads * 16u * kProbeUnroll;   // 16 KiB
    if ((mode != 0 && mode != 1) || workgroups <= 0) return SVLA_ERR_VALUE;
    if (!src || (mode == 1 && !dst) || (mode == 0 && !sink)) return SVLA_ERR_NULL;
    if (bytes % ((size_t)workgroups * chunk) != 0) return SVLA_ERR_SHAPE;
    const size_t per_wg = bytes / (size_t)workgroups;
    if (per_wg >= ((size_t)1 << 31)) return SVLA_ERR_SHAPE;
    if (((uintptr_t)src | (uintptr_t)dst) & 15) return SVLA_ERR_ALIGN;
    (void)hipGetLastError();
    hipStream_t s = (hipStream_t)stream;
    if (mode == 0) svla_probe_read<<<workgroups, kProbeThreads, 0, s>>>(src, (uint32_t)per_wg, sink);
    else svla_probe_copy<<<workgroups, kProbeThreads, 0, s>>>(src, dst, (uint32_t)per_wg);
    return hipGetLastError() == hipSuccess ? SVLA_OK : SVLA_ERR_HIP;
}
