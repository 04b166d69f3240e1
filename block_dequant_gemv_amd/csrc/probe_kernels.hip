// probe_kernels.hip -- measurement kernels of libqgemv (diagnostics, not part
// of any GEMV): a plain streaming read, the ceiling that the GEMVs' weight
// streams are held against, and an empty kernel, the floor of any dispatch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dequant.h"
#include "qgemv_kernels.h"

namespace qgk {

// Streaming read of `bytes` (a multiple of 1 KiB) with 16-byte nontemporal
// loads: wavefront v reads the 8 KiB chunk [8 KiB v, 8 KiB (v + 1)) as 8
// one-KiB load instructions (64 lanes x 16 bytes each), all issued before any
// is used, the way the GEMV kernels stream a unit; loads past the end are not
// issued. The words read are XOR-ed and stored only if they happen to equal a
// value given by the caller, so the loads cannot be removed and nothing is
// written in practice.
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4 *__restrict__ buf, uint64_t n16,
                                                          uint32_t *__restrict__ sink, uint32_t magic)
{
    const uint64_t wave = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t base = wave * 512u + lane;   // 16-byte units: 8 loads of 64
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint64_t u = base + 64u * i;
        v[i] = u < n16 ? __builtin_nontemporal_load(buf + u) : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    if (acc == magic) sink[0] = acc;
}

__global__ void empty_kernel() {}

hipError_t launch_probe_stream(const void *buf, uint64_t bytes, uint32_t *sink, uint32_t magic, hipStream_t s)
{
    const uint64_t n16 = bytes / 16;
    const uint64_t waves = (n16 + 511) / 512;
    const uint64_t grid = (waves + 3) / 4;   // 4 wavefronts per workgroup
    launch_timed(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0u, s, (const u32x4 *)buf, n16, sink, magic);
    return hipGetLastError();
}

hipError_t launch_probe_empty(hipStream_t s)
{
    launch_timed(empty_kernel, dim3(1), dim3(64), 0u, s);
    return hipGetLastError();
}

}  // namespace qgk
