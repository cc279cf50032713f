// attn_tools.hip -- measurement aids of the library (not part of the attention
// path): a plain streaming read, the reference against which the decode
// kernel's HBM rate is compared.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_device.h"
#include "attn_kernels.h"

namespace tpa {

// Each workgroup reads its `per_wg` bytes of [buf, buf + bytes) once, with the
// 16-byte non-temporal buffer loads the decode kernel streams K and V with,
// UNROLL loads in flight per lane. The words read are folded together and
// stored only if they equal a value no input produces in practice, so the
// loads cannot be dropped and almost nothing is written.
template <int UNROLL>
__global__ void __launch_bounds__(256) stream_read_kernel(const char* buf, uint64_t bytes, uint64_t per_wg,
                                                          uint32_t* sink) {
    const uint64_t base = (uint64_t)blockIdx.x * per_wg;
    if (base >= bytes) return;
    const uint64_t left = bytes - base;
    const uint32_t n = (uint32_t)(left < per_wg ? left : per_wg);
    const rsrc_t r = make_rsrc_u(buf + base, n);
    uint32_t acc = 0;
    for (uint32_t off = threadIdx.x * 16u; off < n; off += 256u * 16u * UNROLL) {
        u32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = buf_load16_nt(r, off + (uint32_t)u * 256u * 16u);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= (v[u][0] ^ v[u][1]) ^ (v[u][2] ^ v[u][3]);
    }
    if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, int workgroups, void* sink, hipStream_t stream) {
    const uint64_t per = ((uint64_t)bytes + workgroups - 1) / workgroups;
    const uint64_t per16 = (per + 15) / 16 * 16;
    hipLaunchKernelGGL((stream_read_kernel<16>), dim3(workgroups), dim3(256), 0, stream,
                       static_cast<const char*>(buf), (uint64_t)bytes, per16, static_cast<uint32_t*>(sink));
    return hipGetLastError();
}

}  // namespace tpa
