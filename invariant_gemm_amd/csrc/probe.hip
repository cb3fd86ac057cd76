// probe.hip -- measurement kernels behind the diagnostic entry points
// bi_probe_stream_read and bi_probe_empty: the measured HBM read roof and the
// launch floor the GEMM kernels are compared with.  They compute no GEMM.
#include "common.h"
#include "launch.h"

namespace bigemm {
namespace {

// Workgroup b streams the contiguous byte range [b*per, (b+1)*per) of buf
// (the last one up to `bytes`), each thread loading 16-byte chunks U at a
// time at a stride of the workgroup size; the loaded words are folded by XOR
// into one word per thread so the loads cannot be removed, and that word is
// written to out only in the (never taken) case that it equals `key`, so the
// probe writes nothing in practice yet its result stays observable.
template <int U, bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t* __restrict__ buf, uint64_t bytes,
                                                          uint64_t per, uint32_t key,
                                                          uint32_t* __restrict__ out)
{
    const uint64_t lo = (uint64_t)blockIdx.x * per;
    const uint64_t hi = lo + per < bytes ? lo + per : bytes;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (lo < hi) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(buf + lo, clamp_bytes((int64_t)(hi - lo)));
        const uint32_t n = (uint32_t)(hi - lo);
        for (uint32_t off = threadIdx.x * 16u; off < n; off += 256u * 16u * U) {
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = NT ? buf_load16_nt(r, off + (uint32_t)u * 256u * 16u)
                          : buf_load16(r, off + (uint32_t)u * 256u * 16u);
#pragma unroll
            for (int u = 0; u < U; ++u)
                x ^= v[u];
        }
    }
    const uint32_t w = x[0] ^ x[1] ^ x[2] ^ x[3];
    if (w == key)
        out[(uint64_t)blockIdx.x * blockDim.x + threadIdx.x] = w;
}

__global__ void empty_kernel() {}

}  // namespace

hipError_t launch_probe_stream_read(const uint8_t* buf, uint64_t bytes, int workgroups, int unroll,
                                    bool nt, uint32_t* out, hipStream_t stream)
{
    const uint64_t per = ((bytes + workgroups - 1) / workgroups + 4095) & ~(uint64_t)4095;
    const dim3 grid((unsigned)workgroups), block(256);
    const uint32_t key = 0x9E3779B9u;
    if (unroll == 4) {
        if (nt)
            stream_read_kernel<4, true><<<grid, block, 0, stream>>>(buf, bytes, per, key, out);
        else
            stream_read_kernel<4, false><<<grid, block, 0, stream>>>(buf, bytes, per, key, out);
    } else {
        if (nt)
            stream_read_kernel<8, true><<<grid, block, 0, stream>>>(buf, bytes, per, key, out);
        else
            stream_read_kernel<8, false><<<grid, block, 0, stream>>>(buf, bytes, per, key, out);
    }
    return hipGetLastError();
}

hipError_t launch_probe_empty(hipStream_t stream)
{
    empty_kernel<<<dim3(1), dim3(64), 0, stream>>>();
    return hipGetLastError();
}

}  // namespace bigemm
