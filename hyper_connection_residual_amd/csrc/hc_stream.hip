// hc_stream.hip -- a measurement reference for the short-window kernel: one
// launch of its shape (256 workgroups x 512 threads, one per CU) that only
// streams a buffer from memory into LDS with the same whole-line loads
// (global_load_lds_dwordx4) the kernel's weight tiles use, and does nothing
// else.  Its duration is what a single launch that moves that many bytes can
// reach on the device, the floor the read's duration is compared with.
#include "hc_internal.h"

namespace hc {
namespace {

constexpr int kRing = 32;  // LDS ring of 32 wave-sized (1 KB) slots; its contents are never read

__global__ __launch_bounds__(kDecThreads) void stream_kernel(const uint4* __restrict__ src, int64_t n16,
                                                             uint32_t* __restrict__ sink)
{
    __shared__ __align__(16) uint4 ring[kRing * 64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // workgroup b streams the 16-byte items [b * per, (b + 1) * per), wave by
    // wave in 64-item (1 KB) pieces; items past the end re-read the last one
    const int64_t per = (n16 + kDecWGs - 1) / kDecWGs;
    const int64_t base = (int64_t)blockIdx.x * per;
    const int64_t last = n16 - 1;
    const int pieces = (int)((per + 63) / 64);
    for (int q = wave, k = 0; q < pieces; q += kDecThreads / 64, ++k) {
        int64_t it = base + 64 * (int64_t)q + lane;
        it = it < base + per && it <= last ? it : last;
        __builtin_amdgcn_global_load_lds(src + it, ring + 64 * ((wave + 8 * k) % kRing), 16, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (threadIdx.x == 0)
        sink[blockIdx.x] = ring[0].x;
}

}  // namespace

hipError_t launch_stream(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream)
{
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(stream_kernel, dim3(kDecWGs), dim3(kDecThreads), 0, stream,
                       static_cast<const uint4*>(src), n16, sink);
    return hipGetLastError();
}

}  // namespace hc
