// attn_probe.hip -- a plain streaming read of device memory, the reference
// against which the decode kernel's bandwidth is judged: a decode step reads
// every cached key and value once and is bound by memory bandwidth
// ("RustingBrain" docs, "Generating text"), so the fastest possible decode of a
// cache is a kernel that only reads those bytes.
//
// Every lane reads 16-byte chunks with four loads in flight per iteration
// (grid-stride), XORs them together and writes the result only if it equals a
// sentinel (practically never): the loads cannot be removed, and the write
// traffic is nil.
#include "attn_device.h"
#include "attn_launch.h"

#include <algorithm>

namespace attn {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4 *__restrict__ src,
                                                                   long n16, unsigned *__restrict__ out)
{
    const long stride = (long)gridDim.x * kProbeThreads;
    long i = (long)blockIdx.x * kProbeThreads + threadIdx.x;
    uint4 acc = make_uint4(0, 0, 0, 0);
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        uint4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            acc.x ^= v[u].x; acc.y ^= v[u].y; acc.z ^= v[u].z; acc.w ^= v[u].w;
        }
    }
    for (; i < n16; i += stride) {
        const uint4 v = src[i];
        acc.x ^= v.x; acc.y ^= v.y; acc.z ^= v.z; acc.w ^= v.w;
    }
    const unsigned r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (r == 0x9e3779b9u) *out = r;
}

}  // namespace

hipError_t read_probe(const void *src, long bytes, unsigned *out, hipStream_t st)
{
    const long n16 = bytes / 16;
    const int cus = device_cus();
    // enough lanes that every CU keeps many 16-byte loads in flight: 8
    // workgroups per CU, fewer when there is less than that to read
    const long want = std::max<long>(1, (n16 + kProbeThreads * kProbeUnroll - 1) / (kProbeThreads * kProbeUnroll));
    const long blocks = std::min<long>(want, 8L * cus);
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, st,
                       (const uint4 *)src, n16, out);
    return hipGetLastError();
}

}  // namespace attn
