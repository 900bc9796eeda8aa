// copy.hip -- bitwise slot copies between the live state pools and the
// checkpoint pools (kda_state_checkpoint and copy-on-write kda_resume).
// [vLLM blog "A Preview of Production-Scale Kimi K3 Support on vLLM", section
//  "The Hardest Part: Prefix Caching for KDA": a cached state is copied into a
//  private destination before a request extends it.]
//
// One workgroup per (pair, head): the head's state (dk*dv elements of the
// state dtype) and its conv state (each a multiple of 16 bytes) move as
// 16-byte words.  Ids outside their pool are skipped.

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void copy_kernel(CopyParams p) {
    const int i = blockIdx.x / p.H, h = blockIdx.x % p.H;
    const int src = p.src_idx[i], dst = p.dst_idx[i];
    if (src < 0 || src >= p.src_slots || dst < 0 || dst >= p.dst_slots) return;
    const int64_t sh = static_cast<int64_t>(src) * p.H + h;
    const int64_t dh = static_cast<int64_t>(dst) * p.H + h;
    const uint4* s4 = reinterpret_cast<const uint4*>(static_cast<const char*>(p.src_state) + sh * p.state_bytes);
    uint4* d4 = reinterpret_cast<uint4*>(static_cast<char*>(p.dst_state) + dh * p.state_bytes);
    const int64_t n4 = p.state_bytes / 16;
    for (int64_t e = threadIdx.x; e < n4; e += kCopyThreads) d4[e] = s4[e];
    const uint4* sc = reinterpret_cast<const uint4*>(static_cast<const char*>(p.src_conv) + sh * p.conv_bytes);
    uint4* dc = reinterpret_cast<uint4*>(static_cast<char*>(p.dst_conv) + dh * p.conv_bytes);
    const int64_t c16 = p.conv_bytes / 16;
    for (int64_t e = threadIdx.x; e < c16; e += kCopyThreads) dc[e] = sc[e];
}

hipError_t launch_copy(const CopyParams& p, hipStream_t s) {
    const int64_t blocks = static_cast<int64_t>(p.n) * p.H;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kCopyThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace kda
