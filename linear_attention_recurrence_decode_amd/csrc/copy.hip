// copy.hip -- bitwise slot copies between the live state pools and the
// checkpoint pools (kda_state_checkpoint and copy-on-write kda_resume).
// [vLLM blog "A Preview of Production-Scale Kimi K3 Support on vLLM", section
//  "The Hardest Part: Prefix Caching for KDA": a cached state is copied into a
//  private destination before a request extends it.]
//
// The head's state (dk*dv elements of the state dtype) and its conv state
// (each a multiple of 16 bytes) move as 16-byte words, one per thread, in
// 4 KiB pieces: many short workgroups that each load and store once stream
// better than one long workgroup per (pair, head) looping over its words.
// Ids outside their pool are skipped.

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kCopyThreads = 256;

// One workgroup per 4 KiB piece of a (pair, head): the state's pieces, then
// the conv state's.
__global__ __launch_bounds__(kCopyThreads) void copy_kernel(CopyParams p) {
    const int64_t sw = p.state_bytes / 16, cw = p.conv_bytes / 16;
    const int64_t sblk = (sw + kCopyThreads - 1) / kCopyThreads, cblk = (cw + kCopyThreads - 1) / kCopyThreads;
    const int64_t per = sblk + cblk;
    const int64_t ph = blockIdx.x / per, part = blockIdx.x % per;
    const int i = static_cast<int>(ph / p.H), h = static_cast<int>(ph % p.H);
    const int src = p.src_idx[i], dst = p.dst_idx[i];
    if (src < 0 || src >= p.src_slots || dst < 0 || dst >= p.dst_slots) return;
    const int64_t sh = static_cast<int64_t>(src) * p.H + h;
    const int64_t dh = static_cast<int64_t>(dst) * p.H + h;
    if (part < sblk) {
        const int64_t e = part * kCopyThreads + threadIdx.x;
        if (e < sw) {
            const uint4* s4 = reinterpret_cast<const uint4*>(static_cast<const char*>(p.src_state) + sh * p.state_bytes);
            uint4* d4 = reinterpret_cast<uint4*>(static_cast<char*>(p.dst_state) + dh * p.state_bytes);
            d4[e] = s4[e];
        }
    } else {
        const int64_t e = (part - sblk) * kCopyThreads + threadIdx.x;
        if (e < cw) {
            const uint4* sc = reinterpret_cast<const uint4*>(static_cast<const char*>(p.src_conv) + sh * p.conv_bytes);
            uint4* dc = reinterpret_cast<uint4*>(static_cast<char*>(p.dst_conv) + dh * p.conv_bytes);
            dc[e] = sc[e];
        }
    }
}

hipError_t launch_copy(const CopyParams& p, hipStream_t s) {
    const int64_t per = (p.state_bytes / 16 + kCopyThreads - 1) / kCopyThreads +
                        (p.conv_bytes / 16 + kCopyThreads - 1) / kCopyThreads;
    const int64_t blocks = static_cast<int64_t>(p.n) * p.H * per;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kCopyThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace kda
