// Plain streaming read of a device buffer: the HBM read rate one launch of
// a given size reaches on this part, measured beside the decode kernel (which
// must read K and V once, the same kind of traffic).  Diagnostics only.
//
// 256-thread workgroups, one per CU; each thread keeps eight 16-byte loads in
// flight over a grid-strided range (the fastest of the shapes swept for a
// 33.5 MB read).  The xor of everything read is stored only if it equals a
// fixed pattern, so no load can be dropped and the stores never happen for
// ordinary data.
#pragma once

#include "attn_common.h"

namespace sdpa_dev {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4_t* __restrict__ src, uint64_t nvec,
                                                                     uint32_t* sink) {
    const uint64_t stride = (uint64_t)gridDim.x * kProbeThreads;
    uint64_t i = (uint64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (; i + (kProbeUnroll - 1) * stride < nvec; i += kProbeUnroll * stride) {
        u32x4_t v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(&src[i + u * stride]);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
    }
    for (; i < nvec; i += stride) acc ^= src[i];
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x5d1c0ffeu) sink[0] = acc[0];
}

}  // namespace sdpa_dev
