// A boolean mask tensor turned into the per-lane bit words the head-dim <=
// 128 prefill kernel applies with a bit-field extract and a bit select per
// score (mlx PR #4330, "Proposed changes": the boolean mask kind, nonzero =
// attend).
//
// In prefill_kernel, lane l of a wave holds query row 32 rb + (l mod 32) of
// its 32-row block rb, and in score slot (kb, 4 a4 + r) of key tile kt the
// key 64 kt + 32 kb + 8 a4 + 4 (l / 32) + r (64-key tiles, two 32-key score
// blocks).  For each (mask batch, mask head, rb, kt) this pass writes 64
// words, word l for lane l: bit 16 kb + 4 a4 + r says whether that lane's
// row attends that key (keys >= Lk: 0; rows past Lq repeat row Lq - 1, whose
// outputs are never stored).  A lane then reads one dword per tile (a wave:
// 256 contiguous bytes) instead of 32 mask bytes, and every head that shares
// the mask reads the same words: the byte tests run once per (row, key)
// instead of once per head.
#pragma once

#include "attn_common.h"

namespace sdpa_dev {

struct MaskBitsArgs {
    const uint8_t* mask;
    int64_t ms[4];     // element strides (b, h, row, key); 0 where broadcast
    uint32_t* bits;    // [Bm][Hm][RB][KT][64]
    int Bm, Hm, Lq, Lk, RB, KT;
    int vec;           // key stride 1 and 4-byte aligned 4-key runs: 32-bit loads
};

constexpr int kMaskBitsWords = 64;  // words (one per lane) per (32-row block, 64-key tile)

// One wave per (bm, hm, rb, kt); four per workgroup.
__global__ __launch_bounds__(256) void mask_bits_kernel(const MaskBitsArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (unit >= (int64_t)a.Bm * a.Hm * a.RB * a.KT) return;  // whole wave
    const int kt = (int)(unit % a.KT);
    int64_t t = unit / a.KT;
    const int rb = (int)(t % a.RB);
    t /= a.RB;
    const int hm = (int)(t % a.Hm), bm = (int)(t / a.Hm);
    const int row = min(rb * 32 + (lane & 31), a.Lq - 1), hh = lane >> 5;
    const uint8_t* mrow = a.mask + (int64_t)bm * a.ms[0] + (int64_t)hm * a.ms[1] + (int64_t)row * a.ms[2];
    uint32_t word = 0;
#pragma unroll
    for (int g = 0; g < 8; ++g) {  // g = 4 kb + a4: four keys each
        const int key0 = kt * 64 + 32 * (g >> 2) + 8 * (g & 3) + 4 * hh;
        uint32_t four = 0;
        if (a.vec && key0 + 3 < a.Lk) {
            four = *reinterpret_cast<const uint32_t*>(mrow + key0);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (key0 + r < a.Lk) four |= (uint32_t)mrow[(int64_t)(key0 + r) * a.ms[3]] << (8 * r);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) word |= (((four >> (8 * r)) & 0xffu) != 0u ? 1u : 0u) << (4 * g + r);
    }
    a.bits[unit * kMaskBitsWords + lane] = word;
}

}  // namespace sdpa_dev
