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
    int vec;           // key stride 1 and row starts 16-byte aligned: 16-byte loads
};

constexpr int kMaskBitsWords = 64;  // words (one per lane) per (32-row block, 64-key tile)

// Bit k of the result: byte k of w is nonzero (k = 0..3).  The high bit of
// each byte is set where the byte is nonzero; one multiply gathers the four
// high bits (bits 7, 15, 23, 31) into bits 28..31, their partial products
// landing on distinct bit positions.
__device__ __forceinline__ uint32_t nonzero_bytes4(uint32_t w) {
    const uint32_t t = (((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u;
    return (t * 0x00204081u) >> 28;
}

// One wave per (bm, hm, rb, kt); four per workgroup, consecutive key tiles.
// Lane l reads keys 64 kt + 16 (l % 4) .. + 15 of rows l / 4 and
// 16 + l / 4 of the block, turns them into 16 bits, and parks them in LDS;
// lane l then takes its row's 64 bits (row l % 32) and keeps the 4-key
// groups of its half (the even groups for l < 32, the odd ones above):
// group 2 g + l / 32 becomes bits 4 g .. 4 g + 3 of its word.
__global__ __launch_bounds__(256) void mask_bits_kernel(const MaskBitsArgs a) {
    __shared__ __attribute__((aligned(8))) uint16_t park[4][32][4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t unit = (int64_t)blockIdx.x * 4 + w;
    if (unit >= (int64_t)a.Bm * a.Hm * a.RB * a.KT) return;  // whole wave
    const int kt = (int)(unit % a.KT);
    int64_t t = unit / a.KT;
    const int rb = (int)(t % a.RB);
    t /= a.RB;
    const int hm = (int)(t % a.Hm), bm = (int)(t / a.Hm);
    const uint8_t* mbase = a.mask + (int64_t)bm * a.ms[0] + (int64_t)hm * a.ms[1];
    const int c = lane & 3, key0 = kt * 64 + 16 * c;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int rl = 16 * h + (lane >> 2);  // row within the block
        const uint8_t* mrow = mbase + (int64_t)min(rb * 32 + rl, a.Lq - 1) * a.ms[2];
        uint32_t m16 = 0;
        if (a.vec && key0 + 15 < a.Lk) {
            const uint4 v = *reinterpret_cast<const uint4*>(mrow + key0);
            m16 = nonzero_bytes4(v.x) | nonzero_bytes4(v.y) << 4 | nonzero_bytes4(v.z) << 8 |
                  nonzero_bytes4(v.w) << 12;
        } else {
            for (int k = 0; k < 16; ++k)
                if (key0 + k < a.Lk && mrow[(int64_t)(key0 + k) * a.ms[3]] != 0) m16 |= 1u << k;
        }
        park[w][rl][c] = (uint16_t)m16;
    }
    __builtin_amdgcn_wave_barrier();  // one wave writes and reads its own slice, in order
    const uint64_t row = *reinterpret_cast<const uint64_t*>(&park[w][lane & 31][0]);
    uint64_t x = (row >> (4 * (lane >> 5))) & 0x0f0f0f0f0f0f0f0full;  // this half's 4-key groups
    x = (x | x >> 4) & 0x00ff00ff00ff00ffull;
    x = (x | x >> 8) & 0x0000ffff0000ffffull;
    x = (x | x >> 16) & 0x00000000ffffffffull;
    a.bits[unit * kMaskBitsWords + lane] = (uint32_t)x;
}

}  // namespace sdpa_dev
