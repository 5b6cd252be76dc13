// Tile shapes per (element type, head dim).  Chosen so that each wave's O
// accumulator covers at most 128 head-dim columns (32 x 128 fp32 = 64 VGPRs)
// and each workgroup's LDS fits gfx950's 160 KB.
#pragma once

#include "attn_kernel.h"

namespace sdpa_dev {

// Prefill ("full"): 4 waves x 32 query rows for D <= 128; D = 256 splits the
// head dim over 2 waves and D = 512 over 4 waves per 32-row block.
template <class TR, int D> struct FullCfg { using type = TileCfg<TR, D, 64, 4, 1, 2>; };
template <int D> struct FullCfg<TF32, D> { using type = TileCfg<TF32, D, 64, 4, 1, 1>; };
template <class TR> struct FullCfg<TR, 256> { using type = TileCfg<TR, 256, 32, 2, 2>; };
template <> struct FullCfg<TF32, 256> { using type = TileCfg<TF32, 256, 32, 2, 2>; };
template <class TR> struct FullCfg<TR, 512> { using type = TileCfg<TR, 512, 32, 2, 4>; };
template <> struct FullCfg<TF32, 512> { using type = TileCfg<TF32, 512, 32, 1, 4>; };

// Decode ("vector"): one 32-column block (n_rep x q_len <= 32 per group) per workgroup.
template <class TR, int D> struct DecodeCfg { using type = TileCfg<TR, D, 64, 1, 1>; };
template <int D> struct DecodeCfg<TF32, D> { using type = TileCfg<TF32, D, 32, 1, 1>; };
template <class TR> struct DecodeCfg<TR, 256> { using type = TileCfg<TR, 256, 32, 1, 2>; };
template <class TR> struct DecodeCfg<TR, 512> { using type = TileCfg<TR, 512, 32, 1, 4>; };
template <> struct DecodeCfg<TF32, 256> { using type = TileCfg<TF32, 256, 32, 1, 2>; };
template <> struct DecodeCfg<TF32, 512> { using type = TileCfg<TF32, 512, 32, 1, 4>; };

}  // namespace sdpa_dev
