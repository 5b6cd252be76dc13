// Prefill ("full") kernel for 16-bit inputs and wide heads (D = 256, 512) on gfx950.
//
// At D = 512 a 32-row query block needs 32 x 512 fp32 accumulators (256
// registers per lane) and 32 x 512 16-bit values of Q (128 registers per
// lane): one wave holds a whole query block only at one wave per SIMD, with O
// in the accumulation registers (AGPRs) and Q in the vector registers.  That
// is the layout used here, so every wave contracts the full head dim for its
// own scores and no partial scores cross waves:
//   * a workgroup is 4 waves = 4 (query head, 32-row block) pairs of ONE
//     key/value head: the query heads of a grouped-query group (mlx issue
//     #3885, prefill paragraph: scores [B, n_kv, n_rep, qL, kL]) share every
//     K/V tile loaded into LDS (up to 4 heads per workgroup; with fewer heads
//     in the group the spare waves take further row blocks of the same head);
//   * K/V tiles of BN keys go global -> LDS with buffer_load ... lds, double
//     buffered, one barrier per tile.  LDS rows are unpadded; the 16-byte
//     chunks of row r sit at chunk ^ sw(r) (sw a bijection on r mod 8), which
//     keeps the 128-bit K reads and the transposed 64-bit V reads free of
//     bank conflicts;
//   * S^T = K Q^T with K from LDS and Q from registers, online softmax in
//     base 2 with lazy rescale, O^T += V^T P^T with V^T read from the
//     row-major V tile through ds_read_b64_tr_b16;
//   * LDS reads are software-pipelined one group ahead of the MFMAs that use
//     them; scheduling barriers bound how far the compiler may hoist them,
//     which is what keeps the kernel inside the register file.
#pragma once

#include "attn_common.h"

namespace sdpa_dev {

template <class TR, int D_, int BN_>
struct WideCfg {
    static constexpr int D = D_, BN = BN_, NW = 4, NT = 64 * NW;
    static constexpr int KC = D / 8;             // 16-byte chunks per row
    static constexpr int ROWB = D * 2;           // bytes per LDS row (unpadded)
    static constexpr int TILEB = BN * ROWB;
    static constexpr int NCH = D / 16;           // Q K^T contraction chunks
    static constexpr int NDB = D / 32;           // 32-column O^T blocks
    static constexpr int NKB = BN / 32;          // 32-key score blocks per tile
    static constexpr int RPI = 64 / KC;          // rows filled by one 64-lane load
    static constexpr int NI = BN * KC / (64 * NW);  // load instructions per wave per tile (K, and V)
    static constexpr int RSTEP = NW * RPI;       // rows between a wave's consecutive loads
    static constexpr int SWP = (RSTEP % 8 == 0) ? 1 : 8 / RSTEP;  // period of the swizzle pattern in u
    static constexpr int KG = 4;                 // K chunks per pipelined group
    static constexpr int VG = 4;                 // O^T blocks per pipelined group
    static constexpr int LDS = 4 * TILEB;
    static_assert(D % 32 == 0 && D >= 256 && KC <= 64, "wide head dims");
    static_assert(BN % 32 == 0 && (BN * KC) % (64 * NW) == 0, "key tile");
    static_assert(8 % RSTEP == 0 || RSTEP % 8 == 0, "swizzle period");
    static_assert(NCH % KG == 0 && NDB % VG == 0, "pipeline groups");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// row -> chunk swizzle: rows 0..7 -> 0,2,4,6,1,3,5,7 (bijection on r mod 8);
// four consecutive rows from a multiple of 4 get distinct even (or odd) values.
__device__ __forceinline__ int wide_sw(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

template <bool B> struct WideTag { static constexpr bool value = B; };

template <class TR, class C, int MASK>
__global__ __launch_bounds__(C::NT, 1) void prefill_wide_kernel(const Params p) {
    constexpr int D = C::D, BN = C::BN;
    constexpr float NEG_INF = -__builtin_inff();
    constexpr float kRescale = 8.0f;
    constexpr bool HAS_MT = (MASK == MASK_ADD16 || MASK == MASK_ADD32 || MASK == MASK_BOOL);
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int col = lane & 31, hh = lane >> 5;

    // ---- work item: (batch, kv head, head group, row tile), XCD-aware ----
    const int n_rep = p.n_rep;
    const int HG = (n_rep % 4 == 0) ? 4 : ((n_rep % 2 == 0) ? 2 : 1);  // query heads per workgroup
    const int RB = 4 / HG;                                               // 32-row blocks per head
    const int BMW = 32 * RB;                                             // query rows per workgroup
    const int nrt = (p.Lq + BMW - 1) / BMW;
    const int nhg = n_rep / HG;
    const int total = nrt * nhg * p.Hkv * p.B;
    const int per = (total + 7) / 8;
    const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (item >= total) return;
    const int tt = item % nrt;
    int rest = item / nrt;
    const int hgi = rest % nhg;
    rest /= nhg;
    const int g = rest % p.Hkv, b = rest / p.Hkv;
    const int t = (MASK == MASK_CAUSAL) ? nrt - 1 - tt : tt;  // heavy row tiles first
    const int i0 = t * BMW;
    const int qh = g * n_rep + hgi * HG + (w % HG);
    const int qmin = i0 + 32 * (w / HG);
    const int qi = qmin + col;
    const bool rv = qi < p.Lq;
    const int off = p.Lk - p.Lq;  // bottom-right causal alignment
    int kend = p.Lk;
    if (MASK == MASK_CAUSAL) {
        const int64_t e = (int64_t)i0 + BMW + off;
        kend = (int)(e < 0 ? 0 : (e > p.Lk ? p.Lk : e));
    }
    // keys [0, kplain) need no per-element mask for any row of this wave
    int kplain = kend;
    if (MASK == MASK_CAUSAL) kplain = min(kend, max(0, qmin + off + 1));
    if (HAS_MT || !p.scale_nonneg) kplain = 0;
    const int nplain = kplain / BN;
    const int ntiles = (kend + BN - 1) / BN;

    const uint32_t kstep = (uint32_t)p.ks[2] * 2u, vstep = (uint32_t)p.vs[2] * 2u;
    const char* kglob = reinterpret_cast<const char*>(p.k) + ((int64_t)b * p.ks[0] + (int64_t)g * p.ks[1]) * 2;
    const char* vglob = reinterpret_cast<const char*>(p.v) + ((int64_t)b * p.vs[0] + (int64_t)g * p.vs[1]) * 2;
    // rows at or past kend read as zero (buffer range check)
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kglob, kend > 0 ? (uint32_t)(kend - 1) * kstep + (uint32_t)(D * 2) : 0u);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vglob, kend > 0 ? (uint32_t)(kend - 1) * vstep + (uint32_t)(D * 2) : 0u);

    // ---- Q fragments (MFMA B operand) for the full head dim ----
    u32x4_t qf[C::NCH];
    {
        const char* qrow = reinterpret_cast<const char*>(p.q) +
                           ((int64_t)b * p.qs[0] + (int64_t)qh * p.qs[1] + (int64_t)(rv ? qi : 0) * p.qs[2]) * 2;
#pragma unroll
        for (int ch = 0; ch < C::NCH; ++ch)
            qf[ch] = rv ? *reinterpret_cast<const u32x4_t*>(qrow + (ch * 16 + hh * 8) * 2) : u32x4_t{0u, 0u, 0u, 0u};
    }

    // ---- load slots: instruction u of wave w fills LDS bytes [(u*NW + w) * 1024, +1024) ----
    // lane -> row rl + u*RSTEP of the tile, stored chunk lane % KC holding source
    // chunk (lane % KC) ^ sw(row); the swizzle repeats every SWP instructions.
    const int rl = w * C::RPI + lane / C::KC;
    uint32_t kv0[C::SWP], vv0[C::SWP];
#pragma unroll
    for (int ph = 0; ph < C::SWP; ++ph) {
        const int row = rl + ph * C::RSTEP;
        const uint32_t cb = (uint32_t)(((lane % C::KC) ^ wide_sw(row)) * 16);
        kv0[ph] = (uint32_t)rl * kstep + cb;
        vv0[ph] = (uint32_t)rl * vstep + cb;
    }
    auto issue_tile = [&](int kt, int stage) {
        char* kt_lds = smem + (2 * stage) * C::TILEB;
        char* vt_lds = smem + (2 * stage + 1) * C::TILEB;
        const uint32_t kb0 = (uint32_t)kt * kstep, vb0 = (uint32_t)kt * vstep;
#pragma unroll
        for (int u = 0; u < C::NI; ++u) {
            const int blk = (u * C::NW + w) * 1024;
            buffer_load16_lds(krs, kt_lds + blk, kv0[u % C::SWP] + kb0 + (uint32_t)(u * C::RSTEP) * kstep);
            buffer_load16_lds(vrs, vt_lds + blk, vv0[u % C::SWP] + vb0 + (uint32_t)(u * C::RSTEP) * vstep);
        }
    };

    const int64_t mrow = HAS_MT ? (int64_t)b * p.ms[0] + (int64_t)qh * p.ms[1] + (int64_t)(rv ? qi : 0) * p.ms[2] : 0;
    typename MaskRaw<MASK>::type mr[HAS_MT ? C::NKB : 1][4];
    auto load_mask = [&](int kt) {
        if constexpr (HAS_MT) {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) mr[kb][a4] = load_mask_group<MASK>(p, mrow, kt + kb * 32 + 8 * a4 + 4 * hh);
        }
    };

    // per-lane LDS read offsets
    // K (A operand of S^T): key row kb*32 + col, chunk 2*ch + hh, swizzled by sw(col)
    // chunk c = 2 ch + hh: (c ^ ksw) = 8 (ch >> 2) + ((2 (ch & 3) + hh) ^ ksw), four per-lane values
    const int ksw = wide_sw(col);
    const int kbase = col * C::ROWB;
    int kx[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) kx[m] = ((2 * m + hh) ^ ksw) * 16;
    // V^T (A operand of O^T, transposed reads): key row 16*pc + 4*(grp>>1) + e4 (+8),
    // columns 32*db + 16*(grp&1) + 4*j4 -> chunk 4*db + 2*(grp&1) + (j4>>1), byte 8*(j4&1)
    const int grp = lane >> 4, e4 = (lane >> 2) & 3, j4 = lane & 3;
    const int vrow = 4 * (grp >> 1) + e4;
    const int vsw = wide_sw(vrow);
    const int vbase = vrow * C::ROWB + 8 * (j4 & 1);
    const int vc0 = 2 * (grp & 1) + (j4 >> 1);
    // (4 db + vc0) ^ vsw = 8 (db >> 1) + ((4 (db & 1) + vc0) ^ vsw), two per-lane values
    const int vx[2] = {(vc0 ^ vsw) * 16, ((4 + vc0) ^ vsw) * 16};

    float m_run = NEG_INF, l_run = 0.f;
    f32x16_t oacc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) oacc[db] = f32x16_t{};
    const float c_scale = p.scale_log2;

    auto tile = [&](int it, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int kt = it * BN, stage = it & 1;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // tile `it` is in LDS; every wave is done with the other stage
        if (it + 1 < ntiles) issue_tile(kt + BN, stage ^ 1);
        const char* kt_lds = smem + (2 * stage) * C::TILEB + kbase;
        const char* vt_lds = smem + (2 * stage + 1) * C::TILEB + vbase;

        // ---- S^T blocks, K reads one group ahead ----
        f32x16_t sacc[C::NKB];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
            constexpr int NG = C::NCH / C::KG;
            u32x4_t ka[2][C::KG];
            auto kread = [&](int gi, u32x4_t(&dst)[C::KG]) {
#pragma unroll
                for (int i = 0; i < C::KG; ++i) {
                    const int ch = gi * C::KG + i;
                    dst[i] = *reinterpret_cast<const u32x4_t*>(kt_lds + kb * 32 * C::ROWB + (ch >> 2) * 128 + kx[ch & 3]);
                }
            };
            kread(0, ka[0]);
            f32x16_t s = f32x16_t{};
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                if (gi + 1 < NG) kread(gi + 1, ka[(gi + 1) & 1]);
#pragma unroll
                for (int i = 0; i < C::KG; ++i) s = TR::mma(ka[gi & 1][i], qf[gi * C::KG + i], s);
                __builtin_amdgcn_sched_barrier(0);
            }
            sacc[kb] = s;
        }

        // ---- mask, row max ----
        float mtile, c_eff;
        if constexpr (!MASKED) {
            float mx = NEG_INF;
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mtile = mx * c_scale;
            c_eff = c_scale;
        } else {
            mtile = NEG_INF;
            c_eff = 1.f;
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = kt + kb * 32 + 8 * a4 + 4 * hh + r;
                        float x = sacc[kb][4 * a4 + r] * c_scale;
                        bool ok = j < kend;
                        if constexpr (MASK == MASK_ADD16 || MASK == MASK_ADD32)
                            x = __builtin_fmaf(mask_value<MASK>(mr[kb][a4], r, p.mask_dtype), kLog2e, x);
                        if constexpr (MASK == MASK_CAUSAL) ok = ok && (j <= qi + off);
                        if constexpr (MASK == MASK_BOOL) ok = ok && ((mr[kb][a4] >> (8 * r)) & 0xffu) != 0u;
                        x = ok ? x : NEG_INF;
                        sacc[kb][4 * a4 + r] = x;
                        mtile = fmaxf(mtile, x);
                    }
            if (it + 1 < ntiles) load_mask(kt + BN);
        }

        // ---- online softmax (base 2, lazy rescale) ----
        mtile = fmaxf(mtile, xor32(mtile));
        if (__any(mtile > m_run + kRescale)) {
            const float m_new = fmaxf(m_run, mtile);
            const float alpha = (m_new == NEG_INF) ? 1.f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
            // keeps this block a real branch: speculating it would put 16*NDB
            // multiplies (plus AGPR round trips) on every tile
            asm volatile("" ::: "memory");
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
        const float muse = (m_run == NEG_INF) ? 0.f : m_run;
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = fast_exp2(__builtin_fmaf(sacc[kb][r], c_eff, -muse));
                sacc[kb][r] = e;
                lsum += e;
            }
        l_run += lsum;
        __builtin_amdgcn_sched_barrier(0);

        // ---- O^T += V^T P^T, V reads one group ahead ----
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
            for (int pc = 0; pc < 2; ++pc) {
                u32x4_t bf;
#pragma unroll
                for (int q = 0; q < 4; ++q) bf[q] = TR::pack(sacc[kb][8 * pc + 2 * q], sacc[kb][8 * pc + 2 * q + 1]);
                const char* vrow_p = vt_lds + (kb * 32 + 16 * pc) * C::ROWB;
                constexpr int NG = C::NDB / C::VG;
                u32x4_t va[2][C::VG];
                auto vread = [&](int gi, u32x4_t(&dst)[C::VG]) {
#pragma unroll
                    for (int i = 0; i < C::VG; ++i) {
                        const int db = gi * C::VG + i;
                        const int cofs = (db >> 1) * 128 + vx[db & 1];
                        const u32x2_t y0 = lds_read_tr16(vrow_p + cofs);
                        const u32x2_t y1 = lds_read_tr16(vrow_p + 8 * C::ROWB + cofs);
                        dst[i] = u32x4_t{y0[0], y0[1], y1[0], y1[1]};
                    }
                };
                vread(0, va[0]);
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    if (gi + 1 < NG) vread(gi + 1, va[(gi + 1) & 1]);
#pragma unroll
                    for (int i = 0; i < C::VG; ++i) {
                        const int db = gi * C::VG + i;
                        oacc[db] = TR::mma(va[gi & 1][i], bf, oacc[db]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };

    int it = 0;
    if (ntiles > 0) issue_tile(0, 0);
    if constexpr (!HAS_MT) {
        for (; it < nplain; ++it) tile(it, WideTag<false>{});
    }
    if (it < ntiles) load_mask(it * BN);
    for (; it < ntiles; ++it) tile(it, WideTag<true>{});

    // ---- epilogue: O = O^T / l, written row-major ----
    const float lsum_row = l_run + xor32(l_run);
    if (rv) {
        const float inv = lsum_row > 0.f ? 1.f / lsum_row : 0.f;
        char* orow = reinterpret_cast<char*>(p.o) +
                     ((int64_t)b * p.os[0] + (int64_t)qh * p.os[1] + (int64_t)qi * p.os[2]) * 2;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d0 = 32 * db + 8 * a4 + 4 * hh;
                f32x4_t x = {oacc[db][4 * a4] * inv, oacc[db][4 * a4 + 1] * inv, oacc[db][4 * a4 + 2] * inv,
                             oacc[db][4 * a4 + 3] * inv};
                TR::store4(orow + d0 * 2, x);
            }
    }
}


// ---------------------------------------------------------------------------
// Sixteen query rows per wave (v_mfma_f32_16x16x32): O^T of a 16-row block at
// D = 512 is 128 registers per lane and Q^T 64, so two waves fit per SIMD.
// A workgroup is NW waves = NW (query head, 16-row block) pairs of one
// key/value head (heads of the group first, as above); K/V tiles, swizzle and
// pipelining as in prefill_wide_kernel.
//   S^T block (16 keys x 16 queries) = K (16 x 32 of D) Q^T, D / 32 steps;
//   lane l holds query l % 16 against keys 4 * (l / 16) + i, i = 0..3.
//   O^T block (16 of D x 16 queries) += V^T (16 x 32 keys) P^T: the B operand
//   slot 8 * (l / 16) + j is key 4 * (l / 16) + j of the first 16-key block
//   (j < 4) or of the second (j >= 4) -- exactly the scores lane l holds --
//   and the A operand takes the same keys from two transposed LDS reads.
#ifndef R16_KG
#define R16_KG 2
#endif
#ifndef R16_VG
#define R16_VG 2
#endif
template <class TR, int D_, int BN_, int NW_>
struct R16Cfg {
    static constexpr int D = D_, BN = BN_, NW = NW_, NT = 64 * NW;
    static constexpr int KC = D / 8;             // 16-byte chunks per row
    static constexpr int ROWB = D * 2;           // bytes per LDS row (unpadded)
    static constexpr int TILEB = BN * ROWB;
    static constexpr int NCH = D / 32;           // Q K^T steps
    static constexpr int NDB = D / 16;           // 16-column O^T blocks
    static constexpr int NKB = BN / 16;          // 16-key score blocks per tile
    static constexpr int NKP = BN / 32;          // 32-key P V steps per tile
    static constexpr int RPI = 64 / KC;
    static constexpr int NI = BN * KC / (64 * NW);
    static constexpr int RSTEP = NW * RPI;
    static constexpr int SWP = (RSTEP % 8 == 0) ? 1 : 8 / RSTEP;
    static constexpr int KG = R16_KG;                 // K chunks per pipelined group
    static constexpr int VG = R16_VG;                 // O^T blocks per pipelined group
    static constexpr int LDS = 4 * TILEB;
    static_assert(D % 32 == 0 && KC <= 64, "head dim");
    static_assert(BN % 32 == 0 && (BN * KC) % (64 * NW) == 0, "key tile");
    static_assert(8 % RSTEP == 0 || RSTEP % 8 == 0, "swizzle period");
    static_assert(NCH % KG == 0 && NDB % VG == 0, "pipeline groups");
    static_assert(NW == 8 || NW == 4, "waves per workgroup");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <class TR, class C, int MASK>
__global__ __launch_bounds__(C::NT, 1) void prefill_r16_kernel(const Params p) {
    constexpr int D = C::D, BN = C::BN, NW = C::NW;
    constexpr float NEG_INF = -__builtin_inff();
    constexpr float kRescale = 8.0f;
    constexpr bool HAS_MT = (MASK == MASK_ADD16 || MASK == MASK_ADD32 || MASK == MASK_BOOL);
    using M16 = Mma16<TR>;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int c16 = lane & 15, g4 = lane >> 4;

    // ---- work item: (batch, kv head, head group, row tile), XCD-aware ----
    const int n_rep = p.n_rep;
    const int HG = (NW >= 8 && n_rep % 8 == 0) ? 8 : (n_rep % 4 == 0) ? 4 : ((n_rep % 2 == 0) ? 2 : 1);
    const int RB = NW / HG;
    const int BMW = 16 * RB;
    const int nrt = (p.Lq + BMW - 1) / BMW;
    const int nhg = n_rep / HG;
    const int total = nrt * nhg * p.Hkv * p.B;
    const int per = (total + 7) / 8;
    const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (item >= total) return;
    const int tt = item % nrt;
    int rest = item / nrt;
    const int hgi = rest % nhg;
    rest /= nhg;
    const int g = rest % p.Hkv, b = rest / p.Hkv;
    const int t = (MASK == MASK_CAUSAL) ? nrt - 1 - tt : tt;  // heavy row tiles first
    const int i0 = t * BMW;
    const int qh = g * n_rep + hgi * HG + (w % HG);
    const int qmin = i0 + 16 * (w / HG);
    const int qi = qmin + c16;
    const bool rv = qi < p.Lq;
    const int off = p.Lk - p.Lq;
    int kend = p.Lk;
    if (MASK == MASK_CAUSAL) {
        const int64_t e = (int64_t)i0 + BMW + off;
        kend = (int)(e < 0 ? 0 : (e > p.Lk ? p.Lk : e));
    }
    int kplain = kend;
    if (MASK == MASK_CAUSAL) kplain = min(kend, max(0, qmin + off + 1));
    if (HAS_MT || !p.scale_nonneg) kplain = 0;
    const int nplain = kplain / BN;
    const int ntiles = (kend + BN - 1) / BN;

    const uint32_t kstep = (uint32_t)p.ks[2] * 2u, vstep = (uint32_t)p.vs[2] * 2u;
    const char* kglob = reinterpret_cast<const char*>(p.k) + ((int64_t)b * p.ks[0] + (int64_t)g * p.ks[1]) * 2;
    const char* vglob = reinterpret_cast<const char*>(p.v) + ((int64_t)b * p.vs[0] + (int64_t)g * p.vs[1]) * 2;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kglob, kend > 0 ? (uint32_t)(kend - 1) * kstep + (uint32_t)(D * 2) : 0u);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vglob, kend > 0 ? (uint32_t)(kend - 1) * vstep + (uint32_t)(D * 2) : 0u);

    // ---- Q^T fragments: lane holds Q[qi][32 c + 8 g4 .. +8] ----
    u32x4_t qf[C::NCH];
    {
        const char* qrow = reinterpret_cast<const char*>(p.q) +
                           ((int64_t)b * p.qs[0] + (int64_t)qh * p.qs[1] + (int64_t)(rv ? qi : 0) * p.qs[2]) * 2;
#pragma unroll
        for (int c = 0; c < C::NCH; ++c)
            qf[c] = rv ? *reinterpret_cast<const u32x4_t*>(qrow + (32 * c + 8 * g4) * 2) : u32x4_t{0u, 0u, 0u, 0u};
    }

    const int rl = w * C::RPI + lane / C::KC;
    uint32_t kv0[C::SWP], vv0[C::SWP];
#pragma unroll
    for (int ph = 0; ph < C::SWP; ++ph) {
        const int row = rl + ph * C::RSTEP;
        const uint32_t cb = (uint32_t)(((lane % C::KC) ^ wide_sw(row)) * 16);
        kv0[ph] = (uint32_t)rl * kstep + cb;
        vv0[ph] = (uint32_t)rl * vstep + cb;
    }
    auto issue_tile = [&](int kt, int stage) {
        char* kt_lds = smem + (2 * stage) * C::TILEB;
        char* vt_lds = smem + (2 * stage + 1) * C::TILEB;
        const uint32_t kb0 = (uint32_t)kt * kstep, vb0 = (uint32_t)kt * vstep;
#pragma unroll
        for (int u = 0; u < C::NI; ++u) {
            const int blk = (u * NW + w) * 1024;
            buffer_load16_lds(krs, kt_lds + blk, kv0[u % C::SWP] + kb0 + (uint32_t)(u * C::RSTEP) * kstep);
            buffer_load16_lds(vrs, vt_lds + blk, vv0[u % C::SWP] + vb0 + (uint32_t)(u * C::RSTEP) * vstep);
        }
    };

    const int64_t mrow = HAS_MT ? (int64_t)b * p.ms[0] + (int64_t)qh * p.ms[1] + (int64_t)(rv ? qi : 0) * p.ms[2] : 0;
    typename MaskRaw<MASK>::type mr[HAS_MT ? C::NKB : 1];
    auto load_mask = [&](int kt) {
        if constexpr (HAS_MT) {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) mr[kb] = load_mask_group<MASK>(p, mrow, kt + 16 * kb + 4 * g4);
        }
    };

    // K: row 16 kb + c16, chunk 4 c + g4; V (transposed reads): rows 4 g4 + e4
    // (+16), columns 16 db + 4 j4 -> chunk 2 db + (j4 >> 1), byte 8 (j4 & 1)
    // (4 c + g4) ^ ksw = 8 (c >> 1) + ((4 (c & 1) + g4) ^ ksw); (2 db + vc0) ^ vsw =
    // 8 (db >> 2) + ((2 (db & 3) + vc0) ^ vsw): a few per-lane values, the rest immediate
    const int ksw = wide_sw(c16);
    const int kbase = c16 * C::ROWB;
    const int kx[2] = {(g4 ^ ksw) * 16, ((4 + g4) ^ ksw) * 16};
    const int e4 = (lane >> 2) & 3, j4 = lane & 3;
    const int vsw = wide_sw(4 * g4 + e4);
    const int vbase = (4 * g4 + e4) * C::ROWB + 8 * (j4 & 1);
    const int vc0 = j4 >> 1;
    int vx[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) vx[m] = ((2 * m + vc0) ^ vsw) * 16;

    float m_run = NEG_INF, l_run = 0.f;
    f32x4_t oacc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) oacc[db] = f32x4_t{};
    const float c_scale = p.scale_log2;

    auto tile = [&](int it, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int kt = it * BN, stage = it & 1;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (it + 1 < ntiles) issue_tile(kt + BN, stage ^ 1);
        const char* kt_lds = smem + (2 * stage) * C::TILEB + kbase;
        const char* vt_lds = smem + (2 * stage + 1) * C::TILEB + vbase;

        f32x4_t sacc[C::NKB];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
            constexpr int NG = C::NCH / C::KG;
            u32x4_t ka[2][C::KG];
            auto kread = [&](int gi, u32x4_t(&dst)[C::KG]) {
#pragma unroll
                for (int i = 0; i < C::KG; ++i) {
                    const int c = gi * C::KG + i;
                    dst[i] = *reinterpret_cast<const u32x4_t*>(kt_lds + kb * 16 * C::ROWB + (c >> 1) * 128 + kx[c & 1]);
                }
            };
            kread(0, ka[0]);
            f32x4_t s = f32x4_t{};
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                if (gi + 1 < NG) kread(gi + 1, ka[(gi + 1) & 1]);
#pragma unroll
                for (int i = 0; i < C::KG; ++i) s = M16::mma(ka[gi & 1][i], qf[gi * C::KG + i], s);
                __builtin_amdgcn_sched_barrier(0);
            }
            sacc[kb] = s;
        }

        float mtile, c_eff;
        if constexpr (!MASKED) {
            float mx = NEG_INF;
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mtile = mx * c_scale;
            c_eff = c_scale;
        } else {
            mtile = NEG_INF;
            c_eff = 1.f;
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = kt + 16 * kb + 4 * g4 + r;
                    float x = sacc[kb][r] * c_scale;
                    bool ok = j < kend;
                    if constexpr (MASK == MASK_ADD16 || MASK == MASK_ADD32)
                        x = __builtin_fmaf(mask_value<MASK>(mr[kb], r, p.mask_dtype), kLog2e, x);
                    if constexpr (MASK == MASK_CAUSAL) ok = ok && (j <= qi + off);
                    if constexpr (MASK == MASK_BOOL) ok = ok && ((mr[kb] >> (8 * r)) & 0xffu) != 0u;
                    x = ok ? x : NEG_INF;
                    sacc[kb][r] = x;
                    mtile = fmaxf(mtile, x);
                }
            if (it + 1 < ntiles) load_mask(kt + BN);
        }

        mtile = fmaxf(mtile, __shfl_xor(mtile, 16, 64));
        mtile = fmaxf(mtile, __shfl_xor(mtile, 32, 64));
        if (__any(mtile > m_run + kRescale)) {
            const float m_new = fmaxf(m_run, mtile);
            const float alpha = (m_new == NEG_INF) ? 1.f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
            asm volatile("" ::: "memory");
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) oacc[db][r] *= alpha;
        }
        const float muse = (m_run == NEG_INF) ? 0.f : m_run;
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = fast_exp2(__builtin_fmaf(sacc[kb][r], c_eff, -muse));
                sacc[kb][r] = e;
                lsum += e;
            }
        l_run += lsum;
        __builtin_amdgcn_sched_barrier(0);

#pragma unroll
        for (int kp = 0; kp < C::NKP; ++kp) {
            const u32x4_t bf = {TR::pack(sacc[2 * kp][0], sacc[2 * kp][1]), TR::pack(sacc[2 * kp][2], sacc[2 * kp][3]),
                                TR::pack(sacc[2 * kp + 1][0], sacc[2 * kp + 1][1]),
                                TR::pack(sacc[2 * kp + 1][2], sacc[2 * kp + 1][3])};
            const char* vrow_p = vt_lds + kp * 32 * C::ROWB;
            constexpr int NG = C::NDB / C::VG;
            u32x4_t va[2][C::VG];
            auto vread = [&](int gi, u32x4_t(&dst)[C::VG]) {
#pragma unroll
                for (int i = 0; i < C::VG; ++i) {
                    const int db = gi * C::VG + i;
                    const int cofs = (db >> 2) * 128 + vx[db & 3];
                    const u32x2_t y0 = lds_read_tr16(vrow_p + cofs);
                    const u32x2_t y1 = lds_read_tr16(vrow_p + 16 * C::ROWB + cofs);
                    dst[i] = u32x4_t{y0[0], y0[1], y1[0], y1[1]};
                }
            };
            vread(0, va[0]);
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                if (gi + 1 < NG) vread(gi + 1, va[(gi + 1) & 1]);
#pragma unroll
                for (int i = 0; i < C::VG; ++i) {
                    const int db = gi * C::VG + i;
                    oacc[db] = M16::mma(va[gi & 1][i], bf, oacc[db]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    int it = 0;
    if (ntiles > 0) issue_tile(0, 0);
    if constexpr (!HAS_MT) {
        for (; it < nplain; ++it) tile(it, WideTag<false>{});
    }
    if (it < ntiles) load_mask(it * BN);
    for (; it < ntiles; ++it) tile(it, WideTag<true>{});

    float lsum_row = l_run + __shfl_xor(l_run, 16, 64);
    lsum_row += __shfl_xor(lsum_row, 32, 64);
    if (rv) {
        const float inv = lsum_row > 0.f ? 1.f / lsum_row : 0.f;
        char* orow = reinterpret_cast<char*>(p.o) +
                     ((int64_t)b * p.os[0] + (int64_t)qh * p.os[1] + (int64_t)qi * p.os[2]) * 2;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            f32x4_t x = {oacc[db][0] * inv, oacc[db][1] * inv, oacc[db][2] * inv, oacc[db][3] * inv};
            TR::store4(orow + (16 * db + 4 * g4) * 2, x);
        }
    }
}

}  // namespace sdpa_dev
