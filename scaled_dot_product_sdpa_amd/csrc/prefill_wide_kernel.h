// Prefill ("full") kernel for 16-bit inputs and wide heads (D = 256, 512) on gfx950.
//
// At D = 512 a 32-row query block would need 32 x 512 fp32 accumulators (256
// registers per lane) plus 128 for Q: more than fits next to everything else.
// Each wave therefore takes 16 query rows (v_mfma_f32_16x16x32): O^T is 128
// registers per lane and Q^T 64, so two waves fit per SIMD, and every wave
// contracts the full head dim for its own scores (no partial scores cross
// waves):
//   * a workgroup is 8 waves = 8 (query head, 16-row block) pairs of ONE
//     key/value head: the query heads of a grouped-query group (mlx issue
//     #3885, prefill paragraph: scores [B, n_kv, n_rep, qL, kL]) share every
//     K/V tile loaded into LDS (up to 8 heads per workgroup; with fewer heads
//     in the group the spare waves take further row blocks of the same head);
//   * K/V tiles of BN keys go global -> LDS with buffer_load ... lds, double
//     buffered, one barrier per tile.  LDS rows are unpadded; the 16-byte
//     chunks of row r sit at chunk ^ sw(r) (sw a bijection on r mod 16), which
//     keeps the transposed 64-bit V reads free of bank conflicts;
//   * S^T = K Q^T with K from LDS and Q from registers, online softmax in
//     base 2 with lazy rescale, O^T += V^T P^T with V^T read from the
//     row-major V tile through ds_read_b64_tr_b16;
//   * LDS reads are software-pipelined one group ahead of the MFMAs that use
//     them; scheduling barriers bound how far the compiler may hoist them,
//     which is what keeps the kernel inside the register file.
#pragma once

#include "attn_common.h"
#include "rope_kernel.h"

namespace sdpa_dev {

// Row -> chunk swizzle (XOR on the 16-byte chunk index mod 16).  gfx950's LDS
// serves a 64-bit read 32 lanes at a time, 256 bytes (64 banks) per pass; the
// transposed V reads of a pass cover 8 rows x 2 consecutive chunks.  sw is a
// bijection on r mod 16 whose values for rows 0..7 (and 8..15) differ in bits
// 1-3, so those 8 chunk pairs land on distinct banks; the 128-bit K reads
// (16 consecutive rows, one chunk each) get 16 distinct slots.
__device__ __forceinline__ int wide_sw16(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

template <bool B> struct WideTag { static constexpr bool value = B; };

// Operand layouts (16x16x32):
//   S^T block (16 keys x 16 queries) = K (16 x 32 of D) Q^T, D / 32 steps;
//   lane l holds query l % 16 against keys 4 * (l / 16) + i, i = 0..3.
//   O^T block (16 of D x 16 queries) += V^T (16 x 32 keys) P^T: the B operand
//   slot 8 * (l / 16) + j is key 4 * (l / 16) + j of the first 16-key block
//   (j < 4) or of the second (j >= 4) -- exactly the scores lane l holds --
//   and the A operand takes the same keys from two transposed LDS reads.
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
    static constexpr int SWP = (RSTEP % 16 == 0) ? 1 : 16 / RSTEP;
    static constexpr int KG = 2;                 // K chunks per pipelined group
    static constexpr int VG = 2;                 // O^T blocks per pipelined group
    static constexpr int LDS = 4 * TILEB;
    static_assert(D % 32 == 0 && KC <= 64, "head dim");
    static_assert(BN % 32 == 0 && (BN * KC) % (64 * NW) == 0, "key tile");
    static_assert(16 % RSTEP == 0 || RSTEP % 16 == 0, "swizzle period");
    static_assert(NCH % KG == 0 && NDB % VG == 0, "pipeline groups");
    static_assert(NW == 8 || NW == 4, "waves per workgroup");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <class TR, class C, int MASK, bool ROPE = false>
__global__ __launch_bounds__(C::NT, 1) void prefill_r16_kernel(const Params p) {
    constexpr int D = C::D, BN = C::BN, NW = C::NW;
    constexpr float NEG_INF = -__builtin_inff();
    constexpr float kRescale = 8.0f;
    constexpr bool HAS_MT = (MASK == MASK_ADD16 || MASK == MASK_ADD32 || MASK == MASK_BOOL);
    // masked variants carry mask registers across the tile: pipeline one read ahead only
    constexpr int KGk = HAS_MT ? 1 : C::KG, VGk = HAS_MT ? 1 : C::VG;
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
    // with a mask tensor the head groups of one row tile run next to each other
    // (mask rows shared through L2), otherwise the row tiles of one group do
    int tt, hgi, g, b;
    if constexpr (HAS_MT) {
        hgi = item % nhg;
        int rest = item / nhg;
        g = rest % p.Hkv;
        rest /= p.Hkv;
        tt = rest % nrt;
        b = rest / nrt;
    } else {
        tt = item % nrt;
        int rest = item / nrt;
        hgi = rest % nhg;
        rest /= nhg;
        g = rest % p.Hkv;
        b = rest / p.Hkv;
    }
    constexpr bool CAUSAL_END = (MASK == MASK_CAUSAL || MASK == MASK_SLIDE);
    const int t = CAUSAL_END ? nrt - 1 - tt : tt;  // heavy row tiles first
    const int i0 = t * BMW;
    const int qh = g * n_rep + hgi * HG + (w % HG);
    const int qmin = i0 + 16 * (w / HG);
    const int qi = qmin + c16;
    const bool rv = qi < p.Lq;
    const int off = p.Lk - p.Lq;
    int kend = p.Lk;
    if (CAUSAL_END) {
        const int64_t e = (int64_t)i0 + BMW + off;
        kend = (int)(e < 0 ? 0 : (e > p.Lk ? p.Lk : e));
    }
    const int ntiles = (kend + BN - 1) / BN;
    // key tiles [t0, ntiles) hold every key some row of this workgroup attends;
    // tiles [tp0, tp1) need no per-element mask for any row of this wave
    int t0 = 0;
    if (MASK == MASK_SLIDE) t0 = min(ntiles, max(0, i0 + off - p.window + 1) / BN);
    int tp0 = t0, tp1 = kend / BN;
    if (CAUSAL_END) tp1 = min(tp1, max(0, qmin + off + 1) / BN);
    if (MASK == MASK_SLIDE) {
        const int lo = min(qmin + 15, p.Lq - 1) + off - p.window + 1;  // window's left edge, wave's last row
        tp0 = max(t0, lo <= 0 ? 0 : (lo + BN - 1) / BN);
    }
    if (HAS_MT || !p.scale_nonneg) tp1 = tp0;
    tp0 = min(tp0, ntiles);
    tp1 = max(tp0, min(tp1, ntiles));

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
            qf[c] = *reinterpret_cast<const u32x4_t*>(qrow + (32 * c + 8 * g4) * 2);  // rows >= Lq read row 0, never stored
        if constexpr (ROPE)  // rotary embedding of the query row (columns < rope_dim)
            rope_q_fragments<TR, C::NCH, 32>(qf, qrow, 8 * g4, p.rope_dim, p.rope_cos, p.rope_sin,
                                             (int64_t)p.rope_pos0 + (rv ? qi : 0));
    }

    const int rl = w * C::RPI + lane / C::KC;
    uint32_t kv0[C::SWP], vv0[C::SWP];
#pragma unroll
    for (int ph = 0; ph < C::SWP; ++ph) {
        const int row = rl + ph * C::RSTEP;
        const uint32_t cb = (uint32_t)(((lane % C::KC) ^ wide_sw16(row)) * 16);
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
    // (4 c + g4) ^ ksw = 16 (c >> 2) + ((4 (c & 3) + g4) ^ ksw); (2 db + vc0) ^ vsw =
    // 16 (db >> 3) + ((2 (db & 7) + vc0) ^ vsw): a few per-lane values, the rest immediate
    // (rows 16 apart share a swizzle, so both transposed reads use the same offsets)
    const int ksw = wide_sw16(c16);
    const int kbase = c16 * C::ROWB;
    int kx[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) kx[m] = ((4 * m + g4) ^ ksw) * 16;
    const int e4 = (lane >> 2) & 3, j4 = lane & 3;
    const int vsw = wide_sw16(4 * g4 + e4);
    // (2 m + vc0) ^ vsw = (2 m ^ (vsw & 14)) + ((vc0 ^ vsw) & 1), vc0 = j4 >> 1: one XOR
    // per read pair, no offset table
    const int vbase = (4 * g4 + e4) * C::ROWB + 8 * (j4 & 1) + (((j4 >> 1) ^ vsw) & 1) * 16;
    const int vxm = (vsw & 14) * 16;

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
        // this tile's mask values: issued before the next tile's loads, so waiting
        // for them never waits for the prefetch (and no registers carry them across tiles)
        if constexpr (MASKED) load_mask(kt);
        if (it + 1 < ntiles) issue_tile(kt + BN, stage ^ 1);
        const char* kt_lds = smem + (2 * stage) * C::TILEB + kbase;
        const char* vt_lds = smem + (2 * stage + 1) * C::TILEB + vbase;

        f32x4_t sacc[C::NKB];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
            constexpr int NG = C::NCH / KGk;
            u32x4_t ka[2][KGk];
            auto kread = [&](int gi, u32x4_t(&dst)[KGk]) {
#pragma unroll
                for (int i = 0; i < KGk; ++i) {
                    const int c = gi * KGk + i;
                    dst[i] = *reinterpret_cast<const u32x4_t*>(kt_lds + kb * 16 * C::ROWB + (c >> 2) * 256 + kx[c & 3]);
                }
            };
            kread(0, ka[0]);
            f32x4_t s = f32x4_t{};
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                if (gi + 1 < NG) kread(gi + 1, ka[(gi + 1) & 1]);
#pragma unroll
                for (int i = 0; i < KGk; ++i) s = M16::mma(ka[gi & 1][i], qf[gi * KGk + i], s);
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
                    if constexpr (MASK == MASK_SLIDE) ok = ok && in_window(j, qi + off, p.window);
                    if constexpr (MASK == MASK_BOOL) ok = ok && ((mr[kb] >> (8 * r)) & 0xffu) != 0u;
                    x = ok ? x : NEG_INF;
                    sacc[kb][r] = x;
                    mtile = fmaxf(mtile, x);
                }
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
            constexpr int NG = C::NDB / VGk;
            u32x4_t va[2][VGk];
            auto vread = [&](int gi, u32x4_t(&dst)[VGk]) {
#pragma unroll
                for (int i = 0; i < VGk; ++i) {
                    const int db = gi * VGk + i;
                    const int cofs = (db >> 3) * 256 + ((32 * (db & 7)) ^ vxm);
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
                for (int i = 0; i < VGk; ++i) {
                    const int db = gi * VGk + i;
                    oacc[db] = M16::mma(va[gi & 1][i], bf, oacc[db]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    int it = t0;
    if (it < ntiles) issue_tile(it * BN, it & 1);
    if constexpr (!HAS_MT) {
        for (; it < tp0; ++it) tile(it, WideTag<true>{});
        for (; it < tp1; ++it) tile(it, WideTag<false>{});
    }
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
