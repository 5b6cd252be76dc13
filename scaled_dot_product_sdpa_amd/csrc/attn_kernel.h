// Fused attention tile kernel for gfx950 (MI355X), shared by the prefill
// ("full") path and the split-key decode ("vector") path, plus the decode
// combine kernel.
//
// What it computes: O = softmax(scale * Q K^T + M) V per (batch, query head),
// key/value head = query head / n_rep (mlx issue #3885, prefill paragraph:
// scores are [B, n_kv, n_rep, qL, kL]), masks none / additive / boolean /
// causal (mlx PR #4330, "Proposed changes"), the softmax taken over the keys
// (mlx issue #3585, "Reproduction").  Scores are never written to memory:
// each key tile updates a running maximum m, running sum l and the output
// accumulator, rescaled by 2^(m_old - m_new) (online softmax, base-2
// exponent with log2(e) folded into the scale).
//
// Work decomposition (one workgroup):
//   * WM x WD waves; a wave owns 32 query columns (MFMA N axis) and, when
//     WD > 1, one D/WD slice of the head dimension.  With WD > 1 the waves of
//     one column block each contract their slice of Q K^T and sum the
//     partial scores through LDS in a fixed order (so every wave holds the
//     same scores), then each accumulates its own slice of O: the O
//     accumulator of a 512-wide head is spread over 4 waves instead of one.
//   * K/V tiles of BN keys: global -> registers (prefetched one tile ahead)
//     -> LDS.  K is stored row-major [key][d] (+16 B row pad against bank
//     conflicts); V is stored transposed [d][key] so that each lane reads the
//     four consecutive keys its P registers hold at a fixed d.
//   * Head dims that are not a multiple of the MFMA K step (72 = 4.5 x 16)
//     are zero-padded in LDS and in the Q fragments; when D % 32 != 0 the V^T
//     tile has spare rows and row D is set to ones, so the MFMA produces the
//     softmax row sums along with O (already rescaled with it).
//   * Prefill grid: one dimension, NX x ceil(items / NX) workgroups (NX = the
//     device's XCD count), items = (batch, query head, query tile).
//     Workgroup i runs on XCD i % NX, so
//     XCD x is given the contiguous item range [x * per, (x + 1) * per): the
//     query tiles of one head run on one XCD and share its L2 copy of that
//     head's K/V.  Causal items run longest-first and stop at the diagonal
//     (bottom-right aligned).  Decode grid: (key splits, Hkv * column groups,
//     B); a column enumerates (query head in the group, query row), so all
//     n_rep query heads of a key/value head share every K/V byte read.
//   * Softmax per tile: full tiles without a per-element mask take the row
//     max on unscaled scores and need one FMA and one exp2 per score; the
//     output is rescaled only when a row max grows by more than 2^8
//     (otherwise the stale max is kept, so probabilities stay <= 2^8).
#pragma once

#include "attn_common.h"
#include "rope_kernel.h"

namespace sdpa_dev {

template <class TR, int D_, int BN_, int WM_, int WD_, int OCC_ = 1>
struct TileCfg {
    static constexpr int D = D_, BN = BN_, WM = WM_, WD = WD_;
    static constexpr int OCC = OCC_;  // minimum waves per SIMD the register budget must allow
    static constexpr int NW = WM * WD, NT = 64 * NW;
    static constexpr int ES = TR::ES, EPC = TR::EPC, KCH = TR::KCH;
    static constexpr int DW = D / WD;
    static constexpr int NCH = (DW + KCH - 1) / KCH;           // score chunks per wave
    static constexpr int DKP = (WD == 1) ? NCH * KCH : D;      // K tile columns incl. zero pad
    static constexpr int KP = DKP + 16 / ES;                   // K row pitch (elements)
    static constexpr int NDB = (DW + 31) / 32;                 // 32-row O^T blocks per wave
    static constexpr int DVP = (WD == 1) ? NDB * 32 : D;       // V^T rows incl. pad
    static constexpr int VP = BN + 16 / ES;                    // V^T row pitch (elements)
    static constexpr int NKB = BN / 32;                        // 32-key score blocks per tile
    static constexpr bool ONES = (D % 32) != 0;
    static constexpr int KCPR = D / EPC;                       // 16-byte chunks per K/V row
    static constexpr int UK = (BN * KCPR + NT - 1) / NT;       // K chunks per thread per tile
    static constexpr int UV = ((BN / 4) * KCPR + NT - 1) / NT; // V 4-key units per thread per tile
    static constexpr int LDS_K = BN * KP * ES;
    static constexpr int LDS_V = DVP * VP * ES;
    static constexpr int LDS_X = (WD > 1) ? WM * WD * 32 * BN * 4 : 0;
    static constexpr int LDS = LDS_K + LDS_V + LDS_X;
    static_assert(D % WD == 0, "head dim split");
    static_assert(WD == 1 || (DW % 32 == 0 && DW % KCH == 0), "split-D slices must be whole blocks");
    static_assert(D % EPC == 0, "head dim must be a whole number of 16-byte chunks");
    static_assert(BN % 32 == 0, "key tile");
    static_assert(!ONES || WD == 1, "row-sum row needs a spare V^T row");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <class TR> struct OneBits;
template <> struct OneBits<TBF16> { static constexpr uint32_t v = 0x3F80u; };
template <> struct OneBits<TF16> { static constexpr uint32_t v = 0x3C00u; };
template <> struct OneBits<TF32> { static constexpr uint32_t v = 0x3F800000u; };

template <class TR, class C, int MASK, bool DECODE, bool ROPE = false>
__global__ __launch_bounds__(C::NT, C::OCC) void attn_tile_kernel(const Params p) {
    constexpr int ES = C::ES, EPC = C::EPC, KCH = C::KCH, BN = C::BN, D = C::D, DW = C::DW;
    constexpr int BM = 32 * C::WM;
    constexpr float NEG_INF = -__builtin_inff();
    constexpr float kRescale = 8.0f;  // log2 units
    constexpr bool HAS_MT = (MASK == MASK_ADD16 || MASK == MASK_ADD32 || MASK == MASK_BOOL);
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];
    char* const Ks = smem;
    char* const Vt = smem + C::LDS_K;
    float* const X = reinterpret_cast<float*>(smem + C::LDS_K + C::LDS_V);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WD, wd = wave % C::WD;
    const int col = lane & 31, hh = lane >> 5;

    // ---- columns -> (query head, query row); key range of this workgroup ----
    int b, g, qh, qi, split = 0, qmin;
    bool rv;
    int kbeg, kend;
    if constexpr (!DECODE) {
        const int nqt = (p.Lq + BM - 1) / BM;
        const int total = nqt * p.Hq * p.B;
        const int per = (total + p.nx - 1) / p.nx;
        const int item = (int)(blockIdx.x % p.nx) * per + (int)(blockIdx.x / p.nx);
        if (item >= total) return;  // whole workgroup: no barrier is skipped
        const int tt = item % nqt, bh = item / nqt;
        qh = bh % p.Hq;
        b = bh / p.Hq;
        const int t = (MASK == MASK_CAUSAL || MASK == MASK_SLIDE) ? nqt - 1 - tt : tt;
        g = qh / p.n_rep;
        const int i0 = t * BM;
        qmin = i0 + 32 * wm;
        qi = qmin + col;
        rv = qi < p.Lq;
        kbeg = 0;
        kend = p.Lk;
        if (MASK == MASK_CAUSAL || MASK == MASK_SLIDE) {
            const int64_t e = (int64_t)i0 + BM + (p.Lk - p.Lq);
            kend = (int)(e < 0 ? 0 : (e > p.Lk ? p.Lk : e));
        }
        if (MASK == MASK_SLIDE) {  // first tile holding a key row i0 attends
            const int lo = i0 + (p.Lk - p.Lq) - p.window + 1;
            kbeg = min(kend, lo <= 0 ? 0 : (lo / BN) * BN);
        }
    } else {
        b = blockIdx.z;
        split = blockIdx.x;
        g = blockIdx.y / p.col_groups;
        const int cg = blockIdx.y % p.col_groups;
        const int r = cg * BM + 32 * wm + col;
        rv = r < p.n_rep * p.Lq;
        const int rr = rv ? r : 0;
        qh = g * p.n_rep + rr / p.Lq;
        qi = rr % p.Lq;
        qmin = 0;
        kbeg = p.kbase + split * p.keys_per_split;
        kend = min(p.Lk, kbeg + p.keys_per_split);
    }
    const int off = p.Lk - p.Lq;  // bottom-right causal alignment
    const char* const kglob = reinterpret_cast<const char*>(p.k) +
                              ((int64_t)b * p.ks[0] + (int64_t)g * p.ks[1]) * ES;
    const char* const vglob = reinterpret_cast<const char*>(p.v) +
                              ((int64_t)b * p.vs[0] + (int64_t)g * p.vs[1]) * ES;
    const int64_t kstep = (int64_t)p.ks[2] * ES, vstep = (int64_t)p.vs[2] * ES;

    // ---- Q fragments (MFMA B operand), zero beyond D / beyond the rows ----
    u32x4_t qf[C::NCH];
    {
        const char* qrow = reinterpret_cast<const char*>(p.q) +
                           ((int64_t)b * p.qs[0] + (int64_t)qh * p.qs[1] + (int64_t)qi * p.qs[2]) * ES;
#pragma unroll
        for (int ch = 0; ch < C::NCH; ++ch) {
            const int d = wd * DW + ch * KCH + hh * EPC;
            u32x4_t z = {0u, 0u, 0u, 0u};
            qf[ch] = (rv && d < D) ? *reinterpret_cast<const u32x4_t*>(qrow + (int64_t)d * ES) : z;
        }
        if constexpr (ROPE) {  // rotary embedding of the query row (columns < rope_dim), element by element
            if (rv) {
                const int64_t pos = (int64_t)p.rope_pos0 + qi;
#pragma unroll
                for (int ch = 0; ch < C::NCH; ++ch) {
                    const int d = wd * DW + ch * KCH + hh * EPC;
                    if (d < p.rope_dim) rope_fragment_elems<TR>(qf[ch], qrow, d, p.rope_dim, p.rope_cos, p.rope_sin, pos);
                }
            }
        }
    }

    // ---- constant LDS pads: K columns [D, DKP) = 0; V^T rows [D, DVP) = 0 (row D = 1) ----
    if constexpr (C::DKP > D) {
        constexpr int PADC = C::DKP - D;
        for (int idx = tid; idx < BN * PADC; idx += C::NT) {
            const int key = idx / PADC, c = D + idx % PADC;
            if constexpr (ES == 2) reinterpret_cast<uint16_t*>(Ks)[key * C::KP + c] = 0;
            else reinterpret_cast<uint32_t*>(Ks)[key * C::KP + c] = 0;
        }
    }
    if constexpr (C::DVP > D) {
        for (int idx = tid; idx < (C::DVP - D) * BN; idx += C::NT) {
            const int row = D + idx / BN, j = idx % BN;
            const uint32_t val = (C::ONES && row == D) ? OneBits<TR>::v : 0u;
            if constexpr (ES == 2) reinterpret_cast<uint16_t*>(Vt)[row * C::VP + j] = (uint16_t)val;
            else reinterpret_cast<uint32_t*>(Vt)[row * C::VP + j] = val;
        }
    }

    // ---- per-thread load slots: byte offsets from the (batch, kv head) base ----
    // K and V are read through buffer resources that end with the last byte of
    // key kend - 1, so rows past the keys of this workgroup read as zero (the
    // host guarantees row stride >= D whenever there is more than one key).
    const uint32_t kstep32 = (uint32_t)kstep, vstep32 = (uint32_t)vstep;
    const __amdgpu_buffer_rsrc_t krs =
        make_rsrc(kglob, kend > 0 ? (uint32_t)(kend - 1) * kstep32 + (uint32_t)(D * ES) : 0u);
    const __amdgpu_buffer_rsrc_t vrs =
        make_rsrc(vglob, kend > 0 ? (uint32_t)(kend - 1) * vstep32 + (uint32_t)(D * ES) : 0u);
    bool kok[C::UK], vok[C::UV];
    uint32_t koff[C::UK], voff[C::UV];
    int klds[C::UK], vlds[C::UV], vq[C::UV];
#pragma unroll
    for (int u = 0; u < C::UK; ++u) {
        const int idx = tid + u * C::NT;
        const int key = idx / C::KCPR, c = idx % C::KCPR;
        kok[u] = idx < BN * C::KCPR;
        koff[u] = (uint32_t)key * kstep32 + (uint32_t)(c * 16);
        klds[u] = (key * C::KP + c * EPC) * ES;
    }
#pragma unroll
    for (int u = 0; u < C::UV; ++u) {
        const int idx = tid + u * C::NT;
        const int q4 = idx / C::KCPR, c = idx % C::KCPR;
        vok[u] = idx < (BN / 4) * C::KCPR;
        voff[u] = (uint32_t)(4 * q4) * vstep32 + (uint32_t)(c * 16);
        vq[u] = 4 * q4;
        vlds[u] = c * EPC;  // first d of the chunk; LDS row = d, column = 4 * q4
    }

    // mask row of this lane's query (row 0 for padding columns: never used)
    const int64_t mrow = HAS_MT ? (int64_t)b * p.ms[0] + (int64_t)qh * p.ms[1] + (int64_t)(rv ? qi : 0) * p.ms[2] : 0;

    u32x4_t kr[C::UK];
    u32x4_t vr[C::UV][4];
    typename MaskRaw<MASK>::type mr[HAS_MT ? C::NKB : 1][4];
    auto load_mask = [&](int kt) {
        if constexpr (HAS_MT) {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) mr[kb][a4] = load_mask_group<MASK>(p, mrow, kt + kb * 32 + 8 * a4 + 4 * hh);
        }
    };
    auto load_tile = [&](int kt) {
        const uint32_t kb0 = (uint32_t)kt * kstep32, vb0 = (uint32_t)kt * vstep32;
#pragma unroll
        for (int u = 0; u < C::UK; ++u)
            if (kok[u]) kr[u] = buffer_load16(krs, koff[u] + kb0);
#pragma unroll
        for (int u = 0; u < C::UV; ++u)
            if (vok[u]) {
#pragma unroll
                for (int r = 0; r < 4; ++r) vr[u][r] = buffer_load16(vrs, voff[u] + vb0 + (uint32_t)r * vstep32);
            }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int u = 0; u < C::UK; ++u)
            if (kok[u]) *reinterpret_cast<u32x4_t*>(Ks + klds[u]) = kr[u];
#pragma unroll
        for (int u = 0; u < C::UV; ++u) {
            if (!vok[u]) continue;
            const int q0 = vq[u], d0 = vlds[u];
            if constexpr (ES == 2) {
                // 4 keys x 8 d -> 8 rows of V^T, 4 keys (8 bytes) each
#pragma unroll
                for (int w = 0; w < 4; ++w) {
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const uint32_t sel = e ? 0x07060302u : 0x05040100u;
                        const uint32_t lo = __builtin_amdgcn_perm(vr[u][1][w], vr[u][0][w], sel);
                        const uint32_t hi = __builtin_amdgcn_perm(vr[u][3][w], vr[u][2][w], sel);
                        const int d = d0 + 2 * w + e;
                        *reinterpret_cast<u32x2_t*>(Vt + (d * C::VP + q0) * 2) = u32x2_t{lo, hi};
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int d = d0 + i;
                    *reinterpret_cast<u32x4_t*>(Vt + (d * C::VP + q0) * 4) =
                        u32x4_t{vr[u][0][i], vr[u][1][i], vr[u][2][i], vr[u][3][i]};
                }
            }
        }
    };

    float m_run = NEG_INF, l_run = 0.f;
    f32x16_t oacc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) oacc[db] = f32x16_t{};
    const float c_scale = p.scale_log2;

    if (kbeg < kend) {
        load_tile(kbeg);
        load_mask(kbeg);
    }
    for (int kt = kbeg; kt < kend; kt += BN) {
        __syncthreads();  // every wave is done reading the previous tile
        store_tile();
        __syncthreads();
        if (kt + BN < kend) load_tile(kt + BN);  // next tile in flight during this one

        // ---- S^T = K Q^T over this wave's slice of d ----
        f32x16_t sacc[C::NKB];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
            sacc[kb] = f32x16_t{};
#pragma unroll
            for (int ch = 0; ch < C::NCH; ++ch) {
                const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
                    Ks + ((kb * 32 + col) * C::KP + wd * DW + ch * KCH + hh * EPC) * ES);
                sacc[kb] = TR::mma(a, qf[ch], sacc[kb]);
            }
        }
        if constexpr (C::WD > 1) {
            float* const mine = X + (wm * C::WD + wd) * 32 * BN;
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mine[(kb * 16 + r) * 64 + lane] = sacc[kb][r];
            __syncthreads();
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float s = 0.f;
#pragma unroll
                    for (int w = 0; w < C::WD; ++w) s += X[(wm * C::WD + w) * 32 * BN + (kb * 16 + r) * 64 + lane];
                    sacc[kb][r] = s;
                }
        }

        // ---- tile max; per-element masking only where needed (wave-uniform test) ----
        const bool plain = !HAS_MT && p.scale_nonneg && (kt + BN <= kend) &&
                           (MASK != MASK_CAUSAL || kt + BN - 1 <= qmin + off) &&
                           (MASK != MASK_SLIDE ||
                            (!DECODE && kt + BN - 1 <= qmin + off && kt > min(qmin + 31, p.Lq - 1) + off - p.window));
        float mtile = NEG_INF;
        float c_eff;
        if (plain) {
            float mx = NEG_INF;
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mtile = mx * c_scale;
            c_eff = c_scale;
        } else {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = kt + kb * 32 + 8 * a4 + 4 * hh + r;
                        float x = sacc[kb][4 * a4 + r] * c_scale;
                        bool ok = j < kend;
                        if constexpr (MASK == MASK_ADD16 || MASK == MASK_ADD32)
                            x = __builtin_fmaf(mask_value<MASK>(mr[kb][a4], r, p.mask_dtype), kLog2e, x);
                        if constexpr (MASK == MASK_CAUSAL) ok = ok && (j <= qi + off);
                        if constexpr (MASK == MASK_SLIDE) ok = ok && in_window(j, qi + off, p.window);
                        if constexpr (MASK == MASK_BOOL) ok = ok && ((mr[kb][a4] >> (8 * r)) & 0xffu) != 0u;
                        x = ok ? x : NEG_INF;
                        sacc[kb][4 * a4 + r] = x;
                        mtile = fmaxf(mtile, x);
                    }
                }
            }
            c_eff = 1.f;
        }
        mtile = fmaxf(mtile, xor32(mtile));
        if (kt + BN < kend) load_mask(kt + BN);  // this tile's mask is consumed

        // ---- online softmax: rescale only when some row max grows by > 2^8 ----
        if (__any(mtile > m_run + kRescale)) {
            const float m_new = fmaxf(m_run, mtile);
            const float alpha = (m_new == NEG_INF) ? 1.f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
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
        if constexpr (!C::ONES) l_run += lsum;

        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
            for (int pc = 0; pc < 32 / KCH; ++pc) {
                u32x4_t bf;
                if constexpr (ES == 2) {
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        bf[w] = TR::pack(sacc[kb][8 * pc + 2 * w], sacc[kb][8 * pc + 2 * w + 1]);
                } else {
#pragma unroll
                    for (int w = 0; w < 4; ++w) bf[w] = __float_as_uint(sacc[kb][4 * pc + w]);
                }
#pragma unroll
                for (int db = 0; db < C::NDB; ++db) {
                    const int d = wd * DW + 32 * db + col;
                    u32x4_t af;
                    if constexpr (ES == 2) {
                        const u32x2_t x0 = *reinterpret_cast<const u32x2_t*>(
                            Vt + (d * C::VP + kb * 32 + 16 * pc + 4 * hh) * 2);
                        const u32x2_t x1 = *reinterpret_cast<const u32x2_t*>(
                            Vt + (d * C::VP + kb * 32 + 16 * pc + 8 + 4 * hh) * 2);
                        af = u32x4_t{x0[0], x0[1], x1[0], x1[1]};
                    } else {
                        af = *reinterpret_cast<const u32x4_t*>(Vt + (d * C::VP + kb * 32 + 8 * pc + 4 * hh) * 4);
                    }
                    oacc[db] = TR::mma(af, bf, oacc[db]);
                }
            }
        }
    }

    // ---- epilogue ----
    float lsum_row;
    if constexpr (C::ONES) {
        constexpr int rr = D % 32;
        constexpr int RL = 4 * (rr / 8) + (rr % 4), HL = (rr % 8) / 4, DBL = D / 32;
        const float x = oacc[DBL][RL];
        const float y = xor32(x);
        lsum_row = (hh == HL) ? x : y;
    } else {
        lsum_row = l_run + xor32(l_run);
    }
    if constexpr (!DECODE) {
        if (rv) {
            const float inv = lsum_row > 0.f ? 1.f / lsum_row : 0.f;
            char* orow = reinterpret_cast<char*>(p.o) +
                         ((int64_t)b * p.os[0] + (int64_t)qh * p.os[1] + (int64_t)qi * p.os[2]) * ES;
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int d0 = wd * DW + 32 * db + 8 * a4 + 4 * hh;
                    if (d0 < D) {
                        f32x4_t x = {oacc[db][4 * a4] * inv, oacc[db][4 * a4 + 1] * inv,
                                     oacc[db][4 * a4 + 2] * inv, oacc[db][4 * a4 + 3] * inv};
                        TR::store4(orow + (int64_t)d0 * ES, x);
                    }
                }
        }
    } else {
        if (rv) {
            const int64_t row = ((int64_t)b * p.Hq + qh) * p.Lq + qi;
            float* po = p.ws_o + (row * p.splits + split) * D;
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int d0 = wd * DW + 32 * db + 8 * a4 + 4 * hh;
                    if (d0 < D)
                        *reinterpret_cast<f32x4_t*>(po + d0) =
                            f32x4_t{oacc[db][4 * a4], oacc[db][4 * a4 + 1], oacc[db][4 * a4 + 2], oacc[db][4 * a4 + 3]};
                }
            if (wd == 0 && hh == 0) {
                p.ws_ml[(row * p.splits + split) * 2 + 0] = m_run;
                p.ws_ml[(row * p.splits + split) * 2 + 1] = lsum_row;
            }
        }
    }
}

// Decode combine: O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s, by one
// wave per (output row, 64-wide slice of d), with no cross-wave step: lane l
// takes float4 column group l % 16 and split phase l / 16 (splits
// s = 4 i + l / 16 of each pass of 64), so the first pass's partial loads are
// all in flight at once.  The (m, l) pairs go through LDS once (max, then the
// weights, stored phase-major so each lane reads its 16 weights as four
// 16-byte reads); the four phases are summed by lane swaps in a fixed order
// (deterministic).  grid = (B*Hq*Lq, ceil(D/64)), 64 threads.
constexpr int kMaxSplits = 1024;

template <class TR, int D>
__global__ __launch_bounds__(64) void combine_kernel(const Params p) {
    constexpr float NEG_INF = -__builtin_inff();
    __shared__ __attribute__((aligned(16))) float msh[kMaxSplits], lsh[kMaxSplits], wts[kMaxSplits];
    const int64_t row = blockIdx.x;
    const int lane = threadIdx.x;
    const int S = p.splits, NPASS = (S + 63) / 64;
    const int cgp = lane & 15, ph = lane >> 4;
    const int d = blockIdx.y * 64 + 4 * cgp;
    const bool dv = d < D;
    const float* po = p.ws_o + row * S * D + d;
    const float* ml = p.ws_ml + row * S * 2;
    // the first pass's partial loads go out before anything depends on them
    f32x4_t v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int s = 4 * i + ph;
        v[i] = (dv && s < S) ? *reinterpret_cast<const f32x4_t*>(po + (int64_t)s * D) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    float M = NEG_INF;
    for (int k = 0; k < NPASS; ++k) {
        const int s = 64 * k + lane;
        const float m = s < S ? ml[2 * s] : NEG_INF, l = s < S ? ml[2 * s + 1] : 0.f;
        msh[s] = m;
        lsh[s] = l;
        M = fmaxf(M, m);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    M = max_x32(max_x16(M));
    float den = 0.f;
    for (int k = 0; k < NPASS; ++k) {
        const int s = 64 * k + lane;
        const float m = msh[s];
        const float w = (m == NEG_INF || M == NEG_INF) ? 0.f : fast_exp2(m - M);
        den = __builtin_fmaf(w, lsh[s], den);
        wts[64 * k + 16 * (lane & 3) + (lane >> 2)] = w;  // phase-major within the pass
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) den += __shfl_xor(den, o, 64);
    den = sum_x32(sum_x16(den));
    __syncthreads();  // one wave: orders the weight stores before the reads
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < NPASS; ++k) {
        if (k > 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int s = 64 * k + 4 * i + ph;
                v[i] = (dv && s < S) ? *reinterpret_cast<const f32x4_t*>(po + (int64_t)s * D)
                                     : f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
        const f32x4_t* wp = reinterpret_cast<const f32x4_t*>(wts + 64 * k + 16 * ph);
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4_t w4 = wp[i4];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc += w4[j] * v[4 * i4 + j];
        }
    }
    // the 4 split phases of a column group: lanes l, l ^ 16, l ^ 32, l ^ 48
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = sum_x32(sum_x16(acc[k]));
    if (ph != 0 || !dv) return;
    const float inv = (M != NEG_INF && den > 0.f) ? 1.f / den : 0.f;
    const int qi = (int)(row % p.Lq);
    const int64_t bh = row / p.Lq;
    const int qh = (int)(bh % p.Hq), b = (int)(bh / p.Hq);
    char* dst = reinterpret_cast<char*>(p.o) +
                ((int64_t)b * p.os[0] + (int64_t)qh * p.os[1] + (int64_t)qi * p.os[2] + d) * TR::ES;
    TR::store4(dst, acc * inv);
}

}  // namespace sdpa_dev
