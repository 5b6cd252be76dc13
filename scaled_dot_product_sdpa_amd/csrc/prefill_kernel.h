// Prefill ("full") kernel for 16-bit inputs and head dims up to 128 on gfx950.
//
// Same mathematics and work split as attn_tile_kernel (S^T = K Q^T and
// O^T = V^T P^T on v_mfma_f32_32x32x16, 32 query columns per wave, online
// softmax in base 2, XCD-aware longest-first grid), with the data path
// rebuilt around two gfx950 features:
//   * K and V tiles move global -> LDS with buffer_load_dwordx4 ... lds: each
//     lane of a load writes its 16 bytes at LDS base + 16 * lane, and the
//     global chunk a lane fetches decides the layout.  A tile is stored
//     row-major.  Below D = 128 a row holds KC + 1 sixteen-byte chunks
//     (KC = D / 8); the extra chunk is never loaded: it staggers rows over the
//     LDS banks and holds constants (zeros for K; for V, a one at column D
//     when D is not a multiple of 32, so the P V product also yields the
//     softmax row sums).  At D = 128 rows are 256 bytes with chunk c of row r
//     in slot c ^ sw(r), which puts a 128-bit K read pass (16 lanes: 16
//     consecutive rows, one chunk) and a transposed 64-bit V read pass (32
//     lanes: 4 consecutive rows, 4 consecutive chunks) on 64 distinct banks.
//     Two stages are double-buffered: the loads of tile t + 1 fly during Q K^T
//     and the softmax of tile t, with one barrier per tile.  (hipcc waits for
//     them before tile t's first transposed V read, which it cannot tell apart
//     from the stage being loaded; one LDS array per stage would avoid that,
//     but the two loop bodies it needs cost an occupancy step.)
//   * The A operand of P V (V^T: one head-dim column, eight keys per lane)
//     comes straight from the row-major V tile through ds_read_b64_tr_b16:
//     in each 16-lane group, source lane 4 e + j names the 4 columns
//     4 j .. 4 j + 3 of key e, and output lane i receives column i of keys
//     0..3; two reads give the eight keys a lane's P registers hold.
// Tiles with no per-element mask (full, unmasked, left of the causal
// diagonal) run a separate loop from masked ones, so neither pays for the
// other's code.
#pragma once

#include "attn_common.h"
#include "rope_kernel.h"

namespace sdpa_dev {

template <class TR, int D_, int BN_, int WM_, int OCC_>
struct PfCfg {
    static constexpr int D = D_, BN = BN_, WM = WM_, OCC = OCC_;
    static constexpr int NT = 64 * WM, BM = 32 * WM;
    static constexpr int KC = D / 8;                  // 16-byte chunks per row
    static constexpr bool SWZ = (KC == 16);           // swizzled 256-byte rows, no spare chunk
    static constexpr int RC = SWZ ? KC : KC + 1;      // 16-byte slots per LDS row
    static constexpr int ROWB = RC * 16;              // bytes per LDS row
    static constexpr int TILEB = BN * ROWB;           // bytes per K or V tile
    static constexpr int NCH = (D + 15) / 16;         // Q K^T chunks (16 head-dim columns)
    static constexpr int NDB = (D + 31) / 32;         // 32-column O^T blocks
    static constexpr int NKB = BN / 32;               // 32-key score blocks per tile
    static constexpr bool ONES = (D % 32) != 0;
    // REM: the last O^T columns (the D % 32 real ones, then the row-sum column)
    // fit 16 columns, which take v_mfma_f32_16x16x32 products instead of a third
    // of a 32-column block (head dim 72: 80 O^T columns, not 96)
    static constexpr bool REM = ONES && (D % 32) < 16;
    static constexpr int NDF = REM ? D / 32 : NDB;    // 32-column O^T blocks on 32x32x16 products
    static constexpr int LA = 3;                      // operand reads in flight ahead of the MFMAs
    static constexpr bool PAIRS = true;               // causal: two row tiles per workgroup (see the kernel)
    static constexpr int SLOTS = BN * RC;             // 16-byte slots per tile
    static constexpr int NLD = (SLOTS + NT - 1) / NT; // load instructions per thread per tile (K or V)
    // V0, K0, V1, K1: transposed V reads of a tile's last row may run up to 32
    // bytes past it (head-dim columns beyond D, never stored), into the K tile
    // after it, so the block needs no padding (head dim 72: 40 KiB, a quarter
    // of a CU's LDS).
    static constexpr int LDS = 4 * TILEB;
    static constexpr int KOFF0 = TILEB, VOFF0 = 0;    // stage s: + 2 s TILEB
    static_assert(D % 8 == 0 && D <= 128, "head dim");
    static_assert(BN % 32 == 0, "key tile");
    static_assert(!ONES || (D % 32) <= 16, "ones column must sit in the spare chunk");
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(!SWZ || !ONES, "swizzled rows have no spare chunk");
    // slot of chunk c in row r: a bijection of 16 consecutive rows onto the 16
    // slots, and 4 consecutive rows on the 4 groups of 4 slots (64 bytes)
    static __device__ __forceinline__ int sw(int r) {
        if constexpr (SWZ) return ((r & 3) << 2) | ((r >> 2) & 3);
        else return 0;
    }
};

template <bool B> struct PfTag { static constexpr bool value = B; };

// SMASK: the mask tensor's keys are not 4-element aligned runs (mask_vec == 0);
// its elements are loaded one by one.
// BITS (MASK_BOOL only): the mask comes as precomputed lane masks (mask_bits.h,
// Params::mask_bits), one v_cndmask per score and no mask-tensor loads.
template <class TR, class C, int MASK, bool ROPE = false, bool SMASK = false, bool BITS = false>
__global__ __launch_bounds__(C::NT, C::OCC) void prefill_kernel(const Params p) {
    constexpr int D = C::D, BN = C::BN, BM = C::BM;
    constexpr float NEG_INF = -__builtin_inff();
    constexpr float kRescale = 8.0f;
    constexpr bool HAS_MT = (MASK == MASK_ADD16 || MASK == MASK_ADD32 || MASK == MASK_BOOL);
    constexpr bool LOADS = HAS_MT && !BITS;  // mask-tensor elements loaded by the kernel
    static_assert(!BITS || (MASK == MASK_BOOL && !SMASK && C::BN == 64), "lane masks: boolean, 64-key tiles");
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];
    const uint32_t smem_lds = lds_address(smem);

    const int tid = threadIdx.x, lane = tid & 63, wm = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, hh = lane >> 5;

    // ---- work item (XCD-aware, longest causal tiles first) ----
    const bool pairs = C::PAIRS && MASK == MASK_CAUSAL && p.pairs;  // the host's choice, uniform
    const int nqt = (p.Lq + BM - 1) / BM;
    const int nit = pairs ? (nqt + 1) / 2 : nqt;  // row-tile items per head
    const int total = nit * p.Hq * p.B;
    const int per = (total + p.nx - 1) / p.nx;
    const int item = (int)(blockIdx.x % p.nx) * per + (int)(blockIdx.x / p.nx);
    if (item >= total) return;
    // With mask-tensor bytes, the heads of one row tile run next to each other on
    // one XCD so its mask rows (usually shared by every head) are read from L2;
    // otherwise (lane words too: an eighth of the bytes) the row tiles of one head
    // do, sharing K and V.  (D = 72 boolean, 16 heads x 8192: the heads-together
    // order with lane words missed L2 for 1.19 GB per launch against 0.11 GB.)
    int tt, qh, b;
    if constexpr (LOADS) {
        qh = item % p.Hq;
        const int r = item / p.Hq;
        tt = r % nqt;
        b = r / nqt;
    } else {
        tt = item % nit;
        const int bh = item / nit;
        qh = bh % p.Hq;
        b = bh / p.Hq;
    }
    constexpr bool CAUSAL_END = (MASK == MASK_CAUSAL || MASK == MASK_SLIDE);
    // the row tiles of one workgroup: one, or with pairs (causal) two whose
    // key ranges add up to the same length for every workgroup (t and nqt - 1 - t),
    // so no single long row tile outlasts the rest of the grid (the host pairs
    // only grids that still give every CU a workgroup)
    auto run = [&](const int t) __attribute__((always_inline)) {
        const int g = qh / p.n_rep;
        const int i0 = t * BM;
        const int qmin = i0 + 32 * wm;  // first query row of this wave
        const int qi = qmin + col;
        const bool rv = qi < p.Lq;
        const int off = p.Lk - p.Lq;
        int kend = p.Lk;
        if (CAUSAL_END) {
            const int64_t e = (int64_t)i0 + BM + off;
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
            const int lo = min(qmin + 31, p.Lq - 1) + off - p.window + 1;  // window's left edge, wave's last row
            tp0 = max(t0, lo <= 0 ? 0 : (lo + BN - 1) / BN);
        }
        if (HAS_MT) tp1 = tp0;
        tp0 = min(tp0, ntiles);
        tp1 = max(tp0, min(tp1, ntiles));

        // ---- buffer resources over this (batch, kv head)'s K and V rows ----
        const int64_t kstep = (int64_t)p.ks[2] * 2, vstep = (int64_t)p.vs[2] * 2;
        const char* kglob = reinterpret_cast<const char*>(p.k) + ((int64_t)b * p.ks[0] + (int64_t)g * p.ks[1]) * 2;
        const char* vglob = reinterpret_cast<const char*>(p.v) + ((int64_t)b * p.vs[0] + (int64_t)g * p.vs[1]) * 2;
        const uint32_t kstep32 = (uint32_t)kstep, vstep32 = (uint32_t)vstep;
        const __amdgpu_buffer_rsrc_t krs =
            make_rsrc(kglob, kend > 0 ? (uint32_t)(kend - 1) * kstep32 + (uint32_t)(D * 2) : 0u);
        const __amdgpu_buffer_rsrc_t vrs =
            make_rsrc(vglob, kend > 0 ? (uint32_t)(kend - 1) * vstep32 + (uint32_t)(D * 2) : 0u);

        // ---- Q fragments (MFMA B operand), zero beyond D / beyond the rows ----
        u32x4_t qf[C::NCH];
        {
            const char* qrow = reinterpret_cast<const char*>(p.q) +
                               ((int64_t)b * p.qs[0] + (int64_t)qh * p.qs[1] + (int64_t)qi * p.qs[2]) * 2;
    #pragma unroll
            for (int ch = 0; ch < C::NCH; ++ch) {
                const int d = ch * 16 + hh * 8;
                qf[ch] = (rv && d < D) ? *reinterpret_cast<const u32x4_t*>(qrow + d * 2) : u32x4_t{0u, 0u, 0u, 0u};
            }
            if constexpr (ROPE) {  // rotary embedding of the query row (columns < rope_dim)
                if (rv)
                    rope_q_fragments<TR, C::NCH, 16>(qf, qrow, hh * 8, p.rope_dim, p.rope_cos, p.rope_sin,
                                                     (int64_t)p.rope_pos0 + qi);
            }
            // a negative scale runs as |scale| on -Q (exact: a sign flip) and a zero
            // scale as scale 1 on Q = 0 (every score is 0 either way), so the scale
            // is positive and the row max can always be taken on unscaled scores
            if (p.scale_log2 < 0.f) {
    #pragma unroll
                for (int ch = 0; ch < C::NCH; ++ch) qf[ch] ^= 0x80008000u;
            } else if (p.scale_log2 == 0.f) {
    #pragma unroll
                for (int ch = 0; ch < C::NCH; ++ch) qf[ch] = u32x4_t{0u, 0u, 0u, 0u};
            }
        }

        // ---- spare chunks: K rows 0, V rows (1 at column D if ONES, else 0) ----
        if constexpr (!C::SWZ)
        for (int r = tid; r < 4 * BN; r += C::NT) {
            const int tile = r / BN, row = r % BN;  // tiles V0, K0, V1, K1
            const bool is_v = !(tile & 1);
            u32x4_t z = {0u, 0u, 0u, 0u};
            if (is_v && C::ONES) z[0] = OneBits<TR>::v;
            *reinterpret_cast<u32x4_t*>(smem + tile * C::TILEB + row * C::ROWB + C::KC * 16) = z;
        }

        // ---- load slots: lane slot s -> (row, chunk); a spare chunk is never loaded ----
        uint32_t kofs[C::NLD], vofs[C::NLD];
        bool sok[C::NLD];
    #pragma unroll
        for (int u = 0; u < C::NLD; ++u) {
            const int s = (u * C::WM + wm) * 64 + lane;  // this lane's 16-byte slot of the tile
            const int row = s / C::RC, ch = (s % C::RC) ^ C::sw(row);
            sok[u] = (s < C::SLOTS) && (ch < C::KC);
            kofs[u] = (uint32_t)row * kstep32 + (uint32_t)(ch * 16);
            vofs[u] = (uint32_t)row * vstep32 + (uint32_t)(ch * 16);
        }
        auto issue_tile = [&](int kt, int stage) {
            const uint32_t kt_lds = smem_lds + (uint32_t)(2 * stage * C::TILEB + C::KOFF0);
            const uint32_t vt_lds = smem_lds + (uint32_t)(2 * stage * C::TILEB + C::VOFF0);
            const uint32_t kb0 = (uint32_t)kt * kstep32, vb0 = (uint32_t)kt * vstep32;
    #pragma unroll
            for (int u = 0; u < C::NLD; ++u) {
                const int blk = (u * C::WM + wm) * 64 * 16;  // LDS byte offset of this instruction's 64 slots
                if (blk >= C::SLOTS * 16) break;
                if (sok[u]) {
                    dma16_lds(krs, kt_lds + (uint32_t)blk, kofs[u] + kb0);
                    dma16_lds(vrs, vt_lds + (uint32_t)blk, vofs[u] + vb0);
                }
            }
        };

        // mask rows: rows past Lq read row Lq - 1 (never stored).  One buffer
        // resource per wave starts at the wave's first row and ends at the mask's
        // last byte (32-bit element offsets within it: checked on the host), so
        // every group is one branch-free vector load (or four scalar ones).
        constexpr int MES = MASK == MASK_BOOL ? 1 : (MASK == MASK_ADD16 ? 2 : 4);
        const int q0c = min(qmin, p.Lq - 1), qic = min(qi, p.Lq - 1);
        const int64_t mbase = LOADS ? (int64_t)b * p.ms[0] + (int64_t)qh * p.ms[1] + (int64_t)q0c * p.ms[2] : 0;
        const uint32_t mlane = LOADS ? (uint32_t)((qic - q0c) * p.ms[2]) : 0u;
        const int64_t mleft = LOADS ? p.mask_span - mbase * MES : 0;
        const __amdgpu_buffer_rsrc_t mrs =
            make_rsrc(LOADS ? reinterpret_cast<const char*>(p.mask) + mbase * MES : nullptr,
                      (uint32_t)(mleft > 0xffffffffLL ? 0xffffffffLL : mleft));
        typename MaskRaw<MASK>::type mr[LOADS ? C::NKB : 1][4];
        // lane words of this wave's 32-row block (BITS): 64 per key tile, one per lane,
        // loaded a tile ahead like the mask bytes
        uint32_t mw = 0;
        const __amdgpu_buffer_rsrc_t wrs =
            make_rsrc(BITS ? p.mask_bits + (int64_t)b * p.mb_b + (int64_t)qh * p.mb_h + (int64_t)(qmin / 32) * p.mb_rb
                           : nullptr,
                      BITS ? (uint32_t)(((p.Lk + BN - 1) / BN) * 256) : 0u);
        auto load_mask = [&](int kt) {
            if constexpr (BITS)
                mw = __builtin_amdgcn_raw_buffer_load_b32(wrs, (uint32_t)((kt / BN) * 256 + lane * 4), 0, 0);
            if constexpr (LOADS) {
                if constexpr (!SMASK) {
    #pragma unroll
                    for (int kb = 0; kb < C::NKB; ++kb)
    #pragma unroll
                        for (int a4 = 0; a4 < 4; ++a4)
                            mr[kb][a4] = load_mask_group_rs<MASK>(
                                mrs, (mlane + (uint32_t)(kt + kb * 32 + 8 * a4 + 4 * hh)) * MES);
                } else {
    #pragma unroll
                    for (int kb = 0; kb < C::NKB; ++kb)
    #pragma unroll
                        for (int a4 = 0; a4 < 4; ++a4)
                            mr[kb][a4] = load_mask_group_rs_strided<MASK>(mrs, mlane, kt + kb * 32 + 8 * a4 + 4 * hh,
                                                                          (uint32_t)p.ms[3]);
                }
            }
        };

        float m_run = NEG_INF, l_run = 0.f;
        f32x16_t oacc[C::NDF];
    #pragma unroll
        for (int db = 0; db < C::NDF; ++db) oacc[db] = f32x16_t{};
        // REM: O^T columns 32 NDF .. + 15 of query rows qmin + (lane % 16) (orem[0]) and
        // qmin + 16 + (lane % 16) (orem[1]), head-dim columns 32 NDF + 4 (lane / 16) .. + 3
        f32x4_t orem[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
        const float c_scale = p.scale_log2 == 0.f ? 1.f : __builtin_fabsf(p.scale_log2);

        // per-lane LDS read offsets (loop invariant; the swizzle depends on the
        // row's low 4 bits only, so 32-row and 16-row steps are immediates).
        // K: row col, chunk 2 ch + hh.  V (transposed reads): key rows
        // 4 (grp / 2) + e4 (+ 8 for the second read), head-dim columns
        // 32 db + 16 (grp & 1) + 4 j4 .. + 3, i.e. chunk 4 db + 2 (grp & 1) + j4 / 2, half j4 & 1.
        const int grp = lane >> 4, s16 = lane & 15;
        const int e4 = s16 >> 2, j4 = s16 & 3;
        uint32_t koff[C::NCH], voff[2][C::NDF], voffr[2];
    #pragma unroll
        for (int ch = 0; ch < C::NCH; ++ch) koff[ch] = (uint32_t)(col * C::ROWB + ((2 * ch + hh) ^ C::sw(col)) * 16);
    #pragma unroll
        for (int w = 0; w < 2; ++w) {
            const int kr = 4 * (grp >> 1) + e4 + 8 * w;
    #pragma unroll
            for (int db = 0; db < C::NDF; ++db)
                voff[w][db] = (uint32_t)(kr * C::ROWB + ((4 * db + 2 * (grp & 1) + (j4 >> 1)) ^ C::sw(kr)) * 16 + 8 * (j4 & 1));
            // REM (16x16x32 A operand: head-dim column 32 NDF + lane % 16, eight keys per
            // 16-lane group): group g reads keys 4 (g / 2) + 16 (g % 2) + {0..3, 8..11} of a
            // 32-key block, the key order the swapped P registers hold (below)
            const int krr = 4 * (grp >> 1) + 16 * (grp & 1) + e4 + 8 * w;
            voffr[w] = (uint32_t)(krr * C::ROWB + (4 * C::NDF + (j4 >> 1)) * 16 + 8 * (j4 & 1));
        }

        // S^T of one tile from LDS stage `stage`; operand reads run LA products
        // ahead of their MFMAs (scheduling fences keep them there)
        constexpr int LA = C::LA;
        auto scores = [&](int stage, f32x16_t (&sacc)[C::NKB]) {
            const char* kt_lds = smem + 2 * stage * C::TILEB + C::KOFF0;
            constexpr int N = C::NKB * C::NCH;
            auto rd = [&](int i) {
                return *reinterpret_cast<const u32x4_t*>(kt_lds + (i / C::NCH) * 32 * C::ROWB + koff[i % C::NCH]);
            };
            u32x4_t ring[LA];
    #pragma unroll
            for (int i = 0; i < LA && i < N; ++i) ring[i] = rd(i);
    #pragma unroll
            for (int i = 0; i < N; ++i) {
                const u32x4_t a = ring[i % LA];
                if (i + LA < N) ring[i % LA] = rd(i + LA);
                __builtin_amdgcn_sched_barrier(0);
                const int kb = i / C::NCH, ch = i % C::NCH;
                sacc[kb] = TR::mma(a, qf[ch], ch == 0 ? f32x16_t{} : sacc[kb]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // online softmax on scores already scaled (c_eff = 1) or raw (c_eff = scale)
        auto softmax_pv = [&](int stage, f32x16_t (&sacc)[C::NKB], float mtile, float c_eff) {
            mtile = max_x32(mtile);
            if (__any(mtile > m_run + kRescale)) {
                const float m_new = fmaxf(m_run, mtile);
                const float alpha = (m_new == NEG_INF) ? 1.f : fast_exp2(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
                asm volatile("");  // keep this a branch, not a select on every tile
    #pragma unroll
                for (int db = 0; db < C::NDF; ++db)
    #pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                if constexpr (C::REM) {  // rows lane % 16 and 16 + lane % 16: their lanes' factors
                    const f32x2_t a2 = pair16(alpha);
                    orem[0] *= a2[0];
                    orem[1] *= a2[1];
                }
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
            // O^T += V^T P^T; V^T operands via transposed LDS reads of the row-major V tile
            const char* vt_lds = smem + 2 * stage * C::TILEB + C::VOFF0;
            u32x4_t bf[C::NKB][2];
    #pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
    #pragma unroll
                for (int pc = 0; pc < 2; ++pc)
    #pragma unroll
                    for (int w = 0; w < 4; ++w)
                        bf[kb][pc][w] = TR::pack(sacc[kb][8 * pc + 2 * w], sacc[kb][8 * pc + 2 * w + 1]);
            // operand reads (kb, j): j < 2 NDF the 32-column products (pc, db), db fastest;
            // j = 2 NDF (REM) the 16-column block of the 32 keys.  Reads run LA ahead.
            constexpr int E = 2 * C::NDF + (C::REM ? 1 : 0), N = C::NKB * E, LAV = C::LA;
            auto rd = [&](int i) {
                const int kb = i / E, j = i % E;
                const char* vk = vt_lds + kb * 32 * C::ROWB;
                if (C::REM && j == 2 * C::NDF) {
                    const u32x2_t y0 = lds_read_tr16(vk + voffr[0]);
                    const u32x2_t y1 = lds_read_tr16(vk + voffr[1]);
                    return u32x4_t{y0[0], y0[1], y1[0], y1[1]};
                }
                const int db = j % C::NDF, pc = j / C::NDF;
                const u32x2_t y0 = lds_read_tr16(vk + 16 * pc * C::ROWB + voff[0][db]);
                const u32x2_t y1 = lds_read_tr16(vk + 16 * pc * C::ROWB + voff[1][db]);
                return u32x4_t{y0[0], y0[1], y1[0], y1[1]};
            };
            u32x4_t ring[LAV];
    #pragma unroll
            for (int i = 0; i < LAV && i < N; ++i) ring[i] = rd(i);
    #pragma unroll
            for (int i = 0; i < N; ++i) {
                const u32x4_t a = ring[i % LAV];
                if (i + LAV < N) ring[i % LAV] = rd(i + LAV);
                __builtin_amdgcn_sched_barrier(0);
                const int kb = i / E, j = i % E;
                if (C::REM && j == 2 * C::NDF) {
                    // the 16x16x32 B operand: query rows lane % 16 (first product) and
                    // 16 + lane % 16 (second), eight keys per 16-lane group.  Swapping the
                    // odd 16-lane rows of the pc = 0 registers with the even rows of the
                    // pc = 1 registers gathers them: group g then holds keys
                    // 4 (g / 2) + 16 (g % 2) + {0..3, 8..11} in both registers, for the
                    // first and the second 16 rows.  Both 32-column products of this
                    // block have read these registers already.
    #pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const auto sw2 = __builtin_amdgcn_permlane16_swap(bf[kb][0][w], bf[kb][1][w], false, false);
                        bf[kb][0][w] = sw2[0];
                        bf[kb][1][w] = sw2[1];
                    }
                    orem[0] = Mma16<TR>::mma(a, bf[kb][0], orem[0]);
                    orem[1] = Mma16<TR>::mma(a, bf[kb][1], orem[1]);
                } else {
                    const int db = j % C::NDF, pc = j / C::NDF;
                    oacc[db] = TR::mma(a, bf[kb][pc], oacc[db]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // one key tile; the mask-free and the masked variants run as separate loops
        // so neither carries the other's code (or register copies) around its body.
        // TAIL: the last tile of a mask-free or mask-tensor workgroup, whose keys
        // may run past the end (causal and sliding masks exclude them already).
        auto tile = [&](int it, auto masked_tag, auto tail_tag) __attribute__((always_inline)) {
            constexpr bool MASKED = decltype(masked_tag)::value, TAIL = decltype(tail_tag)::value;
            const int kt = it * BN, stage = it & 1;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            if constexpr (MASKED && BITS) asm volatile("" : "+v"(mw));
            if constexpr (MASKED && LOADS) {
                // this tile's mask registers arrived with the wait above; an asm use says so
                // to the compiler, which would otherwise wait for them where they are read,
                // after the next tile's loads went out, and so for those loads as well
    #pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
    #pragma unroll
                    for (int a4 = 0; a4 < 4; ++a4) asm volatile("" : "+v"(mr[kb][a4]));
            }
            __syncthreads();  // tile `it` is in LDS; every wave is done with the other stage
            if (it + 1 < ntiles) issue_tile(kt + BN, stage ^ 1);
            f32x16_t sacc[C::NKB];
            // a wave issuing its score MFMAs goes first; the other wave on the SIMD
            // fills the gaps with its softmax (D = 72, 8192 x 8192: none 388 -> 381 us,
            // causal 226 -> 219 us; the same around P V gained nothing)
            __builtin_amdgcn_s_setprio(1);
            scores(stage, sacc);
            __builtin_amdgcn_s_setprio(0);
            if constexpr (!MASKED) {
                // no per-element mask: row max on unscaled scores
                float mx = NEG_INF;
    #pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
    #pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
                softmax_pv(stage, sacc, mx * c_scale, c_scale);
            } else {
                constexpr bool ADD = (MASK == MASK_ADD16 || MASK == MASK_ADD32);
                // per-element mask; RAW: on unscaled scores (the scale is positive,
                // so a masked -inf stays -inf once scaled); additive masks add to
                // scaled scores
                auto mask_scores = [&](auto raw_tag) __attribute__((always_inline)) {
                    constexpr bool RAW = decltype(raw_tag)::value;
                    float mtile = NEG_INF;
    #pragma unroll
                    for (int kb = 0; kb < C::NKB; ++kb) {
    #pragma unroll
                        for (int a4 = 0; a4 < 4; ++a4) {
    #pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int j = kt + kb * 32 + 8 * a4 + 4 * hh + r;
                                float x = sacc[kb][4 * a4 + r];
                                if constexpr (!RAW) x *= c_scale;
                                if constexpr (BITS) {  // bit 16 kb + 4 a4 + r: this lane's (row, key j)
                                    // all ones where it attends, else zero; then x or -inf bit by bit
                                    const uint32_t keep =
                                        (uint32_t)__builtin_amdgcn_sbfe((int)mw, kb * 16 + a4 * 4 + r, 1);
                                    const float y = __uint_as_float((__float_as_uint(x) & keep) |
                                                                    (__float_as_uint(NEG_INF) & ~keep));
                                    sacc[kb][4 * a4 + r] = y;
                                    mtile = fmaxf(mtile, y);
                                    continue;
                                }
                                bool ok = true;
                                if constexpr (TAIL) ok = j < kend;
                                if constexpr (ADD)
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
                    return mtile;
                };
                const float mt = mask_scores(PfTag<!ADD>{});
                if (it + 1 < ntiles) load_mask(kt + BN);
                if constexpr (ADD) softmax_pv(stage, sacc, mt, 1.f);
                else softmax_pv(stage, sacc, mt * c_scale, c_scale);
            }
        };

        // masked tiles left of the plain range (window edge), plain tiles, masked
        // tiles right of it (diagonal, ragged end, or every tile of a mask tensor)
        constexpr bool TAIL_CHECK = !CAUSAL_END;
        int it = t0;
        if (it < ntiles) issue_tile(it * BN, it & 1);
        if constexpr (!HAS_MT) {
            for (; it < tp0; ++it) tile(it, PfTag<true>{}, PfTag<false>{});
            for (; it < tp1; ++it) tile(it, PfTag<false>{}, PfTag<false>{});
        }
        if (it < ntiles) load_mask(it * BN);
        if constexpr (TAIL_CHECK) {
            for (; it < ntiles - 1; ++it) tile(it, PfTag<true>{}, PfTag<false>{});
            if (it < ntiles) tile(it, PfTag<true>{}, PfTag<true>{});
        } else {
            for (; it < ntiles; ++it) tile(it, PfTag<true>{}, PfTag<false>{});
        }

        // ---- epilogue ----
        float lsum_row;
        if constexpr (C::REM) {
            // the row-sum column D is element rr % 4 of lane group rr / 4 (rr = D % 32)
            // in orem[0] for rows 0..15 and orem[1] for rows 16..31 of the wave
            constexpr int rr = D % 32, GR = rr / 4, ER = rr % 4;
            const int src = (16 * GR + (col & 15)) * 4;
            const float xl = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(orem[0][ER])));
            const float xh = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(orem[1][ER])));
            lsum_row = col < 16 ? xl : xh;
        } else if constexpr (C::ONES) {
            constexpr int rr = D % 32;
            constexpr int RL = 4 * (rr / 8) + (rr % 4), HL = (rr % 8) / 4, DBL = D / 32;
            const float x = oacc[DBL][RL];
            const float y = xor32(x);
            lsum_row = (hh == HL) ? x : y;
        } else {
            lsum_row = sum_x32(l_run);
        }
        const float inv = lsum_row > 0.f ? 1.f / lsum_row : 0.f;
        if constexpr (C::REM) {  // columns 32 NDF + 4 (lane / 16) .. + 3 of rows lane % 16 and 16 + lane % 16
            const f32x2_t inv2 = pair16(inv);
            const int d0 = 32 * C::NDF + 4 * (lane >> 4);
    #pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int qr = qmin + 16 * h + (lane & 15);
                if (qr < p.Lq && d0 < D) {
                    char* orow = reinterpret_cast<char*>(p.o) +
                                 ((int64_t)b * p.os[0] + (int64_t)qh * p.os[1] + (int64_t)qr * p.os[2]) * 2;
                    TR::store4(orow + d0 * 2, orem[h] * inv2[h]);
                }
            }
        }
        if (rv) {
            char* orow = reinterpret_cast<char*>(p.o) +
                         ((int64_t)b * p.os[0] + (int64_t)qh * p.os[1] + (int64_t)qi * p.os[2]) * 2;
    #pragma unroll
            for (int db = 0; db < C::NDF; ++db)
    #pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int d0 = 32 * db + 8 * a4 + 4 * hh;
                    if (d0 < D) {
                        f32x4_t x = {oacc[db][4 * a4] * inv, oacc[db][4 * a4 + 1] * inv, oacc[db][4 * a4 + 2] * inv,
                                     oacc[db][4 * a4 + 3] * inv};
                        TR::store4(orow + d0 * 2, x);
                    }
                }
        }
    };
    run(CAUSAL_END ? nqt - 1 - tt : tt);
    if (pairs && tt != nqt - 1 - tt) {
        __syncthreads();  // every wave is done with the first row tile's LDS stages
        run(tt);
    }
}

}  // namespace sdpa_dev
