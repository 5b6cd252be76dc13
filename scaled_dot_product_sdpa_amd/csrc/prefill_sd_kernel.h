// Prefill ("full") kernel for 16-bit inputs and wide heads (D = 256, 512) on
// gfx950, with the head dim split across waves.
//
// What bounds a wide-head kernel is LDS bandwidth: every wave reads its K and
// V tiles from LDS, and a 16-row wave (the only row count whose Q and O fit in
// registers at D = 512) uses each byte it reads for 16 rows only.  Here every
// wave works on 32 query rows (v_mfma_f32_32x32x16), and NS waves share those
// rows, each owning D / NS head-dim columns: the split-D accumulators mlx
// issue #3885 ("Requests") suggests for d = 512.
//   * S^T = K Q^T: each wave contracts its own D / NS columns of Q and K and
//     the NS partial score blocks are summed through LDS (every wave of the
//     set adds them in the same order, so all hold the same scores);
//   * every wave runs the same online softmax (base 2, lazy rescale) on those
//     scores and accumulates O^T += V^T P^T for its own columns only, V^T read
//     from the row-major V tile through ds_read_b64_tr_b16;
//   * a workgroup is NW waves = NW / NS sets of 32 rows of one key/value head:
//     query heads of a grouped-query group (mlx issue #3885, prefill
//     paragraph: scores [B, n_kv, n_rep, qL, kL]) share every K/V tile;
//   * K/V tiles of BN keys go global -> LDS with buffer_load ... lds, double
//     buffered, rows unpadded with the 16-byte chunks of row r at
//     chunk ^ sd_sw(r), which keeps the 128-bit K reads (16 rows, one chunk)
//     and the transposed 64-bit V reads (4 rows x 4 chunks) on distinct banks.
// Per tile and wave, LDS reads are 2 * BN * (D / NS) * 2 bytes for a
// 32 x BN x D / NS share of the work: at D = 512, NS = 2, 40 KB per MFLOP
// including the score exchange, against 64 KB for 16-row waves.  At D = 256
// one wave holds all 256 columns (NS = 1, no exchange): 32 KB per MFLOP.
#pragma once

#include "attn_common.h"
#include "rope_kernel.h"

namespace sdpa_dev {

// Row -> chunk swizzle: bits 2-3 from r mod 4 (the 4 rows of a transposed
// read pass land in 4 different 64-byte bank groups), bits 0-1 from
// (r / 4) mod 4 (so 16 consecutive rows take 16 distinct 16-byte slots).
__device__ __forceinline__ int sd_sw(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <bool B> struct SdTag { static constexpr bool value = B; };

template <class TR, int D_, int NS_, int BN_, int NW_>
struct SdCfg {
    static constexpr int D = D_, NS = NS_, BN = BN_, NW = NW_, NT = 64 * NW;
    static constexpr int DH = D / NS;      // head-dim columns per wave
    static constexpr int NP = NW / NS;     // 32-row sets per workgroup
    static constexpr bool PAIRS = true;    // causal: two row tiles per workgroup (see the kernel)
    static constexpr int KC = D / 8;       // 16-byte chunks per LDS row
    static constexpr int ROWB = D * 2;
    static constexpr int TILEB = BN * ROWB;
    static constexpr int NCH = DH / 16;    // Q K^T steps (16 columns each)
    static constexpr int NDB = DH / 32;    // 32-column O^T blocks
    static constexpr int NKB = BN / 32;    // 32-key score blocks per tile
    static constexpr int RPI = 64 / KC;    // LDS rows per 64-lane load
    static constexpr int NI = BN * KC / (64 * NW);  // loads per wave per tile (K; V the same)
    static constexpr int XB = NS > 1 ? NW * NKB * 64 * 16 * 4 : 0;  // partial-score exchange
    static constexpr int LDS = 4 * TILEB + XB;
    // the output tile staged in LDS (each wave's 32 rows x DH columns) where it fits, so
    // that whole rows leave in 16-byte chunks, consecutive lanes on consecutive chunks
    static constexpr int OPB = DH * 2 + 16;  // staged row pitch: 4 banks further per row
    static constexpr bool STAGE_O = NW * 32 * OPB <= LDS;
    static constexpr int WPE = 2;          // waves per SIMD the registers must allow
    static_assert(NS == 1 || NS == 2, "head-dim split");
    static_assert(DH % 128 == 0 && KC <= 64 && 64 % KC == 0, "head dim");
    static_assert(BN % 32 == 0 && (BN * KC) % (64 * NW) == 0, "key tile");
    static_assert(NP == 1 || NP == 2 || NP == 4 || NP == 8, "row sets per workgroup");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// SMASK: the mask tensor's keys are not 4-element aligned runs (mask_vec == 0);
// its elements are loaded one by one.
template <class TR, class C, int MASK, bool ROPE = false, bool SMASK = false>
__global__ __launch_bounds__(C::NT, C::WPE) void prefill_sd_kernel(const Params p) {
    constexpr int D = C::D, BN = C::BN, NW = C::NW, NS = C::NS, DH = C::DH;
    constexpr float NEG_INF = -__builtin_inff();
    constexpr float kRescale = 8.0f;
    constexpr bool HAS_MT = (MASK == MASK_ADD16 || MASK == MASK_ADD32 || MASK == MASK_BOOL);
    constexpr bool CAUSAL_END = (MASK == MASK_CAUSAL || MASK == MASK_SLIDE);
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];
    const uint32_t smem_lds = lds_address(smem);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int col = lane & 31, hh = lane >> 5;
    const int ps = w / NS, hf = w % NS;  // 32-row set, head-dim share

    // ---- work item: (batch, kv head, head group, row tile), XCD-aware ----
    const int n_rep = p.n_rep;
    int HG = 1;  // heads per workgroup: the largest power of two up to NP dividing n_rep
#pragma unroll
    for (int c = C::NP; c > 1; c >>= 1)
        if (HG == 1 && n_rep % c == 0) HG = c;
    const int RB = C::NP / HG;  // 32-row blocks per head
    const int BMW = 32 * RB;
    const bool pairs = C::PAIRS && MASK == MASK_CAUSAL && p.pairs;  // the host's choice, uniform
    const int nrt = (p.Lq + BMW - 1) / BMW;
    const int nit = pairs ? (nrt + 1) / 2 : nrt;  // row-tile items per head group
    const int nhg = n_rep / HG;
    const int total = nit * nhg * p.Hkv * p.B;
    const int per = (total + p.nx - 1) / p.nx;
    const int item = (int)(blockIdx.x % p.nx) * per + (int)(blockIdx.x / p.nx);
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
        tt = item % nit;
        int rest = item / nit;
        hgi = rest % nhg;
        rest /= nhg;
        g = rest % p.Hkv;
        b = rest / p.Hkv;
    }
    // the row tiles of one workgroup: one, or with pairs (causal) two whose
    // key ranges add up to the same length for every workgroup (t and nrt - 1 - t;
    // the host pairs only grids that still give every CU a workgroup)
    auto run = [&](const int t) __attribute__((always_inline)) {
        const int i0 = t * BMW;
        const int qh = g * n_rep + hgi * HG + (ps % HG);
        const int qmin = i0 + 32 * (ps / HG);
        const int qi = qmin + col;
        const bool rv = qi < p.Lq;
        const int qic = min(qi, p.Lq - 1);
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
            const int lo = min(qmin + 31, p.Lq - 1) + off - p.window + 1;  // window's left edge, wave's last row
            tp0 = max(t0, lo <= 0 ? 0 : (lo + BN - 1) / BN);
        }
        if (HAS_MT) tp1 = tp0;
        tp0 = min(tp0, ntiles);
        tp1 = max(tp0, min(tp1, ntiles));

        const uint32_t kstep = (uint32_t)p.ks[2] * 2u, vstep = (uint32_t)p.vs[2] * 2u;
        const char* kglob = reinterpret_cast<const char*>(p.k) + ((int64_t)b * p.ks[0] + (int64_t)g * p.ks[1]) * 2;
        const char* vglob = reinterpret_cast<const char*>(p.v) + ((int64_t)b * p.vs[0] + (int64_t)g * p.vs[1]) * 2;
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(kglob, kend > 0 ? (uint32_t)(kend - 1) * kstep + (uint32_t)(D * 2) : 0u);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vglob, kend > 0 ? (uint32_t)(kend - 1) * vstep + (uint32_t)(D * 2) : 0u);

        // ---- Q^T fragments (B operand): Q[qi][DH hf + 16 c + 8 hh .. +8] ----
        u32x4_t qf[C::NCH];
        {
            const char* qrow = reinterpret_cast<const char*>(p.q) +
                               ((int64_t)b * p.qs[0] + (int64_t)qh * p.qs[1] + (int64_t)qic * p.qs[2]) * 2;
    #pragma unroll
            for (int c = 0; c < C::NCH; ++c)
                qf[c] = *reinterpret_cast<const u32x4_t*>(qrow + (DH * hf + 16 * c + 8 * hh) * 2);  // rows >= Lq: never stored
            if constexpr (ROPE)  // rotary embedding of the query row (columns < rope_dim)
                rope_q_fragments<TR, C::NCH, 16>(qf, qrow, DH * hf + 8 * hh, p.rope_dim, p.rope_cos, p.rope_sin,
                                                 (int64_t)p.rope_pos0 + qic);
            // a negative scale runs as |scale| on -Q (exact: a sign flip) and a zero
            // scale as scale 1 on Q = 0 (every score is 0 either way), so the scale
            // is positive and the row max can always be taken on unscaled scores
            if (p.scale_log2 < 0.f) {
    #pragma unroll
                for (int c = 0; c < C::NCH; ++c) qf[c] ^= 0x80008000u;
            } else if (p.scale_log2 == 0.f) {
    #pragma unroll
                for (int c = 0; c < C::NCH; ++c) qf[c] = u32x4_t{0u, 0u, 0u, 0u};
            }
        }
        const float c_scale = p.scale_log2 == 0.f ? 1.f : __builtin_fabsf(p.scale_log2);

        // ---- K/V tile loads: instruction u of this wave fills LDS rows
        // (u NW + w) RPI + lane / KC, slot lane % KC <- global chunk slot ^ sd_sw(row) ----
        auto issue_tile = [&](int kt, int stage) __attribute__((always_inline)) {
            char* kl = smem + (2 * stage) * C::TILEB;
            char* vl = smem + (2 * stage + 1) * C::TILEB;
            const uint32_t kla = smem_lds + (uint32_t)((2 * stage) * C::TILEB);
            const uint32_t vla = smem_lds + (uint32_t)((2 * stage + 1) * C::TILEB);
    #pragma unroll
            for (int u = 0; u < C::NI; ++u) {
                // row = r0 + lane / KC: r0 (and, with one row per load, the swizzle) is
                // wave-uniform and goes in soffset; only the chunk offset is per lane
                const int ins = u * NW + w;
                const int r0 = ins * C::RPI;
                uint32_t vk, vv;
                if constexpr (C::RPI == 1) {
                    vk = vv = (uint32_t)(lane * 16) ^ (uint32_t)(sd_sw(r0) * 16);
                } else {
                    const int row = r0 + lane / C::KC;
                    const uint32_t cb = (uint32_t)(((lane % C::KC) ^ sd_sw(row)) * 16);
                    vk = (uint32_t)(lane / C::KC) * kstep + cb;
                    vv = (uint32_t)(lane / C::KC) * vstep + cb;
                }
                // a mask tensor's groups are loaded at the top of the tile that uses them,
                // before these: the compiler's count of the loads after them lets it wait
                // for the groups alone, so those variants keep the loads it can see
                if constexpr (HAS_MT) {
                    buffer_load16_lds_so(krs, kl + ins * 1024, vk, (uint32_t)(kt + r0) * kstep);
                    buffer_load16_lds_so(vrs, vl + ins * 1024, vv, (uint32_t)(kt + r0) * vstep);
                } else {
                    dma16_lds_so(krs, kla + (uint32_t)(ins * 1024), vk, (uint32_t)(kt + r0) * kstep);
                    dma16_lds_so(vrs, vla + (uint32_t)(ins * 1024), vv, (uint32_t)(kt + r0) * vstep);
                }
            }
        };

        // ---- mask groups (4 keys): one buffer resource per wave from its first row ----
        constexpr int MES = MASK == MASK_BOOL ? 1 : (MASK == MASK_ADD16 ? 2 : 4);
        const int q0c = min(qmin, p.Lq - 1);
        const int64_t mbase = HAS_MT ? (int64_t)b * p.ms[0] + (int64_t)qh * p.ms[1] + (int64_t)q0c * p.ms[2] : 0;
        const uint32_t mlane = HAS_MT ? (uint32_t)((qic - q0c) * p.ms[2]) : 0u;
        const int64_t mleft = HAS_MT ? p.mask_span - mbase * MES : 0;
        const __amdgpu_buffer_rsrc_t mrs =
            make_rsrc(HAS_MT ? reinterpret_cast<const char*>(p.mask) + mbase * MES : nullptr,
                      (uint32_t)(mleft > 0xffffffffLL ? 0xffffffffLL : mleft));
        typename MaskRaw<MASK>::type mr[HAS_MT ? C::NKB : 1][4];
        auto load_mask = [&](int kt) __attribute__((always_inline)) {
            if constexpr (HAS_MT) {
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

        // ---- LDS read offsets ----
        // K (A operand of S^T): row 32 kb + col, chunk DH/8 hf + 2 c + hh ->
        // slot = DH/8 hf + 16 (c >> 3) + ((2 (c & 7) + hh) ^ ksw)
        // (2 m + hh) ^ ksw = (2 m ^ (ksw & 14)) + ((hh ^ ksw) & 1): one XOR with an
        // immediate per read, no offset table
        const int ksw = sd_sw(col);
        const int kxe = (ksw & 14) * 16;
        const int kbase = col * C::ROWB + DH * hf * 2 + ((hh ^ ksw) & 1) * 16;
        // V^T (A operand of O^T, two transposed reads per MFMA): rows 16 pc + 4 (grp >> 1) + e4 (+ 8),
        // columns DH hf + 32 db + 16 (grp & 1) + 4 j4 -> chunk DH/8 hf + 4 db + cl, byte 8 (j4 & 1)
        const int grp = lane >> 4, e4 = (lane >> 2) & 3, j4 = lane & 3;
        const int cl = 2 * (grp & 1) + (j4 >> 1);
        // rows r and r + 8 differ in sd_sw bits 0-1 only: (4 m + cl) ^ sw =
        // (4 m ^ (4 e4)) + ((cl ^ sw) & 3), one XOR per read pair
        const int vsw0 = (e4 << 2) | ((grp >> 1) & 3), vsw1 = (e4 << 2) | (((grp >> 1) + 2) & 3);
        const int vxe = (e4 << 2) * 16;
        const int vbase = (4 * (grp >> 1) + e4) * C::ROWB + DH * hf * 2 + 8 * (j4 & 1) + ((cl ^ vsw0) & 3) * 16;
        const int vsec = 8 * C::ROWB + (((cl ^ vsw1) & 3) - ((cl ^ vsw0) & 3)) * 16;  // second read, relative

        float m_run = NEG_INF, l_run = 0.f;
        f32x16_t oacc[C::NDB];
    #pragma unroll
        for (int db = 0; db < C::NDB; ++db) oacc[db] = f32x16_t{};

        // TAIL: the last tile of a mask-free or mask-tensor workgroup, whose keys
        // may run past the end (causal and sliding masks exclude them already)
        auto tile = [&](int it, auto masked_tag, auto tail_tag) __attribute__((always_inline)) {
            constexpr bool MASKED = decltype(masked_tag)::value, TAIL = decltype(tail_tag)::value;
            const int kt = it * BN, stage = it & 1;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();  // tile `it` is in LDS; every wave is done with the other stage
            // this tile's mask groups before the next tile's loads: waiting for them
            // never waits for the prefetch
            if constexpr (MASKED) load_mask(kt);
            if (it + 1 < ntiles) issue_tile(kt + BN, stage ^ 1);
            const char* kl = smem + (2 * stage) * C::TILEB + kbase;
            const char* vl = smem + (2 * stage + 1) * C::TILEB + vbase;

            // ---- S^T = K Q^T over this wave's head-dim share ----
            // K reads run one step ahead of the MFMAs that use them (two operand
            // buffers; the scheduling barrier keeps each read ahead of its MFMA)
            f32x16_t sacc[C::NKB];
            __builtin_amdgcn_s_setprio(1);  // score MFMAs first (about 1% on D = 512 causal)
    #pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
                auto kread = [&](int c) __attribute__((always_inline)) {
                    return *reinterpret_cast<const u32x4_t*>(kl + kb * 32 * C::ROWB + (c >> 3) * 256 +
                                                             ((32 * (c & 7)) ^ kxe));
                };
                u32x4_t ka[2];
                ka[0] = kread(0);
                f32x16_t s = f32x16_t{};
    #pragma unroll
                for (int c = 0; c < C::NCH; ++c) {
                    if (c + 1 < C::NCH) ka[(c + 1) & 1] = kread(c + 1);
                    __builtin_amdgcn_sched_barrier(0);
                    s = TR::mma(ka[c & 1], qf[c], s);
                    __builtin_amdgcn_sched_barrier(0);
                }
                sacc[kb] = s;
            }
            __builtin_amdgcn_s_setprio(0);
            // ---- sum the NS partial score blocks (same order in every wave) ----
            if constexpr (NS > 1) {
                char* xb = smem + 4 * C::TILEB;
    #pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
    #pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4)
                        *reinterpret_cast<f32x4_t*>(xb + (((w * C::NKB + kb) * 4 + i4) * 64 + lane) * 16) =
                            f32x4_t{sacc[kb][4 * i4], sacc[kb][4 * i4 + 1], sacc[kb][4 * i4 + 2], sacc[kb][4 * i4 + 3]};
                __syncthreads();
                const int wp = w ^ 1;
    #pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
    #pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4) {
                        const f32x4_t o =
                            *reinterpret_cast<const f32x4_t*>(xb + (((wp * C::NKB + kb) * 4 + i4) * 64 + lane) * 16);
                        // a + b and b + a are the same float: both waves hold the same scores
    #pragma unroll
                        for (int r = 0; r < 4; ++r) sacc[kb][4 * i4 + r] = sacc[kb][4 * i4 + r] + o[r];
                    }
            }

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
                // per-element mask on unscaled scores (the scale is positive); additive
                // masks add to scaled scores
                constexpr bool ADD = (MASK == MASK_ADD16 || MASK == MASK_ADD32);
                float mx = NEG_INF;
    #pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
    #pragma unroll
                    for (int a4 = 0; a4 < 4; ++a4)
    #pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int j = kt + kb * 32 + 8 * a4 + 4 * hh + r;
                            float x = sacc[kb][4 * a4 + r];
                            bool ok = true;
                            if constexpr (TAIL) ok = j < kend;
                            if constexpr (ADD)
                                x = __builtin_fmaf(mask_value<MASK>(mr[kb][a4], r, p.mask_dtype), kLog2e, x * c_scale);
                            if constexpr (MASK == MASK_CAUSAL) ok = ok && (j <= qi + off);
                            if constexpr (MASK == MASK_SLIDE) ok = ok && in_window(j, qi + off, p.window);
                            if constexpr (MASK == MASK_BOOL) ok = ok && ((mr[kb][a4] >> (8 * r)) & 0xffu) != 0u;
                            x = ok ? x : NEG_INF;
                            sacc[kb][4 * a4 + r] = x;
                            mx = fmaxf(mx, x);
                        }
                mtile = ADD ? mx : mx * c_scale;
                c_eff = ADD ? 1.f : c_scale;
            }

            // ---- online softmax (lazy rescale) ----
            mtile = max_x32(mtile);
            if (__any(mtile > m_run + kRescale)) {
                const float m_new = fmaxf(m_run, mtile);
                const float alpha = (m_new == NEG_INF) ? 1.f : fast_exp2(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
                asm volatile("" ::: "memory");  // keep this a branch, not a select on every tile
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

            // ---- O^T += V^T P^T for this wave's columns ----
    #pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
    #pragma unroll
                for (int pc = 0; pc < 2; ++pc) {
                    u32x4_t bf;
    #pragma unroll
                    for (int q = 0; q < 4; ++q) bf[q] = TR::pack(sacc[kb][8 * pc + 2 * q], sacc[kb][8 * pc + 2 * q + 1]);
                    const char* vr = vl + (kb * 32 + 16 * pc) * C::ROWB;
                    // V^T reads one block ahead of the MFMAs (two operand buffers)
                    auto vread = [&](int db) __attribute__((always_inline)) {
                        const char* va = vr + (db >> 2) * 256 + ((64 * (db & 3)) ^ vxe);
                        const u32x2_t y0 = lds_read_tr16(va);
                        const u32x2_t y1 = lds_read_tr16(va + vsec);
                        return u32x4_t{y0[0], y0[1], y1[0], y1[1]};
                    };
                    u32x4_t vb[2];
                    vb[0] = vread(0);
    #pragma unroll
                    for (int db = 0; db < C::NDB; ++db) {
                        if (db + 1 < C::NDB) vb[(db + 1) & 1] = vread(db + 1);
                        __builtin_amdgcn_sched_barrier(0);
                        oacc[db] = TR::mma(vb[db & 1], bf, oacc[db]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        };

        // masked tiles left of the plain range (window edge), plain tiles, masked
        // tiles right of it (diagonal, ragged end, or every tile of a mask tensor)
        constexpr bool TAIL_CHECK = !CAUSAL_END;
        int it = t0;
        if (it < ntiles) issue_tile(it * BN, it & 1);
        if constexpr (!HAS_MT) {
            for (; it < tp0; ++it) tile(it, SdTag<true>{}, SdTag<false>{});
            for (; it < tp1; ++it) tile(it, SdTag<false>{}, SdTag<false>{});
        }
        if constexpr (TAIL_CHECK) {
            for (; it < ntiles - 1; ++it) tile(it, SdTag<true>{}, SdTag<false>{});
            if (it < ntiles) tile(it, SdTag<true>{}, SdTag<true>{});
        } else {
            for (; it < ntiles; ++it) tile(it, SdTag<true>{}, SdTag<false>{});
        }

        // ---- epilogue: lane holds query col, columns DH hf + 32 db + 8 a4 + 4 hh .. +3 ----
        const float lsum_row = sum_x32(l_run);
        if constexpr (C::STAGE_O) {
            // Through LDS: the 8-byte pieces above, written straight to memory, build
            // each 128-byte line of a row from 8 store instructions (c5: 152-156 MB
            // written per launch against 134 MB of output).  The wave's 32 rows x DH
            // columns go to LDS (rows OPB bytes apart: the 32 rows of one write fall on
            // 4-bank steps) and are read back a row pair per instruction, each lane
            // storing one 16-byte chunk, consecutive lanes consecutive chunks.
            constexpr int CPR = DH / 8;  // 16-byte chunks per row of the wave's share
            const float inv = lsum_row > 0.f ? 1.f / lsum_row : 0.f;
            __syncthreads();  // every wave is done with the K/V stages and the score exchange
            char* const ob = smem + w * (32 * C::OPB);
            char* const obw = ob + col * C::OPB + 8 * hh;
    #pragma unroll
            for (int db = 0; db < C::NDB; ++db)
    #pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const u32x2_t x = {TR::pack(oacc[db][4 * a4] * inv, oacc[db][4 * a4 + 1] * inv),
                                       TR::pack(oacc[db][4 * a4 + 2] * inv, oacc[db][4 * a4 + 3] * inv)};
                    *reinterpret_cast<u32x2_t*>(obw + (4 * db + a4) * 16) = x;
                }
            __syncthreads();
            const int c = lane % CPR, r0 = lane / CPR;  // this lane's chunk, first row
            char* const obase = reinterpret_cast<char*>(p.o) +
                                ((int64_t)b * p.os[0] + (int64_t)qh * p.os[1] + (int64_t)(qmin + r0) * p.os[2]) * 2 +
                                (DH * hf + 8 * c) * 2;
            const int64_t ostep = (int64_t)p.os[2] * 2 * (64 / CPR);  // bytes between this lane's rows
    #pragma unroll 1
            for (int i = 0; i < 32 * CPR / 64; ++i) {
                const int r = r0 + (64 / CPR) * i;
                const u32x4_t y = *reinterpret_cast<const u32x4_t*>(ob + r * C::OPB + c * 16);
                if (qmin + r < p.Lq) *reinterpret_cast<u32x4_t*>(obase + ostep * i) = y;
            }
        } else if (rv) {
            const float inv = lsum_row > 0.f ? 1.f / lsum_row : 0.f;
            char* orow = reinterpret_cast<char*>(p.o) +
                         ((int64_t)b * p.os[0] + (int64_t)qh * p.os[1] + (int64_t)qi * p.os[2]) * 2;
    #pragma unroll
            for (int db = 0; db < C::NDB; ++db)
    #pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int d0 = DH * hf + 32 * db + 8 * a4 + 4 * hh;
                    f32x4_t x = {oacc[db][4 * a4] * inv, oacc[db][4 * a4 + 1] * inv, oacc[db][4 * a4 + 2] * inv,
                                 oacc[db][4 * a4 + 3] * inv};
                    TR::store4(orow + d0 * 2, x);
                }
        }
    };
    run(CAUSAL_END ? nrt - 1 - tt : tt);  // heavy row tiles first
    if (pairs && tt != nrt - 1 - tt) {
        __syncthreads();  // every wave is done with the first row tile's LDS stages
        run(tt);
    }
}

}  // namespace sdpa_dev
