// Split-key decode ("vector") kernel for 16-bit inputs on gfx950.
//
// Decode (q_len <= 8, mlx issue #3885: "vector" kernel, and its 2-pass
// variant that splits the keys over nkv x blocks threadgroups before a
// combine) is bound by reading K and V once from HBM.  One workgroup handles
// one (batch, kv head, key split) and all n_rep x q_len query rows of that kv
// head (up to 16 per column group), so every K/V byte serves every query head
// of its group.  Per chunk of KS = 16 * NW keys:
//   1. all K and V loads of the chunk are issued at once: each wave loads the
//      K rows of its 16 keys straight into v_mfma_f32_16x16x32 A-operand
//      registers (lane l: key l % 16, head-dim columns 32 i + 8 (l / 16) .. +7)
//      and its V rows into registers bound for LDS;
//   2. S^T = K Q^T on the matrix cores (16 keys x 16 query rows per wave);
//   3. exact softmax statistics of the chunk: row maxima and sums reduced
//      over lanes (shuffles) and over waves (LDS); the chunk is merged into
//      the running state with the usual 2^(m_old - m_new) rescale;
//   4. P (rounded to the input type) goes to LDS; O^T += V^T P^T on the matrix
//      cores, each wave owning every NW-th 16-column block of the head dim.
//      V is stored transposed in LDS ([d][key], 4-key x 8-column register
//      transposes on the way in), so each A operand is one 16-byte read.
// The workgroup writes its unnormalised partial output, running max (log2
// domain) and sum; combine_kernel merges the splits.  With a single split
// (enough batch x kv-head groups to fill the chip) it writes the output itself
// and no combine runs.
#pragma once

#include "attn_common.h"
#include "rope_kernel.h"

namespace sdpa_dev {

// D: head dim of Q and K; DO: head dim of V and of the output (equal to D
// except for the (192, 128) pairing of mlx issue #3885, "Current routing").
template <class TR, int D_, int NW_, int DO_ = D_>
struct DecCfg {
    static constexpr int D = D_, DO = DO_, NW = NW_, NT = 64 * NW;
    static constexpr int KS = 16 * NW;               // keys per chunk
    static constexpr int NCH = (D + 31) / 32;        // Q K^T steps (32 head-dim columns each)
    static constexpr int DV = (DO + 15) / 16 * 16;   // V columns incl. zero pad
    static constexpr int NDB = DV / 16;              // 16-column O^T blocks
    static constexpr int NDBW = (NDB + NW - 1) / NW; // blocks per wave (round robin)
    static constexpr int TP = KS + 4;                // V^T row pitch: 8-byte rows skew, so the 8 rows a
                                                     // transposed store hits at once fall on distinct banks
    static constexpr int PP = KS + 8;                // P row pitch (elements)
    static constexpr int CPR = DO / 8;               // 16-byte chunks per V row
    static constexpr int VU = (4 * CPR + 63) / 64;   // (4-key, 8-column) V units per lane
    static constexpr int LDS = DV * TP * 2 + 16 * PP * 2 + 2 * NW * 16 * 4;
    static constexpr bool PREFETCH = D <= 256;       // registers for a second chunk in flight
    static_assert(D % 8 == 0 && DO % 8 == 0, "head dims must be whole numbers of 16-byte chunks");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <class TR, class C, int MASK, bool ROPE = false>
__global__ __launch_bounds__(C::NT) void decode_split_kernel(const Params p) {
    constexpr int D = C::D, DO = C::DO, NW = C::NW, KS = C::KS;
    constexpr float NEG_INF = -__builtin_inff();
    constexpr bool HAS_MT = (MASK == MASK_ADD16 || MASK == MASK_ADD32 || MASK == MASK_BOOL);
    __shared__ __attribute__((aligned(16))) uint16_t Vt[C::DV * C::TP];
    __shared__ __attribute__((aligned(16))) uint16_t Ps[16 * C::PP];
    __shared__ float red[2][NW][16];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int b = blockIdx.z, split = blockIdx.x;
    const int grp = blockIdx.y / p.col_groups, cg = blockIdx.y % p.col_groups;
    const int r = cg * 16 + col;
    const bool rv = r < p.n_rep * p.Lq;
    const int rr = rv ? r : 0;
    const int qh = grp * p.n_rep + rr / p.Lq, qi = rr % p.Lq;
    const int kbeg = p.kbase + split * p.keys_per_split;
    const int kend = min(p.Lk, kbeg + p.keys_per_split);
    const int off = p.Lk - p.Lq;

    const int64_t kstep = p.ks[2] * 2, vstep = p.vs[2] * 2;
    const char* kglob = reinterpret_cast<const char*>(p.k) + ((int64_t)b * p.ks[0] + (int64_t)grp * p.ks[1]) * 2;
    const char* vglob = reinterpret_cast<const char*>(p.v) + ((int64_t)b * p.vs[0] + (int64_t)grp * p.vs[1]) * 2;
    const uint32_t kstep32 = (uint32_t)kstep, vstep32 = (uint32_t)vstep;
    const __amdgpu_buffer_rsrc_t krs =
        make_rsrc(kglob, kend > 0 ? (uint32_t)(kend - 1) * kstep32 + (uint32_t)(D * 2) : 0u);
    const __amdgpu_buffer_rsrc_t vrs =
        make_rsrc(vglob, kend > 0 ? (uint32_t)(kend - 1) * vstep32 + (uint32_t)(DO * 2) : 0u);

    const int64_t mrow = HAS_MT ? (int64_t)b * p.ms[0] + (int64_t)qh * p.ms[1] + (int64_t)qi * p.ms[2] : 0;

    // ---- loads of one chunk (keys k0 .. k0 + KS - 1): this wave's 16 keys of
    // K as A operands (lane: key col, head-dim columns 32 i + 8 g .. +7), its
    // V rows bound for LDS and, for mask tensors, its mask groups ----
    u32x4_t kf[C::NCH];
    // V unit u of this lane: keys kw + 4 * q4 .. +3, head-dim columns 8 c .. +7
    // (the key quad varies fastest across lanes, so the transposed LDS stores
    // of one instruction spread over 16 column groups x 4 quads of banks)
    u32x4_t vr[C::VU][4];
    typename MaskRaw<MASK>::type mr{};
    // (K first: loads return in order, and S = K Q^T waits only for K, Q and
    // the mask while V is still arriving)
    auto issue_k = [&](int k0) __attribute__((always_inline)) {
        const int kw = k0 + 16 * w;
#pragma unroll
        for (int i = 0; i < C::NCH; ++i) {
            const int d = 32 * i + 8 * g;
            kf[i] = u32x4_t{0u, 0u, 0u, 0u};
            if (d < D) kf[i] = buffer_load16(krs, (uint32_t)(kw + col) * kstep32 + (uint32_t)(d * 2));
        }
    };
    auto issue_v = [&](int k0) __attribute__((always_inline)) {
        const int kw = k0 + 16 * w;
        if constexpr (HAS_MT) mr = load_mask_group<MASK>(p, mrow, kw + 4 * g);
#pragma unroll
        for (int u = 0; u < C::VU; ++u) {
            const int idx = lane + 64 * u;
            const int q4 = idx & 3, c = idx >> 2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vr[u][e] = u32x4_t{0u, 0u, 0u, 0u};
                if (idx < 4 * C::CPR)
                    vr[u][e] = buffer_load16(vrs, (uint32_t)(kw + 4 * q4 + e) * vstep32 + (uint32_t)(c * 16));
            }
        }
    };
    // with prefetching, the first chunk's K loads go out before anything else
    // (its V loads right after Q's)
    if constexpr (C::PREFETCH) {
        if (kbeg < kend) issue_k(kbeg);
    }

    // Q fragments (B operand): row col, head-dim columns 32 i + 8 g .. +7;
    // rows past n_rep * Lq read row 0 (their results are never stored)
    u32x4_t qf[C::NCH];
    {
        const char* qrow = reinterpret_cast<const char*>(p.q) +
                           ((int64_t)b * p.qs[0] + (int64_t)qh * p.qs[1] + (int64_t)qi * p.qs[2]) * 2;
#pragma unroll
        for (int i = 0; i < C::NCH; ++i) {
            const int d = 32 * i + 8 * g;
            const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qrow + min(d, D - 8) * 2);
            qf[i] = d < D ? x : u32x4_t{0u, 0u, 0u, 0u};
        }
        if constexpr (ROPE)  // rotary embedding of the query row (columns < rope_dim)
            rope_q_fragments<TR, C::NCH, 32>(qf, qrow, 8 * g, p.rope_dim, p.rope_cos, p.rope_sin,
                                             (int64_t)p.rope_pos0 + qi);
    }
    if constexpr (C::PREFETCH) {
        if (kbeg < kend) issue_v(kbeg);
    }
    // zero V^T pad rows [DO, DV) once (they feed the last O^T block)
    if constexpr (C::DV > DO) {
        for (int idx = tid; idx < (C::DV - DO) * C::TP; idx += C::NT) Vt[DO * C::TP + idx] = 0;
    }
    const float c_scale = p.scale_log2;

    float m_run = NEG_INF, l_run = 0.f;
    f32x4_t oacc[C::NDBW];
#pragma unroll
    for (int i = 0; i < C::NDBW; ++i) oacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int k0 = kbeg; k0 < kend; k0 += KS) {
        const int kw = k0 + 16 * w;  // this wave's first key
        if constexpr (!C::PREFETCH) {
            issue_k(k0);
            issue_v(k0);
        }

        // ---- 2. S^T = K Q^T (lane: row col, keys kw + 4 g + e) ----
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < C::NCH; ++i) s = Mma16<TR>::mma(kf[i], qf[i], s);

        // ---- 3. chunk statistics ----
        float x[4];
        float mx = NEG_INF;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = kw + 4 * g + e;
            float t = s[e] * c_scale;
            bool ok = j < kend;
            if constexpr (MASK == MASK_ADD16 || MASK == MASK_ADD32)
                t = __builtin_fmaf(mask_value<MASK>(mr, e, p.mask_dtype), kLog2e, t);
            if constexpr (MASK == MASK_CAUSAL) ok = ok && (j <= qi + off);
            if constexpr (MASK == MASK_SLIDE) ok = ok && in_window(j, qi + off, p.window);
            if constexpr (MASK == MASK_BOOL) ok = ok && ((mr >> (8 * e)) & 0xffu) != 0u;
            x[e] = ok ? t : NEG_INF;
            mx = fmaxf(mx, x[e]);
        }
        mx = max_x32(max_x16(mx));
        if (g == 0) red[0][w][col] = mx;
        // V -> LDS transposed: 4 keys x 8 columns -> 8 rows of V^T, 4 keys (8 bytes) each
#pragma unroll
        for (int u = 0; u < C::VU; ++u) {
            const int idx = lane + 64 * u;
            if (idx < 4 * C::CPR) {
                const int q4 = idx & 3, c = idx >> 2;
#pragma unroll
                for (int wd = 0; wd < 4; ++wd) {
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const uint32_t sel = e ? 0x07060302u : 0x05040100u;
                        const uint32_t lo = __builtin_amdgcn_perm(vr[u][1][wd], vr[u][0][wd], sel);
                        const uint32_t hi = __builtin_amdgcn_perm(vr[u][3][wd], vr[u][2][wd], sel);
                        *reinterpret_cast<u32x2_t*>(&Vt[(8 * c + 2 * wd + e) * C::TP + 16 * w + 4 * q4]) =
                            u32x2_t{lo, hi};
                    }
                }
            }
        }
        // K, V and the mask of this chunk are consumed: the next chunk's loads
        // overlap this chunk's softmax and P V
        if constexpr (C::PREFETCH) {
            if (k0 + KS < kend) {
                issue_k(k0 + KS);
                issue_v(k0 + KS);
            }
        }
        __syncthreads();
        float mc = NEG_INF;
#pragma unroll
        for (int i = 0; i < NW; ++i) mc = fmaxf(mc, red[0][i][col]);
        const float m_new = fmaxf(m_run, mc);
        const float alpha = (m_new == NEG_INF) ? 1.f : fast_exp2(m_run - m_new);
        const float muse = (m_new == NEG_INF) ? 0.f : m_new;
        m_run = m_new;
        float ls = 0.f;
        float pe[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pe[e] = fast_exp2(x[e] - muse);
            ls += pe[e];
        }
        ls = sum_x32(sum_x16(ls));
        if (g == 0) red[1][w][col] = ls;
        *reinterpret_cast<u32x2_t*>(&Ps[col * C::PP + 16 * w + 4 * g]) =
            u32x2_t{TR::pack(pe[0], pe[1]), TR::pack(pe[2], pe[3])};
        __syncthreads();
        float lc = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) lc += red[1][i][col];
        l_run = l_run * alpha + lc;

        // ---- 4. O^T += V^T P^T over the chunk, this wave's head-dim blocks ----
#pragma unroll
        for (int i = 0; i < C::NDBW; ++i) {
            const int db = w + NW * i;
            if (db >= C::NDB) break;
            f32x4_t acc = oacc[i] * alpha;
#pragma unroll
            for (int ks = 0; ks < KS / 32; ++ks) {
                const u32x4_t bf = *reinterpret_cast<const u32x4_t*>(&Ps[col * C::PP + 32 * ks + 8 * g]);
                const uint16_t* vt = &Vt[(16 * db + col) * C::TP + 32 * ks + 8 * g];
                const u32x2_t a0 = reinterpret_cast<const u32x2_t*>(vt)[0];
                const u32x2_t a1 = reinterpret_cast<const u32x2_t*>(vt)[1];
                const u32x4_t af = {a0[0], a0[1], a1[0], a1[1]};
                acc = Mma16<TR>::mma(af, bf, acc);
            }
            oacc[i] = acc;
        }
        __syncthreads();  // Vt / Ps / red are rewritten by the next chunk
    }

    // ---- one split: this workgroup saw every key of its rows; normalise and
    // store the output (what the merge of a single split computes) ----
    if (p.splits == 1) {
        if (rv) {
            const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
            char* orow = reinterpret_cast<char*>(p.o) +
                         ((int64_t)b * p.os[0] + (int64_t)qh * p.os[1] + (int64_t)qi * p.os[2]) * 2;
#pragma unroll
            for (int i = 0; i < C::NDBW; ++i) {
                const int db = w + NW * i;
                if (db >= C::NDB) break;
                const int d = 16 * db + 4 * g;
                if (d < DO) TR::store4(orow + d * 2, oacc[i] * inv);
            }
        }
        return;
    }
    // ---- partial state of this split ----
    if (rv) {
        const int64_t row = ((int64_t)b * p.Hq + qh) * p.Lq + qi;
        float* po = p.ws_o + (row * p.splits + split) * DO;
#pragma unroll
        for (int i = 0; i < C::NDBW; ++i) {
            const int db = w + NW * i;
            if (db >= C::NDB) break;
            const int d = 16 * db + 4 * g;
            if (d < DO) *reinterpret_cast<f32x4_t*>(po + d) = oacc[i];
        }
        if (w == 0 && g == 0) {
            p.ws_ml[(row * p.splits + split) * 2 + 0] = m_run;
            p.ws_ml[(row * p.splits + split) * 2 + 1] = l_run;
        }
    }
}

}  // namespace sdpa_dev
