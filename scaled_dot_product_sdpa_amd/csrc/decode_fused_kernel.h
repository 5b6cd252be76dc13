// Single-launch split-key decode ("vector") kernel for 16-bit inputs on gfx950.
//
// Decode (q_len <= 8; mlx issue #3885, "Current routing": the vector kernel
// and its 2-pass variant that splits the keys over several threadgroups and
// merges them) is bound by reading K and V once from HBM.  Here the split and
// the merge happen in one launch:
//
//   * A group is (batch, kv head, column group): up to 16 query rows (query
//     heads of the kv head x query positions) that share every K/V byte.  Its
//     keys are split over S workgroups.
//   * Workgroup i of the 1-D grid serves group x + NX * ((i / NX) / S), split
//     (i / NX) % S, x = i % NX, with NX the device's XCD count.  Workgroups are
//     dispatched round-robin over the XCDs, so all S splits of a group run on
//     one XCD and exchange their partial results through that XCD's L2.
//   * Each wave streams 16-key blocks of its split: K rows straight into
//     v_mfma_f32_16x16x32 A-operand registers, V rows into registers and then
//     into a wave-private LDS block (rows padded to an odd multiple of 32
//     bytes, so the transposed reads below hit 64 distinct banks), with NB
//     blocks in flight.  Per block: S^T = K Q^T (keys x rows), the online
//     softmax (base 2, lazy rescale), and O^T += V^T P^T on
//     v_mfma_f32_16x16x16 with P^T straight from the score registers and V^T
//     from ds_read_b64_tr_b16.  No barrier inside the key loop.
//   * The waves' (O, m, l) are merged through LDS into the workgroup's
//     partial, which is stored to the workspace.  Then one atomic add on the
//     group's arrival word (count, sum and sum of squares of the XCC ids)
//     tells the workgroup whether it is the group's last; the last one merges
//     the S partials from L2 (log-sum-exp weights, fixed split order), writes
//     the output and resets the word to zero for the next call.
//   * Visibility: every store of a partial completes in L2 (s_waitcnt
//     vmcnt(0)) before the arrival add; the last workgroup invalidates its
//     vector L1 (buffer_inv sc0) before reading the partials -- the
//     release/acquire pair the compiler itself uses between the CUs of one
//     workgroup in threadgroup-split mode, i.e. between CUs sharing an L2.
//     That is only valid when the group's splits all ran on the last
//     workgroup's XCD, which the XCC-id sums prove (equal ids <=> sum = S x
//     and sum of squares = S x^2).  If they did not, the last workgroup
//     recomputes the whole group from K and V itself (never reading other
//     workgroups' partials) and counts the event in the workspace.
//   * S = 1 (enough groups to fill the chip): the workgroup normalises and
//     writes its output directly; no workspace traffic.
#pragma once

#include "attn_common.h"
#include "rope_kernel.h"

namespace sdpa_dev {

// Arrival word of a group: bits 0..7 count, 8..17 sum of XCC ids, 18..31 sum
// of their squares (S <= 32 splits, ids < 16).
// Each group's word sits on its own 128-byte line: the splits of one group add
// to it at nearly the same moment, and words sharing a line would serialise
// every group's adds in one L2 channel.
constexpr int kFusedMaxSplits = 32;
constexpr int kFusedCounterStride = 32;                      // words between two groups' arrival words
constexpr int kFusedCounterSlots = 256;
constexpr int kFusedCounterWords = kFusedCounterStride * kFusedCounterSlots;  // 32 KiB of the workspace
constexpr int kFusedFallbackWord = kFusedCounterStride * (kFusedCounterSlots - 1);  // groups recomputed by their last workgroup
constexpr int kFusedMaxGroups = kFusedCounterSlots - 1;

template <class TR, int D_, int DO_, int NW_>
struct DfCfg {
    static constexpr int D = D_, DO = DO_, NW = NW_, NT = 64 * NW;
    static constexpr int DOW = DO;                        // V / output columns of a group
    static constexpr int NCH = (D + 31) / 32;              // Q K^T steps of 32 head-dim columns
    static constexpr int DVP = (DOW + 15) / 16 * 16;       // V columns incl. pad to whole 16-column blocks
    static constexpr int NDB = DVP / 16;                   // O^T blocks (16 columns each)
    static constexpr int VCH = DOW / 8;                    // 16-byte chunks of a V row slice
    static constexpr int VCHP = DVP / 8;
    // LDS row pitch in 16-byte units: 2 x odd, so the 8 rows a transposed read
    // pass touches start on 8 distinct even bank groups
    static constexpr int PITCH = ((VCHP / 2) % 2 == 1) ? VCHP : VCHP + 2;
    static constexpr int VSLOTS = 16 * VCHP;               // 16-byte slots of one V block (incl. pad chunks)
    static constexpr int VU = (VSLOTS + 63) / 64;          // V load slots per lane per block
    static constexpr int LDS_V = NW * 16 * PITCH * 16;     // one V block per wave
    // per-wave O^T rows for the merge, padded to 16 banks past a multiple of 64: the
    // 4 x 4 lanes (row, column quad) of one 16-byte write per row then cover the 64
    // banks instead of 4-way conflicting on 1 KB rows
    static constexpr int OP = DVP + (80 - DVP % 64) % 64;
    // groups of up to RS rows keep the per-wave O^T beside the V blocks, so a wave
    // writes it as soon as its keys are done; more rows reuse the V blocks' LDS
    static constexpr int RS = 4;
    static constexpr int LDS_OS = LDS_V + NW * RS * OP * 4;  // V blocks + separate O^T
    static constexpr int LDS_OA = NW * 16 * OP * 4;          // O^T over the V blocks
    static constexpr int ML_OFF = LDS_OS > LDS_OA ? LDS_OS : LDS_OA;  // per-wave (m, l)
    static constexpr int LDS_M = ML_OFF + 2 * NW * 16 * 4;
    static constexpr int LDS_G = 16 * 32 * 4 + 2 * 16 * (DOW / 4) * 16;  // group merge: weights, half sums
    static constexpr int LDS_W = LDS_V > LDS_M ? (LDS_V > LDS_G ? LDS_V : LDS_G) : (LDS_M > LDS_G ? LDS_M : LDS_G);
    static constexpr int LDS = LDS_W;
    static_assert(DOW % 8 == 0, "V rows must be whole 16-byte chunks");
    static_assert(D % 8 == 0, "head dim must be whole 16-byte chunks");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Waves per workgroup of the single-launch kernel: eight (two per SIMD, one
// 16-key block each in flight) unless the per-wave output rows no longer fit
// the LDS merge area.
template <int DVP> struct DfWaves { static constexpr int value = DVP <= 256 ? 8 : 4; };

// v_mfma_f32_16x16x16: lane l holds A[l % 16][4 (l / 16) .. +3] and
// B[4 (l / 16) .. +3][l % 16]; C lane l: column l % 16, rows 4 (l / 16) .. +3.
template <class TR> struct Mma16k16;
template <> struct Mma16k16<TBF16> {
    static __device__ __forceinline__ f32x4_t mma(u32x2_t a, u32x2_t b, f32x4_t c) {
        typedef short s4_t __attribute__((ext_vector_type(4)));
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bitcast<s4_t>(a), bitcast<s4_t>(b), c, 0, 0, 0);
    }
};
template <> struct Mma16k16<TF16> {
    static __device__ __forceinline__ f32x4_t mma(u32x2_t a, u32x2_t b, f32x4_t c) {
        typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
        return __builtin_amdgcn_mfma_f32_16x16x16f16(bitcast<h4_t>(a), bitcast<h4_t>(b), c, 0, 0, 0);
    }
};

// Timeline build (SDPA_TRACE_DECODE=1, a separate library; off in the product
// build): each workgroup of a split group records the constant 100 MHz clock at
// the points below and writes them, 8 x 64 bits, to the workspace after the
// (m, l) partials (kTraceWords x 8 bytes per workgroup more workspace).
//   0 entry   1 wave 0's first block in registers   2 wave 0's keys done
//   3 every wave's keys done   4 partial stored in L2   5 arrival add returned
//   6 (last workgroup) output stored   7 xcc | last << 4 | split << 8 | group << 16
//   8 wave partials in LDS   9 partial stores issued   10 (last) weights in LDS
//   11 (last) weighted sums in LDS   12, 13 a second clock read right after 3 and 9
//   (the cost of a read)
#ifndef SDPA_TRACE_DECODE
#define SDPA_TRACE_DECODE 0
#endif
constexpr int kTraceWords = 14;
__device__ __forceinline__ uint64_t trace_clock() {
    uint64_t t;
    asm volatile("s_memrealtime %0\n s_waitcnt lgkmcnt(0)" : "=s"(t)::"memory");
    return t;
}

__device__ __forceinline__ uint32_t xcc_id() {
    return (uint32_t)__builtin_amdgcn_s_getreg((20) | (0 << 6) | ((16 - 1) << 11)) & 0xfu;  // HW_REG_XCC_ID[3:0]
}

template <class TR, class C, int MASK, bool ROPE = false>
__global__ __launch_bounds__(C::NT) void decode_fused_kernel(const Params p, const FusedGeom fg) {
    constexpr int D = C::D, NW = C::NW, NDB = C::NDB, DOW = C::DOW;
    constexpr float NEG_INF = -__builtin_inff();
    constexpr float kRescale = 8.0f;
    constexpr bool HAS_MT = (MASK == MASK_ADD16 || MASK == MASK_ADD32 || MASK == MASK_BOOL);
    constexpr int MES = MASK == MASK_BOOL ? 1 : (MASK == MASK_ADD16 ? 2 : 4);
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];
    __shared__ uint32_t s_word;
    char* const work = smem;

    // Every 64-byte line of the argument block into the scalar cache in one
    // batch (a load every 32 bytes reaches every line whatever the block's
    // alignment).  Left to itself the compiler issues the argument loads in
    // several batches, each waited for before the next, and every batch that
    // misses the scalar cache is another round trip to memory before the first
    // K/V load can go out.  The loads complete inside the asm statement.
    static_assert(sizeof(Params) + sizeof(FusedGeom) <= 0x1a0, "argument block larger than the lines touched");
    {
        const __attribute__((address_space(4))) char* ka =
            (const __attribute__((address_space(4))) char*)__builtin_amdgcn_kernarg_segment_ptr();
        uint32_t t0, t1, t2, t3, t4, t5, t6, t7, t8, t9, t10, t11, t12;
        asm volatile(
            "s_load_dword %0, %13, 0x0\n s_load_dword %1, %13, 0x20\n s_load_dword %2, %13, 0x40\n"
            "s_load_dword %3, %13, 0x60\n s_load_dword %4, %13, 0x80\n s_load_dword %5, %13, 0xa0\n"
            "s_load_dword %6, %13, 0xc0\n s_load_dword %7, %13, 0xe0\n s_load_dword %8, %13, 0x100\n"
            "s_load_dword %9, %13, 0x120\n s_load_dword %10, %13, 0x140\n s_load_dword %11, %13, 0x160\n"
            "s_load_dword %12, %13, 0x180\n s_waitcnt lgkmcnt(0)"
            : "=&s"(t0), "=&s"(t1), "=&s"(t2), "=&s"(t3), "=&s"(t4), "=&s"(t5), "=&s"(t6), "=&s"(t7), "=&s"(t8),
              "=&s"(t9), "=&s"(t10), "=&s"(t11), "=&s"(t12)
            : "s"(ka));
        asm volatile("" ::"s"(t0 ^ t1 ^ t2 ^ t3 ^ t4 ^ t5 ^ t6 ^ t7 ^ t8 ^ t9 ^ t10 ^ t11 ^ t12));
    }

    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g4 = lane >> 4;
    uint64_t tr[kTraceWords] = {};
    if constexpr (SDPA_TRACE_DECODE) tr[0] = trace_clock();

    // ---- group and split of this workgroup (32-bit: the host keeps nblk * S below 2^31) ----
    const int i = blockIdx.x;
    const int j = fast_div(i, fg.nx), x = i - j * fg.nx.d;
    const int js = fast_div(j, fg.splits), split = j - js * fg.splits.d;
    const int grp = x + fg.nx.d * js;
    // grp -> (b, kv head, column group); column group fastest
    const int bk = fast_div(grp, fg.colg), cg = grp - bk * fg.colg.d;
    const int b = fast_div(bk, fg.hkv), kvh = bk - b * fg.hkv.d;
    // split s streams the 16-key blocks [s nblk / S, (s + 1) nblk / S); wave w takes
    // blocks blk0 + w + NW n
    int blk0 = fast_div(split * fg.nblk, fg.splits), blk1 = fast_div((split + 1) * fg.nblk, fg.splits);

    // ---- K / V: buffer resources over this (batch, kv head); rows past Lk read as zero ----
    const uint32_t kstep32 = (uint32_t)(p.ks[2] * 2), vstep32 = (uint32_t)(p.vs[2] * 2);
    const char* kglob = reinterpret_cast<const char*>(p.k) + ((int64_t)b * p.ks[0] + (int64_t)kvh * p.ks[1]) * 2;
    const char* vglob = reinterpret_cast<const char*>(p.v) + ((int64_t)b * p.vs[0] + (int64_t)kvh * p.vs[1]) * 2;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kglob, (uint32_t)(p.Lk - 1) * kstep32 + (uint32_t)(D * 2));
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vglob, (uint32_t)(p.Lk - 1) * vstep32 + (uint32_t)(DOW * 2));

    // this lane's row of the group
    const int rows_g = min(16, p.n_rep * p.Lq - cg * 16);  // valid rows (<= fg.rv)
    const int r = col;
    const int rr = cg * 16 + (r < rows_g ? r : 0);
    const int rq = fast_div(rr, fg.lq), qh = kvh * p.n_rep + rq, qi = rr - rq * fg.lq.d;
    const int off = p.Lk - p.Lq;
    // mask tensor (key-contiguous, 4-key aligned rows, below 4 GiB: checked on the host): one
    // range-checked vector load per 4 keys
    const uint32_t mrow = HAS_MT ? (uint32_t)((int64_t)b * p.ms[0] + (int64_t)qh * p.ms[1] + (int64_t)qi * p.ms[2]) : 0u;
    const __amdgpu_buffer_rsrc_t mrs = make_rsrc(HAS_MT ? p.mask : nullptr, HAS_MT ? (uint32_t)p.mask_span : 0u);

    uint32_t* const words = reinterpret_cast<uint32_t*>(p.ws_o);
    float* const part_o = reinterpret_cast<float*>(reinterpret_cast<char*>(p.ws_o) + kFusedCounterWords * 4);
    float* const part_ml = p.ws_ml;
    const int S = fg.splits.d, RV = fg.rv;
    bool direct = S == 1;
    // timeline build: this workgroup's record, past the (m, l) partials (256-byte aligned)
    auto trace_store = [&](bool last) __attribute__((always_inline)) {
        if constexpr (SDPA_TRACE_DECODE) {
            if (tid == 0 && S > 1) {
                const size_t slots = (size_t)fg.groups * S * RV;
                uint64_t* rec = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(part_ml) +
                                                            (slots * 8 + 255) / 256 * 256) +
                                (size_t)blockIdx.x * kTraceWords;
                tr[7] = (uint64_t)xcc_id() | ((uint64_t)last << 4) | ((uint64_t)split << 8) | ((uint64_t)grp << 16);
#pragma unroll
                for (int k = 0; k < kTraceWords; ++k) rec[k] = tr[k];
            }
        }
    };
    char* const vlds = work + w * (16 * C::PITCH * 16);
    // transposed-read offsets: lane (g4, e = (lane % 16) / 4, q = lane % 4) names row 4 g4 + e,
    // columns 16 db + 4 q .. + 3
    const uint32_t tr_off = (uint32_t)((4 * g4 + ((lane & 15) >> 2)) * C::PITCH * 16 + (lane & 3) * 8);

    // Q fragments (B operand of S^T = K Q^T): row r, head-dim columns 32 c + 8 g4 .. +7,
    // zero for rows past the group (finite scores that are never stored; no load).
    // Loaded first: a wave's loads return in order, and S needs Q with the first K.
    u32x4_t qf[C::NCH];
    {
        const char* qrow = reinterpret_cast<const char*>(p.q) +
                           ((int64_t)b * p.qs[0] + (int64_t)qh * p.qs[1] + (int64_t)qi * p.qs[2]) * 2;
#pragma unroll
        for (int c = 0; c < C::NCH; ++c) {
            const int d = 32 * c + 8 * g4;
            qf[c] = (d < D && r < rows_g) ? *reinterpret_cast<const u32x4_t*>(qrow + d * 2) : u32x4_t{0u, 0u, 0u, 0u};
        }
        if constexpr (ROPE)
            rope_q_fragments<TR, C::NCH, 32>(qf, qrow, 8 * g4, p.rope_dim, p.rope_cos, p.rope_sin,
                                             (int64_t)p.rope_pos0 + qi);
    }
    const float c_scale = p.scale_log2;

    // one 16-key block in flight per wave: K straight into A-operand registers, V rows, mask group
    u32x4_t kf[C::NCH];
    u32x4_t vr[C::VU];
    typename MaskRaw<MASK>::type mr{};
    auto issue = [&](int n) __attribute__((always_inline)) {
        const int k0 = p.kbase + (blk0 + w + NW * n) * 16;
#pragma unroll
        for (int c = 0; c < C::NCH; ++c) {
            const int d = 32 * c + 8 * g4;
            kf[c] = u32x4_t{0u, 0u, 0u, 0u};
            if (d < D) kf[c] = buffer_load16_nt(krs, (uint32_t)(k0 + col) * kstep32 + (uint32_t)(d * 2));
        }
#pragma unroll
        for (int u = 0; u < C::VU; ++u) {
            const int s = 64 * u + lane;
            const int row = s / C::VCHP, ch = s % C::VCHP;
            vr[u] = u32x4_t{0u, 0u, 0u, 0u};
            if (s < C::VSLOTS && ch < C::VCH)
                vr[u] = buffer_load16_nt(vrs, (uint32_t)(k0 + row) * vstep32 + (uint32_t)(ch * 16));
        }
        if constexpr (HAS_MT) mr = load_mask_group_rs<MASK>(mrs, (mrow + (uint32_t)(k0 + 4 * g4)) * MES);
    };
    auto count_mine = [&]() { return blk1 - blk0 > w ? (blk1 - blk0 - w + NW - 1) / NW : 0; };
    int nmine = count_mine();
    if (nmine > 0) issue(0);

    // ---- the keys of this split's blocks, merged over the waves into this workgroup's
    // (O, m, l) for the group's rows; `direct`: normalise and write the output ----
    for (;;) {
        float m_run = NEG_INF, l_run = 0.f;
        f32x4_t oacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        for (int n = 0; n < nmine; ++n) {
            const int k0 = p.kbase + (blk0 + w + NW * n) * 16;
            // V block -> LDS (row-major, padded rows)
#pragma unroll
            for (int u = 0; u < C::VU; ++u) {
                const int s = 64 * u + lane;
                if (s < C::VSLOTS) {
                    const int row = s / C::VCHP, ch = s % C::VCHP;
                    *reinterpret_cast<u32x4_t*>(vlds + (row * C::PITCH + ch) * 16) = vr[u];
                }
            }
            // S^T = K Q^T: lane (row r, keys k0 + 4 g4 + e)
            f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < C::NCH; ++c) sc = Mma16<TR>::mma(kf[c], qf[c], sc);
            if constexpr (SDPA_TRACE_DECODE) {
                if (n == 0 && tr[1] == 0) {
                    asm volatile("" ::"v"(sc[0]) : "memory");  // after this block's products
                    tr[1] = trace_clock();
                }
            }
            const typename MaskRaw<MASK>::type mk = mr;
            // K, V registers consumed: the next block streams during this one's softmax and P V
            if (n + 1 < nmine) issue(n + 1);

            float xs[4];
            float bm = NEG_INF;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int jk = k0 + 4 * g4 + e;
                float v = sc[e] * c_scale;
                bool ok = jk < p.Lk;
                if constexpr (MASK == MASK_ADD16 || MASK == MASK_ADD32)
                    v = __builtin_fmaf(mask_value<MASK>(mk, e, p.mask_dtype), kLog2e, v);
                if constexpr (MASK == MASK_CAUSAL) ok = ok && (jk <= qi + off);
                if constexpr (MASK == MASK_SLIDE) ok = ok && in_window(jk, qi + off, p.window);
                if constexpr (MASK == MASK_BOOL) ok = ok && ((mk >> (8 * e)) & 0xffu) != 0u;
                xs[e] = ok ? v : NEG_INF;
                bm = fmaxf(bm, xs[e]);
            }
            bm = max_x32(max_x16(bm));  // the block max of row r, in all four lanes of the row
            // lazy rescale: a row's max moves only when the block's max exceeds it by
            // more than 2^8; a row that has seen no finite score has nothing to rescale
            const bool grow = bm > m_run + kRescale;
            if (__any(grow)) {
                const float m_new = grow ? bm : m_run;
                if (__any(grow && m_run != NEG_INF)) {
                    const float alpha = (grow && m_run != NEG_INF) ? fast_exp2(m_run - m_new) : 1.f;
                    l_run *= alpha;
#pragma unroll
                    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
                }
                m_run = m_new;
            }
            const float muse = (m_run == NEG_INF) ? 0.f : m_run;
            float pe[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pe[e] = fast_exp2(xs[e] - muse);
                l_run += pe[e];
            }
            const u32x2_t pb = {TR::pack(pe[0], pe[1]), TR::pack(pe[2], pe[3])};
            // O^T += V^T P^T, V^T through transposed LDS reads of this wave's block
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const u32x2_t a = lds_read_tr16(vlds + tr_off + db * 32);
                oacc[db] = Mma16k16<TR>::mma(a, pb, oacc[db]);
            }
        }
        const float l_row = sum_x32(sum_x16(l_run));
        if constexpr (SDPA_TRACE_DECODE) {
            asm volatile("" ::"v"(l_row) : "memory");
            if (tr[2] == 0) tr[2] = trace_clock();
        }

        // ---- merge the waves through LDS: wave w's O^T, m, l of rows < RV ----
        // (up to RS rows: written beside the V blocks as soon as this wave is done;
        // more: over the V blocks, once every wave is done with its block)
        const bool sep = RV <= C::RS;
        const int orw = sep ? C::RS : 16;  // O^T rows per wave in LDS
        float* lo = reinterpret_cast<float*>(work + (sep ? C::LDS_V : 0));
        float* lml = reinterpret_cast<float*>(work + C::ML_OFF);
        auto put = [&]() __attribute__((always_inline)) {
            if (r < RV) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    *reinterpret_cast<f32x4_t*>(lo + ((w * orw + r) * C::OP + 16 * db + 4 * g4)) = oacc[db];
                if (g4 == 0) {
                    lml[(w * 16 + r) * 2] = m_run;
                    lml[(w * 16 + r) * 2 + 1] = l_row;
                }
            }
        };
        if (sep) put();
        __syncthreads();  // every wave is done with its keys (and, up to RS rows, its partial is in LDS)
        if constexpr (SDPA_TRACE_DECODE) {
            if (tr[3] == 0) {
                tr[3] = trace_clock();
                tr[12] = trace_clock();
            }
        }
        if (!sep) {
            put();
            __syncthreads();
        }
        if constexpr (SDPA_TRACE_DECODE) {
            if (tr[8] == 0) tr[8] = trace_clock();
        }
        // thread -> (row, 4 columns) items of the group's partial
        constexpr int QPR = DOW / 4;  // column quads per row
        const int nitems = RV * QPR;
        for (int it = tid; it < nitems; it += C::NT) {
            const int row = it / QPR, c4 = (it % QPR) * 4;
            // every wave's (m, l) and O^T quad read at once (left to itself the compiler
            // waited for each wave's read before issuing the next)
            f32x2_t mlw[NW];
            f32x4_t ow[NW];
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                mlw[ww] = *reinterpret_cast<const f32x2_t*>(lml + (ww * 16 + row) * 2);
                ow[ww] = *reinterpret_cast<const f32x4_t*>(lo + ((ww * orw + row) * C::OP + c4));
            }
            float M = NEG_INF;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, mlw[ww][0]);
            f32x4_t o = {0.f, 0.f, 0.f, 0.f};
            float l = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                const float wt = (mlw[ww][0] == NEG_INF) ? 0.f : fast_exp2(mlw[ww][0] - M);
                l = __builtin_fmaf(wt, mlw[ww][1], l);
                o += wt * ow[ww];
            }
            if (direct) {
                if (row < rows_g) {
                    const int rg = cg * 16 + row;
                    const int rgq = fast_div(rg, fg.lq), oqh = kvh * p.n_rep + rgq, oqi = rg - rgq * fg.lq.d;
                    const float inv = l > 0.f ? 1.f / l : 0.f;
                    char* dst = reinterpret_cast<char*>(p.o) +
                                ((int64_t)b * p.os[0] + (int64_t)oqh * p.os[1] + (int64_t)oqi * p.os[2] + c4) * 2;
                    TR::store4(dst, o * inv);
                }
            } else {
                const int64_t slot = ((int64_t)grp * S + split) * RV + row;
                *reinterpret_cast<f32x4_t*>(part_o + slot * DOW + c4) = o;
                if (c4 == 0) *reinterpret_cast<f32x2_t*>(part_ml + slot * 2) = f32x2_t{M, l};
            }
        }
        if (direct) return;
        if constexpr (SDPA_TRACE_DECODE) {
            tr[9] = trace_clock();
            tr[13] = trace_clock();
        }

        // ---- arrival: partial stores complete in L2, then one add on the group's word ----
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if constexpr (SDPA_TRACE_DECODE) tr[4] = trace_clock();
        const uint32_t xc = xcc_id();
        if (tid == 0) {
            const uint32_t add = 1u + (xc << 8) + ((xc * xc) << 18);
            s_word = __hip_atomic_fetch_add(&words[grp * kFusedCounterStride], add, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) + add;
        }
        __syncthreads();
        const uint32_t word = s_word;
        if constexpr (SDPA_TRACE_DECODE) tr[5] = trace_clock();
        if ((int)(word & 0xffu) != S) {  // not the last split of the group
            trace_store(false);
            return;
        }
        if (tid == 0)
            __hip_atomic_exchange(&words[grp * kFusedCounterStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool one_xcd = ((word >> 8) & 0x3ffu) == (uint32_t)S * xc && (word >> 18) == (uint32_t)S * xc * xc;
        if (!one_xcd) {
            // the splits ran on several XCDs: their partials may sit in other L2s.
            // Recompute the whole group here and write the output directly.
            if (tid == 0) __hip_atomic_fetch_add(&words[kFusedFallbackWord], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            blk0 = 0;
            blk1 = fg.nblk;
            nmine = count_mine();
            direct = true;
            __syncthreads();  // LDS of the merge is reused by the next pass
            if (nmine > 0) issue(0);
            continue;
        }
        asm volatile("buffer_inv sc0" ::: "memory");  // this CU's L1 holds no stale partial lines

        // ---- merge the S partials of the group (fixed split order) ----
        // buffer resources over the group's partials: loads past them (splits >= S,
        // rows or items without a partial) read zero
        const int64_t gbase = (int64_t)grp * S * RV;
        const __amdgpu_buffer_rsrc_t ors = make_rsrc(part_o + gbase * DOW, (uint32_t)(S * RV * DOW * 4));
        const __amdgpu_buffer_rsrc_t mls = make_rsrc(part_ml + gbase * 2, (uint32_t)(S * RV * 8));
        // (m, l) of the group's S x RV slots (wave w, lane s: split s of rows w, w + NW, ...),
        // requested together with the first item's S partial rows
        constexpr int RPW = (16 + NW - 1) / NW;
        f32x2_t ml[RPW];
#pragma unroll
        for (int k = 0; k < RPW; ++k) {
            const int rw = w + NW * k;
            const uint32_t o8 = (rw < rows_g && lane < S) ? (uint32_t)((lane * RV + rw) * 8) : 0x80000000u;
            ml[k] = bitcast<f32x2_t>(__builtin_amdgcn_raw_buffer_load_b64(mls, o8, 0, 0));
        }
        // work units (item, half of the splits): 16 partial loads in flight per thread
        constexpr int MAXS = kFusedMaxSplits, HS = MAXS / 2;
        const int halves = (S + HS - 1) / HS;
        const int nunits = nitems * halves;
        f32x4_t pv[HS];
        auto load_unit = [&](int u) __attribute__((always_inline)) {
            const int it = u % nitems, h = u / nitems;
            const int row = it / QPR, c4 = (it % QPR) * 4;
            // (a unit without a partial starts 2 GiB out, past the range for every split)
            const uint32_t vo = (u < nunits && row < rows_g) ? (uint32_t)(((h * HS) * RV * DOW + row * DOW + c4) * 4)
                                                             : 0x80000000u;
#pragma unroll
            for (int k = 0; k < HS; ++k)  // split h HS + k at byte offset k * RV * DOW * 4 further on
                pv[k] = bitcast<f32x4_t>(
                    __builtin_amdgcn_raw_buffer_load_b128(ors, vo + (uint32_t)(k * RV * DOW * 4), 0, 0));
        };
        load_unit(tid);
        // per row: M = max_s m_s and normalised weights 2^(m_s - M) / sum_s 2^(m_s - M) l_s
        float* const wts = reinterpret_cast<float*>(work);  // [16 rows][MAXS]
        f32x4_t* const ob = reinterpret_cast<f32x4_t*>(work + 16 * MAXS * 4);  // [halves][nitems] sums
#pragma unroll
        for (int k = 0; k < RPW; ++k) {
            const int rw = w + NW * k;
            if (rw >= rows_g) break;
            const float M = wave_max(ml[k][0]);
            const float wt = (ml[k][0] == NEG_INF) ? 0.f : fast_exp2(ml[k][0] - M);
            const float den = wave_sum(wt * ml[k][1]);
            if (lane < MAXS) wts[rw * MAXS + lane] = (den > 0.f && lane < S) ? wt / den : 0.f;
        }
        __syncthreads();
        if constexpr (SDPA_TRACE_DECODE) tr[10] = trace_clock();
        for (int u = tid; u < nunits; u += C::NT) {
            if (u != tid) load_unit(u);
            const int it = u % nitems, h = u / nitems;
            const int row = it / QPR;
            f32x4_t o = {0.f, 0.f, 0.f, 0.f};
            if (row < rows_g) {
#pragma unroll
                for (int k = 0; k < HS; k += 4) {
                    const f32x4_t w4 = *reinterpret_cast<const f32x4_t*>(wts + row * MAXS + h * HS + k);
#pragma unroll
                    for (int e = 0; e < 4; ++e) o += w4[e] * pv[k + e];
                }
            }
            ob[h * nitems + it] = o;
        }
        __syncthreads();
        if constexpr (SDPA_TRACE_DECODE) tr[11] = trace_clock();
        for (int it = tid; it < nitems; it += C::NT) {
            const int row = it / QPR, c4 = (it % QPR) * 4;
            if (row >= rows_g) continue;
            f32x4_t o = ob[it];
            for (int h = 1; h < halves; ++h) o += ob[h * nitems + it];
            const int rg = cg * 16 + row;
            const int rgq = fast_div(rg, fg.lq), oqh = kvh * p.n_rep + rgq, oqi = rg - rgq * fg.lq.d;
            char* dst = reinterpret_cast<char*>(p.o) +
                        ((int64_t)b * p.os[0] + (int64_t)oqh * p.os[1] + (int64_t)oqi * p.os[2] + c4) * 2;
            TR::store4(dst, o);
        }
        if constexpr (SDPA_TRACE_DECODE) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            tr[6] = trace_clock();
            trace_store(true);
        }
        return;
    }
}

}  // namespace sdpa_dev
