// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// Layout conventions used throughout (CDNA matrix-core operand layout of
// v_mfma_f32_32x32x{16 bf16|16 f16|2 f32}: 64 lanes, lane l works on row/column
// l % 32 and on the K-half h = l / 32):
//   * scores are computed transposed, S^T = K Q^T: keys are the MFMA's M axis,
//     queries its N axis, head_dim its K axis.  The 16 accumulator registers
//     of lane l then hold query (l % 32) against keys
//         key(r, h) = 8 * (r / 4) + 4 * h + (r % 4),   r = 0..15
//     of a 32-key block, so each query's softmax runs inside one lane plus
//     one exchange with lane l ^ 32;
//   * O is accumulated transposed too, O^T = V^T P^T: the probabilities P^T
//     stay in the registers the scores came from and feed the MFMA's B operand
//     directly; V^T (head_dim x keys) is the A operand, read from an LDS copy
//     of the V tile stored transposed.
// Any permutation of the contraction index is allowed as long as A and B use
// the same one; the code pairs them explicitly ("chunk" = 16 bytes per lane).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa_dev {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Kernel mask variants.  The C ABI's additive kind maps to MASK_ADD16
// (bf16 / f16 mask) or MASK_ADD32 (float32 mask); MASK_SLIDE is the causal
// mask limited to a window of the most recent `window` keys.
enum { MASK_NONE = 0, MASK_ADD16 = 1, MASK_BOOL = 2, MASK_CAUSAL = 3, MASK_ADD32 = 4, MASK_SLIDE = 5, MASK_VARIANTS = 6 };

// key j is live for the query at position pos (= row + Lk - Lq) under MASK_SLIDE
__device__ __forceinline__ bool in_window(int j, int pos, int window) { return j <= pos && j > pos - window; }
enum { MDT_F32 = 0, MDT_F16 = 1, MDT_BF16 = 2, MDT_U8 = 3 };

constexpr float kLog2e = 1.4426950408889634f;

// Everything a launch needs; strides in elements, logical (b, h, l, d) order.
struct Params {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int64_t qs[4], ks[4], vs[4], os[4];
    const void* mask;
    int64_t ms[4];
    int mask_dtype;   // MDT_*
    int mask_vec;     // 1: key stride 1 and 4-element runs aligned -> vector loads
    int64_t mask_span;  // bytes from `mask` to one past its last element
    int B, Lq, Lk, Hq, Hkv, n_rep;
    float scale_log2;  // scale * log2(e)
    int scale_nonneg;  // scale >= 0: the row max can be taken on unscaled scores
    // vector (decode) kernel
    float* ws_o;      // [B*Hq*Lq][splits][D] unnormalised partial outputs
    float* ws_ml;     // [B*Hq*Lq][splits][2] running max (log2 domain) and sum
    int splits;
    int keys_per_split;
    int col_groups;   // decode: column groups per kv head
    int kbase;        // decode: first key of split 0 (keys before it are masked for every row)
    int window;       // MASK_SLIDE: keys per query (>= 1)
    int pairs;        // prefill, causal: a workgroup takes row tiles t and last - t
    int nx;           // XCD count of the device: workgroup i runs on XCD i % nx
    // rotary embedding of Q (0 = none): columns [0, rope_dim) of query row i
    // turn by the table angles of position rope_pos0 + i ([n_pos][rope_dim / 2] fp32)
    int rope_dim;
    int rope_pos0;
    const float* rope_cos;
    const float* rope_sin;
    // boolean mask as lane words (prefill, head dim <= 128; mask_bits.h): the 64 words
    // of (b, h, 32-row block rb, key tile kt) start at b * mb_b + h * mb_h + rb * mb_rb
    // + 64 kt (mb_b, mb_h 0 where the mask is broadcast)
    const uint32_t* mask_bits;
    int mb_b, mb_h, mb_rb, mb_pad;
};

template <class To, class From>
__device__ __forceinline__ To bitcast(const From& x) {
    static_assert(sizeof(To) == sizeof(From), "bitcast size");
    return __builtin_bit_cast(To, x);
}

// Round-to-nearest-even float -> bf16 / f16 pairs, packed low = a, high = b
// (one v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 per pair).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return bitcast<uint32_t>(__builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    return bitcast<uint32_t>(__builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}

// ---------------------------------------------------------------------------
// Element-type traits.  A "chunk" is 16 bytes per lane: EPC elements.  One
// chunk of A and one of B per lane feed CH_MFMA matrix instructions that
// together contract KCH indices (both lane halves).
// ---------------------------------------------------------------------------
struct TBF16 {
    static constexpr int ES = 2, EPC = 8, KCH = 16, DT = MDT_BF16;
    static __device__ __forceinline__ f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8_t>(a), bitcast<bf16x8_t>(b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_bf16(a, b); }
    static __device__ __forceinline__ float unpack_lo(uint32_t u) { return __uint_as_float(u << 16); }
    static __device__ __forceinline__ float unpack_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
    static __device__ __forceinline__ void store4(void* dst, f32x4_t x) {
        u32x2_t w = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
        *reinterpret_cast<u32x2_t*>(dst) = w;
    }
    static __device__ __forceinline__ void store1(void* dst, float x) {
        *reinterpret_cast<uint16_t*>(dst) = bitcast<uint16_t>((__bf16)x);
    }
};

struct TF16 {
    static constexpr int ES = 2, EPC = 8, KCH = 16, DT = MDT_F16;
    static __device__ __forceinline__ f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<f16x8_t>(a), bitcast<f16x8_t>(b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_f16(a, b); }
    static __device__ __forceinline__ float unpack_lo(uint32_t u) { return (float)bitcast<_Float16>((uint16_t)u); }
    static __device__ __forceinline__ float unpack_hi(uint32_t u) {
        return (float)bitcast<_Float16>((uint16_t)(u >> 16));
    }
    static __device__ __forceinline__ void store4(void* dst, f32x4_t x) {
        u32x2_t w = {pack_f16(x[0], x[1]), pack_f16(x[2], x[3])};
        *reinterpret_cast<u32x2_t*>(dst) = w;
    }
    static __device__ __forceinline__ void store1(void* dst, float x) {
        *reinterpret_cast<uint16_t*>(dst) = bitcast<uint16_t>((_Float16)x);
    }
};

// 16x16x32 MFMA (lane l: column l % 16, rows 4 * (l / 16) + i of the output)
template <class TR> struct Mma16;
template <> struct Mma16<TBF16> {
    static __device__ __forceinline__ f32x4_t mma(u32x4_t a, u32x4_t b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(a), bitcast<bf16x8_t>(b), c, 0, 0, 0);
    }
};
template <> struct Mma16<TF16> {
    static __device__ __forceinline__ f32x4_t mma(u32x4_t a, u32x4_t b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8_t>(a), bitcast<f16x8_t>(b), c, 0, 0, 0);
    }
};

// float32 stays float32 end to end: v_mfma_f32_32x32x2_f32, no reduced-precision mode.
struct TF32 {
    static constexpr int ES = 4, EPC = 4, KCH = 8, DT = MDT_F32;
    static __device__ __forceinline__ f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i]), __uint_as_float(b[i]), c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ void store4(void* dst, f32x4_t x) {
        *reinterpret_cast<f32x4_t*>(dst) = x;
    }
    static __device__ __forceinline__ void store1(void* dst, float x) { *reinterpret_cast<float*>(dst) = x; }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer resource over [base, base + bytes): a load whose 32-bit offset is
// >= bytes returns zero without touching memory (hardware range check).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return bitcast<u32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// The same with the non-temporal cache policy (nt): for K / V bytes a decode
// call reads exactly once.  The lines stream through the caches instead of
// being kept; the single-launch decode of 33.5 MB ran 7% faster with it (the
// sc0 / sc1 bits on top made no further difference).  The split kernel, whose
// two halves of a K line are requested far apart, ran 2% slower with it and
// keeps the default policy.
__device__ __forceinline__ u32x4_t buffer_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return bitcast<u32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

// 16 bytes per lane, global -> LDS without passing through registers: lane l
// writes at lds_base + 16 * l (buffer_load_dwordx4 ... lds).  The builtin
// exists for the device target only; the host pass sees an empty body.
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, off, 0, 0, 0);
#endif
}
// The same with a wave-uniform part of the offset in soffset (an SGPR).
__device__ __forceinline__ void buffer_load16_lds_so(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t voff,
                                                     uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, soff, 0, 0);
#endif
}
// The same two loads issued from inline assembly, unseen by the compiler's
// wait-count pass.  That pass takes every ds_read_b64_tr_b16 as aliasing
// every LDS DMA in flight and puts an s_waitcnt vmcnt(0) in front of the
// first one: a P V step would wait for the NEXT tile's loads, and the
// prefetch would overlap only the score half of a tile.  The kernels that
// use these order their DMA themselves: each tile starts with an explicit
// vmcnt(0) and a barrier before any wave reads it, and a stage is refilled
// only after that barrier, once every wave is done reading it.  The loads
// have no register results (nothing for the compiler to track); M0 carries
// the LDS base, with the one wait state the DMA needs after writing it.
// Compiler-issued vector loads newer than these get waits counted without
// them, which only makes those waits stricter.
// LDS byte address of a pointer into a __shared__ array (the M0 value the
// DMA wants).  Taken once from the array itself, where the compiler knows
// the address space; offsets are then plain integer adds.
__device__ __forceinline__ uint32_t lds_address(const void* shared_array) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)shared_array;
}
__device__ __forceinline__ void dma16_lds(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "memory");
#endif
}
__device__ __forceinline__ void dma16_lds_so(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, uint32_t voff,
                                             uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r),
                 "s"(__builtin_amdgcn_readfirstlane(soff)), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "memory");
#endif
}

// ds_read_b64_tr_b16: in each 16-lane group, output lane i element e is
// element i % 4 of the 4 values at the address of source lane 4 e + i / 4.
__device__ __forceinline__ u32x2_t lds_read_tr16(const void* addr) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef short v4i16_t __attribute__((ext_vector_type(4)));
    return bitcast<u32x2_t>(__builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16_t*)(const_cast<void*>(addr))));
#else
    return u32x2_t{0u, 0u};
#endif
}

// Cross-lane exchanges without an LDS round trip.  v_permlane32_swap on (x, x)
// leaves lane i holding (x[i mod 32], x[i mod 32 + 32]) and v_permlane16_swap
// (x[i & ~16], x[i | 16]) for each 32-lane half: both partners of an xor-32
// (xor-16) pair, in the same order in both lanes of the pair.
__device__ __forceinline__ f32x2_t pair32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return f32x2_t{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ f32x2_t pair16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return f32x2_t{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// the value of lane i ^ 32
__device__ __forceinline__ float xor32(float x) {
    const f32x2_t r = pair32(x);
    return (threadIdx.x & 32) ? r[0] : r[1];
}
// max / sum over lanes i and i ^ 32 (i ^ 16): the same float in both lanes
__device__ __forceinline__ float max_x32(float x) { const f32x2_t r = pair32(x); return fmaxf(r[0], r[1]); }
__device__ __forceinline__ float sum_x32(float x) { const f32x2_t r = pair32(x); return r[0] + r[1]; }
__device__ __forceinline__ float max_x16(float x) { const f32x2_t r = pair16(x); return fmaxf(r[0], r[1]); }
__device__ __forceinline__ float sum_x16(float x) { const f32x2_t r = pair16(x); return r[0] + r[1]; }

// max / sum over all 64 lanes of a wave, the result in every lane: quad
// exchanges and row mirrors (DPP) reduce each 16-lane row, then the two lane
// swaps above combine the rows.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_mov<0xB1>(x));   // quad_perm [1, 0, 3, 2]
    x = fmaxf(x, dpp_mov<0x4E>(x));   // quad_perm [2, 3, 0, 1]
    x = fmaxf(x, dpp_mov<0x141>(x));  // row_half_mirror
    x = fmaxf(x, dpp_mov<0x140>(x));  // row_mirror
    return max_x32(max_x16(x));
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_mov<0xB1>(x);
    x += dpp_mov<0x4E>(x);
    x += dpp_mov<0x141>(x);
    x += dpp_mov<0x140>(x);
    return sum_x32(sum_x16(x));
}

// ---------------------------------------------------------------------------
// Masks are read in groups of 4 consecutive keys (the 4 keys one lane holds
// per accumulator group).  Raw form kept in registers until use:
//   MASK_BOOL  : 1 dword, byte r = key r (nonzero = attend)
//   MASK_ADD16 : 2 dwords, 16-bit values of keys 0..3 (bf16 or f16)
//   MASK_ADD32 : 4 dwords, float32 values of keys 0..3
// A tile's groups are loaded right after the previous tile's softmax, so the
// load overlaps that tile's P V products and the next tile's Q K^T.
// Keys >= Lk read as "masked" / 0 and are masked separately.
// ---------------------------------------------------------------------------
template <int MASK> struct MaskRaw { using type = uint32_t; };           // MASK_BOOL: 4 bytes
template <> struct MaskRaw<MASK_ADD16> { using type = u32x2_t; };         // 4 x 16-bit
template <> struct MaskRaw<MASK_ADD32> { using type = u32x4_t; };         // 4 x float32

template <int MASK>
__device__ __forceinline__ typename MaskRaw<MASK>::type load_mask_group(const Params& p, int64_t mrow, int key0) {
    using R = typename MaskRaw<MASK>::type;
    const char* base = reinterpret_cast<const char*>(p.mask);
    if (p.mask_vec && key0 + 3 < p.Lk) {
        if constexpr (MASK == MASK_BOOL) return *reinterpret_cast<const uint32_t*>(base + mrow + key0);
        else if constexpr (MASK == MASK_ADD16) return *reinterpret_cast<const u32x2_t*>(base + (mrow + key0) * 2);
        else return *reinterpret_cast<const u32x4_t*>(base + (mrow + key0) * 4);
    }
    R r{};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int j = key0 + k;
        if (j >= p.Lk) continue;
        const int64_t o = mrow + (int64_t)j * p.ms[3];
        if constexpr (MASK == MASK_BOOL) {
            r |= (base[o] ? 1u : 0u) << (8 * k);
        } else if constexpr (MASK == MASK_ADD16) {
            const uint32_t u = reinterpret_cast<const uint16_t*>(base)[o];
            r[k >> 1] |= u << (16 * (k & 1));
        } else {
            r[k] = reinterpret_cast<const uint32_t*>(base)[o];
        }
    }
    return r;
}

// The same group through a buffer resource whose range ends at the mask's
// last byte (mask_vec layouts only): one vector load, no branch; bytes past
// the range read as zero.
template <int MASK>
__device__ __forceinline__ typename MaskRaw<MASK>::type load_mask_group_rs(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (MASK == MASK_BOOL) return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    else if constexpr (MASK == MASK_ADD16) return bitcast<u32x2_t>(__builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    else return bitcast<u32x4_t>(__builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Any other layout: the group's 4 elements one by one (element offsets
// row_off + (key0 + k) * key_stride), through the same kind of resource.
// The prefill kernels take this path in a separate instantiation (SMASK):
// the compiler keeps a per-lane offset for every group of a tile live across
// the key loop, registers the vector path must not pay for.
template <int MASK>
__device__ __forceinline__ typename MaskRaw<MASK>::type load_mask_group_rs_strided(__amdgpu_buffer_rsrc_t r,
                                                                                    uint32_t row_off, int key0,
                                                                                    uint32_t key_stride) {
    typename MaskRaw<MASK>::type g{};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t e = row_off + (uint32_t)(key0 + k) * key_stride;
        if constexpr (MASK == MASK_BOOL) {
            g |= (__builtin_amdgcn_raw_buffer_load_b8(r, e, 0, 0) ? 1u : 0u) << (8 * k);
        } else if constexpr (MASK == MASK_ADD16) {
            g[k >> 1] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, e * 2, 0, 0) << (16 * (k & 1));
        } else {
            g[k] = __builtin_amdgcn_raw_buffer_load_b32(r, e * 4, 0, 0);
        }
    }
    return g;
}

// Additive mask value of key k (0..3) of a raw group, widened to float.
template <int MASK>
__device__ __forceinline__ float mask_value(const typename MaskRaw<MASK>::type& r, int k, int mdt) {
    if constexpr (MASK == MASK_ADD32) {
        return __uint_as_float(r[k]);
    } else {
        const uint32_t w = r[k >> 1];
        const uint32_t h = (k & 1) ? (w >> 16) : (w & 0xffffu);
        if (mdt == MDT_BF16) return __uint_as_float(h << 16);
        return (float)bitcast<_Float16>((uint16_t)h);
    }
}

// Geometry of the single-launch decode kernel (decode_fused_kernel.h).
// Division by a divisor fixed for a launch, after Granlund and Montgomery,
// "Division by Invariant Integers using Multiplication" (PLDI 1994), with the
// rounded-up multiplier: for 1 <= d < 2^31 let l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, which fits 32 bits; then for
// 0 <= n < 2^31, n / d = (umulhi(n, m) + n) >> l.  The sum cannot overflow
// (umulhi(n, m) <= n < 2^31).  One multiply-high, one add and one shift in
// place of the thirty-odd instructions of a general 32-bit division.
struct FastDiv {
    int d;
    uint32_t m;
    uint32_t l;
};

inline FastDiv make_fastdiv(int d) {
    uint32_t l = 0;
    while ((1ull << l) < (unsigned long long)d) ++l;
    const unsigned long long m = ((1ull << 32) * ((1ull << l) - (unsigned long long)d)) / (unsigned long long)d + 1;
    return FastDiv{d, (uint32_t)m, l};
}

__host__ __device__ __forceinline__ int fast_div(int n, const FastDiv& f) {
    const uint32_t hi = (uint32_t)(((unsigned long long)(uint32_t)n * f.m) >> 32);
    return (int)((hi + (uint32_t)n) >> f.l);
}

struct FusedGeom {
    FastDiv nx;      // XCD count (grid stride of one group's splits)
    FastDiv splits;  // S
    FastDiv colg;    // column groups per kv head
    FastDiv hkv;     // kv heads
    FastDiv lq;      // query rows per head
    int groups;      // G = B * Hkv * col_groups * VS
    int nblk;        // 16-key blocks of the keys every group reads (from kbase)
    int rv;          // rows per group partial (min(16, n_rep * Lq))
};

}  // namespace sdpa_dev
