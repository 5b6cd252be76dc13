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

enum { MASK_NONE = 0, MASK_ADD = 1, MASK_BOOL = 2, MASK_CAUSAL = 3 };
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
    int B, Lq, Lk, Hq, Hkv, n_rep;
    float scale_log2;  // scale * log2(e)
    // vector (decode) kernel
    float* ws_o;      // [B*Hq*Lq][splits][D] unnormalised partial outputs
    float* ws_ml;     // [B*Hq*Lq][splits][2] running max (log2 domain) and sum
    int splits;
    int keys_per_split;
    int col_groups;   // decode: column groups per kv head
};

template <class To, class From>
__device__ __forceinline__ To bitcast(const From& x) {
    static_assert(sizeof(To) == sizeof(From), "bitcast size");
    return __builtin_bit_cast(To, x);
}

// Round-to-nearest-even float -> bf16 / f16 pairs, packed low = a, high = b.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    __bf16 x = (__bf16)a, y = (__bf16)b;
    return (uint32_t)bitcast<uint16_t>(x) | ((uint32_t)bitcast<uint16_t>(y) << 16);
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    _Float16 x = (_Float16)a, y = (_Float16)b;
    return (uint32_t)bitcast<uint16_t>(x) | ((uint32_t)bitcast<uint16_t>(y) << 16);
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
    static __device__ __forceinline__ void store4(void* dst, f32x4_t x) {
        u32x2_t w = {pack_f16(x[0], x[1]), pack_f16(x[2], x[3])};
        *reinterpret_cast<u32x2_t*>(dst) = w;
    }
    static __device__ __forceinline__ void store1(void* dst, float x) {
        *reinterpret_cast<uint16_t*>(dst) = bitcast<uint16_t>((_Float16)x);
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

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Mask value for one (row, key) of an additive mask, widened to float.
__device__ __forceinline__ float load_mask_scalar(const void* base, int64_t off, int mdt) {
    if (mdt == MDT_F32) return reinterpret_cast<const float*>(base)[off];
    uint16_t u = reinterpret_cast<const uint16_t*>(base)[off];
    if (mdt == MDT_BF16) return __uint_as_float((uint32_t)u << 16);
    return (float)bitcast<_Float16>(u);
}

// Four consecutive keys of an additive mask (key stride 1, 4-element aligned run).
__device__ __forceinline__ f32x4_t load_mask4(const void* base, int64_t off, int mdt) {
    if (mdt == MDT_F32) return *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(base) + off);
    u32x2_t w = *reinterpret_cast<const u32x2_t*>(reinterpret_cast<const uint16_t*>(base) + off);
    f32x4_t r;
    if (mdt == MDT_BF16) {
        r[0] = __uint_as_float(w[0] << 16);
        r[1] = __uint_as_float(w[0] & 0xffff0000u);
        r[2] = __uint_as_float(w[1] << 16);
        r[3] = __uint_as_float(w[1] & 0xffff0000u);
    } else {
        r[0] = (float)bitcast<_Float16>((uint16_t)(w[0] & 0xffffu));
        r[1] = (float)bitcast<_Float16>((uint16_t)(w[0] >> 16));
        r[2] = (float)bitcast<_Float16>((uint16_t)(w[1] & 0xffffu));
        r[3] = (float)bitcast<_Float16>((uint16_t)(w[1] >> 16));
    }
    return r;
}

}  // namespace sdpa_dev
