// Rotary position embedding on gfx950: the step in front of Q K^T.
//
// The convention is the rotate-half one of the pre-computed cos/sin tables
// named in mlx issue #3585 [Model config]: with R rotated columns and
// h = R / 2, column pairs (j, j + h), j < h, of a row at position pos turn by
// the table angle of (pos, j):
//     y[j]     = x[j] * cos[pos][j] - x[j + h] * sin[pos][j]
//     y[j + h] = x[j + h] * cos[pos][j] + x[j] * sin[pos][j]
// and columns >= R pass through (partial RoPE, mlx issue #3885 [Summary]).
//
// rope_kernel rotates a whole strided [B, H, L, D] tensor (a key tensor on
// its way into a cache, once); rope_q_fragments builds the rotated Q
// fragments an attention kernel keeps in registers, so queries are never
// written back rotated.  Both compute each output as fma(x, c, -(x' * s)) /
// fma(x', c, x * s) in fp32 and round once to the element type, so the two
// paths give the same bits.
#pragma once

#include "attn_common.h"

namespace sdpa_dev {

struct RopeArgs {
    const void* x;
    void* y;
    int64_t xs[4], ys[4];  // element strides, logical (b, h, l, d)
    int B, H, L, D;
    int R;                 // rotated columns (even)
    int pos0;              // position of row 0
    const float* cos;      // [n_pos][R / 2]
    const float* sin;
};

template <class T> struct RopeElem;
template <> struct RopeElem<float> {
    static __device__ __forceinline__ float load(const void* p) { return *reinterpret_cast<const float*>(p); }
    static __device__ __forceinline__ void store(void* p, float v) { *reinterpret_cast<float*>(p) = v; }
};
template <> struct RopeElem<__bf16> {
    static __device__ __forceinline__ float load(const void* p) {
        return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16);
    }
    static __device__ __forceinline__ void store(void* p, float v) { *reinterpret_cast<__bf16*>(p) = (__bf16)v; }
};
template <> struct RopeElem<_Float16> {
    static __device__ __forceinline__ float load(const void* p) {
        return (float)*reinterpret_cast<const _Float16*>(p);
    }
    static __device__ __forceinline__ void store(void* p, float v) { *reinterpret_cast<_Float16*>(p) = (_Float16)v; }
};

__device__ __forceinline__ float rope_lo(float a, float b, float c, float s) { return __builtin_fmaf(a, c, -(b * s)); }
__device__ __forceinline__ float rope_hi(float a, float b, float c, float s) { return __builtin_fmaf(b, c, a * s); }

// One thread per (row, column): pairs for j < h, pass-through copies for
// j >= R when y is not x.  Grid: ceil(B * H * L * D / 256) workgroups.
template <class T>
__global__ __launch_bounds__(256) void rope_kernel(const RopeArgs a) {
    using E = RopeElem<T>;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n = (int64_t)a.B * a.H * a.L * a.D;
    if (t >= n) return;
    const int j = (int)(t % a.D);
    int64_t r = t / a.D;
    const int l = (int)(r % a.L);
    r /= a.L;
    const int hh = (int)(r % a.H), b = (int)(r / a.H);
    const int h = a.R / 2;
    const char* xr = reinterpret_cast<const char*>(a.x) +
                     ((int64_t)b * a.xs[0] + (int64_t)hh * a.xs[1] + (int64_t)l * a.xs[2]) * sizeof(T);
    char* yr = reinterpret_cast<char*>(a.y) +
               ((int64_t)b * a.ys[0] + (int64_t)hh * a.ys[1] + (int64_t)l * a.ys[2]) * sizeof(T);
    if (j < h) {
        const float x0 = E::load(xr + j * sizeof(T)), x1 = E::load(xr + (j + h) * sizeof(T));
        const int64_t pos = (int64_t)a.pos0 + l;
        const float c = a.cos[pos * h + j], s = a.sin[pos * h + j];
        E::store(yr + j * sizeof(T), rope_lo(x0, x1, c, s));
        E::store(yr + (j + h) * sizeof(T), rope_hi(x0, x1, c, s));
    } else if (j >= a.R && a.y != a.x) {
        E::store(yr + j * sizeof(T), E::load(xr + j * sizeof(T)));
    }
}

// One element of a 16-byte MFMA fragment (8 halves or 4 floats) as a float,
// and back: a 16-bit element is rounded once, to nearest even (the same bits
// RopeElem::store and TR::pack give).
template <class TR> struct FragElem {
    static constexpr int NE = 8;
    static __device__ __forceinline__ float get(const u32x4_t& f, int e) {
        return (e & 1) ? TR::unpack_hi(f[e >> 1]) : TR::unpack_lo(f[e >> 1]);
    }
    static __device__ __forceinline__ void set(u32x4_t& f, int e, float v) {
        const uint32_t b = TR::pack(v, v);
        f[e >> 1] = (e & 1) ? ((f[e >> 1] & 0x0000ffffu) | (b & 0xffff0000u)) : ((f[e >> 1] & 0xffff0000u) | (b & 0x0000ffffu));
    }
    static __device__ __forceinline__ float load(const char* p) {
        return TR::unpack_lo((uint32_t)*reinterpret_cast<const uint16_t*>(p));
    }
};
template <> struct FragElem<TF32> {
    static constexpr int NE = 4;
    static __device__ __forceinline__ float get(const u32x4_t& f, int e) { return __uint_as_float(f[e]); }
    static __device__ __forceinline__ void set(u32x4_t& f, int e, float v) { f[e] = __float_as_uint(v); }
    static __device__ __forceinline__ float load(const char* p) { return *reinterpret_cast<const float*>(p); }
};

// Any even R: each of a fragment's columns below R turns on its own, with its
// partner column (h = R / 2 away) and its two table entries read one by one.
// `frag` holds the row's columns d0 .. d0 + NE - 1 as loaded.
template <class TR>
__device__ __forceinline__ void rope_fragment_elems(u32x4_t& frag, const char* qrow, int d0, int R,
                                                    const float* cos, const float* sin, int64_t pos) {
    using E = FragElem<TR>;
    constexpr int ES = 16 / E::NE;
    const int h = R / 2;
    const u32x4_t own = frag;
#pragma unroll
    for (int e = 0; e < E::NE; ++e) {
        const int j = d0 + e;
        if (j < R) {
            const bool low = j < h;
            const int jc = low ? j : j - h;  // table column
            const float x = E::get(own, e);
            const float xp = E::load(qrow + (int64_t)(low ? j + h : j - h) * ES);
            const float c = cos[pos * h + jc], sn = sin[pos * h + jc];
            E::set(frag, e, low ? rope_lo(x, xp, c, sn) : rope_hi(xp, x, c, sn));
        }
    }
}

// The same rotation, 16 bytes at a time: one thread per (row, unit), a unit
// being one 16-byte chunk of the low half [0, h) together with its partner
// chunk h further on (both written), or, out of place, one chunk of the
// pass-through columns [R, D).  Needs R a multiple of two chunks, D a whole
// number of chunks and 16-byte aligned rows and tables (the host checks);
// gives the bits of rope_kernel.  Grid: ceil(B * H * L * nunit / 256).
template <class TR>
__global__ __launch_bounds__(256) void rope_kernel_vec(const RopeArgs a, int nunit) {
    using E = FragElem<TR>;
    constexpr int NE = E::NE, ES = 16 / NE;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)a.B * a.H * a.L * nunit) return;
    const int u = (int)(t % nunit);
    int64_t r = t / nunit;
    const int l = (int)(r % a.L);
    r /= a.L;
    const int hh = (int)(r % a.H), b = (int)(r / a.H);
    const int h = a.R / 2, nrot = h / NE;
    const char* xr = reinterpret_cast<const char*>(a.x) +
                     ((int64_t)b * a.xs[0] + (int64_t)hh * a.xs[1] + (int64_t)l * a.xs[2]) * ES;
    char* yr = reinterpret_cast<char*>(a.y) + ((int64_t)b * a.ys[0] + (int64_t)hh * a.ys[1] + (int64_t)l * a.ys[2]) * ES;
    if (u < nrot) {
        const int j = u * NE;
        const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(xr + (int64_t)j * ES);
        const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(xr + (int64_t)(j + h) * ES);
        const int64_t pos = (int64_t)a.pos0 + l;
        float cv[NE], sv[NE];
#pragma unroll
        for (int q = 0; q < NE / 4; ++q) {
            const f32x4_t c4 = *reinterpret_cast<const f32x4_t*>(a.cos + pos * h + j + 4 * q);
            const f32x4_t s4 = *reinterpret_cast<const f32x4_t*>(a.sin + pos * h + j + 4 * q);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                cv[4 * q + e] = c4[e];
                sv[4 * q + e] = s4[e];
            }
        }
        u32x4_t y0 = x0, y1 = x1;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const float xa = E::get(x0, e), xb = E::get(x1, e);
            E::set(y0, e, rope_lo(xa, xb, cv[e], sv[e]));
            E::set(y1, e, rope_hi(xa, xb, cv[e], sv[e]));
        }
        *reinterpret_cast<u32x4_t*>(yr + (int64_t)j * ES) = y0;
        *reinterpret_cast<u32x4_t*>(yr + (int64_t)(j + h) * ES) = y1;
    } else {
        const int j = a.R + (u - nrot) * NE;
        *reinterpret_cast<u32x4_t*>(yr + (int64_t)j * ES) = *reinterpret_cast<const u32x4_t*>(xr + (int64_t)j * ES);
    }
}

// Rotated 16-bit MFMA fragments of one query row: frag[i] holds head-dim
// columns d0 .. d0 + 7, d0 = i * STEP + off.  With R a multiple of 16 a
// fragment lies wholly on one side of h = R / 2 and is rebuilt from two
// 16-byte loads of the row (its own 8 columns and the partner's) and 16-byte
// table loads; any other even R takes the element path above.  Fragments
// with d0 >= R keep what the caller loaded.  Indices into `frag` stay
// compile-time (no register spilling).
template <class TR, int N, int STEP>
__device__ __forceinline__ void rope_q_fragments(u32x4_t (&frag)[N], const char* qrow, int off, int R,
                                                 const float* cos, const float* sin, int64_t pos) {
    const int h = R / 2;
    const bool vec = (R & 15) == 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int d0 = i * STEP + off;
        if (d0 < R && !vec) {
            rope_fragment_elems<TR>(frag[i], qrow, d0, R, cos, sin, pos);
        } else if (d0 < R) {
            const bool low = d0 < h;
            const int jc = low ? d0 : d0 - h;     // table column
            const int dp = low ? d0 + h : d0 - h; // partner columns
            const u32x4_t own = *reinterpret_cast<const u32x4_t*>(qrow + d0 * 2);
            const u32x4_t par = *reinterpret_cast<const u32x4_t*>(qrow + dp * 2);
            const float* cr = cos + pos * h + jc;
            const float* sr = sin + pos * h + jc;
            const f32x4_t c0 = *reinterpret_cast<const f32x4_t*>(cr), c1 = *reinterpret_cast<const f32x4_t*>(cr + 4);
            const f32x4_t s0 = *reinterpret_cast<const f32x4_t*>(sr), s1 = *reinterpret_cast<const f32x4_t*>(sr + 4);
            u32x4_t out;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float ca = (w < 2) ? c0[2 * w] : c1[2 * w - 4], cb = (w < 2) ? c0[2 * w + 1] : c1[2 * w - 3];
                const float sa = (w < 2) ? s0[2 * w] : s1[2 * w - 4], sb = (w < 2) ? s0[2 * w + 1] : s1[2 * w - 3];
                const float xa = TR::unpack_lo(own[w]), xb = TR::unpack_hi(own[w]);
                const float ya = TR::unpack_lo(par[w]), yb = TR::unpack_hi(par[w]);
                out[w] = low ? TR::pack(rope_lo(xa, ya, ca, sa), rope_lo(xb, yb, cb, sb))
                             : TR::pack(rope_hi(ya, xa, ca, sa), rope_hi(yb, xb, cb, sb));
            }
            frag[i] = out;
        }
        __builtin_amdgcn_sched_barrier(0);  // one fragment's loads at a time: no register spike
    }
}

}  // namespace sdpa_dev
