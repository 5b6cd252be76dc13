/*
 * sdpa.h -- C ABI of libsdpa.so: fused scaled dot-product attention on
 * AMD Instinct MI355X (gfx950).
 *
 *     O = softmax(scale * Q K^T + M) V
 *
 * computed tile by tile with an online softmax, so the [B, Hq, Lq, Lk]
 * score tensor is never stored.  Definition and sources:
 *   - mlx issue "mx.fast.scaled_dot_product_attention produces incorrect
 *     attention scores (MLX 0.31.2)", section "Reproduction": the manual
 *     attention (Q K^T times scale, softmax over the key axis, times V) that
 *     the fused operation must equal;  same page, root-cause comment: the
 *     kernel addresses Q, K, V through explicit batch / head / sequence
 *     strides, and reading a [B,L,H,D] tensor as if it were [B,H,L,D] is the
 *     bug that page reports.  This ABI therefore takes every dimension as an
 *     explicit argument and every tensor with its own logical strides; it
 *     never infers a shape from memory order.
 *   - mlx issue #3885 "Metal SDPA: no fused path for head_dim=512 (vector or
 *     full kernel), and the fallback is silent": queries of length <= 8 take
 *     the "vector" (decode) kernel, longer ones the "full" (prefill) kernel;
 *     grouped-query heads (scores [B, n_kv, n_rep, qL, kL]); a silent
 *     unfused fallback is the failure to avoid, and a queryable predicate
 *     plus a once-per-shape route log are the remedies asked for.
 *   - mlx PR #4330 "Support head dimension 72 in Metal full attention":
 *     mask kinds none / additive / boolean / causal, aligned and unaligned
 *     lengths, float16 / bfloat16 / float32.
 *   - mlxcel issue #1065 "f32 matmul and single-query SDPA lose ~fp16
 *     precision on M5": float32 inputs must be computed in float32.
 *
 * Conventions shared by every entry point
 *   - Shapes are logical: Q [B, Hq, Lq, D], K and V [B, Hkv, Lk, D],
 *     O [B, Hq, Lq, D], mask broadcastable to [B, Hq, Lq, Lk].
 *   - Strides are in ELEMENTS, in logical (b, h, l, d) order.  A [B,L,H,D]
 *     tensor has strides (L*H*D, D, H*D, 1); a [B,H,L,D] one (H*L*D, L*D, D, 1).
 *     The d stride must be 1.  For Q, K, V and O every other stride and the
 *     base address must be 16-byte aligned (a multiple of 8 elements for
 *     16-bit types, 4 for float32).  K and V rows may not overlap (row
 *     stride >= head_dim when kv_len > 1) and kv_len * row stride of one
 *     key/value head must stay below 4 GiB.
 *   - Grouped-query attention: Hq must be a multiple of Hkv; query head h
 *     reads key/value head h / (Hq / Hkv).
 *   - Device pointers are HIP device pointers on the current device; the
 *     caller owns every buffer (including the workspace) and must keep it
 *     alive until `stream` has executed the call.  The library allocates
 *     nothing on this path and keeps no pointer after returning.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; errors from kernels that already ran
 *     surface on a later HIP call, as for any HIP launch.
 *   - Every argument is checked before anything is enqueued: on any error
 *     nothing is written.  No entry point aborts, throws or prints (except
 *     the opt-in route log, SDPA_LOG_ROUTE=1, to stderr).
 */
#ifndef SDPA_H
#define SDPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  SDPA_U8 is only valid as the element type of a boolean mask. */
typedef enum { SDPA_F32 = 0, SDPA_F16 = 1, SDPA_BF16 = 2, SDPA_U8 = 3 } sdpa_dtype;

/* Mask kinds (mlx PR #4330, "Proposed changes": unmasked, additive, boolean, causal).
 *   NONE      M = 0.
 *   ADDITIVE  M[b,h,i,j] = stored value (element type = dtype or SDPA_F32), added
 *             after the scale, not scaled.  -inf entries are allowed.
 *   BOOLEAN   one byte per element: nonzero = attend (M = 0), zero = masked (M = -inf).
 *   CAUSAL    no tensor; bottom-right aligned: query i attends key j iff
 *             j <= i + (Lk - Lq).
 *   SLIDING   no tensor; the causal mask limited to the `window` most recent
 *             keys: query i at position pos = i + (Lk - Lq) attends key j iff
 *             pos - window < j <= pos (the local layers of the d=256 model in
 *             mlx issue #3885, "Summary").  Only sdpa_forward_sliding takes it.
 * Mask strides use the same logical (b, h, l, d) order with `d` meaning the key
 * index j; a zero stride broadcasts that axis; `h` indexes QUERY heads.
 * A query row whose every key is masked produces an all-zero output row. */
typedef enum {
    SDPA_MASK_NONE = 0,
    SDPA_MASK_ADDITIVE = 1,
    SDPA_MASK_BOOLEAN = 2,
    SDPA_MASK_CAUSAL = 3,
    SDPA_MASK_SLIDING = 4
} sdpa_mask_kind;

/* Kernels (mlx issue #3885, "Current routing": vector for qL <= 8, full for qL > 8). */
typedef enum {
    SDPA_KERNEL_UNSUPPORTED = 0, /* this shape has no fused kernel: an error, never a fallback */
    SDPA_KERNEL_FULL = 1,        /* prefill: q_len > 8, MFMA tiles, online softmax        */
    SDPA_KERNEL_VECTOR = 2       /* decode: q_len <= 8, split keys + log-sum-exp combine  */
} sdpa_kernel;

typedef struct {
    int64_t b, h, l, d;
} sdpa_strides;

/* Rotary position embedding tables (rotate-half convention of the
 * pre-computed cos/sin tables in mlx issue #3585, "Model config"; partial
 * rotation as the "25% partial RoPE" layers of mlx issue #3885, "Summary").
 * A row at position pos has its head-dim columns j and j + R/2 (j < R/2)
 * turned by the angle of (pos, j):
 *     y[j]       = x[j] cos[pos][j] - x[j + R/2] sin[pos][j]
 *     y[j + R/2] = x[j + R/2] cos[pos][j] + x[j] sin[pos][j]
 * columns >= R are unchanged.  Computed in fp32, rounded once to the element
 * type.  cos and sin are device float32 [n_pos][R/2] row-major, 16-byte aligned. */
typedef struct {
    int rotary_dim;   /* R: even; 0 = no rotation                      */
    const float* cos; /* [n_pos][R / 2]                                  */
    const float* sin; /* [n_pos][R / 2]                                  */
    int n_pos;        /* table rows; every position used must be < n_pos */
} sdpa_rope_table;

/* Status codes. */
#define SDPA_OK 0
#define SDPA_EINVAL (-1)       /* null pointer, non-positive size, Hq % Hkv != 0, bad mask args */
#define SDPA_EUNSUPPORTED (-2) /* head dim / dtype not built, d stride != 1, misaligned          */
#define SDPA_EWORKSPACE (-3)   /* workspace smaller than sdpa_workspace_size()                   */
#define SDPA_ELAUNCH (-4)      /* launch shape rejected by the kernel's own limits               */
#define SDPA_EHIP (-5)         /* a HIP runtime call failed (detail: sdpa_last_hip_error())      */

/* Reasons reported by sdpa_select_kernel (0 when a kernel is selected). */
#define SDPA_REASON_OK 0
#define SDPA_REASON_HEAD_DIM 1   /* head_dim is not one of the built sizes      */
#define SDPA_REASON_DTYPE 2      /* dtype is not F32 / F16 / BF16              */
#define SDPA_REASON_GROUPS 3     /* n_q_heads is not a multiple of n_kv_heads  */
#define SDPA_REASON_SIZE 4       /* a size is non-positive or too large        */
#define SDPA_REASON_MASK 5       /* unknown mask kind                          */
#define SDPA_REASON_V_HEAD_DIM 6 /* v_head_dim != head_dim outside the built pairs (see sdpa_forward_ex) */

/*
 * sdpa_forward -- O = softmax(scale * Q K^T + M) V.
 *
 *   q, k, v, out   device pointers of element type `dtype`, with the logical
 *                  strides q_st, k_st, v_st, o_st described above.  `out` may
 *                  not overlap q, k, v or the workspace.
 *   batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim   all >= 1.
 *   scale          multiplies Q K^T (pass 1/sqrt(head_dim) for the usual scale).
 *   mask_kind      see sdpa_mask_kind (SLIDING: use sdpa_forward_sliding; here it
 *                  is SDPA_EINVAL).  `mask`, `mask_st` and `mask_dtype` are read
 *                  only for ADDITIVE (mask_dtype = SDPA_F32, SDPA_F16 or
 *                  SDPA_BF16, any of them for any dtype) and BOOLEAN
 *                  (mask_dtype = SDPA_U8); mask must then be non-null.
 *   workspace      device scratch of at least sdpa_workspace_size(...) bytes,
 *                  256-byte aligned (may be NULL when that size is 0), not
 *                  overlapping q, k, v, out or the mask.  The vector kernel
 *                  splits the keys over several workgroups (the 2-pass vector
 *                  kernel of mlx issue #3885, "Current routing") and keeps
 *                  their partial results there.  Its first 32768 bytes are
 *                  arrival counters: they must be ZERO before the first call
 *                  that uses the workspace (allocate it zero-filled once) and
 *                  every call leaves them zero again; the rest needs no
 *                  initialisation and is garbage afterwards.  Calls that
 *                  share a workspace must be ordered on one stream.  The full
 *                  kernel uses the bytes after the counters for the lane masks
 *                  of a BOOLEAN mask (one bit per mask element, built by a
 *                  pre-pass and read by every head that shares the mask) when
 *                  they fit; otherwise it reads the mask bytes themselves, with
 *                  the same result bit for bit.
 *   stream         hipStream_t as void*.
 * Returns SDPA_OK or a negative status; nothing is enqueued on error.
 */
int sdpa_forward(const void* q, sdpa_strides q_st,
                 const void* k, sdpa_strides k_st,
                 const void* v, sdpa_strides v_st,
                 void* out, sdpa_strides o_st,
                 int batch, int q_len, int kv_len,
                 int n_q_heads, int n_kv_heads, int head_dim,
                 sdpa_dtype dtype, float scale,
                 sdpa_mask_kind mask_kind, const void* mask, sdpa_strides mask_st,
                 sdpa_dtype mask_dtype,
                 void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * sdpa_forward_sliding -- sdpa_forward with mask kind SLIDING: causal
 * attention over the `window` (>= 1) most recent keys of each query
 * (bottom-right aligned).  Same operands, workspace, stream and status codes
 * as sdpa_forward; window < 1 is SDPA_EINVAL.  The full kernel skips the key
 * tiles left of every row's window; the vector kernel splits only the keys
 * the window can reach, so sdpa_workspace_size() for the same shape is enough.
 */
int sdpa_forward_sliding(const void* q, sdpa_strides q_st,
                         const void* k, sdpa_strides k_st,
                         const void* v, sdpa_strides v_st,
                         void* out, sdpa_strides o_st,
                         int batch, int q_len, int kv_len,
                         int n_q_heads, int n_kv_heads, int head_dim,
                         sdpa_dtype dtype, float scale, int window,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * sdpa_forward_ex -- the general call: sdpa_forward plus a V head dim and the
 * sliding window.
 *   v_head_dim     head dim of V and of `out` (and of their strides' extents).
 *                  Equal to head_dim for every built head dim; the one distinct
 *                  pairing built is head_dim 192 with v_head_dim 128, for the
 *                  vector (decode, q_len <= 8) kernel and 16-bit types (the
 *                  pairing mlx issue #3885 lists for its vector kernel under
 *                  "Current routing").  Other pairings: SDPA_EUNSUPPORTED,
 *                  reason SDPA_REASON_V_HEAD_DIM.
 *   window         keys per query when mask_kind is SDPA_MASK_SLIDING (>= 1,
 *                  else SDPA_EINVAL); ignored for the other kinds.
 *   q_rope, q_pos0 rotary embedding of Q inside the attention kernels (NULL or
 *                  rotary_dim 0: none).  Query row i sits at position q_pos0 + i
 *                  (q_pos0 = kv_len - q_len continues the keys).  K is taken as
 *                  already rotated: rotate keys once with sdpa_rope when they
 *                  are written (a cache keeps rotated keys), not on every call.
 *                  Any dtype; rotary_dim even and at most head_dim (a multiple
 *                  of 16 rotates 8 columns per 16-byte load, any other even
 *                  value column by column), 16-byte aligned tables, and
 *                  0 <= q_pos0, q_pos0 + q_len <= n_pos (SDPA_EUNSUPPORTED /
 *                  SDPA_EINVAL otherwise).  When v_head_dim == head_dim and
 *                  rotary_dim is above 128, 128 of 128, or not a multiple of
 *                  16 and above 32, Q is first rotated into `out` by a pass of
 *                  its own and the attention kernels read it from there: the
 *                  same bits as the in-kernel rotation, one more launch.
 * Everything else as sdpa_forward; the workspace is sdpa_workspace_size_ex().
 */
int sdpa_forward_ex(const void* q, sdpa_strides q_st,
                    const void* k, sdpa_strides k_st,
                    const void* v, sdpa_strides v_st,
                    void* out, sdpa_strides o_st,
                    int batch, int q_len, int kv_len,
                    int n_q_heads, int n_kv_heads, int head_dim, int v_head_dim,
                    sdpa_dtype dtype, float scale,
                    sdpa_mask_kind mask_kind, const void* mask, sdpa_strides mask_st,
                    sdpa_dtype mask_dtype, int window,
                    const sdpa_rope_table* q_rope, int q_pos0,
                    void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * sdpa_forward_noalloc -- sdpa_forward_ex for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): no workspace argument; the vector kernel keeps its
 * per-split partial results and arrival counters in a static device array of
 * sdpa_noalloc_scratch_bytes() bytes (8 MiB) that every GPU the library runs
 * on holds until the process ends.  The call allocates and frees nothing; the
 * first call on a device looks up that device's copy of the array.  A shape
 * whose sdpa_workspace_size_ex() exceeds the array returns SDPA_EWORKSPACE
 * (use sdpa_forward_ex with a workspace).  The arrival counters are zero when
 * the library is loaded and every completed call leaves them zero.  All calls
 * on one GPU share the array: calls that may overlap on one GPU (different
 * streams, or host threads without ordering) race and give wrong results.
 * Every other argument, status and rule as sdpa_forward_ex.
 */
int sdpa_forward_noalloc(const void* q, sdpa_strides q_st,
                         const void* k, sdpa_strides k_st,
                         const void* v, sdpa_strides v_st,
                         void* out, sdpa_strides o_st,
                         int batch, int q_len, int kv_len,
                         int n_q_heads, int n_kv_heads, int head_dim, int v_head_dim,
                         sdpa_dtype dtype, float scale,
                         sdpa_mask_kind mask_kind, const void* mask, sdpa_strides mask_st,
                         sdpa_dtype mask_dtype, int window,
                         const sdpa_rope_table* q_rope, int q_pos0,
                         void* stream);

/* sdpa_noalloc_scratch_bytes -- size of the static scratch of sdpa_forward_noalloc. */
size_t sdpa_noalloc_scratch_bytes(void);

/*
 * sdpa_rope -- y = the rotary embedding of x (see sdpa_rope_table): row l of
 * every (batch, head) sits at position pos0 + l.  x and y are device
 * [batch, n_heads, len, head_dim] tensors of `dtype` (F32, F16, BF16) with
 * logical strides (d stride 1); y may be x (in place) but may not otherwise
 * overlap it.  rotary_dim: even, 2 .. head_dim.  0 <= pos0, pos0 + len <= n_pos.
 * HBM-bound elementwise kernel on `stream`; returns SDPA_OK or a status.
 */
int sdpa_rope(const void* x, sdpa_strides x_st, void* y, sdpa_strides y_st,
              int batch, int n_heads, int len, int head_dim, sdpa_dtype dtype,
              const sdpa_rope_table* rope, int pos0, void* stream);

/*
 * sdpa_select_kernel -- the predicate sdpa_forward itself uses (one shared
 * function, so the query and the launch can never disagree; mlxcel issue
 * #1065 shows an inline copy of such a test drifting from the shared one).
 * Host only; touches no GPU.  Writes the kernel to *kernel and the reason
 * (SDPA_REASON_*) to *reason (either pointer may be NULL).  Returns SDPA_OK
 * when a kernel is selected, SDPA_EUNSUPPORTED or SDPA_EINVAL otherwise.
 */
int sdpa_select_kernel(int batch, int q_len, int kv_len, int n_q_heads, int n_kv_heads,
                       int head_dim, sdpa_dtype dtype, sdpa_mask_kind mask_kind,
                       sdpa_kernel* kernel, int* reason);

/* sdpa_select_kernel_ex -- the same predicate with a V head dim (sdpa_forward_ex). */
int sdpa_select_kernel_ex(int batch, int q_len, int kv_len, int n_q_heads, int n_kv_heads,
                          int head_dim, int v_head_dim, sdpa_dtype dtype, sdpa_mask_kind mask_kind,
                          sdpa_kernel* kernel, int* reason);

/*
 * sdpa_describe_route -- human-readable route for the same arguments: kernel,
 * tile shape, waves, key splits (e.g. "vector bf16 d512 additive splits=64").
 * Host only.  Writes a NUL-terminated string of at most `len` bytes into buf.
 * Returns the same status as sdpa_select_kernel.
 */
int sdpa_describe_route(int batch, int q_len, int kv_len, int n_q_heads, int n_kv_heads,
                        int head_dim, sdpa_dtype dtype, sdpa_mask_kind mask_kind,
                        char* buf, size_t len);

/* sdpa_describe_route_ex -- the same with a V head dim (sdpa_forward_ex). */
int sdpa_describe_route_ex(int batch, int q_len, int kv_len, int n_q_heads, int n_kv_heads,
                           int head_dim, int v_head_dim, sdpa_dtype dtype, sdpa_mask_kind mask_kind,
                           char* buf, size_t len);

/*
 * sdpa_workspace_size -- bytes of workspace sdpa_forward needs for this shape
 * (the 2-pass vector kernel of mlx issue #3885, "Current routing", keeps one
 * partial result per key split): 0 for a vector call whose key range is not
 * split; otherwise 32768 bytes of arrival counters (zero-initialised once, see
 * sdpa_forward) followed by the per-split partial results (an fp32 output row
 * plus running max and sum, per split, query head and query row).  An upper
 * bound over every mask kind, mask layout, sliding window and rotary option
 * for the same shape, on the current device.  For the full kernel: 0 where it
 * reads boolean masks as bytes (head dims above 128, fp32), else the counters
 * plus the lane masks of one boolean mask shared by every batch and head,
 * ceil(q_len / 32) * ceil(kv_len / 64) * 256 bytes; a mask that differs per
 * batch or head needs that many per (batch, head) and runs on its bytes when
 * the workspace is smaller.
 * Returns 0 for unsupported shapes as well.
 */
size_t sdpa_workspace_size(int batch, int q_len, int kv_len, int n_q_heads, int n_kv_heads,
                           int head_dim, sdpa_dtype dtype);

/* sdpa_workspace_size_ex -- the same with a V head dim (the partial outputs are v_head_dim wide). */
size_t sdpa_workspace_size_ex(int batch, int q_len, int kv_len, int n_q_heads, int n_kv_heads,
                              int head_dim, int v_head_dim, sdpa_dtype dtype);

/* sdpa_head_dims -- writes up to n built head dims (ascending) to out; returns how many exist.
 * Part of the queryable answer to "which shapes have a fused kernel" that mlx
 * issue #3885 asks for under "Requests" (head dims as template parameters,
 * not an enumerated list discovered by a silent fallback). */
int sdpa_head_dims(int* out, int n);

/* sdpa_strerror -- static description of a status code (never NULL).  Every
 * refusal is a status the caller sees: mlx issue #3885 (the comments after
 * "Requests") shows an unchecked launch returning silent zeros and turns it
 * into a loud error; here no call falls back or fails silently. */
const char* sdpa_strerror(int status);

/* sdpa_last_hip_error -- the hipError_t of the last SDPA_EHIP on this thread (0 if none). */
int sdpa_last_hip_error(void);

/*
 * sdpa_route_counters -- diagnostics: copies up to n counters into out and
 * returns how many exist: [0] calls, [1] full launches, [2] vector launches,
 * [3] rejected (any error status).  calls == full + vector + rejected.  The
 * counters are relaxed atomics, as the per-route hit / fallback counters of
 * the commits merged in mlx PR #4330 (their C diagnostics ABI and the
 * invariant attempts == hits + fallbacks).
 */
int sdpa_route_counters(uint64_t* out, int n);

/*
 * Diagnostics: per-kernel timing with HIP events on the call's own stream.
 * sdpa_timing_start(max_calls) creates 3 * max_calls events and arms the next
 * max_calls calls of sdpa_forward made by this thread: each records an event
 * before its first kernel and after each kernel it launches (the attention
 * kernel, then the decode combine kernel when there is one).  Must not be
 * active while a stream is being captured into a graph.
 * sdpa_timing_stop(ms, cap) waits for the recorded events, writes
 * ms[2*i] = attention-kernel milliseconds and ms[2*i+1] = combine-kernel
 * milliseconds (0 for the full kernel) of call i, for at most cap/2 calls,
 * destroys the events and returns the number of calls recorded (negative
 * status on a HIP error).  Calls beyond max_calls are not recorded.
 */
int sdpa_timing_start(int max_calls);
int sdpa_timing_stop(float* ms, int cap);

/*
 * sdpa_probe_stream_read -- diagnostics, not attention: one launch of a plain
 * streaming read of `bytes` bytes at device address `src` (16-byte aligned,
 * bytes a multiple of 16), one 256-thread workgroup per CU, on `stream`.
 * Decode is bound by reading K and V once (mlx issue #3885, "Measured
 * impact": decode time follows the K/V bytes); this kernel reads the same
 * amount with nothing else to do, which is the practical ceiling a launch of
 * that size reaches.  `sink` is a 4-byte device word that is written only for
 * one specific data pattern (it keeps the reads from being optimised away).
 * Returns SDPA_OK, SDPA_EINVAL or SDPA_EHIP.
 */
int sdpa_probe_stream_read(const void* src, size_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_H */
