// Internal host-side launch table: one KernelSet per (element type, head dim).
// Not part of the public ABI (see include/sdpa.h).
#pragma once

#include <hip/hip_runtime.h>

#include "attn_common.h"

namespace sdpa_host {

using sdpa_dev::Params;

typedef hipError_t (*launch_fn)(const Params&, dim3 grid, hipStream_t stream);
typedef hipError_t (*fused_fn)(const Params&, const sdpa_dev::FusedGeom&, dim3 grid, hipStream_t stream);

struct TileInfo {
    int bn;   // keys per tile (decode: keys per chunk; a split is a whole number of chunks)
    int cols; // query columns per workgroup (prefill: query rows; decode: query-head x row pairs)
    int wm;   // 32-column blocks per workgroup
    int wd;   // waves splitting the head dim
    int nt;   // threads per workgroup
    int lds;  // bytes of LDS per workgroup
    int heads = 1;  // prefill: query heads of one grouped-query group sharing a workgroup (at most)
    int causal_pairs = 0;  // prefill, causal mask: a workgroup takes two row tiles (t, last - t)
};

struct KernelSet {
    launch_fn full[sdpa_dev::MASK_VARIANTS];    // indexed by kernel mask variant (MASK_*)
    launch_fn decode[sdpa_dev::MASK_VARIANTS];  // indexed by kernel mask variant (MASK_*)
    launch_fn full_rope[sdpa_dev::MASK_VARIANTS];    // the same with the rotary prologue on Q (16-bit only)
    launch_fn decode_rope[sdpa_dev::MASK_VARIANTS];
    launch_fn combine;
    TileInfo full_cfg;
    TileInfo dec_cfg;
    // causal prefill with fewer rows per workgroup, for grids too small to pair
    // with full_cfg's workgroups (null where not built)
    launch_fn full_small[sdpa_dev::MASK_VARIANTS];
    launch_fn full_small_rope[sdpa_dev::MASK_VARIANTS];
    TileInfo full_small_cfg;
    // prefill with a mask tensor whose keys are not aligned 4-element runs
    // (Params::mask_vec == 0), same tiles as full_cfg (null where full[]
    // handles both layouts)
    launch_fn full_strided[sdpa_dev::MASK_VARIANTS];
    launch_fn full_strided_rope[sdpa_dev::MASK_VARIANTS];
    // prefill with a boolean mask given as precomputed lane masks
    // (Params::mask_bits; null where not built)
    launch_fn full_bits;
    launch_fn full_bits_rope;
    // 16-bit decode in one launch (split keys merged in L2 by the last
    // workgroup of each group), by V column slices (index VS - 1; null where
    // not built) and mask variant
    fused_fn decode_fused[sdpa_dev::MASK_VARIANTS];
    fused_fn decode_fused_rope[sdpa_dev::MASK_VARIANTS];
    int fused_nt;  // threads per workgroup of those kernels (0: none built)
};

// Returns hipErrorInvalidConfiguration when the compiled kernel cannot run
// `nt` threads per workgroup (register or LDS limits): such a launch would be
// dropped by the hardware, so it is refused before it is made.  Callers keep
// the result in a function-local static (initialised once, thread-safe).
template <class K>
hipError_t check_launch(K kernel, int nt) {
    hipFuncAttributes a;
    hipError_t e = hipFuncGetAttributes(&a, reinterpret_cast<const void*>(kernel));
    if (e == hipSuccess && a.maxThreadsPerBlock < nt) e = hipErrorInvalidConfiguration;
    return e;
}

// Head dims with built kernels; one getter per head dim (index = sdpa_dtype: F32, F16, BF16).
#define SDPA_HEAD_DIMS(X) X(64) X(72) X(80) X(96) X(128) X(256) X(512)
#define SDPA_DECLARE_GETTER(D) const KernelSet* kernels_d##D(int dtype);
SDPA_HEAD_DIMS(SDPA_DECLARE_GETTER)
#undef SDPA_DECLARE_GETTER

// (Q/K head dim, V head dim) pairs with built kernels: the vector (decode)
// kernel only, 16-bit inputs only (null entries elsewhere), as in the routing
// mlx issue #3885 describes ("Current routing": vector kernel (192, 128)).
#define SDPA_HEAD_DIM_PAIRS(X) X(192, 128)
#define SDPA_DECLARE_PAIR_GETTER(DQ, DV) const KernelSet* kernels_q##DQ##_v##DV(int dtype);
SDPA_HEAD_DIM_PAIRS(SDPA_DECLARE_PAIR_GETTER)
#undef SDPA_DECLARE_PAIR_GETTER

}  // namespace sdpa_host
