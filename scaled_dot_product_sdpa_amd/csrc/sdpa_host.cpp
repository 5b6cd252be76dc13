// Host side of libsdpa.so: argument checks, the routing predicate, workspace
// sizing, launches, diagnostics.  Implements include/sdpa.h.
//
// Routing follows mlx issue #3885 ("Current routing"): query length <= 8 ->
// vector (decode) kernel, longer -> full (prefill) kernel.  Unlike the
// routing that page describes, there is no unfused fallback: a head dim or
// element type without a built kernel is reported as unsupported by the same
// predicate the caller can query, and sdpa_forward returns an error for it.
#include "../../include/sdpa.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <set>
#include <string>
#include <vector>

#include "attn_kernel.h"
#include "decode_fused_kernel.h"
#include "mask_bits.h"
#include "launch.h"
#include "rope_kernel.h"
#include "stream_probe.h"

using sdpa_dev::Params;
using sdpa_host::KernelSet;
using sdpa_host::launch_fn;

namespace {

constexpr int kVectorMaxQLen = 8;     // qL <= 8 -> vector kernel
constexpr int kMaxGridYZ = 65535;
constexpr int kMaxDevices = 64;

// Compute units and XCDs of the current device (grid heuristics and the XCD
// mapping of workgroups), queried once per device.  Without a device (host
// only queries) an MI355X is assumed: 256 CUs in 8 XCDs.
struct DevInfo {
    int cus;
    int nx;
};
DevInfo device_info() {
    static std::atomic<uint64_t> cache[kMaxDevices];  // (cus << 32 | nx), 0 = not queried yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DevInfo{256, 8};
    uint64_t v = cache[dev].load(std::memory_order_acquire);
    if (v == 0) {
        int cus = 0, nx = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipDeviceGetAttribute(&nx, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || nx <= 0 || nx > 16)
            nx = 1;
        v = ((uint64_t)cus << 32) | (uint64_t)nx;
        cache[dev].store(v, std::memory_order_release);
    }
    return DevInfo{(int)(v >> 32), (int)(v & 0xffffffffu)};
}

std::atomic<uint64_t> g_counters[4];  // calls, full, vector, rejected
thread_local int g_last_hip_error = 0;

const int kHeadDims[] = {
#define SDPA_LIST_D(D) D,
    SDPA_HEAD_DIMS(SDPA_LIST_D)
#undef SDPA_LIST_D
};

// Kernels for (Q/K head dim d, V head dim dv); null when none are built.
const KernelSet* kernel_set(sdpa_dtype dt, int d, int dv) {
    if (dt != SDPA_F32 && dt != SDPA_F16 && dt != SDPA_BF16) return nullptr;
    if (dv == d) {
        switch (d) {
#define SDPA_CASE_D(D) \
    case D:            \
        return sdpa_host::kernels_d##D((int)dt);
            SDPA_HEAD_DIMS(SDPA_CASE_D)
#undef SDPA_CASE_D
            default:
                return nullptr;
        }
    }
#define SDPA_CASE_PAIR(DQ, DV) \
    if (d == DQ && dv == DV) return sdpa_host::kernels_q##DQ##_v##DV((int)dt);
    SDPA_HEAD_DIM_PAIRS(SDPA_CASE_PAIR)
#undef SDPA_CASE_PAIR
    return nullptr;
}

bool head_dim_built(int d) {
    for (int x : kHeadDims)
        if (x == d) return true;
    return false;
}

int elem_size(sdpa_dtype dt) {
    switch (dt) {
        case SDPA_F32: return 4;
        case SDPA_F16: return 2;
        case SDPA_BF16: return 2;
        case SDPA_U8: return 1;
    }
    return 0;
}

// The one routing predicate (also behind sdpa_select_kernel).
int select(int batch, int q_len, int kv_len, int hq, int hkv, int d, int dv, sdpa_dtype dt, sdpa_mask_kind mk,
           sdpa_kernel* kernel, int* reason) {
    sdpa_kernel k = SDPA_KERNEL_UNSUPPORTED;
    int why = SDPA_REASON_OK, st = SDPA_OK;
    if (batch <= 0 || q_len <= 0 || kv_len <= 0 || hq <= 0 || hkv <= 0 || d <= 0 || dv <= 0 ||
        batch > kMaxGridYZ || hq > kMaxGridYZ) {
        why = SDPA_REASON_SIZE;
        st = SDPA_EINVAL;
    } else if (hq % hkv != 0) {
        why = SDPA_REASON_GROUPS;
        st = SDPA_EINVAL;
    } else if (mk < SDPA_MASK_NONE || mk > SDPA_MASK_SLIDING) {
        why = SDPA_REASON_MASK;
        st = SDPA_EINVAL;
    } else if (dt != SDPA_F32 && dt != SDPA_F16 && dt != SDPA_BF16) {
        why = SDPA_REASON_DTYPE;
        st = SDPA_EUNSUPPORTED;
    } else if (dv == d && !head_dim_built(d)) {
        why = SDPA_REASON_HEAD_DIM;
        st = SDPA_EUNSUPPORTED;
    } else {
        k = (q_len <= kVectorMaxQLen) ? SDPA_KERNEL_VECTOR : SDPA_KERNEL_FULL;
        // a distinct V head dim exists only where a kernel for the pair was built
        const KernelSet* ks = (dv == d) ? nullptr : kernel_set(dt, d, dv);
        if (dv != d && (!ks || (k == SDPA_KERNEL_FULL ? !ks->full[0] : !ks->decode[0]))) {
            k = SDPA_KERNEL_UNSUPPORTED;
            why = SDPA_REASON_V_HEAD_DIM;
            st = SDPA_EUNSUPPORTED;
        }
    }
    if (kernel) *kernel = k;
    if (reason) *reason = why;
    return st;
}

struct DecodePlan {
    int col_groups;
    int splits;
    int keys_per_split;
};

// Split the key axis so the decode grid covers the chip about twice; a
// test-only environment override (SDPA_DECODE_SPLITS) pins the count.
// The split count never exceeds split_cap(kv_len), which grows with kv_len:
// the workspace is sized with it (a sliding window plans over fewer keys).
long split_cap(int batch, int q_len, int kv_len, int hq, int hkv, const sdpa_host::TileInfo& t, int cus) {
    const int rows = (hq / hkv) * q_len;
    const long groups = (long)batch * hkv * ((rows + t.cols - 1) / t.cols);
    const int max_splits = (kv_len + t.bn - 1) / t.bn;
    long s = (2L * cus + groups - 1) / groups;
    if (const char* env = std::getenv("SDPA_DECODE_SPLITS")) {
        const long v = std::strtol(env, nullptr, 10);
        if (v > 0) s = v;
    }
    if (s < 1) s = 1;
    if (s > max_splits) s = max_splits;
    if (s > sdpa_dev::kMaxSplits) s = sdpa_dev::kMaxSplits;
    return s;
}

DecodePlan decode_plan(int batch, int q_len, int kv_len, int hq, int hkv, const sdpa_host::TileInfo& t) {
    DecodePlan p;
    const int rows = (hq / hkv) * q_len;
    const int cols = t.cols;
    p.col_groups = (rows + cols - 1) / cols;
    const long groups = (long)batch * hkv * p.col_groups;
    const int max_splits = (kv_len + t.bn - 1) / t.bn;
    long s = (2L * device_info().cus + groups - 1) / groups;
    if (const char* env = std::getenv("SDPA_DECODE_SPLITS")) {
        const long v = std::strtol(env, nullptr, 10);
        if (v > 0) s = v;
    }
    if (s < 1) s = 1;
    if (s > max_splits) s = max_splits;
    if (s > sdpa_dev::kMaxSplits) s = sdpa_dev::kMaxSplits;
    const int per = (int)((kv_len + s - 1) / s);
    p.keys_per_split = ((per + t.bn - 1) / t.bn) * t.bn;
    p.splits = (kv_len + p.keys_per_split - 1) / p.keys_per_split;
    return p;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Every decode workspace starts with kFusedCounterWords arrival words of the
// single-launch kernel (zero before and after every call); the split + combine
// kernels place their partial results after them and never touch them.
constexpr size_t kCounterBytes = (size_t)sdpa_dev::kFusedCounterWords * 4;

// Lane masks of a boolean mask for the head-dim <= 128 prefill kernel
// (mask_bits.h), per (mask batch, mask head): 32 words per (32-row block,
// 64-key tile).  They too sit after the arrival words, which a workspace
// shared with decode calls must keep zero.
size_t mask_bits_bytes(int q_len, int kv_len) {
    return (size_t)((q_len + 31) / 32) * (size_t)((kv_len + 63) / 64) * sdpa_dev::kMaskBitsWords * sizeof(uint32_t);
}

// (a single split of the 16-bit split kernel writes the output itself: no workspace)
size_t decode_ws_bytes(int batch, int q_len, int hq, int d, long splits, sdpa_dtype dt) {
    if (splits == 1 && dt != SDPA_F32) return 0;
    const size_t rows = (size_t)batch * hq * q_len;
    return kCounterBytes + align256(rows * splits * d * sizeof(float)) + align256(rows * splits * 2 * sizeof(float));
}

// Single-launch decode (16-bit, D <= 256): groups of (batch, kv head, column
// group of <= 16 rows) whose splits all run on one XCD.  Taken when the groups
// spread evenly over the XCDs; otherwise the split + combine kernels run.
struct FusedPlan {
    bool use = false;
    int groups = 0;   // G
    int splits = 1;   // S
    int nblk = 0;     // 16-key blocks from kbase
    int rv = 0;       // rows per partial
    int col_groups = 0;
};
constexpr int kFusedKeys = 16;  // keys per block of the single-launch kernel

FusedPlan fused_plan(const KernelSet* ks, int batch, int q_len, int kv_len_eff, int hq, int hkv, int rope,
                     int variant, bool mask_ok = true) {
    FusedPlan f;
    if (!ks || !ks->fused_nt || !mask_ok) return f;
    // SDPA_DECODE_FUSED=0: the split + combine kernels for every decode shape (comparisons, tests)
    if (const char* env = std::getenv("SDPA_DECODE_FUSED"))
        if (env[0] == '0') return f;
    if ((rope ? ks->decode_fused_rope[variant] : ks->decode_fused[variant]) == nullptr) return f;
    const DevInfo di = device_info();
    const int nx = di.nx;
    const int rows = (hq / hkv) * q_len;
    f.col_groups = (rows + 15) / 16;
    f.rv = rows < 16 ? rows : 16;
    const long G = (long)batch * hkv * f.col_groups;
    if (G % nx != 0 || G > (1L << 30)) return FusedPlan{};
    f.groups = (int)G;
    f.nblk = (kv_len_eff + kFusedKeys - 1) / kFusedKeys;
    // one workgroup per CU: S splits per group
    long s = (long)di.cus / G;
    const long by_keys = f.nblk / 2;  // at least two 16-key blocks per split
    if (s > by_keys) s = by_keys;
    if (const char* env = std::getenv("SDPA_DECODE_SPLITS")) {
        const long v = std::strtol(env, nullptr, 10);
        if (v > 0) s = v;
    }
    if (s > sdpa_dev::kFusedMaxSplits) s = sdpa_dev::kFusedMaxSplits;
    if (s > f.nblk) s = f.nblk;
    if (s < 1) s = 1;
    // block indices are computed in 32-bit arithmetic; merged groups need an arrival word each
    if ((long long)f.nblk * s >= (1LL << 31)) return FusedPlan{};
    if (s > 1 && G > sdpa_dev::kFusedMaxGroups) return FusedPlan{};
    f.splits = (int)s;
    f.use = true;
    return f;
}

size_t fused_ws_bytes(const FusedPlan& f, int dv) {
    if (f.splits == 1) return 0;
    const size_t slots = (size_t)f.groups * f.splits * f.rv;
    // the timeline build appends one record per workgroup (decode_fused_kernel.h)
    const size_t trace = SDPA_TRACE_DECODE ? align256((size_t)f.groups * f.splits * sdpa_dev::kTraceWords * 8) : 0;
    return kCounterBytes + align256(slots * dv * sizeof(float)) + align256(slots * 2 * sizeof(float)) + trace;
}

// Byte extent of a strided tensor: [base, base + span).
size_t span_bytes(const int64_t* n, const sdpa_strides& s, int es) {
    const int64_t st[4] = {s.b, s.h, s.l, s.d};
    int64_t last = 0;
    for (int i = 0; i < 4; ++i) last += (n[i] - 1) * st[i];
    return (size_t)(last + 1) * es;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Strides must be non-negative, d stride 1, and every non-trivial axis a whole
// number of 16-byte chunks (the kernels move Q, K, V, O in 16-byte vectors).
int check_operand(const void* ptr, const sdpa_strides& s, const int64_t* n, int es) {
    if (!ptr) return SDPA_EINVAL;
    if (s.b < 0 || s.h < 0 || s.l < 0 || s.d < 0) return SDPA_EINVAL;
    if (s.d != 1) return SDPA_EUNSUPPORTED;
    if (((uintptr_t)ptr) % 16 != 0) return SDPA_EUNSUPPORTED;
    const int64_t st[3] = {s.b, s.h, s.l};
    for (int i = 0; i < 3; ++i)
        if (n[i] > 1 && (st[i] * es) % 16 != 0) return SDPA_EUNSUPPORTED;
    return SDPA_OK;
}

const char* dtype_name(sdpa_dtype dt) {
    switch (dt) {
        case SDPA_F32: return "f32";
        case SDPA_F16: return "f16";
        case SDPA_BF16: return "bf16";
        case SDPA_U8: return "u8";
    }
    return "?";
}

const char* mask_name(sdpa_mask_kind mk) {
    switch (mk) {
        case SDPA_MASK_NONE: return "none";
        case SDPA_MASK_ADDITIVE: return "additive";
        case SDPA_MASK_BOOLEAN: return "boolean";
        case SDPA_MASK_CAUSAL: return "causal";
        case SDPA_MASK_SLIDING: return "sliding";
    }
    return "?";
}

// Prefill grid: work items of (batch, head group, row tile).  A causal grid
// pairs row tiles t and last - t in one workgroup (the same key count for
// every workgroup, so no long row tile outlasts the rest) when the kernel
// supports it and the halved grid still covers every CU.
struct FullGrid {
    long items;
    int pairs;
};
FullGrid full_grid(const sdpa_host::TileInfo& t, bool causal, int batch, int q_len, int n_q_heads, int n_kv_heads) {
    // heads of one group that share a workgroup: the largest power of two up
    // to t.heads dividing the group size (the kernel derives the same number)
    const int rep = n_q_heads / n_kv_heads;
    int hg = 1;
    for (int c = t.heads; c > 1; c >>= 1)
        if (rep % c == 0) {
            hg = c;
            break;
        }
    const int bm = t.cols / hg;
    const long qtiles = (q_len + bm - 1) / bm;
    const long groups = (long)(n_q_heads / hg) * batch;
    if (t.causal_pairs && causal && (qtiles + 1) / 2 * groups >= device_info().cus) return FullGrid{(qtiles + 1) / 2 * groups, 1};
    return FullGrid{qtiles * groups, 0};
}

// The prefill kernel, its tile shape and grid: the default set, or, for a
// causal grid that cannot pair, the variant with fewer rows per workgroup when
// that one can pair or the default grid leaves CUs without a workgroup.
struct FullPlan {
    const sdpa_host::TileInfo* cfg;
    FullGrid grid;
    bool small;
};
FullPlan full_plan(const KernelSet* ks, int variant, int batch, int q_len, int n_q_heads, int n_kv_heads) {
    const bool causal = variant == sdpa_dev::MASK_CAUSAL;
    FullPlan fp{&ks->full_cfg, full_grid(ks->full_cfg, causal, batch, q_len, n_q_heads, n_kv_heads), false};
    if (causal && !fp.grid.pairs && ks->full_small[variant]) {
        const FullGrid gs = full_grid(ks->full_small_cfg, causal, batch, q_len, n_q_heads, n_kv_heads);
        if (gs.pairs || fp.grid.items < device_info().cus) fp = FullPlan{&ks->full_small_cfg, gs, true};
    }
    return fp;
}

// Kernel mask variant of a mask kind (additive splits by mask element width).
int kernel_variant(sdpa_mask_kind mk, sdpa_dtype mask_dtype) {
    if (mk == SDPA_MASK_ADDITIVE) return mask_dtype == SDPA_F32 ? sdpa_dev::MASK_ADD32 : sdpa_dev::MASK_ADD16;
    if (mk == SDPA_MASK_SLIDING) return sdpa_dev::MASK_SLIDE;
    return (int)mk;
}

std::string route_string(int batch, int q_len, int kv_len, int hq, int hkv, int d, int dv, sdpa_dtype dt,
                         sdpa_mask_kind mk, int st, sdpa_kernel k, int reason) {
    char buf[256];
    char dn[32];
    if (dv == d)
        std::snprintf(dn, sizeof dn, "%d", d);
    else
        std::snprintf(dn, sizeof dn, "%d/v%d", d, dv);
    if (st != SDPA_OK) {
        std::snprintf(buf, sizeof buf, "unsupported (%s) B=%d Lq=%d Lk=%d Hq=%d Hkv=%d D=%s %s %s: reason %d",
                      sdpa_strerror(st), batch, q_len, kv_len, hq, hkv, dn, dtype_name(dt), mask_name(mk), reason);
        return buf;
    }
    const KernelSet* ks = kernel_set(dt, d, dv);
    if (k == SDPA_KERNEL_FULL) {
        const int variant = mk == SDPA_MASK_CAUSAL ? sdpa_dev::MASK_CAUSAL : sdpa_dev::MASK_NONE;
        const FullPlan fp = full_plan(ks, variant, batch, q_len, hq, hkv);
        const auto& t = *fp.cfg;
        const FullGrid fg = fp.grid;
        // a boolean mask with the workspace sdpa_workspace_size() names: lane words
        // built by a pre-pass launch, then the kernel
        const bool words = mk == SDPA_MASK_BOOLEAN && ks->full_bits && !fp.small;
        std::snprintf(buf, sizeof buf,
                      "full %s d%s %s B=%d Lq=%d Lk=%d Hq=%d Hkv=%d tile=%dx%d waves=%dx%d lds=%d workgroups=%ld%s%s",
                      dtype_name(dt), dn, mask_name(mk), batch, q_len, kv_len, hq, hkv, t.cols, t.bn, t.wm, t.wd,
                      t.lds, fg.items, fg.pairs ? " causal-pairs" : "", words ? " lane-words+prepass" : "");
    } else {
        const auto& t = ks->dec_cfg;
        const FusedPlan f = fused_plan(ks, batch, q_len, kv_len, hq, hkv, 0, kernel_variant(mk, SDPA_BF16));
        if (f.use) {
            std::snprintf(buf, sizeof buf,
                          "vector-fused %s d%s %s B=%d Lq=%d Lk=%d Hq=%d Hkv=%d groups=%d splits=%d "
                          "blocks/split=%d colgroups=%d threads=%d xcds=%d",
                          dtype_name(dt), dn, mask_name(mk), batch, q_len, kv_len, hq, hkv, f.groups, f.splits,
                          (f.nblk + f.splits - 1) / f.splits, f.col_groups, ks->fused_nt,
                          device_info().nx);
        } else {
            DecodePlan p = decode_plan(batch, q_len, kv_len, hq, hkv, t);
            std::snprintf(buf, sizeof buf,
                          "vector %s d%s %s B=%d Lq=%d Lk=%d Hq=%d Hkv=%d splits=%d keys/split=%d colgroups=%d "
                          "cols=%d threads=%d lds=%d",
                          dtype_name(dt), dn, mask_name(mk), batch, q_len, kv_len, hq, hkv, p.splits,
                          p.keys_per_split, p.col_groups, t.cols, t.nt, t.lds);
        }
    }
    return buf;
}

void log_route_once(const std::string& s) {
    static const bool on = [] {
        const char* e = std::getenv("SDPA_LOG_ROUTE");
        return e && e[0] && e[0] != '0';
    }();
    if (!on) return;
    static std::mutex mu;
    static std::set<std::string> seen;
    std::lock_guard<std::mutex> lock(mu);
    if (seen.insert(s).second) std::fprintf(stderr, "[sdpa] %s\n", s.c_str());
}

// Event ring for sdpa_timing_start / sdpa_timing_stop (per thread).
struct Timing {
    std::vector<hipEvent_t> ev;  // 3 per call
    std::vector<int> nkern;      // kernels recorded per call
    int armed = 0;
    int used = 0;
};
thread_local Timing g_timing;

hipEvent_t timing_event(int call, int k) { return g_timing.ev[3 * call + k]; }

int reject(int st) {
    g_counters[3].fetch_add(1, std::memory_order_relaxed);
    return st;
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return SDPA_OK;
    g_last_hip_error = (int)e;
    if (e == hipErrorInvalidConfiguration) return SDPA_ELAUNCH;
    return SDPA_EHIP;
}

}  // namespace

extern "C" {

int sdpa_select_kernel(int batch, int q_len, int kv_len, int n_q_heads, int n_kv_heads, int head_dim,
                       sdpa_dtype dtype, sdpa_mask_kind mask_kind, sdpa_kernel* kernel, int* reason) {
    return select(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, head_dim, dtype, mask_kind, kernel, reason);
}

int sdpa_select_kernel_ex(int batch, int q_len, int kv_len, int n_q_heads, int n_kv_heads, int head_dim,
                          int v_head_dim, sdpa_dtype dtype, sdpa_mask_kind mask_kind, sdpa_kernel* kernel,
                          int* reason) {
    return select(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, v_head_dim, dtype, mask_kind, kernel,
                  reason);
}

int sdpa_describe_route_ex(int batch, int q_len, int kv_len, int n_q_heads, int n_kv_heads, int head_dim,
                           int v_head_dim, sdpa_dtype dtype, sdpa_mask_kind mask_kind, char* buf, size_t len) {
    sdpa_kernel k;
    int reason;
    const int st =
        select(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, v_head_dim, dtype, mask_kind, &k, &reason);
    if (buf && len) {
        const std::string s = route_string(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, v_head_dim, dtype,
                                           mask_kind, st, k, reason);
        std::snprintf(buf, len, "%s", s.c_str());
    }
    return st;
}

int sdpa_describe_route(int batch, int q_len, int kv_len, int n_q_heads, int n_kv_heads, int head_dim,
                        sdpa_dtype dtype, sdpa_mask_kind mask_kind, char* buf, size_t len) {
    return sdpa_describe_route_ex(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, head_dim, dtype, mask_kind,
                                  buf, len);
}

size_t sdpa_workspace_size_ex(int batch, int q_len, int kv_len, int n_q_heads, int n_kv_heads, int head_dim,
                              int v_head_dim, sdpa_dtype dtype) {
    sdpa_kernel k;
    if (select(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, v_head_dim, dtype, SDPA_MASK_NONE, &k,
               nullptr) != SDPA_OK)
        return 0;
    const KernelSet* ks = kernel_set(dtype, head_dim, v_head_dim);
    // prefill: room for the lane masks of a boolean mask shared by every batch
    // and head (a per-head mask needs more and otherwise runs on the bytes)
    if (k != SDPA_KERNEL_VECTOR) return (ks && ks->full_bits) ? kCounterBytes + mask_bits_bytes(q_len, kv_len) : 0;
    // an upper bound over every mask kind, window and rotary option: the
    // single-launch plan (its split count only grows with the key count), and
    // the split + combine plan's largest split count
    size_t need = 0;
    for (int rope = 0; rope < 2; ++rope)
        for (int var = 0; var < sdpa_dev::MASK_VARIANTS; ++var) {
            // (a mask tensor without aligned 4-key runs takes the split + combine kernels)
            const FusedPlan f = fused_plan(ks, batch, q_len, kv_len, n_q_heads, n_kv_heads, rope, var);
            const size_t bf = f.use ? fused_ws_bytes(f, v_head_dim) : 0;
            const size_t bs = decode_ws_bytes(batch, q_len, n_q_heads, v_head_dim,
                                              split_cap(batch, q_len, kv_len, n_q_heads, n_kv_heads, ks->dec_cfg,
                                                        device_info().cus),
                                              dtype);
            const bool tensor = var == sdpa_dev::MASK_ADD16 || var == sdpa_dev::MASK_ADD32 || var == sdpa_dev::MASK_BOOL;
            const size_t b = (f.use && !tensor) ? bf : (bf > bs ? bf : bs);
            if (b > need) need = b;
        }
    return need;
}

size_t sdpa_workspace_size(int batch, int q_len, int kv_len, int n_q_heads, int n_kv_heads, int head_dim,
                           sdpa_dtype dtype) {
    return sdpa_workspace_size_ex(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, head_dim, dtype);
}

int sdpa_head_dims(int* out, int n) {
    const int total = (int)(sizeof(kHeadDims) / sizeof(kHeadDims[0]));
    for (int i = 0; out && i < n && i < total; ++i) out[i] = kHeadDims[i];
    return total;
}

const char* sdpa_strerror(int status) {
    switch (status) {
        case SDPA_OK: return "ok";
        case SDPA_EINVAL: return "invalid argument";
        case SDPA_EUNSUPPORTED: return "unsupported shape, type or layout (no fused kernel; no fallback)";
        case SDPA_EWORKSPACE: return "workspace too small";
        case SDPA_ELAUNCH: return "launch shape exceeds the kernel's limits";
        case SDPA_EHIP: return "HIP runtime error";
    }
    return "unknown status";
}

int sdpa_last_hip_error(void) { return g_last_hip_error; }

int sdpa_timing_start(int max_calls) {
    float dummy;
    if (!g_timing.ev.empty()) sdpa_timing_stop(&dummy, 0);
    if (max_calls <= 0) return SDPA_EINVAL;
    g_timing.ev.assign(3 * (size_t)max_calls, nullptr);
    g_timing.nkern.assign(max_calls, 0);
    for (auto& e : g_timing.ev) {
        const hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) {
            g_last_hip_error = (int)r;
            return SDPA_EHIP;
        }
    }
    g_timing.armed = max_calls;
    g_timing.used = 0;
    return SDPA_OK;
}

int sdpa_timing_stop(float* ms, int cap) {
    int st = g_timing.used;
    for (int i = 0; i < g_timing.used; ++i) {
        for (int k = 0; k < 2; ++k) {
            float t = 0.f;
            if (k < g_timing.nkern[i]) {
                hipError_t r = hipEventSynchronize(timing_event(i, k + 1));
                if (r == hipSuccess) r = hipEventElapsedTime(&t, timing_event(i, k), timing_event(i, k + 1));
                if (r != hipSuccess) {
                    g_last_hip_error = (int)r;
                    st = SDPA_EHIP;
                }
            }
            if (ms && 2 * i + k < cap) ms[2 * i + k] = t;
        }
    }
    for (auto e : g_timing.ev)
        if (e) (void)hipEventDestroy(e);
    g_timing = Timing();
    return st;
}

int sdpa_route_counters(uint64_t* out, int n) {
    for (int i = 0; out && i < n && i < 4; ++i) out[i] = g_counters[i].load(std::memory_order_relaxed);
    return 4;
}

}  // extern "C"

// The allocation-free entry point's scratch: one static device array per GPU
// (the code object is loaded on every device the library runs on), zero at
// load.  Host code never passes the array's name to a kernel: it keeps the
// device address hipGetSymbolAddress returns for each device, taken once with
// that device current.
constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_pointer(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return SDPA_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!ptr || ((uintptr_t)ptr) % 256 != 0) return SDPA_EHIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SDPA_OK;
}

// The rotary embedding of a strided [B, H, L, D] tensor into y (arguments
// already checked): 16 bytes per thread when R is a multiple of two 16-byte
// chunks and rows and tables are 16-byte aligned, else one thread per column.
// Both kernels give the same bits.
int launch_rope(const void* x, const sdpa_strides& x_st, void* y, const sdpa_strides& y_st, int batch, int n_heads,
                int len, int head_dim, sdpa_dtype dtype, int r, int pos0, const float* cos, const float* sin,
                hipStream_t s) {
    const int es = elem_size(dtype), ne = 16 / es;
    sdpa_dev::RopeArgs a{};
    a.x = x;
    a.y = y;
    const int64_t xs[4] = {x_st.b, x_st.h, x_st.l, x_st.d}, ys[4] = {y_st.b, y_st.h, y_st.l, y_st.d};
    for (int i = 0; i < 4; ++i) {
        a.xs[i] = xs[i];
        a.ys[i] = ys[i];
    }
    a.B = batch;
    a.H = n_heads;
    a.L = len;
    a.D = head_dim;
    a.R = r;
    a.pos0 = pos0;
    a.cos = cos;
    a.sin = sin;
    const bool same = x == y && x_st.b == y_st.b && x_st.h == y_st.h && x_st.l == y_st.l;
    bool vec = r % (2 * ne) == 0 && head_dim % ne == 0 && ((uintptr_t)x) % 16 == 0 && ((uintptr_t)y) % 16 == 0 &&
               ((uintptr_t)cos) % 16 == 0 && ((uintptr_t)sin) % 16 == 0;
    for (int i = 0; i < 3; ++i) vec = vec && xs[i] % ne == 0 && ys[i] % ne == 0;
    if (vec) {
        const int nunit = r / 2 / ne + (same ? 0 : (head_dim - r) / ne);
        if (nunit == 0) return SDPA_OK;
        const int64_t total = (int64_t)batch * n_heads * len * nunit;
        if ((total + 255) / 256 > 0x7fffffffLL) return SDPA_EUNSUPPORTED;
        const dim3 grid((unsigned)((total + 255) / 256));
        if (dtype == SDPA_F32)
            hipLaunchKernelGGL(sdpa_dev::rope_kernel_vec<sdpa_dev::TF32>, grid, dim3(256), 0, s, a, nunit);
        else if (dtype == SDPA_F16)
            hipLaunchKernelGGL(sdpa_dev::rope_kernel_vec<sdpa_dev::TF16>, grid, dim3(256), 0, s, a, nunit);
        else
            hipLaunchKernelGGL(sdpa_dev::rope_kernel_vec<sdpa_dev::TBF16>, grid, dim3(256), 0, s, a, nunit);
        return hip_status(hipGetLastError());
    }
    const int64_t total = (int64_t)batch * n_heads * len * head_dim;
    if ((total + 255) / 256 > 0x7fffffffLL) return SDPA_EUNSUPPORTED;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (dtype == SDPA_F32)
        hipLaunchKernelGGL(sdpa_dev::rope_kernel<float>, grid, dim3(256), 0, s, a);
    else if (dtype == SDPA_F16)
        hipLaunchKernelGGL(sdpa_dev::rope_kernel<_Float16>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(sdpa_dev::rope_kernel<__bf16>, grid, dim3(256), 0, s, a);
    return hip_status(hipGetLastError());
}

int forward_impl(const void* q, sdpa_strides q_st, const void* k, sdpa_strides k_st, const void* v,
                 sdpa_strides v_st, void* out, sdpa_strides o_st, int batch, int q_len, int kv_len, int n_q_heads,
                 int n_kv_heads, int head_dim, int v_head_dim, sdpa_dtype dtype, float scale, sdpa_mask_kind mask_kind,
                 const void* mask, sdpa_strides mask_st, sdpa_dtype mask_dtype, int window,
                 const sdpa_rope_table* q_rope, int q_pos0, void* workspace, size_t workspace_bytes, void* stream) {
    sdpa_kernel kern;
    int reason;
    int st = select(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, v_head_dim, dtype, mask_kind, &kern,
                    &reason);
    if (st != SDPA_OK) return reject(st);
    if (!std::isfinite(scale)) return reject(SDPA_EINVAL);

    const int es = elem_size(dtype);
    const int64_t nq[4] = {batch, n_q_heads, q_len, head_dim};
    const int64_t nk[4] = {batch, n_kv_heads, kv_len, head_dim};
    const int64_t nv[4] = {batch, n_kv_heads, kv_len, v_head_dim};
    const int64_t no[4] = {batch, n_q_heads, q_len, v_head_dim};
    if ((st = check_operand(q, q_st, nq, es)) != SDPA_OK) return reject(st);
    if ((st = check_operand(k, k_st, nk, es)) != SDPA_OK) return reject(st);
    if ((st = check_operand(v, v_st, nv, es)) != SDPA_OK) return reject(st);
    if ((st = check_operand(out, o_st, no, es)) != SDPA_OK) return reject(st);
    // K/V rows are read through 32-bit buffer offsets from each (batch, kv head)
    // base: rows may not overlap and one head's keys must span < 4 GiB.
    if (kv_len > 1 && (k_st.l < head_dim || v_st.l < v_head_dim)) return reject(SDPA_EUNSUPPORTED);
    if ((double)kv_len * (double)(k_st.l > 0 ? k_st.l : 1) * es >= 4294967296.0 ||
        (double)kv_len * (double)(v_st.l > 0 ? v_st.l : 1) * es >= 4294967296.0)
        return reject(SDPA_EUNSUPPORTED);
    const size_t oq = span_bytes(no, o_st, es);
    const size_t sq = span_bytes(nq, q_st, es), sk = span_bytes(nk, k_st, es), sv = span_bytes(nv, v_st, es);
    if (overlaps(out, oq, q, sq) || overlaps(out, oq, k, sk) || overlaps(out, oq, v, sv)) return reject(SDPA_EINVAL);

    Params p{};
    int mvec = 0;
    if (mask_kind == SDPA_MASK_ADDITIVE || mask_kind == SDPA_MASK_BOOLEAN) {
        if (!mask) return reject(SDPA_EINVAL);
        if (mask_kind == SDPA_MASK_BOOLEAN && mask_dtype != SDPA_U8) return reject(SDPA_EINVAL);
        if (mask_kind == SDPA_MASK_ADDITIVE && mask_dtype != SDPA_F32 && mask_dtype != SDPA_F16 &&
            mask_dtype != SDPA_BF16)
            return reject(SDPA_EINVAL);
        if (mask_st.b < 0 || mask_st.h < 0 || mask_st.l < 0 || mask_st.d < 0) return reject(SDPA_EINVAL);
        const int mes = elem_size(mask_dtype);
        if (((uintptr_t)mask) % mes != 0) return reject(SDPA_EUNSUPPORTED);
        // Mask offsets within a wave's rows are 32-bit: 64 rows plus one tile
        // past the last key must stay below 4 GiB.
        if (((double)mask_st.l * 64.0 + (double)(kv_len + 256) * (double)mask_st.d) * mes >= 4294967295.0)
            return reject(SDPA_EUNSUPPORTED);
        // Vector mask loads need 4-key runs aligned to 4 elements.
        mvec = mask_st.d == 1 && ((uintptr_t)mask) % (4 * mes) == 0 && mask_st.b % 4 == 0 && mask_st.h % 4 == 0 &&
               mask_st.l % 4 == 0;
        p.mask = mask;
        const int64_t mn[4] = {batch, n_q_heads, q_len, kv_len};
        p.mask_span = (int64_t)span_bytes(mn, mask_st, mes);
        if (overlaps(out, oq, mask, (size_t)p.mask_span)) return reject(SDPA_EINVAL);
        p.ms[0] = mask_st.b;
        p.ms[1] = mask_st.h;
        p.ms[2] = mask_st.l;
        p.ms[3] = mask_st.d;
        p.mask_dtype = (int)mask_dtype;
    }
    p.mask_vec = mvec;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = out;
    const sdpa_strides* sts[4] = {&q_st, &k_st, &v_st, &o_st};
    int64_t* dst[4] = {p.qs, p.ks, p.vs, p.os};
    for (int i = 0; i < 4; ++i) {
        dst[i][0] = sts[i]->b;
        dst[i][1] = sts[i]->h;
        dst[i][2] = sts[i]->l;
        dst[i][3] = sts[i]->d;
    }
    p.B = batch;
    p.Lq = q_len;
    p.Lk = kv_len;
    p.Hq = n_q_heads;
    p.Hkv = n_kv_heads;
    p.n_rep = n_q_heads / n_kv_heads;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);
    p.scale_nonneg = scale >= 0.f;
    p.window = window;
    p.kbase = 0;
    size_t rope_bytes = 0;
    if (q_rope && q_rope->rotary_dim != 0) {
        const int r = q_rope->rotary_dim;
        if (r < 0 || r % 2 != 0 || r > head_dim) return reject(SDPA_EUNSUPPORTED);
        if (!q_rope->cos || !q_rope->sin || q_pos0 < 0 || (long)q_pos0 + q_len > (long)q_rope->n_pos)
            return reject(SDPA_EINVAL);
        if (((uintptr_t)q_rope->cos) % 16 != 0 || ((uintptr_t)q_rope->sin) % 16 != 0) return reject(SDPA_EUNSUPPORTED);
        const size_t tb = (size_t)q_rope->n_pos * (size_t)(r / 2) * sizeof(float);
        if (overlaps(out, oq, q_rope->cos, tb) || overlaps(out, oq, q_rope->sin, tb)) return reject(SDPA_EINVAL);
        rope_bytes = tb;
        p.rope_dim = r;
        p.rope_pos0 = q_pos0;
        p.rope_cos = q_rope->cos;
        p.rope_sin = q_rope->sin;
    }
    // Where the in-kernel rotation of Q costs more than a pass of its own (many
    // fragments per lane: rotary dims above 128, a full rotation of 128; or the
    // column-by-column path beyond 32 columns), Q is rotated into `out` first and
    // the kernels read it from there without a table.  `out` has Q's shape when
    // v_head_dim == head_dim, and every workgroup reads the query rows it later
    // overwrites with their output before it writes them, so no buffer is needed.
    const bool q_prepass =
        p.rope_dim > 0 && v_head_dim == head_dim &&
        (p.rope_dim > 128 || (p.rope_dim == 128 && head_dim == 128) || (p.rope_dim % 16 != 0 && p.rope_dim > 32));
    const bool rope_k = p.rope_dim > 0 && !q_prepass;  // kernels with the rotary prologue
    auto rotate_q_into_out = [&]() -> int {
        if (!q_prepass) return SDPA_OK;
        const int rs = launch_rope(q, q_st, out, o_st, batch, n_q_heads, q_len, head_dim, dtype, p.rope_dim,
                                   p.rope_pos0, p.rope_cos, p.rope_sin, reinterpret_cast<hipStream_t>(stream));
        if (rs != SDPA_OK) return rs;
        p.q = out;
        for (int i = 0; i < 4; ++i) p.qs[i] = p.os[i];
        p.rope_dim = 0;
        return SDPA_OK;
    };

    const KernelSet* ks = kernel_set(dtype, head_dim, v_head_dim);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int mk = kernel_variant(mask_kind, mask_dtype);
    const DevInfo di = device_info();
    p.nx = di.nx;
    // optional per-kernel timing (diagnostics): events bracket each launch on `s`
    int tcall = -1;
    if (g_timing.used < g_timing.armed) tcall = g_timing.used++;
    auto mark = [&](int k) {
        if (tcall >= 0) {
            (void)hipEventRecord(timing_event(tcall, k), s);
            g_timing.nkern[tcall] = k;
        }
    };

    // bytes a kernel writes in the workspace must not be an operand any kernel reads
    // or the output it writes
    auto ws_overlaps = [&](const void* w, size_t n) {
        return overlaps(out, oq, w, n) || overlaps(q, sq, w, n) || overlaps(k, sk, w, n) || overlaps(v, sv, w, n) ||
               (p.mask && overlaps(p.mask, (size_t)p.mask_span, w, n)) ||
               (rope_bytes && (overlaps(p.rope_cos, rope_bytes, w, n) || overlaps(p.rope_sin, rope_bytes, w, n)));
    };

    if (kern == SDPA_KERNEL_FULL) {
        const FullPlan fp = full_plan(ks, mk, batch, q_len, n_q_heads, n_kv_heads);
        p.pairs = fp.grid.pairs;
        const long items = fp.grid.items;
        if (items > (1L << 30)) return reject(SDPA_EUNSUPPORTED);
        dim3 grid((unsigned)(di.nx * ((items + di.nx - 1) / di.nx)), 1, 1);
        log_route_once(route_string(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, v_head_dim, dtype,
                                    mask_kind, st, kern, reason));
        const bool strided = !p.mask_vec && ks->full_strided[mk];
        // a boolean mask goes in as lane masks when the workspace holds them (one
        // pass over the mask, shared by every head that reads it)
        const int bm = (mask_kind == SDPA_MASK_BOOLEAN && p.ms[0] != 0) ? batch : 1;
        const int hm = (mask_kind == SDPA_MASK_BOOLEAN && p.ms[1] != 0) ? n_q_heads : 1;
        const size_t bits_need = mask_bits_bytes(q_len, kv_len) * (size_t)bm * (size_t)hm;
        // (word offsets per mask head and batch are ints: under 2^31 words)
        const bool bits = mask_kind == SDPA_MASK_BOOLEAN && !fp.small && ks->full_bits && workspace &&
                          workspace_bytes >= kCounterBytes + bits_need && ((uintptr_t)workspace) % 256 == 0 &&
                          bits_need < ((size_t)1 << 34);
        char* const bits_at = reinterpret_cast<char*>(workspace) + kCounterBytes;
        if (bits && ws_overlaps(bits_at, bits_need)) return reject(SDPA_EINVAL);
        const launch_fn f = bits         ? (rope_k ? ks->full_bits_rope : ks->full_bits)
                            : fp.small   ? (rope_k ? ks->full_small_rope[mk] : ks->full_small[mk])
                            : strided    ? (rope_k ? ks->full_strided_rope[mk] : ks->full_strided[mk])
                                         : (rope_k ? ks->full_rope[mk] : ks->full[mk]);
        if (!f) return reject(SDPA_EUNSUPPORTED);
        mark(0);
        if ((st = rotate_q_into_out()) != SDPA_OK) return reject(st);
        if (bits) {
            const int rbn = (q_len + 31) / 32, ktn = (kv_len + 63) / 64;
            sdpa_dev::MaskBitsArgs a{};
            a.mask = reinterpret_cast<const uint8_t*>(p.mask);
            for (int i = 0; i < 4; ++i) a.ms[i] = p.ms[i];
            a.bits = reinterpret_cast<uint32_t*>(bits_at);
            a.Bm = bm;
            a.Hm = hm;
            a.Lq = q_len;
            a.Lk = kv_len;
            a.RB = rbn;
            a.KT = ktn;
            // 16-byte loads: key stride 1 and every row start 16-byte aligned
            const uintptr_t mp = (uintptr_t)p.mask;
            a.vec = p.ms[3] == 1 && mp % 16 == 0 && p.ms[0] % 16 == 0 && p.ms[1] % 16 == 0 && p.ms[2] % 16 == 0;
            const int64_t units = (int64_t)bm * hm * rbn * ktn;
            hipLaunchKernelGGL(sdpa_dev::mask_bits_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, s, a);
            if ((st = hip_status(hipGetLastError())) != SDPA_OK) return reject(st);
            const int64_t per_rb = (int64_t)ktn * sdpa_dev::kMaskBitsWords;
            p.mask_bits = a.bits;
            p.mb_rb = (int)per_rb;
            p.mb_h = hm > 1 ? (int)(per_rb * rbn) : 0;
            p.mb_b = bm > 1 ? (int)(per_rb * rbn * hm) : 0;
        }
        st = hip_status(f(p, grid, s));
        if (st != SDPA_OK) return reject(st);
        mark(1);
        g_counters[1].fetch_add(1, std::memory_order_relaxed);
        return SDPA_OK;
    }

    // vector (decode): split keys, then combine the splits
    const auto& t = ks->dec_cfg;
    // a sliding window reaches no key left of (first row's position - window + 1):
    // split only the keys from there on
    if (mask_kind == SDPA_MASK_SLIDING) {
        const long lo = (long)(kv_len - q_len) - window + 1;
        p.kbase = lo > 0 ? (int)lo : 0;
    }
    // the single-launch kernel reads mask tensors in aligned 4-key vectors with 32-bit offsets
    const bool mask_ok = !p.mask || (p.mask_vec && p.mask_span < (int64_t)0xffffffffLL);
    const FusedPlan fpl = fused_plan(ks, batch, q_len, kv_len - p.kbase, n_q_heads, n_kv_heads, rope_k, mk,
                                     mask_ok);
    if (fpl.use) {
        const size_t need = fused_ws_bytes(fpl, v_head_dim);
        if (need && (!workspace || workspace_bytes < need)) return reject(SDPA_EWORKSPACE);
        if (need && ((uintptr_t)workspace) % 256 != 0) return reject(SDPA_EINVAL);
        if (need && ws_overlaps(workspace, need)) return reject(SDPA_EINVAL);
        const size_t slots = (size_t)fpl.groups * fpl.splits * fpl.rv;
        p.ws_o = reinterpret_cast<float*>(workspace);
        p.ws_ml = need ? reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + kCounterBytes +
                                                  align256(slots * v_head_dim * sizeof(float)))
                       : nullptr;
        p.col_groups = fpl.col_groups;
        sdpa_dev::FusedGeom fg{sdpa_dev::make_fastdiv(di.nx), sdpa_dev::make_fastdiv(fpl.splits),
                               sdpa_dev::make_fastdiv(fpl.col_groups), sdpa_dev::make_fastdiv(n_kv_heads),
                               sdpa_dev::make_fastdiv(q_len), fpl.groups, fpl.nblk, fpl.rv};
        // test-only: another XCD stride scatters a group's splits over several XCDs,
        // which the kernel must detect (and recompute the group)
        if (const char* env = std::getenv("SDPA_FUSED_XCD_STRIDE")) {
            const long v = std::strtol(env, nullptr, 10);
            if (v > 0 && fpl.groups % v == 0) fg.nx = sdpa_dev::make_fastdiv((int)v);
        }
        log_route_once(route_string(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, v_head_dim, dtype,
                                    mask_kind, st, kern, reason));
        const sdpa_host::fused_fn f = rope_k ? ks->decode_fused_rope[mk] : ks->decode_fused[mk];
        if (!f) return reject(SDPA_EUNSUPPORTED);
        mark(0);
        if ((st = rotate_q_into_out()) != SDPA_OK) return reject(st);
        st = hip_status(f(p, fg, dim3((unsigned)(fpl.groups * fpl.splits)), s));
        if (st != SDPA_OK) return reject(st);
        mark(1);
        g_counters[2].fetch_add(1, std::memory_order_relaxed);
        return SDPA_OK;
    }
    const DecodePlan plan = decode_plan(batch, q_len, kv_len - p.kbase, n_q_heads, n_kv_heads, t);
    const size_t need = decode_ws_bytes(batch, q_len, n_q_heads, v_head_dim, plan.splits, dtype);
    if (need && (!workspace || workspace_bytes < need)) return reject(SDPA_EWORKSPACE);
    if (need && ((uintptr_t)workspace) % 256 != 0) return reject(SDPA_EINVAL);
    if (need && ws_overlaps(workspace, need)) return reject(SDPA_EINVAL);
    if ((long)n_kv_heads * plan.col_groups > kMaxGridYZ) return reject(SDPA_EUNSUPPORTED);
    const size_t rows = (size_t)batch * n_q_heads * q_len;
    p.ws_o = need ? reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + kCounterBytes) : nullptr;
    p.ws_ml = need ? reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + kCounterBytes +
                                              align256(rows * plan.splits * v_head_dim * sizeof(float)))
                   : nullptr;
    p.splits = plan.splits;
    p.keys_per_split = plan.keys_per_split;
    p.col_groups = plan.col_groups;
    log_route_once(route_string(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, v_head_dim, dtype, mask_kind,
                                st, kern, reason));
    dim3 grid((unsigned)plan.splits, (unsigned)(n_kv_heads * plan.col_groups), (unsigned)batch);
    const launch_fn f = rope_k ? ks->decode_rope[mk] : ks->decode[mk];
    if (!f) return reject(SDPA_EUNSUPPORTED);
    mark(0);
    if ((st = rotate_q_into_out()) != SDPA_OK) return reject(st);
    st = hip_status(f(p, grid, s));
    if (st != SDPA_OK) return reject(st);
    mark(1);
    // a single split of the 16-bit kernel writes the output itself
    if (!(plan.splits == 1 && dtype != SDPA_F32)) {
        dim3 cgrid((unsigned)rows, (unsigned)((v_head_dim + 63) / 64), 1);
        st = hip_status(ks->combine(p, cgrid, s));
        if (st != SDPA_OK) return reject(st);
        mark(2);
    }
    g_counters[2].fetch_add(1, std::memory_order_relaxed);
    return SDPA_OK;
}

}  // namespace

extern "C" {

int sdpa_forward(const void* q, sdpa_strides q_st, const void* k, sdpa_strides k_st, const void* v,
                 sdpa_strides v_st, void* out, sdpa_strides o_st, int batch, int q_len, int kv_len, int n_q_heads,
                 int n_kv_heads, int head_dim, sdpa_dtype dtype, float scale, sdpa_mask_kind mask_kind,
                 const void* mask, sdpa_strides mask_st, sdpa_dtype mask_dtype, void* workspace,
                 size_t workspace_bytes, void* stream) {
    g_counters[0].fetch_add(1, std::memory_order_relaxed);
    if (mask_kind == SDPA_MASK_SLIDING) return reject(SDPA_EINVAL);  // needs a window: sdpa_forward_sliding
    return forward_impl(q, q_st, k, k_st, v, v_st, out, o_st, batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim,
                        head_dim, dtype, scale, mask_kind, mask, mask_st, mask_dtype, 0, nullptr, 0, workspace,
                        workspace_bytes, stream);
}

int sdpa_forward_sliding(const void* q, sdpa_strides q_st, const void* k, sdpa_strides k_st, const void* v,
                         sdpa_strides v_st, void* out, sdpa_strides o_st, int batch, int q_len, int kv_len,
                         int n_q_heads, int n_kv_heads, int head_dim, sdpa_dtype dtype, float scale, int window,
                         void* workspace, size_t workspace_bytes, void* stream) {
    g_counters[0].fetch_add(1, std::memory_order_relaxed);
    if (window < 1) return reject(SDPA_EINVAL);
    const sdpa_strides none{0, 0, 0, 0};
    return forward_impl(q, q_st, k, k_st, v, v_st, out, o_st, batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim,
                        head_dim, dtype, scale, SDPA_MASK_SLIDING, nullptr, none, SDPA_F32, window, nullptr, 0,
                        workspace, workspace_bytes, stream);
}

int sdpa_forward_ex(const void* q, sdpa_strides q_st, const void* k, sdpa_strides k_st, const void* v,
                    sdpa_strides v_st, void* out, sdpa_strides o_st, int batch, int q_len, int kv_len, int n_q_heads,
                    int n_kv_heads, int head_dim, int v_head_dim, sdpa_dtype dtype, float scale,
                    sdpa_mask_kind mask_kind, const void* mask, sdpa_strides mask_st, sdpa_dtype mask_dtype, int window,
                    const sdpa_rope_table* q_rope, int q_pos0, void* workspace, size_t workspace_bytes, void* stream) {
    g_counters[0].fetch_add(1, std::memory_order_relaxed);
    if (mask_kind == SDPA_MASK_SLIDING && window < 1) return reject(SDPA_EINVAL);
    return forward_impl(q, q_st, k, k_st, v, v_st, out, o_st, batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim,
                        v_head_dim, dtype, scale, mask_kind, mask, mask_st, mask_dtype,
                        mask_kind == SDPA_MASK_SLIDING ? window : 0, q_rope, q_pos0, workspace, workspace_bytes,
                        stream);
}

int sdpa_forward_noalloc(const void* q, sdpa_strides q_st, const void* k, sdpa_strides k_st, const void* v,
                         sdpa_strides v_st, void* out, sdpa_strides o_st, int batch, int q_len, int kv_len,
                         int n_q_heads, int n_kv_heads, int head_dim, int v_head_dim, sdpa_dtype dtype, float scale,
                         sdpa_mask_kind mask_kind, const void* mask, sdpa_strides mask_st, sdpa_dtype mask_dtype,
                         int window, const sdpa_rope_table* q_rope, int q_pos0, void* stream) {
    g_counters[0].fetch_add(1, std::memory_order_relaxed);
    if (mask_kind == SDPA_MASK_SLIDING && window < 1) return reject(SDPA_EINVAL);
    size_t need = sdpa_workspace_size_ex(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, v_head_dim, dtype);
    if (need > kScratchBytes) {
        // a prefill's workspace only speeds up boolean masks (lane masks): run without it
        sdpa_kernel kk;
        if (select(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, v_head_dim, dtype, mask_kind, &kk,
                   nullptr) == SDPA_OK &&
            kk == SDPA_KERNEL_FULL)
            need = 0;
        else
            return reject(SDPA_EWORKSPACE);
    }
    void* ws = nullptr;
    if (need) {
        const int st = scratch_pointer(&ws);
        if (st != SDPA_OK) return reject(st);
    }
    return forward_impl(q, q_st, k, k_st, v, v_st, out, o_st, batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim,
                        v_head_dim, dtype, scale, mask_kind, mask, mask_st, mask_dtype,
                        mask_kind == SDPA_MASK_SLIDING ? window : 0, q_rope, q_pos0, ws, need ? kScratchBytes : 0,
                        stream);
}

size_t sdpa_noalloc_scratch_bytes(void) { return kScratchBytes; }

int sdpa_rope(const void* x, sdpa_strides x_st, void* y, sdpa_strides y_st, int batch, int n_heads, int len,
              int head_dim, sdpa_dtype dtype, const sdpa_rope_table* rope, int pos0, void* stream) {
    if (batch <= 0 || n_heads <= 0 || len <= 0 || head_dim <= 0 || !rope || !x || !y) return SDPA_EINVAL;
    if (dtype != SDPA_F32 && dtype != SDPA_F16 && dtype != SDPA_BF16) return SDPA_EUNSUPPORTED;
    const int r = rope->rotary_dim;
    if (r <= 0 || r % 2 != 0 || r > head_dim) return SDPA_EINVAL;
    if (!rope->cos || !rope->sin || pos0 < 0 || (long)pos0 + len > (long)rope->n_pos) return SDPA_EINVAL;
    if (x_st.b < 0 || x_st.h < 0 || x_st.l < 0 || y_st.b < 0 || y_st.h < 0 || y_st.l < 0) return SDPA_EINVAL;
    if (x_st.d != 1 || y_st.d != 1) return SDPA_EUNSUPPORTED;
    const int es = elem_size(dtype);
    const int64_t n[4] = {batch, n_heads, len, head_dim};
    const bool same = x == y && x_st.b == y_st.b && x_st.h == y_st.h && x_st.l == y_st.l;
    if (!same && overlaps(y, span_bytes(n, y_st, es), x, span_bytes(n, x_st, es))) return SDPA_EINVAL;
    const int64_t total = (int64_t)batch * n_heads * len * head_dim;
    if ((total + 255) / 256 > 0x7fffffffLL) return SDPA_EUNSUPPORTED;
    return launch_rope(x, x_st, y, y_st, batch, n_heads, len, head_dim, dtype, r, pos0, rope->cos, rope->sin,
                       reinterpret_cast<hipStream_t>(stream));
}

int sdpa_probe_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
    if (!src || !sink || bytes == 0) return SDPA_EINVAL;
    if (bytes % 16 != 0 || ((uintptr_t)src) % 16 != 0 || ((uintptr_t)sink) % 4 != 0) return SDPA_EINVAL;
    const DevInfo di = device_info();
    hipLaunchKernelGGL(sdpa_dev::stream_read_kernel, dim3((unsigned)di.cus), dim3(sdpa_dev::kProbeThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const sdpa_dev::u32x4_t*>(src),
                       (uint64_t)(bytes / 16), reinterpret_cast<uint32_t*>(sink));
    return hip_status(hipGetLastError());
}

}  // extern "C"
