// Host-side checks of libsdpa's planner and argument validation, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (see
// test_host_harness.py).  The library's host source is compiled in directly
// and its kernel tables are replaced by recording stubs: nothing is ever
// launched and no device pointer is dereferenced, so this runs on a machine
// without a GPU.  Device pointers below are made-up, aligned, non-overlapping
// addresses.
#include "sdpa_host.cpp"

#include <random>
#include <thread>
#include <vector>

#include "decode_kernel.h"

namespace {

int g_fail = 0;
long g_checks = 0;
#define CHECK(cond, ...)                                  \
    do {                                                  \
        ++g_checks;                                       \
        if (!(cond)) {                                    \
            if (g_fail < 20) {                            \
                std::fprintf(stderr, "FAIL %s: ", #cond); \
                std::fprintf(stderr, __VA_ARGS__);        \
                std::fprintf(stderr, "\n");               \
            }                                             \
            ++g_fail;                                     \
        }                                                 \
    } while (0)

struct Launch {
    int calls = 0;
    bool fused = false;
    sdpa_dev::Params p{};
    sdpa_dev::FusedGeom fg{};
    unsigned grid = 0;
};
Launch g_last;

hipError_t stub(const sdpa_dev::Params& p, dim3 grid, hipStream_t) {
    ++g_last.calls;
    g_last.fused = false;
    g_last.p = p;
    g_last.grid = grid.x * grid.y * grid.z;
    return hipSuccess;
}
hipError_t stub_fused(const sdpa_dev::Params& p, const sdpa_dev::FusedGeom& fg, dim3 grid, hipStream_t) {
    ++g_last.calls;
    g_last.fused = true;
    g_last.p = p;
    g_last.fg = fg;
    g_last.grid = grid.x * grid.y * grid.z;
    return hipSuccess;
}

template <class TR, int D, int DV = D>
sdpa_host::KernelSet make_set() {
    sdpa_host::KernelSet k{};
    for (int m = 0; m < sdpa_dev::MASK_VARIANTS; ++m) {
        if (DV == D) {
            k.full[m] = stub;
            if (TR::ES == 2) k.full_rope[m] = stub;
        }
        k.decode[m] = stub;
        if (TR::ES == 2) {
            k.decode_rope[m] = stub;
            if (D <= 256) {  // as the instantiation units: the single-launch kernel up to D = 256
                k.decode_fused[m] = stub_fused;
                k.decode_fused_rope[m] = stub_fused;
            }
        }
    }
    k.combine = stub;
    if (TR::ES == 2 && D <= 256) k.fused_nt = 512;
    // tile shapes as the instantiation units declare them (the planner reads bn, cols, nt)
    if constexpr (TR::ES == 2) {
        using V = sdpa_dev::DecCfg<TR, D, 4, DV>;
        k.dec_cfg = sdpa_host::TileInfo{V::KS, 16, 1, 1, V::NT, V::LDS};
    } else {
        k.dec_cfg = sdpa_host::TileInfo{32, 32, 1, 1, 64, 0};
    }
    k.full_cfg = sdpa_host::TileInfo{64, 128, 4, 1, 256, 0, D >= 256 ? 4 : 1, 1};
    return k;
}

}  // namespace

namespace sdpa_host {
#define SDPA_STUB_GETTER(D)                                                                      \
    const KernelSet* kernels_d##D(int dt) {                                                      \
        static const KernelSet s[3] = {make_set<sdpa_dev::TF32, D>(), make_set<sdpa_dev::TF16, D>(), \
                                       make_set<sdpa_dev::TBF16, D>()};                          \
        return (dt >= 0 && dt < 3) ? &s[dt] : nullptr;                                           \
    }
SDPA_HEAD_DIMS(SDPA_STUB_GETTER)
const KernelSet* kernels_q192_v128(int dt) {
    static const KernelSet s[2] = {make_set<sdpa_dev::TF16, 192, 128>(), make_set<sdpa_dev::TBF16, 192, 128>()};
    return (dt == 1 || dt == 2) ? &s[dt - 1] : nullptr;
}
}  // namespace sdpa_host

namespace {

constexpr uintptr_t kQ = 0x100000000000ull, kK = 0x200000000000ull, kV = 0x300000000000ull,
                    kO = 0x400000000000ull, kM = 0x500000000000ull, kW = 0x600000000000ull;

sdpa_strides bhld(int H, int L, int D) { return sdpa_strides{(int64_t)H * L * D, (int64_t)L * D, D, 1}; }

// Bytes of the workspace (at kW) the recorded decode launch touches; the
// partial outputs must end before the (max, sum) pairs begin.
size_t touched(const Launch& l, int dv) {
    const char* base = (const char*)kW;
    if (l.fused) {
        if (l.fg.splits.d == 1) return 0;
        const size_t slots = (size_t)l.fg.groups * l.fg.splits.d * l.fg.rv;
        const size_t o_end = (size_t)((const char*)l.p.ws_o - base) + 32768 + slots * (dv / (l.fg.groups / (l.p.B * l.p.Hkv * l.p.col_groups))) * 4;
        const size_t ml_beg = (size_t)((const char*)l.p.ws_ml - base);
        if (o_end > ml_beg) return (size_t)-1;
        return ml_beg + slots * 2 * sizeof(float);
    }
    const size_t rows = (size_t)l.p.B * l.p.Hq * l.p.Lq;
    if (!l.p.ws_o) return 0;  // a single split writes the output itself
    if ((const char*)l.p.ws_o - base < 32768) return (size_t)-1;  // the arrival words are not the combine's
    const size_t o_end = (size_t)((const char*)l.p.ws_o - base) + rows * l.p.splits * dv * sizeof(float);
    const size_t ml_beg = (size_t)((const char*)l.p.ws_ml - base);
    if (o_end > ml_beg) return (size_t)-1;
    return ml_beg + rows * l.p.splits * 2 * sizeof(float);
}

int call(int B, int lq, int lk, int hq, int hkv, int d, int dv, sdpa_dtype dt, sdpa_mask_kind mk, int window,
         size_t wsb, uintptr_t ws = kW) {
    const sdpa_strides qs = bhld(hq, lq, d), ks = bhld(hkv, lk, d), vs = bhld(hkv, lk, dv), os = bhld(hq, lq, dv);
    const sdpa_strides ms{0, 0, lk, 1};
    const void* mask = (mk == SDPA_MASK_ADDITIVE || mk == SDPA_MASK_BOOLEAN) ? (const void*)kM : nullptr;
    const sdpa_dtype mdt = mk == SDPA_MASK_BOOLEAN ? SDPA_U8 : dt;
    return sdpa_forward_ex((const void*)kQ, qs, (const void*)kK, ks, (const void*)kV, vs, (void*)kO, os, B, lq, lk, hq,
                           hkv, d, dv, dt, 0.125f, mk, mask, ms, mdt, window, nullptr, 0, (void*)ws, wsb, nullptr);
}

void sweep_workspace_bound() {
    const int Ls[] = {1, 15, 16, 17, 63, 64, 65, 100, 1000, 4096, 4100, 4160, 5000};
    const int Ws[] = {1, 7, 64, 1000, 4096, 5000};
    const int Hkvs[] = {1, 2, 3, 4, 8};
    const int reps[] = {1, 2, 4, 8};
    const int Ds[] = {64, 128, 256, 512};
    const sdpa_dtype dts[] = {SDPA_F32, SDPA_F16, SDPA_BF16};
    for (sdpa_dtype dt : dts)
        for (int d : Ds)
            for (int hkv : Hkvs)
                for (int rep : reps)
                    for (int lq : {1, 3, 8})
                        for (int lk : Ls) {
                            if (lq > lk) continue;
                            const int hq = hkv * rep;
                            const size_t ws = sdpa_workspace_size(1, lq, lk, hq, hkv, d, dt);
                            for (int mki = 0; mki <= 4; ++mki) {
                                const sdpa_mask_kind mk = (sdpa_mask_kind)mki;
                                for (int w : Ws) {
                                    if (mk != SDPA_MASK_SLIDING && w != Ws[0]) continue;
                                    g_last = Launch{};
                                    const int st = call(1, lq, lk, hq, hkv, d, d, dt, mk, w, ws);
                                    CHECK(st == SDPA_OK, "st=%d d=%d hkv=%d hq=%d lq=%d lk=%d mk=%d w=%d ws=%zu", st, d,
                                          hkv, hq, lq, lk, mki, w, ws);
                                    if (st != SDPA_OK) continue;
                                    CHECK(g_last.calls >= 1, "no launch");
                                    const size_t t = touched(g_last, d);
                                    CHECK(t <= ws, "touches %zu of %zu (d=%d hkv=%d hq=%d lq=%d lk=%d mk=%d w=%d fused=%d)",
                                          t, ws, d, hkv, hq, lq, lk, mki, w, (int)g_last.fused);
                                    if (ws > 0 && t > 0)
                                        CHECK(call(1, lq, lk, hq, hkv, d, d, dt, mk, w, t - 1) == SDPA_EWORKSPACE,
                                              "a workspace one byte short was accepted");
                                }
                            }
                        }
}

void check_fused_geometry() {
    // the bench decode shapes: one group per XCD, 32 splits of 128 keys
    g_last = Launch{};
    const size_t ws = sdpa_workspace_size(1, 1, 4096, 32, 8, 256, SDPA_BF16);
    CHECK(call(1, 1, 4096, 32, 8, 256, 256, SDPA_BF16, SDPA_MASK_ADDITIVE, 0, ws) == SDPA_OK, "c2");
    CHECK(g_last.fused && g_last.fg.groups == 8 && g_last.fg.splits.d == 32 && g_last.grid == 256 &&
              g_last.fg.nblk == 256 && g_last.fg.rv == 4,
          "c2 geometry fused=%d G=%d S=%d grid=%u", (int)g_last.fused, g_last.fg.groups, g_last.fg.splits.d,
          g_last.grid);
    g_last = Launch{};
    const size_t ws3 = sdpa_workspace_size(1, 1, 4096, 32, 4, 512, SDPA_BF16);
    CHECK(call(1, 1, 4096, 32, 4, 512, 512, SDPA_BF16, SDPA_MASK_ADDITIVE, 0, ws3) == SDPA_OK, "c3");
    CHECK(!g_last.fused && g_last.calls == 2, "c3 (D = 512): split + combine, fused=%d launches=%d",
          (int)g_last.fused, g_last.calls);
    // groups that do not spread evenly over the XCDs: split + combine kernels
    g_last = Launch{};
    const size_t ws4 = sdpa_workspace_size(1, 2, 3000, 12, 3, 128, SDPA_BF16);
    CHECK(call(1, 2, 3000, 12, 3, 128, 128, SDPA_BF16, SDPA_MASK_NONE, 0, ws4) == SDPA_OK, "3 kv heads");
    CHECK(!g_last.fused && g_last.calls == 2, "3 kv heads: fused=%d launches=%d", (int)g_last.fused, g_last.calls);
    // a full batch: one split per group, the kernel writes the output, no workspace
    CHECK(sdpa_workspace_size(64, 1, 512, 16, 8, 128, SDPA_BF16) == 0, "batch 64 needs no workspace");
    g_last = Launch{};
    CHECK(call(64, 1, 512, 16, 8, 128, 128, SDPA_BF16, SDPA_MASK_NONE, 0, 0, 0) == SDPA_OK, "batch 64");
    CHECK(g_last.fused && g_last.fg.splits.d == 1, "batch 64: S=%d", g_last.fg.splits.d);
}

// fast_div against the hardware division: divisors at and around every power
// of two and random ones, numerators at the edges of each quotient step and
// random ones below 2^31
void check_fast_div() {
    std::mt19937_64 rng(7);
    std::vector<int> ds;
    for (int l = 0; l < 31; ++l)
        for (int e = -2; e <= 2; ++e) {
            const long long d = (1LL << l) + e;
            if (d >= 1 && d < (1LL << 31)) ds.push_back((int)d);
        }
    for (int r = 0; r < 2000; ++r) ds.push_back(1 + (int)(rng() % ((1ULL << 31) - 1)));
    for (int r = 0; r < 2000; ++r) ds.push_back(1 + (int)(rng() % 300));
    for (const int d : ds) {
        const sdpa_dev::FastDiv f = sdpa_dev::make_fastdiv(d);
        std::vector<long long> ns = {0, 1, d - 1LL, d, d + 1LL, (1LL << 31) - 1, (1LL << 31) - 2, (1LL << 31) - d};
        const long long qmax = ((1LL << 31) - 1) / d;
        for (int r = 0; r < 64; ++r) {
            const long long q = (long long)(rng() % (unsigned long long)(qmax + 1));
            ns.push_back(q * d);
            ns.push_back(q * d - 1);
            ns.push_back(q * d + d - 1);
            ns.push_back((long long)(rng() % (1ULL << 31)));
        }
        for (const long long n : ns) {
            if (n < 0 || n >= (1LL << 31)) continue;
            CHECK(sdpa_dev::fast_div((int)n, f) == (int)(n / d), "fast_div(%lld, %d) = %d", n, d,
                  sdpa_dev::fast_div((int)n, f));
        }
    }
}

// The single-launch decode kernel's workgroup -> (group, split) mapping, taken
// on the host with the geometry the planner launched: every (group, split)
// exactly once, the splits of a group on one XCD (workgroup i on XCD i % nx),
// and the split key ranges tile [0, nblk) in order.
void check_fused_mapping() {
    struct Shape { int b, lq, lk, hq, hkv, d; };
    const Shape shapes[] = {{1, 1, 4096, 32, 8, 256}, {1, 1, 4096, 32, 4, 512}, {2, 3, 1000, 16, 4, 128},
                            {1, 8, 5000, 64, 8, 64},   {4, 1, 333, 8, 2, 96},    {1, 2, 70000, 16, 16, 128}};
    for (const Shape& sh : shapes) {
        g_last = Launch{};
        const size_t ws = sdpa_workspace_size(sh.b, sh.lq, sh.lk, sh.hq, sh.hkv, sh.d, SDPA_BF16);
        CHECK(call(sh.b, sh.lq, sh.lk, sh.hq, sh.hkv, sh.d, sh.d, SDPA_BF16, SDPA_MASK_NONE, 0, ws) == SDPA_OK,
              "mapping shape Hq=%d Hkv=%d", sh.hq, sh.hkv);
        if (!g_last.fused) continue;
        const sdpa_dev::FusedGeom& fg = g_last.fg;
        const int S = fg.splits.d, G = fg.groups, nx = fg.nx.d;
        CHECK((long)G * S == (long)g_last.grid, "grid %u for G=%d S=%d", g_last.grid, G, S);
        CHECK(fg.colg.d == g_last.p.col_groups && fg.hkv.d == sh.hkv && fg.lq.d == sh.lq, "divisors");
        std::vector<int> seen((size_t)G * S, 0), xcd(G, -1);
        std::vector<int> lo((size_t)G * S), hi((size_t)G * S);
        for (int i = 0; i < (int)g_last.grid; ++i) {
            const int j = sdpa_dev::fast_div(i, fg.nx), x = i - j * nx;
            const int js = sdpa_dev::fast_div(j, fg.splits), split = j - js * S;
            const int grp = x + nx * js;
            CHECK(grp >= 0 && grp < G && split >= 0 && split < S, "workgroup %d -> group %d split %d", i, grp,
                  split);
            if (grp < 0 || grp >= G) continue;
            ++seen[(size_t)grp * S + split];
            if (xcd[grp] < 0) xcd[grp] = i % nx;
            CHECK(xcd[grp] == i % nx, "group %d on XCDs %d and %d", grp, xcd[grp], i % nx);
            lo[(size_t)grp * S + split] = sdpa_dev::fast_div(split * fg.nblk, fg.splits);
            hi[(size_t)grp * S + split] = sdpa_dev::fast_div((split + 1) * fg.nblk, fg.splits);
        }
        for (int g = 0; g < G; ++g)
            for (int s2 = 0; s2 < S; ++s2) {
                const size_t k = (size_t)g * S + s2;
                CHECK(seen[k] == 1, "group %d split %d seen %d times", g, s2, seen[k]);
                CHECK(lo[k] == (s2 ? hi[k - 1] : 0) && lo[k] < hi[k], "split %d keys [%d, %d)", s2, lo[k], hi[k]);
            }
        CHECK(hi[(size_t)S - 1] == fg.nblk, "last split ends at %d of %d", hi[(size_t)S - 1], fg.nblk);
    }
}

void check_overlaps() {
    const size_t ws = sdpa_workspace_size(1, 1, 4096, 32, 8, 256, SDPA_BF16);
    CHECK(ws > 0, "c2 workspace");
    // a workspace that overlaps q, k, v or the mask is refused
    for (uintptr_t w : {kQ, kK, kV, kM})
        CHECK(call(1, 1, 4096, 32, 8, 256, 256, SDPA_BF16, SDPA_MASK_ADDITIVE, 0, ws, w) == SDPA_EINVAL,
              "workspace at %#lx accepted", (unsigned long)w);
    // an output that overlaps the mask
    const sdpa_strides qs = bhld(8, 100, 64), os = bhld(8, 100, 64);
    const int st = sdpa_forward((const void*)kQ, qs, (const void*)kK, qs, (const void*)kV, qs, (void*)kM, os, 1, 100,
                                100, 8, 8, 64, SDPA_BF16, 0.125f, SDPA_MASK_BOOLEAN, (const void*)(kM + 64),
                                sdpa_strides{0, 0, 100, 1}, SDPA_U8, nullptr, 0, nullptr);
    CHECK(st == SDPA_EINVAL, "out over the mask: %d", st);
    // a workspace over the rotary tables (read by the kernels that write the workspace)
    const sdpa_strides q2 = bhld(32, 1, 256), k2 = bhld(8, 4096, 256);
    const sdpa_rope_table tab{64, (const float*)(kW + 4096), (const float*)(kM + (1u << 20)), 8192};
    const int st2 = sdpa_forward_ex((const void*)kQ, q2, (const void*)kK, k2, (const void*)kV, k2, (void*)kO, q2, 1, 1,
                                    4096, 32, 8, 256, 256, SDPA_BF16, 0.0625f, SDPA_MASK_NONE, nullptr,
                                    sdpa_strides{0, 0, 0, 0}, SDPA_BF16, 0, &tab, 4095, (void*)kW, ws, nullptr);
    CHECK(st2 == SDPA_EINVAL, "workspace over the rope tables: %d", st2);
    const sdpa_rope_table tab_ok{64, (const float*)(kM + (2u << 20)), (const float*)(kM + (1u << 20)), 8192};
    const int st3 = sdpa_forward_ex((const void*)kQ, q2, (const void*)kK, k2, (const void*)kV, k2, (void*)kO, q2, 1, 1,
                                    4096, 32, 8, 256, 256, SDPA_BF16, 0.0625f, SDPA_MASK_NONE, nullptr,
                                    sdpa_strides{0, 0, 0, 0}, SDPA_BF16, 0, &tab_ok, 4095, (void*)kW, ws, nullptr);
    CHECK(st3 == SDPA_OK, "tables apart from the workspace: %d", st3);
}

void concurrent_queries() {
    std::vector<std::thread> th;
    std::atomic<int> bad{0};
    for (int t = 0; t < 8; ++t)
        th.emplace_back([&bad, t] {
            for (int i = 0; i < 200; ++i) {
                const size_t a = sdpa_workspace_size(1, 1, 1000 + 16 * i, 8 * (1 + t % 4), 8, 128, SDPA_BF16);
                const size_t b = sdpa_workspace_size(1, 1, 1000 + 16 * i, 8 * (1 + t % 4), 8, 128, SDPA_BF16);
                if (a != b) bad.fetch_add(1);
                char buf[256];
                sdpa_describe_route(1, 1 + i % 8, 4096, 32, 8, 256, SDPA_BF16, SDPA_MASK_CAUSAL, buf, sizeof buf);
            }
        });
    for (auto& x : th) x.join();
    CHECK(bad.load() == 0, "workspace size changed between identical queries");
}

}  // namespace

int main() {
    sweep_workspace_bound();
    check_fused_geometry();
    check_fast_div();
    check_fused_mapping();
    check_overlaps();
    concurrent_queries();
    std::printf("host harness: %ld checks, %d failed\n", g_checks, g_fail);
    return g_fail ? 1 : 0;
}
