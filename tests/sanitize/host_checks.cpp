// Host paths of the library under AddressSanitizer and UndefinedBehaviorSanitizer:
// the argument checks of every entry point (each call below is rejected before
// anything reaches the GPU), the host repack and its inverse, the launch
// planners, the workspace-size queries, the KV-cache host packing and the
// tree-MTP planner.  Built together with the library's sources into one
// executable (host code instrumented, GPU code not); exits 0 when every check
// holds, and a sanitizer report aborts it.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "sk_attention.h"
#include "sk_mtp.h"
#include "sk_repack.h"
#include "sk_repack_test.h"

static int g_fails = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++g_fails;                                                        \
        }                                                                     \
    } while (0)

// 16-byte aligned and never dereferenced: every call that receives it is rejected first.
static void* const FAKE = reinterpret_cast<void*>(uintptr_t(0x7F0000000000ull));
static char* fake(size_t off) { return static_cast<char*>(FAKE) + off; }

static size_t weight_bytes(int fmt, int n, int k, int g) {
    const int bits = fmt == SK_W6_SYM ? 6 : 4;
    return (size_t)n * k * bits / 8 + (size_t)n * (k / g) * 4;
}

static sk_weight make_w(int fmt, int n, int k, int g, int layout, void* data) {
    sk_weight w;
    std::memset(&w, 0, sizeof(w));
    w.n = n;
    w.k = k;
    w.group = g;
    w.format = fmt;
    w.layout = layout;
    w.data = data;
    w.bytes = weight_bytes(fmt, n, k, g);
    w.codebook = fmt == SK_W4_CODEBOOK ? static_cast<const float*>(FAKE) : nullptr;
    return w;
}

static void check_gemm_rejections() {
    sk_weight w = make_w(SK_W4_SYM, 64, 256, 32, SK_LAYOUT_STREAM, FAKE);
    void* y = FAKE;
    CHECK(sk_gemm_w4a8(nullptr, FAKE, SK_F32, 1, static_cast<float*>(y), nullptr, 0, nullptr) == SK_ERR_NULL);
    CHECK(sk_gemm_w4a8(&w, nullptr, SK_F32, 1, static_cast<float*>(y), nullptr, 0, nullptr) == SK_ERR_NULL);
    CHECK(sk_gemm_w4a8(&w, FAKE, SK_F32, 0, static_cast<float*>(y), nullptr, 0, nullptr) == SK_ERR_SHAPE);
    CHECK(sk_gemm_w4a8(&w, FAKE, SK_F32, 9, static_cast<float*>(y), nullptr, 0, nullptr) == SK_ERR_SHAPE);
    CHECK(sk_gemm_w4a8(&w, FAKE, 7, 1, static_cast<float*>(y), nullptr, 0, nullptr) == SK_ERR_FORMAT);
    CHECK(sk_gemm_w4a8(&w, fake(4), SK_F32, 1, static_cast<float*>(y), nullptr, 0, nullptr) == SK_ERR_ALIGN);
    sk_weight canon = make_w(SK_W4_SYM, 64, 256, 32, SK_LAYOUT_CANONICAL, FAKE);
    CHECK(sk_gemm_w4a8(&canon, FAKE, SK_F32, 1, static_cast<float*>(y), nullptr, 0, nullptr) == SK_ERR_LAYOUT);
    sk_weight w6 = make_w(SK_W6_SYM, 64, 256, 64, SK_LAYOUT_STREAM, FAKE);
    CHECK(sk_gemm_w4a8(&w6, FAKE, SK_F32, 1, static_cast<float*>(y), nullptr, 0, nullptr) == SK_ERR_FORMAT);
    CHECK(sk_gemm_w6a8(&w, FAKE, SK_F32, 1, static_cast<float*>(y), nullptr, 0, nullptr) == SK_ERR_FORMAT);
    sk_weight bad = w;
    bad.bytes += 1;
    CHECK(sk_gemm_w4a8(&bad, FAKE, SK_F32, 1, static_cast<float*>(y), nullptr, 0, nullptr) == SK_ERR_SHAPE);
    sk_weight wide = make_w(SK_W4_SYM, 64, 20480, 32, SK_LAYOUT_STREAM, FAKE);
    CHECK(sk_gemm_w4a8(&wide, FAKE, SK_F32, 1, static_cast<float*>(y), nullptr, 0, nullptr) == SK_ERR_UNSUPPORTED);
    // a K-split call without its workspace
    sk_weight down = make_w(SK_W4_SYM, 5120, 17408, 32, SK_LAYOUT_STREAM, FAKE);
    CHECK(sk_gemm_w4a8(&down, FAKE, SK_BF16, 8, static_cast<float*>(y), nullptr, 0, nullptr) == SK_ERR_WORKSPACE);
    CHECK(sk_gemm_w4a8_noalloc(&canon, FAKE, SK_F32, 1, static_cast<float*>(y), nullptr) == SK_ERR_LAYOUT);
    const float* gam = static_cast<const float*>(FAKE);
    CHECK(sk_gemm_fused_rmsnorm(&w, FAKE, SK_F32, nullptr, 1e-6f, 1, static_cast<float*>(y), nullptr, 0, nullptr) ==
          SK_ERR_NULL);
    CHECK(sk_gemm_fused_rmsnorm(&w, FAKE, SK_F32, reinterpret_cast<const float*>(fake(8)), 1e-6f, 1,
                                static_cast<float*>(y), nullptr, 0, nullptr) == SK_ERR_ALIGN);
    CHECK(sk_gemm_fused_swiglu(&w, FAKE, nullptr, 256, SK_F32, 1, static_cast<float*>(y), nullptr, 0, nullptr) ==
          SK_ERR_NULL);
    CHECK(sk_gemm_fused_swiglu(&w, FAKE, FAKE, 128, SK_F32, 1, static_cast<float*>(y), nullptr, 0, nullptr) ==
          SK_ERR_SHAPE);
    CHECK(sk_gemm_fused_swiglu(&w, FAKE, FAKE, 260, SK_BF16, 1, static_cast<float*>(y), nullptr, 0, nullptr) ==
          SK_ERR_ALIGN);
    (void)gam;
    const int32_t* ids = static_cast<const int32_t*>(FAKE);
    CHECK(sk_gemm_experts(&w, 16, nullptr, 1, FAKE, SK_F32, 1, static_cast<float*>(y), nullptr, 0, nullptr) ==
          SK_ERR_NULL);
    CHECK(sk_gemm_experts(&w, 10, ids, 1, FAKE, SK_F32, 1, static_cast<float*>(y), nullptr, 0, nullptr) ==
          SK_ERR_SHAPE);
    CHECK(sk_quantize_rows(nullptr, SK_F32, 1, 256, static_cast<int8_t*>(FAKE), static_cast<float*>(FAKE),
                           nullptr) == SK_ERR_NULL);
    CHECK(sk_quantize_rows(FAKE, SK_F32, 1, 24, static_cast<int8_t*>(FAKE), static_cast<float*>(FAKE), nullptr) ==
          SK_ERR_SHAPE);
    CHECK(sk_prologue_rmsnorm(FAKE, SK_F32, gam, 1e-6f, 9, 256, static_cast<float*>(FAKE), nullptr) == SK_ERR_SHAPE);
    CHECK(sk_prologue_swiglu(FAKE, FAKE, 255, SK_F32, 1, 256, static_cast<float*>(FAKE), nullptr) == SK_ERR_SHAPE);
    CHECK(sk_gemm_w4a8_canonical(&w, FAKE, SK_F32, 1, static_cast<float*>(y), nullptr, 0, nullptr) == SK_ERR_LAYOUT);
    CHECK(sk_gemm_w4a8_canonical_q(&canon, static_cast<const int8_t*>(FAKE), nullptr, 1, static_cast<float*>(y),
                                   nullptr, 0, nullptr) == SK_ERR_NULL);
    CHECK(sk_debug_gemm(&w, 3, FAKE, nullptr, 0, SK_F32, nullptr, 0.0f, 1, static_cast<float*>(y), nullptr, nullptr,
                        nullptr, nullptr, 0, nullptr) != SK_OK);
    sk_weight rep = make_w(SK_W4_SYM, 64, 256, 32, SK_LAYOUT_CANONICAL, fake(8));
    CHECK(sk_repack_w4a8(&rep, nullptr) == SK_ERR_ALIGN);
    CHECK(rep.layout == SK_LAYOUT_CANONICAL);
    sk_weight rep2 = make_w(SK_W4_SYM, 64, 256, 32, SK_LAYOUT_STREAM, FAKE);
    CHECK(sk_repack_w4a8(&rep2, nullptr) == SK_ERR_LAYOUT);
    CHECK(sk_unrepack_w4a8(&canon, nullptr) == SK_ERR_LAYOUT);
    for (int s = 0; s <= 9; ++s) CHECK(sk_status_string((sk_status)s) != nullptr);
    CHECK(sk_status_string((sk_status)99) != nullptr);
}

static void check_attention_rejections() {
    const uint16_t* q = static_cast<const uint16_t*>(FAKE);
    float* out = static_cast<float*>(FAKE);
    CHECK(sk_decode_attention(nullptr, 1, 32, 8, FAKE, 64, 32, 0.088f, out, nullptr, 0, nullptr) == SK_ERR_NULL);
    CHECK(sk_decode_attention(q, 9, 32, 8, FAKE, 64, 32, 0.088f, out, nullptr, 0, nullptr) == SK_ERR_SHAPE);
    CHECK(sk_decode_attention(q, 1, 30, 8, FAKE, 64, 32, 0.088f, out, nullptr, 0, nullptr) == SK_ERR_SHAPE);
    CHECK(sk_decode_attention(q, 1, 32, 8, FAKE, 64, 80, 0.088f, out, nullptr, 0, nullptr) == SK_ERR_SHAPE);
    CHECK(sk_kv_append(nullptr, 8, 64, 0, 1, q, q, nullptr) == SK_ERR_NULL);
    CHECK(sk_kv_append(FAKE, 8, 60, 0, 1, q, q, nullptr) == SK_ERR_SHAPE);
    CHECK(sk_kv_append(FAKE, 8, 64, 60, 8, q, q, nullptr) == SK_ERR_SHAPE);
    size_t bytes = 0;
    CHECK(sk_attention_workspace_size(1, 32, 8, 4096, nullptr) == SK_ERR_NULL);
    CHECK(sk_attention_workspace_size(9, 32, 8, 4096, &bytes) == SK_ERR_SHAPE);
}

// The host repack and its inverse restore every byte, for each format and
// ragged shapes, with buffers of exactly the weight's size.
static void check_host_repack(std::mt19937& rng) {
    struct Case { int fmt, n, k, g; };
    const Case cases[] = {{SK_W4_SYM, 40, 256, 32}, {SK_W4_SYM, 16, 128, 128}, {SK_W4_SYM, 5, 1024, 64},
                          {SK_W6_SYM, 17, 512, 64}, {SK_W6_SYM, 33, 256, 32}, {SK_W4_CODEBOOK, 33, 384, 16},
                          {SK_W4_CODEBOOK, 1, 128, 32}, {SK_W4_SYM, 1000, 2048, 32}};
    for (const Case& c : cases) {
        const size_t nb = weight_bytes(c.fmt, c.n, c.k, c.g);
        std::vector<uint8_t> orig(nb), buf(nb);
        for (auto& b : orig) b = (uint8_t)(rng() & 0xFF);
        buf = orig;
        sk_weight w = make_w(c.fmt, c.n, c.k, c.g, SK_LAYOUT_CANONICAL, FAKE);
        CHECK(sk_test_repack_on_host(&w, buf.data(), 0) == SK_OK);
        w.layout = SK_LAYOUT_STREAM;
        CHECK(sk_test_repack_on_host(&w, buf.data(), 1) == SK_OK);
        CHECK(buf == orig);
    }
    sk_weight w = make_w(SK_W4_SYM, 40, 256, 32, SK_LAYOUT_CANONICAL, FAKE);
    CHECK(sk_test_repack_on_host(&w, nullptr, 0) == SK_ERR_NULL);
}

// Plans over a grid of shapes, row counts, prologues and device sizes.
static void check_planners() {
    const int ns[] = {1, 15, 16, 100, 4096, 34816, 151936};
    const int ks[] = {128, 1024, 4096, 5120, 12288, 17408, 20480};
    const int gs[] = {16, 32, 64, 128};
    const int cus[] = {1, 64, 256, 304};
    int ok = 0;
    for (int fmt = 0; fmt < 3; ++fmt)
        for (int n : ns)
            for (int k : ks)
                for (int g : gs)
                    for (int m = 1; m <= 8; ++m)
                        for (int pro = 0; pro < 3; ++pro)
                            for (int cu : cus) {
                                int64_t f[15];
                                const sk_status st = sk_test_gemm_plan(n, k, g, fmt, m, pro, cu, f);
                                CHECK(st == SK_OK || st == SK_ERR_UNSUPPORTED || st == SK_ERR_SHAPE ||
                                      st == SK_ERR_FORMAT);
                                if (st == SK_OK) {
                                    ++ok;
                                    CHECK(f[0] >= 1 && f[1] >= 1 && f[2] == f[0] * f[1] && f[3] >= 1 && f[4] >= 1);
                                    CHECK(f[13] == 4 || f[13] == 5);
                                    CHECK(f[14] >= 0 && f[14] < f[4] && (f[0] > 1 || f[14] == 0));
                                }
                            }
    CHECK(ok > 1000);
    int splits = 0, bps = 0;
    for (int m = 1; m <= 8; ++m)
        for (int hkv : {1, 8, 64})
            for (int len : {1, 31, 32, 4096, 65536})
                if (len >= m) {
                    const sk_status st = sk_test_attention_plan(m, hkv * 4, hkv, len, 256, &splits, &bps);
                    CHECK(st == SK_OK || st == SK_ERR_UNSUPPORTED);
                    if (st == SK_OK) CHECK(splits >= 1 && bps >= 1);
                }
    CHECK(sk_test_set_split(33) == SK_ERR_SHAPE);
    CHECK(sk_test_set_spin_limit(-1) == SK_ERR_SHAPE);
}

static void check_kv_pack(std::mt19937& rng) {
    const int hkv = 2, len = 40, cap = 64;
    std::vector<uint16_t> k((size_t)hkv * len * 128), v(k.size());
    for (auto& x : k) x = (uint16_t)rng();
    for (auto& x : v) x = (uint16_t)rng();
    std::vector<uint8_t> out((size_t)hkv * (cap / 32) * 16384, 0xAB);
    CHECK(sk_kv_pack_host(k.data(), v.data(), hkv, len, cap, out.data()) == SK_OK);
    CHECK(sk_kv_pack_host(k.data(), v.data(), hkv, len, 48, out.data()) == SK_ERR_SHAPE);
    CHECK(sk_kv_pack_host(nullptr, v.data(), hkv, len, cap, out.data()) == SK_ERR_NULL);
}

static void check_mtp(std::mt19937& rng) {
    sk_mtp_planner* p = nullptr;
    CHECK(sk_mtp_create(1.5, 32, 1.03, &p) != SK_OK);
    CHECK(sk_mtp_create(0.95, 32, 1.03, nullptr) == SK_ERR_NULL);
    CHECK(sk_mtp_create(0.95, 32, 1.03, &p) == SK_OK && p != nullptr);
    std::uniform_int_distribution<int> rank(0, 7), levels(0, 7);
    int32_t widths[7], depth = 0;
    for (int step = 0; step < 3000; ++step) {
        int32_t r[7];
        const int nl = levels(rng);
        for (int i = 0; i < nl; ++i) r[i] = rank(rng) % (step % 3 == 0 ? 2 : 8);
        CHECK(sk_mtp_observe(p, r, nl, 1.7, 0.04, widths, &depth) == SK_OK);
        CHECK(depth >= 1 && depth <= 7);
    }
    int32_t index = -1;
    CHECK(sk_mtp_layout(p, &index, widths, &depth) == SK_OK && index >= 0 && index < 64);
    std::vector<double> counts(56);
    double vm = 0, dm = 0;
    int64_t steps = 0;
    CHECK(sk_mtp_state(p, counts.data(), &vm, &dm, &steps) == SK_OK && steps == 3000);
    for (int b = 0; b < 64; ++b) {
        CHECK(sk_mtp_layout_of(b, widths, &depth) == SK_OK);
        int sum = 0;
        for (int i = 0; i < depth; ++i) sum += widths[i];
        CHECK(sum == 7);
        int32_t r[7], acc = -1, obs = -1;
        for (int i = 0; i < depth; ++i) r[i] = rank(rng);
        CHECK(sk_mtp_accept(widths, depth, r, &acc, &obs) == SK_OK && acc >= 0 && obs >= 1);
        double pr[56];
        for (double& x : pr) x = 1.0 / 8.0;
        double e = 0;
        CHECK(sk_mtp_expected_tokens(pr, widths, depth, &e) == SK_OK && e >= 1.0);
    }
    CHECK(sk_mtp_layout_of(64, widths, &depth) != SK_OK);
    int32_t bad[1] = {9};
    CHECK(sk_mtp_observe(p, bad, 1, 1.0, 1.0, nullptr, nullptr) != SK_OK);
    sk_mtp_destroy(p);
    sk_mtp_destroy(nullptr);
}

int main() {
    std::mt19937 rng(20261202u);
    check_gemm_rejections();
    check_attention_rejections();
    check_host_repack(rng);
    check_planners();
    check_kv_pack(rng);
    check_mtp(rng);
    if (g_fails) {
        std::fprintf(stderr, "%d checks failed\n", g_fails);
        return 1;
    }
    std::printf("host checks passed\n");
    return 0;
}
