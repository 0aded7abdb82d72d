// Host-only driver of libmbq's C ABI for the sanitizer build: packing and
// unpacking in every format, the size queries, and every argument check
// that returns before any device work.  Device pointers here are fake
// addresses the library only inspects (alignment, overlap), never reads.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "mbq.h"

static int failures = 0;
#define CHECK(cond)                                                       \
    do {                                                                  \
        if (!(cond)) {                                                    \
            std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);   \
            failures++;                                                   \
        }                                                                 \
    } while (0)

static const uintptr_t BASE = 0x7F0000000000ull;
static void* fake(uintptr_t off) { return (void*)(BASE + off); }

static void pack_round_trips() {
    std::mt19937_64 rng(7);
    const int shapes[][2] = {{1, 256}, {7, 512}, {3, 4096}, {2, 12288}};
    for (int fmt = 0; fmt <= 3; fmt++)
        for (auto& sh : shapes) {
            const int64_t N = sh[0], K = sh[1];
            size_t sz[4];
            CHECK(mbq_plane_sizes(fmt, N, K, sz) == MBQ_OK);
            double bpw = 0;
            int bk = 0;
            CHECK(mbq_format_info(fmt, &bpw, &bk) == MBQ_OK);
            CHECK(sz[0] + sz[1] + sz[2] + sz[3] == (size_t)(N * K * bpw / 8));
            const int bits = fmt == 1 ? 4 : fmt == 2 ? 6 : 2;
            std::vector<uint8_t> codes(fmt == 0 ? 2 * N * K : N * K);
            for (auto& c : codes) c = (uint8_t)(fmt == 0 ? rng() : rng() % (1u << bits));
            std::vector<uint16_t> sc16(N * K / 32), su(N * K / 256);
            std::vector<int8_t> sc8(N * K / 16);
            for (auto& v : sc16) v = (uint16_t)(0x2000 + rng() % 0x1000);
            for (auto& v : su) v = (uint16_t)(0x1800 + rng() % 0x800);
            for (auto& v : sc8) v = (int8_t)rng();
            const void* scales = fmt == 0 ? nullptr : fmt == 2 ? (const void*)sc8.data() : (const void*)sc16.data();
            const void* supers = fmt == 2 ? su.data() : nullptr;
            std::vector<std::vector<uint8_t>> planes(4);
            void* pp[4];
            for (int i = 0; i < 4; i++) {
                planes[i].resize(sz[i] + 1);
                pp[i] = sz[i] ? planes[i].data() : nullptr;
            }
            CHECK(mbq_pack(fmt, N, K, codes.data(), scales, supers, pp) == MBQ_OK);
            std::vector<uint8_t> c2(codes.size());
            std::vector<uint8_t> s2(sc16.size() * 2 + sc8.size() + 16), u2(su.size() * 2 + 16);
            const void* cp[4] = {pp[0], pp[1], pp[2], pp[3]};
            CHECK(mbq_unpack(fmt, N, K, cp, c2.data(), fmt ? s2.data() : nullptr, fmt == 2 ? u2.data() : nullptr) == MBQ_OK);
            CHECK(c2 == codes);
            if (fmt == 1 || fmt == 3) CHECK(std::memcmp(s2.data(), sc16.data(), sc16.size() * 2) == 0);
            if (fmt == 2) {
                CHECK(std::memcmp(s2.data(), sc8.data(), sc8.size()) == 0);
                CHECK(std::memcmp(u2.data(), su.data(), su.size() * 2) == 0);
            }
            if (fmt != 0) {   // a code one past the format's range is rejected
                codes[codes.size() / 2] = (uint8_t)(1u << bits);
                CHECK(mbq_pack(fmt, N, K, codes.data(), scales, supers, pp) == MBQ_EINVAL);
            }
        }
}

static mbq_qweight qw(int fmt, int64_t N, int64_t K) {
    mbq_qweight w;
    std::memset(&w, 0, sizeof w);
    w.fmt = fmt;
    w.N = N;
    w.K = K;
    w.codes = fake(0);
    w.codes_hi = fmt == 2 ? fake(0x100000) : nullptr;
    w.scales = fmt ? fake(0x200000) : nullptr;
    w.super_scales = fmt == 2 ? fake(0x300000) : nullptr;
    return w;
}

static void argument_checks() {
    mbq_qweight w = qw(1, 64, 256);
    float* x = (float*)fake(0x400000);
    float* y = (float*)fake(0x800000);
    CHECK(mbq_gemv_q(nullptr, x, 1, 256, y, 64, 0, nullptr) == MBQ_EINVAL);
    mbq_qweight bad = qw(7, 64, 256);
    CHECK(mbq_gemv_q(&bad, x, 1, 256, y, 64, 0, nullptr) == MBQ_EINVAL);
    bad = qw(1, 64, 48);
    CHECK(mbq_gemv_q(&bad, x, 1, 48, y, 64, 0, nullptr) == MBQ_EINVAL);
    CHECK(mbq_gemv_q(&w, x, -1, 256, y, 64, 0, nullptr) == MBQ_EINVAL);
    CHECK(mbq_gemv_q(&w, x, 2, 100, y, 64, 0, nullptr) == MBQ_EINVAL);
    CHECK(mbq_gemv_q(&w, x, 1, 256, y, 64, 2, nullptr) == MBQ_EINVAL);
    CHECK(mbq_gemv_q(&w, x, 0, 256, y, 64, 0, nullptr) == MBQ_OK);
    CHECK(mbq_gemv_q(&w, (float*)fake(0x400004), 1, 256, y, 64, 0, nullptr) == MBQ_EALIGN);
    CHECK(mbq_gemv_q(&w, x, 1, 256, (float*)fake(0x100), 64, 0, nullptr) == MBQ_EINVAL);   // y over the codes
    size_t b = 0;
    CHECK(mbq_xq_bytes(1, 16, 4096, &b) == MBQ_OK && b > 0);
    CHECK(mbq_xq_bytes(1, 16, 100, &b) == MBQ_EINVAL);
    CHECK(mbq_xq_bytes(9, 16, 4096, &b) == MBQ_EINVAL);
    CHECK(mbq_stage_x(1, x, 2, 100, 4096, fake(0xA00000), nullptr) == MBQ_EINVAL);
    {
        // the K-split product: the workspace size is host arithmetic, the
        // workspace is checked before any launch
        mbq_qweight d = qw(1, 4096, 12288);
        CHECK(mbq_gemv_xq_workspace_bytes(&d, 16, &b) == MBQ_OK && b == 256 + 4ull * 16 * 4096 * 4);
        CHECK(mbq_gemv_xq_workspace_bytes(&d, 3, &b) == MBQ_OK && b == 0);
        CHECK(mbq_gemv_xq_workspace_bytes(nullptr, 16, &b) == MBQ_EINVAL);
        const size_t need = 256 + 4ull * 16 * 4096 * 4;
        void* xq = fake(0x4000000);
        float* yq = (float*)fake(0x5000000);
        CHECK(mbq_gemv_xq_ws(&d, xq, 16, yq, 4096, 0, nullptr, need, nullptr) == MBQ_EINVAL);
        CHECK(mbq_gemv_xq_ws(&d, xq, 16, yq, 4096, 0, fake(0x6000000), need - 1, nullptr) == MBQ_EINVAL);
        CHECK(mbq_gemv_xq_ws(&d, xq, 16, yq, 4096, 0, fake(0x6000010), need, nullptr) == MBQ_EALIGN);
        CHECK(mbq_gemv_xq_ws(&d, xq, 16, yq, 4096, 0, fake(0x5000100), need, nullptr) == MBQ_EINVAL);
        CHECK(mbq_gemv_xq_ws(&d, xq, 16, yq, 4096, 0, fake(0), need, nullptr) == MBQ_EINVAL);
    }
    CHECK(mbq_rmsnorm(x, (float*)fake(0x500000), -1.0f, 1, 4096, y, nullptr) == MBQ_EINVAL);
    CHECK(mbq_layernorm(x, nullptr, nullptr, 1e-5f, 1, 2048, y, nullptr) == MBQ_EINVAL);
    void* pl[4] = {fake(0x1000000), nullptr, fake(0x3000000), nullptr};
    CHECK(mbq_quantize(9, x, 4, 256, 256, pl, nullptr) == MBQ_EINVAL);
    CHECK(mbq_quantize(1, x, 4, 48, 48, pl, nullptr) == MBQ_EINVAL);
    CHECK(mbq_quantize(1, x, 0, 256, 256, pl, nullptr) == MBQ_OK);
    CHECK(mbq_quantize(1, (float*)fake(0x400004), 4, 256, 256, pl, nullptr) == MBQ_EALIGN);
    CHECK(mbq_attention_workspace_bytes(512, 32, 8, 128, &b) == MBQ_OK && b > 0);
    CHECK(mbq_attention_workspace_bytes(0, 32, 8, 128, &b) == MBQ_EINVAL);
    CHECK(mbq_attention_workspace_bytes(512, 24, 8, 128, &b) == MBQ_EUNSUPPORTED);
    CHECK(mbq_attention_decode(x, fake(0x1000000), fake(0x2000000), 512, 1028, 32, 8, 128, y,
                               fake(0x4000000), 1 << 24, nullptr) == MBQ_EALIGN);
    CHECK(mbq_attention_decode(x, fake(0x1000000), fake(0x2000000), 512, 1024, 32, 8, 128, y,
                               fake(0x4000000), 16, nullptr) == MBQ_EINVAL);
    // the fused append: T counts cached positions, the workspace covers T + 1
    CHECK(mbq_attention_decode_append(x, (float*)fake(0x10000), (float*)fake(0x20000), fake(0x1000000),
                                      fake(0x2000000), -1, 1024, 32, 8, 128, y, fake(0x4000000), 1 << 24,
                                      nullptr) == MBQ_EINVAL);
    CHECK(mbq_attention_decode_append(x, (float*)fake(0x10004), (float*)fake(0x20000), fake(0x1000000),
                                      fake(0x2000000), 511, 1024, 32, 8, 128, y, fake(0x4000000), 1 << 24,
                                      nullptr) == MBQ_EALIGN);
    CHECK(mbq_attention_decode_append(x, (float*)fake(0x10000), (float*)fake(0x20000), fake(0x1000000),
                                      fake(0x2000000), 511, 1024, 32, 8, 128, y, fake(0x4000000),
                                      32 * 16 * 132 * 4 - 4, nullptr) == MBQ_EINVAL);
    CHECK(mbq_attention_decode_append(x, (float*)fake(0x1000000 + 511 * 2048), (float*)fake(0x20000),
                                      fake(0x1000000), fake(0x2000000), 511, 1024, 32, 8, 128, y,
                                      fake(0x4000000), 1 << 24, nullptr) == MBQ_EINVAL);
    mbq_decode_model m;
    std::memset(&m, 0, sizeof m);
    CHECK(mbq_decode_workspace_bytes(nullptr, &b) == MBQ_EINVAL);
    m.n_layers = -1;
    CHECK(mbq_decode_workspace_bytes(&m, &b) == MBQ_EINVAL);
    // the step with attention over the caches: size queries and argument
    // checks on a model without layers (nothing reaches a launch)
    m.n_layers = 0;
    m.eps = 1e-6f;
    m.d = 4096;
    m.dq = 4096;
    m.dkv = 1024;
    m.gamma_f = (const float*)fake(0x700000);
    CHECK(mbq_decode_kv_workspace_bytes(&m, 511, &b) == MBQ_OK &&
          b == (4096 + 2048) * 4 + 4096 * 4 + 32 * 16 * 132 * 4);
    CHECK(mbq_decode_kv_workspace_bytes(&m, -1, &b) == MBQ_EINVAL);
    CHECK(mbq_decode_kv_workspace_bytes(nullptr, 5, &b) == MBQ_EINVAL);
    m.dkv = 1000;
    CHECK(mbq_decode_kv_workspace_bytes(&m, 5, &b) == MBQ_EUNSUPPORTED);
    m.dkv = 1024;
    const size_t kvb = b;
    float* hh = (float*)fake(0x8000000);
    CHECK(mbq_decode_step_kv(&m, hh, nullptr, nullptr, nullptr, -1, 1024, fake(0x9000000), 1 << 24,
                             nullptr) == MBQ_EINVAL);
    CHECK(mbq_decode_step_kv(&m, (float*)fake(0x8000004), nullptr, nullptr, nullptr, 511, 1024,
                             fake(0x9000000), 1 << 24, nullptr) == MBQ_EALIGN);
    CHECK(mbq_decode_step_kv(&m, hh, nullptr, nullptr, nullptr, 511, 1024, fake(0x9000000), kvb - 1,
                             nullptr) == MBQ_EINVAL);
    CHECK(mbq_decode_step_kv(&m, hh, nullptr, nullptr, nullptr, 511, 1020, fake(0x9000000), 1 << 24,
                             nullptr) == MBQ_EINVAL);
    CHECK(mbq_decode_step_kv(&m, hh, nullptr, nullptr, nullptr, 511, 1028, fake(0x9000000), 1 << 24,
                             nullptr) == MBQ_EALIGN);
    std::memset(&m, 0, sizeof m);
    CHECK(mbq_probe_mixed(nullptr, 1024, nullptr, 1024, 5, 256, y, nullptr) == MBQ_EINVAL);
    CHECK(mbq_probe_read(fake(0), 15, y, nullptr) == MBQ_EALIGN);
    CHECK(std::strlen(mbq_status_str(MBQ_EINVAL)) > 0);
    CHECK(std::strlen(mbq_last_error()) > 0);
    CHECK(mbq_version() == 1);
}

int main() {
    pack_round_trips();
    argument_checks();
    std::printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
