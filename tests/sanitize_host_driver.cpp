// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py): the planner
// on random and extreme shapes, and every validation path of every entry
// point.  The kernel launches are replaced by stubs
// (sanitize_host_stubs.cpp), so nothing here touches a device.
#include <cinttypes>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <vector>

#include "fd.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint32_t rnd() {
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(g_state >> 33);
}

int g_failures = 0;
#define CHECK(c)                                                                   \
    do {                                                                           \
        if (!(c)) {                                                                \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++g_failures;                                                          \
        }                                                                          \
    } while (0)

void* fake(int i) { return reinterpret_cast<void*>((uintptr_t)0x100000 * (uintptr_t)(i + 1)); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

void random_plans() {
    for (int it = 0; it < 4000; ++it) {
        fd_dims d;
        d.batch = (int32_t)(rnd() % 40);
        d.num_kv_heads = 1 + (int32_t)(rnd() % 8);
        d.num_q_heads = d.num_kv_heads * (1 + (int32_t)(rnd() % 8));
        d.head_dim = (rnd() & 1) ? 64 : 128;
        d.q_len = (rnd() % 4 == 0) ? 1 + (int32_t)(rnd() % 600) : 1;
        d.max_cache_len = (int32_t)(rnd() % 300000);
        d.dtype = (int32_t)(rnd() % 2);
        std::vector<int32_t> lens(d.batch + 1);
        for (int b = 0; b < d.batch; ++b) lens[b] = (int32_t)(rnd() % ((uint32_t)d.max_cache_len + 1));
        const int32_t ns = (rnd() % 3 == 0) ? (int32_t)(rnd() % 257) : 0;
        const int32_t cus = 1 + (int32_t)(rnd() % 512);
        fd_plan p;
        std::vector<int32_t> splits(d.batch + 1, -7);
        const fd_status st = fd_plan_splits(&d, lens.data(), ns, cus, &p, splits.data());
        CHECK(st == FD_OK);
        if (st != FD_OK) continue;
        CHECK(p.max_splits >= 1 && p.max_splits <= FD_MAX_SPLITS);
        int64_t units = 0, max_len = 0;
        for (int b = 0; b < d.batch; ++b) {
            max_len = std::max<int64_t>(max_len, lens[b]);
            const int64_t L = lens[b];
            const int64_t T = p.tile_len > 0 ? p.tile_len : (ns > 0 ? std::max<int64_t>(1, ceil_div(L, ns)) : 1);
            int64_t S = L == 0 ? 0 : ceil_div(L, T);
            if (S > p.max_splits) S = p.max_splits;
            CHECK(splits[b] == S);
            units += S;
        }
        CHECK(splits[d.batch] == -7);  // nothing written past the batch
        CHECK(units >= 0);
        CHECK(p.workspace_bytes == (p.max_splits > 1 ? fd_workspace_bytes(&d, p.max_splits) : 0));
        // multiples of 64 keys, at least 256 unless the longest sequence is shorter
        if (p.tile_len > 0) CHECK(p.tile_len % 64 == 0 && (p.tile_len >= 256 || p.tile_len >= max_len));
    }
}

void extreme_plans() {
    // The largest shapes the ABI accepts: planner arithmetic must not
    // overflow.
    fd_dims d{65535, 65535, 1, 128, 1, INT32_MAX, FD_BF16};
    std::vector<int32_t> lens(65535, INT32_MAX);
    fd_plan p;
    fd_status st = fd_plan_splits(&d, lens.data(), 0, 256, &p, nullptr);
    CHECK(st == FD_OK || st == FD_ERR_UNSUPPORTED);
    if (st == FD_OK) CHECK(p.max_splits <= FD_MAX_SPLITS && (int64_t)p.tile_len * p.max_splits >= INT32_MAX);
    st = fd_plan_splits(&d, lens.data(), FD_MAX_SPLITS, 1, &p, nullptr);
    CHECK(st == FD_OK || st == FD_ERR_UNSUPPORTED);
    d = fd_dims{1, 64, 8, 128, 70000, 80000, FD_BF16};  // long chunk: many row blocks
    int32_t L = 80000;
    st = fd_plan_splits(&d, &L, 0, 256, &p, nullptr);
    CHECK(st == FD_OK || st == FD_ERR_UNSUPPORTED);
    (void)fd_workspace_bytes(&d, FD_MAX_SPLITS);
    d = fd_dims{65535, 1024, 1, 64, 65535, 16, FD_F32};  // rows above INT32_MAX
    CHECK(fd_plan_splits(&d, lens.data(), 0, 256, &p, nullptr) == FD_ERR_UNSUPPORTED);
    CHECK(std::strlen(fd_last_error()) > 0);
    CHECK(fd_workspace_bytes(&d, 4) == 0);
}

void validation_paths() {
    const fd_dims good{2, 32, 8, 128, 1, 64, FD_BF16};
    const int32_t lens[2] = {64, 3};
    fd_plan p;
    CHECK(fd_plan_splits(nullptr, lens, 0, 256, &p, nullptr) == FD_ERR_INVALID);
    CHECK(fd_plan_splits(&good, nullptr, 0, 256, &p, nullptr) == FD_ERR_INVALID);
    CHECK(fd_plan_splits(&good, lens, 0, 256, nullptr, nullptr) == FD_ERR_INVALID);
    CHECK(fd_plan_splits(&good, lens, -1, 256, &p, nullptr) == FD_ERR_INVALID);
    CHECK(fd_plan_splits(&good, lens, 0, -3, &p, nullptr) == FD_ERR_INVALID);
    const int32_t bad_lens[2] = {65, 3};
    CHECK(fd_plan_splits(&good, bad_lens, 0, 256, &p, nullptr) == FD_ERR_INVALID);
    const fd_dims bads[] = {
        {-1, 32, 8, 128, 1, 64, FD_BF16}, {1, 0, 8, 128, 1, 64, FD_BF16}, {1, 12, 8, 128, 1, 64, FD_BF16},
        {1, 32, 8, 96, 1, 64, FD_BF16},   {1, 32, 8, 128, 0, 64, FD_BF16}, {1, 32, 8, 128, 1, -5, FD_BF16},
        {1, 32, 8, 128, 1, 64, 7},        {70000, 32, 8, 128, 1, 64, FD_BF16},
    };
    for (const fd_dims& d : bads) {
        CHECK(fd_plan_splits(&d, lens, 0, 256, &p, nullptr) < 0);
        CHECK(fd_decode_attention(&d, fake(0), fake(1), fake(2), (const int32_t*)fake(3), 0.1f, 0, nullptr,
                                  nullptr, 0, fake(4), (float*)fake(5), nullptr) < 0);
        CHECK(fd_workspace_bytes(&d, 4) == 0);
    }
    // pointers, alignment, workspace
    const int32_t* dl = (const int32_t*)fake(3);
    CHECK(fd_decode_attention(&good, nullptr, fake(1), fake(2), dl, 0.1f, 0, nullptr, nullptr, 0, fake(4),
                              nullptr, nullptr) == FD_ERR_INVALID);
    CHECK(fd_decode_attention(&good, (char*)fake(0) + 8, fake(1), fake(2), dl, 0.1f, 0, nullptr, nullptr, 0,
                              fake(4), nullptr, nullptr) == FD_ERR_INVALID);
    CHECK(fd_decode_attention(&good, fake(0), fake(1), fake(2), dl, 0.1f, 4, nullptr, nullptr, 0, fake(4),
                              nullptr, nullptr) == FD_ERR_WORKSPACE);
    CHECK(fd_decode_attention(&good, fake(0), fake(1), fake(2), dl, 0.1f, 300, nullptr, nullptr, 0, fake(4),
                              nullptr, nullptr) == FD_ERR_INVALID);
    CHECK(fd_decode_partials(&good, fake(0), fake(1), fake(2), dl, 0.1f, 0, nullptr, (float*)fake(4),
                             (float*)fake(5), (float*)fake(6), nullptr) == FD_ERR_INVALID);
    CHECK(fd_combine_splits(1, 32, 1, 128, 0, (float*)fake(0), (float*)fake(1), nullptr, FD_BF16, fake(2), nullptr,
                            nullptr) == FD_ERR_INVALID);
    CHECK(fd_combine_splits(1, 32, 1, 100, 4, (float*)fake(0), (float*)fake(1), nullptr, FD_BF16, fake(2), nullptr,
                            nullptr) == FD_ERR_UNSUPPORTED);
    // paged and fp8 descriptions
    fd_kv_pages pg{(const int32_t*)fake(7), 4, 16, 10, FD_PAGES_NHD};
    CHECK(fd_decode_attention_paged(&good, fake(0), fake(1), fake(2), nullptr, dl, 0.1f, 0, nullptr, nullptr, 0,
                                    fake(4), nullptr, nullptr) == FD_ERR_INVALID);
    fd_kv_pages bad = pg;
    bad.page_size = 24;
    CHECK(fd_decode_attention_paged(&good, fake(0), fake(1), fake(2), &bad, dl, 0.1f, 0, nullptr, nullptr, 0,
                                    fake(4), nullptr, nullptr) == FD_ERR_UNSUPPORTED);
    bad = pg;
    bad.max_pages_per_seq = 3;
    CHECK(fd_decode_attention_paged(&good, fake(0), fake(1), fake(2), &bad, dl, 0.1f, 0, nullptr, nullptr, 0,
                                    fake(4), nullptr, nullptr) == FD_ERR_INVALID);
    bad = pg;
    bad.num_pages = INT32_MAX;  // pool too large for element offsets
    (void)fd_decode_attention_paged(&good, fake(0), fake(1), fake(2), &bad, dl, 0.1f, 0, nullptr, nullptr, 0,
                                    fake(4), nullptr, nullptr);
    CHECK(fd_decode_attention_fp8(&good, fake(0), fake(1), fake(2), nullptr, NAN, 1.f, dl, 0.1f, 0, nullptr,
                                  nullptr, 0, fake(4), nullptr, nullptr) == FD_ERR_INVALID);
    const fd_dims f32q{1, 32, 8, 128, 9, 64, FD_F32};
    CHECK(fd_decode_attention_fp8(&f32q, fake(0), fake(1), fake(2), nullptr, 1.f, 1.f, dl, 0.1f, 0, nullptr,
                                  nullptr, 0, fake(4), nullptr, nullptr) == FD_ERR_UNSUPPORTED);
    // Calls that pass validation reach the (stubbed) launch and report a
    // device error, with the message recorded.
    CHECK(fd_decode_attention(&good, fake(0), fake(1), fake(2), dl, 0.1f, 0, nullptr, nullptr, 0, fake(4),
                              nullptr, nullptr) == FD_ERR_DEVICE);
    CHECK(std::strstr(fd_last_error(), "launch") != nullptr);
    CHECK(fd_decode_attention_paged(&good, fake(0), fake(1), fake(2), &pg, dl, 0.1f, 0, nullptr, nullptr, 0,
                                    fake(4), nullptr, nullptr) == FD_ERR_DEVICE);
    CHECK(fd_decode_attention_fp8(&good, fake(0), fake(1), fake(2), &pg, 0.5f, 2.f, dl, 0.1f, 3, nullptr, fake(6),
                                  1 << 20, fake(4), nullptr, nullptr) == FD_ERR_DEVICE);
    CHECK(fd_decode_attention_int8(&good, fake(0), fake(1), fake(2), nullptr, 1.f, INFINITY, dl, 0.1f, 0, nullptr,
                                   nullptr, 0, fake(4), nullptr, nullptr) == FD_ERR_INVALID);
    CHECK(fd_decode_attention_int8(&f32q, fake(0), fake(1), fake(2), nullptr, 1.f, 1.f, dl, 0.1f, 0, nullptr,
                                   nullptr, 0, fake(4), nullptr, nullptr) == FD_ERR_UNSUPPORTED);
    CHECK(std::strstr(fd_last_error(), "int8") != nullptr);
    CHECK(fd_decode_partials_int8(&good, fake(0), fake(1), fake(2), &pg, 0.5f, 2.f, dl, 0.1f, 3, nullptr,
                                  (float*)fake(5), (float*)fake(6), (float*)fake(7), nullptr) == FD_ERR_DEVICE);
    // status strings and a long error message
    for (int s = -10; s <= 1; ++s) CHECK(std::strlen(fd_status_string(s)) > 0);
    const fd_dims huge{1, 32, 8, 128, 1, 64, FD_BF16};
    const int32_t big[1] = {INT32_MAX};
    CHECK(fd_plan_splits(&huge, big, 0, 256, &p, nullptr) == FD_ERR_INVALID);
    CHECK(std::strlen(fd_last_error()) < 512);
}

}  // namespace

int main() {
    random_plans();
    extreme_plans();
    validation_paths();
    if (g_failures) {
        std::fprintf(stderr, "%d host checks failed\n", g_failures);
        return 1;
    }
    std::printf("host checks ok\n");
    return 0;
}
