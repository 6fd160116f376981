// Drives the host side of the C ABI (configuration checks, arena layout,
// argument checks, error paths, cleanup on failure) without a GPU, for a build
// of dms_api.cpp with AddressSanitizer and UndefinedBehaviorSanitizer on the
// host: any out-of-bounds access, leak-free cleanup violation or undefined
// operation (a signed overflow in the layout arithmetic, say) aborts the run.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "dms.h"

static int fails = 0;
#define CHECK(c)                                                           \
    do {                                                                   \
        if (!(c)) {                                                        \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++fails;                                                       \
        }                                                                  \
    } while (0)

static dms_pool_config qwen() {
    dms_pool_config c;
    std::memset(&c, 0, sizeof(c));
    c.n_layers = 36; c.n_q_heads = 32; c.n_kv_heads = 8; c.head_dim = 128; c.window = 512;
    c.max_seqs = 1; c.max_positions = 8320; c.max_pages = 36 * 8 * 131;
    return c;
}

int main() {
    // valid configurations across the parameter ranges, extremes included
    const int dims[] = {64, 128}, groups[] = {1, 2, 4, 8};
    for (int d : dims)
        for (int g : groups)
            for (int fmt = 0; fmt < 2; ++fmt)
                for (int w : {1, 7, 512, 1 << 30}) {
                    dms_pool_config c = qwen();
                    c.head_dim = d; c.n_kv_heads = 4; c.n_q_heads = 4 * g; c.kv_format = fmt; c.window = w;
                    c.n_layers = 3; c.max_seqs = 5; c.max_positions = 1000; c.max_pages = 3 * 4 * 5 * 16;
                    const size_t n = dms_pool_bytes(&c);
                    CHECK(n > 0 && n % 256 == 0);
                    CHECK(std::strlen(dms_last_error()) == 0);
                }
    {   // the largest shapes the checks admit, and just past them
        dms_pool_config c = qwen();
        c.max_positions = 1 << 30; c.max_pages = 1; c.n_kv_heads = 128; c.n_q_heads = 128; c.n_layers = 1;
        CHECK(dms_pool_bytes(&c) == 0);  // 128 x 2^24 scratch pages: the page arrays reach 2^31
        c.n_kv_heads = 64; c.n_q_heads = 64;
        CHECK(dms_pool_bytes(&c) > 0);   // 2^30 + 1 pages
        c.max_positions = 1 << 20;
        CHECK(dms_pool_bytes(&c) > 0);
        c = qwen(); c.max_pages = (int64_t)INT32_MAX;
        CHECK(dms_pool_bytes(&c) == 0);
        c = qwen(); c.max_pages = (int64_t)INT32_MAX + 1;
        CHECK(dms_pool_bytes(&c) == 0);
        c = qwen(); c.max_seqs = INT32_MAX;
        CHECK(dms_pool_bytes(&c) == 0);
        c = qwen(); c.n_layers = 4032 / 8 + 1;
        CHECK(dms_pool_bytes(&c) == 0);
    }
    {   // each invalid field on its own
        dms_pool_config c;
        c = qwen(); c.head_dim = 96; CHECK(dms_pool_bytes(&c) == 0);
        c = qwen(); c.n_q_heads = 12; CHECK(dms_pool_bytes(&c) == 0);
        c = qwen(); c.n_q_heads = 128; CHECK(dms_pool_bytes(&c) == 0);
        c = qwen(); c.window = 0; CHECK(dms_pool_bytes(&c) == 0);
        c = qwen(); c.max_positions = 0; CHECK(dms_pool_bytes(&c) == 0);
        c = qwen(); c.max_positions = (1 << 30) + 1; CHECK(dms_pool_bytes(&c) == 0);
        c = qwen(); c.page_slots = 32; CHECK(dms_pool_bytes(&c) == 0);
        c = qwen(); c.softmax_scale = NAN; CHECK(dms_pool_bytes(&c) == 0);
        c = qwen(); c.softmax_scale = -1.f; CHECK(dms_pool_bytes(&c) == 0);
        c = qwen(); c.softmax_scale = INFINITY; CHECK(dms_pool_bytes(&c) == 0);
        c = qwen(); c.kv_format = 2; CHECK(dms_pool_bytes(&c) == 0);
        c = qwen(); c.logit_source = 1; c.logit_channel = 128; CHECK(dms_pool_bytes(&c) == 0);
        c = qwen(); c.logit_channel = 1; CHECK(dms_pool_bytes(&c) == 0);
        c = qwen(); c.reserved[0] = 1; CHECK(dms_pool_bytes(&c) == 0);
        CHECK(dms_pool_bytes(nullptr) == 0);
        CHECK(std::strlen(dms_last_error()) > 0);
    }
    {   // create: argument checks before any device call
        dms_pool_config c = qwen();
        const size_t n = dms_pool_bytes(&c);
        dms_pool* p = nullptr;
        CHECK(dms_pool_create(&c, nullptr, n, nullptr, &p) == DMS_E_INVAL && p == nullptr);
        CHECK(dms_pool_create(&c, reinterpret_cast<void*>(0x1008), n, nullptr, &p) == DMS_E_INVAL);
        CHECK(dms_pool_create(&c, reinterpret_cast<void*>(0x1000), n - 256, nullptr, &p) == DMS_E_NOMEM);
        CHECK(dms_pool_create(&c, reinterpret_cast<void*>(0x1000), n, nullptr, nullptr) == DMS_E_INVAL);
        CHECK(dms_pool_create(nullptr, reinterpret_cast<void*>(0x1000), n, nullptr, &p) == DMS_E_INVAL);
    }
    {   // every entry point on a NULL pool
        dms_stats st;
        dms_timing tm;
        int32_t ids[1] = {0}, n = 0;
        CHECK(dms_pool_destroy(nullptr) == DMS_E_INVAL);
        CHECK(dms_prefill(nullptr, 0, 0, 1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == DMS_E_INVAL);
        CHECK(dms_extend(nullptr, 0, 0, 1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == DMS_E_INVAL);
        CHECK(dms_decode_step(nullptr, 1, ids, 0, 1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) ==
              DMS_E_INVAL);
        CHECK(dms_query_stats(nullptr, 0, &st, nullptr) == DMS_E_INVAL);
        CHECK(dms_export_live(nullptr, 0, 0, 0, nullptr, 0, &n) == DMS_E_INVAL);
        CHECK(dms_export_kv(nullptr, 0, 0, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, &n) == DMS_E_INVAL);
        CHECK(dms_seq_release(nullptr, 0, nullptr) == DMS_E_INVAL);
        CHECK(dms_timing_enable(nullptr, 1) == DMS_E_INVAL);
        CHECK(dms_timing_read(nullptr, &tm) == DMS_E_INVAL);
    }
    if (fails) {
        std::fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    std::printf("abi driver ok\n");
    return 0;
}
