// Host side of the DMS C ABI (include/dms.h): configuration checks, arena
// layout, per-(sequence, layer) bookkeeping, kernel launches and stats.
#include "dms.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "dms_internal.h"

namespace {

thread_local std::string g_err;

dms_status fail(dms_status s, const std::string& msg) {
    g_err = msg;
    return s;
}

dms_status hip_fail(hipError_t e, const char* what) {
    return fail(DMS_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

enum Section { S_K, S_V, S_KS, S_VS, S_POS, S_STACK, S_RCACHE, S_HSTATE, S_PTABLE, S_RING, S_PART, S_PREFIX,
               S_INV, S_PCNT, S_VT, S_VT16, S_MBITS, S_Q8, S_CTL, S_N };

struct Layout {
    size_t off[S_N + 1];
    int64_t heads;
    int32_t pages_per_head, ring_len, max_items, max_call_heads;
};

bool make_layout(const dms_pool_config* c, Layout* L, std::string* why) {
    auto bad = [&](const char* m) { *why = m; return false; };
    if (!c) return bad("config is NULL");
    if (c->n_layers < 1) return bad("n_layers must be >= 1");
    if (c->n_kv_heads < 1) return bad("n_kv_heads must be >= 1");
    if (c->n_q_heads < c->n_kv_heads || c->n_q_heads % c->n_kv_heads) return bad("n_q_heads must be a multiple of n_kv_heads");
    const int g = c->n_q_heads / c->n_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8) return bad("n_q_heads / n_kv_heads must be 1, 2, 4 or 8");
    if (c->head_dim != 64 && c->head_dim != 128) return bad("head_dim must be 64 or 128");
    if (c->window < 1) return bad("window must be >= 1");
    if (c->max_seqs < 1) return bad("max_seqs must be >= 1");
    if (c->max_positions < 1 || c->max_positions > (1 << 30)) return bad("max_positions must be in [1, 2^30]");
    if (c->page_slots != 0 && c->page_slots != DMS_PAGE_SLOTS) return bad("page_slots must be 0 or 64");
    if (c->max_pages < 1 || c->max_pages > (int64_t)INT32_MAX) return bad("max_pages must be in [1, 2^31)");
    if (!(c->softmax_scale >= 0.f) || !std::isfinite(c->softmax_scale)) return bad("softmax_scale must be finite and >= 0");
    if (c->kv_format != DMS_KV_BF16 && c->kv_format != DMS_KV_FP8_E4M3)
        return bad("kv_format must be DMS_KV_BF16 or DMS_KV_FP8_E4M3");
    if (c->logit_source == DMS_LOGITS_INPUT) {
        if (c->logit_channel != 0) return bad("logit_channel must be 0 unless logit_source is DMS_LOGITS_K_CHANNEL");
    } else if (c->logit_source == DMS_LOGITS_K_CHANNEL) {
        if (c->logit_channel < 0 || c->logit_channel >= c->head_dim) return bad("logit_channel must be in [0, head_dim)");
    } else {
        return bad("logit_source must be DMS_LOGITS_INPUT or DMS_LOGITS_K_CHANNEL");
    }
    if (c->reserved[0] != 0) return bad("reserved fields must be 0");
    const int64_t heads = (int64_t)c->max_seqs * c->n_layers * c->n_kv_heads;
    if (heads > (int64_t)INT32_MAX / 4) return bad("max_seqs * n_layers * n_kv_heads too large");
    if ((int64_t)c->n_layers * c->n_kv_heads > dms::kMaxCallHeads) return bad("n_layers * n_kv_heads too large");
    const int64_t D = c->head_dim;
    L->heads = heads;
    L->pages_per_head = (c->max_positions + dms::kPage - 1) / dms::kPage;
    L->ring_len = c->window < c->max_positions ? c->window : 0;
    L->max_call_heads = (int32_t)std::min<int64_t>(heads, dms::kMaxCallHeads);
    // partial slots: one per (attention wave, call head) pair that can occur
    L->max_items = dms::kMaxAttendBlocks * dms::kAttendWaves + L->max_call_heads;
    const bool fp8 = c->kv_format == DMS_KV_FP8_E4M3;
    size_t sz[S_N];
    // K / V pages: the shared pool's max_pages, then pages_per_head scratch pages
    // per kv head (extend calls gather the chunk's unmarked rows there)
    const int64_t all_pages = c->max_pages + (int64_t)c->n_kv_heads * L->pages_per_head;
    if (all_pages > (int64_t)INT32_MAX) return bad("max_pages + n_kv_heads * ceil(max_positions / 64) must be below 2^31");
    sz[S_K] = (size_t)all_pages * dms::kPage * D * (fp8 ? 1 : 2);
    sz[S_V] = sz[S_K];
    sz[S_KS] = fp8 ? (size_t)all_pages * dms::kPage * 4 : 0;
    sz[S_VS] = sz[S_KS];
    sz[S_POS] = (size_t)c->max_pages * dms::kPage * 4;
    sz[S_STACK] = (size_t)c->max_pages * 4;
    sz[S_HSTATE] = (size_t)heads * dms::kHS * 4;
    sz[S_PTABLE] = (size_t)heads * L->pages_per_head * 4;
    sz[S_RING] = (size_t)heads * L->ring_len * 4;
    sz[S_PART] = (size_t)L->max_items * dms::part_stride(g, (int)D) * 4;
    sz[S_PREFIX] = (size_t)(L->max_call_heads + 1) * 4;
    sz[S_INV] = (size_t)c->n_kv_heads * c->max_positions * 4;
    sz[S_PCNT] = sz[S_INV];
    sz[S_VT] = (size_t)c->n_kv_heads * ((c->max_positions + 31) / 32 * 32) * D * 2;
    sz[S_VT16] = fp8 ? 0 : sz[S_VT];
    sz[S_MBITS] = (size_t)c->n_kv_heads * ((c->max_positions + 63) / 64) * 2 * 4;
    sz[S_Q8] = fp8 ? (size_t)2 * c->max_positions * c->n_kv_heads * (D + 4) : 0;
    sz[S_RCACHE] = dms::kRunCacheBytes;
    sz[S_CTL] = 64 * 4;
    size_t o = 0;
    for (int i = 0; i < S_N; ++i) {
        L->off[i] = o;
        o = align_up(o + sz[i]);
    }
    L->off[S_N] = o;
    // the decode attention finds the page cache from the head-record pointer
    if (L->off[S_HSTATE] != L->off[S_RCACHE] + dms::kRunCacheBytes) return bad("arena layout: cache placement");
    return true;
}

// SplitMix64 step, used only to shuffle the initial page order on request.
uint64_t mix64(uint64_t& s) {
    uint64_t z = (s += 0x9E3779B97F4A7C15ULL);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

}  // namespace

struct dms_pool {
    // streams the pool's work was enqueued on (synchronising calls wait for
    // these, not for the whole device); beyond kMaxStreams distinct streams the
    // synchronising calls fall back to the whole device
    static constexpr int kMaxStreams = 16;
    hipStream_t streams[kMaxStreams];
    int n_streams = 0;
    bool streams_overflow = false;
    void note(hipStream_t s) {
        for (int i = 0; i < n_streams; ++i)
            if (streams[i] == s) return;
        if (n_streams < kMaxStreams) streams[n_streams++] = s;
        else streams_overflow = true;
    }
    hipError_t sync() const {
        if (streams_overflow) return hipDeviceSynchronize();
        for (int i = 0; i < n_streams; ++i) {
            const hipError_t e = hipStreamSynchronize(streams[i]);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    dms_pool_config cfg;
    bool timing = false;
    std::vector<hipEvent_t> events;   // 4 per decode launch while timing (attend, merge start/stop)
    std::vector<hipEvent_t> pevents;  // 4 per prefill with output while timing (compaction with V copy, attend)
    std::vector<hipEvent_t> xevents;  // 4 per extend with output while timing (preparation, attend)
    Layout layout;
    dms::PoolDev dev;
    char* arena;
    std::vector<int32_t> pos;  // [max_seqs][n_layers]: next position, -1 = empty
    std::vector<uint32_t> seen;  // [max_seqs]: call stamp of the last decode call naming the sequence
    uint32_t call_stamp = 0;
    uint64_t rewrites = 0;       // releases and prefills (each advances the device's page-cache epoch once at most)
    void* scratch = nullptr;     // device address of the static decode scratch on the pool's device
    int cu_count;
    int attend_per_cu;  // attention blocks per compute unit (checked once, for the largest call)
    int32_t& position(int seq, int layer) { return pos[(size_t)seq * cfg.n_layers + layer]; }
};

extern "C" {

const char* dms_last_error(void) { return g_err.c_str(); }

size_t dms_pool_bytes(const dms_pool_config* cfg) {
    Layout L;
    std::string why;
    if (!make_layout(cfg, &L, &why)) {
        g_err = why;
        return 0;
    }
    g_err.clear();
    return L.off[S_N];
}

dms_status dms_pool_create(const dms_pool_config* cfg, void* arena, size_t arena_bytes, void* stream,
                           dms_pool** out) {
    if (!out) return fail(DMS_E_INVAL, "out is NULL");
    *out = nullptr;
    Layout L;
    std::string why;
    if (!make_layout(cfg, &L, &why)) return fail(DMS_E_INVAL, why);
    if (!arena) return fail(DMS_E_INVAL, "arena is NULL");
    if (reinterpret_cast<uintptr_t>(arena) % kAlign) return fail(DMS_E_INVAL, "arena must be 256-byte aligned");
    if (arena_bytes < L.off[S_N]) return fail(DMS_E_NOMEM, "arena smaller than dms_pool_bytes()");
    hipStream_t s = static_cast<hipStream_t>(stream);

    dms_pool* p = new dms_pool();
    p->note(s);
    p->cfg = *cfg;
    if (p->cfg.page_slots == 0) p->cfg.page_slots = DMS_PAGE_SLOTS;
    p->layout = L;
    p->arena = static_cast<char*>(arena);
    p->pos.assign((size_t)cfg->max_seqs * cfg->n_layers, -1);
    p->seen.assign((size_t)cfg->max_seqs, 0);
    p->cu_count = dms::device_cu_count();
    char* a = p->arena;
    dms::PoolDev& d = p->dev;
    d.kpages = reinterpret_cast<uint16_t*>(a + L.off[S_K]);
    d.vpages = reinterpret_cast<uint16_t*>(a + L.off[S_V]);
    d.kscale = reinterpret_cast<float*>(a + L.off[S_KS]);
    d.vscale = reinterpret_cast<float*>(a + L.off[S_VS]);
    d.q8 = reinterpret_cast<uint8_t*>(a + L.off[S_Q8]);
    d.slot_pos = reinterpret_cast<int32_t*>(a + L.off[S_POS]);
    d.stack = reinterpret_cast<int32_t*>(a + L.off[S_STACK]);
    d.hstate = reinterpret_cast<int32_t*>(a + L.off[S_HSTATE]);
    d.ptable = reinterpret_cast<int32_t*>(a + L.off[S_PTABLE]);
    d.ring = reinterpret_cast<int32_t*>(a + L.off[S_RING]);
    d.partials = reinterpret_cast<float*>(a + L.off[S_PART]);
    d.prefix = reinterpret_cast<int32_t*>(a + L.off[S_PREFIX]);
    d.inv = reinterpret_cast<int32_t*>(a + L.off[S_INV]);
    d.pcnt = reinterpret_cast<int32_t*>(a + L.off[S_PCNT]);
    d.vt = reinterpret_cast<uint16_t*>(a + L.off[S_VT]);
    d.vt16 = reinterpret_cast<uint16_t*>(a + L.off[S_VT16]);
    d.mbits = reinterpret_cast<uint32_t*>(a + L.off[S_MBITS]);
    d.rcache = reinterpret_cast<int32_t*>(a + L.off[S_RCACHE]);
    d.ctl = reinterpret_cast<int32_t*>(a + L.off[S_CTL]);
    d.max_pages = cfg->max_pages;
    d.n_layers = cfg->n_layers;
    d.n_q_heads = cfg->n_q_heads;
    d.n_kv_heads = cfg->n_kv_heads;
    d.head_dim = cfg->head_dim;
    d.window = cfg->window;
    d.ring_len = L.ring_len;
    d.pages_per_head = L.pages_per_head;
    d.max_positions = cfg->max_positions;
    d.max_pos32 = (cfg->max_positions + 31) / 32 * 32;
    d.max_items = L.max_items;
    d.fp8 = cfg->kv_format == DMS_KV_FP8_E4M3 ? 1 : 0;
    d.logit_ch = cfg->logit_source == DMS_LOGITS_K_CHANNEL ? cfg->logit_channel : -1;
    const double scale = cfg->softmax_scale > 0.f ? (double)cfg->softmax_scale : 1.0 / std::sqrt((double)cfg->head_dim);
    d.scale_log2 = (float)(scale * 1.4426950408889634);

    // free stack: pops take stack[top-1] first, so store the hand-out order reversed
    std::vector<int32_t> order((size_t)cfg->max_pages);
    for (int64_t i = 0; i < cfg->max_pages; ++i) order[i] = (int32_t)i;
    if (cfg->page_order_seed) {
        uint64_t st = cfg->page_order_seed;
        for (int64_t i = cfg->max_pages - 1; i > 0; --i) std::swap(order[i], order[mix64(st) % (uint64_t)(i + 1)]);
    }
    std::reverse(order.begin(), order.end());
    int32_t ctl[64] = {0};
    ctl[dms::kCtlTop] = (int32_t)cfg->max_pages;

    std::vector<int32_t> rec((size_t)L.heads * dms::kHS, 0);  // empty heads: no expiring slot
    for (int64_t h = 0; h < L.heads; ++h) rec[(size_t)h * dms::kHS + dms::kHsExp] = -1;
    hipError_t e = hipMemsetAsync(arena, 0, L.off[S_N], s);
    if (e == hipSuccess) e = hipMemcpyAsync(d.stack, order.data(), order.size() * 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(d.hstate, rec.data(), rec.size() * 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(d.ctl, ctl, sizeof(ctl), hipMemcpyHostToDevice, s);
    const int32_t epoch = 1;
    if (e == hipSuccess) e = hipMemcpyAsync(d.rcache, &epoch, sizeof(epoch), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = dms::launch_page_cache_clear(d, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = dms::static_scratch_address(&p->scratch);  // once per device, here
    if (e != hipSuccess) {
        delete p;
        return hip_fail(e, "pool initialisation");
    }
    {
        dms::DecodeArgs probe{};
        probe.pool = d;
        probe.n_call_heads = L.max_call_heads;
        const int want = d.fp8 ? dms::kAttendBlocksPerCUFp8 : dms::kAttendBlocksPerCU;
        p->attend_per_cu = std::min(want, dms::decode_blocks_per_cu(probe));
        if (p->attend_per_cu < 1) {
            delete p;
            return fail(DMS_E_INVAL, "the decode kernel does not fit a compute unit with this configuration");
        }
    }
    *out = p;
    g_err.clear();
    return DMS_OK;
}

dms_status dms_pool_destroy(dms_pool* pool) {
    if (!pool) return fail(DMS_E_INVAL, "pool is NULL");
    hipError_t e = pool->sync();
    for (hipEvent_t ev : pool->events) (void)hipEventDestroy(ev);
    for (hipEvent_t ev : pool->pevents) (void)hipEventDestroy(ev);
    for (hipEvent_t ev : pool->xevents) (void)hipEventDestroy(ev);
    delete pool;
    if (e != hipSuccess) return hip_fail(e, "synchronise");
    g_err.clear();
    return DMS_OK;
}

namespace {
// n fresh events appended to v (for one timed call), or nullptr on failure
hipEvent_t* timing_events(std::vector<hipEvent_t>& v, size_t n, hipError_t* err) {
    const size_t base = v.size();
    v.resize(base + n, nullptr);
    for (size_t i = base; i < base + n; ++i) {
        *err = hipEventCreate(&v[i]);
        if (*err != hipSuccess) return nullptr;
    }
    return &v[base];
}
}  // namespace

dms_status dms_prefill(dms_pool* pool, int32_t seq, int32_t layer, int32_t n_tokens, const void* q, const void* k,
                       const void* v, const float* logits, void* out, void* stream) {
    if (!pool) return fail(DMS_E_INVAL, "pool is NULL");
    const dms_pool_config& c = pool->cfg;
    if (seq < 0 || seq >= c.max_seqs) return fail(DMS_E_INVAL, "seq out of range");
    if (layer < 0 || layer >= c.n_layers) return fail(DMS_E_INVAL, "layer out of range");
    if (n_tokens < 1 || n_tokens > c.max_positions) return fail(DMS_E_INVAL, "n_tokens must be in [1, max_positions]");
    const bool need_logits = c.logit_source == DMS_LOGITS_INPUT;
    if (!k || !v || (need_logits && !logits)) return fail(DMS_E_INVAL, "k, v and logits must not be NULL");
    if (out && !q) return fail(DMS_E_INVAL, "q must not be NULL when out is given");
    if (pool->position(seq, layer) >= 0) return fail(DMS_E_STATE, "this (seq, layer) already holds tokens");
    dms::PrefillArgs a;
    a.pool = pool->dev;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.logits = logits;
    a.out = static_cast<uint16_t*>(out);
    a.seq = seq;
    a.layer = layer;
    a.n_tokens = n_tokens;
    a.t0 = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    pool->note(s);
    hipError_t e = hipSuccess;
    hipEvent_t* ev = nullptr;
    if (pool->timing && out) {
        ev = timing_events(pool->pevents, 4, &e);
        if (!ev) return hip_fail(e, "timing event");
    }
    e = dms::launch_prefill_compact(a, out != nullptr, s, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr);
    if (e != hipSuccess) return hip_fail(e, "prefill compaction launch");
    if (out) {
        e = dms::launch_prefill_attend(a, s, ev ? ev + 2 : nullptr);
        if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
    }
    pool->position(seq, layer) = n_tokens;
    if (++pool->rewrites % dms::kRunCacheRefill == 0) {
        e = dms::launch_page_cache_clear(pool->dev, s);
        if (e != hipSuccess) return hip_fail(e, "page cache clear launch");
    }
    g_err.clear();
    return DMS_OK;
}

dms_status dms_extend(dms_pool* pool, int32_t seq, int32_t layer, int32_t n_tokens, const void* q, const void* k,
                      const void* v, const float* logits, void* out, void* stream) {
    if (!pool) return fail(DMS_E_INVAL, "pool is NULL");
    const dms_pool_config& c = pool->cfg;
    if (seq < 0 || seq >= c.max_seqs) return fail(DMS_E_INVAL, "seq out of range");
    if (layer < 0 || layer >= c.n_layers) return fail(DMS_E_INVAL, "layer out of range");
    if (n_tokens < 1) return fail(DMS_E_INVAL, "n_tokens must be >= 1");
    if (!k || !v || (c.logit_source == DMS_LOGITS_INPUT && !logits))
        return fail(DMS_E_INVAL, "k, v and logits must not be NULL");
    if (out && !q) return fail(DMS_E_INVAL, "q must not be NULL when out is given");
    const int32_t t0 = pool->position(seq, layer);
    if (t0 < 0) return fail(DMS_E_STATE, "extend on a (seq, layer) that was not prefilled");
    if ((int64_t)t0 + n_tokens > c.max_positions) return fail(DMS_E_STATE, "the chunk runs past max_positions");
    dms::PrefillArgs a;
    a.pool = pool->dev;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.logits = logits;
    a.out = static_cast<uint16_t*>(out);
    a.seq = seq;
    a.layer = layer;
    a.n_tokens = n_tokens;
    a.t0 = t0;
    hipError_t e = hipSuccess;
    hipEvent_t* ev = nullptr;
    if (pool->timing && out) {
        ev = timing_events(pool->xevents, 4, &e);
        if (!ev) return hip_fail(e, "timing event");
    }
    pool->note(static_cast<hipStream_t>(stream));
    e = dms::launch_extend(a, out != nullptr, static_cast<hipStream_t>(stream), ev);
    if (e != hipSuccess) return hip_fail(e, "extend launch");
    pool->position(seq, layer) = t0 + n_tokens;
    g_err.clear();
    return DMS_OK;
}

}  // extern "C"

namespace {

// Bytes of split-K partials and page-axis prefix one decode launch of up to
// `heads` call heads needs at most (the largest attention grid the pool uses).
size_t decode_scratch_bytes(const dms_pool* pool, int heads) {
    const dms_pool_config& c = pool->cfg;
    const int64_t blocks = std::min<int64_t>((int64_t)pool->cu_count * pool->attend_per_cu, dms::kMaxAttendBlocks);
    const int64_t items = blocks * dms::kAttendWaves + heads;
    const size_t part = (size_t)items * dms::part_stride(c.n_q_heads / c.n_kv_heads, c.head_dim) * 4;
    return align_up(part) + (size_t)(heads + 1) * 4;
}

// One decode step; the partials and prefix live in the pool's arena, or (with
// scratch) in the given device buffer.  Allocates nothing per call: no device
// memory, no host containers; with scratch, no timing events either.
dms_status decode_step(dms_pool* pool, int32_t n_seqs, const int32_t* seq_ids, int32_t layer0, int32_t n_layers,
                       const void* q, const void* k, const void* v, const float* logits, void* out, void* stream,
                       char* scratch, size_t scratch_bytes) {
    if (!pool) return fail(DMS_E_INVAL, "pool is NULL");
    const dms_pool_config& c = pool->cfg;
    if (n_seqs < 1 || n_seqs > c.max_seqs) return fail(DMS_E_INVAL, "n_seqs must be in [1, max_seqs]");
    if (!seq_ids) return fail(DMS_E_INVAL, "seq_ids is NULL");
    if (layer0 < 0 || n_layers < 1 || layer0 + n_layers > c.n_layers) return fail(DMS_E_INVAL, "layer range out of bounds");
    if (!q || !k || !v || !out || (c.logit_source == DMS_LOGITS_INPUT && !logits))
        return fail(DMS_E_INVAL, "q, k, v, logits and out must not be NULL");
    const int hkv = c.n_kv_heads;
    const int per_launch = std::max(1, std::min(dms::kMaxCallSeqs, dms::kMaxCallHeads / (n_layers * hkv)));
    if (scratch) {
        const size_t need = decode_scratch_bytes(pool, std::min(n_seqs, per_launch) * n_layers * hkv);
        if (need > scratch_bytes)
            return fail(DMS_E_INVAL, "this call needs " + std::to_string(need) + " bytes of decode scratch, above the " +
                                         std::to_string(scratch_bytes) + " the static array holds");
    }
    if (++pool->call_stamp == 0) {  // the stamp wrapped: forget every older stamp
        std::fill(pool->seen.begin(), pool->seen.end(), 0u);
        pool->call_stamp = 1;
    }
    for (int i = 0; i < n_seqs; ++i) {
        const int s = seq_ids[i];
        if (s < 0 || s >= c.max_seqs) return fail(DMS_E_INVAL, "seq id out of range");
        if (pool->seen[s] == pool->call_stamp) return fail(DMS_E_INVAL, "seq ids must be distinct");
        pool->seen[s] = pool->call_stamp;
        for (int l = layer0; l < layer0 + n_layers; ++l) {
            const int p = pool->position(s, l);
            if (p < 0) return fail(DMS_E_STATE, "decode on a (seq, layer) that was not prefilled");
            if (p >= c.max_positions) return fail(DMS_E_STATE, "sequence reached max_positions");
        }
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    pool->note(st);
    for (int sb = 0; sb < n_seqs; sb += per_launch) {
        dms::DecodeArgs a;
        a.pool = pool->dev;
        if (scratch) {  // every launch of the call reuses the buffer, in stream order
            a.pool.partials = reinterpret_cast<float*>(scratch);
            const int heads = std::min(per_launch, n_seqs - sb) * n_layers * hkv;
            a.pool.prefix = reinterpret_cast<int32_t*>(scratch + decode_scratch_bytes(pool, heads) -
                                                       (size_t)(heads + 1) * 4);
        }
        a.q = static_cast<const uint16_t*>(q);
        a.k = static_cast<const uint16_t*>(k);
        a.v = static_cast<const uint16_t*>(v);
        a.logits = logits;
        a.out = static_cast<uint16_t*>(out);
        a.n_seqs_total = n_seqs;
        a.seq_base = sb;
        a.n_seqs = std::min(per_launch, n_seqs - sb);
        a.layer0 = layer0;
        a.n_layers = n_layers;
        a.n_call_heads = a.n_layers * a.n_seqs * hkv;
        int64_t bound = 0;  // pages of the call: n_live <= position, ceil(n_live / 64) per head
        for (int i = 0; i < a.n_seqs; ++i) {
            a.seq_ids[i] = seq_ids[sb + i];
            for (int l = layer0; l < layer0 + n_layers; ++l)
                bound += (int64_t)hkv * ((pool->position(a.seq_ids[i], l) + dms::kPage - 1) / dms::kPage);
        }
        int64_t grid = std::min<int64_t>((int64_t)pool->cu_count * pool->attend_per_cu, dms::kMaxAttendBlocks);
        grid = std::max<int64_t>(1, std::min<int64_t>(grid, (bound + dms::kAttendWaves - 1) / dms::kAttendWaves));
        a.n_waves = (int32_t)grid * dms::kAttendWaves;
        hipEvent_t* ev = nullptr;
        if (pool->timing && !scratch) {
            hipError_t ce = hipSuccess;
            ev = timing_events(pool->events, 4, &ce);
            if (!ev) return hip_fail(ce, "timing event");
        }
        hipError_t e = dms::launch_decode(a, (int)grid, st, ev);
        if (e != hipSuccess) return hip_fail(e, "decode launch");
    }
    for (int i = 0; i < n_seqs; ++i)
        for (int l = layer0; l < layer0 + n_layers; ++l) pool->position(seq_ids[i], l) += 1;
    g_err.clear();
    return DMS_OK;
}

}  // namespace

extern "C" {

dms_status dms_decode_step(dms_pool* pool, int32_t n_seqs, const int32_t* seq_ids, int32_t layer0, int32_t n_layers,
                           const void* q, const void* k, const void* v, const float* logits, void* out,
                           void* stream) {
    return decode_step(pool, n_seqs, seq_ids, layer0, n_layers, q, k, v, logits, out, stream, nullptr, 0);
}

dms_status dms_decode_step_static(dms_pool* pool, int32_t n_seqs, const int32_t* seq_ids, int32_t layer0,
                                  int32_t n_layers, const void* q, const void* k, const void* v, const float* logits,
                                  void* out, void* stream) {
    if (!pool) return fail(DMS_E_INVAL, "pool is NULL");
    if (!pool->scratch) return fail(DMS_E_STATE, "no static scratch on this pool's device");
    return decode_step(pool, n_seqs, seq_ids, layer0, n_layers, q, k, v, logits, out, stream,
                       static_cast<char*>(pool->scratch), dms::kStaticScratchBytes);
}

dms_status dms_query_stats(dms_pool* pool, int32_t seq, dms_stats* out, int32_t* live_per_layer_head) {
    if (!pool || !out) return fail(DMS_E_INVAL, "pool and out must not be NULL");
    const dms_pool_config& c = pool->cfg;
    if (seq < -1 || seq >= c.max_seqs) return fail(DMS_E_INVAL, "seq out of range");
    if (live_per_layer_head && seq < 0) return fail(DMS_E_INVAL, "live_per_layer_head needs seq >= 0");
    hipError_t e = pool->sync();
    if (e != hipSuccess) return hip_fail(e, "synchronise");
    const int64_t per_seq = (int64_t)c.n_layers * c.n_kv_heads;
    const int s0 = seq < 0 ? 0 : seq, s1 = seq < 0 ? c.max_seqs : seq + 1;
    std::vector<int32_t> hs((size_t)(s1 - s0) * per_seq * dms::kHS);
    int32_t ctl[64];
    e = hipMemcpy(hs.data(), pool->dev.hstate + (size_t)s0 * per_seq * dms::kHS, hs.size() * 4, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(ctl, pool->dev.ctl, sizeof(ctl), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "read pool state");
    const int64_t D = c.head_dim;
    std::memset(out, 0, sizeof(*out));
    int64_t dense_tokens = 0;
    for (int s = s0; s < s1; ++s) {
        for (int l = 0; l < c.n_layers; ++l) {
            int32_t& hp = pool->position(s, l);
            const int32_t* h0 = &hs[(((size_t)(s - s0) * c.n_layers + l) * c.n_kv_heads) * dms::kHS];
            if (hp >= 0) hp = h0[dms::kHsPos];  // device counters are authoritative (graph replays bypass the host)
            if (hp > 0) dense_tokens += (int64_t)hp * c.n_kv_heads;
            for (int h = 0; h < c.n_kv_heads; ++h) {
                const int32_t* x = h0 + h * dms::kHS;
                out->live_slots += x[dms::kHsLive];
                out->pages_used += x[dms::kHsPages];
                if (live_per_layer_head) live_per_layer_head[l * c.n_kv_heads + h] = x[dms::kHsLive];
            }
        }
    }
    const int64_t slot_bytes = c.kv_format == DMS_KV_FP8_E4M3 ? 2 * (D + 4) : 2 * D * 2;
    out->kv_bytes_live = out->live_slots * slot_bytes;
    out->kv_bytes_allocated = out->pages_used * dms::kPage * slot_bytes;
    out->kv_bytes_dense_equiv = dense_tokens * 2 * D * 2;
    out->pages_free = ctl[dms::kCtlTop];
    out->workspace_bytes = (int64_t)(pool->layout.off[S_N] - pool->layout.off[S_POS]);
    out->position = seq >= 0 ? pool->position(seq, 0) : -1;
    out->device_error = ctl[dms::kCtlError] ? DMS_E_CAPACITY : (ctl[dms::kCtlPosError] ? DMS_E_STATE : DMS_OK);
    if (ctl[dms::kCtlError]) return fail(DMS_E_CAPACITY, "the shared page pool ran out on the device");
    if (ctl[dms::kCtlPosError])
        return fail(DMS_E_STATE, "a decode or extend call ran past max_positions on the device (tokens dropped)");
    g_err.clear();
    return DMS_OK;
}

dms_status dms_export_live(dms_pool* pool, int32_t seq, int32_t layer, int32_t kv_head, int32_t* positions,
                           int32_t cap, int32_t* n) {
    if (!pool || !n) return fail(DMS_E_INVAL, "pool and n must not be NULL");
    const dms_pool_config& c = pool->cfg;
    if (seq < 0 || seq >= c.max_seqs || layer < 0 || layer >= c.n_layers || kv_head < 0 || kv_head >= c.n_kv_heads)
        return fail(DMS_E_INVAL, "(seq, layer, kv_head) out of range");
    hipError_t e = pool->sync();
    if (e != hipSuccess) return hip_fail(e, "synchronise");
    const int64_t gh = ((int64_t)seq * c.n_layers + layer) * c.n_kv_heads + kv_head;
    int32_t hs[dms::kHS];
    e = hipMemcpy(hs, pool->dev.hstate + gh * dms::kHS, sizeof(hs), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "read head state");
    const int live = hs[dms::kHsLive], np = hs[dms::kHsPages];
    *n = live;
    if (live > cap || (live > 0 && !positions)) return fail(DMS_E_INVAL, "positions array too small");
    std::vector<int32_t> pages((size_t)np);
    if (np > 0) {
        e = hipMemcpy(pages.data(), pool->dev.ptable + gh * pool->layout.pages_per_head, (size_t)np * 4,
                      hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(e, "read page table");
    }
    std::vector<int32_t> buf(dms::kPage);
    int got = 0;
    for (int j = 0; j < np && got < live; ++j) {
        e = hipMemcpy(buf.data(), pool->dev.slot_pos + (size_t)pages[j] * dms::kPage, dms::kPage * 4,
                      hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(e, "read slot positions");
        const int take = std::min(dms::kPage, live - got);
        std::memcpy(positions + got, buf.data(), (size_t)take * 4);
        got += take;
    }
    std::sort(positions, positions + live);
    g_err.clear();
    return DMS_OK;
}

dms_status dms_export_kv(dms_pool* pool, int32_t seq, int32_t layer, int32_t kv_head, int32_t cap,
                         int32_t* positions, void* k, void* v, float* k_scale, float* v_scale, int32_t* n) {
    if (!pool || !n) return fail(DMS_E_INVAL, "pool and n must not be NULL");
    const dms_pool_config& c = pool->cfg;
    if (seq < 0 || seq >= c.max_seqs || layer < 0 || layer >= c.n_layers || kv_head < 0 || kv_head >= c.n_kv_heads)
        return fail(DMS_E_INVAL, "(seq, layer, kv_head) out of range");
    hipError_t e = pool->sync();
    if (e != hipSuccess) return hip_fail(e, "synchronise");
    const int64_t gh = ((int64_t)seq * c.n_layers + layer) * c.n_kv_heads + kv_head;
    int32_t hs[dms::kHS];
    e = hipMemcpy(hs, pool->dev.hstate + gh * dms::kHS, sizeof(hs), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "read head state");
    const int live = hs[dms::kHsLive], np = hs[dms::kHsPages];
    *n = live;
    if (live > cap) return fail(DMS_E_INVAL, "output arrays too small");
    const bool fp8 = c.kv_format == DMS_KV_FP8_E4M3;
    const int D = c.head_dim;
    const size_t page_bytes = (size_t)dms::kPage * D * (fp8 ? 1 : 2);
    std::vector<int32_t> pages((size_t)np);
    if (np > 0) {
        e = hipMemcpy(pages.data(), pool->dev.ptable + gh * pool->layout.pages_per_head, (size_t)np * 4,
                      hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(e, "read page table");
    }
    // rows in slot order, then sorted by position
    std::vector<int32_t> pos((size_t)live);
    std::vector<uint8_t> kr((size_t)live * D * (fp8 ? 1 : 2)), vr(kr.size());
    std::vector<float> ksr((size_t)live, 1.f), vsr((size_t)live, 1.f);
    std::vector<uint8_t> kpg(page_bytes), vpg(page_bytes);
    std::vector<int32_t> spos(dms::kPage);
    std::vector<float> ksc(dms::kPage), vsc(dms::kPage);
    const char* kbase = reinterpret_cast<const char*>(pool->dev.kpages);
    const char* vbase = reinterpret_cast<const char*>(pool->dev.vpages);
    for (int j = 0; j < np && j * dms::kPage < live; ++j) {
        const size_t pg = (size_t)pages[j];
        e = hipMemcpy(spos.data(), pool->dev.slot_pos + pg * dms::kPage, dms::kPage * 4, hipMemcpyDeviceToHost);
        if (e == hipSuccess) e = hipMemcpy(kpg.data(), kbase + pg * page_bytes, page_bytes, hipMemcpyDeviceToHost);
        if (e == hipSuccess) e = hipMemcpy(vpg.data(), vbase + pg * page_bytes, page_bytes, hipMemcpyDeviceToHost);
        if (e == hipSuccess && fp8) e = hipMemcpy(ksc.data(), pool->dev.kscale + pg * dms::kPage, dms::kPage * 4,
                                                  hipMemcpyDeviceToHost);
        if (e == hipSuccess && fp8) e = hipMemcpy(vsc.data(), pool->dev.vscale + pg * dms::kPage, dms::kPage * 4,
                                                  hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(e, "read pages");
        for (int i = 0; i < dms::kPage && j * dms::kPage + i < live; ++i) {
            const size_t r = (size_t)j * dms::kPage + i;
            pos[r] = spos[i];
            for (int d = 0; d < D; ++d) {
                if (fp8) {  // K [D/16][64][16], V [4][D][16]
                    kr[r * D + d] = kpg[((size_t)(d / 16) * dms::kPage + i) * 16 + d % 16];
                    vr[r * D + d] = vpg[((size_t)(i / 16) * D + d) * 16 + i % 16];
                } else {    // K [D/8][64][8], V [8][D][8] (2-byte values)
                    std::memcpy(&kr[(r * D + d) * 2], &kpg[(((size_t)(d / 8) * dms::kPage + i) * 8 + d % 8) * 2], 2);
                    std::memcpy(&vr[(r * D + d) * 2], &vpg[(((size_t)(i / 8) * D + d) * 8 + i % 8) * 2], 2);
                }
            }
            if (fp8) {
                ksr[r] = ksc[i];
                vsr[r] = vsc[i];
            }
        }
    }
    std::vector<int> order((size_t)live);
    for (int r = 0; r < live; ++r) order[r] = r;
    std::sort(order.begin(), order.end(), [&](int x, int y) { return pos[x] < pos[y]; });
    const size_t row = (size_t)D * (fp8 ? 1 : 2);
    for (int i = 0; i < live; ++i) {
        const int r = order[i];
        if (positions) positions[i] = pos[r];
        if (k) std::memcpy(static_cast<char*>(k) + i * row, &kr[r * row], row);
        if (v) std::memcpy(static_cast<char*>(v) + i * row, &vr[r * row], row);
        if (k_scale) k_scale[i] = ksr[r];
        if (v_scale) v_scale[i] = vsr[r];
    }
    g_err.clear();
    return DMS_OK;
}

dms_status dms_seq_release(dms_pool* pool, int32_t seq, void* stream) {
    if (!pool) return fail(DMS_E_INVAL, "pool is NULL");
    if (seq < 0 || seq >= pool->cfg.max_seqs) return fail(DMS_E_INVAL, "seq out of range");
    pool->note(static_cast<hipStream_t>(stream));
    hipError_t e = dms::launch_seq_release(pool->dev, seq, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "release launch");
    if (++pool->rewrites % dms::kRunCacheRefill == 0) {
        e = dms::launch_page_cache_clear(pool->dev, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "page cache clear launch");
    }
    for (int l = 0; l < pool->cfg.n_layers; ++l) pool->position(seq, l) = -1;
    g_err.clear();
    return DMS_OK;
}

dms_status dms_timing_enable(dms_pool* pool, int32_t enable) {
    if (!pool) return fail(DMS_E_INVAL, "pool is NULL");
    pool->timing = enable != 0;
    g_err.clear();
    return DMS_OK;
}

dms_status dms_timing_read(dms_pool* pool, dms_timing* out) {
    if (!pool || !out) return fail(DMS_E_INVAL, "NULL argument");
    hipError_t e = pool->sync();
    if (e != hipSuccess) return hip_fail(e, "synchronise");
    std::memset(out, 0, sizeof(*out));
    // events come in start/stop pairs; group g of each call adds to acc[slot[g]]
    auto sum = [&](std::vector<hipEvent_t>& v, size_t per_call, const int* slot, double* const* acc,
                   int64_t* n) -> hipError_t {
        *n = (int64_t)(v.size() / per_call);
        for (size_t i = 0; i + per_call <= v.size(); i += per_call) {
            for (size_t g = 0; g < per_call / 2; ++g) {
                float t = 0;
                const hipError_t r = hipEventElapsedTime(&t, v[i + 2 * g], v[i + 2 * g + 1]);
                if (r != hipSuccess) return r;
                *acc[slot[g]] += t;
            }
        }
        for (hipEvent_t ev : v) (void)hipEventDestroy(ev);
        v.clear();
        return hipSuccess;
    };
    double* dacc[2] = {&out->decode_attend_ms, &out->decode_merge_ms};
    const int dslot[2] = {0, 1};
    e = sum(pool->events, 4, dslot, dacc, &out->decode_launches);
    double* pacc[2] = {&out->prefill_compact_ms, &out->prefill_attend_ms};
    const int pslot[2] = {0, 1};  // compaction with the V copy, attention
    if (e == hipSuccess) e = sum(pool->pevents, 4, pslot, pacc, &out->prefill_calls);
    double vcopy = 0;
    double* xacc[2] = {&vcopy, &out->extend_attend_ms};
    const int xslot[2] = {0, 1};
    if (e == hipSuccess) e = sum(pool->xevents, 4, xslot, xacc, &out->extend_calls);
    if (e != hipSuccess) return hip_fail(e, "event elapsed time");
    g_err.clear();
    return DMS_OK;
}

}  // extern "C"
