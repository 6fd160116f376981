/*
 * dms.h -- C ABI of the DMS compact-KV decode library for MI355X (gfx950).
 *
 * Dynamic Memory Sparsification (DMS) lets every attention head decide, per
 * token, whether to keep that token's key/value or to evict it; an evicted
 * token stays readable for a delay window of w further steps and is then
 * dropped (delayed eviction).  Sources: "NVIDIA veroeffentlicht
 * Qwen3-8B-DMS-8x ..." (mindverse news page), section "Dynamic Memory
 * Sparsification (DMS): Eine innovative Loesung"; "Nvidia DMS: szhatie pamyati
 * LLM v 8 raz" (stiva.ai), sections on the keep/evict signal and on delayed
 * eviction.  The FastDMS announcement ("FastDMS: vLLM BF16/FP8 ... 6.4x KV
 * cache", molayo1419.me) describes the compact store this library keeps: the
 * slots of evicted tokens are physically reclaimed, so token counts vary per
 * layer and per head and the saving shows up in real device memory (its
 * memory table and its "What's the catch?" table, PagedAttention row).
 *
 * Visibility rule (the plain reading of those pages, stated once here):
 *   token s is marked for eviction iff its logit is > 0 (strictly);
 *   token s is visible to the query at position t iff s <= t and
 *   (s is unmarked or t < s + w).
 * So a marked token is seen by the w queries s .. s+w-1, its own included.
 * A window w >= max_positions never expires anything (the FastDMS quality
 * method's "eviction disabled" reference is a 1M-token window).
 *
 * Conventions shared by every entry point
 *  - All tensor arguments are device pointers owned by the caller; they must
 *    stay valid until the work enqueued on `stream` has finished.  bf16 values
 *    are passed as their 16-bit patterns.  Rows are contiguous, 16-byte aligned.
 *    K and V values must be finite (bf16 and FP8 pools alike): a query whose
 *    key tile holds a non-finite value it does not see can still come out
 *    non-finite (a zero weight times an infinite value).
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls
 *    enqueue kernels and return without waiting, except dms_pool_create,
 *    dms_pool_destroy, dms_query_stats, dms_export_live, dms_export_kv and
 *    dms_timing_read, which first wait for the streams the pool's calls were
 *    enqueued on (not for the whole device).
 *  - Errors found on the host are returned at once and nothing is enqueued.
 *    Device-side failures set sticky flags that the next synchronising call
 *    returns: DMS_E_CAPACITY when the shared page pool ran out (the token or
 *    chunk that needed a page is dropped), DMS_E_STATE when a decode or extend
 *    call ran past max_positions (the tokens past it are dropped).
 *  - HIP graph capture: dms_decode_step, dms_extend, dms_prefill and
 *    dms_seq_release may be captured.  The positions live in the device's
 *    per-head records, which every replay advances and every kernel reads; the
 *    host keeps a copy for its argument checks, which replays do not advance
 *    and which dms_query_stats refreshes from the device.  So a check the host
 *    makes at call time may pass on a stale copy; the kernels check again
 *    (the sticky DMS_E_STATE above).  Work replayed on a stream the pool's
 *    calls never used must be finished by the caller before a synchronising
 *    call.
 *  - Error text for the last failing call on the calling thread:
 *    dms_last_error().  No C++ exception crosses this interface.
 *  - A pool is not thread-safe; use it from one host thread and order all of
 *    its work on one stream (or synchronise between streams).
 *  - The library never allocates device memory: the caller hands over one
 *    arena of dms_pool_bytes() bytes and keeps ownership of it.
 */
#ifndef DMS_H_
#define DMS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dms_status;
enum {
    DMS_OK = 0,
    DMS_E_INVAL = -1,     /* bad argument, shape or pointer */
    DMS_E_NOMEM = -2,     /* arena smaller than dms_pool_bytes() */
    DMS_E_CAPACITY = -3,  /* the shared page pool ran out (device-side, sticky) */
    DMS_E_STATE = -4,     /* call not valid in the pool's current state */
    DMS_E_HIP = -5        /* a HIP runtime call failed */
};

/* Slots per page of the compact store.  Fixed: one page is one 64-lane
 * wavefront's worth of keys. */
#define DMS_PAGE_SLOTS 64

/* Storage format of K and V in the compact store (dms_pool_config.kv_format).
 *  DMS_KV_BF16      K and V rows as given (2 bytes per value).
 *  DMS_KV_FP8_E4M3  every (token, kv head) row of K, and of V, is stored as
 *                   OCP FP8 E4M3 codes (1 byte per value) with one fp32 scale:
 *                   scale = amax / 448 in fp32 (amax = the row's largest |x|;
 *                   1 for an all-zero row), code = the finite E4M3 value nearest
 *                   to x / scale (fp32 quotient; ties to the even code; beyond
 *                   +-448 it is +-448), and attention, in prefill and decode,
 *                   reads value(code) * scale in place of x.  Halves the bytes
 *                   decode streams.  (The FastDMS announcement on molayo1419.me
 *                   compares against FP8 KV caches; the format follows the OCP
 *                   8-bit floating point specification.)  K/V inputs must be
 *                   finite. */
#define DMS_KV_BF16 0
#define DMS_KV_FP8_E4M3 1

/* Where the eviction logit of a (token, kv head) comes from
 * (dms_pool_config.logit_source).
 *  DMS_LOGITS_INPUT      the caller's logits array (prefill and decode calls).
 *  DMS_LOGITS_K_CHANNEL  channel logit_channel of the token's K row for that kv
 *                        head: one existing neuron of the attention layer emits
 *                        the keep/evict signal ("NVIDIA veroeffentlicht
 *                        Qwen3-8B-DMS-8x ..." news page, section "Technische
 *                        Details und Implementierung"; stiva.ai "Nvidia DMS ...",
 *                        section on the model managing its own memory).  The
 *                        channel keeps its value in attention; the logits
 *                        argument of the calls is ignored and may be NULL.
 *                        K arrives after positional encoding, so a model with
 *                        rotary embeddings must carry the logit in a channel
 *                        the rotation leaves alone (past its rotary dims, or
 *                        written after the rotation): a rotated channel mixes
 *                        with its partner and would vary with position. */
#define DMS_LOGITS_INPUT 0
#define DMS_LOGITS_K_CHANNEL 1

typedef struct dms_pool dms_pool; /* opaque; owned by the library */

typedef struct {
    int32_t n_layers;      /* >= 1 */
    int32_t n_q_heads;     /* multiple of n_kv_heads; n_q_heads / n_kv_heads in {1,2,4,8} */
    int32_t n_kv_heads;    /* >= 1 */
    int32_t head_dim;      /* 64 or 128 */
    int32_t window;        /* delay window w >= 1 */
    int32_t max_seqs;      /* sequences sharing the pool's one page allocator */
    int32_t max_positions; /* most tokens (prompt + generated) one sequence may hold */
    int32_t page_slots;    /* 0 or DMS_PAGE_SLOTS */
    int64_t max_pages;     /* pages in the shared pool; each page holds 64 slots of K and V */
    float softmax_scale;   /* 0 => 1/sqrt(head_dim) */
    uint32_t page_order_seed; /* 0: pages are handed out in ascending order; otherwise
                                 in a seeded shuffled order (physical placement must
                                 not change any result) */
    int32_t kv_format;     /* DMS_KV_BF16 (0) or DMS_KV_FP8_E4M3 */
    int32_t logit_source;  /* DMS_LOGITS_INPUT (0) or DMS_LOGITS_K_CHANNEL */
    int32_t logit_channel; /* DMS_LOGITS_K_CHANNEL: channel in [0, head_dim); else 0 */
    int32_t reserved[1];   /* must be 0 */
} dms_pool_config;

/* Bytes of device memory (the arena) a pool with this configuration needs, or 0
 * if the configuration is invalid (dms_last_error() says why).  Besides the
 * max_pages shared pages it holds the head records, page tables, window rings,
 * split-K partials and the prefill / extend scratch, which includes
 * ceil(max_positions / 64) scratch pages per kv head (max_pages plus these must
 * stay below 2^31).  (The store is paged per (layer, kv head) with variable
 * token counts and pages handed back one by one: the FastDMS announcement on
 * molayo1419.me, "What's the catch?" table, PagedAttention row.) */
size_t dms_pool_bytes(const dms_pool_config* cfg);

/* Create a pool inside the caller's arena (device memory, >= dms_pool_bytes()
 * bytes, 256-byte aligned).  Clears the arena and fills the page free list on
 * `stream`, then synchronises.  The arena stays owned by the caller and must
 * outlive the pool.  (A compact store whose evicted slots are reclaimed, one
 * shared page allocator for all sequences: the FastDMS announcement on
 * molayo1419.me, release paragraph and "What's the catch?" table, PagedAttention
 * row.)  Errors: DMS_E_INVAL (configuration, NULL or misaligned arena),
 * DMS_E_NOMEM (arena too small), DMS_E_HIP. */
dms_status dms_pool_create(const dms_pool_config* cfg, void* arena, size_t arena_bytes,
                           void* stream, dms_pool** out);

/* Wait for the pool's streams and free the host-side handle (not the arena,
 * which the caller owns). */
dms_status dms_pool_destroy(dms_pool* pool);

/* Prefill: the first n_tokens tokens (positions 0 .. n_tokens-1) of one
 * (sequence, layer).  Marks every token from its logit, stores exactly the
 * tokens visible to the last position n_tokens-1 in the compact store (unmarked
 * tokens older than the window, plus the last min(n_tokens, w) tokens) in
 * position order, and records the marks of the window so that decode can
 * expire them on time.  When out is not NULL it also writes the masked causal
 * attention output of every position (query t sees the keys visible to t).
 *   q      bf16 [n_tokens][n_q_heads][head_dim]  (may be NULL when out is NULL)
 *   k, v   bf16 [n_tokens][n_kv_heads][head_dim]
 *   logits fp32 [n_tokens][n_kv_heads] (ignored, may be NULL, with
 *          DMS_LOGITS_K_CHANNEL)
 *   out    bf16 [n_tokens][n_q_heads][head_dim] or NULL
 * q and k arrive after any positional encoding.  Returns DMS_E_STATE if this
 * (seq, layer) already holds tokens (release the sequence first), DMS_E_INVAL
 * for out-of-range arguments or NULL inputs.  (Masks from delayed eviction:
 * "NVIDIA veroeffentlicht Qwen3-8B-DMS-8x ..." news page, section "Dynamic
 * Memory Sparsification (DMS): Eine innovative Loesung"; prefill throughput is
 * one of the two columns of the FastDMS announcement's speed table, on
 * molayo1419.me.)
 * Precision: fp32 accumulation; each output is within 2e-3 + 1e-2 |ref| of the
 * masked attention over the inputs (FP8 pools: over value(code) * scale).  A
 * bf16 pool that has seen a V value of magnitude 2^16 or more (in any prompt,
 * chunk or decode step) keeps its prefill and extend attention on a slower
 * path for good; the bound is the same. */
dms_status dms_prefill(dms_pool* pool, int32_t seq, int32_t layer, int32_t n_tokens,
                       const void* q, const void* k, const void* v, const float* logits,
                       void* out, void* stream);

/* One decode step for n_seqs sequences over layers layer0 .. layer0+n_layers-1.
 * For every (layer, sequence, kv head), in this order: mark the new token from
 * its logit; expire the token whose delay window has just run out (position
 * t-w, if it was marked) and put its slot on the free list; take a slot for the
 * new token from the free list or the end of the store (a fresh page from the
 * shared pool when needed); write the new K/V; and attend the head's query
 * group over every live token, the new one included.
 *   seq_ids host int32 [n_seqs], distinct, each already prefilled on every
 *           layer of the call
 *   q       bf16 [n_layers][n_seqs][n_q_heads][head_dim]
 *   k, v    bf16 [n_layers][n_seqs][n_kv_heads][head_dim]
 *   logits  fp32 [n_layers][n_seqs][n_kv_heads] (ignored, may be NULL, with
 *           DMS_LOGITS_K_CHANNEL)
 *   out     bf16 [n_layers][n_seqs][n_q_heads][head_dim]
 * Each (seq, layer) keeps its own position counter; the new token's position
 * is that counter.  A model calls this once per layer (n_layers = 1); a caller
 * whose layers have independent inputs may step several layers in one call.
 * Errors: DMS_E_INVAL (arguments), DMS_E_STATE (a (seq, layer) not prefilled or
 * at max_positions by the host's count), DMS_E_HIP; a page-pool exhaustion or a
 * position past max_positions found on the device is reported by the next
 * synchronising call.  (The step order is the delayed eviction of "NVIDIA
 * veroeffentlicht Qwen3-8B-DMS-8x ..." news page, section "Dynamic Memory
 * Sparsification (DMS): Eine innovative Loesung", and of stiva.ai "Nvidia DMS
 * ...", section "Klyuchevoe izobretenie: delayed eviction": a marked token
 * stays readable for w steps, its own included, then its slot is reclaimed.) */
dms_status dms_decode_step(dms_pool* pool, int32_t n_seqs, const int32_t* seq_ids,
                           int32_t layer0, int32_t n_layers, const void* q, const void* k,
                           const void* v, const float* logits, void* out, void* stream);

/* dms_decode_step for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, same kernels and results bit for bit; the call allocates nothing
 * (no device memory, no host containers, no timing events even when timing is
 * enabled).  Its split-K partials and page-axis prefix live in one file-scope
 * device array of 16 MiB per GPU (held until the process ends), not in the
 * pool's arena.  A call whose largest launch needs more returns DMS_E_INVAL
 * (that is (attention waves + call heads) x (8 + G x head_dim) x 4 bytes, G =
 * n_q_heads / n_kv_heads: about 2.8 MB for 36 layers x 8 kv heads at G = 4,
 * D = 128; up to 256 sequences x n_layers x n_kv_heads heads per launch).
 * Nothing in the array needs clearing: each launch writes what it reads.
 * Every call on one GPU shares that GPU's array, across all pools: calls that
 * overlap on one GPU (other streams, other pools, other threads) race. */
dms_status dms_decode_step_static(dms_pool* pool, int32_t n_seqs, const int32_t* seq_ids,
                                  int32_t layer0, int32_t n_layers, const void* q, const void* k,
                                  const void* v, const float* logits, void* out, void* stream);

/* Append n_tokens new tokens to one (sequence, layer) that already holds
 * tokens, at positions t .. t+n_tokens-1 (t = its position counter): the same
 * result as n_tokens decode steps of that (seq, layer), in position order (for
 * each token: mark it from its logit, expire the token w positions earlier if
 * that one was marked and reuse its slot, else take the next slot; attend over
 * the live tokens at its own position, itself included), with every token's
 * inputs given at once, as in chunked prefill or in the check of several
 * proposed tokens.  Several expiries per call are the point of this entry: a
 * slot can change hands several times within one call.  (Delayed eviction:
 * "NVIDIA veroeffentlicht Qwen3-8B-DMS-8x ..." news page, section "Dynamic
 * Memory Sparsification (DMS): Eine innovative Loesung"; stiva.ai "Nvidia DMS
 * ...", section on delayed eviction; slots of evicted tokens reclaimed in a
 * compact store: the FastDMS announcement on molayo1419.me, "What's the catch?"
 * table.)
 *   q      bf16 [n_tokens][n_q_heads][head_dim]  (may be NULL when out is NULL)
 *   k, v   bf16 [n_tokens][n_kv_heads][head_dim]
 *   logits fp32 [n_tokens][n_kv_heads] (ignored, may be NULL, with
 *          DMS_LOGITS_K_CHANNEL)
 *   out    bf16 [n_tokens][n_q_heads][head_dim] or NULL (no attention)
 * Returns DMS_E_STATE if the (seq, layer) was not prefilled or the chunk would
 * run past max_positions.  Uses the pool's prefill scratch: calls that touch
 * one pool must be ordered (one stream). */
dms_status dms_extend(dms_pool* pool, int32_t seq, int32_t layer, int32_t n_tokens, const void* q,
                      const void* k, const void* v, const float* logits, void* out, void* stream);

typedef struct {
    int64_t live_slots;           /* tokens held, summed over the queried layers and kv heads */
    int64_t kv_bytes_live;        /* live_slots * bytes per slot: 2 (K,V) * head_dim * 2 bytes
                                     (bf16), or 2 * (head_dim + 4) bytes (FP8 codes + scales) */
    int64_t kv_bytes_allocated;   /* pages held * 64 slots * bytes per slot */
    int64_t kv_bytes_dense_equiv; /* what a store keeping every token would hold */
    int64_t pages_used;           /* pages held by the queried sequence(s) */
    int64_t pages_free;           /* free pages in the whole pool */
    int64_t workspace_bytes;      /* arena bytes outside the K/V pages (tables, split-K partials) */
    int32_t position;             /* seq >= 0: the next position of layer 0; -1 if not prefilled */
    int32_t device_error;         /* sticky device status: DMS_OK or DMS_E_CAPACITY */
} dms_stats;

/* Wait for the pool's streams and report the store's size for one sequence
 * (seq >= 0) or for all sequences (seq = -1).  live_per_layer_head, when not
 * NULL, is a host array [n_layers][n_kv_heads] (seq >= 0 only) that receives the
 * live counts.  The byte figures are the memory the store really holds, as the
 * FastDMS announcement's memory table reports KV memory (molayo1419.me):
 * live bytes follow the live tokens, allocated bytes the whole pages behind
 * them.  Also refreshes the host's copy of the positions from the device.
 * Returns DMS_E_CAPACITY or DMS_E_STATE (after filling *out) if a sticky
 * device flag is set. */
dms_status dms_query_stats(dms_pool* pool, int32_t seq, dms_stats* out,
                           int32_t* live_per_layer_head);

/* Wait for the pool's streams and list the positions of the tokens one (seq,
 * layer, kv_head) holds, ascending, into the host array positions[cap]; *n
 * receives the count (DMS_E_INVAL if it exceeds cap).  The list is what a
 * comparison with the eviction-disabled reference needs (the FastDMS
 * announcement's quality-method paragraph, molayo1419.me: the same engine with
 * a 1M-token window keeps every token). */
dms_status dms_export_live(dms_pool* pool, int32_t seq, int32_t layer, int32_t kv_head,
                           int32_t* positions, int32_t cap, int32_t* n);

/* Wait for the pool's streams and copy what one (seq, layer, kv_head) stores,
 * row by row in ascending position order, to host arrays (eviction decides
 * first and FP8 quantisation applies to what stays: the FastDMS announcement's
 * quality-method paragraph, molayo1419.me):
 *   positions int32 [cap]
 *   k, v      [cap][head_dim]: bf16 bits (bf16 pools) or E4M3 codes (FP8 pools)
 *   k_scale, v_scale fp32 [cap]: the row scales (FP8 pools), 1 (bf16 pools)
 * Any output pointer may be NULL to skip it.  *n receives the row count
 * (DMS_E_INVAL if it exceeds cap). */
dms_status dms_export_kv(dms_pool* pool, int32_t seq, int32_t layer, int32_t kv_head, int32_t cap,
                         int32_t* positions, void* k, void* v, float* k_scale, float* v_scale, int32_t* n);

/* Return every page of a sequence to the shared pool and forget its tokens on
 * all layers (enqueued on `stream`).  The sequence may then be prefilled again.
 * Another sequence may get these pages next; their old rows are never read as
 * live tokens (slots past a head's live count are cleared when a page is
 * taken).  (Pages handed back one by one: the FastDMS announcement,
 * "What's the catch?" table, PagedAttention row.) */
dms_status dms_seq_release(dms_pool* pool, int32_t seq, void* stream);

/* Kernel timing for measurement.  While enabled, the kernels of every decode
 * launch and of every prefill that produces an output are dispatched with HIP
 * start/stop events that the dispatches themselves record, so the times cover
 * kernel execution only.  dms_timing_read waits for the pool's streams, adds up
 * the times of everything recorded since the last read (milliseconds), counts
 * the calls, and releases the events.  Disabled by default.  (Decode and
 * prefill throughput are what the FastDMS announcement's speed table reports.) */
typedef struct {
    double decode_attend_ms;   /* split-K attention kernels */
    double decode_merge_ms;    /* merge + evict/append kernels */
    double prefill_compact_ms; /* mark scan + compaction kernels and the prompt-V copy */
    double prefill_attend_ms;  /* masked causal attention (MFMA) kernels */
    int64_t decode_launches;
    int64_t prefill_calls;     /* prefills that produced an output */
    double extend_attend_ms;   /* attention (MFMA) kernels of extend calls with output */
    int64_t extend_calls;      /* extend calls that produced an output */
} dms_timing;
dms_status dms_timing_enable(dms_pool* pool, int32_t enable);
dms_status dms_timing_read(dms_pool* pool, dms_timing* out);

/* Text of the last error on the calling thread ("" if none). */
const char* dms_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DMS_H_ */
