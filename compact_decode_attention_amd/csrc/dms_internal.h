// Internal layout of a DMS pool and the kernel launchers (not part of the ABI).
//
// Arena layout (every section 256-byte aligned).  The page arrays (K, V and FP8
// scales) hold NP = max_pages + n_kv_heads * pages_per_head pages: the shared
// pool, then pages_per_head scratch pages per kv head, where an extend call
// gathers the chunk's unmarked rows (xpage(h) below).  K/V pages of bf16 pools:
//   kpages   bf16 [NP][head_dim/8][64][8]          K, 16-byte dim chunks, key-major:
//                                                  chunk c of 64 consecutive slots is
//                                                  1 KB contiguous (lane = slot loads)
//   vpages   bf16 [NP][8][head_dim][8]             V, 8-slot blocks, dim-major: the
//                                                  16 bytes at (block, d) are 8
//                                                  consecutive slots of dim d
// K/V pages of FP8 pools (E4M3 codes, one fp32 scale per slot):
//   kpages   u8   [NP][head_dim/16][64][16]        K, 16 dims per 16-byte chunk, key-major
//   vpages   u8   [NP][4][head_dim][16]            V, 16-slot blocks, dim-major
//   kscale   f32  [NP][64], vscale f32 [NP][64]
//   q8       prefill scratch: the prompt quantised, codes u8 [2][max_positions]
//            [n_kv_heads][head_dim] (K, V) then scales f32 [2][max_positions][n_kv_heads]
//   slot_pos int32 [max_pages][64]                 position held by each slot
//   stack    int32 [max_pages]                     free pages, stack[0 .. top)
//   rcache   int32 [kRunCacheHeader + kRunCacheRows * kRunCacheRuns * 4]
//                                                  decode attention: the pool's epoch, then the
//                                                  pages of earlier small calls' blocks (directly
//                                                  before hstate; kRunCache* below)
//   hstate   int32 [heads][8]                      per-head record (kHs* below)
//   ptable   int32 [heads][pages_per_head]         page of slots 64j .. 64j+63
//   ring     int32 [heads][ring_len]               entry of position s at s % w:
//                                                  (slot << 1) | mark, -1 = none
//   partials f32   [max_items][part_stride(G, D)] split-K partials {m[G], l[G], pad, acc[G][D]},
//                                                  slot w + ch for wave w and call head ch
//   prefix   int32 [max_call_heads + 1]            first page of each call head on the page
//                                                  axis of the last decode launch
//   inv      int32 [n_kv_heads][max_positions]     prefill scratch: slot -> position
//   pcnt     int32 [n_kv_heads][max_positions]     prefill scratch: live tokens in [0, s]; extend
//                                                  calls: unmarked chunk rows in [0, r]
//   vt       bf16 [n_kv_heads][max_pos32/8][head_dim][8]
//                                                  prefill scratch: the prompt's V (FP8 pools:
//                                                  its codes as bf16) with 8 consecutive tokens
//                                                  per 16 bytes (max_pos32 = max_positions
//                                                  rounded up to 32)
//   vt16     fp16 [n_kv_heads][max_pos32/8][head_dim][8]
//                                                  bf16 pools: the same copy as fp16 values
//                                                  (read by the prefill attention while no V
//                                                  value is wide; FP8 pools: empty)
//   mbits    u32  [n_kv_heads][2 * ceil(max_positions / 64)]
//                                                  prefill scratch: bit j of word k is the
//                                                  mark of prompt position 32k + j
//   ctl      int32 [64]                            pool counters (kCtl* below)
// heads = max_seqs * n_layers * n_kv_heads, head id = (seq * n_layers + layer) * n_kv_heads + h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dms {

// Decode attention: blocks of kAttendWaves waves (one per SIMD), at most
// kAttendBlocksPerCU per compute unit and kMaxAttendBlocks per launch; the
// partials hold one slot per (wave, call head) pair that can occur.
// (Tuning constants; overridable at build time.)
#ifndef DMS_ATTEND_WAVES
#define DMS_ATTEND_WAVES 4
#endif
#ifndef DMS_ATTEND_BLOCKS_PER_CU
#define DMS_ATTEND_BLOCKS_PER_CU 1
#endif
#ifndef DMS_ATTEND_BLOCKS_PER_CU_FP8
#define DMS_ATTEND_BLOCKS_PER_CU_FP8 2
#endif
constexpr int kPage = 64;          // slots per page
constexpr int kAttendWaves = DMS_ATTEND_WAVES;
constexpr int kAttendBlocksPerCU = DMS_ATTEND_BLOCKS_PER_CU;          // bf16 pools
constexpr int kAttendBlocksPerCUFp8 = DMS_ATTEND_BLOCKS_PER_CU_FP8;   // FP8 pools (half the registers)
constexpr int kMaxAttendBlocks = 4096 / kAttendWaves;
// Split-K partial of G q heads: m[G], l[G], padding to 16 bytes, acc[G][D].
constexpr int part_acc_off(int g) { return (2 * g + 3) & ~3; }
constexpr int part_stride(int g, int d) { return part_acc_off(g) + g * d; }  // floats
constexpr int kMaxCallSeqs = 256;  // sequences per kernel launch (larger calls are split)
constexpr int kMaxCallHeads = 4032;  // heads per launch (4 ints of plan per head in LDS, < 64 KB)

// Size of the file-scope device array that holds the split-K partials and the
// page-axis prefix of dms_decode_step_static (per GPU, for the process's life).
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;

// ctl words
constexpr int kCtlTop = 0;    // free pages on the stack
constexpr int kCtlError = 1;  // sticky: nonzero once the page pool ran out
constexpr int kCtlVWide = 2;  // sticky: nonzero once a bf16 V value of magnitude >= 2^16 (or inf/NaN) was seen
constexpr int kCtlPosError = 3;  // sticky: nonzero once a decode or extend call ran past max_positions (the
                                 // device's position counters decide; tokens past the limit are dropped)

// Page cache of the decode attention's calls of one layer of one sequence:
// a header of kRunCacheHeader ints, whose first is the pool's epoch (advanced by
// every release and prefill: a head's page-table entries below its page count
// change only when a release frees them), then kRunCacheRows rows (the first
// head of a call of one sequence picks the row) of kRunCacheRuns entries {page
// id, global head, page index, epoch}, one per wave group's page (block b's
// first group: entry b; its second: entry b + grid).  The arena places it
// directly before the head records, so the attention finds it from the
// head-record pointer it gets in registers.
constexpr int kRunCacheRows = 64;
constexpr int kRunCacheRuns = 1024;
constexpr int kRunCacheHeader = 64;
constexpr size_t kRunCacheBytes = ((size_t)kRunCacheHeader + (size_t)kRunCacheRows * kRunCacheRuns * 4) * 4;
static_assert(kRunCacheBytes % 256 == 0, "the head records follow the cache without padding");

// Nonzero if one of the two bf16 values in w has magnitude >= 2^16, is inf or
// is NaN (exponent field >= 143): such a value has no fp16 counterpart.
__device__ __forceinline__ uint32_t bf16x2_wide(uint32_t w) {
    return ((w & 0x7fffu) >= 0x4780u) | ((w & 0x7fff0000u) >= 0x47800000u);
}
__device__ __forceinline__ uint32_t bf16x8_wide(uint4 u) {
    return bf16x2_wide(u.x) | bf16x2_wide(u.y) | bf16x2_wide(u.z) | bf16x2_wide(u.w);
}

// 8 bf16 values as 8 fp16 values: exact for |v| < 65536 down to 2^-17 (below
// that, fp16 subnormal spacing 2^-24).  Used only while no stored V value is
// wide (the kCtlVWide flag is clear).
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 u) {
    typedef _Float16 f16x2_v __attribute__((ext_vector_type(2)));
    auto cv = [](uint32_t w) -> uint32_t {
        const f16x2_v x = {(_Float16)__uint_as_float(w << 16), (_Float16)__uint_as_float(w & 0xffff0000u)};
        return __builtin_bit_cast(uint32_t, x);
    };
    return make_uint4(cv(u.x), cv(u.y), cv(u.z), cv(u.w));
}

// Per-head record, 8 int32:
//   [0] n_live       tokens held, in slots 0 .. n_live-1
//   [1] n_pages      pages in the head's page table
//   [2] position     position of the next token
//   [3] e_next       slot of the token that expires when `position` is appended
//                    (position - w, if it was marked), or -1
//   [4..7]           unused
constexpr int kHS = 8;
constexpr int kHsLive = 0, kHsPages = 1, kHsPos = 2, kHsExp = 3;  // [0..3] is one 16-byte load

struct PoolDev {
    uint16_t* kpages;  // bf16 pools; FP8 pools hold bytes here (see kp8 / vp8)
    uint16_t* vpages;
    float* kscale;     // FP8 pools only
    float* vscale;
    uint8_t* q8;       // FP8 pools only: prefill scratch
    int32_t* slot_pos;
    int32_t* stack;
    int32_t* hstate;
    int32_t* ptable;
    int32_t* ring;
    float* partials;
    int32_t* prefix;
    int32_t* inv;
    int32_t* pcnt;
    uint16_t* vt;
    uint16_t* vt16;    // bf16 pools only
    uint32_t* mbits;
    int32_t* rcache;
    int32_t* ctl;
    int64_t max_pages;
    int32_t n_layers, n_q_heads, n_kv_heads, head_dim;
    int32_t window, ring_len, pages_per_head, max_positions, max_pos32;
    int32_t max_items;
    int32_t fp8;       // kv_format == DMS_KV_FP8_E4M3
    int32_t logit_ch;  // channel of K holding the eviction logit, or -1: the logits input
    float scale_log2;  // softmax scale * log2(e): scores are kept in base-2 units
    __host__ __device__ uint8_t* kp8() const { return reinterpret_cast<uint8_t*>(kpages); }
    __host__ __device__ uint8_t* vp8() const { return reinterpret_cast<uint8_t*>(vpages); }
    // prefill scratch of an FP8 pool: codes of tensor x (0 = K, 1 = V) and their scales
    __host__ __device__ uint8_t* q8_codes(int x) const {
        return q8 + (size_t)x * max_positions * n_kv_heads * head_dim;
    }
    __host__ __device__ float* q8_scales(int x) const {
        return reinterpret_cast<float*>(q8 + (size_t)2 * max_positions * n_kv_heads * head_dim) +
               (size_t)x * max_positions * n_kv_heads;
    }
    // mark bits of kv head h's prompt positions (prefill scratch)
    __host__ __device__ uint32_t* mbits_of(int h) const {
        return mbits + (size_t)h * ((max_positions + 63) / 64) * 2;
    }
    // first scratch page of kv head h (extend calls: the chunk's unmarked rows, in order)
    __host__ __device__ int xpage(int h) const { return (int)max_pages + h * pages_per_head; }
};

// ---- raw buffer loads ----------------------------------------------------------
// Resource over [base, base + bytes): loads beyond it return 0 and touch no
// memory, so a dead request is a load through a zero-size resource.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Streaming loads of K/V pages: the non-temporal cache policy (nt, bit 1 of the
// buffer instruction's cache-policy operand on gfx950), which a read-once
// stream of pages larger than the caches wants.
#ifndef DMS_KV_AUX
#define DMS_KV_AUX 2
#endif
__device__ __forceinline__ uint4 buffer_load16_stream(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, DMS_KV_AUX);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    return make_uint2(v[0], v[1]);
}

__device__ __forceinline__ float buffer_load4f(__amdgpu_buffer_rsrc_t r, int voff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}

__device__ __forceinline__ int buffer_load4i(__amdgpu_buffer_rsrc_t r, int voff) {
    return (int)__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
}

__device__ __forceinline__ uint32_t buffer_load2(__amdgpu_buffer_rsrc_t r, int voff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0);
}

// ---- OCP FP8 E4M3 (FP8 pools) -------------------------------------------------
// Code of x: the finite E4M3 value nearest to x, ties to the code with an even
// last bit, +-448 beyond the largest finite value, the sign kept (so -0 and
// values rounding to zero from below give 0x80); NaN gives 0x7f.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return 0x7fu;
    const float af = __uint_as_float(a);
    if (af >= 448.0f) return sign | 0x7eu;
    if (af < 0.015625f) {  // below 2^-6: multiples of 2^-9 (code = multiple, 8 = 2^-6)
        return sign | (uint32_t)__builtin_rintf(af * 512.0f);
    }
    // normal: round the fp32 mantissa to 3 bits, nearest-even (a carry moves the exponent)
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
    return sign | (((r >> 3) - 120u) << 3) | (r & 7u);
}

// Value of an E4M3 code (NaN codes are never stored).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    return (c & 0x80u) ? -mag : mag;
}

// Two codes (bytes 0-1 or 2-3 of w) as a bf16 pair (low half = the lower byte):
// exact, every E4M3 value is a bf16 value.
__device__ __forceinline__ uint32_t fp8x2_lo(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
__device__ __forceinline__ uint32_t fp8x2_hi(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}
// 8 codes as 8 bf16 values
__device__ __forceinline__ uint4 fp8x8_bf16(uint2 w) {
    return make_uint4(fp8x2_lo(w.x), fp8x2_hi(w.x), fp8x2_lo(w.y), fp8x2_hi(w.y));
}

// Row scale: amax / 448 in fp32 (1 for an all-zero row); codes are
// e4m3_encode(x / scale) with the fp32 quotient.
__device__ __forceinline__ float e4m3_row_scale(float amax) { return amax > 0.f ? amax / 448.0f : 1.0f; }

// Eviction logit of input row r (token s of a prefill; call row of a decode)
// and kv head h: the logits input, or one channel of the row's K.
__device__ __forceinline__ float eviction_logit(const PoolDev& P, const float* logits, const uint16_t* k, size_t r,
                                                int h) {
    if (P.logit_ch >= 0)
        return __uint_as_float((uint32_t)k[(r * P.n_kv_heads + h) * P.head_dim + P.logit_ch] << 16);
    return logits[r * P.n_kv_heads + h];
}

struct DecodeArgs {
    PoolDev pool;
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* logits;
    uint16_t* out;
    int32_t n_seqs_total;  // sequences of the whole call (row stride of the inputs)
    int32_t seq_base;      // first sequence of this launch within the call
    int32_t n_seqs;        // sequences in this launch
    int32_t layer0, n_layers;
    int32_t n_call_heads;  // n_layers * n_seqs * n_kv_heads
    int32_t n_waves;       // waves of the attention kernel's grid
    int32_t seq_ids[kMaxCallSeqs];
};

struct PrefillArgs {
    PoolDev pool;
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* logits;
    uint16_t* out;
    int32_t seq, layer, n_tokens;
    int32_t t0;  // extend calls: position of input row 0 (the head's position counter); prefill: 0
};

// ---------------------------------------------------------------------------
// prompt V -> vt[h][s/8][d][8] (8 consecutive tokens of one dim per 16 bytes),
// zero beyond the prompt up to the next multiple of 32.  FP8 pools: the values
// of the prompt V's codes (exact in bf16; the row scales are applied to P).
// bf16 pools: a V value without an fp16 counterpart sets the pool's sticky
// kCtlVWide flag, which keeps the attention on its bf16 path.
// ---------------------------------------------------------------------------
// Rows s0 .. s0+63 of kv head h, by the 256 threads of a block (all of them
// call it together: it synchronises the block once), staged in s_v.  With
// V16 (bf16 pools, prefill) the copy is also written as fp16 values to vt16.
template <int D, bool F8, bool V16 = false>
__device__ __forceinline__ void vt_rows(const PrefillArgs& a, int s0, int h, uint16_t (*s_v)[D + 8]) {
    const PoolDev& P = a.pool;
    const int tid = threadIdx.x;
    const int T = a.n_tokens, hkv = P.n_kv_heads;
    const int T32 = (T + 31) / 32 * 32;
    constexpr int NC = D / 8;
    uint32_t wide = 0;
    for (int u = tid; u < 64 * NC; u += 256) {
        const int j = u / NC, cc = u - j * NC;
        const int s = s0 + j;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (s < T) {
            if constexpr (F8)
                val = fp8x8_bf16(*reinterpret_cast<const uint2*>(P.q8_codes(1) + ((size_t)s * hkv + h) * D + cc * 8));
            else
                val = *reinterpret_cast<const uint4*>(a.v + ((size_t)s * hkv + h) * D + cc * 8);
        }
        if (!F8) wide |= bf16x8_wide(val);
        *reinterpret_cast<uint4*>(&s_v[j][cc * 8]) = val;
    }
    if (wide) atomicOr(&P.ctl[kCtlVWide], 1);
    __syncthreads();
    uint16_t* vt = P.vt + (size_t)h * (P.max_pos32 / 8) * D * 8;
    for (int u = tid; u < 8 * D; u += 256) {
        const int b = u / D, d = u - b * D;
        const int blk = s0 / 8 + b;
        if (blk * 8 >= T32) continue;
        uint32_t w4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w4[i] = (uint32_t)s_v[8 * b + 2 * i][d] | ((uint32_t)s_v[8 * b + 2 * i + 1][d] << 16);
        const uint4 unit = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        *reinterpret_cast<uint4*>(vt + ((size_t)blk * D + d) * 8) = unit;
        if constexpr (V16 && !F8)
            *reinterpret_cast<uint4*>(P.vt16 + (size_t)h * (P.max_pos32 / 8) * D * 8 + ((size_t)blk * D + d) * 8) =
                bf16x8_to_f16x8(unit);
    }
}


// ev (optional, 4 events): start/stop of the attention kernel and of the merge
// kernel, taken by the kernel dispatches (execution time only)
hipError_t launch_decode(const DecodeArgs& a, int grid, hipStream_t s, hipEvent_t* ev);
// blocks of the attention kernel one compute unit holds at once for this call (0: does not fit)
int decode_blocks_per_cu(const DecodeArgs& a);
// start / stop (optional): taken by the first and the last kernel dispatch.
// with_vt: the compaction launch also copies the prompt V for the attention's band
hipError_t launch_prefill_compact(const PrefillArgs& a, bool with_vt, hipStream_t s, hipEvent_t start,
                                  hipEvent_t stop);
// after launch_prefill_compact with with_vt; ev (optional, 2 events): start/stop of
// the attention kernel
hipError_t launch_prefill_attend(const PrefillArgs& a, hipStream_t s, hipEvent_t* ev);
// extend calls (several new tokens of one (seq, layer) appended to its store):
// the prompt-side kernels of the chunk (FP8: quantisation; with output: one
// preparation kernel -- V copy, expiry rows of the stored slots, the chunk's
// unmarked rows gathered into the scratch pages -- and the attention of the
// chunk's queries over the store and the chunk), then the slot assignment, page
// allocation, ring and record, then the writes
hipError_t launch_extend(const PrefillArgs& a, bool with_out, hipStream_t s, hipEvent_t* ev);
// ev (optional, 4 events): start/stop of the preparation kernel, then of the attention kernel
hipError_t launch_extend_attend(const PrefillArgs& a, hipStream_t s, hipEvent_t* ev);
hipError_t launch_seq_release(const PoolDev& p, int32_t seq, hipStream_t s);
// Every entry of the decode attention's page cache set to -1 (its global head
// then matches no head): at pool creation, and every kRunCacheRefill releases
// and prefills, so that no entry outlives 2^30 advances of the 32-bit epoch.
hipError_t launch_page_cache_clear(const PoolDev& p, hipStream_t s);
constexpr uint64_t kRunCacheRefill = (uint64_t)1 << 30;
int device_cu_count();
// Device address of the static decode scratch (kStaticScratchBytes) on the
// current device, looked up once per device.
hipError_t static_scratch_address(void** out);

}  // namespace dms
