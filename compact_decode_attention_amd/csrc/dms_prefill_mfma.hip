// Masked causal prefill attention on MFMA (gfx950, v_mfma_f32_32x32x16_bf16 and
// _f16).
//
// Query t sees key s iff s <= t and (s is unmarked or t < s + w) (DMS delayed
// eviction: "NVIDIA veroeffentlicht Qwen3-8B-DMS-8x ..." news page, section
// "Dynamic Memory Sparsification (DMS): Eine innovative Loesung"; stiva.ai
// "Nvidia DMS ...", section on delayed eviction).  For a tile of 32 queries
// starting at t0 the keys split in two:
//   far field  s <= t0 - w: visible iff unmarked, for every query of the tile.
//              These are exactly the first U = #live[0, t0-w] slots of the
//              compacted store the compaction kernels just wrote (unmarked
//              tokens older than the window, in position order), so the far
//              field is a dense, unmasked contraction over pool pages.
//   band       t0 - w < s <= t0 + 31: taken from the prompt K and from a copy of
//              the prompt V with 8 consecutive tokens per 16 bytes, masked per
//              (query, key) pair.
//
// Each wave owns one q head and the tile's 32 queries and computes, per tile of
// 32 keys, S^T = K Q^T (rows = keys, columns = queries), so that the softmax
// over keys of one query is a reduction over a lane's 16 accumulators plus one
// exchange with lane ^ 32.  K rows are fed with bits 2 and 3 of the key index
// swapped; with that order the MFMA accumulator layout of P^T is exactly the
// B-operand layout of the next MFMA, O^T += V^T P^T, so P never leaves
// registers.  V^T's A operand (8 consecutive keys of one dim) is one 16-byte
// unit of the dim-major V page (far field) or of the V copy (band).
// The waves of a block are the G q heads sharing one kv head (for QT query
// tiles), so each K/V tile is read by one block for all of them.
#include "dms_internal.h"

#include <hip/hip_ext.h>
#include <algorithm>
#include <type_traits>
#include <limits.h>
#include <math.h>

namespace dms {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ f16x8_t as_f16x8(uint4 u) { return __builtin_bit_cast(f16x8_t, u); }

__device__ __forceinline__ uint16_t bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// max and sum of x over lanes l and l ^ 32 (v_permlane32_swap exchanges the two
// halves of the wave in one VALU instruction; either result pair holds x of both)
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wait until at most N vector memory operations of this wave are in flight
// (for loads the compiler does not see: those with an LDS destination).
template <int N>
__device__ __forceinline__ void wait_older_loads() {
    static_assert(N == 2 || N == 4, "one or two units per thread and operand");
    if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
}

// row index of the S^T tile -> key index within the 32-key tile: bits 2 and 3 swapped
__device__ __forceinline__ int swap23(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }


// ---------------------------------------------------------------------------
// masked prefill attention.  One block = (kv head, QT consecutive 32-query
// tiles), max(4, G) waves: wave qt * G + g computes q head h * G + g on query
// tile qt.  Two blocks share a compute unit (two waves per SIMD); blocks are
// not synchronised with each other, so one block's matrix work overlaps the
// other's vector work.
// Key tiles of 32 are staged in LDS, double-buffered, by all threads of the
// block: K as [D/8][32] 16-byte units (A operand of S^T = K Q^T: lane = key row,
// 16 bytes = 8 dims), V as [4][D] units (A operand of O^T = V^T P^T: lane = dim,
// 16 bytes = 8 keys).  While tile i is folded, S_{i+1} is computed and the
// global loads of K_{i+3} and V_{i+2} are in flight.
//
// Key tiles of a block whose first query tile starts at t0b (xf = t0b - w):
//   far field  the first U = #live[0, xf] pool slots: unmarked keys older than
//              every query's window, visible to all queries of the block
//   band       prompt keys in (xf, t0b + 32 QT), masked per (query, key) pair
// ---------------------------------------------------------------------------
#ifndef DMS_PREFILL_WAVES
#define DMS_PREFILL_WAVES 4
#endif
constexpr int kPrefillWaves = DMS_PREFILL_WAVES;  // waves per block (tuning constant; G if larger)
constexpr int prefill_waves(int g) { return kPrefillWaves > g ? kPrefillWaves : g; }

//
// FP8 pools: K and V are staged as the bf16 values of their codes (far field
// from the pages, band from the quantised prompt and its V copy) and the row
// scales of the tile's keys go to LDS with V: a key's scores are multiplied by
// its K scale before the softmax, its weights by its V scale before P.V.
//
// EXT (extend calls: the T = n_tokens input rows are new tokens at positions
// t0 .. t0+T-1 of a (seq, layer) whose store already holds n_old live tokens):
// queries and band keys are input rows (the band rule is the same in rows as in
// positions, with no far-field boundary); the far field is every stored slot
// 0 .. n_old-1, in slot order, each visible to the rows below its expiry row X
// (position + w - t0 if marked, else never), staged per tile with V.
//
// H16 (bf16 pools whose V values all lie in the fp16 range): V is staged in LDS
// as fp16 and P enters P.V as one fp16 part, p * 2^7 (11 significant bits;
// the factor keeps small weights out of the fp16 subnormals and cancels in
// O / l).  Otherwise (FP8 pools, or a bf16 pool that has held a V value of
// magnitude 2^16 or more) P enters as two bf16 parts.
//
// DIR (prompt prefill on a bf16 pool with fp16 weights, four-wave blocks): the
// tiles go from memory straight to LDS (buffer loads with the LDS destination),
// so no register set stages them; three LDS buffers per operand, because a tile
// lands while the two before it are read; the band's V comes from the fp16 copy
// and its marks from the scan's bit mask (a scalar load).  Its kernel runs
// three waves per SIMD.  The loads are counted by hand: every step issues the
// same 2 UPT of them, and waits at its end until only its own are in flight.
template <int D, int G, bool F8, bool EXT, bool H16, bool DIR = false>
__device__ __forceinline__ void prefill_attend_body(const PrefillArgs& a) {
    constexpr int NWV = prefill_waves(G);
    constexpr int NT = 64 * NWV;
    static_assert(NWV % G == 0, "a block holds whole kv-head groups");
    constexpr int QT = NWV / G;  // query tiles per block
    constexpr int KS = D / 16;             // k-steps of S^T over the head dim
    constexpr int DT = D / 32;             // 32-row tiles of O^T
    constexpr int UNITS = 4 * D;           // 16-byte units of a K (or V) tile of 32 keys
    constexpr int UPT = (UNITS + NT - 1) / NT;  // units per thread
    static_assert(!DIR || (!F8 && !EXT && H16 && UNITS % NT == 0), "direct staging: prompt prefill, fp16 weights");
    constexpr int NB = DIR ? 3 : 2;  // LDS buffers per operand
    __shared__ uint4 s_k[NB][D / 8][32];
    __shared__ uint4 s_v[NB][4][D];
    __shared__ uint32_t s_marks[NB];
    __shared__ float4 s_ks[2][8], s_vs[2][8];  // FP8: K and V scales of the tile's 32 keys
    __shared__ int4 s_x[2][8];                  // EXT: expiry rows of the tile's 32 stored keys
    const PoolDev& P = a.pool;
    const int T = a.n_tokens, w = P.window, hkv = P.n_kv_heads, hq_n = P.n_q_heads;
    const int nqb = (T + 32 * QT - 1) / (32 * QT);
    // Blocks b, b+8, b+16, ... are placed on the same XCD; hand each XCD a run of
    // consecutive (kv head, query block) pairs so that a head's keys stay in that
    // XCD's L2.  Later query blocks (more keys) first.
    const int total = hkv * nqb;
    const int per_xcd = (total + 7) / 8;
    const int pidx = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (pidx >= total) return;
    const int h = pidx / nqb;
    const int t0b = (nqb - 1 - pidx % nqb) * (32 * QT);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qt = wave / G, hq = h * G + wave % G;
    const int gh = (a.seq * P.n_layers + a.layer) * hkv + h;
    const int col = lane & 31, half = lane >> 5;
    const int tq = t0b + 32 * qt + col;  // this lane's query
    const float sl = P.scale_log2;

    // Q^T as the B operand: column = query, 8 consecutive dims per half-wave
    uint4 qb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qb[ks] = tq < T ? *reinterpret_cast<const uint4*>(a.q + ((size_t)tq * hq_n + hq) * D + ks * 16 + half * 8)
                        : make_uint4(0, 0, 0, 0);

    // ---- the block's key tiles: far field, then the band (xf, kend) of prompt rows.
    // Prefill: the far field is the first U slots of the compacted store (the
    // unmarked keys at or below xf).  Extend: the U stored slots (each visible to
    // the rows below its expiry row), then the first Uc gathered unmarked rows of
    // the chunk (those at or below xf) in the scratch pages.
    const int xf = t0b - w;
    const int U = EXT ? P.hstate[(size_t)gh * kHS + kHsLive]
                      : (xf >= 0 ? P.pcnt[(size_t)h * P.max_positions + xf] : 0);
    const int Uc = EXT && xf >= 0 ? P.pcnt[(size_t)h * P.max_positions + xf] : 0;
    const int Ufar = EXT ? Uc : U;  // slots of the unmasked far segment (its last tile is cut at Ufar)
    const int nfar1 = (U + 31) / 32;
    const int nfar = nfar1 + (Uc + 31) / 32;
    const int band0 = max(0, xf + 1) / 32 * 32;
    const int kend = min(T, t0b + 32 * QT);
    const int ntiles = nfar + (kend > band0 ? (kend - band0 + 31) / 32 : 0);
    const int32_t* ptab = P.ptable + (size_t)gh * P.pages_per_head;
    const uint16_t* vt = (DIR ? P.vt16 : P.vt) + (size_t)h * (P.max_pos32 / 8) * D * 8;
    const size_t rowk = (size_t)hkv * D;  // elements from one prompt row of K to the next

    // Staging, thread t: K units u = t, t + NT, ... (chunk u / 32, key u % 32) and the
    // same V units.
    // K runs one tile ahead of V: while tile i is folded (scores S_i, computed one
    // iteration earlier, and V_i) the block computes S_{i+1} from K_{i+1}.  The
    // global loads run one step further ahead: those of K_{i+3} and V_{i+2} are
    // issued in step i into one of two register sets and written to LDS at the
    // end of step i+1, so every load has a whole step to land.  (FP8 codes are
    // converted to bf16 when written.)  Every load is issued by every thread:
    // rows past the prompt, units past the tile and tiles past the last are
    // read through short or zero-size resources, return 0 and touch no memory,
    // so each step issues the same loads and waits only for the older set.
    // (far tiles: slot of the first key within the tile's segment; band: prompt row)
    auto tile_kb = [&](int i) { return i < nfar1 ? 32 * i : i < nfar ? 32 * (i - nfar1) : band0 + 32 * (i - nfar); };
    // (Loaded values stay untouched in their registers until they are written:
    // any use would make the wave wait for them in the step that issues them.)
    uint4 rk[2][UPT], rv[2][UPT];
    uint32_t rlg[2];             // band: bits of the eviction logit of key kb + (lane & 31) (K channel: bf16)
    float rks[2], rvs[2];        // FP8: K and V scales of key kb + (lane & 31)
    int rx[2];                   // EXT: expiry row of stored slot kb + (lane & 31)
    const int kl = lane & 31;
    constexpr int kFar = 1 << 30;  // an offset past every resource below
    // resources are wave-uniform: base and size go through readfirstlane so that a
    // value the compiler cannot prove uniform (a loaded page id) never turns a
    // load into a per-lane loop
    auto rsrc = [](const void* base, int bytes) {
        const uint64_t b = reinterpret_cast<uint64_t>(base);
        const uint64_t ub = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b) |
                            ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) << 32);
        return buffer_rsrc(reinterpret_cast<const void*>(ub), __builtin_amdgcn_readfirstlane(bytes));
    };
    // page id of far-field tile t: a scalar load (the page table is read-only
    // here), so it is counted with the LDS operations, not with the tile loads
    typedef const int32_t __attribute__((address_space(4))) cint32_t;
    cint32_t* cptab = (cint32_t*)ptab;
    auto page_of = [&](int t) -> int {
        return t < nfar1 ? cptab[(32 * t) / kPage] : t < nfar ? P.xpage(h) + (32 * (t - nfar1)) / kPage : 0;
    };
    auto upage = [](int pg) -> size_t { return (size_t)(uint32_t)__builtin_amdgcn_readfirstlane(pg); };
    auto rows_left = [&](int kb) { return kb + 32 <= T ? 32 : kb < T ? T - kb : 0; };  // prompt rows kb .. kb+31
    const __amdgpu_buffer_rsrc_t rx_rsrc = rsrc(P.inv + (size_t)h * P.max_positions, EXT ? U * 4 : 0);
    // Per-thread offsets that do not change from tile to tile (bytes; kFar for
    // units past the tile): K unit (chunk cc, key j) in a page at slot 0 and in
    // the prompt at row 0; V unit u of a tile.
    int koff_far[UPT], koff_band[UPT], voff[UPT];
#pragma unroll
    for (int x = 0; x < UPT; ++x) {
        const int u = tid + x * NT, cc = u >> 5, j = u & 31;
        if constexpr (F8) {
            koff_far[x] = u >= UNITS ? kFar : ((cc >> 1) * kPage + j) * 16 + (cc & 1) * 8;
            koff_band[x] = u >= UNITS ? kFar : j * (int)rowk + cc * 8;
            voff[x] = u >= UNITS ? kFar : ((8 * (u / D)) / 16 * D + u % D) * 16 + (8 * (u / D)) % 16;
        } else {
            koff_far[x] = u >= UNITS ? kFar : ((cc * kPage + j) * 8) * 2;
            koff_band[x] = u >= UNITS ? kFar : (j * (int)rowk + cc * 8) * 2;
            voff[x] = u >= UNITS ? kFar : u * 16;
        }
    }
    constexpr int EB = F8 ? 1 : 2;  // bytes per stored K/V element
    const char* const kfar0 = reinterpret_cast<const char*>(F8 ? (const void*)P.kp8() : (const void*)P.kpages);
    const char* const vfar0 = reinterpret_cast<const char*>(F8 ? (const void*)P.vp8() : (const void*)P.vpages);
    const char* const kband0 = F8 ? reinterpret_cast<const char*>(P.q8_codes(0) + h * D)
                                  : reinterpret_cast<const char*>(a.k + h * D);
    const int rowb = (int)rowk * EB;  // bytes from one prompt row of K to the next
    // md (compile time): 1 if tile i is a full tile of the first far-field
    // segment (the compacted prompt; extend: the stored slots), 2 if it is a full
    // band tile (32 prompt rows), 0 if any kind may hold
    // DIR: 16 bytes per lane from r at voff into LDS at lds + 16 lane (lds:
    // this wave's 1 KB of the buffer, passed in M0; a lane past the resource
    // reads 0 and touches no memory, as with the register loads)
    // (LDS byte addresses: the low half of a shared variable's generic address)
    const uint32_t lds_k = (uint32_t)(uintptr_t)&s_k[0][0][0], lds_v = (uint32_t)(uintptr_t)&s_v[0][0][0];
    auto dma16 = [&](__amdgpu_buffer_rsrc_t r, int voff, uint32_t lds) {
        const uint32_t la = __builtin_amdgcn_readfirstlane((int)lds);
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" : : "s"(la), "v"(voff), "s"(r) : "memory");
    };
    auto load_k = [&](int i, int X, int pg, auto md) {
        constexpr bool FP = decltype(md)::value == 1, BP = decltype(md)::value == 2;
        const int kb = FP ? 32 * i : BP ? band0 + 32 * (i - nfar) : tile_kb(i);
        const bool far = FP || (!BP && i < nfar), live = FP || BP || i < ntiles;
        const char* base = far ? kfar0 + upage(pg) * (kPage * D * EB) : kband0 + (size_t)kb * rowb;
        const int bytes = !live ? 0 : far ? kPage * D * EB : (BP ? 32 : rows_left(kb)) * rowb;
        const __amdgpu_buffer_rsrc_t r = rsrc(base, bytes);
        const int slot16 = (kb % kPage) * 16;  // far: the tile's first slot within the page
        if constexpr (DIR) {  // unit u = 64 wave + lane + NT x: chunk u / 32, key u % 32
#pragma unroll
            for (int x = 0; x < UPT; ++x)
                dma16(r, far ? koff_far[x] + slot16 : koff_band[x],
                      lds_k + (uint32_t)(((i % NB) * UNITS + 64 * wave + NT * x) * 16));
            return;
        }
#pragma unroll
        for (int x = 0; x < UPT; ++x) {
            const int off = far ? koff_far[x] + slot16 : koff_band[x];
            if constexpr (F8) {
                const uint2 c = buffer_load8(r, off, 0);
                rk[X][x] = make_uint4(c.x, c.y, 0u, 0u);
            } else {
                rk[X][x] = buffer_load16(r, off, 0);
            }
        }
    };
    auto load_v = [&](int i, int X, int pg, auto md) {
        constexpr bool FP = decltype(md)::value == 1, BP = decltype(md)::value == 2;
        const int kb = FP ? 32 * i : BP ? band0 + 32 * (i - nfar) : tile_kb(i);
        const bool far = FP || (!BP && i < nfar), live = FP || BP || i < ntiles;
        const int rows = BP ? 32 : rows_left(kb);
        if (F8 && far) {  // keys kb % 64 + 8 (u / D) .. +7 of dim u % D: half a 16-slot unit
            const __amdgpu_buffer_rsrc_t r =
                rsrc(vfar0 + upage(pg) * (kPage * D) + (size_t)(kb % kPage / 16) * D * 16, live ? 2 * D * 16 : 0);
#pragma unroll
            for (int x = 0; x < UPT; ++x) {
                const uint2 c = buffer_load8(r, voff[x], 0);
                rv[X][x] = make_uint4(c.x, c.y, 0u, 0u);
            }
        } else {
            // (prefill on fp16 weights: the far field's V from the fp16 copy the
            // compaction left in the kv head's scratch pages, in slot order)
            const char* base = !far ? reinterpret_cast<const char*>(vt) + (size_t)(kb / 8) * D * 16
                               : H16 && !EXT ? vfar0 + (size_t)(P.xpage(h) + kb / kPage) * (kPage * D * 2) +
                                                   (size_t)(kb % kPage / 8) * D * 16
                                             : vfar0 + upage(pg) * (kPage * D * 2) + (size_t)(kb % kPage / 8) * D * 16;
            const __amdgpu_buffer_rsrc_t r = rsrc(base, live ? UNITS * 16 : 0);
            if constexpr (DIR) {  // unit u = 64 wave + lane + NT x: key block u / D, dim u % D
#pragma unroll
                for (int x = 0; x < UPT; ++x)
                    dma16(r, voff[x], lds_v + (uint32_t)(((i % NB) * UNITS + 64 * wave + NT * x) * 16));
            } else {
#pragma unroll
                for (int x = 0; x < UPT; ++x)
                    rv[X][x] = buffer_load16(r, F8 ? (tid + x * NT >= UNITS ? kFar : (tid + x * NT) * 16) : voff[x], 0);
            }
        }
        // per-key data of the tile (lanes l and l + 32 read the same key)
        const bool band = live && !far;
        if (FP) {
        } else if (DIR) {  // marks of keys kb .. kb+31 (bits past the prompt are 0)
            typedef const uint32_t __attribute__((address_space(4))) cu32_t;
            rlg[X] = band ? ((cu32_t*)P.mbits_of(h))[kb / 32] : 0u;
        } else if (P.logit_ch >= 0) {
            const __amdgpu_buffer_rsrc_t r =
                rsrc(a.k + (size_t)kb * rowk + h * D + P.logit_ch, band ? rows * (int)rowk * 2 : 0);
            rlg[X] = buffer_load2(r, kl * (int)rowk * 2);
        } else {
            const __amdgpu_buffer_rsrc_t r = rsrc(a.logits + (size_t)kb * hkv + h, band ? rows * hkv * 4 : 0);
            rlg[X] = (uint32_t)buffer_load4i(r, kl * hkv * 4);
        }
        if constexpr (EXT && !BP) rx[X] = buffer_load4i(rx_rsrc, (kb + kl) * 4 + (live && (FP || i < nfar1) ? 0 : kFar));
        if constexpr (F8) {
            if (far) {
                const size_t sl0 = upage(pg) * kPage + kb % kPage;
                rks[X] = buffer_load4f(rsrc(P.kscale + sl0, live ? 32 * 4 : 0), kl * 4);
                rvs[X] = buffer_load4f(rsrc(P.vscale + sl0, live ? 32 * 4 : 0), kl * 4);
            } else {
                const int bytes = live ? rows * hkv * 4 : 0;
                rks[X] = buffer_load4f(rsrc(P.q8_scales(0) + (size_t)kb * hkv + h, bytes), kl * hkv * 4);
                rvs[X] = buffer_load4f(rsrc(P.q8_scales(1) + (size_t)kb * hkv + h, bytes), kl * hkv * 4);
            }
        }
    };
    auto store_k = [&](int i, int X) {
        if constexpr (DIR) return;  // already in LDS
#pragma unroll
        for (int x = 0; x < UPT; ++x) {
            const int u = tid + x * NT;
            if (UNITS % NT == 0 || u < UNITS)
                s_k[i % NB][u >> 5][u & 31] = F8 ? fp8x8_bf16(make_uint2(rk[X][x].x, rk[X][x].y)) : rk[X][x];
        }
    };
    auto store_v = [&](int i, int X, auto md) {
        constexpr int MD = decltype(md)::value;
        const bool far = MD == 1 || (MD != 2 && i < nfar);
        if constexpr (DIR) {  // V is already in LDS; the tile's marks
            if (!far && tid == 0) s_marks[i % NB] = rlg[X];
            return;
        }
#pragma unroll
        for (int x = 0; x < UPT; ++x) {
            const int u = tid + x * NT;
            if (UNITS % NT == 0 || u < UNITS)
                s_v[i % NB][u / D][u % D] = (F8 && far)           ? fp8x8_bf16(make_uint2(rv[X][x].x, rv[X][x].y))
                                           : H16 && (EXT || !far) ? bf16x8_to_f16x8(rv[X][x])
                                                                  : rv[X][x];
        }
        if (!far && wave == 0) {  // keys past the prompt read logit 0: unmarked
            const float lg = __uint_as_float(P.logit_ch >= 0 ? rlg[X] << 16 : rlg[X]);
            const uint32_t mk = (uint32_t)__ballot(lg > 0.f);
            if (lane == 0) s_marks[i % NB] = mk;
        }
        if constexpr (EXT) {
            if (tid < 32 && (MD == 1 || (MD != 2 && i < nfar1)))
                reinterpret_cast<int*>(s_x[i & 1])[tid] = tile_kb(i) + tid < U ? rx[X] : INT_MIN;
        }
        if constexpr (F8) {
            if (tid < 32) {
                reinterpret_cast<float*>(s_ks[i & 1])[tid] = rks[X];
                reinterpret_cast<float*>(s_vs[i & 1])[tid] = rvs[X];
            }
        }
    };
    const int krow = swap23(col);  // key this lane feeds as A-operand row
    auto scores = [&](int i) {
        uint4 ka[KS];  // every K operand of the tile first: one wait for LDS
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) ka[ks] = s_k[i % NB][2 * ks + half][krow];
        f32x16_t sc = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[ks]), as_bf16x8(qb[ks]), sc, 0, 0, 0);
        return sc;
    };

    f32x16_t o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16_t{};
    float m = -INFINITY, lsum = 0.f;

    // prologue: K_0, V_0, K_1 in LDS, S_0; K_2 and V_1 in flight (register set 1)
    int pg2, pg3;
    {
        const int pg0 = page_of(0), pg1 = page_of(1);
        pg2 = page_of(2);
        pg3 = page_of(3);
        const std::integral_constant<int, 0> gen;
        load_k(0, 0, pg0, gen);
        load_v(0, 0, pg0, gen);
        load_k(1, 1, pg1, gen);
        store_k(0, 0);
        store_v(0, 0, gen);
        if (ntiles > 1) store_k(1, 1);
        load_k(2, 1, pg2, gen);
        load_v(1, 1, pg1, gen);
    }
    if constexpr (DIR) wait_older_loads<2 * UPT>();  // K_0, V_0 and K_1 are in LDS
    __syncthreads();
    // one tile: fold S_i (in cur) while S_{i+1} (into nxt) and the next loads run.
    // md (compile time): 1 if tiles i .. i+3 are full tiles of the first
    // far-field segment, 2 if they are full band tiles, 0 otherwise
    auto step = [&](int i, f32x16_t& cur, f32x16_t& nxt, int X, auto md) {
        constexpr bool FP = decltype(md)::value == 1, BP = decltype(md)::value == 2;
        const int pg4 = BP ? 0 : page_of(i + 4);
        load_k(i + 3, X, pg3, md);
        load_v(i + 2, X, pg2, md);

        // ---- fold tile i: row r of S_i holds key kb + (r & 7) + 8 half + 16 (r >> 3)
        const int kb = FP ? 32 * i : BP ? band0 + 32 * (i - nfar) : tile_kb(i);
        // z: the scores (FP8: times the keys' K scales) with invisible keys at
        // -inf, computed in place in S_i's registers (dead after this step)
        f32x16_t& z = cur;
        // (FP8: rows r0 .. r0+3 hold keys 4 kk .. 4 kk + 3, whose K scales are
        // applied here and whose V scales are read where the weights are formed)
        auto scale_q4 = [&](int r) { return 2 * half + ((r >> 2) & 1) + 4 * (r >> 3); };  // kk of row r
        if constexpr (F8) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int r0 = 4 * (q4 & 1) + 8 * (q4 >> 1);
                const float4 k4 = s_ks[i & 1][scale_q4(r0)];
                z[r0] *= k4.x;
                z[r0 + 1] *= k4.y;
                z[r0 + 2] *= k4.z;
                z[r0 + 3] *= k4.w;
            }
        }
        if (EXT && !BP && (FP || i < nfar1)) {  // stored keys: visible to the rows below their expiry row
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int4 x4 = s_x[i & 1][2 * half + (q4 & 1) + 4 * (q4 >> 1)];
                const int r0 = 4 * (q4 & 1) + 8 * (q4 >> 1);
                if (tq >= x4.x) z[r0] = -INFINITY;
                if (tq >= x4.y) z[r0 + 1] = -INFINITY;
                if (tq >= x4.z) z[r0 + 2] = -INFINITY;
                if (tq >= x4.w) z[r0 + 3] = -INFINITY;
            }
        } else if (!FP && (BP || !(i < nfar && kb + 32 <= Ufar))) {  // (a whole far tile is visible as it is)
            // visible keys of this lane's query as one 32-bit mask over the tile.
            // Last far tile: kb + kr < Ufar.  Band: kb + kr <= tq, kb + kr > xf,
            // and unmarked or kb + kr > tq - w.
            uint32_t vis;
            if (!BP && i < nfar) {
                vis = (1u << (Ufar - kb)) - 1u;  // Ufar - kb in [1, 31]
            } else {
                const uint32_t marks = s_marks[i % NB];
                auto above = [](int c) -> uint32_t {  // bits kr > c
                    return c < 0 ? 0xffffffffu : (c >= 31 ? 0u : (0xffffffffu << (c + 1)));
                };
                vis = ~above(tq - kb) & above(xf - kb) & (~marks | above(tq - w - kb));
                if (tq >= T) vis = 0;
            }
            // (tiles every query of the wave sees whole, e.g. inside the window and
            // below the diagonal, keep their scores as they are)
            if (__ballot(vis != 0xffffffffu)) {
                vis >>= 8 * half;  // this lane's rows: kr = (r & 7) + 8 half + 16 (r >> 3)
#pragma unroll
                for (int r = 0; r < 16; ++r) {  // bit -> all-ones or zero, then a bit select
                    const int mk = __builtin_amdgcn_sbfe((int)vis, (r & 7) + 16 * (r >> 3), 1);
                    z[r] = __int_as_float((__float_as_int(z[r]) & mk) | (int)(0xff800000u & ~(uint32_t)mk));
                }
            }
        }
        float tmax = z[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, z[r]);
        tmax = max_xor32(tmax) * sl;  // base-2 units (sl > 0)
        // lazy rescale: the running maximum moves only when a score exceeds it by
        // more than 8 (base 2), so weights stay below 256
        const bool grow = tmax > m + 8.f;
        if (__ballot(grow)) {
            const float mn = grow ? tmax : m;
            const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mn);
            lsum *= alpha;
            m = mn;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        }
        // ---- branch-free part: S_{i+1} on the matrix cores (after the last tile
        // the K buffer holds an older tile: the result is not used) interleaved
        // with the weights of tile i on the vector ALUs.  P^T enters the PV
        // product as two bf16 parts, hi = bf16(p) and lo = bf16(p - hi): about
        // 16 significant bits, fp32 accumulation.  (v_exp_f32: exact to about
        // 1 ulp; results below 2^-126 flush to 0.)
        // (extend calls: the two blocks that share a compute unit start together
        // and stay in phase; a raised wave priority over the matrix part of the
        // step lets one block's products run while the other's vector work
        // issues: 143 -> 134.6 us per chunk and layer on the 32K chunked
        // prefill.  The prompt prefill, whose blocks start staggered, gains
        // nothing from it.)
        if constexpr (EXT) __builtin_amdgcn_s_setprio(1);
        // (DIR: each K operand read where its product is issued, to keep the
        // register count within three waves per SIMD)
        uint4 ka[KS];
        if constexpr (!DIR)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) ka[ks] = s_k[(i + 1) % NB][2 * ks + half][krow];
        f32x16_t sc = f32x16_t{};
        uint32_t ph[8], pl[8];
        float ps = 0.f;
        // m == -inf only while every score so far (this tile's included) is masked:
        // then z = -inf and exp2(-inf) = 0.  (H16: weights times 2^7, l alike.)
        const float nm = (m == -INFINITY ? 0.f : -m) + (H16 ? 7.f : 0.f);
#pragma unroll
        for (int i2 = 0; i2 < 8; ++i2) {
            if (i2 % (8 / KS) == 0) {
                if constexpr (DIR) ka[i2 / (8 / KS)] = s_k[(i + 1) % NB][2 * (i2 / (8 / KS)) + half][krow];
                sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[i2 / (8 / KS)]), as_bf16x8(qb[i2 / (8 / KS)]),
                                                             sc, 0, 0, 0);
            }
            const float p0 = __builtin_amdgcn_exp2f(fmaf(z[2 * i2], sl, nm));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(z[2 * i2 + 1], sl, nm));
            if constexpr (H16) {
                const f16x2_t hv = {(_Float16)p0, (_Float16)p1};
                ph[i2] = __builtin_bit_cast(uint32_t, hv);
            } else {
                float w0 = p0, w1 = p1;
                if constexpr (F8) {  // V scales of the keys in rows 2 i2 and 2 i2 + 1
                    const float2 v2 = reinterpret_cast<const float2*>(&s_vs[i & 1][scale_q4(2 * i2)])[(i2 & 1)];
                    w0 *= v2.x;
                    w1 *= v2.y;
                }
                const bf16x2_t hv = {(__bf16)w0, (__bf16)w1};
                const bf16x2_t lv = {(__bf16)(w0 - (float)hv[0]), (__bf16)(w1 - (float)hv[1])};
                ph[i2] = __builtin_bit_cast(uint32_t, hv);
                pl[i2] = __builtin_bit_cast(uint32_t, lv);
            }
            ps += p0 + p1;
        }
        nxt = sc;
        lsum += ps;
        uint4 va[DT][2];
        if constexpr (!DIR)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) va[dt][kk] = s_v[i % NB][2 * kk + half][dt * 32 + col];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if constexpr (DIR)  // (DIR: half the V operands at a time)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) va[dt][kk] = s_v[i % NB][2 * kk + half][dt * 32 + col];
            const uint4 hb = make_uint4(ph[4 * kk], ph[4 * kk + 1], ph[4 * kk + 2], ph[4 * kk + 3]);
            if constexpr (H16) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(va[dt][kk]), as_f16x8(hb), o[dt], 0, 0, 0);
            } else {
                const uint4 lb = make_uint4(pl[4 * kk], pl[4 * kk + 1], pl[4 * kk + 2], pl[4 * kk + 3]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[dt][kk]), as_bf16x8(hb), o[dt], 0, 0,
                                                                    0);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[dt][kk]), as_bf16x8(lb), o[dt], 0, 0,
                                                                    0);
            }
        }
        // K_{i+2} replaces K_i (read for S_i one iteration ago), V_{i+1} replaces
        // V_{i-1}; both were loaded in step i-1 (the other register set)
        if constexpr (EXT) __builtin_amdgcn_s_setprio(0);
        if (FP || BP || i + 2 < ntiles) store_k(i + 2, X ^ 1);
        if (FP || BP || i + 1 < ntiles) store_v(i + 1, X ^ 1, md);
        pg2 = pg3;
        pg3 = pg4;
        if constexpr (DIR) wait_older_loads<2 * UPT>();  // K_{i+2} and V_{i+1} are in LDS
        __syncthreads();
    };
    // S and the in-flight loads alternate between two register sets (no copies
    // between iterations)
    // (steps whose tile and in-flight loads are all full tiles of the first
    // far-field segment, then general steps up to the band (extend: through the
    // gathered chunk rows), steps on full band tiles, general steps)
    const std::integral_constant<int, 0> gen;
    const std::integral_constant<int, 1> farc;
    const std::integral_constant<int, 2> bandc;
    f32x16_t sa = scores(0), sb;
    // (DIR: step 0 loads K_3 into K_0's buffer, which every wave has just read
    // for S_0; with staging through registers that write came two barriers later)
    if constexpr (DIR) __syncthreads();
    int i = 0;
    for (; i + 6 <= nfar1; i += 2) {
        step(i, sa, sb, 0, farc);
        step(i + 1, sb, sa, 1, farc);
    }
    for (; i < nfar && i < ntiles; i += 2) {
        step(i, sa, sb, 0, gen);
        if (i + 1 < ntiles) step(i + 1, sb, sa, 1, gen);
    }
    for (; i + 6 <= ntiles; i += 2) {
        step(i, sa, sb, 0, bandc);
        step(i + 1, sb, sa, 1, bandc);
    }
    for (; i < ntiles; i += 2) {
        step(i, sa, sb, 0, gen);
        if (i + 1 < ntiles) step(i + 1, sb, sa, 1, gen);
    }

    // (DIR: the last steps' loads, of tiles past the end, land before the block
    // can leave and its LDS be handed to another)
    if constexpr (DIR) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- normalise and store: lane holds dims dt*32 + 8*(r/4) + 4*half + r%4 of query tq
    const float ltot = sum_xor32(lsum);
    if (tq < T) {
        const float inv = 1.f / ltot;
        uint16_t* orow = a.out + ((size_t)tq * hq_n + hq) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = dt * 32 + 8 * r4 + 4 * half;
                const uint32_t lo = (uint32_t)bf16_bits(o[dt][4 * r4] * inv) | ((uint32_t)bf16_bits(o[dt][4 * r4 + 1] * inv) << 16);
                const uint32_t hi = (uint32_t)bf16_bits(o[dt][4 * r4 + 2] * inv) | ((uint32_t)bf16_bits(o[dt][4 * r4 + 3] * inv) << 16);
                *reinterpret_cast<uint2*>(orow + d) = make_uint2(lo, hi);
            }
    }
}

// Prompt prefill on bf16 pools with four-wave blocks: the fp16-weights case runs
// in prefill_attend3_kernel (below), this kernel only when a V value is wide.
template <int D, int G, bool EXT>
constexpr bool prefill_direct() { return !EXT && prefill_waves(G) == 4; }

template <int D, int G, bool F8, bool EXT>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * prefill_waves(G), 64 * prefill_waves(G)),
                          amdgpu_waves_per_eu(2, 2)))
void prefill_attend_kernel(PrefillArgs a) {
    if constexpr (F8) {
        prefill_attend_body<D, G, true, EXT, false>(a);
    } else {
        typedef const int32_t __attribute__((address_space(4))) cint32_t;  // a scalar load
        if (((cint32_t*)a.pool.ctl)[kCtlVWide] == 0) {
            if constexpr (!prefill_direct<D, G, EXT>()) prefill_attend_body<D, G, false, EXT, true>(a);
        } else {
            prefill_attend_body<D, G, false, EXT, false>(a);
        }
    }
}

// The same for the fp16-weights case of a prompt prefill with direct staging:
// three waves per SIMD (at most 168 registers), 49 KB of LDS per block.
template <int D, int G>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(3, 3)))
void prefill_attend3_kernel(PrefillArgs a) {
    typedef const int32_t __attribute__((address_space(4))) cint32_t;
    if (((cint32_t*)a.pool.ctl)[kCtlVWide] == 0) prefill_attend_body<D, G, false, false, true, true>(a);
}

// Extend calls: expiry row of every stored slot j < n_old of the (seq, layer),
// relative to the chunk's first position t0: position + w - t0 if the token is
// marked (its mark is in the window ring while it is within w of t0), else
// INT_MAX.  Written to the inv scratch ([kv head][slot]), which the attention
// reads per far-field tile and the chain resolution overwrites afterwards.
// n_old and t0 come from the head record (the device's counters decide); the
// nb blocks of a kv head stride over its slots.
__device__ __forceinline__ void expiry_block(const PrefillArgs& a, int bx, int nb, int h) {
    const PoolDev& P = a.pool;
    const int w = P.window;
    const int gh = (a.seq * P.n_layers + a.layer) * P.n_kv_heads + h;
    const int n_old = P.hstate[(size_t)gh * kHS + kHsLive], t0 = P.hstate[(size_t)gh * kHS + kHsPos];
    for (int j = bx * 256 + threadIdx.x; j < n_old; j += nb * 256) {
        const int page = P.ptable[(size_t)gh * P.pages_per_head + j / kPage];
        const int pos = P.slot_pos[(size_t)page * kPage + j % kPage];
        int mk = 0;
        if (P.ring_len > 0 && pos >= t0 - w) {
            const int e = P.ring[(size_t)gh * P.ring_len + pos % w];
            mk = e >= 0 && (e & 1);
        }
        P.inv[(size_t)h * P.max_positions + j] = mk ? pos + w - t0 : INT_MAX;
    }
}

// Extend calls with output: the chunk's unmarked rows (never evicted, so every
// query at least w rows later sees them) gathered in row order into the scratch
// pages of their kv head, with the running count of unmarked rows per row in
// pcnt.  The attention reads them as a dense far field, as the prefill reads
// the compacted prompt.  Block bx of kv head h: rows 64bx .. 64bx+63; it
// counts the unmarked rows before its segment itself (up to 8 logits per thread
// per pass, all requested before any is used), and every copy load is issued
// before the stores.
template <int D, bool F8>
__device__ __forceinline__ void compact_block(const PrefillArgs& a, int bx, int h) {
    const PoolDev& P = a.pool;
    __shared__ int s_prev[4];  // per wave: unmarked rows before the segment
    __shared__ int s_row[64];  // the segment's unmarked rows, in order
    __shared__ int s_n;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r0 = bx * 64;
    const int T = a.n_tokens, hkv = P.n_kv_heads;
    int prev = 0;  // unmarked rows in [0, r0) seen by this wave (wave-uniform)
    for (int c0 = 0; c0 < r0; c0 += 2048) {
        bool u[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int c = c0 + 256 * k + tid;
            u[k] = c < r0 && !(eviction_logit(P, a.logits, a.k, c, h) > 0.f);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) prev += __popcll(__ballot(u[k]));
    }
    if (lane == 0) s_prev[wave] = prev;
    const int r = r0 + lane;  // wave 0: the segment's rows
    bool um = false;
    int rank = 0;
    if (wave == 0) {
        um = r < T && !(eviction_logit(P, a.logits, a.k, r, h) > 0.f);
        const uint64_t b = __ballot(um);
        rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0));
        if (um) s_row[rank] = r;
        if (lane == 0) s_n = __popcll(b);
    }
    __syncthreads();
    const int n = s_n, base = s_prev[0] + s_prev[1] + s_prev[2] + s_prev[3];
    if (wave == 0 && r < T) P.pcnt[(size_t)h * P.max_positions + r] = base + rank + (um ? 1 : 0);
    const int xp = P.xpage(h);
    if constexpr (F8) {
        constexpr int NC = D / 16;
        for (int u = tid; u < n * NC; u += 256) {  // K: 16 codes per chunk
            const int j = u / NC, cc = u - j * NC, slot = base + j;
            const size_t row = (size_t)s_row[j] * hkv + h;
            uint8_t* kp = P.kp8() + (size_t)(xp + slot / kPage) * (kPage * D);
            *reinterpret_cast<uint4*>(kp + ((size_t)cc * kPage + slot % kPage) * 16) =
                *reinterpret_cast<const uint4*>(P.q8_codes(0) + row * D + cc * 16);
        }
        for (int u = tid; u < n * D; u += 256) {  // V: one code per (row, dim)
            const int j = u / D, d = u - j * D, slot = base + j;
            const size_t row = (size_t)s_row[j] * hkv + h;
            uint8_t* vp = P.vp8() + (size_t)(xp + slot / kPage) * (kPage * D);
            vp[((size_t)(slot % kPage / 16) * D + d) * 16 + slot % 16] = P.q8_codes(1)[row * D + d];
        }
        if (tid < n) {
            const int slot = base + tid;
            const size_t row = (size_t)s_row[tid] * hkv + h, sl = (size_t)(xp + slot / kPage) * kPage + slot % kPage;
            P.kscale[sl] = P.q8_scales(0)[row];
            P.vscale[sl] = P.q8_scales(1)[row];
        }
    } else {
        // item u < n NC: K chunk u % NC of row u / NC; then the same for V
        constexpr int NC = D / 8, IT = (64 * 2 * NC) / 256;
        uint4 x[IT];
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int u = tid + 256 * k, uv = u - n * NC;
            const bool isk = u < n * NC, isv = !isk && uv < n * NC;
            const int j = isk ? u / NC : uv / NC, cc = isk ? u % NC : uv % NC;
            x[k] = make_uint4(0, 0, 0, 0);
            if (isk || isv) {
                const size_t row = (size_t)s_row[j] * hkv + h;
                x[k] = *reinterpret_cast<const uint4*>((isk ? a.k : a.v) + row * D + cc * 8);
            }
        }
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const int u = tid + 256 * k, uv = u - n * NC;
            const bool isk = u < n * NC, isv = !isk && uv < n * NC;
            if (!isk && !isv) continue;
            const int j = isk ? u / NC : uv / NC, cc = isk ? u % NC : uv % NC, slot = base + j;
            if (isk) {
                uint16_t* kp = P.kpages + (size_t)(xp + slot / kPage) * (kPage * D);
                *reinterpret_cast<uint4*>(kp + ((size_t)cc * kPage + slot % kPage) * 8) = x[k];
            } else {  // V: 8 dims of the row, one value per 8-slot unit
                uint16_t* vp = P.vpages + (size_t)(xp + slot / kPage) * (kPage * D) +
                               (size_t)(slot % kPage / 8) * D * 8 + slot % 8;
                const uint32_t xw[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    vp[(size_t)(cc * 8 + q) * 8] = (uint16_t)(q & 1 ? xw[q / 2] >> 16 : xw[q / 2] & 0xffffu);
            }
        }
    }
}


// Extend calls with output: the three independent preparations of the attention
// in one launch, blocks (x, kv head): the V copy of the chunk (x < NV), the
// expiry rows of the stored slots (next NE), the gathered unmarked rows (rest).
template <int D, bool F8>
__global__ __launch_bounds__(256) void extend_prep_kernel(PrefillArgs a) {
    const int nv = (a.n_tokens + 63) / 64, ne = max(1, (a.t0 + 255) / 256);  // t0: the host's count (a size hint)
    __shared__ uint16_t s_v[64][D + 8];
    const int bx = blockIdx.x, h = blockIdx.y;
    if (bx < nv) vt_rows<D, F8>(a, bx * 64, h, s_v);
    else if (bx < nv + ne) expiry_block(a, bx - nv, ne, h);
    else compact_block<D, F8>(a, bx - nv - ne, h);
}

template <int D, int G, bool EXT>
hipError_t launch_attend_t(const PrefillArgs& a, hipStream_t s, hipEvent_t* ev) {
    constexpr int QT = prefill_waves(G) / G;
    const int nqb = (a.n_tokens + 32 * QT - 1) / (32 * QT);
    const int total = a.pool.n_kv_heads * nqb;
    const int grid = 8 * ((total + 7) / 8);
    if (a.pool.fp8) {
        hipExtLaunchKernelGGL((prefill_attend_kernel<D, G, true, EXT>), dim3(grid), dim3(64 * prefill_waves(G)), 0,
                              s, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr, 0, a);
    } else if constexpr (prefill_direct<D, G, EXT>()) {
        // whether a V value is wide is known on the device only: both kernels
        // are launched, and the one that does not apply returns at once
        hipExtLaunchKernelGGL((prefill_attend3_kernel<D, G>), dim3(grid), dim3(256), 0, s, ev ? ev[0] : nullptr,
                              nullptr, 0, a);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        hipExtLaunchKernelGGL((prefill_attend_kernel<D, G, false, EXT>), dim3(grid), dim3(64 * prefill_waves(G)), 0,
                              s, nullptr, ev ? ev[1] : nullptr, 0, a);
    } else {
        hipExtLaunchKernelGGL((prefill_attend_kernel<D, G, false, EXT>), dim3(grid), dim3(64 * prefill_waves(G)), 0,
                              s, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr, 0, a);
    }
    return hipGetLastError();
}

// ev (optional): extend, 4 events (preparation, then attention start/stop);
// prefill, 2 events (attention; its V copy ran with the compaction)
template <int D, bool EXT>
hipError_t launch_attend_d(const PrefillArgs& a, hipStream_t s, hipEvent_t* ev) {
    if (EXT) {
        const int nv = (a.n_tokens + 63) / 64;
        // the store holds at most t0 slots per head (expiry rows); the chunk's
        // rows are copied and gathered 64 per block
        const dim3 pgrid(nv + std::max(1, (a.t0 + 255) / 256) + nv, a.pool.n_kv_heads);
        if (a.pool.fp8)
            hipExtLaunchKernelGGL((extend_prep_kernel<D, true>), pgrid, dim3(256), 0, s, ev ? ev[0] : nullptr,
                                  ev ? ev[1] : nullptr, 0, a);
        else
            hipExtLaunchKernelGGL((extend_prep_kernel<D, false>), pgrid, dim3(256), 0, s, ev ? ev[0] : nullptr,
                                  ev ? ev[1] : nullptr, 0, a);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        if (ev) ev += 2;
    }
    switch (a.pool.n_q_heads / a.pool.n_kv_heads) {
        case 1: return launch_attend_t<D, 1, EXT>(a, s, ev);
        case 2: return launch_attend_t<D, 2, EXT>(a, s, ev);
        case 4: return launch_attend_t<D, 4, EXT>(a, s, ev);
        case 8: return launch_attend_t<D, 8, EXT>(a, s, ev);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// Runs after the compaction kernels of the same prefill (same stream): the far
// field reads the pages and the live-count prefix they wrote.
hipError_t launch_prefill_attend(const PrefillArgs& a, hipStream_t s, hipEvent_t* ev) {
    if (a.pool.head_dim == 128) return launch_attend_d<128, false>(a, s, ev);
    if (a.pool.head_dim == 64) return launch_attend_d<64, false>(a, s, ev);
    return hipErrorInvalidValue;
}

// Extend calls: the chunk's queries over the store (read before the chunk's
// tokens are written) and the chunk; after the FP8 quantisation of the chunk.
hipError_t launch_extend_attend(const PrefillArgs& a, hipStream_t s, hipEvent_t* ev) {
    if (a.pool.head_dim == 128) return launch_attend_d<128, true>(a, s, ev);
    if (a.pool.head_dim == 64) return launch_attend_d<64, true>(a, s, ev);
    return hipErrorInvalidValue;
}

}  // namespace dms
