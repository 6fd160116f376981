// DMS compact-store kernels for CDNA4 (gfx950): decode (split-K flash-decode
// over the live slots, then merge and eviction/append), prefill compaction, and
// sequence release.
//
// What a decode step computes for one (sequence, layer, kv head) at position t
// (DMS delayed eviction: "NVIDIA veroeffentlicht Qwen3-8B-DMS-8x ..." news page,
// section "Dynamic Memory Sparsification (DMS): Eine innovative Loesung"; stiva.ai
// "Nvidia DMS ...", section on delayed eviction; compact store with reclaimed
// slots: the FastDMS announcement on molayo1419.me):
//   live set before the step  V(t-1), stored in slots 0 .. n_old-1 of the head
//   the token at t-w leaves if it was marked; its slot e is reused by token t,
//   otherwise token t takes slot n_old (a new page every 64 slots)
//   out[g] = softmax over V(t) = V(t-1) \ {t-w if marked} + {t}
//
// Kernels of one decode launch:
//   decode_attend  -- one block per compute unit; every block derives the page
//                     axis of the call (ceil(n_old / 64) pages per head, heads in
//                     call order) from the head records, then each wave folds an
//                     equal run of consecutive pages into a running softmax:
//                     QK^T with lane = slot (v_dot2_f32_bf16 over 16-byte K chunks
//                     loaded 1 KB-coalesced from the key-major K page), page max
//                     and sum by DPP wavefront reductions, PV with lane = dim
//                     (v_dot2 over key pairs of the dim-major V page), the next
//                     page's K and V in flight meanwhile.  One partial per (wave,
//                     head) pair.  This kernel only reads the pool.
//   decode_merge   -- per head: log-sum-exp merge of the partials with the new
//                     token (bf16 output), and, in separate blocks, mark, expiry,
//                     slot reuse or page allocation, K/V append and the record.
// The kernel boundary orders every read of this step before every write.
#include "dms_internal.h"

#include <hip/hip_ext.h>
#include <math.h>

#include <mutex>

namespace dms {

// Scratch of the decode entry point that allocates nothing: the split-K
// partials and the page-axis prefix of one launch, in a file-scope device array
// (each GPU the library runs on holds its own copy until the process ends).
// Host code never passes the array's name to a kernel: in host code the name
// stands for a host-side stand-in, not for the device memory.  It uses the
// address hipGetSymbolAddress gives for the current device instead.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch_address(void** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {  // once per device, with that device current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // keep NaN a NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// a.lo*b.lo + a.hi*b.hi + c, bf16 pairs, fp32 accumulate
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Wavefront reductions on DPP (no LDS): butterflies inside each 16-lane row,
// then row_bcast:15 / row_bcast:31 fold the four rows into lane 63, which is
// read back as a wave-uniform value.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float old, float x) {
    return __builtin_amdgcn_update_dpp(old, x, CTRL, ROW_MASK, 0xf, false);
}

// readlane on the bit pattern (the builtin takes an int; a float argument would
// be converted by value)
__device__ __forceinline__ float readlane_f(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x, x));        // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_f<0x4E>(x, x));        // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_f<0x141>(x, x));       // row_half_mirror
    x = fmaxf(x, dpp_f<0x140>(x, x));       // row_mirror
    x = fmaxf(x, dpp_f<0x142, 0xa>(x, x));  // row_bcast:15 into rows 1, 3
    x = fmaxf(x, dpp_f<0x143, 0xc>(x, x));  // row_bcast:31 into rows 2, 3
    return readlane_f(x, 63);
}

__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_f<0xB1>(0.f, x);
    x += dpp_f<0x4E>(0.f, x);
    x += dpp_f<0x141>(0.f, x);
    x += dpp_f<0x140>(0.f, x);
    x += dpp_f<0x142, 0xa>(0.f, x);
    x += dpp_f<0x143, 0xc>(0.f, x);
    return readlane_f(x, 63);
}

// The kernel arguments sit in memory the command processor wrote just before
// the dispatch, so the first read of each 64-byte line of them misses the
// caches; read lazily under branches, those misses come one after another.
// Touching every line the kernel reads puts them in flight together (the
// decode kernels do it right after their first loads, whose addresses come in
// the preloaded leading arguments).
// (with: uniform values loaded just before, which are waited for together with
// the lines)
template <int BYTES>
__device__ __forceinline__ void touch_args(const void* args, int with = 0) {
    typedef const int __attribute__((address_space(4))) cint_t;
    cint_t* p = (cint_t*)args;
    int acc = with;
#pragma unroll
    for (int o = 0; o < BYTES / 4; o += 16) acc ^= p[o];
    asm volatile("" ::"s"(acc));
}

// x where c holds, zeros elsewhere, component by component (a select of the
// whole vector struct is lowered through private memory)
__device__ __forceinline__ uint4 keep_if(bool c, uint4 x) {
    const uint32_t m = c ? ~0u : 0u;
    return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
}

// Reduce x over the lanes that share lane % G (G a power of two up to 32) with
// op, all on the VALU: the halves and quarters of the wave are exchanged by
// v_permlane32_swap / v_permlane16_swap (either result pair holds x of both
// partners), the lanes of a 16-lane row by DPP rotations (combining lane l with
// l + o mod 16 for o = 8, 4, ... covers the row's lanes with l's residue).
template <int G, typename Op>
__device__ __forceinline__ float reduce_mod_g(float x, Op op) {
    if constexpr (G <= 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    if constexpr (G <= 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    if constexpr (G <= 8) x = op(x, dpp_f<0x128>(x, x));  // row_ror:8
    if constexpr (G <= 4) x = op(x, dpp_f<0x124>(x, x));  // row_ror:4
    if constexpr (G <= 2) x = op(x, dpp_f<0x122>(x, x));  // row_ror:2
    if constexpr (G <= 1) x = op(x, dpp_f<0x121>(x, x));  // row_ror:1
    return x;
}

// Scheduling fence for register values: an empty volatile asm that reads and
// writes x.  Volatile asm keeps its place among memory operations, so the
// arithmetic producing x stays ahead of the loads issued after this point.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

// Exclusive scan of one int per thread over a block of NT threads (NT % 64 == 0).
template <int NT>
__device__ int block_excl_scan(int x, int* total, int* s_wave) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int NW = NT / 64;
    int incl = wave_incl_scan(x, lane);
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int v = lane < NW ? s_wave[lane] : 0;
        int vi = wave_incl_scan(v, lane);
        if (lane < NW) s_wave[NW + lane] = vi - v;  // exclusive wave offsets
        if (lane == NW - 1) s_wave[2 * NW] = vi;
    }
    __syncthreads();
    int r = s_wave[NW + wave] + incl - x;
    *total = s_wave[2 * NW];
    __syncthreads();
    return r;
}

// Intra-wave LDS hand-off: order this wave's LDS writes before its later reads.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct CallHead {
    int gh;   // global head id
    int row;  // input row (layer-in-call, sequence-in-call)
    int h;    // kv head
};

__device__ __forceinline__ CallHead call_head(const DecodeArgs& a, int ch) {
    const int hkv = a.pool.n_kv_heads;
    const int per_layer = a.n_seqs * hkv;
    const int li = ch / per_layer;
    const int rem = ch - li * per_layer;
    const int si = rem / hkv;
    const int h = rem - si * hkv;
    CallHead c;
    c.h = h;
    c.gh = ((a.seq_ids[si] * a.pool.n_layers) + a.layer0 + li) * hkv + h;
    c.row = li * a.n_seqs_total + a.seq_base + si;
    return c;
}

// ---------------------------------------------------------------------------
// decode, kernel 1: split-K attention over the live slots
//
// Work split.  The pages of the call's heads, concatenated in call-head order,
// form one axis: head ch owns pages pp[ch] .. pp[ch+1]-1, pp being the exclusive
// prefix of ceil(n_old / 64).  Its P pages are cut into W = min(waves, P) equal
// runs; wave w takes pages [w*P/W, (w+1)*P/W) and folds them into a running
// softmax, writing one partial per head its run touches, at partial slot w + ch
// (distinct for all (w, ch) pairs that occur, and contiguous per head).  Waves
// never wait for each other after the plan is built.  Small calls: with fewer
// pages than waves, run w (one page) goes to wave w / grid of block w % grid;
// with at most one page per block, block b takes page b and its waves share
// out the page's q heads.
//
// Pipeline of one wave: K and V of page k+1 are requested while page k is being
// computed (K right after QK^T has consumed the K registers, V right after P.V
// has consumed the V registers), so each wave keeps 16-32 KB of loads in flight.
// ---------------------------------------------------------------------------

// K chunks of one page (lane = slot; chunk cc of the page's 64 slots is 1 KB
// contiguous).  A dead request gets a zero-size resource: no memory traffic.
template <int D>
__device__ __forceinline__ void issue_k(const PoolDev& P, int page, bool live, int lane, uint4 (&kc)[D / 8]) {
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(P.kpages + (size_t)page * (kPage * D), live ? kPage * D * 2 : 0);
#pragma unroll
    for (int cc = 0; cc < D / 8; ++cc) kc[cc] = buffer_load16_stream(r, lane * 16, cc * kPage * 16);
}

// V units of one page (lane = dim: unit (b, j) holds slots 8b .. 8b+7 of dim j*64 + lane).
template <int D>
__device__ __forceinline__ void issue_v(const PoolDev& P, int page, bool live, int lane, uint4 (&vc)[8][D / 64]) {
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(P.vpages + (size_t)page * (kPage * D), live ? kPage * D * 2 : 0);
#pragma unroll
    for (int b = 0; b < 8; ++b)
#pragma unroll
        for (int j = 0; j < D / 64; ++j) vc[b][j] = buffer_load16_stream(r, lane * 16, (b * D + j * 64) * 16);
}

// QK^T of one page, lane = slot.  q comes from LDS (every lane reads the same
// address: a broadcast), the G heads' pieces of a chunk one chunk ahead of their
// use; the G heads are G independent chains of dot products over the 16-byte K
// chunks.
template <int D, int G>
__device__ __forceinline__ void qk_page(const uint4 (&kc)[D / 8], const uint4* s_q, float (&z)[G]) {
    constexpr int NC = D / 8;
    uint4 qa[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        z[g] = 0.f;
        qa[g] = s_q[g * NC];
    }
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
        uint4 qb[G];
        if (cc + 1 < NC) {
#pragma unroll
            for (int g = 0; g < G; ++g) qb[g] = s_q[g * NC + cc + 1];
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            z[g] = dot2(qa[g].x, kc[cc].x, z[g]);
            z[g] = dot2(qa[g].y, kc[cc].y, z[g]);
            z[g] = dot2(qa[g].z, kc[cc].z, z[g]);
            z[g] = dot2(qa[g].w, kc[cc].w, z[g]);
            pin(z[g]);
        }
        if (cc + 1 < NC) {
#pragma unroll
            for (int g = 0; g < G; ++g) qa[g] = qb[g];
        }
    }
}

// Online-softmax update with the scores of one page (slots base + lane; slots at
// or beyond n_old and the expiring slot e are masked).  The page's weights go to
// LDS as two bf16 parts, hi = bf16(p) and lo = bf16(p - hi), for the PV step.
// (FP8 pages: one fp16 part, p times vmul / vmax, vmul = the slot's V scale and
// vmax = the largest over the page's valid slots, returned for P.V; l sums p.)
template <int D, int G, bool F8>
__device__ __forceinline__ void softmax_page(const float (&z)[G], float scale_log2, int base, int n_old, int e,
                                             int lane, float vmul, uint16_t (*s_p)[G][kPage], float (&m)[G],
                                             float (&l)[G], float (&acc)[G][D / 64], float& vmax) {
    const int slot = base + lane;
    const bool valid = slot < n_old && slot != e;
    float pscale = 1.f;
    if constexpr (F8) {
        vmax = wave_max(valid ? vmul : 0.f);
        pscale = vmax > 0.f ? vmul * __builtin_amdgcn_rcpf(vmax) : 0.f;
    }
    float zz[G], mn[G], p[G];
    // the G heads' reductions are independent: issue them side by side
#pragma unroll
    for (int g = 0; g < G; ++g) zz[g] = valid ? z[g] * scale_log2 : -INFINITY;  // masked by a select
#pragma unroll
    for (int g = 0; g < G; ++g) mn[g] = fmaxf(m[g], wave_max(zz[g]));
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float alpha = 1.f;
        p[g] = 0.f;
        if (mn[g] != -INFINITY) {
            p[g] = exp2f(zz[g] - mn[g]);
            alpha = exp2f(m[g] - mn[g]);
        }
        if constexpr (F8) {
            s_p[0][g][lane] = __builtin_bit_cast(uint16_t, (_Float16)(p[g] * pscale));
        } else {
            const uint16_t ph = f32_to_bf16(p[g]);
            s_p[0][g][lane] = ph;
            s_p[1][g][lane] = f32_to_bf16(p[g] - bf16_to_f32(ph));
        }
        l[g] *= alpha;
        m[g] = mn[g];
#pragma unroll
        for (int j = 0; j < D / 64; ++j) acc[g][j] *= alpha;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) l[g] += wave_sum(p[g]);
}

// P.V of one page, lane = dim: each 16-byte V unit holds 8 consecutive slots of
// one dim, i.e. 4 key pairs, matched by 4 bf16 pairs of p (broadcast reads),
// once for the high and once for the low part of p.
template <int D, int G>
__device__ __forceinline__ void pv_page(const uint4 (&vc)[8][D / 64], const uint16_t (*s_p)[G][kPage],
                                        float (&acc)[G][D / 64]) {
    constexpr int VJ = D / 64;
#pragma unroll
    for (int part = 0; part < 2; ++part) {
        uint4 pn[G];
#pragma unroll
        for (int g = 0; g < G; ++g) pn[g] = *reinterpret_cast<const uint4*>(&s_p[part][g][0]);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            uint4 pp[G];
#pragma unroll
            for (int g = 0; g < G; ++g) pp[g] = pn[g];
            if (b + 1 < 8) {
#pragma unroll
                for (int g = 0; g < G; ++g) pn[g] = *reinterpret_cast<const uint4*>(&s_p[part][g][(b + 1) * 8]);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
#pragma unroll
                for (int j = 0; j < VJ; ++j) {
                    acc[g][j] = dot2(pp[g].x, vc[b][j].x, acc[g][j]);
                    acc[g][j] = dot2(pp[g].y, vc[b][j].y, acc[g][j]);
                    acc[g][j] = dot2(pp[g].z, vc[b][j].z, acc[g][j]);
                    acc[g][j] = dot2(pp[g].w, vc[b][j].w, acc[g][j]);
                    pin(acc[g][j]);
                }
            }
        }
    }
}

// ---- FP8 pages (E4M3 codes, one fp32 scale per slot) -----------------------
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// a.lo*b.lo + a.hi*b.hi + c, fp16 pairs, fp32 accumulate
__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

// Two E4M3 codes (bytes 0-1 or 2-3 of w) as an fp16 pair: exact (every E4M3
// value is an fp16 value).
__device__ __forceinline__ uint32_t fp8x2_h_lo(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}
__device__ __forceinline__ uint32_t fp8x2_h_hi(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

// K chunks of one FP8 page (lane = slot; chunk cc = 16 dims of 64 slots, 1 KB
// contiguous), then the K and V scales of slot lane (behind the K chunks in the
// load queue, so waiting for them never waits for the page's V).
template <int D>
__device__ __forceinline__ void issue_k8(const PoolDev& P, int page, bool live, int lane, uint4 (&kc)[D / 16],
                                         float& ks, float& vs) {
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(P.kp8() + (size_t)page * (kPage * D), live ? kPage * D : 0);
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) kc[cc] = buffer_load16_stream(r, lane * 16, cc * kPage * 16);
    ks = buffer_load4f(buffer_rsrc(P.kscale + (size_t)page * kPage, live ? kPage * 4 : 0), lane * 4);
    vs = buffer_load4f(buffer_rsrc(P.vscale + (size_t)page * kPage, live ? kPage * 4 : 0), lane * 4);
}

// V units of one FP8 page (lane = dim: unit (b, j) holds slots 16b .. 16b+15 of
// dim j*64 + lane).
template <int D>
__device__ __forceinline__ void issue_v8(const PoolDev& P, int page, bool live, int lane, uint4 (&vc)[4][D / 64]) {
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(P.vp8() + (size_t)page * (kPage * D), live ? kPage * D : 0);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int j = 0; j < D / 64; ++j) vc[b][j] = buffer_load16_stream(r, lane * 16, (b * D + j * 64) * 16);
}

// QK^T of one FP8 page, lane = slot: chunk cc (dims 16cc .. 16cc+15) against q
// pieces 2cc and 2cc+1; the codes become bf16 pairs once for all G heads.  The
// result is in code units (times the slot's K scale = the score).
template <int D, int G>
__device__ __forceinline__ void qk_page8(const uint4 (&kc)[D / 16], const uint4* s_q, float (&z)[G]) {
    constexpr int NC = D / 8;
#pragma unroll
    for (int g = 0; g < G; ++g) z[g] = 0.f;
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
        const uint32_t k0 = fp8x2_lo(kc[cc].x), k1 = fp8x2_hi(kc[cc].x);
        const uint32_t k2 = fp8x2_lo(kc[cc].y), k3 = fp8x2_hi(kc[cc].y);
        const uint32_t k4 = fp8x2_lo(kc[cc].z), k5 = fp8x2_hi(kc[cc].z);
        const uint32_t k6 = fp8x2_lo(kc[cc].w), k7 = fp8x2_hi(kc[cc].w);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint4 qa = s_q[g * NC + 2 * cc], qb = s_q[g * NC + 2 * cc + 1];
            z[g] = dot2(qa.x, k0, z[g]);
            z[g] = dot2(qa.y, k1, z[g]);
            z[g] = dot2(qa.z, k2, z[g]);
            z[g] = dot2(qa.w, k3, z[g]);
            z[g] = dot2(qb.x, k4, z[g]);
            z[g] = dot2(qb.y, k5, z[g]);
            z[g] = dot2(qb.z, k6, z[g]);
            z[g] = dot2(qb.w, k7, z[g]);
            pin(z[g]);
        }
    }
}

// P.V of one FP8 page, lane = dim: unit (b, j) holds 16 slots of one dim, i.e.
// 8 key pairs as fp16 pairs, matched by two 16-byte pieces of the page's fp16
// weights (p times the slot's V scale over the page's largest, vmax); the
// page's sums enter the accumulators times vmax.
template <int D, int G>
__device__ __forceinline__ void pv_page8(const uint4 (&vc)[4][D / 64], const uint16_t (*s_p)[G][kPage],
                                         float vmax, float (&acc)[G][D / 64]) {
    constexpr int VJ = D / 64;
    float t[G][VJ];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < VJ; ++j) t[g][j] = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        uint32_t vb[VJ][8];
#pragma unroll
        for (int j = 0; j < VJ; ++j) {
            vb[j][0] = fp8x2_h_lo(vc[b][j].x);
            vb[j][1] = fp8x2_h_hi(vc[b][j].x);
            vb[j][2] = fp8x2_h_lo(vc[b][j].y);
            vb[j][3] = fp8x2_h_hi(vc[b][j].y);
            vb[j][4] = fp8x2_h_lo(vc[b][j].z);
            vb[j][5] = fp8x2_h_hi(vc[b][j].z);
            vb[j][6] = fp8x2_h_lo(vc[b][j].w);
            vb[j][7] = fp8x2_h_hi(vc[b][j].w);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint4 pa = *reinterpret_cast<const uint4*>(&s_p[0][g][16 * b]);
            const uint4 pb = *reinterpret_cast<const uint4*>(&s_p[0][g][16 * b + 8]);
#pragma unroll
            for (int j = 0; j < VJ; ++j) {
                t[g][j] = dot2h(pa.x, vb[j][0], t[g][j]);
                t[g][j] = dot2h(pa.y, vb[j][1], t[g][j]);
                t[g][j] = dot2h(pa.z, vb[j][2], t[g][j]);
                t[g][j] = dot2h(pa.w, vb[j][3], t[g][j]);
                t[g][j] = dot2h(pb.x, vb[j][4], t[g][j]);
                t[g][j] = dot2h(pb.y, vb[j][5], t[g][j]);
                t[g][j] = dot2h(pb.z, vb[j][6], t[g][j]);
                t[g][j] = dot2h(pb.w, vb[j][7], t[g][j]);
                pin(t[g][j]);
            }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < VJ; ++j) acc[g][j] = fmaf(t[g][j], vmax, acc[g][j]);
}

// q of call head ch's G query heads: G * D bf16, contiguous in the input.
__device__ __forceinline__ const uint16_t* q_group(const DecodeArgs& a, int ch) {
    const CallHead c = call_head(a, ch);
    return a.q + ((size_t)c.row * a.pool.n_q_heads + c.h * (a.pool.n_q_heads / a.pool.n_kv_heads)) * a.pool.head_dim;
}

template <int D, int G, bool F8, bool RC>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kAttendWaves, 64 * kAttendWaves),
                          amdgpu_waves_per_eu(2, 2)))
void decode_attend_kernel(const int32_t* __restrict__ hs_plan, int32_t gh0, int32_t n_heads, int32_t n_kv,
                          int32_t n_seqs, int32_t pool_layers, int32_t layer0, DecodeArgs a) {
    constexpr int NT = 64 * kAttendWaves;
    constexpr int VJ = D / 64;
    constexpr int QV = G * D / 8;  // 16-byte pieces of one head group's q
    constexpr int QR = (QV + 63) / 64;
    constexpr int PSTR = part_stride(G, D);
    constexpr int ACC = part_acc_off(G);
    const int H = n_heads;
    extern __shared__ int32_t s_dyn[];
    int32_t* s_pp = s_dyn;            // [H + 1] first page of each head on the call's page axis
    int32_t* s_nold = s_pp + H + 1;   // [H] live count before this step
    int32_t* s_exp = s_nold + H;      // [H] slot expiring at this step, or -1
    int32_t* s_gh = s_exp + H;        // [H] global head id
    __shared__ uint4 s_q[kAttendWaves][QV];
    __shared__ uint16_t s_p[kAttendWaves][2][G][kPage];
    __shared__ int s_scan[2 * kAttendWaves + 1];

    const PoolDev& P = a.pool;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // Calls with at most NG pages per block (below): each group of NA waves of
    // a block takes a page, GW q heads per wave (group k of block b: page
    // b + k * grid).  A 32 KB page (D = 128) goes to at most two waves: four
    // copies of it load one compute unit's memory path more than the shorter
    // dot products save.
    constexpr int NAX = D == 128 ? 2 : kAttendWaves;
    constexpr int NA = G < NAX ? G : NAX;  // waves per page
    constexpr int NG = kAttendWaves / NA;  // pages per block
    constexpr int GW = G / NA;             // q heads per wave
    constexpr int QW = GW * D / 8;         // 16-byte pieces of their q
    const int grp = NG == 1 ? 0 : wave / NA, role = NG == 1 ? wave : wave % NA;
    const int ei = (int)blockIdx.x + grp * (int)gridDim.x;  // this group's page (and cache entry)
    // Their page, K/V and q registers, which the block may fill before the plan
    // is done: from the page cache entry of this block in the row of the call's
    // head group, when it is of the pool's current epoch.  Only calls of one
    // layer of one sequence (the calls a model makes at batch 1) use the cache
    // (RC, chosen at launch): other calls run the kernel without its code.  The
    // cache sits directly before the head records.
    const int32_t* const rc0 = hs_plan - kRunCacheBytes / 4;
    const bool rc_on = RC && gh0 >= 0 && n_heads == n_kv && ei < kRunCacheRuns;
    int32_t* const rce_at = const_cast<int32_t*>(rc0) + kRunCacheHeader +
                            ((size_t)(rc_on ? gh0 / n_kv % kRunCacheRows : 0) * kRunCacheRuns + (rc_on ? ei : 0)) * 4;
    uint4 kc[F8 ? D / 16 : D / 8], vc[F8 ? 4 : 8][VJ];
    float ksn = 1.f, vsn = 1.f;
    uint4 qv = make_uint4(0u, 0u, 0u, 0u);
    int rpid = -1, rgh = -1, rj = -1, epoch = 0;

    // ---- plan: pages per head and their prefix (every block builds its own);
    // a thread's head records (16 bytes each) are all requested before any is used
    {
        constexpr int MAXPER = (kMaxCallHeads + NT - 1) / NT;
        const int per = (H + NT - 1) / NT;
        const int h0 = min(tid * per, H), h1 = min(h0 + per, H);
        int4 rec[MAXPER];
        int ghs[MAXPER];
#pragma unroll
        for (int i = 0; i < MAXPER; ++i) {
            if (h0 + i < h1) {
                // (the global head id as call_head computes it, from the leading
                // arguments; a call of one sequence needs no sequence id)
                const int ch = h0 + i, li = ch / (n_seqs * n_kv), si = (ch - li * n_seqs * n_kv) / n_kv;
                ghs[i] = gh0 >= 0 ? gh0 + ch : (a.seq_ids[si] * pool_layers + layer0 + li) * n_kv + ch % n_kv;
                rec[i] = *reinterpret_cast<const int4*>(hs_plan + (size_t)ghs[i] * kHS);
            }
        }
        // the page cache entry and the epoch, behind the head records (blocks
        // past the cache read through empty resources: no memory access)
        uint4 e = make_uint4(~0u, ~0u, ~0u, ~0u);
        int ep = 0;
        if constexpr (RC) {
            e = buffer_load16(buffer_rsrc(rce_at, rc_on ? 16 : 0), 0, 0);
            ep = buffer_load4i(buffer_rsrc(rc0, rc_on ? 4 : 0), 0);
        }
        // (after the head records are requested: the fixed part of the
        // arguments and the first sequence ids, one word of every line)
        touch_args<offsetof(DecodeArgs, seq_ids) + 64>(&a);
        if constexpr (RC) {
            rpid = __builtin_amdgcn_readfirstlane((int)e.x);
            rgh = __builtin_amdgcn_readfirstlane((int)e.y);
            rj = __builtin_amdgcn_readfirstlane((int)e.z);
            epoch = __builtin_amdgcn_readfirstlane(ep);
            if (__builtin_amdgcn_readfirstlane((int)e.w) != epoch) rgh = -1;
            // the cached page, if this call covers its head: its K, V and this
            // wave's q go out now, while the plan is being built
            const int64_t all_pages = P.max_pages + (int64_t)P.n_kv_heads * P.pages_per_head;
            if (rc_on && rgh >= gh0 && rgh - gh0 < H && rpid >= 0 && rpid < all_pages) {
                if constexpr (F8) {
                    issue_k8<D>(P, rpid, true, lane, kc, ksn, vsn);
                    issue_v8<D>(P, rpid, true, lane, vc);
                } else {
                    issue_k<D>(P, rpid, true, lane, kc);
                    issue_v<D>(P, rpid, true, lane, vc);
                }
                qv = buffer_load16(buffer_rsrc(q_group(a, rgh - gh0) + role * GW * D, QW * 16), lane * 16, 0);
            } else {
                rgh = -1;
            }
        }
        int local = 0;
#pragma unroll
        for (int i = 0; i < MAXPER; ++i) {
            if (h0 + i < h1) {
                const int ch = h0 + i;
                const int n = rec[i].x;  // [kHsLive]
                s_nold[ch] = n;
                s_exp[ch] = rec[i].w;    // [kHsExp]
                s_gh[ch] = ghs[i];
                const int c = (n + kPage - 1) / kPage;
                s_pp[ch] = c;
                local += c;
            }
        }
        int total;
        int off = block_excl_scan<NT>(local, &total, s_scan);
        for (int ch = h0; ch < h1; ++ch) {
            const int c = s_pp[ch];
            s_pp[ch] = off;
            off += c;
        }
        if (tid == 0) s_pp[H] = total;
        __syncthreads();
        if (blockIdx.x == 0)
            for (int i = tid; i <= H; i += NT) P.prefix[i] = s_pp[i];
    }
    // ---- this wave's run of pages (no block-wide synchronisation below)
    const int total = __builtin_amdgcn_readfirstlane(s_pp[H]);
    if (total <= (int)gridDim.x * NG) {
        // A call with at most NG pages per block (e.g. one layer of one
        // sequence): group k of block b takes page b + k * grid (run pg of W =
        // total), and its NA waves split the page's G q heads, GW each, every
        // wave with its own copy of the page.  Each head's arithmetic is the
        // general path's, so the partial holds the same bits; the page's dot
        // products are spread over the block's SIMDs.  The page is the cached
        // one if the group's cache entry names the same (head, page index) in
        // the current epoch (a head's page-table entries below its page count
        // change only after a release, which advances the epoch); else it is
        // read from the page table and the entry rewritten.
        const int pg = ei;
        if (pg >= total) return;
        int lo = 0, hi = H;  // s_pp[lo] <= pg < s_pp[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_pp[mid] <= pg) lo = mid; else hi = mid;
        }
        const int hd = __builtin_amdgcn_readfirstlane(lo);
        const int j = pg - __builtin_amdgcn_readfirstlane(s_pp[hd]);
        const int gh = __builtin_amdgcn_readfirstlane(s_gh[hd]);
        if (!RC || rgh != gh || rj != j) {
            // (registers still awaiting the cached page are refilled after it:
            // loads return in order)
            const int pid = __builtin_amdgcn_readfirstlane(P.ptable[(size_t)gh * P.pages_per_head + j]);
            if constexpr (F8) {
                issue_k8<D>(P, pid, true, lane, kc, ksn, vsn);
                issue_v8<D>(P, pid, true, lane, vc);
            } else {
                issue_k<D>(P, pid, true, lane, kc);
                issue_v<D>(P, pid, true, lane, vc);
            }
            qv = buffer_load16(buffer_rsrc(q_group(a, hd) + role * GW * D, QW * 16), lane * 16, 0);
            if (RC && rc_on && role == 0 && lane == 0) *reinterpret_cast<int4*>(rce_at) = make_int4(pid, gh, j, epoch);
        }
        if (lane < QW) s_q[wave][lane] = qv;
        wave_lds_sync();
        float z[GW], m[GW], l[GW], acc[GW][VJ], vmax = 1.f, vsc = 1.f;
#pragma unroll
        for (int g = 0; g < GW; ++g) {
            m[g] = -INFINITY;
            l[g] = 0.f;
#pragma unroll
            for (int jj = 0; jj < VJ; ++jj) acc[g][jj] = 0.f;
        }
        if constexpr (F8) {
            qk_page8<D, GW>(kc, s_q[wave], z);
#pragma unroll
            for (int g = 0; g < GW; ++g) z[g] *= ksn;
            vsc = vsn;
        } else {
            qk_page<D, GW>(kc, s_q[wave], z);
        }
        uint16_t(*sp)[GW][kPage] = reinterpret_cast<uint16_t(*)[GW][kPage]>(&s_p[wave][0][0][0]);
        softmax_page<D, GW, F8>(z, P.scale_log2, j * kPage, __builtin_amdgcn_readfirstlane(s_nold[hd]),
                                __builtin_amdgcn_readfirstlane(s_exp[hd]), lane, vsc, sp, m, l, acc, vmax);
        wave_lds_sync();
        if constexpr (F8) pv_page8<D, GW>(vc, sp, vmax, acc);
        else pv_page<D, GW>(vc, sp, acc);
        float* part = P.partials + (size_t)(pg + hd) * PSTR;
        if (lane == 0) {
#pragma unroll
            for (int g = 0; g < GW; ++g) {
                part[role * GW + g] = m[g];
                part[G + role * GW + g] = l[g];
            }
        }
#pragma unroll
        for (int g = 0; g < GW; ++g)
#pragma unroll
            for (int jj = 0; jj < VJ; ++jj) part[ACC + (role * GW + g) * D + jj * 64 + lane] = acc[g][jj];
        return;
    }
    const int NW = (int)gridDim.x * kAttendWaves;
    const int W = min(NW, total);
    // Run w of W.  A call with fewer pages than waves (one page per run, e.g.
    // one layer of one sequence) hands its runs to wave 0 of every block first,
    // so that each run has a compute unit's load path to itself; otherwise the
    // waves of a block take consecutive runs.
    const int w = W < NW ? wave * (int)gridDim.x + (int)blockIdx.x : (int)blockIdx.x * kAttendWaves + wave;
    if (w >= W) return;
    const int p0 = (int)(((int64_t)w * total) / W);
    const int p1 = (int)(((int64_t)(w + 1) * total) / W);

    // page id and head of pages b0 + lane (a batch of 64): lane-parallel search
    auto batch = [&](int b0, int& pid, int& hd) {
        const int p = b0 + lane;
        int lo = 0;
        pid = 0;
        if (p < p1) {
            int hi = H;  // s_pp[lo] <= p < s_pp[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_pp[mid] <= p) lo = mid; else hi = mid;
            }
            pid = P.ptable[(size_t)s_gh[lo] * P.pages_per_head + (p - s_pp[lo])];
        }
        hd = lo;
    };
    auto load_q = [&](int ch, bool live, uint4 (&qr)[QR]) {
        const __amdgpu_buffer_rsrc_t r = buffer_rsrc(q_group(a, ch), live ? QV * 16 : 0);
#pragma unroll
        for (int i = 0; i < QR; ++i) qr[i] = buffer_load16(r, (lane + 64 * i) * 16, 0);
    };
    auto store_q = [&](const uint4 (&qr)[QR]) {
#pragma unroll
        for (int i = 0; i < QR; ++i)
            if (lane + 64 * i < QV) s_q[wave][lane + 64 * i] = qr[i];
        wave_lds_sync();
    };

    // page ids and heads of pages b0 .. b0+63 (cur) and b0+64 .. b0+127 (nxt)
    int b0 = p0;
    int cpid, chd, npid = 0, nhd = 0;
    batch(b0, cpid, chd);
    if (b0 + 64 < p1) batch(b0 + 64, npid, nhd);  // the next batch, in flight
    auto head_at = [&](int j) {                   // j - b0 in [0, 128), wave-uniform
        const int i = j - b0;
        return i < 64 ? __builtin_amdgcn_readlane(chd, i) : __builtin_amdgcn_readlane(nhd, i - 64);
    };
    auto page_at = [&](int j) {
        const int i = j - b0;
        return i < 64 ? __builtin_amdgcn_readlane(cpid, i) : __builtin_amdgcn_readlane(npid, i - 64);
    };
    int hd = __builtin_amdgcn_readfirstlane(chd);
    uint4 qr[QR];
    load_q(hd, true, qr);
    // kc, vc: K and V registers of one page (FP8 pages: half as many, plus the
    // slot's scales, loaded with K into ksn / vsn and taken over at the top of
    // the page); once consumed they are refilled with the next page.
    auto ik = [&](int page, bool live) {
        if constexpr (F8) issue_k8<D>(P, page, live, lane, kc, ksn, vsn);
        else issue_k<D>(P, page, live, lane, kc);
    };
    auto iv = [&](int page, bool live) {
        if constexpr (F8) issue_v8<D>(P, page, live, lane, vc);
        else issue_v<D>(P, page, live, lane, vc);
    };
    ik(__builtin_amdgcn_readfirstlane(cpid), true);
    iv(__builtin_amdgcn_readfirstlane(cpid), true);
    store_q(qr);

    float m[G], l[G], acc[G][VJ];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int j = 0; j < VJ; ++j) acc[g][j] = 0.f;
    }
    for (int k = p0; k < p1; ++k) {
        if (k - b0 == 64) {  // page k enters the next batch
            b0 += 64;
            cpid = npid;
            chd = nhd;
            if (b0 + 64 < p1) batch(b0 + 64, npid, nhd);
        }
        const bool more = k + 1 < p1;
        const int hd1 = more ? head_at(k + 1) : hd;
        const bool new_head = more && hd1 != hd;
        const int pid1 = more ? page_at(k + 1) : 0;
        const int n_old = __builtin_amdgcn_readfirstlane(s_nold[hd]);
        const int e = __builtin_amdgcn_readfirstlane(s_exp[hd]);
        const int base = (k - __builtin_amdgcn_readfirstlane(s_pp[hd])) * kPage;

        float z[G];
        float vsc = 1.f, vmax = 1.f;
        if constexpr (F8) {
            const float ksc = ksn;
            vsc = vsn;
            qk_page8<D, G>(kc, s_q[wave], z);
#pragma unroll
            for (int g = 0; g < G; ++g) z[g] *= ksc;
        } else {
            qk_page<D, G>(kc, s_q[wave], z);
        }
        load_q(hd1, new_head, qr);  // the next head's q, if the run moves on
        ik(pid1, more);             // K registers are free again
        softmax_page<D, G, F8>(z, P.scale_log2, base, n_old, e, lane, vsc, s_p[wave], m, l, acc, vmax);
        wave_lds_sync();
        if constexpr (F8) pv_page8<D, G>(vc, s_p[wave], vmax, acc);
        else pv_page<D, G>(vc, s_p[wave], acc);
        iv(pid1, more);             // V registers are free again
        wave_lds_sync();            // s_p is rewritten by the next page

        if (!more || new_head) {
            // the run leaves head hd: its partial goes to slot w + hd
            float* part = P.partials + (size_t)(w + hd) * PSTR;
            if (lane == 0) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    part[g] = m[g];
                    part[G + g] = l[g];
                }
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
#pragma unroll
                for (int j = 0; j < VJ; ++j) {
                    part[ACC + g * D + j * 64 + lane] = acc[g][j];
                    acc[g][j] = 0.f;
                }
                m[g] = -INFINITY;
                l[g] = 0.f;
            }
            if (new_head) store_q(qr);
        }
        hd = hd1;
    }
}

// ---------------------------------------------------------------------------
// decode, kernel 2: merge (blocks 0 .. H-1) and evict / append (blocks H .. 2H-1).
// The two halves touch disjoint data: the merge reads the partials and the
// inputs, the append writes the pool and the head records.  Each issues its
// independent loads together, so a head costs two round trips to memory.
// ---------------------------------------------------------------------------

// Log-sum-exp merge of a head's partials with the new token; bf16 output of the
// head's G q heads, or of its part ds of DS equal parts (calls with many partials
// per head spread a head over DS blocks, so that fewer loads queue per thread and
// one round holds DS times as many partials).  256 threads.  Once the head's
// partial range is known the loads go out together, 16 bytes per lane: thread t
// owns output float4 ds * NF + t % NF for the partials u = t / NF, t / NF + NPH,
// ... (a round of RU of them in registers), and the maxima and sums (thread t:
// q head t % G of partials t / G, t / G + 256 / G, ...).  The NPH phases are
// summed through LDS.
// (FP8 pools: the new token enters as its quantised K and V rows, value(code) *
// row scale, like every stored token.)
template <int D, int G, bool F8, int DS>
__device__ void merge_head(const DecodeArgs& a, const int32_t* __restrict__ prefix, int H, int ch, int ds) {
    const PoolDev& P = a.pool;
    constexpr int PSTR = part_stride(G, D);  // floats per partial
    constexpr int ACC = part_acc_off(G);
    constexpr int NF = G * D / 4 / DS;       // float4 outputs of the block
    constexpr int NPH = 256 / NF;            // partial phases (NF divides 256)
    constexpr int RU = 16;                   // accumulators per thread per round
    constexpr int STEP = 256 / G;
    constexpr int KT = G;                    // partials per thread whose m, l stay in registers
    constexpr int NW_MAX = KT * STEP;        // partials whose weights are kept in LDS (256)
    static_assert(NF * NPH == 256, "output float4s must tile the block");
    __shared__ float s_zn[G];
    __shared__ float s_red[2][4][G];  // per wave: max, then sum
    __shared__ float s_w[NW_MAX][G];  // weights
    __shared__ float4 s_o[NPH > 1 ? NPH - 1 : 1][NF];
    // partial slots of this head: w + ch for the waves w whose runs of the page
    // axis meet the head's pages [pf, pl); wave of page p: ((p + 1) * W - 1) / total
    const int pf = prefix[ch], pl = prefix[ch + 1], total = prefix[H];
    // the argument lines requested beside the prefix (whose pointer and
    // count are leading arguments), one wait for both
    touch_args<offsetof(DecodeArgs, seq_ids) + 64>(&a, pf ^ pl ^ total);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const CallHead c = call_head(a, ch);
    int i0 = 0, n = 0;
    if (pl > pf) {
        const int64_t W = min(a.n_waves, total);
        const int wf = (int)(((int64_t)(pf + 1) * W - 1) / total);
        const int wl = (int)(((int64_t)pl * W - 1) / total);
        i0 = wf + ch;
        n = wl - wf + 1;
    }
    const float* part0 = P.partials + (size_t)i0 * PSTR;
    const uint16_t* qg = a.q + ((size_t)c.row * P.n_q_heads + c.h * G) * D;
    const uint16_t* kn = a.k + ((size_t)c.row * P.n_kv_heads + c.h) * D;
    const uint16_t* vn = a.v + ((size_t)c.row * P.n_kv_heads + c.h) * D;
    const int ph = tid / NF;
    const int f = ds * NF + tid % NF;  // this thread's output float4 within the head
    const int gf = (4 * f) / D;        // q head of this thread's outputs

    // first round of accumulators, and every maximum and sum
    float4 xv[RU];
#pragma unroll
    for (int j = 0; j < RU; ++j) {
        const int u = ph + j * NPH;
        xv[j] = u < n ? *reinterpret_cast<const float4*>(part0 + (size_t)u * PSTR + ACC + 4 * f)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const int gt = tid % G;
    float mi[KT], li[KT];
    float mloc = -INFINITY;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
        const int i = tid / G + k * STEP;
        mi[k] = i < n ? part0[(size_t)i * PSTR + gt] : -INFINITY;
        li[k] = i < n ? part0[(size_t)i * PSTR + G + gt] : 0.f;
        mloc = fmaxf(mloc, mi[k]);
    }
    for (int i = tid / G + NW_MAX; i < n; i += STEP) mloc = fmaxf(mloc, part0[(size_t)i * PSTR + gt]);
    // the new token: its value row and the score of each q head (one wave per q head)
    const uint2 vraw = *reinterpret_cast<const uint2*>(vn + (4 * f) % D);
    float kx[D / 64], ks = 1.f, vs = 1.f;
#pragma unroll
    for (int j = 0; j < D / 64; ++j) kx[j] = bf16_to_f32(kn[j * 64 + lane]);
    if constexpr (F8) {
        float ka = 0.f, va = 0.f;
#pragma unroll
        for (int j = 0; j < D / 64; ++j) {
            ka = fmaxf(ka, fabsf(kx[j]));
            va = fmaxf(va, fabsf(bf16_to_f32(vn[j * 64 + lane])));
        }
        ks = e4m3_row_scale(wave_max(ka));
        vs = e4m3_row_scale(wave_max(va));
#pragma unroll
        for (int j = 0; j < D / 64; ++j) kx[j] = e4m3_to_f32(e4m3_encode(kx[j] / ks));
    }
    for (int g = wave; g < G; g += 4) {
        float dp = 0.f;
#pragma unroll
        for (int j = 0; j < D / 64; ++j) dp = fmaf(bf16_to_f32(qg[g * D + j * 64 + lane]), kx[j], dp);
        const float zn = F8 ? wave_sum(dp) * ks * P.scale_log2 : wave_sum(dp) * P.scale_log2;
        if (lane == 0) s_zn[g] = zn;
    }

    // maximum per q head: the lanes with the same lane % G hold the same q head
    mloc = reduce_mod_g<G>(mloc, [](float a, float b) { return fmaxf(a, b); });
    if (lane < G) s_red[0][wave][lane] = mloc;
    __syncthreads();
    float Mt = s_red[0][0][gt];
#pragma unroll
    for (int w = 1; w < 4; ++w) Mt = fmaxf(Mt, s_red[0][w][gt]);
    float lloc = 0.f;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
        const int i = tid / G + k * STEP;
        const float wgt = (i < n && Mt != -INFINITY) ? exp2f(mi[k] - Mt) : 0.f;
        lloc = fmaf(wgt, li[k], lloc);
        s_w[i][gt] = wgt;
    }
    if (Mt != -INFINITY)
        for (int i = tid / G + NW_MAX; i < n; i += STEP)
            lloc = fmaf(exp2f(part0[(size_t)i * PSTR + gt] - Mt), part0[(size_t)i * PSTR + G + gt], lloc);
    lloc = reduce_mod_g<G>(lloc, [](float a, float b) { return a + b; });
    if (lane < G) s_red[1][wave][lane] = lloc;
    __syncthreads();

    float M = s_red[0][0][gf], L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        M = fmaxf(M, s_red[0][w][gf]);
        L += s_red[1][w][gf];
    }
    auto weight = [&](int u) -> float {
        if (u < NW_MAX) return s_w[u][gf];
        return M == -INFINITY ? 0.f : exp2f(part0[(size_t)u * PSTR + gf] - M);
    };
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int u0 = 0; u0 < n; u0 += RU * NPH) {
        if (u0 > 0) {  // a further round: its loads first
#pragma unroll
            for (int j = 0; j < RU; ++j) {
                const int u = u0 + ph + j * NPH;
                xv[j] = u < n ? *reinterpret_cast<const float4*>(part0 + (size_t)u * PSTR + ACC + 4 * f)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int j = 0; j < RU; ++j) {
            const int u = u0 + ph + j * NPH;
            if (u < n) {
                const float wgt = weight(u);
                o.x = fmaf(wgt, xv[j].x, o.x);
                o.y = fmaf(wgt, xv[j].y, o.y);
                o.z = fmaf(wgt, xv[j].z, o.z);
                o.w = fmaf(wgt, xv[j].w, o.w);
            }
        }
    }
    if (NPH > 1) {
        if (ph > 0) s_o[ph - 1][tid % NF] = o;
        __syncthreads();
        if (ph > 0) return;
#pragma unroll
        for (int q = 0; q < NPH - 1; ++q) {
            const float4 t = s_o[q][tid % NF];
            o.x += t.x;
            o.y += t.y;
            o.z += t.z;
            o.w += t.w;
        }
    }
    const float zn = s_zn[gf];
    const float mn = fmaxf(M, zn);
    const float sc = M == -INFINITY ? 0.f : exp2f(M - mn), sn = exp2f(zn - mn);
    const float den = 1.f / (L * sc + sn);
    float v0 = bf16_to_f32((uint16_t)(vraw.x & 0xffffu)), v1 = bf16_to_f32((uint16_t)(vraw.x >> 16));
    float v2 = bf16_to_f32((uint16_t)(vraw.y & 0xffffu)), v3 = bf16_to_f32((uint16_t)(vraw.y >> 16));
    if constexpr (F8) {
        v0 = e4m3_to_f32(e4m3_encode(v0 / vs)) * vs;
        v1 = e4m3_to_f32(e4m3_encode(v1 / vs)) * vs;
        v2 = e4m3_to_f32(e4m3_encode(v2 / vs)) * vs;
        v3 = e4m3_to_f32(e4m3_encode(v3 / vs)) * vs;
    }
    uint2 packed;
    packed.x = (uint32_t)f32_to_bf16((o.x * sc + sn * v0) * den) | ((uint32_t)f32_to_bf16((o.y * sc + sn * v1) * den) << 16);
    packed.y = (uint32_t)f32_to_bf16((o.z * sc + sn * v2) * den) | ((uint32_t)f32_to_bf16((o.w * sc + sn * v3) * den) << 16);
    *reinterpret_cast<uint2*>(a.out + ((size_t)c.row * P.n_q_heads + c.h * G) * D + 4 * f) = packed;
}

// Mark the new token, expire position t-w if it was marked (its slot e is
// reused), otherwise take slot n_old (a page from the shared pool when a new
// page starts), write K/V, and advance the head record.  One wave.
// FP8 pools store the token's K and V rows as E4M3 codes with their row scales.
// A page fresh from the shared pool may hold rows of a released sequence: its
// other 63 slots are cleared, so the slots past a head's live count always
// hold zeros.  The record's position is authoritative (calls replayed from a
// captured graph advance it without the host): at max_positions the token is
// dropped and the pool's sticky position flag is set.
template <int D, bool F8>
__device__ void append_head(const DecodeArgs& a, int ch) {
    constexpr int VJ = D / 64;
    const PoolDev& P = a.pool;
    const int lane = threadIdx.x & 63;
    const CallHead c = call_head(a, ch);
    int32_t* hs = P.hstate + (size_t)c.gh * kHS;
    const int n_old = hs[kHsLive];
    const int n_pages = hs[kHsPages];
    const int t = hs[kHsPos];
    const int e = hs[kHsExp];
    if (t >= P.max_positions) {
        if (lane == 0) atomicOr(&P.ctl[kCtlPosError], 1);
        return;
    }
    const uint16_t* kn = a.k + ((size_t)c.row * P.n_kv_heads + c.h) * D;
    const uint16_t* vn = a.v + ((size_t)c.row * P.n_kv_heads + c.h) * D;
    uint4 kchunk = make_uint4(0, 0, 0, 0);
    if (lane < D / 8) kchunk = *reinterpret_cast<const uint4*>(kn + lane * 8);
    uint16_t vv[VJ];
#pragma unroll
    for (int jj = 0; jj < VJ; ++jj) vv[jj] = vn[jj * 64 + lane];
    const int mark = eviction_logit(P, a.logits, a.k, c.row, c.h) > 0.f ? 1 : 0;
    // the entry of position t+1-w (expires at the next step); for w = 1 that is
    // the token written now
    const int sx = t + 1 - P.window;
    const int ring_next = (P.ring_len > 0 && sx >= 0 && P.window > 1)
                              ? P.ring[(size_t)c.gh * P.ring_len + (sx % P.window)] : -1;
    int slot, n_new, np = n_pages, page;
    bool fresh = false;  // a page just taken from the shared pool (the token goes to its slot 0)
    if (e >= 0) {
        slot = e;
        n_new = n_old;
        page = P.ptable[(size_t)c.gh * P.pages_per_head + slot / kPage];
    } else {
        slot = n_old;
        n_new = n_old + 1;
        if ((slot % kPage) == 0) {
            int pg = -1;
            if (lane == 0) {
                const int old = atomicSub(&P.ctl[kCtlTop], 1);
                if (old < 1) {
                    atomicAdd(&P.ctl[kCtlTop], 1);
                    atomicOr(&P.ctl[kCtlError], 1);
                } else {
                    pg = P.stack[old - 1];
                }
            }
            page = __shfl(pg, 0, 64);
            if (page < 0) return;  // pool exhausted: the sticky flag is set, the token is dropped
            if (lane == 0) P.ptable[(size_t)c.gh * P.pages_per_head + slot / kPage] = page;
            np = slot / kPage + 1;
            fresh = true;
        } else {
            page = P.ptable[(size_t)c.gh * P.pages_per_head + slot / kPage];
        }
    }
    const int j = slot % kPage;
    if constexpr (F8) {
        float ka = 0.f, va = 0.f;
#pragma unroll
        for (int jj = 0; jj < VJ; ++jj) {
            ka = fmaxf(ka, fabsf(bf16_to_f32(kn[jj * 64 + lane])));
            va = fmaxf(va, fabsf(bf16_to_f32(vv[jj])));
        }
        const float ks = e4m3_row_scale(wave_max(ka)), vs = e4m3_row_scale(wave_max(va));
        uint8_t* kp = P.kp8() + (size_t)page * (kPage * D);
        uint8_t* vp = P.vp8() + (size_t)page * (kPage * D);
        // every lane encodes its dims d = lane + 64 jj (the values it read for the
        // maximum) and stores each code as the byte d % 16 of chunk d / 16
#pragma unroll
        for (int jj = 0; jj < VJ; ++jj) {
            const int d = jj * 64 + lane;
            kp[((size_t)(d / 16) * kPage + j) * 16 + d % 16] = (uint8_t)e4m3_encode(bf16_to_f32(kn[d]) / ks);
        }
        if (fresh) {  // j = 0: slots 1..63 cleared (codes and scales), V units written whole
            if (lane > 0) {
#pragma unroll
                for (int cc = 0; cc < D / 16; ++cc)
                    *reinterpret_cast<uint4*>(kp + ((size_t)cc * kPage + lane) * 16) = make_uint4(0, 0, 0, 0);
                P.kscale[(size_t)page * kPage + lane] = 0.f;
                P.vscale[(size_t)page * kPage + lane] = 0.f;
            }
#pragma unroll
            for (int jj = 0; jj < VJ; ++jj) {
                const uint32_t code = e4m3_encode(bf16_to_f32(vv[jj]) / vs);
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    *reinterpret_cast<uint4*>(vp + ((size_t)b * D + jj * 64 + lane) * 16) =
                        make_uint4(b == 0 ? code : 0u, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int jj = 0; jj < VJ; ++jj)
                vp[((size_t)(j / 16) * D + jj * 64 + lane) * 16 + (j % 16)] =
                    (uint8_t)e4m3_encode(bf16_to_f32(vv[jj]) / vs);
        }
        if (lane == 0) {
            P.kscale[(size_t)page * kPage + j] = ks;
            P.vscale[(size_t)page * kPage + j] = vs;
        }
    } else {
        uint16_t* kp = P.kpages + (size_t)page * (kPage * D);
        uint16_t* vp = P.vpages + (size_t)page * (kPage * D);
        if (lane < D / 8) *reinterpret_cast<uint4*>(kp + ((size_t)lane * kPage + j) * 8) = kchunk;
        uint32_t wide = 0;  // a stored V value without an fp16 counterpart: sticky pool flag
        if (fresh) {  // j = 0: slots 1..63 cleared, V units written whole
            if (lane > 0) {
#pragma unroll
                for (int cc = 0; cc < D / 8; ++cc)
                    *reinterpret_cast<uint4*>(kp + ((size_t)cc * kPage + lane) * 8) = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int jj = 0; jj < VJ; ++jj) {
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    *reinterpret_cast<uint4*>(vp + ((size_t)b * D + jj * 64 + lane) * 8) =
                        make_uint4(b == 0 ? (uint32_t)vv[jj] : 0u, 0, 0, 0);
                wide |= bf16x2_wide(vv[jj]);
            }
        } else {
#pragma unroll
            for (int jj = 0; jj < VJ; ++jj) {
                vp[((size_t)(j / 8) * D + jj * 64 + lane) * 8 + (j % 8)] = vv[jj];
                wide |= bf16x2_wide(vv[jj]);
            }
        }
        if (wide) atomicOr(&P.ctl[kCtlVWide], 1);
    }
    if (lane == 0) {
        P.slot_pos[(size_t)page * kPage + j] = t;
        if (P.ring_len > 0) P.ring[(size_t)c.gh * P.ring_len + (t % P.window)] = (slot << 1) | mark;
        int e_next = -1;
        if (P.ring_len > 0 && sx >= 0) {
            if (P.window == 1) e_next = mark ? slot : -1;
            else if (ring_next >= 0 && (ring_next & 1)) e_next = ring_next >> 1;
        }
        hs[kHsLive] = n_new;
        hs[kHsPages] = np;
        hs[kHsPos] = t + 1;
        hs[kHsExp] = e_next;
    }
}

// Blocks 0 .. DS*H-1 merge (head b / DS, part b % DS), the next H append.
template <int D, int G, bool F8, int DS>
__global__ __launch_bounds__(256) void decode_merge_kernel(const int32_t* __restrict__ prefix, int32_t n_heads,
                                                          DecodeArgs a) {
    const int H = n_heads;
    const int b = blockIdx.x;
    if (b < DS * H) {
        merge_head<D, G, F8, DS>(a, prefix, H, b / DS, b % DS);
    } else if (threadIdx.x < 64) {
        touch_args<offsetof(DecodeArgs, seq_ids) + 64>(&a);
        append_head<D, F8>(a, b - DS * H);
    }
}

// ---------------------------------------------------------------------------
// prefill: marks, live set of the last position, page allocation, ring
// ---------------------------------------------------------------------------
constexpr int kScanChunk = 16 * 64 * 8;  // prompt positions per scan block

// Block (c, h): positions [c kScanChunk, (c+1) kScanChunk) of kv head h.  The
// live positions before the chunk are counted first (all their logits requested
// at once), so the chunks of a long prompt run side by side; the block of the
// last chunk, which then knows the head's live count, pops its pages and writes
// its record and window ring.
__global__ __launch_bounds__(1024) void prefill_scan_kernel(PrefillArgs a) {
    const PoolDev& P = a.pool;
    __shared__ int s_scan[2 * 16 + 1];
    __shared__ int s_base;
    const int tid = threadIdx.x;
    const int h = blockIdx.y;
    const int chunk = blockIdx.x;
    const int hkv = P.n_kv_heads;
    const int gh = (a.seq * P.n_layers + a.layer) * hkv + h;
    const int T = a.n_tokens, w = P.window;
    int32_t* inv = P.inv + (size_t)h * P.max_positions;
    int32_t* pcnt = P.pcnt + (size_t)h * P.max_positions;
    // live at the last position T-1: unmarked, or inside the window (s >= T - w).
    // Chunks of 8192 positions: wave v takes positions c0 + 512 v + 64 k + lane
    // (k < 8; neighbouring lanes read and write neighbouring positions, all 8
    // logits requested before any is used); ranks within the wave come from
    // ballots, the waves' offsets from one exchange through LDS.
    constexpr int KW = 8;
    const int lane = tid & 63, wave = tid >> 6;
    int n = 0;  // live positions before the current chunk
    if (chunk > 0) {
        // live(s) = s >= T - w or s unmarked; thread t reads positions t, t + 1024, ...
        // (all below chunk * kScanChunk <= T - 1)
        int cnt = 0;  // live positions of this wave's share
        const int end = chunk * kScanChunk;
        for (int s0 = 0; s0 < end; s0 += 1024 * KW) {
            float lg[KW];
#pragma unroll
            for (int k = 0; k < KW; ++k) lg[k] = eviction_logit(P, a.logits, a.k, s0 + 1024 * k + tid, h);
#pragma unroll
            for (int k = 0; k < KW; ++k) cnt += __popcll(__ballot(s0 + 1024 * k + tid >= T - w || !(lg[k] > 0.f)));
        }
        if (lane == 0) s_scan[wave] = cnt;
        __syncthreads();
#pragma unroll
        for (int v = 0; v < 16; ++v) n += s_scan[v];
        __syncthreads();  // s_scan is rewritten below
    }
    for (int c0 = chunk * kScanChunk; c0 < min(T, (chunk + 1) * kScanChunk); c0 += 16 * 64 * KW) {
        const int seg0 = c0 + wave * 64 * KW + lane;
        float lg[KW];
#pragma unroll
        for (int k = 0; k < KW; ++k) lg[k] = seg0 + 64 * k < T ? eviction_logit(P, a.logits, a.k, seg0 + 64 * k, h) : 0.f;
        uint64_t bal[KW];
        int wcount = 0;
#pragma unroll
        for (int k = 0; k < KW; ++k) {
            const int s = seg0 + 64 * k;
            bal[k] = __ballot(s < T && (s >= T - w || !(lg[k] > 0.f)));
            wcount += __popcll(bal[k]);
            // the marks of these 64 positions, for the attention's band tiles
            const uint64_t mk = __ballot(s < T && lg[k] > 0.f);
            const int s64 = s - lane;
            if (lane == 0 && s64 < T) {
                uint32_t* mb = P.mbits_of(h) + s64 / 32;
                mb[0] = (uint32_t)mk;
                mb[1] = (uint32_t)(mk >> 32);
            }
        }
        if (lane == 0) s_scan[wave] = wcount;
        __syncthreads();
        int woff = 0, tot = 0;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int c = s_scan[v];
            woff += v < wave ? c : 0;
            tot += c;
        }
        __syncthreads();  // s_scan is rewritten by the next chunk
        int off = n + woff;
#pragma unroll
        for (int k = 0; k < KW; ++k) {
            const int s = seg0 + 64 * k;
            const int rank = off + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[k] >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)bal[k], 0));
            const int live = (int)((bal[k] >> lane) & 1u);
            if (live) inv[rank] = s;
            if (s < T) pcnt[s] = rank + live;  // live tokens in [0, s]
            off += __popcll(bal[k]);
        }
        n += tot;
    }
    if (chunk != (T - 1) / kScanChunk) return;  // the head's last chunk finishes it
    const int np = (n + kPage - 1) / kPage;
    if (tid == 0) {
        const int old = atomicSub(&P.ctl[kCtlTop], np);
        if (old < np) {
            atomicAdd(&P.ctl[kCtlTop], np);
            atomicOr(&P.ctl[kCtlError], 1);
            s_base = -1;
        } else {
            s_base = old;
        }
    }
    __syncthreads();
    int32_t* hs = P.hstate + (size_t)gh * kHS;
    if (s_base < 0) {
        if (tid == 0)
            for (int i = 0; i < kHS; ++i) hs[i] = i == kHsPos ? T : (i == kHsExp ? -1 : 0);
        return;
    }
    for (int j = tid; j < np; j += 1024)
        P.ptable[(size_t)gh * P.pages_per_head + j] = P.stack[s_base - 1 - j];
    if (tid == 0) {
        // the token expiring when position T is appended: T - w, if marked; it
        // lies in the window, so its slot is n - T + (T - w)
        int e = -1;
        if (P.ring_len > 0 && T >= w && eviction_logit(P, a.logits, a.k, T - w, h) > 0.f) e = n - w;
        for (int i = 0; i < kHS; ++i) hs[i] = 0;
        hs[kHsLive] = n;
        hs[kHsPages] = np;
        hs[kHsPos] = T;
        hs[kHsExp] = e;
        if (h == 0) atomicAdd(P.rcache, 1);  // epoch: a page table written afresh
    }
    // ring entry idx holds the newest position s < T with s % w == idx (all of
    // them lie in the window, so their slots are the last ones: n - T + s)
    for (int idx = tid; idx < P.ring_len; idx += 1024) {
        int entry = -1;
        if (idx <= T - 1) {
            const int s = idx + w * ((T - 1 - idx) / w);
            const int mark = eviction_logit(P, a.logits, a.k, s, h) > 0.f ? 1 : 0;
            entry = ((n - T + s) << 1) | mark;
        }
        P.ring[(size_t)gh * P.ring_len + idx] = entry;
    }
}

// Gather the live rows into the head's pages: one block per destination page.
// Blocks past the prompt's page count copy the prompt V for the attention's band
// instead (vt_rows), alongside the gathering.
template <int D>
__global__ __launch_bounds__(256) void prefill_compact_kernel(PrefillArgs a) {
    constexpr int NC = D / 8;
    const PoolDev& P = a.pool;
    __shared__ int s_src[kPage];
    __shared__ uint16_t s_v[kPage][D + 8];
    const int ncomp = (a.n_tokens + kPage - 1) / kPage;  // blocks past these copy the prompt V
    if ((int)blockIdx.x >= ncomp) {
        vt_rows<D, false, true>(a, ((int)blockIdx.x - ncomp) * 64, blockIdx.y, s_v);
        return;
    }
    const int tid = threadIdx.x;
    const int pj = blockIdx.x, h = blockIdx.y;
    const int hkv = P.n_kv_heads;
    const int gh = (a.seq * P.n_layers + a.layer) * hkv + h;
    const int n = P.hstate[(size_t)gh * kHS + kHsLive];
    if (pj * kPage >= n) return;
    const int page = P.ptable[(size_t)gh * P.pages_per_head + pj];
    const int cnt = min(kPage, n - pj * kPage);
    if (tid < kPage) s_src[tid] = tid < cnt ? P.inv[(size_t)h * P.max_positions + pj * kPage + tid] : -1;
    __syncthreads();
    uint16_t* __restrict__ kp = P.kpages + (size_t)page * (kPage * D);
    uint16_t* vp = P.vpages + (size_t)page * (kPage * D);
    const uint16_t* __restrict__ kin = a.k;
    const uint16_t* __restrict__ vin = a.v;
    // Every K and V unit of the thread is requested before any is stored.  (Slots
    // past the live count read row 0 and store zeros: every load is a plain
    // global load, with the value selected afterwards.)
    constexpr int UT = NC * kPage / 256;  // units per thread
    static_assert(NC * kPage % 256 == 0, "K and V units tile the block");
    uint4 kx[UT], vx[UT];
#pragma unroll
    for (int x = 0; x < UT; ++x) {
        const int u = tid + 256 * x;
        const int sk = s_src[u % kPage], sv = s_src[u / NC];
        kx[x] = *reinterpret_cast<const uint4*>(kin + ((size_t)max(sk, 0) * hkv + h) * D + (u / kPage) * 8);
        vx[x] = *reinterpret_cast<const uint4*>(vin + ((size_t)max(sv, 0) * hkv + h) * D + (u % NC) * 8);
    }
    uint32_t wide = 0;  // a stored V value without an fp16 counterpart: sticky pool flag
#pragma unroll
    for (int x = 0; x < UT; ++x) {
        const int u = tid + 256 * x;
        const int j = u % kPage, cc = u / kPage;  // K unit: chunk cc of slot j
        const int vj = u / NC, vc = u % NC;       // V unit: chunk vc of slot vj
        *reinterpret_cast<uint4*>(kp + ((size_t)cc * kPage + j) * 8) = keep_if(s_src[j] >= 0, kx[x]);
        const uint4 val = keep_if(s_src[vj] >= 0, vx[x]);
        wide |= bf16x8_wide(val);
        *reinterpret_cast<uint4*>(&s_v[vj][vc * 8]) = val;
    }
    if (wide) atomicOr(&P.ctl[kCtlVWide], 1);
    __syncthreads();
    // the page, and its fp16 copy in the kv head's scratch page pj, which the
    // attention reads on its fp16-weights path (the copy is exact whenever that
    // path runs: no stored V value is wide)
    uint16_t* vh = P.vpages + (size_t)(P.xpage(h) + pj) * (kPage * D);
    for (int u = tid; u < 8 * D; u += 256) {
        const int b = u / D, d = u - b * D;
        uint32_t w4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w4[i] = (uint32_t)s_v[8 * b + 2 * i][d] | ((uint32_t)s_v[8 * b + 2 * i + 1][d] << 16);
        const uint4 x = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        *reinterpret_cast<uint4*>(vp + ((size_t)b * D + d) * 8) = x;
        *reinterpret_cast<uint4*>(vh + ((size_t)b * D + d) * 8) = bf16x8_to_f16x8(x);
    }
    if (tid < kPage) P.slot_pos[(size_t)page * kPage + tid] = s_src[tid];
}

// FP8 pools: the prompt's K and V rows as E4M3 codes and row scales, into the
// prefill scratch (row r = s * n_kv_heads + h of tensor x = K, V).  D / 8 lanes
// per row, 8 dims each; the row maximum is reduced over the row's lanes.
template <int D>
__global__ __launch_bounds__(256) void prefill_quant_kernel(PrefillArgs a) {
    constexpr int LPR = D / 8;
    const PoolDev& P = a.pool;
    const int64_t rows = (int64_t)a.n_tokens * P.n_kv_heads;  // per tensor
    const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gt / LPR;
    const int part = (int)(gt % LPR);
    const bool live = row < 2 * rows;
    const int x = live && row >= rows ? 1 : 0;
    const int64_t r = live ? row - x * rows : 0;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (live) u = *reinterpret_cast<const uint4*>((x ? a.v : a.k) + r * D + part * 8);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_to_f32((uint16_t)(w[i] & 0xffffu));
        f[2 * i + 1] = bf16_to_f32((uint16_t)(w[i] >> 16));
    }
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(f[i]));
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    const float sc = e4m3_row_scale(am);
    uint32_t c[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i / 4] |= e4m3_encode(f[i] / sc) << (8 * (i % 4));
    if (live) {
        *reinterpret_cast<uint2*>(P.q8_codes(x) + r * D + part * 8) = make_uint2(c[0], c[1]);
        if (part == 0) P.q8_scales(x)[r] = sc;
    }
}

// FP8 pools: gather the live rows' codes and scales into the head's pages, one
// block per destination page (K chunks of 16 dims key-major; V through LDS into
// 16-slot dim-major units).  Slots past the live count get zero codes and scales.
// Blocks past the prompt's page count copy the values of the prompt V's codes.
template <int D>
__global__ __launch_bounds__(256) void prefill_compact8_kernel(PrefillArgs a) {
    constexpr int NC = D / 16;
    const PoolDev& P = a.pool;
    __shared__ int s_src[kPage];
    __shared__ __attribute__((aligned(16))) uint8_t s_v[kPage][D + 16];
    __shared__ uint16_t s_vt[kPage][D + 8];
    const int ncomp = (a.n_tokens + kPage - 1) / kPage;  // blocks past these copy the prompt V's values
    if ((int)blockIdx.x >= ncomp) {
        vt_rows<D, true>(a, ((int)blockIdx.x - ncomp) * 64, blockIdx.y, s_vt);
        return;
    }
    const int tid = threadIdx.x;
    const int pj = blockIdx.x, h = blockIdx.y;
    const int hkv = P.n_kv_heads;
    const int gh = (a.seq * P.n_layers + a.layer) * hkv + h;
    const int n = P.hstate[(size_t)gh * kHS + kHsLive];
    if (pj * kPage >= n) return;
    const int page = P.ptable[(size_t)gh * P.pages_per_head + pj];
    const int cnt = min(kPage, n - pj * kPage);
    if (tid < kPage) s_src[tid] = tid < cnt ? P.inv[(size_t)h * P.max_positions + pj * kPage + tid] : -1;
    __syncthreads();
    const uint8_t* __restrict__ kq = P.q8_codes(0);
    const uint8_t* __restrict__ vq = P.q8_codes(1);
    uint8_t* __restrict__ kp = P.kp8() + (size_t)page * (kPage * D);
    uint8_t* vp = P.vp8() + (size_t)page * (kPage * D);
    // (slots past the live count read row 0 and store zeros, as above)
#pragma unroll
    for (int u = tid; u < NC * kPage; u += 256) {
        const int cc = u / kPage, j = u - cc * kPage;
        const int s = s_src[j];
        const uint4 x = *reinterpret_cast<const uint4*>(kq + ((size_t)max(s, 0) * hkv + h) * D + cc * 16);
        *reinterpret_cast<uint4*>(kp + ((size_t)cc * kPage + j) * 16) = keep_if(s >= 0, x);
    }
#pragma unroll
    for (int u = tid; u < kPage * NC; u += 256) {
        const int j = u / NC, cc = u - j * NC;
        const int s = s_src[j];
        const uint4 x = *reinterpret_cast<const uint4*>(vq + ((size_t)max(s, 0) * hkv + h) * D + cc * 16);
        *reinterpret_cast<uint4*>(&s_v[j][cc * 16]) = keep_if(s >= 0, x);
    }
    __syncthreads();
    for (int u = tid; u < 4 * D; u += 256) {
        const int b = u / D, d = u - b * D;
        uint32_t w4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w4[i] = (uint32_t)s_v[16 * b + 4 * i][d] | ((uint32_t)s_v[16 * b + 4 * i + 1][d] << 8) |
                    ((uint32_t)s_v[16 * b + 4 * i + 2][d] << 16) | ((uint32_t)s_v[16 * b + 4 * i + 3][d] << 24);
        *reinterpret_cast<uint4*>(vp + ((size_t)b * D + d) * 16) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
    if (tid < kPage) {
        const int s = s_src[tid];
        P.slot_pos[(size_t)page * kPage + tid] = s;
        P.kscale[(size_t)page * kPage + tid] = s >= 0 ? P.q8_scales(0)[(size_t)s * hkv + h] : 0.f;
        P.vscale[(size_t)page * kPage + tid] = s >= 0 ? P.q8_scales(1)[(size_t)s * hkv + h] : 0.f;
    }
}

// ---------------------------------------------------------------------------
// extend: T new tokens (input rows r = 0 .. T-1 at positions t0 + r) appended
// to the store of one (seq, layer), in position order, as T decode steps would.
// Token t reuses the slot of the token t - w expiring at its step when that one
// was marked, and takes the next fresh slot otherwise:
//   slot(r) = slot(r - w)                  if t - w >= t0 was marked (a chain)
//           = ring slot of t - w           if t0 - w <= t - w < t0 was marked
//           = n_old + #fresh rows before r otherwise
// The chains are resolved by pointer jumping (log2(T / w) rounds).  Only the
// last token of each chain is still live after the chunk, so only it is written.
// One block per kv head; slot of each row and chain parents in LDS (chunks up to
// 4096 rows; else in the inv and pcnt scratch); the slots end in inv.
// t0 is the head record's position (authoritative: calls replayed from a
// captured graph advance it without the host); a chunk that would run past
// max_positions is dropped and sets the pool's sticky position flag.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool ext_marked(const PrefillArgs& a, int r, int h) {
    return eviction_logit(a.pool, a.logits, a.k, r, h) > 0.f;
}

// the ring entry (slot << 1 | mark) of stored position u (t0 - w <= u < t0), or -1
__device__ __forceinline__ int ext_ring(const PoolDev& P, int gh, int u) {
    return (P.ring_len > 0 && u >= 0) ? P.ring[(size_t)gh * P.ring_len + u % P.window] : -1;
}

__global__ __launch_bounds__(1024) void extend_update_kernel(PrefillArgs a) {
    const PoolDev& P = a.pool;
    constexpr int kLdsRows = 4096;  // chunks up to this many rows keep the arrays in LDS
    __shared__ int s_scan[2 * 16 + 1];
    __shared__ int s_base, s_enext;
    __shared__ int s_val[kLdsRows], s_par[kLdsRows];
    const int tid = threadIdx.x, h = blockIdx.x;
    const int gh = (a.seq * P.n_layers + a.layer) * P.n_kv_heads + h;
    int32_t* hs = P.hstate + (size_t)gh * kHS;
    const int n_old = hs[kHsLive], np_old = hs[kHsPages];
    const int T = a.n_tokens, t0 = hs[kHsPos], w = P.window;
    const bool in_lds = T <= kLdsRows;
    int32_t* const gval = P.inv + (size_t)h * P.max_positions;
    int32_t* val = in_lds ? s_val : gval;                                    // slot of row r (roots: final)
    int32_t* par = in_lds ? s_par : P.pcnt + (size_t)h * P.max_positions;  // chain parent of row r (itself at a root)
    auto publish = [&]() {  // the write kernel reads the slots from the inv scratch
        if (in_lds) {
            __syncthreads();
            for (int r = tid; r < T; r += 1024) gval[r] = s_val[r];
        }
    };
    if ((int64_t)t0 + T > P.max_positions) {  // nothing is stored: every row's slot is -1
        if (tid == 0) atomicOr(&P.ctl[kCtlPosError], 1);
        for (int r = tid; r < T; r += 1024) gval[r] = -1;
        return;
    }
    const bool evict = P.ring_len > 0;
    const int per = (T + 1023) / 1024;
    const int r0 = min(tid * per, T), r1 = min(r0 + per, T);
    // fresh rows and their ranks
    int cnt = 0;
    for (int r = r0; r < r1; ++r) {
        const int u = t0 + r - w;  // expires at this step if marked
        bool reuse = false;
        if (evict && u >= 0) {
            if (u >= t0) reuse = ext_marked(a, u - t0, h);
            else { const int e = ext_ring(P, gh, u); reuse = e >= 0 && (e & 1); }
        }
        par[r] = reuse ? -1 : r;
        cnt += reuse ? 0 : 1;
    }
    int fresh;
    int off = block_excl_scan<1024>(cnt, &fresh, s_scan);
    for (int r = r0; r < r1; ++r) {
        const int u = t0 + r - w;
        if (par[r] == r) {
            val[r] = n_old + off++;
        } else if (u >= t0) {
            par[r] = u - t0;
        } else {
            par[r] = r;
            val[r] = ext_ring(P, gh, u) >> 1;
        }
    }
    __syncthreads();
    // pointer jumping: every parent read is an ancestor, so in-place is safe
    for (;;) {
        int changed = 0;
        for (int r = r0; r < r1; ++r) {
            const int p = par[r], pp = par[p];
            if (pp != p) {
                par[r] = pp;
                changed = 1;
            }
        }
        if (!__syncthreads_or(changed)) break;
    }
    for (int r = r0; r < r1; ++r) val[r] = val[par[r]];  // roots keep their value
    // the slot expiring when position t0 + T is appended (before the ring changes)
    if (tid == 0) {
        int e = -1;
        const int u = t0 + T - w;
        if (evict && u >= 0) {
            if (u >= t0) {
                if (ext_marked(a, u - t0, h)) e = -2;  // a new row: its slot, below
            } else {
                const int re = ext_ring(P, gh, u);
                if (re >= 0 && (re & 1)) e = re >> 1;
            }
        }
        s_enext = e;
    }
    __syncthreads();
    // pages for the fresh slots
    const int n_new = n_old + fresh;
    const int np_new = (n_new + kPage - 1) / kPage;
    const int need = np_new - np_old;
    if (tid == 0) {
        s_base = 0;
        if (need > 0) {
            const int old = atomicSub(&P.ctl[kCtlTop], need);
            if (old < need) {
                atomicAdd(&P.ctl[kCtlTop], need);
                atomicOr(&P.ctl[kCtlError], 1);
                s_base = -1;
            } else {
                s_base = old;
            }
        }
    }
    __syncthreads();
    if (s_base < 0) {  // pool exhausted: the sticky flag is set, the chunk is dropped
        if (tid == 0) hs[kHsPos] = t0 + T;
        for (int r = r0; r < r1; ++r) val[r] = -1;
        publish();
        return;
    }
    for (int j = tid; j < need; j += 1024)
        P.ptable[(size_t)gh * P.pages_per_head + np_old + j] = P.stack[s_base - 1 - j];
    // Pages fresh from the shared pool may hold rows of a released sequence.
    // Every new page but the last is filled by the chunk's fresh slots; the last
    // one is cleared here whole (the write kernel, which runs after this one,
    // fills its slots below n_new), so slots past the live count hold zeros.
    if (need > 0) {
        const size_t pg = (size_t)P.stack[s_base - need];
        const int D = P.head_dim;
        const int pbytes = kPage * D * (P.fp8 ? 1 : 2);
        uint4* kz = reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(P.kpages) + pg * pbytes);
        uint4* vz = reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(P.vpages) + pg * pbytes);
        for (int u = tid; u < pbytes / 16; u += 1024) {
            kz[u] = make_uint4(0, 0, 0, 0);
            vz[u] = make_uint4(0, 0, 0, 0);
        }
        if (P.fp8 && tid < kPage) {
            P.kscale[pg * kPage + tid] = 0.f;
            P.vscale[pg * kPage + tid] = 0.f;
        }
    }
    // ring entries of the last w positions that are new
    if (evict)
        for (int r = max(0, T - w) + tid; r < T; r += 1024)
            P.ring[(size_t)gh * P.ring_len + (t0 + r) % w] = (val[r] << 1) | (ext_marked(a, r, h) ? 1 : 0);
    if (tid == 0) {
        int e = s_enext;
        if (e == -2) e = val[t0 + T - w - t0];
        hs[kHsLive] = n_new;
        hs[kHsPages] = np_new;
        hs[kHsPos] = t0 + T;
        hs[kHsExp] = e;
    }
    publish();
}

// K/V (FP8: codes and scales) of the rows still live after the chunk into their
// slots: row r is overwritten within the chunk iff it is marked and r + w < T.
// Grid (ceil(T / 64), n_kv_heads), 256 threads.
template <int D, bool F8>
__global__ __launch_bounds__(256) void extend_write_kernel(PrefillArgs a) {
    const PoolDev& P = a.pool;
    __shared__ int s_slot[64], s_page[64];  // per row: destination slot (-1: not written) and its page
    const int tid = threadIdx.x, h = blockIdx.y, rb = blockIdx.x * 64;
    const int hkv = P.n_kv_heads, T = a.n_tokens, w = P.window;
    const int gh = (a.seq * P.n_layers + a.layer) * hkv + h;
    if (tid < 64) {
        const int r = rb + tid;
        int slot = -1;
        if (r < T) {
            slot = P.inv[(size_t)h * P.max_positions + r];
            if (P.ring_len > 0 && r + w < T && ext_marked(a, r, h)) slot = -1;  // replaced within the chunk
        }
        s_slot[tid] = slot;
        s_page[tid] = slot >= 0 ? P.ptable[(size_t)gh * P.pages_per_head + slot / kPage] : 0;
    }
    __syncthreads();
    if constexpr (F8) {
        constexpr int NC = D / 16;
        for (int u = tid; u < 64 * NC; u += 256) {  // K: 16 codes per chunk
            const int j = u / NC, cc = u - j * NC;
            const int slot = s_slot[j];
            if (slot < 0) continue;
            const size_t row = (size_t)(rb + j) * hkv + h;
            uint8_t* kp = P.kp8() + (size_t)s_page[j] * (kPage * D);
            *reinterpret_cast<uint4*>(kp + ((size_t)cc * kPage + slot % kPage) * 16) =
                *reinterpret_cast<const uint4*>(P.q8_codes(0) + row * D + cc * 16);
        }
        for (int u = tid; u < 64 * D; u += 256) {  // V: one code per (row, dim)
            const int j = u / D, d = u - j * D;
            const int slot = s_slot[j];
            if (slot < 0) continue;
            const size_t row = (size_t)(rb + j) * hkv + h;
            uint8_t* vp = P.vp8() + (size_t)s_page[j] * (kPage * D);
            vp[((size_t)(slot % kPage / 16) * D + d) * 16 + slot % 16] = P.q8_codes(1)[row * D + d];
        }
    } else {
        constexpr int NC = D / 8;
        for (int u = tid; u < 64 * NC; u += 256) {  // K: 8 dims per chunk
            const int j = u / NC, cc = u - j * NC;
            const int slot = s_slot[j];
            if (slot < 0) continue;
            const size_t row = (size_t)(rb + j) * hkv + h;
            uint16_t* kp = P.kpages + (size_t)s_page[j] * (kPage * D);
            *reinterpret_cast<uint4*>(kp + ((size_t)cc * kPage + slot % kPage) * 8) =
                *reinterpret_cast<const uint4*>(a.k + row * D + cc * 8);
        }
        uint32_t wide = 0;  // a stored V value without an fp16 counterpart: sticky pool flag
        for (int u = tid; u < 64 * NC; u += 256) {  // V: 8 dims of a row per thread, one value per unit
            const int j = u / NC, cc = u - j * NC;
            const int slot = s_slot[j];
            if (slot < 0) continue;
            const size_t row = (size_t)(rb + j) * hkv + h;
            uint16_t* vp = P.vpages + (size_t)s_page[j] * (kPage * D) + (size_t)(slot % kPage / 8) * D * 8 + slot % 8;
            const uint4 x = *reinterpret_cast<const uint4*>(a.v + row * D + cc * 8);
            wide |= bf16x8_wide(x);
            const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int q = 0; q < 8; ++q)
                vp[(size_t)(cc * 8 + q) * 8] = (uint16_t)(q & 1 ? xw[q / 2] >> 16 : xw[q / 2] & 0xffffu);
        }
        if (wide) atomicOr(&P.ctl[kCtlVWide], 1);
    }
    if (tid < 64 && s_slot[tid] >= 0) {
        const int slot = s_slot[tid];
        const size_t sl = (size_t)s_page[tid] * kPage + slot % kPage;
        // the update kernel advanced the record's position past the chunk
        P.slot_pos[sl] = P.hstate[(size_t)gh * kHS + kHsPos] - T + rb + tid;
        if constexpr (F8) {
            const size_t row = (size_t)(rb + tid) * hkv + h;
            P.kscale[sl] = P.q8_scales(0)[row];
            P.vscale[sl] = P.q8_scales(1)[row];
        }
    }
}

__global__ __launch_bounds__(64) void seq_release_kernel(PoolDev P, int seq) {
    const int gh = seq * P.n_layers * P.n_kv_heads + blockIdx.x;
    int32_t* hs = P.hstate + (size_t)gh * kHS;
    const int np = hs[kHsPages];
    int base = 0;
    if (threadIdx.x == 0 && np > 0) base = atomicAdd(&P.ctl[kCtlTop], np);
    base = __shfl(base, 0, 64);
    for (int j = threadIdx.x; j < np; j += 64) P.stack[base + j] = P.ptable[(size_t)gh * P.pages_per_head + j];
    if (threadIdx.x == 0) {
        for (int i = 0; i < kHS; ++i) hs[i] = i == kHsExp ? -1 : 0;
        if (blockIdx.x == 0) atomicAdd(P.rcache, 1);  // epoch: the freed pages' table entries are stale
    }
}

size_t decode_shm(const DecodeArgs& a) { return (size_t)(4 * a.n_call_heads + 1) * sizeof(int32_t); }

// ev (optional): start/stop of the attention kernel, then of the merge kernel,
// taken by the dispatches themselves (kernel execution only)
template <int D, int G, bool F8>
hipError_t launch_decode_f(const DecodeArgs& a, int grid, hipStream_t s, hipEvent_t* ev) {
    // the plan's first loads need the head records, the call's head count and
    // what the global head ids are made of (for a call of one sequence, the id
    // of its first head: the others follow it): leading arguments, which the
    // dispatch places in registers (kernel-argument preloading)
    const int32_t gh0 = a.n_seqs == 1 ? (a.seq_ids[0] * a.pool.n_layers + a.layer0) * a.pool.n_kv_heads : -1;
    // calls of one layer of one sequence: the kernel with the page cache
    if (a.n_seqs == 1 && a.n_layers == 1)
        hipExtLaunchKernelGGL((decode_attend_kernel<D, G, F8, true>), dim3(grid), dim3(64 * kAttendWaves),
                              decode_shm(a), s, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr, 0,
                              (const int32_t*)a.pool.hstate, gh0, a.n_call_heads, a.pool.n_kv_heads, a.n_seqs,
                              a.pool.n_layers, a.layer0, a);
    else
        hipExtLaunchKernelGGL((decode_attend_kernel<D, G, F8, false>), dim3(grid), dim3(64 * kAttendWaves),
                              decode_shm(a), s, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr, 0,
                              (const int32_t*)a.pool.hstate, gh0, a.n_call_heads, a.pool.n_kv_heads, a.n_seqs,
                              a.pool.n_layers, a.layer0, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // A head whose outputs fill 128 or more threads' float4s holds at most 32
    // partials per round.  In a call with many partials per head (few heads, e.g.
    // one layer of one sequence) its merge is spread over 4 blocks.  (The
    // attention grid never exceeds the call's page bound by a block, so
    // n_waves / H bounds the partials of an average head.)
    if (G * D / 4 >= 128 && a.n_waves > 8 * a.n_call_heads)
        hipExtLaunchKernelGGL((decode_merge_kernel<D, G, F8, 4>), dim3(5 * a.n_call_heads), dim3(256), 0, s,
                              ev ? ev[2] : nullptr, ev ? ev[3] : nullptr, 0, (const int32_t*)a.pool.prefix,
                              a.n_call_heads, a);
    else
        hipExtLaunchKernelGGL((decode_merge_kernel<D, G, F8, 1>), dim3(2 * a.n_call_heads), dim3(256), 0, s,
                              ev ? ev[2] : nullptr, ev ? ev[3] : nullptr, 0, (const int32_t*)a.pool.prefix,
                              a.n_call_heads, a);
    return hipGetLastError();
}

template <int D, int G>
hipError_t launch_decode_t(const DecodeArgs& a, int grid, hipStream_t s, hipEvent_t* ev) {
    return a.pool.fp8 ? launch_decode_f<D, G, true>(a, grid, s, ev) : launch_decode_f<D, G, false>(a, grid, s, ev);
}

template <int D, int G>
int blocks_per_cu_t(const DecodeArgs& a) {
    // (the smaller count of the kernel's two forms, with and without the page cache)
    int n = 0, m = 0;
    hipError_t e, f;
    if (a.pool.fp8) {
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_attend_kernel<D, G, true, false>,
                                                         64 * kAttendWaves, decode_shm(a));
        f = hipOccupancyMaxActiveBlocksPerMultiprocessor(&m, decode_attend_kernel<D, G, true, true>,
                                                         64 * kAttendWaves, decode_shm(a));
    } else {
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_attend_kernel<D, G, false, false>,
                                                         64 * kAttendWaves, decode_shm(a));
        f = hipOccupancyMaxActiveBlocksPerMultiprocessor(&m, decode_attend_kernel<D, G, false, true>,
                                                         64 * kAttendWaves, decode_shm(a));
    }
    return e == hipSuccess && f == hipSuccess ? std::min(n, m) : 0;
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, int grid, hipStream_t s, hipEvent_t* ev) {
    switch (a.pool.n_q_heads / a.pool.n_kv_heads) {
        case 1: return launch_decode_t<D, 1>(a, grid, s, ev);
        case 2: return launch_decode_t<D, 2>(a, grid, s, ev);
        case 4: return launch_decode_t<D, 4>(a, grid, s, ev);
        case 8: return launch_decode_t<D, 8>(a, grid, s, ev);
    }
    return hipErrorInvalidValue;
}

template <int D>
int blocks_per_cu_d(const DecodeArgs& a) {
    switch (a.pool.n_q_heads / a.pool.n_kv_heads) {
        case 1: return blocks_per_cu_t<D, 1>(a);
        case 2: return blocks_per_cu_t<D, 2>(a);
        case 4: return blocks_per_cu_t<D, 4>(a);
        case 8: return blocks_per_cu_t<D, 8>(a);
    }
    return 0;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int grid, hipStream_t s, hipEvent_t* ev) {
    if (a.pool.head_dim == 128) return launch_decode_d<128>(a, grid, s, ev);
    if (a.pool.head_dim == 64) return launch_decode_d<64>(a, grid, s, ev);
    return hipErrorInvalidValue;
}

int decode_blocks_per_cu(const DecodeArgs& a) {
    return a.pool.head_dim == 128 ? blocks_per_cu_d<128>(a) : blocks_per_cu_d<64>(a);
}

hipError_t launch_prefill_compact(const PrefillArgs& a, bool with_vt, hipStream_t s, hipEvent_t start,
                                  hipEvent_t stop) {
    const bool d128 = a.pool.head_dim == 128;
    if (a.pool.fp8) {  // quantise the prompt first (the compaction gathers codes)
        const int64_t threads = (int64_t)2 * a.n_tokens * a.pool.n_kv_heads * (a.pool.head_dim / 8);
        const dim3 qgrid((unsigned)((threads + 255) / 256));
        if (d128) hipExtLaunchKernelGGL(prefill_quant_kernel<128>, qgrid, dim3(256), 0, s, start, nullptr, 0, a);
        else hipExtLaunchKernelGGL(prefill_quant_kernel<64>, qgrid, dim3(256), 0, s, start, nullptr, 0, a);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        start = nullptr;
    }
    hipExtLaunchKernelGGL(prefill_scan_kernel, dim3((a.n_tokens + kScanChunk - 1) / kScanChunk, a.pool.n_kv_heads),
                          dim3(1024), 0, s, start, nullptr, 0, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // one block per page of live slots (those past the head's count return at
    // once), then with_vt one block per 64 prompt rows for the V copy
    const int ncomp = (a.n_tokens + kPage - 1) / kPage;
    const dim3 grid(ncomp + (with_vt ? (a.n_tokens + 63) / 64 : 0), a.pool.n_kv_heads);
    if (a.pool.fp8) {
        if (d128) hipExtLaunchKernelGGL(prefill_compact8_kernel<128>, grid, dim3(256), 0, s, nullptr, stop, 0, a);
        else hipExtLaunchKernelGGL(prefill_compact8_kernel<64>, grid, dim3(256), 0, s, nullptr, stop, 0, a);
    } else {
        if (d128) hipExtLaunchKernelGGL(prefill_compact_kernel<128>, grid, dim3(256), 0, s, nullptr, stop, 0, a);
        else hipExtLaunchKernelGGL(prefill_compact_kernel<64>, grid, dim3(256), 0, s, nullptr, stop, 0, a);
    }
    return hipGetLastError();
}

hipError_t launch_extend(const PrefillArgs& a, bool with_out, hipStream_t s, hipEvent_t* ev) {
    const bool d128 = a.pool.head_dim == 128;
    hipError_t err;
    if (a.pool.fp8) {  // the chunk's codes and scales: read by the attention and the writes
        const int64_t threads = (int64_t)2 * a.n_tokens * a.pool.n_kv_heads * (a.pool.head_dim / 8);
        const dim3 qgrid((unsigned)((threads + 255) / 256));
        if (d128) hipLaunchKernelGGL(prefill_quant_kernel<128>, qgrid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL(prefill_quant_kernel<64>, qgrid, dim3(256), 0, s, a);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (with_out && (err = launch_extend_attend(a, s, ev)) != hipSuccess) return err;
    hipLaunchKernelGGL(extend_update_kernel, dim3(a.pool.n_kv_heads), dim3(1024), 0, s, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const dim3 grid((a.n_tokens + 63) / 64, a.pool.n_kv_heads);
    if (a.pool.fp8) {
        if (d128) hipLaunchKernelGGL((extend_write_kernel<128, true>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((extend_write_kernel<64, true>), grid, dim3(256), 0, s, a);
    } else {
        if (d128) hipLaunchKernelGGL((extend_write_kernel<128, false>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((extend_write_kernel<64, false>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void page_cache_clear_kernel(int32_t* e, int32_t n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) e[i] = -1;
}

hipError_t launch_page_cache_clear(const PoolDev& p, hipStream_t s) {
    constexpr int n = kRunCacheRows * kRunCacheRuns * 4;
    hipLaunchKernelGGL(page_cache_clear_kernel, dim3(256), dim3(256), 0, s, p.rcache + kRunCacheHeader, n);
    return hipGetLastError();
}

hipError_t launch_seq_release(const PoolDev& p, int32_t seq, hipStream_t s) {
    hipLaunchKernelGGL(seq_release_kernel, dim3(p.n_layers * p.n_kv_heads), dim3(64), 0, s, p, seq);
    return hipGetLastError();
}

int device_cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
}

}  // namespace dms
