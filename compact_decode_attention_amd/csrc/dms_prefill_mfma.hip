// Masked causal prefill attention on MFMA (gfx950, v_mfma_f32_32x32x16_bf16).
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
// The G waves of a block are the G q heads sharing one kv head, so each K/V
// tile is read by one block for all of them.
#include "dms_internal.h"

#include <math.h>

namespace dms {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    auto rne = [](float f) -> uint32_t {
        uint32_t u = __float_as_uint(f);
        u += 0x7fffu + ((u >> 16) & 1u);
        return u >> 16;
    };
    return rne(lo) | (rne(hi) << 16);
}

__device__ __forceinline__ uint16_t bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// row index of the S^T tile -> key index within the 32-key tile: bits 2 and 3 swapped
__device__ __forceinline__ int swap23(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// ---------------------------------------------------------------------------
// prompt V -> vt[h][s/8][d][8] (8 consecutive tokens of one dim per 16 bytes),
// zero beyond the prompt up to the next multiple of 32
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void prefill_vt_kernel(PrefillArgs a) {
    const PoolDev& P = a.pool;
    __shared__ uint16_t s_v[64][D + 8];
    const int tid = threadIdx.x;
    const int s0 = blockIdx.x * 64, h = blockIdx.y;
    const int T = a.n_tokens, hkv = P.n_kv_heads;
    const int T32 = (T + 31) / 32 * 32;
    constexpr int NC = D / 8;
    for (int u = tid; u < 64 * NC; u += 256) {
        const int j = u / NC, cc = u - j * NC;
        const int s = s0 + j;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (s < T) val = *reinterpret_cast<const uint4*>(a.v + ((size_t)s * hkv + h) * D + cc * 8);
        *reinterpret_cast<uint4*>(&s_v[j][cc * 8]) = val;
    }
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
        *reinterpret_cast<uint4*>(vt + ((size_t)blk * D + d) * 8) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
}

// ---------------------------------------------------------------------------
// masked prefill attention, one block = (kv head, 32-query tile), one wave per q head
// ---------------------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(64 * G) void prefill_attend_kernel(PrefillArgs a) {
    constexpr int KS = D / 16;  // k-steps of S^T = K Q^T over the head dim
    constexpr int DT = D / 32;  // 32-row tiles of O^T
    const PoolDev& P = a.pool;
    const int T = a.n_tokens, w = P.window, hkv = P.n_kv_heads, hq_n = P.n_q_heads;
    const int nqt = (T + 31) / 32;
    // Blocks b, b+8, b+16, ... are placed on the same XCD; hand each XCD a run of
    // consecutive (kv head, query tile) pairs so that a head's keys stay in that
    // XCD's L2.  Later tiles (more keys) first.
    const int total = hkv * nqt;
    const int per_xcd = (total + 7) / 8;
    const int pidx = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (pidx >= total) return;
    const int h = pidx / nqt;
    const int t0 = (nqt - 1 - pidx % nqt) * 32;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hq = h * G + wave;
    const int gh = (a.seq * P.n_layers + a.layer) * hkv + h;
    const int col = lane & 31, half = lane >> 5;
    const int tq = t0 + col;  // this lane's query
    const float sl = P.scale_log2;

    // Q^T as the B operand: column = query, 8 consecutive dims per half-wave
    uint4 qb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qb[ks] = tq < T ? *reinterpret_cast<const uint4*>(a.q + ((size_t)tq * hq_n + hq) * D + ks * 16 + half * 8)
                        : make_uint4(0, 0, 0, 0);

    f32x16_t o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16_t{};
    float m = -INFINITY, lsum = 0.f;
    const int krow = swap23(col);  // key this lane feeds as A-operand row

    // fold one 32-key tile (scores in s) into the running state; valid per reg
    auto fold = [&](f32x16_t s, const uint32_t (&vmask)[1], const uint4 (&va)[DT][2]) {
        float z[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            z[r] = ((vmask[0] >> r) & 1u) ? s[r] * sl : -INFINITY;
            tmax = fmaxf(tmax, z[r]);
        }
        tmax = fmaxf(tmax, xor32(tmax));
        const float mn = fmaxf(m, tmax);
        float alpha = 1.f;
        // P^T enters the PV product as two bf16 parts, hi = bf16(p) and
        // lo = bf16(p - hi): about 16 significant bits, fp32 accumulation
        uint32_t ph[8], pl[8];
        if (mn == -INFINITY) {
#pragma unroll
            for (int i = 0; i < 8; ++i) ph[i] = pl[i] = 0;
        } else {
            alpha = exp2f(m - mn);
            float ps = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p0 = exp2f(z[2 * i] - mn), p1 = exp2f(z[2 * i + 1] - mn);
                ph[i] = pack_bf16x2(p0, p1);
                pl[i] = pack_bf16x2(p0 - bf16_f(ph[i] & 0xffffu), p1 - bf16_f(ph[i] >> 16));
                ps += p0 + p1;
            }
            lsum = lsum * alpha + ps;
            m = mn;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const uint4 hb = make_uint4(ph[4 * kk], ph[4 * kk + 1], ph[4 * kk + 2], ph[4 * kk + 3]);
                const uint4 lb = make_uint4(pl[4 * kk], pl[4 * kk + 1], pl[4 * kk + 2], pl[4 * kk + 3]);
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[dt][kk]), as_bf16x8(hb), o[dt], 0, 0, 0);
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[dt][kk]), as_bf16x8(lb), o[dt], 0, 0, 0);
            }
        }
    };

    // ---- far field: the first U slots of the compacted store
    const int xf = t0 - w;
    const int U = xf >= 0 ? P.pcnt[(size_t)h * P.max_positions + xf] : 0;
    for (int kb = 0; kb < U; kb += 32) {
        const int page = P.ptable[(size_t)gh * P.pages_per_head + kb / kPage];
        const uint16_t* kp = P.kpages + (size_t)page * (kPage * D);
        const uint16_t* vp = P.vpages + (size_t)page * (kPage * D);
        const int off = kb % kPage;
        f32x16_t s = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint4 ka = *reinterpret_cast<const uint4*>(kp + ((size_t)(2 * ks + half) * kPage + off + krow) * 8);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka), as_bf16x8(qb[ks]), s, 0, 0, 0);
        }
        uint4 va[DT][2];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                va[dt][kk] = *reinterpret_cast<const uint4*>(
                    vp + ((size_t)((off + 16 * kk + 8 * half) / 8) * D + dt * 32 + col) * 8);
        uint32_t vmask[1] = {0};
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kb + (r & 7) + 8 * half + 16 * (r >> 3);
            vmask[0] |= (key < U ? 1u : 0u) << r;
        }
        fold(s, vmask, va);
    }

    // ---- band: keys (t0 - w, t0 + 31], from the prompt, masked per pair
    const int sb0 = max(0, t0 - w + 1);
    const int kend = min(T, t0 + 32);
    const uint16_t* vt = P.vt + (size_t)h * (P.max_pos32 / 8) * D * 8;
    for (int kb = sb0 / 32 * 32; kb < kend; kb += 32) {
        const int sk = kb + krow;
        f32x16_t s = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint4 ka = sk < T ? *reinterpret_cast<const uint4*>(a.k + ((size_t)sk * hkv + h) * D + ks * 16 + half * 8)
                                    : make_uint4(0, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka), as_bf16x8(qb[ks]), s, 0, 0, 0);
        }
        uint4 va[DT][2];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                va[dt][kk] = *reinterpret_cast<const uint4*>(
                    vt + ((size_t)((kb + 16 * kk + 8 * half) / 8) * D + dt * 32 + col) * 8);
        // marks of the tile's 32 keys, one bit per key
        const int sm = kb + col;
        const bool mk = sm < T && a.logits[(size_t)sm * hkv + h] > 0.f;
        const uint32_t marks = (uint32_t)__ballot(mk && half == 0);
        uint32_t vmask[1] = {0};
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kr = (r & 7) + 8 * half + 16 * (r >> 3);
            const int key = kb + kr;
            const bool marked = (marks >> kr) & 1u;
            const bool vis = key > xf && key <= tq && tq < T && (!marked || tq < key + w);
            vmask[0] |= (vis ? 1u : 0u) << r;
        }
        fold(s, vmask, va);
    }

    // ---- normalise and store: lane holds dims dt*32 + 8*(r/4) + 4*half + r%4 of query tq
    const float ltot = lsum + xor32(lsum);
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

template <int D, int G>
hipError_t launch_attend_t(const PrefillArgs& a, hipStream_t s) {
    const int nqt = (a.n_tokens + 31) / 32;
    const int total = a.pool.n_kv_heads * nqt;
    const int grid = 8 * ((total + 7) / 8);
    hipLaunchKernelGGL((prefill_attend_kernel<D, G>), dim3(grid), dim3(64 * G), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_attend_d(const PrefillArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(prefill_vt_kernel<D>, dim3((a.n_tokens + 63) / 64, a.pool.n_kv_heads), dim3(256), 0, s, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    switch (a.pool.n_q_heads / a.pool.n_kv_heads) {
        case 1: return launch_attend_t<D, 1>(a, s);
        case 2: return launch_attend_t<D, 2>(a, s);
        case 4: return launch_attend_t<D, 4>(a, s);
        case 8: return launch_attend_t<D, 8>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// Runs after the compaction kernels of the same prefill (same stream): the far
// field reads the pages and the live-count prefix they wrote.
hipError_t launch_prefill_attend(const PrefillArgs& a, hipStream_t s) {
    if (a.pool.head_dim == 128) return launch_attend_d<128>(a, s);
    if (a.pool.head_dim == 64) return launch_attend_d<64>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace dms
