// Device helpers shared by the gfx950 kernels of libspecv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specv.h"

namespace specv {

constexpr int kWave = 64;   // CDNA wavefront width

// Workspace header, padded to 256 bytes. `status` holds the data-error bits of
// the last completed call (specv_read_status reads this first word).
struct WsHeader {
    uint32_t status;
    uint32_t pad[63];
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// A pointer into device global memory, for loads through pointers the compiler
// cannot trace to a kernel argument (read from LDS, say): without it they become
// flat loads, which also count in lgkmcnt, so every later LDS wait would wait for
// them as well.
template <typename U>
__device__ __forceinline__ const __attribute__((address_space(1))) U* as_global(const U* p) {
    return (const __attribute__((address_space(1))) U*)(p);
}

// Storage traits: 16-byte vector of logits, widened to float.
template <int DT> struct Logit;

template <> struct Logit<SPECV_BF16> {
    using T = uint16_t;
    static constexpr int kVec = 8;                 // elements per 16-byte load
    __device__ static __forceinline__ float load1(const T* p) {
        return __uint_as_float(static_cast<uint32_t>(*as_global(p)) << 16);
    }
    __device__ static __forceinline__ void unpack(const uint4& v, float (&x)[8]) {
        x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
        x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
        x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
        x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
    }
};

template <> struct Logit<SPECV_F32> {
    using T = float;
    static constexpr int kVec = 4;
    __device__ static __forceinline__ float load1(const T* p) { return *as_global(p); }
    __device__ static __forceinline__ void unpack(const uint4& v, float (&x)[4]) {
        x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
        x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
    }
};

// ---- wavefront reductions (xor butterflies: every lane ends with the result) ----

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
    return v;
}

// (value, index) maximum: larger value wins, equal values go to the lower index.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float v2 = __shfl_xor(v, o, kWave);
        int i2 = __shfl_xor(i, o, kWave);
        argmax_merge(v, i, v2, i2);
    }
}

// Online log-sum-exp state in base 2: the sum of exp2(a - m) over the elements
// seen, a = logit * log2(e) / tau. An empty state is (-inf, 0).
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
    float mm = fmaxf(m, m2);
    if (mm == -INFINITY) return;
    float e1 = (m == -INFINITY) ? 0.f : exp2f(m - mm);
    float e2 = (m2 == -INFINITY) ? 0.f : exp2f(m2 - mm);
    s = s * e1 + s2 * e2;
    m = mm;
}

__device__ __forceinline__ void wave_lse(float& m, float& s) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float m2 = __shfl_xor(m, o, kWave);
        float s2 = __shfl_xor(s, o, kWave);
        lse_merge(m, s, m2, s2);
    }
}

// ---- DPP wavefront reductions: quad permutes, row mirrors and the two row
// broadcasts leave the reduction of all 64 lanes in lane 63, which is then read
// into a scalar. Every lane of the wave must be active.

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_i(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, false);
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float old, float v) {
    return __int_as_float(dpp_i<CTRL, ROW_MASK>(__float_as_int(old), __float_as_int(v)));
}
__device__ __forceinline__ float lane63(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over the wave (fixed order, identical on every call with the same data).
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += dpp_f<0xb1>(0.f, v);          // quad_perm [1,0,3,2]
    v += dpp_f<0x4e>(0.f, v);          // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(0.f, v);         // row_half_mirror
    v += dpp_f<0x140>(0.f, v);         // row_mirror
    v += dpp_f<0x142, 0xa>(0.f, v);    // row_bcast:15 into rows 1 and 3
    v += dpp_f<0x143, 0xc>(0.f, v);    // row_bcast:31 into rows 2 and 3
    return lane63(v);
}

__device__ __forceinline__ float wave_max_dpp(float v) {
    v = fmaxf(v, dpp_f<0xb1>(v, v));
    v = fmaxf(v, dpp_f<0x4e>(v, v));
    v = fmaxf(v, dpp_f<0x141>(v, v));
    v = fmaxf(v, dpp_f<0x140>(v, v));
    v = fmaxf(v, dpp_f<0x142, 0xa>(v, v));
    v = fmaxf(v, dpp_f<0x143, 0xc>(v, v));
    return lane63(v);
}

// Minimum of an int over the wave (all lanes active), as a scalar.
__device__ __forceinline__ int wave_min_int_dpp(int v) {
    v = min(v, dpp_i<0xb1>(v, v));
    v = min(v, dpp_i<0x4e>(v, v));
    v = min(v, dpp_i<0x141>(v, v));
    v = min(v, dpp_i<0x140>(v, v));
    v = min(v, dpp_i<0x142, 0xa>(v, v));
    v = min(v, dpp_i<0x143, 0xc>(v, v));
    return __builtin_amdgcn_readlane(v, 63);
}

// (value, index) maximum over the wave, larger value first, then lower index.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ void argmax_dpp_step(float& v, int& i) {
    const float v2 = dpp_f<CTRL, ROW_MASK>(v, v);
    const int i2 = dpp_i<CTRL, ROW_MASK>(i, i);
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}
__device__ __forceinline__ void wave_argmax_dpp(float& v, int& i) {
    argmax_dpp_step<0xb1>(v, i);
    argmax_dpp_step<0x4e>(v, i);
    argmax_dpp_step<0x141>(v, i);
    argmax_dpp_step<0x140>(v, i);
    argmax_dpp_step<0x142, 0xa>(v, i);
    argmax_dpp_step<0x143, 0xc>(v, i);
    v = lane63(v);
    i = __builtin_amdgcn_readlane(i, 63);
}

// Inclusive prefix sum of an int across the wave in lane order (all lanes
// active): sums of 4 within each row of 16 lanes, then of 8 and 16 under bank
// masks, then the two row broadcasts carry row totals forward.
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
    const int v0 = v;
    v += __builtin_amdgcn_update_dpp(0, v0, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v0, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v0, 0x113, 0xf, 0xf, false);   // row_shr:3
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xe, false);    // row_shr:4, lanes 4-15 of a row
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xc, false);    // row_shr:8, lanes 8-15 of a row
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);    // row_bcast:15 into rows 1 and 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);    // row_bcast:31 into rows 2 and 3
    return v;
}

// Inclusive prefix sum of a float across the wave in lane order (all lanes
// active), same pattern as wave_incl_scan_i32.
__device__ __forceinline__ float wave_incl_scan_f32(float v) {
    const float v0 = v;
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v0), 0x111, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v0), 0x112, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v0), 0x113, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xe, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xc, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));
    return v;
}

// Block-wide exclusive scan of one int per thread (DPP within each wave, wave
// totals through LDS); returns the block total too. Totals stay below 2^31.
// nw: wavefronts in the workgroup (0: from blockDim). A source built with
// -mno-amdgpu-ieee cannot inline the device-library function behind blockDim, and
// that call waits for every outstanding memory operation, so callers with loads
// in flight pass nw.
__device__ __forceinline__ int block_exclusive_scan_i32(int v, int* sh, int& total, int nw = 0) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (nw == 0) nw = blockDim.x >> 6;
    const int incl = wave_incl_scan_i32(v);
    if (lane == 63) sh[w] = incl;
    __syncthreads();
    int before = 0, tot = 0;
    for (int q = 0; q < nw; ++q) {
        const int t = sh[q];
        tot += t;
        if (q < w) before += t;
    }
    total = tot;
    __syncthreads();
    return before + incl - v;
}

// Inclusive prefix sum across the wave in lane order.
__device__ __forceinline__ float wave_inclusive_scan(float v, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        float t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    return v;
}

// Two-level inverse-CDF draw by one wavefront: the smallest index e with
// w_0 + ... + w_e > thr, where the weights come in chunks of `chunk_len`.
// chunk_mass(ch) must return the chunk's total weight and weight(e) one
// element's; the chunk totals select the chunk, an in-order scan of its
// elements selects the index. When rounding leaves no crossing, the last index
// with positive weight (in the last chunk with mass) is returned.
// With c0 > 0 the search covers chunks [c0, C) only, its running sum starting
// at carry0 (the mass before chunk c0; -inf: no crossing, the last positive
// weight of those chunks).
template <class ChunkMass, class Weight>
__device__ int inv_cdf_pick(int C, int V, int chunk_len, float thr, ChunkMass chunk_mass, Weight weight,
                            int lane, int c0 = 0, float carry0 = 0.f) {
    float carry = carry0, base = 0.f;
    int sel = -1, last_pos = -1;
    for (int ch0 = c0; ch0 < C && sel < 0; ch0 += kWave) {
        const int ch = ch0 + lane;
        const float mch = ch < C ? chunk_mass(ch) : 0.f;
        const float inc = wave_inclusive_scan(mch, lane) + carry;
        int cand = (ch < C && inc > thr) ? ch : 0x7fffffff;
        const int pos = (ch < C && mch > 0.f) ? ch : -1;
        cand = wave_min_int(cand);
        last_pos = max(last_pos, -wave_min_int(-pos));
        if (cand != 0x7fffffff) {
            sel = cand;
            base = __shfl(inc - mch, cand - ch0, kWave);
        }
        carry = __shfl(inc, kWave - 1, kWave);
    }
    if (sel < 0) {
        sel = last_pos < 0 ? 0 : last_pos;
        base = -INFINITY;                      // no crossing: fall back to the last positive weight
    }
    const int beg = sel * chunk_len, end = min(V, beg + chunk_len);
    float run = base;
    int found = 0x7fffffff, lastw = -1;
    for (int e0 = beg; e0 < end && found == 0x7fffffff; e0 += kWave * 8) {
        float w[8];
        float lsum = 0.f;
        const int my = e0 + lane * 8;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            w[q] = (my + q < end) ? weight(my + q) : 0.f;
            lsum += w[q];
            if (w[q] > 0.f) lastw = max(lastw, my + q);
        }
        const float incl = wave_inclusive_scan(lsum, lane);
        float cum = run + (incl - lsum);
        int hit = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            cum += w[q];
            if (hit == 0x7fffffff && my + q < end && cum > thr) hit = my + q;
        }
        found = wave_min_int(hit);
        run += __shfl(incl, kWave - 1, kWave);
    }
    lastw = -wave_min_int(-lastw);
    return found != 0x7fffffff ? found : (lastw >= 0 ? lastw : beg);
}

__device__ __forceinline__ void set_status(WsHeader* h, uint32_t bits) {
    atomicOr(&h->status, bits);
}

// Float classes from the bits, behind an empty asm statement so that the
// optimiser cannot turn them back into floating-point class tests: sources
// built with -fno-honor-nans may fold those to "no NaN".
__device__ __forceinline__ uint32_t opaque_bits(float x) {
    uint32_t b = __float_as_uint(x);
    asm volatile("" : "+v"(b));
    return b;
}
// finite (neither infinite nor NaN)
__device__ __forceinline__ bool finite_bits(float x) { return (opaque_bits(x) & 0x7f800000u) != 0x7f800000u; }
// NaN or +inf (-inf is a valid logit: a token that can never be drawn)
__device__ __forceinline__ bool nan_or_posinf_bits(float x) {
    const uint32_t b = opaque_bits(x);
    return b == 0x7f800000u || (b & 0x7fffffffu) > 0x7f800000u;
}

// ---- counter-based uniforms --------------------------------------------------
// Philox4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11). A round multiplies counter words 0 and
// 2 by two fixed 64-bit constants into 128-bit products; the new counter is
// (hi(w2 * M1) ^ w1 ^ k0, lo(w2 * M1), hi(w0 * M0) ^ w3 ^ k1, lo(w0 * M0)); the
// key is bumped by two Weyl constants before every round but the first. Only
// word 0 of the block is used.
//
// Every uniform of the step is addressed by what it decides:
//   U(seed, step, purpose, r, i) = (word 0 of the block at counter
//       (i + 1, r, purpose, 0) under key (seed, step)) >> 40, times 2^-24,
// a float multiple of 2^-24 in [0, 1), exact. Purposes below.
enum : uint32_t { kPurposeAccept = 0, kPurposeDraw = 1, kPurposeDraft = 2 };

// The block of counter (w0, w1, w2, w3) under key (k0, k1), in place.
__device__ __forceinline__ void philox4x64_10(uint64_t& w0, uint64_t& w1, uint64_t& w2, uint64_t& w3, uint64_t k0,
                                              uint64_t k1) {
    constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    constexpr uint64_t K0 = 0x9E3779B97F4A7C15ull, K1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int n = 0; n < 10; ++n) {
        if (n > 0) {
            k0 += K0;
            k1 += K1;
        }
        const uint64_t hi0 = __umul64hi(M0, w0), lo0 = M0 * w0;
        const uint64_t hi1 = __umul64hi(M1, w2), lo1 = M1 * w2;
        const uint64_t n0 = hi1 ^ w1 ^ k0, n2 = hi0 ^ w3 ^ k1;
        w0 = n0;
        w1 = lo1;
        w2 = n2;
        w3 = lo0;
    }
}

__device__ __forceinline__ float philox_uniform(uint64_t seed, uint64_t step, uint32_t purpose, uint32_t r,
                                                uint32_t i) {
    uint64_t w0 = uint64_t(i) + 1u, w1 = r, w2 = purpose, w3 = 0u;
    philox4x64_10(w0, w1, w2, w3, seed, step);
    return float(uint32_t(w0 >> 40)) * 0x1p-24f;
}

// The two uniforms of trial t of the residual draw at position i of request r:
// words 0 and 1 of the block at counter (i + 1, r, 1, t), each >> 40 and times
// 2^-24 (trial 0's first uniform is U(seed, step, 1, r, i)).
__device__ __forceinline__ void philox_trial(uint64_t seed, uint64_t step, uint32_t r, uint32_t i, uint32_t t,
                                             float& u1, float& u2) {
    uint64_t w0 = uint64_t(i) + 1u, w1 = r, w2 = kPurposeDraw, w3 = t;
    philox4x64_10(w0, w1, w2, w3, seed, step);
    u1 = float(uint32_t(w0 >> 40)) * 0x1p-24f;
    u2 = float(uint32_t(w1 >> 40)) * 0x1p-24f;
}

}  // namespace specv
