// markov_draft: the Markov head of the semi-autoregressive drafter.
//
// Pages: the drafter keeps a parallel backbone that proposes the whole block in
// one pass and adds a light sequential module that injects prefix information
// token by token; the default is a Markov head that looks only at the previous
// token ("刚融完500亿创始人亲自下场写代码…", section "1. 半自回归生成";
// "DSpark 的 661% 提速…", section 3.1). The head is read here as a low-rank
// additive correction: dl_i = backbone_i + E[x_{i-1}] . P^T.
//
// Per position i (sequential: x_i feeds position i+1):
//   markov_logits_mfma (bf16)  one workgroup per 64-entry vocabulary slice:
//       the slice of P (64 x d_m) is staged in LDS; four wavefronts sweep the
//       requests in blocks of 64, multiplying gathered embedding rows E[x_{i-1}]
//       by the slice with v_mfma_f32_16x16x32_bf16 (fp32 accumulation). The
//       epilogue adds the backbone logits, rounds to bf16 (nearest-even),
//       stores the draft logits and emits per-(request, slice) softmax or
//       argmax partials of the rounded values.
//   markov_logits_fma (fp32)   the same with one lane per output and plain FMA.
//   markov_pick                one wavefront per request: merges the partials;
//       greedy argmax, or the two-level inverse-CDF draw over softmax(dl / tau).
//
// rnn_draft: the RNN head, the pages' other sequential module, which carries
// the whole prefix of the block in a recurrent state (same sections). Read as
// h_i = round(tanh(E[x_{i-1}] + A h_{i-1})), h_{-1} = 0, dl_i = bk_i + h_i . P^T:
//   rnn_state                  one workgroup per request: h_i from h_{i-1} and
//       the embedding row, float32 accumulation, tanh, rounded to the storage
//       type (the operand of the projection);
//   then the same logits and pick kernels, with the state rows in place of the
//       gathered embedding rows.
#include <climits>

#include "common.h"
#include "host.h"

namespace specv {

constexpr int kSlice = 64;          // vocabulary entries per workgroup / partial

struct MarkovArgs {
    int R, k, V, d_m, S;            // S = slices per row
    int pos;                        // current position i
    int mode;
    float c;                        // log2(e) / tau
    const void* bk;                 // [R,k,V]
    const void* emb;                // [V,d_m]
    const void* proj;               // [V,d_m]
    const int32_t* prev;            // [R]
    const void* rec;                // RNN head: [d_m,d_m] recurrence A (NULL: Markov head)
    void* state;                    // RNN head: [R,k,d_m] states, storage type
    const float* uniforms;          // [R,k]
    int32_t* tokens;                // [R,k]
    void* dl;                       // [R,k,V]
    float2* part;                   // [R * S]
    WsHeader* hdr;
};

__device__ __forceinline__ int prev_token(const MarkovArgs& a, int m) {
    int p = a.pos == 0 ? a.prev[m] : a.tokens[long(m) * a.k + a.pos - 1];
    return p;
}

// round-to-nearest-even float -> bf16 bits (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Partial of one (request, slice): argmax (greedy) or base-2 online softmax.
struct Part {
    float a;
    float b;   // greedy: index bits; sampling: sum
};

__device__ __forceinline__ void part_add(int mode, Part& p, float x, int idx, float c) {
    if (mode == SPECV_GREEDY) {
        if (__float_as_int(p.b) == INT_MAX || x > p.a || (x == p.a && idx < __float_as_int(p.b))) {
            p.a = x;
            p.b = __int_as_float(idx);
        }
    } else {
        const float am = x * c;
        if (am > p.a) { p.b *= __builtin_amdgcn_exp2f(p.a - am); p.a = am; }
        p.b += __builtin_amdgcn_exp2f(fmaf(x, c, -p.a));
    }
}

__device__ __forceinline__ void part_merge(int mode, Part& p, Part q) {
    if (mode == SPECV_GREEDY) {
        int i1 = __float_as_int(p.b), i2 = __float_as_int(q.b);
        if (q.a > p.a || (q.a == p.a && i2 < i1) || i1 == INT_MAX) {
            if (i2 != INT_MAX) { p.a = q.a; p.b = q.b; }
        }
    } else {
        lse_merge(p.a, p.b, q.a, q.b);
    }
}

__device__ __forceinline__ Part part_empty(int mode) {
    Part p;
    if (mode == SPECV_GREEDY) { p.a = -INFINITY; p.b = __int_as_float(INT_MAX); }
    else { p.a = -INFINITY; p.b = 0.f; }
    return p;
}

// Partial of the 16 rounded logits one lane holds for one request (vocabulary
// n_x + e for x, e in 0..3; entries at or past V excluded): the maximum first,
// then one exp2 per value (sampling), or the first argmax (greedy).
__device__ __forceinline__ Part lane_part(int mode, const float (&v)[4][4], const int (&n)[4], int V, float c) {
    Part p = part_empty(mode);
    if (mode == SPECV_GREEDY) {
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n[x] + e < V && (v[x][e] > p.a || __float_as_int(p.b) == INT_MAX)) {
                    p.a = v[x][e];
                    p.b = __int_as_float(n[x] + e);
                }
        return p;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n[x] + e < V) mx = fmaxf(mx, v[x][e]);
    if (mx == -INFINITY) return p;
    const float m = mx * c;
    float sum = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n[x] + e < V) sum += __builtin_amdgcn_exp2f(fmaf(v[x][e], c, -m));
    p.a = m;
    p.b = sum;
    return p;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// bf16: MFMA projection
// ---------------------------------------------------------------------------

template <bool VEC4>
__global__ __launch_bounds__(256) void markov_logits_mfma(MarkovArgs a) {
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * kSlice;
    const int dm = a.d_m;
    if (a.pos == 0 && blockIdx.x == 0 && tid == 0) a.hdr->status = 0u;   // this kernel sets no bits
    const int row_bytes = dm * 2 + 16;              // padded LDS row (bank spread)
    const uint16_t* P = static_cast<const uint16_t*>(a.proj);
    const uint16_t* E = static_cast<const uint16_t*>(a.emb);

    // stage P[n0 .. n0+63, :] in LDS (zeros past V)
    const int vec_per_row = dm / 8;
    for (int q = tid; q < kSlice * vec_per_row; q += blockDim.x) {
        const int rr = q / vec_per_row, cc = q % vec_per_row;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n0 + rr < a.V) v = reinterpret_cast<const uint4*>(P + long(n0 + rr) * dm)[cc];
        *reinterpret_cast<uint4*>(lds_raw + rr * row_bytes + cc * 16) = v;
    }
    __syncthreads();

    const uint16_t* bk = static_cast<const uint16_t*>(a.bk);
    uint16_t* dl = static_cast<uint16_t*>(a.dl);
    const int g = lane >> 4, l16 = lane & 15;

    for (int mb = wave * 64; mb < a.R; mb += 4 * 64) {
        f32x4 acc[4][4];
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
        // gathered operand rows (embedding of the previous token, or the RNN state)
        // of this lane's four request columns
        const uint16_t* erow[4];
        bool mok[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int m = mb + 16 * b + l16;
            mok[b] = m < a.R;
            int p = mok[b] ? prev_token(a, m) : 0;
            if (p < 0 || p >= a.V) p = 0;             // reported by markov_pick
            erow[b] = a.state ? static_cast<const uint16_t*>(a.state) + (long(mok[b] ? m : 0) * a.k + a.pos) * dm
                              : E + long(p) * dm;
        }
        // the epilogue's backbone values, loaded now so that they arrive during the
        // products: lane holds vocab n0 + 16x + 4g + {0..3} of request mb + 16b + l16
        uint2 bkw[4][4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int m = mb + 16 * b + l16;
            const long rowoff = (long(mok[b] ? m : 0) * a.k + a.pos) * long(a.V);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int n = n0 + 16 * x + 4 * g;
                bkw[b][x] = make_uint2(0u, 0u);
                if (VEC4 && mok[b] && n + 3 < a.V) bkw[b][x] = *reinterpret_cast<const uint2*>(bk + rowoff + n);
            }
        }
        // products, with the next k-step's operand rows in flight during this one
        auto load_b = [&](bf16x8 (&f)[4], int k0) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint4 v = mok[b] ? *reinterpret_cast<const uint4*>(erow[b] + k0 + 8 * g) : make_uint4(0, 0, 0, 0);
                f[b] = __builtin_bit_cast(bf16x8, v);
            }
        };
        bf16x8 bfr[4], bnx[4];
        load_b(bfr, 0);
        for (int k0 = 0; k0 < dm; k0 += 32) {
            if (k0 + 32 < dm) load_b(bnx, k0 + 32);
            bf16x8 afr[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                uint4 v = *reinterpret_cast<const uint4*>(lds_raw + (16 * x + l16) * row_bytes + (k0 + 8 * g) * 2);
                afr[x] = __builtin_bit_cast(bf16x8, v);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[x][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[x], bfr[b], acc[x][b], 0, 0, 0);
#pragma unroll
            for (int b = 0; b < 4; ++b) bfr[b] = bnx[b];
        }
        // epilogue
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int m = mb + 16 * b + l16;
            Part pp = part_empty(a.mode);
            if (m < a.R) {
                const long rowoff = (long(m) * a.k + a.pos) * long(a.V);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int n = n0 + 16 * x + 4 * g;
                    float bkv[4];
                    if (VEC4 && n + 3 < a.V) {
                        bkv[0] = bf16_lo(bkw[b][x].x); bkv[1] = bf16_hi(bkw[b][x].x);
                        bkv[2] = bf16_lo(bkw[b][x].y); bkv[3] = bf16_hi(bkw[b][x].y);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            bkv[e] = n + e < a.V ? __uint_as_float(uint32_t(bk[rowoff + n + e]) << 16) : 0.f;
                    }
                    uint32_t hb[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        hb[e] = f32_to_bf16_rne(acc[x][b][e] + bkv[e]);
                        if (n + e < a.V) part_add(a.mode, pp, __uint_as_float(hb[e] << 16), n + e, a.c);
                    }
                    if (VEC4 && n + 3 < a.V) {
                        *reinterpret_cast<uint2*>(dl + rowoff + n) =
                            make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < a.V) dl[rowoff + n + e] = uint16_t(hb[e]);
                    }
                }
            }
            // merge the four lanes that share this request (lane ^ 16, lane ^ 32)
#pragma unroll
            for (int o = 16; o <= 32; o <<= 1) {
                Part q;
                q.a = __shfl_xor(pp.a, o, 64);
                q.b = __shfl_xor(pp.b, o, 64);
                part_merge(a.mode, pp, q);
            }
            if (g == 0 && m < a.R) a.part[long(m) * a.S + blockIdx.x] = make_float2(pp.a, pp.b);
        }
    }
}

// bf16, d_m <= 256: one 512-thread workgroup per 256-entry vocabulary tile. The
// tile's 256 rows of P sit in LDS (135 KB at d_m = 256); each wavefront keeps
// its 64 requests' operand rows in registers (d_m / 2 VGPRs) and sweeps the
// tile's four 64-entry sub-slices, so the gathered rows are read once per 256
// vocabulary entries instead of once per 64, and a workgroup's logits are 512
// contiguous bytes per row. Partials stay per 64-entry sub-slice.
constexpr int kTileN = 256;
constexpr int kTileThreads = 512;

template <bool VEC4, int KS>
__global__ __launch_bounds__(kTileThreads) void markov_logits_tile(MarkovArgs a) {
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * kTileN;
    constexpr int dm = KS * 32;
    if (a.pos == 0 && blockIdx.x == 0 && tid == 0) a.hdr->status = 0u;   // this kernel sets no bits
    constexpr int row_bytes = dm * 2 + 16;
    const uint16_t* P = static_cast<const uint16_t*>(a.proj);
    const uint16_t* E = static_cast<const uint16_t*>(a.emb);
    constexpr int vec_per_row = dm / 8;
    for (int q = tid; q < kTileN * vec_per_row; q += kTileThreads) {
        const int rr = q / vec_per_row, cc = q % vec_per_row;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (t0 + rr < a.V) v = reinterpret_cast<const uint4*>(P + long(t0 + rr) * dm)[cc];
        *reinterpret_cast<uint4*>(lds_raw + rr * row_bytes + cc * 16) = v;
    }
    __syncthreads();

    const uint16_t* bk = static_cast<const uint16_t*>(a.bk);
    uint16_t* dl = static_cast<uint16_t*>(a.dl);
    const int g = lane >> 4, l16 = lane & 15;
    constexpr int KB = 2;                        // 16-request blocks per wavefront
    for (int mb = wave * 16 * KB; mb < a.R; mb += (kTileThreads / 64) * 16 * KB) {
        bool mok[KB];
        bf16x8 bfr[KS][KB];                      // this lane's operand rows, all of d_m
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            const int m = mb + 16 * b + l16;
            mok[b] = m < a.R;
            int p = mok[b] ? prev_token(a, m) : 0;
            if (p < 0 || p >= a.V) p = 0;             // reported by markov_pick
            const uint16_t* erow = a.state
                ? static_cast<const uint16_t*>(a.state) + (long(mok[b] ? m : 0) * a.k + a.pos) * dm
                : E + long(p) * dm;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint4 v = mok[b] ? *reinterpret_cast<const uint4*>(erow + 32 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
                bfr[ks][b] = __builtin_bit_cast(bf16x8, v);
            }
        }
        // backbone values of a sub-slice (VEC4 path), one sub-slice ahead of its epilogue
        auto load_bk = [&](uint2 (&w)[KB][4], int n0) {
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                const int m = mb + 16 * b + l16;
                const long rowoff = (long(mok[b] ? m : 0) * a.k + a.pos) * long(a.V);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int n = n0 + 16 * x + 4 * g;
                    w[b][x] = make_uint2(0u, 0u);
                    if (VEC4 && mok[b] && n + 3 < a.V) w[b][x] = *reinterpret_cast<const uint2*>(bk + rowoff + n);
                }
            }
        };
        uint2 bkc[KB][4], bkn[KB][4];
        load_bk(bkc, t0);
        for (int sub = 0; sub < kTileN / kSlice; ++sub) {
            const int n0 = t0 + sub * kSlice;
            if (n0 >= a.V) break;
            if (sub + 1 < kTileN / kSlice) load_bk(bkn, n0 + kSlice);
            f32x4 acc[4][KB];
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y < KB; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 afr[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const uint4 v = *reinterpret_cast<const uint4*>(
                        lds_raw + (sub * kSlice + 16 * x + l16) * row_bytes + (32 * ks + 8 * g) * 2);
                    afr[x] = __builtin_bit_cast(bf16x8, v);
                }
#pragma unroll
                for (int x = 0; x < 4; ++x)
#pragma unroll
                    for (int b = 0; b < KB; ++b)
                        acc[x][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[x], bfr[ks][b], acc[x][b], 0, 0, 0);
            }
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                const int m = mb + 16 * b + l16;
                Part pp = part_empty(a.mode);
                if (m < a.R) {
                    const long rowoff = (long(m) * a.k + a.pos) * long(a.V);
                    float vals[4][4];
                    int ns[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const int n = n0 + 16 * x + 4 * g;
                        ns[x] = n;
                        float bkv[4];
                        if (VEC4 && n + 3 < a.V) {
                            const uint2 w = bkc[b][x];
                            bkv[0] = bf16_lo(w.x); bkv[1] = bf16_hi(w.x);
                            bkv[2] = bf16_lo(w.y); bkv[3] = bf16_hi(w.y);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                bkv[e] = n + e < a.V ? __uint_as_float(uint32_t(bk[rowoff + n + e]) << 16) : 0.f;
                        }
                        uint32_t hb[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            hb[e] = f32_to_bf16_rne(acc[x][b][e] + bkv[e]);
                            vals[x][e] = __uint_as_float(hb[e] << 16);
                        }
                        if (VEC4 && n + 3 < a.V) {
                            *reinterpret_cast<uint2*>(dl + rowoff + n) =
                                make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (n + e < a.V) dl[rowoff + n + e] = uint16_t(hb[e]);
                        }
                    }
                    pp = lane_part(a.mode, vals, ns, a.V, a.c);
                }
#pragma unroll
                for (int o = 16; o <= 32; o <<= 1) {
                    Part q;
                    q.a = __shfl_xor(pp.a, o, 64);
                    q.b = __shfl_xor(pp.b, o, 64);
                    part_merge(a.mode, pp, q);
                }
                if (g == 0 && m < a.R) a.part[long(m) * a.S + n0 / kSlice] = make_float2(pp.a, pp.b);
            }
#pragma unroll
            for (int b = 0; b < KB; ++b)
#pragma unroll
                for (int x = 0; x < 4; ++x) bkc[b][x] = bkn[b][x];
        }
    }
}

// ---------------------------------------------------------------------------
// fp32: plain FMA projection, one wavefront per (request, slice)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void markov_logits_fma(MarkovArgs a) {
    const int lane = threadIdx.x & 63;
    const long item = long(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (item >= long(a.R) * a.S) return;
    const int m = int(item / a.S), sl = int(item % a.S);
    const int n = sl * kSlice + lane;
    const float* E = static_cast<const float*>(a.emb);
    const float* P = static_cast<const float*>(a.proj);
    const float* bk = static_cast<const float*>(a.bk);
    float* dl = static_cast<float*>(a.dl);
    if (a.pos == 0 && item == 0 && lane == 0) a.hdr->status = 0u;   // this kernel sets no bits
    int p = prev_token(a, m);
    if (p < 0 || p >= a.V) p = 0;                 // reported by markov_pick
    const float* erow = a.state ? static_cast<const float*>(a.state) + (long(m) * a.k + a.pos) * a.d_m
                                : E + long(p) * a.d_m;
    Part pp = part_empty(a.mode);
    if (n < a.V) {
        float acc = 0.f;
        for (int d = 0; d < a.d_m; ++d) acc = fmaf(erow[d], P[long(n) * a.d_m + d], acc);
        const long off = (long(m) * a.k + a.pos) * long(a.V) + n;
        const float v = acc + bk[off];
        dl[off] = v;
        part_add(a.mode, pp, v, n, a.c);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        Part q;
        q.a = __shfl_xor(pp.a, o, 64);
        q.b = __shfl_xor(pp.b, o, 64);
        part_merge(a.mode, pp, q);
    }
    if (lane == 0) a.part[long(m) * a.S + sl] = make_float2(pp.a, pp.b);
}

// ---------------------------------------------------------------------------
// RNN head: h_i = round(tanh(E[x_{i-1}] + A h_{i-1})), one workgroup per request
// ---------------------------------------------------------------------------

template <int DT>
__global__ __launch_bounds__(256) void rnn_state(MarkovArgs a) {
    using LT = Logit<DT>;
    using T = typename LT::T;
    __shared__ float h[512];
    const int m = blockIdx.x, dm = a.d_m;
    const T* A = static_cast<const T*>(a.rec);
    const T* E = static_cast<const T*>(a.emb);
    T* st = static_cast<T*>(a.state);
    for (int q = threadIdx.x; q < dm; q += blockDim.x)
        h[q] = a.pos == 0 ? 0.f : LT::load1(st + (long(m) * a.k + a.pos - 1) * dm + q);
    int p = prev_token(a, m);
    if (p < 0 || p >= a.V) p = 0;                 // reported by markov_pick
    __syncthreads();
    for (int j = threadIdx.x; j < dm; j += blockDim.x) {
        float s = LT::load1(E + long(p) * dm + j);
        const T* row = A + long(j) * dm;
        for (int q = 0; q < dm; ++q) s = fmaf(LT::load1(row + q), h[q], s);
        const float t = tanhf(s);
        if constexpr (DT == SPECV_BF16)
            st[(long(m) * a.k + a.pos) * dm + j] = uint16_t(f32_to_bf16_rne(t));
        else
            st[(long(m) * a.k + a.pos) * dm + j] = t;
    }
}

// ---------------------------------------------------------------------------
// next token per request
// ---------------------------------------------------------------------------

template <int DT>
__global__ __launch_bounds__(256) void markov_pick(MarkovArgs a) {
    using LT = Logit<DT>;
    using T = typename LT::T;
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= a.R) return;
    if (a.pos == 0 && lane == 0 && (a.prev[m] < 0 || a.prev[m] >= a.V)) set_status(a.hdr, SPECV_STATUS_BAD_TOKEN);
    const float2* pr = a.part + long(m) * a.S;
    Part tot = part_empty(a.mode);
    for (int s = lane; s < a.S; s += 64) {
        Part q;
        q.a = pr[s].x;
        q.b = pr[s].y;
        part_merge(a.mode, tot, q);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        Part q;
        q.a = __shfl_xor(tot.a, o, 64);
        q.b = __shfl_xor(tot.b, o, 64);
        part_merge(a.mode, tot, q);
    }
    int y;
    if (a.mode == SPECV_GREEDY) {
        y = __float_as_int(tot.b);
    } else {
        const float M = tot.a;
        const float thr = a.uniforms[long(m) * a.k + a.pos] * tot.b;
        const T* row = static_cast<const T*>(a.dl) + (long(m) * a.k + a.pos) * long(a.V);
        const float c = a.c;
        y = inv_cdf_pick(
            a.S, a.V, kSlice, thr,
            [&](int s) { float2 q = pr[s]; return q.x == -INFINITY ? 0.f : q.y * exp2f(q.x - M); },
            [&](int e) { return exp2f(fmaf(LT::load1(row + e), c, -M)); }, lane);
    }
    if (lane == 0) a.tokens[long(m) * a.k + a.pos] = y;
}

}  // namespace specv

namespace specv {
namespace {

size_t head_workspace_bytes(int R, int k, int V, int d_m, bool state) {
    if (R < 1 || k < 1 || k > SPECV_MAX_K || V < 1 || d_m < 1) return 0;
    const size_t S = (size_t(V) + kSlice - 1) / kSlice;
    size_t n = 256 + ((size_t(R) * S * sizeof(float2) + 255) & ~size_t(255));
    if (state) n += (size_t(R) * k * d_m * sizeof(float) + 255) & ~size_t(255);
    return n;
}

// Markov head (rec == NULL) or RNN head: validation and the per-position launches.
int head_draft(const char* fn, int mode, int dtype, int R, int k, int V, int d_m, const void* backbone_logits,
               const void* emb, const void* rec, const void* proj, const int32_t* prev_token, float temperature,
               const float* uniforms, int32_t* draft_tokens_out, void* draft_logits_out, void* state_out, void* ws,
               size_t ws_bytes, hipStream_t s) {
    clear_error();
    const bool rnn = rec != nullptr;
    if (mode != SPECV_GREEDY && mode != SPECV_SAMPLE)
        return fail(SPECV_EINVAL, "%s: mode %d is neither greedy (0) nor sample (1)", fn, mode);
    if (dtype != SPECV_BF16 && dtype != SPECV_F32) return fail(SPECV_EUNSUPPORTED, "%s: dtype %d unsupported", fn, dtype);
    if (R < 1 || k < 1 || k > SPECV_MAX_K || V < 1 || d_m < 1)
        return fail(SPECV_EINVAL, "%s: need R >= 1, 1 <= k <= %d, V >= 1, d_m >= 1", fn, SPECV_MAX_K);
    if (dtype == SPECV_BF16 && (d_m % 32 != 0 || d_m > 480))
        return fail(SPECV_EUNSUPPORTED, "%s: bf16 needs d_m %% 32 == 0 and d_m <= 480 (got %d)", fn, d_m);
    if (rnn && d_m > 512) return fail(SPECV_EUNSUPPORTED, "%s: d_m %d above 512", fn, d_m);
    if (!backbone_logits || !emb || !proj || !prev_token || !draft_tokens_out || !draft_logits_out || !ws)
        return fail(SPECV_EINVAL, "%s: NULL required pointer", fn);
    if (mode == SPECV_SAMPLE) {
        if (!uniforms) return fail(SPECV_EINVAL, "%s: sampling needs uniforms", fn);
        if (!(temperature > 0.f) || !(temperature < INFINITY))
            return fail(SPECV_EINVAL, "%s: temperature must be finite and > 0", fn);
    }
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(SPECV_EINVAL, "%s: workspace must be 256-byte aligned", fn);
    const size_t need = head_workspace_bytes(R, k, V, d_m, rnn && !state_out);
    if (ws_bytes < need) return fail(SPECV_EINVAL, "%s: workspace of %zu bytes, need %zu", fn, ws_bytes, need);
    if (dtype == SPECV_BF16 && (!aligned16(emb) || !aligned16(proj) || (state_out && !aligned16(state_out))))
        return fail(SPECV_EINVAL, "%s: emb, proj and state_out must be 16-byte aligned", fn);

    MarkovArgs a;
    a.R = R; a.k = k; a.V = V; a.d_m = d_m;
    a.S = (V + kSlice - 1) / kSlice;
    a.mode = mode;
    a.c = mode == SPECV_SAMPLE ? float(1.4426950408889634 / double(temperature)) : 1.f;
    a.bk = backbone_logits; a.emb = emb; a.proj = proj; a.prev = prev_token;
    a.uniforms = uniforms; a.tokens = draft_tokens_out; a.dl = draft_logits_out;
    a.hdr = static_cast<WsHeader*>(ws);
    a.part = reinterpret_cast<float2*>(static_cast<char*>(ws) + 256);
    a.rec = rec;
    a.state = nullptr;
    if (rnn)
        a.state = state_out ? state_out : static_cast<char*>(ws) + head_workspace_bytes(R, k, V, d_m, false);
    const bool vec4 = (V % 4) == 0 && (reinterpret_cast<uintptr_t>(backbone_logits) & 7u) == 0 &&
                      (reinterpret_cast<uintptr_t>(draft_logits_out) & 7u) == 0;
    const size_t lds = size_t(kSlice) * size_t(d_m * 2 + 16);
    if (dtype == SPECV_BF16 && d_m == 256) {
        const int tlds = int(size_t(kTileN) * size_t(d_m * 2 + 16));
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(markov_logits_tile<true, 8>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, tlds) != hipSuccess ||
            hipFuncSetAttribute(reinterpret_cast<const void*>(markov_logits_tile<false, 8>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, tlds) != hipSuccess)
            return fail(SPECV_EDEVICE, "%s: cannot raise the LDS limit of the projection kernel", fn);
    }
    // The status word is cleared by position 0's logits kernel (which sets no
    // bits) and set by position 0's pick kernel, which checks prev_token.
    for (int i = 0; i < k; ++i) {
        a.pos = i;
        if (dtype == SPECV_BF16) {
            if (rnn) SPECV_LAUNCH("rnn_state", rnn_state<SPECV_BF16>, R, 256, 0, s, a);
            if (d_m == 256) {
                const int tiles = (V + kTileN - 1) / kTileN;
                const size_t tlds = size_t(kTileN) * size_t(d_m * 2 + 16);
                if (vec4)
                    SPECV_LAUNCH("markov_logits", (markov_logits_tile<true, 8>), tiles, kTileThreads, tlds, s, a);
                else
                    SPECV_LAUNCH("markov_logits", (markov_logits_tile<false, 8>), tiles, kTileThreads, tlds, s, a);
            } else if (vec4)
                SPECV_LAUNCH("markov_logits", markov_logits_mfma<true>, a.S, 256, lds, s, a);
            else
                SPECV_LAUNCH("markov_logits", markov_logits_mfma<false>, a.S, 256, lds, s, a);
            SPECV_LAUNCH("markov_pick", markov_pick<SPECV_BF16>, (R + 3) / 4, 256, 0, s, a);
        } else {
            if (rnn) SPECV_LAUNCH("rnn_state", rnn_state<SPECV_F32>, R, 256, 0, s, a);
            const long items = long(R) * a.S;
            SPECV_LAUNCH("markov_logits", markov_logits_fma, (items + 3) / 4, 256, 0, s, a);
            SPECV_LAUNCH("markov_pick", markov_pick<SPECV_F32>, (R + 3) / 4, 256, 0, s, a);
        }
    }
    return SPECV_OK;
}

}  // namespace
}  // namespace specv

extern "C" size_t markov_draft_workspace_bytes(int R, int k, int V, int d_m) {
    return specv::head_workspace_bytes(R, k, V, d_m, false);
}

extern "C" int markov_draft(int mode, int dtype, int R, int k, int V, int d_m, const void* backbone_logits,
                            const void* emb, const void* proj, const int32_t* prev_token,
                            float temperature, const float* uniforms, int32_t* draft_tokens_out,
                            void* draft_logits_out, void* ws, size_t ws_bytes, specv_stream stream) {
    return specv::head_draft("markov_draft", mode, dtype, R, k, V, d_m, backbone_logits, emb, nullptr, proj,
                             prev_token, temperature, uniforms, draft_tokens_out, draft_logits_out, nullptr, ws,
                             ws_bytes, static_cast<hipStream_t>(stream));
}

extern "C" size_t rnn_draft_workspace_bytes(int R, int k, int V, int d_m) {
    return specv::head_workspace_bytes(R, k, V, d_m, true);
}

extern "C" int rnn_draft(int mode, int dtype, int R, int k, int V, int d_m, const void* backbone_logits,
                         const void* emb, const void* rec, const void* proj, const int32_t* prev_token,
                         float temperature, const float* uniforms, int32_t* draft_tokens_out, void* draft_logits_out,
                         void* state_out, void* ws, size_t ws_bytes, specv_stream stream) {
    if (!rec) {
        specv::clear_error();
        return specv::fail(SPECV_EINVAL, "rnn_draft: NULL required pointer (rec)");
    }
    return specv::head_draft("rnn_draft", mode, dtype, R, k, V, d_m, backbone_logits, emb, rec, proj, prev_token,
                             temperature, uniforms, draft_tokens_out, draft_logits_out, state_out, ws, ws_bytes,
                             static_cast<hipStream_t>(stream));
}
