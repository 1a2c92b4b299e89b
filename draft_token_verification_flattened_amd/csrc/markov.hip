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
//   markov_logits_run (bf16, d_m = 256)  the persistent projection (below); it
//       also leaves each request's partial merged over each contiguous range of
//       slices.
//   markov_logits_fma (fp32)   the same with one lane per output and plain FMA.
//   markov_pick_ranges         after markov_logits_run: one wavefront per
//       request, the draw in three levels (range, slice, entry).
//   markov_pick_wg             otherwise one workgroup per request: merges the
//       partials; greedy argmax, or the two-level inverse-CDF draw over
//       softmax(dl / tau) (markov_pick, one wavefront per request, for rows of
//       more than 4096 slices).
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
    const float* uniforms;          // [R,k], or NULL: counter-based uniforms (common.h)
    uint64_t seed, step;            // their key
    int32_t* tokens;                // [R,k]
    void* dl;                       // [R,k,V]
    specv_draft_stat* stats;        // [R,k] or NULL (sampling): the rows' softmax states for verification
    float2* part;                   // [R * S]
    float2* part_rng;               // [R * nr] the projection's merged partial per (request, slice range)
    int nr;                         // slice ranges (markov_logits_run's grid)
    WsHeader* hdr;
};

// The sampling uniform of request m at the current position.
__device__ __forceinline__ float draft_uniform(const MarkovArgs& a, int m) {
    return a.uniforms ? a.uniforms[long(m) * a.k + a.pos] : philox_uniform(a.seed, a.step, kPurposeDraft, m, a.pos);
}

// A merged (max, sum) state (sampling) or (max, index) (greedy) that is not
// finite: a NaN or +inf draft logit (sampling also: a row of -inf only).
__device__ __forceinline__ bool part_nonfinite(int mode, float a_, float b_) {
    if (mode == SPECV_GREEDY) return __float_as_uint(a_) == 0x7f800000u;
    return !(finite_bits(a_) && finite_bits(b_));
}

// The partial of (request m, slice s) sits at part[((m / 16) * S + s) * 16 + m % 16]:
// the 16 requests of one MFMA tile write one contiguous 128-byte record per
// slice (a request-major layout scatters 8-byte stores 19 KB apart, each
// costing the memory a whole sector), and request m's partials are 16 entries
// apart.
constexpr int kPartBlock = 16;
__host__ __device__ __forceinline__ long part_at(int m, int s, int S) {
    return (long(m / kPartBlock) * S + s) * kPartBlock + m % kPartBlock;
}

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

// lane_part for 16 values that all lie inside the row (no masks).
__device__ __forceinline__ Part lane_part_full(int mode, const float (&v)[4][4], const int (&n)[4], float c) {
    Part p;
    if (mode == SPECV_GREEDY) {
        p.a = v[0][0];
        p.b = __int_as_float(n[0]);
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (v[x][e] > p.a) {
                    p.a = v[x][e];
                    p.b = __int_as_float(n[x] + e);
                }
        return p;
    }
    float mx = fmaxf(v[0][0], v[0][1]);
#pragma unroll
    for (int q = 2; q < 16; q += 2) mx = fmaxf(mx, fmaxf(v[q / 4][q % 4], v[q / 4][q % 4 + 1]));
    const float m = mx * c;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int q = 0; q < 16; q += 2) {
        s0 += __builtin_amdgcn_exp2f(fmaf(v[q / 4][q % 4], c, -m));
        s1 += __builtin_amdgcn_exp2f(fmaf(v[q / 4][q % 4 + 1], c, -m));
    }
    p.a = m;
    p.b = s0 + s1;
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
            if (g == 0 && m < a.R) a.part[part_at(m, blockIdx.x, a.S)] = make_float2(pp.a, pp.b);
        }
    }
}

// bf16, d_m = 32 * KS (256 at KS = 8): a persistent grid of 1024-thread
// workgroups, one per compute unit. Workgroup (range, group) owns the 64-entry
// vocabulary slices [range S / nr, (range + 1) S / nr) and a group of 256
// requests (it also leaves each request's partial merged over its slices, in
// vocabulary order, for the pick's first level); the
// groups of one range are launched on the same XCD (blockIdx modulo 8), so the
// second group's reads of P find the first group's in that XCD's L2. Each
// wavefront keeps its 16 requests' operand rows in registers for the whole
// launch and sweeps the range slice by slice:
//   - P slices go through two LDS buffers: the next slice's rows are loaded
//     into registers during the current slice and written to the other buffer
//     after it, one barrier per slice. Rows are 512 bytes, unpadded; the
//     16-byte chunk c of LDS row L is stored at position c ^ (L % 16), so the
//     16 lanes that read one chunk of 16 consecutive rows hit 16 different
//     bank groups. A slice's rows are stored permuted so
//     that the MFMA output puts 16 consecutive vocabulary entries of one
//     request in one lane: vocabulary entry v = 16q + 4x + r of the slice is
//     row 4q + r of MFMA tile x, at LDS row 16x + 4q + r (conflict-free reads);
//   - backbone values come in 16-byte loads two slices ahead of their epilogue;
//   - the epilogue adds them, rounds to bf16 with the hardware conversion
//     (nearest-even), emits the per-(request, slice) partials and stores the
//     logits through a per-wavefront LDS tile, so that each store instruction
//     writes whole 128-byte lines (8 lanes per request row): non-temporal
//     stores that cover half of each line per instruction move 1.43 times the
//     bytes at half the rate.
constexpr int kTileRow = 144;                // LDS row of the store tile: 128 bytes + 16 of padding
constexpr int kTileBytes = 16 * kTileRow;    // one wavefront's 16 requests x 64 entries, bf16
constexpr int kRunKB = 1;                    // 16-request blocks per wavefront (2: 8 wavefronts of
                                             // 228 VGPRs, 5% slower than 16 of 120)
constexpr int kRunThreads = 1024 / kRunKB;   // 16 / kRunKB wavefronts
constexpr int kRunGroup = 256;               // requests per workgroup

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// grid of the persistent projection for R requests and S slices: nr ranges
// (a multiple of 8) times ng request groups
__host__ __device__ inline void run_grid(int R, int S, int& ng, int& nr) {
    ng = (R + kRunGroup - 1) / kRunGroup;
    nr = (256 / ng) / 8 * 8;
    if (nr < 8) nr = 8;
    (void)S;
}

template <bool VEC, int KS>
__global__ __launch_bounds__(kRunThreads) void markov_logits_run(MarkovArgs a, int ng, int nr) {
    extern __shared__ __align__(16) unsigned char lds_raw[];
    constexpr int dm = KS * 32;
    constexpr int row_bytes = dm * 2;                  // LDS row; 16-byte chunk c of row L sits at c ^ (L % 16)
    constexpr int buf_bytes = kSlice * row_bytes;
    constexpr int vpr = dm / 8;                        // 16-byte vectors per P row
    constexpr int PT = kSlice * vpr / kRunThreads;     // P vectors per thread per slice
    static_assert(PT * kRunThreads == kSlice * vpr, "P slice must split evenly over the threads");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (a.pos == 0 && blockIdx.x == 0 && tid == 0) a.hdr->status = 0u;   // this kernel sets no bits
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int range = (idx / ng) * 8 + xcd, grp = idx % ng;
    const int S = a.S, V = a.V;
    // a contiguous run of slices [s_first, s_last]
    const int s_first = int(long(range) * S / nr), s_last = int(long(range + 1) * S / nr) - 1;

    // Every load in the slice loop is issued on every path (addresses clamped
    // into the tensors), so the compiler's count of outstanding memory
    // operations stays exact and a wait for one slice's backbone values never
    // waits for the next slice's.
    const uint16_t* P = static_cast<const uint16_t*>(a.proj);
    const uint16_t* E = static_cast<const uint16_t*>(a.emb);
    const uint16_t* bk = static_cast<const uint16_t*>(a.bk);
    uint16_t* dl = static_cast<uint16_t*>(a.dl);
    const int g = lane >> 4, l16 = lane & 15;

    // P slice s: thread vectors q = tid + j * threads (row q / vpr, vector q % vpr);
    // rows past V repeat row V - 1 (their outputs are never stored)
    auto load_p = [&](u32x4 (&pr)[PT], int s) {
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            const int q = tid + j * kRunThreads, row = q / vpr, cc = q % vpr;
            const int v = min(s * kSlice + row, V - 1);
            pr[j] = *reinterpret_cast<const u32x4*>(P + long(v) * dm + cc * 8);
        }
    };
    auto store_p = [&](const u32x4 (&pr)[PT], int buf) {
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            const int q = tid + j * kRunThreads, row = q / vpr, cc = q % vpr;
            const int L = 16 * ((row >> 2) & 3) + 4 * (row >> 4) + (row & 3);
            *reinterpret_cast<u32x4*>(lds_raw + buf * buf_bytes + L * row_bytes + ((cc ^ (L & 15)) * 16)) = pr[j];
        }
    };

    // the store tile: lane (row, q) = (lane / 8 + 8 j, lane % 8) stores bytes 16 q .. 16 q + 15
    // of request row's 128-byte segment, for j = 0, 1
    unsigned char* tile = lds_raw + 2 * buf_bytes + wave * kTileBytes;
    // (row j = 1 is request m + 8, eight rows of k V further than row 0; it is
    // stored only when present, and then so is row 0)
    bool stok[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) stok[j] = grp * kRunGroup + wave * 16 + 8 * j + (lane >> 3) < a.R;
    const int m_st = grp * kRunGroup + wave * 16 + (lane >> 3);
    const long strow0 = (long(stok[0] ? m_st : 0) * a.k + a.pos) * long(V);
    const long strow_step = 8L * a.k * long(V);

    // this wavefront's first request, in a scalar register
    const int m_wave = __builtin_amdgcn_readfirstlane(grp * kRunGroup + wave * 16 * kRunKB);
    // this wavefront's requests (rows of absent requests read request 0's) and their operand rows
    int mreq[kRunKB];
    bool mok[kRunKB];
    long rowoff[kRunKB];
    bf16x8 bfr[KS][kRunKB];
#pragma unroll
    for (int b = 0; b < kRunKB; ++b) {
        const int m = grp * kRunGroup + wave * 16 * kRunKB + 16 * b + l16;
        mreq[b] = m;
        mok[b] = m < a.R;
        const int mc = mok[b] ? m : 0;
        rowoff[b] = (long(mc) * a.k + a.pos) * long(V);
        int p = prev_token(a, mc);
        if (p < 0 || p >= V) p = 0;                    // reported by markov_pick
        const uint16_t* erow = a.state ? static_cast<const uint16_t*>(a.state) + (long(mc) * a.k + a.pos) * dm
                                       : E + long(p) * dm;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            bfr[ks][b] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(erow + 32 * ks + 8 * g));
    }

    // backbone values of slice s for this lane: entries 16g .. 16g + 15 of its two
    // requests (clamped into the row; entries past V are never stored)
    auto load_bk = [&](u32x4 (&w)[kRunKB][2], int s) {
        if constexpr (VEC) {
#pragma unroll
            for (int b = 0; b < kRunKB; ++b)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int n = min(s * kSlice + 16 * g + 8 * h, V - 8);
                    w[b][h] = *reinterpret_cast<const u32x4*>(bk + rowoff[b] + n);
                }
        }
    };

    if (s_first > s_last) {
        // a range without slices (a row of fewer slices than ranges): empty partials, no loads
#pragma unroll
        for (int b = 0; b < kRunKB; ++b)
            if (g == 0 && mok[b]) {
                const Part e = part_empty(a.mode);
                a.part_rng[long(mreq[b]) * nr + range] = make_float2(e.a, e.b);
            }
        return;
    }
    // P slices ahead in registers: vector rows two (sets prA / prB hold slices
    // s + 1 and s + 2 while slice s is computed, roles alternating with the
    // slice), scalar rows one (prA only: their epilogue needs the registers)
    constexpr int kPAhead = VEC ? 2 : 1;
    u32x4 prA[PT], prB[PT];
    load_p(prA, s_first);
    store_p(prA, 0);
    load_p(prA, min(s_first + 1, s_last));
    if constexpr (VEC) load_p(prB, min(s_first + 2, s_last));
    // backbone values one slice ahead, in two buffers whose roles alternate
    // with the slice (as the two LDS buffers of P do); the loop below is
    // unrolled twice so that every role is fixed at compile time: a rotation
    // by register moves would make each slice wait for every load in flight,
    // the next P slice included
    u32x4 bkA[kRunKB][2], bkB[kRunKB][2];
    load_bk(bkA, s_first);
    Part run[kRunKB];
#pragma unroll
    for (int b = 0; b < kRunKB; ++b) run[b] = part_empty(a.mode);
    __syncthreads();

    // one slice: cur holds slice s's backbone values, ahead receives slice s + 1's
    auto slice = [&](int s, int lb, const u32x4 (&cur)[kRunKB][2], u32x4 (&ahead)[kRunKB][2], u32x4 (&pr)[PT]) {
        load_bk(ahead, min(s + 1, s_last));
        f32x4 acc[4][kRunKB];
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int b = 0; b < kRunKB; ++b) acc[x][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        const unsigned char* buf = lds_raw + lb * buf_bytes;
        // the MFMA phase issues ahead of other wavefronts' epilogues on the same SIMD
        // (raised wave priority; about 0.6% per launch at R = 512)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const bf16x8 afr = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const uint4*>(buf + (16 * x + l16) * row_bytes + (((4 * ks + g) ^ l16) * 16)));
#pragma unroll
                for (int b = 0; b < kRunKB; ++b)
                    acc[x][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[ks][b], acc[x][b], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // epilogue: lane holds entries n16 + 4x + e (x, e < 4) of request mreq[b]
        const int n16 = s * kSlice + 16 * g;
#pragma unroll
        for (int b = 0; b < kRunKB; ++b) {
            float bkv[16];
            if constexpr (VEC) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const u32x4 w = cur[b][h];
                    bkv[8 * h + 0] = bf16_lo(w.x); bkv[8 * h + 1] = bf16_hi(w.x);
                    bkv[8 * h + 2] = bf16_lo(w.y); bkv[8 * h + 3] = bf16_hi(w.y);
                    bkv[8 * h + 4] = bf16_lo(w.z); bkv[8 * h + 5] = bf16_hi(w.z);
                    bkv[8 * h + 6] = bf16_lo(w.w); bkv[8 * h + 7] = bf16_hi(w.w);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    bkv[j] = __uint_as_float(uint32_t(bk[rowoff[b] + min(n16 + j, V - 1)]) << 16);
            }
            uint32_t wd[8];
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int e = 0; e < 4; e += 2)
                    wd[2 * x + e / 2] = pack_bf16_rne(acc[x][b][e] + bkv[4 * x + e], acc[x][b][e + 1] + bkv[4 * x + e + 1]);
            float vals[4][4];
            int ns[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                ns[x] = n16 + 4 * x;
                vals[x][0] = bf16_lo(wd[2 * x]);     vals[x][1] = bf16_hi(wd[2 * x]);
                vals[x][2] = bf16_lo(wd[2 * x + 1]); vals[x][3] = bf16_hi(wd[2 * x + 1]);
            }
            if constexpr (VEC) {
                // through the tile: this lane's 32 bytes in, then 16 bytes of each of two rows out.
                // V % 8 == 0: each 8-entry piece is wholly inside the row or wholly past it.
                // Non-temporal stores: the logits go to HBM now, while this kernel leaves
                // bandwidth spare, instead of sitting dirty in the Infinity Cache until
                // the verify stream's reads evict them
                u32x4* tw = reinterpret_cast<u32x4*>(tile + l16 * kTileRow + 32 * g);
                tw[0] = u32x4{wd[0], wd[1], wd[2], wd[3]};
                tw[1] = u32x4{wd[4], wd[5], wd[6], wd[7]};
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                const int q = lane & 7, nq = s * kSlice + 8 * q;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(tile + (8 * j + (lane >> 3)) * kTileRow + 16 * q);
                    if (stok[j] && nq + 8 <= V)
                        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dl + strow0 + j * strow_step + nq));
                }
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (mok[b] && n16 + j < V) dl[rowoff[b] + n16 + j] = uint16_t(wd[j / 2] >> (16 * (j & 1)));
            }
            Part pp = (s + 1) * kSlice <= V ? lane_part_full(a.mode, vals, ns, a.c)
                                            : lane_part(a.mode, vals, ns, V, a.c);
#pragma unroll
            for (int o = 16; o <= 32; o <<= 1) {
                Part q;
                q.a = __shfl_xor(pp.a, o, 64);
                q.b = __shfl_xor(pp.b, o, 64);
                part_merge(a.mode, pp, q);
            }
            if (g == 0 && mok[b]) a.part[part_at(mreq[b], s, S)] = make_float2(pp.a, pp.b);
            part_merge(a.mode, run[b], pp);
        }
        // the next slice into the other buffer (last read before the previous
        // barrier); its registers then take slice s + 1 + kPAhead
        store_p(pr, lb ^ 1);
        load_p(pr, min(s + 1 + kPAhead, s_last));
        __syncthreads();
    };

    for (int s = s_first; s <= s_last;) {
        slice(s, 0, bkA, bkB, prA);
        s += 1;
        if (s > s_last) break;
        if constexpr (VEC) slice(s, 1, bkB, bkA, prB);
        else slice(s, 1, bkB, bkA, prA);
        s += 1;
    }
    // the requests' partials merged over this workgroup's slices
#pragma unroll
    for (int b = 0; b < kRunKB; ++b)
        if (g == 0 && mok[b]) {
            // the request recomputed here (the lane count in an asm statement, which
            // the compiler cannot merge with the earlier one), so that no vector
            // register has to hold it across the loop
            int l;
            asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
            const int m = m_wave + 16 * b + (l & 15);
            a.part_rng[long(m) * nr + range] = make_float2(run[b].a, run[b].b);
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
    if (lane == 0) a.part[part_at(m, sl, a.S)] = make_float2(pp.a, pp.b);
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
    const float2* pr = a.part + part_at(m, 0, a.S);      // slice s at pr[kPartBlock * s]
    Part tot = part_empty(a.mode);
    for (int s = lane; s < a.S; s += 64) {
        Part q;
        q.a = pr[kPartBlock * s].x;
        q.b = pr[kPartBlock * s].y;
        part_merge(a.mode, tot, q);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        Part q;
        q.a = __shfl_xor(tot.a, o, 64);
        q.b = __shfl_xor(tot.b, o, 64);
        part_merge(a.mode, tot, q);
    }
    if (lane == 0 && part_nonfinite(a.mode, tot.a, tot.b)) set_status(a.hdr, SPECV_STATUS_NONFINITE);
    int y;
    if (a.mode == SPECV_GREEDY) {
        y = __float_as_int(tot.b);
    } else {
        const float M = tot.a;
        const float thr = draft_uniform(a, m) * tot.b;
        const T* row = static_cast<const T*>(a.dl) + (long(m) * a.k + a.pos) * long(a.V);
        const float c = a.c;
        y = inv_cdf_pick(
            a.S, a.V, kSlice, thr,
            [&](int s) { float2 q = pr[kPartBlock * s]; return q.x == -INFINITY ? 0.f : q.y * exp2f(q.x - M); },
            [&](int e) { return exp2f(fmaf(LT::load1(row + e), c, -M)); }, lane);
        if (a.stats && lane == 0)
            a.stats[long(m) * a.k + a.pos] = specv_draft_stat{M, tot.b, LT::load1(row + y), c, y, {0, 0, 0}};
    }
    if (lane == 0) a.tokens[long(m) * a.k + a.pos] = y;
}

// The draw from markov_logits_run's range partials, one wavefront per request,
// in three levels, each in vocabulary order: the request's nr range partials
// (one contiguous record; range p covers slices [p S / nr, (p + 1) S / nr))
// give the row's state (M, Z) and the first range where the running mass
// exceeds u Z; that range's slice partials give the slice; the slice's 64
// logits give the token. When rounding leaves no crossing at a level, the
// last range, slice or entry with positive weight is taken. Greedy: the merged
// (max, first index) of the range partials is the token.
constexpr int kRangePer = 4;                 // range partials per lane: nr <= 256

// Levels 2 and 3 of markov_pick_ranges for a range of at most kPrefetchSlices
// slices of a bf16 row with V % 8 == 0, with every load in one round trip: the
// range's slice partials (one per lane) and all its logits (16-byte vectors,
// four per lane) are loaded together, the slice is chosen from the partials,
// and the chosen slice's eight vectors move by lane shuffles to lanes 0..7,
// where the entry is chosen. The arithmetic, its order and the no-crossing
// fallbacks are inv_cdf_pick's for chunks [s0, s1) from carry `base`; the
// drawn token's logit for the statistics comes from the same registers.
// Returns false, having stored nothing, when no slice of the range has mass
// (inv_cdf_pick then falls back to slice 0, outside the loaded range).
constexpr int kPrefetchSlices = 32;          // 32 x 8 vectors = 4 per lane
__device__ __forceinline__ bool pick_in_range(const MarkovArgs& a, int m, const uint16_t* row, const float2* ps,
                                              int s0, int s1, float thr, float M, float base, float Z) {
    const int lane = threadIdx.x & (kWave - 1);
    const int V = a.V, ns = s1 - s0, nvec = min(ns * (kSlice / 8), (V - s0 * kSlice) / 8);
    const float c = a.c;
    const float2 sp = lane < ns ? ps[kPartBlock * (s0 + lane)] : make_float2(-INFINITY, 0.f);
    uint4 vec[kPrefetchSlices * (kSlice / 8) / kWave];
#pragma unroll
    for (int i = 0; i < kPrefetchSlices * (kSlice / 8) / kWave; ++i) {
        const int j = lane + kWave * i;
        vec[i] = j < nvec ? *reinterpret_cast<const uint4*>(row + long(s0) * kSlice + 8 * j) : uint4{0, 0, 0, 0};
    }
    // level 2: the slice, from the partials (inv_cdf_pick's chunk level, one window)
    const float mch = lane < ns ? (sp.x == -INFINITY ? 0.f : sp.y * exp2f(sp.x - M)) : 0.f;
    const float inc = wave_inclusive_scan(mch, lane) + base;
    int cand = (lane < ns && inc > thr) ? s0 + lane : 0x7fffffff;
    const int pos = (lane < ns && mch > 0.f) ? s0 + lane : -1;
    cand = wave_min_int(cand);
    const int last_pos = max(-1, -wave_min_int(-pos));
    if (cand == 0x7fffffff && last_pos < 0) return false;
    int sel;
    float run;
    if (cand != 0x7fffffff) {
        sel = cand;
        run = __shfl(inc - mch, cand - s0, kWave);
    } else {
        sel = last_pos;
        run = -INFINITY;
    }
    // level 3: lane t < 8 takes entries beg + 8t .. beg + 8t + 7 of the slice
    const int beg = sel * kSlice, end = min(V, beg + kSlice);
    const int j0 = (sel - s0) * (kSlice / 8);                  // its first vector: slot j0 / 64, lanes j0 % 64 ..
    const int slot = j0 / kWave, src = (j0 % kWave) + (lane & 7);
    uint4 mine = vec[0];
#pragma unroll
    for (int i = 1; i < kPrefetchSlices * (kSlice / 8) / kWave; ++i)
        if (slot == i) mine = vec[i];
    uint4 v;
    v.x = __shfl(mine.x, src, kWave);
    v.y = __shfl(mine.y, src, kWave);
    v.z = __shfl(mine.z, src, kWave);
    v.w = __shfl(mine.w, src, kWave);
    float x[8];
    Logit<SPECV_BF16>::unpack(v, x);
    const int my = beg + lane * 8;
    float w[8], lsum = 0.f;
    int lastw = -1;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        w[q] = (lane < 8 && my + q < end) ? exp2f(fmaf(x[q], c, -M)) : 0.f;
        lsum += w[q];
        if (w[q] > 0.f) lastw = max(lastw, my + q);
    }
    const float incl = wave_inclusive_scan(lsum, lane);
    float cum = run + (incl - lsum);
    int hit = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        cum += w[q];
        if (hit == 0x7fffffff && lane < 8 && my + q < end && cum > thr) hit = my + q;
    }
    const int found = wave_min_int(hit);
    lastw = -wave_min_int(-lastw);
    const int y = found != 0x7fffffff ? found : (lastw >= 0 ? lastw : beg);
    // y's logit from the lane that holds it
    const int yl = (y - beg) >> 3, yq = (y - beg) & 7;
    float xy = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q)
        if (q == yq) xy = x[q];
    xy = __shfl(xy, yl, kWave);
    if (lane == 0) {
        a.tokens[long(m) * a.k + a.pos] = y;
        if (a.stats) a.stats[long(m) * a.k + a.pos] = specv_draft_stat{M, Z, xy, c, y, {0, 0, 0}};
    }
    return true;
}
static_assert(kRangePer * kWave >= 256, "run_grid makes at most 256 ranges");

template <int DT>
__global__ __launch_bounds__(256) void markov_pick_ranges(MarkovArgs a) {
    using LT = Logit<DT>;
    using T = typename LT::T;
    const int lane = threadIdx.x & (kWave - 1);
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= a.R) return;
    if (a.pos == 0 && lane == 0 && (a.prev[m] < 0 || a.prev[m] >= a.V)) set_status(a.hdr, SPECV_STATUS_BAD_TOKEN);
    const int nr = a.nr, S = a.S;
    const float2* pr = a.part_rng + long(m) * nr;
    // lane holds ranges [lane kRangePer, lane kRangePer + kRangePer)
    float2 q[kRangePer];
    Part tot = part_empty(a.mode);
#pragma unroll
    for (int i = 0; i < kRangePer; ++i) {
        const int rr = lane * kRangePer + i;
        q[i] = rr < nr ? pr[rr] : make_float2(-INFINITY, a.mode == SPECV_GREEDY ? __int_as_float(INT_MAX) : 0.f);
        Part p;
        p.a = q[i].x;
        p.b = q[i].y;
        if (rr < nr) part_merge(a.mode, tot, p);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        Part p;
        p.a = __shfl_xor(tot.a, o, 64);
        p.b = __shfl_xor(tot.b, o, 64);
        part_merge(a.mode, tot, p);
    }
    if (lane == 0 && part_nonfinite(a.mode, tot.a, tot.b)) set_status(a.hdr, SPECV_STATUS_NONFINITE);
    if (a.mode == SPECV_GREEDY) {
        if (lane == 0) a.tokens[long(m) * a.k + a.pos] = __float_as_int(tot.b);
        return;
    }
    const float M = tot.a;
    const float thr = draft_uniform(a, m) * tot.b;
    // level 1: the range
    float w[kRangePer], lsum = 0.f;
    int lastpos = -1;
#pragma unroll
    for (int i = 0; i < kRangePer; ++i) {
        const int rr = lane * kRangePer + i;
        w[i] = (rr < nr && q[i].x != -INFINITY) ? q[i].y * exp2f(q[i].x - M) : 0.f;
        lsum += w[i];
        if (w[i] > 0.f) lastpos = rr;
    }
    const float incl = wave_inclusive_scan(lsum, lane);
    float cum = incl - lsum, base = 0.f;
    int hit = INT_MAX;
#pragma unroll
    for (int i = 0; i < kRangePer; ++i) {
        const float prev = cum;
        cum += w[i];
        if (hit == INT_MAX && lane * kRangePer + i < nr && cum > thr) {
            hit = lane * kRangePer + i;
            base = prev;
        }
    }
    int rsel = wave_min_int(hit);
    if (rsel != INT_MAX) {
        base = __shfl(base, rsel / kRangePer, kWave);
    } else {                                  // no crossing: the last range with mass
        rsel = max(0, -wave_min_int(-lastpos));
        base = -INFINITY;
    }
    // levels 2 and 3: the slice inside the range, then the entry
    const int s0 = int(long(rsel) * S / nr), s1 = int(long(rsel + 1) * S / nr);
    const float2* ps = a.part + part_at(m, 0, S);        // slice s at ps[kPartBlock * s]
    const T* row = static_cast<const T*>(a.dl) + (long(m) * a.k + a.pos) * long(a.V);
    const float c = a.c;
    if constexpr (DT == SPECV_BF16) {
        if (s1 - s0 <= kPrefetchSlices && a.V % 8 == 0 && (reinterpret_cast<uintptr_t>(row) & 15u) == 0 &&
            pick_in_range(a, m, row, ps, s0, s1, thr, M, base, tot.b))
            return;
    }
    const int y = inv_cdf_pick(
        s1, a.V, kSlice, thr,
        [&](int s) { const float2 p = ps[kPartBlock * s]; return p.x == -INFINITY ? 0.f : p.y * exp2f(p.x - M); },
        [&](int e) { return exp2f(fmaf(LT::load1(row + e), c, -M)); }, lane, s0, base);
    if (lane == 0) {
        a.tokens[long(m) * a.k + a.pos] = y;
        if (a.stats) a.stats[long(m) * a.k + a.pos] = specv_draft_stat{M, tot.b, LT::load1(row + y), c, y, {0, 0, 0}};
    }
}

// The same draw by one 256-thread workgroup per request, for rows of at most
// kPickThreads * kPickPer slices. Thread t holds the contiguous slices
// [t J, t J + J), J = ceil(S / kPickThreads), in registers: one round trip for
// all of a row's partials, a workgroup merge, then (sampling) the slice masses
// exp2(M_s - M) S_s in slice order, a workgroup exclusive scan of the threads'
// sums, each thread's walk over its own slices for the first running sum above
// u Z, and one wavefront's scan of the chosen 64-entry slice.
constexpr int kPickThreads = 256;
constexpr int kPickPer = 16;
constexpr int kXcds = 8;                     // workgroups are dealt to the XCDs round-robin

// Workgroup b of the pick grid takes request pick_request(b): the 16 requests
// of one partial block (part_at) go to workgroups b, b + 8, ... of one XCD, so
// that XCD's L2 fetches each 128-byte record of the block once instead of up
// to eight L2s fetching it. The grid has pick_grid(R) workgroups; those past R
// return at once.
__host__ __device__ inline int pick_grid(int R) {
    return (R + kXcds * kPartBlock - 1) / (kXcds * kPartBlock) * (kXcds * kPartBlock);
}
__device__ __forceinline__ int pick_request(int b) {
    const int xcd = b % kXcds, i = b / kXcds;
    return (xcd + kXcds * (i / kPartBlock)) * kPartBlock + i % kPartBlock;
}

template <int DT>
__global__ __launch_bounds__(kPickThreads) void markov_pick_wg(MarkovArgs a) {
    using LT = Logit<DT>;
    using T = typename LT::T;
    constexpr int NW = kPickThreads / kWave;
    __shared__ float sh_a[NW], sh_b[NW];
    __shared__ int sh_i[NW];
    __shared__ float sh_base[NW];
    __shared__ int sh_last[NW];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int m = pick_request(int(blockIdx.x));
    if (m >= a.R) return;
    if (a.pos == 0 && tid == 0 && (a.prev[m] < 0 || a.prev[m] >= a.V)) set_status(a.hdr, SPECV_STATUS_BAD_TOKEN);
    const int S = a.S;
    const int J = (S + kPickThreads - 1) / kPickThreads;
    const int beg = tid * J, end = min(S, beg + J);
    const float2* pr = a.part + part_at(m, 0, S);         // slice s at pr[kPartBlock * s]
    float2 q[kPickPer];
#pragma unroll
    for (int j = 0; j < kPickPer; ++j)
        q[j] = (j < J && beg + j < end) ? pr[kPartBlock * (beg + j)] : make_float2(-INFINITY, __int_as_float(INT_MAX));
    Part tot = part_empty(a.mode);
#pragma unroll
    for (int j = 0; j < kPickPer; ++j) {
        if (!(j < J && beg + j < end)) continue;
        Part p;
        p.a = q[j].x;
        p.b = q[j].y;
        part_merge(a.mode, tot, p);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        Part p;
        p.a = __shfl_xor(tot.a, o, 64);
        p.b = __shfl_xor(tot.b, o, 64);
        part_merge(a.mode, tot, p);
    }
    if (lane == 0) { sh_a[w] = tot.a; sh_b[w] = tot.b; }
    __syncthreads();
    tot = part_empty(a.mode);
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        Part p;
        p.a = sh_a[v];
        p.b = sh_b[v];
        part_merge(a.mode, tot, p);
    }
    if (tid == 0 && part_nonfinite(a.mode, tot.a, tot.b)) set_status(a.hdr, SPECV_STATUS_NONFINITE);
    if (a.mode == SPECV_GREEDY) {
        if (tid == 0) a.tokens[long(m) * a.k + a.pos] = __float_as_int(tot.b);
        return;
    }
    const float M = tot.a;
    const float thr = draft_uniform(a, m) * tot.b;
    float wm[kPickPer];
    float lsum = 0.f;
    int lastpos = -1;
#pragma unroll
    for (int j = 0; j < kPickPer; ++j) {
        const bool in = j < J && beg + j < end;
        wm[j] = (in && q[j].x != -INFINITY) ? q[j].y * exp2f(q[j].x - M) : 0.f;
        lsum += wm[j];
        if (wm[j] > 0.f) lastpos = beg + j;
    }
    // workgroup exclusive scan of the threads' sums (slice order = thread order)
    const float incl = wave_incl_scan_f32(lsum);
    __syncthreads();                                  // sh_a / sh_b reads are done
    if (lane == 63) sh_a[w] = incl;
    __syncthreads();
    float before = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v)
        if (v < w) before += sh_a[v];
    float cum = before + (incl - lsum);
    int hit = INT_MAX;
    float base = 0.f;
#pragma unroll
    for (int j = 0; j < kPickPer; ++j) {
        const bool in = j < J && beg + j < end;
        const float prev_cum = cum;
        cum += wm[j];
        if (hit == INT_MAX && in && cum > thr) { hit = beg + j; base = prev_cum; }
    }
    // first crossing over the workgroup, with its running sum before the slice
    const int whit = wave_min_int(hit);
    const int wlast = -wave_min_int(-lastpos);
    if (hit == whit && whit != INT_MAX) { sh_i[w] = whit; sh_base[w] = base; }
    if (lane == 0 && whit == INT_MAX) sh_i[w] = INT_MAX;
    if (lane == 0) sh_last[w] = wlast;
    __syncthreads();
    if (w != 0) return;
    int sel = INT_MAX, lastall = -1;
    float sbase = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        if (sel == INT_MAX && sh_i[v] != INT_MAX) { sel = sh_i[v]; sbase = sh_base[v]; }
        lastall = max(lastall, sh_last[v]);
    }
    if (sel == INT_MAX) {                             // rounding left no crossing: last slice with mass
        sel = lastall < 0 ? 0 : lastall;
        sbase = -INFINITY;
    }
    // the chosen slice: one entry per lane
    const T* row = static_cast<const T*>(a.dl) + (long(m) * a.k + a.pos) * long(a.V);
    const int e = sel * kSlice + lane;
    const float we = e < a.V ? exp2f(fmaf(LT::load1(row + e), a.c, -M)) : 0.f;
    const float run = sbase + wave_incl_scan_f32(we);
    const int ehit = wave_min_int((e < a.V && run > thr) ? e : INT_MAX);
    const int elast = -wave_min_int((we > 0.f) ? -e : 1);
    const int y = ehit != INT_MAX ? ehit : (elast >= 0 ? elast : sel * kSlice);
    if (lane == 0) {
        a.tokens[long(m) * a.k + a.pos] = y;
        if (a.stats)     // the row's softmax state and the drawn token's stored logit, for verification
            a.stats[long(m) * a.k + a.pos] = specv_draft_stat{M, tot.b, LT::load1(row + y), a.c, y, {0, 0, 0}};
    }
}

}  // namespace specv

namespace specv {
namespace {

size_t head_workspace_bytes(int R, int k, int V, int d_m, bool state) {
    if (R < 1 || k < 1 || k > SPECV_MAX_K || V < 1 || d_m < 1) return 0;
    const size_t S = (size_t(V) + kSlice - 1) / kSlice;
    const size_t Rb = (size_t(R) + kPartBlock - 1) / kPartBlock * kPartBlock;     // part_at's blocks
    size_t n = 256 + ((Rb * S * sizeof(float2) + 255) & ~size_t(255));
    n += (size_t(R) * 256 * sizeof(float2) + 255) & ~size_t(255);          // range partials (nr <= 256)
    if (state) n += (size_t(R) * k * d_m * sizeof(float) + 255) & ~size_t(255);
    return n;
}

// Markov head (rec == NULL) or RNN head: validation and the per-position launches.
int head_draft(const char* fn, int mode, int dtype, int R, int k, int V, int d_m, const void* backbone_logits,
               const void* emb, const void* rec, const void* proj, const int32_t* prev_token, float temperature,
               uint64_t seed, uint64_t step, const float* uniforms, int32_t* draft_tokens_out,
               void* draft_logits_out, specv_draft_stat* stats_out, void* state_out, void* ws, size_t ws_bytes,
               hipStream_t s) {
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
    a.uniforms = uniforms; a.seed = seed; a.step = step;
    a.tokens = draft_tokens_out; a.dl = draft_logits_out;
    a.stats = mode == SPECV_SAMPLE ? stats_out : nullptr;
    a.hdr = static_cast<WsHeader*>(ws);
    a.part = reinterpret_cast<float2*>(static_cast<char*>(ws) + 256);
    {
        const size_t S = size_t(a.S), Rb = (size_t(R) + kPartBlock - 1) / kPartBlock * kPartBlock;
        a.part_rng = reinterpret_cast<float2*>(static_cast<char*>(ws) + 256 + ((Rb * S * sizeof(float2) + 255) & ~size_t(255)));
    }
    a.rec = rec;
    a.state = nullptr;
    if (rnn)
        a.state = state_out ? state_out : static_cast<char*>(ws) + head_workspace_bytes(R, k, V, d_m, false);
    const bool vec4 = (V % 4) == 0 && (reinterpret_cast<uintptr_t>(backbone_logits) & 7u) == 0 &&
                      (reinterpret_cast<uintptr_t>(draft_logits_out) & 7u) == 0;
    const bool vec8 = (V % 8) == 0 && (reinterpret_cast<uintptr_t>(backbone_logits) & 15u) == 0 &&
                      (reinterpret_cast<uintptr_t>(draft_logits_out) & 15u) == 0;
    const size_t lds = size_t(kSlice) * size_t(d_m * 2 + 16);
    const int run_lds = 2 * kSlice * (d_m * 2) + (kRunThreads / kWave) * kTileBytes;
    if (dtype == SPECV_BF16 && d_m == 256) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(markov_logits_run<true, 8>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, run_lds) != hipSuccess ||
            hipFuncSetAttribute(reinterpret_cast<const void*>(markov_logits_run<false, 8>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, run_lds) != hipSuccess)
            return fail(SPECV_EDEVICE, "%s: cannot raise the LDS limit of the projection kernel", fn);
    }
    int run_ng = 1, run_nr = 8;
    run_grid(R, a.S, run_ng, run_nr);
    a.nr = run_nr;
    const bool pick_wg = a.S <= kPickThreads * kPickPer;   // else one wavefront per request
    // The status word is cleared by position 0's logits kernel (which sets no
    // bits) and set by position 0's pick kernel, which checks prev_token.
    for (int i = 0; i < k; ++i) {
        a.pos = i;
        if (dtype == SPECV_BF16) {
            if (rnn) SPECV_LAUNCH("rnn_state", rnn_state<SPECV_BF16>, R, 256, 0, s, a);
            if (d_m == 256) {
                if (vec8)
                    SPECV_LAUNCH("markov_logits", (markov_logits_run<true, 8>), run_ng * run_nr, kRunThreads,
                                 size_t(run_lds), s, a, run_ng, run_nr);
                else
                    SPECV_LAUNCH("markov_logits", (markov_logits_run<false, 8>), run_ng * run_nr, kRunThreads,
                                 size_t(run_lds), s, a, run_ng, run_nr);
            } else if (vec4)
                SPECV_LAUNCH("markov_logits", markov_logits_mfma<true>, a.S, 256, lds, s, a);
            else
                SPECV_LAUNCH("markov_logits", markov_logits_mfma<false>, a.S, 256, lds, s, a);
            if (d_m == 256)                      // markov_logits_run left range partials
                SPECV_LAUNCH("markov_pick", markov_pick_ranges<SPECV_BF16>, (R + 3) / 4, 256, 0, s, a);
            else if (pick_wg)
                SPECV_LAUNCH("markov_pick", markov_pick_wg<SPECV_BF16>, pick_grid(R), kPickThreads, 0, s, a);
            else
                SPECV_LAUNCH("markov_pick", markov_pick<SPECV_BF16>, (R + 3) / 4, 256, 0, s, a);
        } else {
            if (rnn) SPECV_LAUNCH("rnn_state", rnn_state<SPECV_F32>, R, 256, 0, s, a);
            const long items = long(R) * a.S;
            SPECV_LAUNCH("markov_logits", markov_logits_fma, (items + 3) / 4, 256, 0, s, a);
            if (pick_wg)
                SPECV_LAUNCH("markov_pick", markov_pick_wg<SPECV_F32>, pick_grid(R), kPickThreads, 0, s, a);
            else
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
                            const void* emb, const void* proj, const int32_t* prev_token, float temperature,
                            uint64_t seed, uint64_t step, const float* uniforms, int32_t* draft_tokens_out,
                            void* draft_logits_out, specv_draft_stat* draft_stats_out, void* ws, size_t ws_bytes,
                            specv_stream stream) {
    return specv::head_draft("markov_draft", mode, dtype, R, k, V, d_m, backbone_logits, emb, nullptr, proj,
                             prev_token, temperature, seed, step, uniforms, draft_tokens_out, draft_logits_out,
                             draft_stats_out, nullptr, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

extern "C" size_t rnn_draft_workspace_bytes(int R, int k, int V, int d_m) {
    return specv::head_workspace_bytes(R, k, V, d_m, true);
}

extern "C" int rnn_draft(int mode, int dtype, int R, int k, int V, int d_m, const void* backbone_logits,
                         const void* emb, const void* rec, const void* proj, const int32_t* prev_token,
                         float temperature, uint64_t seed, uint64_t step, const float* uniforms,
                         int32_t* draft_tokens_out, void* draft_logits_out, specv_draft_stat* draft_stats_out,
                         void* state_out, void* ws, size_t ws_bytes, specv_stream stream) {
    if (!rec) {
        specv::clear_error();
        return specv::fail(SPECV_EINVAL, "rnn_draft: NULL required pointer (rec)");
    }
    return specv::head_draft("rnn_draft", mode, dtype, R, k, V, d_m, backbone_logits, emb, rec, proj, prev_token,
                             temperature, seed, step, uniforms, draft_tokens_out, draft_logits_out, draft_stats_out,
                             state_out, ws, ws_bytes, static_cast<hipStream_t>(stream));
}
