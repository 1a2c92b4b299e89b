// spec_verify: the exact acceptance rule over a flattened, tagged varlen batch.
//
// Pages: every selected draft token becomes one element of a single batch and a
// tag tensor (request, position) carries the in-sequence dependency ("刚融完500亿
// 创始人亲自下场写代码…", engineering table, row "内核利用率暴跌"); verified tokens
// are kept and the first divergence is resampled ("DSpark 的 661% 提速，是真突破
// 还是数字游戏？", section 一); rejection sampling keeps the target's distribution
// ("DeepSeek服务器不再卡顿！…", section "成本与质量的考量").
//
// Batch layout (spec_schedule / spec_flatten): rows [0, N) are the verified rows,
// request-major, request r's at [cu_rows[r], cu_rows[r+1]); rows [N, N + R) are
// the bonus rows, request r's at N + r. N = cu_rows[R]; n_rows = N + R.
//
// Kernels, in stream order:
//   verify_stream    (spec_verify; under spec_step verify_step_stream, which
//                    runs this round's schedule in its workgroup 0 and streams
//                    the rows (r, 0) in the others meanwhile, then streams the
//                    batch like verify_stream in all of them)
//                    the HBM stream. Work item = one chunk of 64 * kNV 16-byte
//                    vectors of one logit row. Items: the target chunks of all
//                    rows, then (sampling) the draft chunks of the verified rows,
//                    so every item costs the same. Wavefront w of the persistent
//                    grid takes items w, w + nw, w + 2 nw, ... (at any moment the
//                    grid reads one dense window of the item range). Each
//                    wavefront loads item i+1 while it reduces item i to a
//                    partial: (max, lowest index) in greedy mode, the base-2
//                    softmax state (M, S) of the chunk in sampling mode (M = max
//                    of logit * log2(e) / tau, S = sum of exp2(that - M)). No
//                    atomics, no waits: all of the step's logit traffic is here.
//   verify_decide    one 1024-thread workgroup per request (sampling with
//                    fewer requests than compute units: two or four; with more
//                    requests than compute units: 512 threads, two per unit,
//                    so that all are resident at once): merges
//                    each row's chunk partials, decides every verified row,
//                    finds the first rejection a_r and writes the accepted
//                    length and tokens. Greedy: complete. Sampling: a request
//                    with a_r < L_r draws from max(0, p - q). With the library's
//                    uniforms its wavefronts run rejection trials from p side by
//                    side (chunk masses from the partials, one chunk read per
//                    trial); with the caller's uniforms, or when all trials are
//                    rejected, it re-reads its rejected row pair with all its
//                    wavefronts for the chunk masses of the residual (kept in
//                    LDS; split over the request's workgroups, which exchange
//                    their masses through device-scope stores and one arrival
//                    counter, the last to arrive drawing) and draws the token by
//                    the inverse CDF. With every row kept it draws the bonus
//                    token from p of the bonus row (chunk masses from the
//                    partials).
#include <atomic>
#include <chrono>
#include <climits>
#include <mutex>
#include <random>

#include "common.h"
#include "host.h"
#include "schedule_dev.h"

namespace specv {

constexpr int kStreamThreads = 1024;        // verify_stream: one workgroup per compute unit
constexpr int kPhaseSlots = 2 * kStreamThreads;   // slots described in LDS at a time
constexpr int kDecideThreads = 1024;        // verify_decide: 16 wavefronts per workgroup, or
constexpr int kDecideHalf = 512;            // 8 (two workgroups per compute unit)
constexpr int kMaxChunks = 4096;            // sampling: chunks per row (residual masses live in LDS)
constexpr int kResidualTrials = 16;         // counter-based uniforms: rejection trials of the residual draw per
                                            // round (the first round's uniforms are tabled in phase 1)
constexpr int kTrialsMax = 64;              // trials before the inverse-CDF fallback (at most four rounds)
constexpr int kNV = 4;                      // 16-byte vectors per lane per item
constexpr int kChunkVecs = kWave * kNV;     // vectors per chunk

__host__ __device__ constexpr int chunk_elems(int vec) { return kChunkVecs * vec; }
static int chunk_len(int dtype) { return chunk_elems(dtype == SPECV_BF16 ? 8 : 4); }

struct RowRec {                             // one per flattened row (sampling)
    float ax, bx;                           // target / draft logit at the draft token
};

struct VerifyArgs {
    int R, k, V, C, CH, Bmax;               // C chunks of CH logits per row
    const void* target;
    const void* draft;
    const int32_t* tokens;
    const int32_t* tags;
    const int32_t* cu_rows;
    const int32_t* n_rows;
    const float* uniforms;                  // [R, k+1], or NULL: counter-based uniforms (common.h)
    const specv_draft_stat* stats;          // [R, k] or NULL (sampling): q's state per draft row; no draft items
    uint64_t seed, step;                    // the key of those uniforms
    float c;                                // log2(e) / tau
    int32_t* acc_len;
    int32_t* out_tokens;
    float* diag;
    WsHeader* hdr;
    float2* part_p;                         // [Bmax * C] target chunk partials
    float2* part_q;                         // [Bmax * C] draft chunk partials (sampling)
    RowRec* rec;                            // [Bmax]
    float* res_mass;                        // [R * C] sampling: residual chunk masses shared by a request's decide workgroups
    int* res_cnt;                           // [R] arrivals per request (zeroed by verify_stream)
    int nsplit;                             // sampling: decide workgroups per request (1, 2 or 4)
    SchedArgs next;                         // the next round's schedule (spec_verify_ex)
    int has_next;                           // 1: verify_decide runs `next` as workgroup R
    int pre0;                               // 1: rows streamed beside the schedule (spec_step): npre kinds
    int npre;                               //    of row per request, kind 0 target (r, 0), kind 1 target
                                            //    (r, 1), kind 2 draft (r, 0), into part0 / ax0
    float2* part0;                          // [npre * R * C] chunk partials of those rows (kind-major)
    float* ax0;                             // [npre * R] their logits at draft tokens x[r, 0], x[r, 1], x[r, 0]
    uint64_t* flag;                         // spec_step: [0] the schedule's completion mark, [1] a late waiter's
    uint64_t token;                         // spec_step: this call's mark (unique per call, never 0)
    int grid;                               // workgroups of the streaming launch (gridDim.x, which this
                                            // source would read through a call and a memory round trip)
};

struct Layout {
    size_t part_p, part_q, rec, res_mass, res_cnt, part0, ax0, flag, total;
};

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static Layout ws_layout(int R, int k, int V) {
    Layout l;
    const size_t C = (size_t(V) + chunk_elems(4) - 1) / chunk_elems(4);   // fp32 has the most chunks
    const size_t B = size_t(R) * size_t(k + 1);
    size_t off = align256(sizeof(WsHeader));
    l.part_p = off;  off = align256(off + B * C * sizeof(float2));
    l.part_q = off;  off = align256(off + B * C * sizeof(float2));
    l.rec = off;     off = align256(off + B * sizeof(RowRec));
    l.res_mass = off; off = align256(off + size_t(R) * C * sizeof(float));
    l.res_cnt = off; off = align256(off + size_t(R) * sizeof(int));
    l.part0 = off;   off = align256(off + 3 * size_t(R) * C * sizeof(float2));
    l.ax0 = off;     off = align256(off + 3 * size_t(R) * sizeof(float));
    l.flag = off;    off = align256(off + 2 * sizeof(uint64_t));
    l.total = off;
    return l;
}

// ---------------------------------------------------------------------------
// chunk loads
// ---------------------------------------------------------------------------

// Raw logits of one chunk for one lane: kNV 16-byte vectors (VEC) or kNV * kVec
// scalars (unaligned rows, or V not a multiple of the vector width).
template <int DT, bool VEC>
struct Raw {
    using LT = Logit<DT>;
    using T = typename LT::T;
    static constexpr int kVec = LT::kVec;
    static constexpr int kE = kNV * kVec;           // logits per lane per chunk
    uint4 v[VEC ? kNV : 1];
    float s[VEC ? 1 : kE];

    // Lane's element q of a chunk sits at chunk offset
    // (q / kVec * 64 + lane) * kVec + q % kVec in both layouts; for fixed q the
    // offsets increase with the lane, for a fixed lane they increase with q.
    __device__ __forceinline__ static int offset(int q, int lane) {
        return ((q / kVec) * kWave + lane) * kVec + q % kVec;
    }

    // Load the chunk starting at element `beg`; `full` = the whole chunk lies
    // inside the row (else the elements past V are read from the row's last
    // position and masked by widen). Every call issues the same loads whatever
    // the arguments, so the compiler's load counting stays exact across the
    // streaming loop's branches (a path with fewer loads makes it wait for all).
    __device__ __forceinline__ void load(const T* row, int beg, int V, int lane, bool full) {
        if constexpr (VEC) {
            using U4 = unsigned int __attribute__((ext_vector_type(4)));
            const auto* vr = as_global(reinterpret_cast<const U4*>(row));
            const int first = beg / kVec + lane, last = V / kVec - 1;
            (void)full;
#pragma unroll
            for (int u = 0; u < kNV; ++u) {
                // read once per call: non-temporal, so the stream does not fill the
                // caches (and the Infinity Cache) with rows nothing reads again soon
                const U4 t = __builtin_nontemporal_load(vr + min(first + u * kWave, last));
                v[u] = make_uint4(t.x, t.y, t.z, t.w);
            }
        } else {
#pragma unroll
            for (int q = 0; q < kE; ++q) {
                const int e = beg + offset(q, lane);
                const float t = LT::load1(row + min(e, V - 1));
                s[q] = e < V ? t : -INFINITY;
            }
        }
    }

    // Widen to float; with !full the elements past the end of the row are -inf.
    __device__ __forceinline__ void widen(int beg, int V, int lane, bool full, float (&x)[kE]) const {
        if constexpr (VEC) {
#pragma unroll
            for (int u = 0; u < kNV; ++u) {
                float t[kVec];
                LT::unpack(v[u], t);
#pragma unroll
                for (int e = 0; e < kVec; ++e) x[u * kVec + e] = t[e];
            }
            if (!full) {
                const int nv = V / kVec - beg / kVec - lane;
#pragma unroll
                for (int u = 0; u < kNV; ++u)
                    if (u * kWave >= nv) {
#pragma unroll
                        for (int e = 0; e < kVec; ++e) x[u * kVec + e] = -INFINITY;
                    }
            }
        } else {
#pragma unroll
            for (int q = 0; q < kE; ++q) x[q] = s[q];
        }
    }
};

// Largest of a lane's values (pairs folded with three-input max).
template <int E>
__device__ __forceinline__ float lane_max(const float (&x)[E]) {
    float m = fmaxf(x[0], x[1]);
#pragma unroll
    for (int q = 2; q + 1 < E; q += 2) m = fmaxf(m, fmaxf(x[q], x[q + 1]));
    if (E % 2) m = fmaxf(m, x[E - 1]);
    return m;
}

// Base-2 softmax state of one chunk of x * c over the wave: M = max, S = sum
// of exp2(x * c - M); (-inf, 0) for a chunk of padding only.
template <int E>
__device__ __forceinline__ float2 chunk_softmax(const float (&x)[E], float c) {
    const float M = wave_max_dpp(lane_max(x)) * c;
    if (M == -INFINITY) return make_float2(-INFINITY, 0.f);
    float acc[4];                                       // four chains for latency
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = __builtin_amdgcn_exp2f(fmaf(x[q], c, -M));
#pragma unroll
    for (int q = 4; q < E; ++q) acc[q % 4] += __builtin_amdgcn_exp2f(fmaf(x[q], c, -M));
    return make_float2(M, wave_sum_dpp((acc[0] + acc[1]) + (acc[2] + acc[3])));
}

// (max, lowest index) of one chunk over the wave. A chunk holding a NaN or +inf
// gives (+inf, INT_MIN), which wins every merge: the row's maximum is then +inf,
// the mark of a row that is not finite. Each logit is folded into a scaled sum,
// in which any NaN or +inf survives and finite values cannot overflow (-inf
// alone, a valid logit, leaves -inf).
template <class RW, int E>
__device__ __forceinline__ float2 chunk_argmax(const float (&x)[E], int beg, int lane) {
    float fold = 0.f;
#pragma unroll
    for (int q = 0; q < E; ++q) fold = fmaf(x[q], 0x1p-64f, fold);
    if (__ballot(nan_or_posinf_bits(fold))) return make_float2(INFINITY, __int_as_float(INT_MIN));
    const float lm = lane_max(x);
    const float M = wave_max_dpp(lm);
    int idx = INT_MAX;
    if (lm == M && M != -INFINITY) {
#pragma unroll
        for (int q = E - 1; q >= 0; --q)               // offsets increase with q: keep the first
            if (x[q] == M) idx = beg + RW::offset(q, lane);
    }
    return make_float2(M, __int_as_float(wave_min_int_dpp(idx)));
}

// ---------------------------------------------------------------------------
// verify_stream
// ---------------------------------------------------------------------------

// One workgroup of kStreamThreads per compute unit. The slot space is static:
// the target chunks of all Bmax = R (k+1) possible rows, then (sampling) the
// draft chunks of all of them; a slot is live when its row exists in this
// call's batch (target: row < n_rows; draft: row < N, the verified rows).
// Workgroup b owns slots b, b + G, b + 2G, ... (so the grid sweeps one dense
// window of the slot space). It describes up to kPhaseSlots of them at a time
// in LDS (tag -> row pointer, row, chunk, token index), live ones only, in slot
// order; its wavefronts then take the items one at a time from an LDS counter,
// so a wavefront that the compute unit serves faster simply takes more items
// and all of them finish together. Each wavefront loads its next item while it
// reduces the current one.
//
// The slot descriptions and results of a phase live in LDS (StreamLds, carved
// from one byte range): verify_stream declares it, verify_step_stream reuses
// the schedule's dynamic LDS for it.
struct StreamLds {
    uint64_t* d_row;         // row pointer
    float2* st_p;            // the items' partials, written out after the phase
    int* d_t;                // flattened row
    int* d_cf;               // chunk << 2 | draft << 1 | ok
    int* d_tok;              // the row's draft token (sampling, verified rows), or -1
    float* st_x;             // logit at the draft token, if the item holds it
    int* sh;                 // [64] scan scratch
    int* next_item;          // the phase's item counter
    unsigned char* st_f;     // 1: st_x holds the item's value
};
constexpr size_t kStreamLdsBytes = size_t(kPhaseSlots) * (8 + 8 + 4 + 4 + 4 + 4 + 1) + 64 * 4 + 16;

__device__ __forceinline__ StreamLds stream_lds_at(unsigned char* p) {
    StreamLds l;
    l.d_row = reinterpret_cast<uint64_t*>(p);
    l.st_p = reinterpret_cast<float2*>(p + 8 * kPhaseSlots);
    l.d_t = reinterpret_cast<int*>(p + 16 * kPhaseSlots);
    l.d_cf = reinterpret_cast<int*>(p + 20 * kPhaseSlots);
    l.d_tok = reinterpret_cast<int*>(p + 24 * kPhaseSlots);
    l.st_x = reinterpret_cast<float*>(p + 28 * kPhaseSlots);
    l.sh = reinterpret_cast<int*>(p + 32 * kPhaseSlots);
    l.next_item = reinterpret_cast<int*>(p + 32 * kPhaseSlots + 64 * 4);
    l.st_f = p + 32 * kPhaseSlots + 64 * 4 + 16;
    return l;
}

// The batch (tags, cu_rows, n_rows) is read with device-scope atomic loads:
// under spec_step it is written by another workgroup of the same launch
// (device-scope atomic stores), and such loads see it without invalidating
// any cache.
__device__ __forceinline__ int load_dev(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT, int MODE, bool VEC, bool PRE = false>
__device__ __forceinline__ void stream_slots(const VerifyArgs& a, const StreamLds& lds) {
    using RW = Raw<DT, VEC>;
    using T = typename RW::T;
    constexpr int E = RW::kE;
    constexpr int GW = RW::kVec;
    constexpr bool SAMPLE = MODE == SPECV_SAMPLE;
    uint64_t* const d_row = lds.d_row;
    int* const d_t = lds.d_t;
    int* const d_cf = lds.d_cf;
    int* const d_tok = lds.d_tok;
    float2* const st_p = lds.st_p;
    float* const st_x = lds.st_x;
    unsigned char* const st_f = lds.st_f;
    int* const sh = lds.sh;
    int& next_item = *lds.next_item;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const uint32_t G = uint32_t(a.grid), b = blockIdx.x;
    if (b == 0 && tid == 0) a.hdr->status = 0u;
    if (SAMPLE && b == 0 && a.nsplit > 1)            // verify_decide's per-request arrival counters
        for (int i = tid; i < a.R; i += kStreamThreads) a.res_cnt[i] = 0;
    const int C = a.C, CH = a.CH, V = a.V, K = a.k;
    // rows streamed beside the schedule (spec_step): the target rows (r, 0); with PRE
    // also target (r, 1) and, if npre > 2, draft (r, 0)
    const bool pre_d0 = PRE && a.npre > 2;
    const uint32_t region = uint32_t(a.Bmax) * uint32_t(C);          // slots per tensor
    const uint32_t slots = (SAMPLE && !a.stats) ? 2 * region : region;
    if (b >= slots) return;
    const uint32_t mine = (slots - 1 - b) / G + 1;                   // slots b + i G, i < mine
    const float c = a.c;

    for (uint32_t p0 = 0; p0 < mine; p0 += kPhaseSlots) {
        const uint32_t np = min(uint32_t(kPhaseSlots), mine - p0);
        // 1. describe this phase's slots; thread tid owns slots 2 tid and 2 tid + 1, and
        //    every thread of wavefront w also describes slot w: the first kWaves slots
        //    are the wavefronts' first items, taken before the scan and kept out of the
        //    shared list. All tag loads are unconditional (a past-the-end slot reads the
        //    phase's last one), so they are in flight together with n_rows: one memory
        //    round trip before the scan instead of a chain of three.
        constexpr int kWaves = kStreamThreads / kWave;
        const int wv = tid >> 6;
        uint32_t sl[3];
        int2 tg[3];
#pragma unroll
        for (int h = 0; h < 3; ++h) {
            const uint32_t i = min(h < 2 ? 2u * uint32_t(tid) + uint32_t(h) : uint32_t(wv), np - 1);
            sl[h] = b + (p0 + i) * G;
            const uint32_t rel = sl[h] >= region ? sl[h] - region : sl[h];
            const int t = int(rel / uint32_t(C));                       // t < Bmax
            tg[h] = make_int2(load_dev(a.tags + 2 * t), load_dev(a.tags + 2 * t + 1));
        }
        // all values at one point: the loads are issued ahead of it and waited for once
        // (otherwise the compiler waits for n_rows first and sinks each tag load into its branch)
        int nr = load_dev(a.n_rows), nv = load_dev(a.cu_rows + a.R);
        asm volatile("" : "+v"(nr), "+v"(nv) : "v"(tg[0].x), "v"(tg[0].y), "v"(tg[1].x), "v"(tg[1].y),
                     "v"(tg[2].x), "v"(tg[2].y));
        const int nrows = min(max(nr, 0), a.Bmax);
        const int nver = min(max(nv, 0), nrows);
        // items with a bad tag keep the first target row as a (harmless) load address
        const uint64_t row0 = reinterpret_cast<uint64_t>(a.target);
        uint64_t rp[3] = {row0, row0, row0};
        int tt[3] = {0, 0, -1}, cf[3] = {0, 0, 0}, tk[3] = {-1, -1, -1}, lv[3] = {0, 0, 0};
#pragma unroll
        for (int h = 0; h < 3; ++h) {
            const uint32_t i = h < 2 ? 2u * uint32_t(tid) + uint32_t(h) : uint32_t(wv);
            const uint32_t slot = sl[h];
            const int tensor = slot >= region ? 1 : 0;
            const uint32_t rel = tensor ? slot - region : slot;
            const int t = int(rel / uint32_t(C));
            const int ch = int(rel - uint32_t(t) * uint32_t(C));
            const int r = tg[h].x, j = tg[h].y;
            if (i >= np || t >= (tensor ? nver : nrows)) continue;
            if (a.pre0 && j == 0 && (tensor == 0 || pre_d0)) continue;   // streamed beside the schedule
            if (PRE && tensor == 0 && j == 1) continue;
            const bool ok = r >= 0 && r < a.R && j >= 0 && j <= K && (tensor == 0 || j < K);
            lv[h] = (h < 2 && i < uint32_t(kWaves)) ? 0 : 1;       // slots 0 .. kWaves-1: not listed
            tt[h] = t;
            cf[h] = (ch << 2) | (tensor << 1) | (ok ? 1 : 0);
            if (ok) {
                const T* row = tensor == 0 ? static_cast<const T*>(a.target) + (long(r) * (K + 1) + j) * long(V)
                                           : static_cast<const T*>(a.draft) + (long(r) * K + j) * long(V);
                rp[h] = reinterpret_cast<uint64_t>(row);
                if (SAMPLE && t < nver && j < K) tk[h] = r * K + j;
            }
        }
        // the draft tokens, loaded while the scan runs (no small loads in the streaming
        // loop: a reused load destination there makes the compiler drain every load)
        int tv[3];
#pragma unroll
        for (int h = 0; h < 3; ++h) tv[h] = tk[h] >= 0 ? a.tokens[tk[h]] : -1;

        struct Cur {
            const T* row;
            int i, cf, x;
        };
        auto issue_at = [&](RW& buf, Cur& m, uint64_t rw, int cfv) {
            m.row = reinterpret_cast<const T*>(
                (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(rw >> 32)))) << 32) |
                uint32_t(__builtin_amdgcn_readfirstlane(int(rw))));
            m.cf = __builtin_amdgcn_readfirstlane(cfv);
            const int beg = (m.cf >> 2) * CH;
            buf.load(m.row, beg, V, lane, beg + CH <= V);    // also for a bad tag: same loads on every path
        };
        // The wavefront's first item (slot w, the same for all its lanes). If that slot is
        // not live, one chunk of the first target row stands in (not reduced, not
        // written; a different chunk per wavefront), so that every wavefront issues the
        // same loads here and the loop below needs no other entry.
        RW q0, q1;
        Cur m0, m1;
        const int pre = lv[2];
        const int pre_t = pre ? tt[2] : -1;
        const int pre_cf = pre ? cf[2] : int((uint32_t(b) * kWaves + uint32_t(wv)) % uint32_t(C)) << 2;
        issue_at(q0, m0, rp[2], pre_cf);
        m0.x = tv[2];

        int nl;
        const int pos = block_exclusive_scan_i32(lv[0] + lv[1], sh, nl, kWaves);
#pragma unroll
        for (int h = 0, q = pos; h < 2; ++h) {
            if (!lv[h]) continue;
            d_row[q] = rp[h];
            d_t[q] = tt[h];
            d_cf[q] = cf[h];
            d_tok[q] = tv[h];
            st_f[q] = 0;
            ++q;
        }
        // the wavefronts' first items are entries nl + w (row -1: none), for the write-out
        m0.i = nl + wv;
        if (lane == 0) {
            d_t[nl + wv] = pre_t;
            d_cf[nl + wv] = pre_cf;
            st_f[nl + wv] = 0;
        }
        if (tid == 0) next_item = 0;
        __syncthreads();

        // 2. stream the live items, one at a time per wavefront
        auto grab = [&]() {
            int i = 0;
            if (lane == 0) i = atomicAdd(&next_item, 1);
            return __builtin_amdgcn_readfirstlane(i);
        };
        auto issue = [&](RW& buf, Cur& m, int i) {
            m.i = i;
            m.x = __builtin_amdgcn_readfirstlane(d_tok[i]);
            issue_at(buf, m, d_row[i], d_cf[i]);
        };
        auto process = [&](const RW& buf, const Cur& m) {
            const int beg = (m.cf >> 2) * CH;
            const bool full = beg + CH <= V;
            float2 P = SAMPLE ? make_float2(-INFINITY, 0.f) : make_float2(-INFINITY, __int_as_float(INT_MAX));
            if (m.cf & 1) {
                float xv[E];
                buf.widen(beg, V, lane, full, xv);
                P = SAMPLE ? chunk_softmax(xv, c) : chunk_argmax<RW>(xv, beg, lane);
                if (SAMPLE && m.x >= beg && m.x < beg + CH && m.x < V) {
                    // the draft token's logit, from the lane that holds it
                    const int off = m.x - beg, vi = off / GW;
                    const int qx = (vi >> 6) * GW + off % GW;
                    if (lane == (vi & (kWave - 1))) {
                        float lx = 0.f;
#pragma unroll
                        for (int q = 0; q < E; ++q)
                            if (q == qx) lx = xv[q];
                        st_x[m.i] = lx;
                        st_f[m.i] = 1;
                    }
                }
            }
            if (lane == 0) st_p[m.i] = P;
        };
        // Two items per wavefront: the next one's loads are issued before the current
        // one is reduced. The last item is handled on its own exit path, so that in
        // the loop every issue is unconditional. Scalar rows: one item at a time
        // (their loads fill twice the registers).
        if constexpr (!VEC) {
            while (true) {                         // q0 holds an issued item here
                process(q0, m0);
                const int i0 = grab();
                if (i0 >= nl) break;
                issue(q0, m0, i0);
            }
        } else {
            while (true) {                         // q0 holds an issued item here
                const int i1 = grab();
                if (i1 >= nl) {
                    process(q0, m0);
                    break;
                }
                issue(q1, m1, i1);
                process(q0, m0);
                const int i0 = grab();
                if (i0 >= nl) {
                    process(q1, m1);
                    break;
                }
                issue(q0, m0, i0);
                process(q1, m1);
            }
        }
        __syncthreads();

        // 3. write the phase's results (no stores while the loads stream: a
        //    store ahead of a load in the memory queue would delay its wait)
        for (int i = tid; i < nl + kStreamThreads / kWave; i += kStreamThreads) {
            const int t = d_t[i], cf = d_cf[i];
            if (t < 0) continue;
            ((cf & 2) ? a.part_q : a.part_p)[long(t) * C + (cf >> 2)] = st_p[i];
            if (st_f[i]) {
                if (cf & 2) a.rec[t].bx = st_x[i]; else a.rec[t].ax = st_x[i];
            }
        }
        __syncthreads();                             // the next phase rewrites the descriptions
    }
}

template <int DT, int MODE, bool VEC>
__global__ __launch_bounds__(kStreamThreads) void verify_stream(VerifyArgs a) {
    __shared__ __align__(16) unsigned char lds[kStreamLdsBytes];
    stream_slots<DT, MODE, VEC>(a, stream_lds_at(lds));
}

// ---------------------------------------------------------------------------
// verify_step_stream (spec_step)
// ---------------------------------------------------------------------------

// spec_step's streaming launch, one workgroup per compute unit. Workgroup 0
// runs this round's schedule (the single-workgroup bucket schedule, `a.next`),
// a latency-bound job that keeps one compute unit busy for ~10 us, and
// publishes its completion. The others meanwhile stream the target row (r, 0)
// of every request, which the batch holds whatever lengths the schedule picks
// (verified row 0 when L_r > 0, the bonus row when L_r = 0), into part0 (and
// ax0, the logit at draft token (r, 0)); when those rows alone would be done
// well before the schedule (PRE, npre > 1: light loads, long blocks), also
// the target rows (r, 1) and the draft rows (r, 0), which every request with
// L_r > 0 needs. Then every workgroup, the schedule's included, streams its
// slots of the batch's other rows as verify_stream does; the others start once
// the schedule is published, which it normally is by the time those rows are
// done. One launch instead of two: the grid does not drain between the rows
// streamed beside the schedule and the rest.
//
// Rows beside the schedule: work items are (kind, request, chunk) triples,
// taken grid-stride by the streaming wavefronts in batches of at most
// kRow0Batch (scalar rows: one item at a time, so that no registers spill). A
// wavefront has only a few items (about five at 256 requests), so the loads go
// through a ring of kRow0Ring buffers: the first kRow0Ring are issued at once,
// and each later one as soon as a buffer is free. Every batch size is its own
// unrolled instance, so the compiler counts the loads in flight exactly. The
// batch's results are stored after its last load.
constexpr int kRow0Batch = 3;        // (more spill registers beside the stream's code)
constexpr int kRow0Ring = 3;         // 16-byte loads; scalar rows (kE floats per buffer) use one buffer

template <int DT, int MODE, bool VEC, int NB, bool PRE>
__device__ __forceinline__ void row0_batch(const VerifyArgs& a, uint32_t i0, uint32_t nw, int lane) {
    using RW = Raw<DT, VEC>;
    using T = typename RW::T;
    constexpr int E = RW::kE;
    constexpr int GW = RW::kVec;
    constexpr bool SAMPLE = MODE == SPECV_SAMPLE;
    const int C = a.C, CH = a.CH, V = a.V, K = a.k;
    constexpr int kRing = VEC ? kRow0Ring : 1;
    // item it: kind it / (R C), request (it % (R C)) / C, chunk it % C; the kind's
    // row and the draft token its logit is taken at (kind 1 with k = 1: none)
    const uint32_t RC = uint32_t(a.R) * uint32_t(C);
    auto kind_of = [&](uint32_t it) { return !PRE || it < RC ? 0u : (it < 2 * RC ? 1u : 2u); };
    auto row_of = [&](uint32_t it) {
        const uint32_t kind = kind_of(it);
        const long r = long((it - kind * RC) / uint32_t(C));
        return kind < 2 ? static_cast<const T*>(a.target) + (r * (K + 1) + kind) * long(V)
                        : static_cast<const T*>(a.draft) + r * K * long(V);
    };
    int xt[NB];
    // the draft tokens of the batch's rows first: a small load issued after
    // the chunk loads would make its wait drain them
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const uint32_t it = i0 + uint32_t(b) * nw, kind = kind_of(it);
        const int j = kind == 1 ? 1 : 0;
        xt[b] = (SAMPLE && j < K) ? a.tokens[long((it - kind * RC) / uint32_t(C)) * K + j] : -1;
    }
    auto issue = [&](RW& buf, int b) {
        const uint32_t it = i0 + uint32_t(b) * nw;
        const int beg = int(it % uint32_t(C)) * CH;
        buf.load(row_of(it), beg, V, lane, beg + CH <= V);
    };
    RW ring[kRing];
#pragma unroll
    for (int b = 0; b < NB && b < kRing; ++b) issue(ring[b], b);
    float2 res[NB];
    float xv[NB];
    bool xf[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const uint32_t it = i0 + uint32_t(b) * nw;
        const int beg = int(it % uint32_t(C)) * CH;
        float x[E];
        ring[b % kRing].widen(beg, V, lane, beg + CH <= V, x);
        if (b + kRing < NB) issue(ring[b % kRing], b + kRing);      // the buffer is free again
        res[b] = SAMPLE ? chunk_softmax(x, a.c) : chunk_argmax<RW>(x, beg, lane);
        xf[b] = false;
        xv[b] = 0.f;
        if (SAMPLE) {
            const int xb = __builtin_amdgcn_readfirstlane(xt[b]);
            if (xb >= 0 && xb >= beg && xb < beg + CH && xb < V) {
                const int off = xb - beg, vi = off / GW;
                const int qx = (vi >> 6) * GW + off % GW;
                if (lane == (vi & (kWave - 1))) {
#pragma unroll
                    for (int q = 0; q < E; ++q)
                        if (q == qx) xv[b] = x[q];
                    xf[b] = true;
                }
            }
        }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const uint32_t it = i0 + uint32_t(b) * nw;
        if (lane == 0) a.part0[it] = res[b];                    // part0[(kind R + r) C + ch]
        if (xf[b]) a.ax0[it / uint32_t(C)] = xv[b];              // ax0[kind R + r]
    }
}

// Streaming wavefront gw of nw: the (kind, request, chunk) items of the rows
// streamed beside the schedule.
template <int DT, int MODE, bool VEC, bool PRE>
__device__ __forceinline__ void row0_items(const VerifyArgs& a, uint32_t gw, uint32_t nw) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t items = uint32_t(PRE ? a.npre : 1) * uint32_t(a.R) * uint32_t(a.C);
    if constexpr (!VEC) {                 // scalar rows: one item at a time (registers)
        for (uint32_t i0 = gw; i0 < items; i0 += nw) row0_batch<DT, MODE, VEC, 1, PRE>(a, i0, nw, lane);
        return;
    }
    static_assert(kRow0Batch == 3, "one case per batch size");
    for (uint32_t i0 = gw; i0 < items; i0 += kRow0Batch * nw) {
        const int nb = int(min(uint32_t(kRow0Batch), (items - 1 - i0) / nw + 1));   // items of this batch
        switch (nb) {
            case 1: row0_batch<DT, MODE, VEC, 1, PRE>(a, i0, nw, lane); break;
            case 2: row0_batch<DT, MODE, VEC, 2, PRE>(a, i0, nw, lane); break;
            default: row0_batch<DT, MODE, VEC, 3, PRE>(a, i0, nw, lane); break;
        }
    }
}

// The wait for the schedule gives up after this long (100 MHz clock ticks):
// only a workgroup 0 kept off the device by other work can take that long.
constexpr uint64_t kScheduleWaitTicks = 100000000ull;    // one second

template <int DT, int MODE, bool VEC, bool PRE>
__global__ __launch_bounds__(kStreamThreads) void verify_step_stream(VerifyArgs a) {
    extern __shared__ __align__(16) uint64_t step_lds[];
    const int tid = threadIdx.x;
    if (blockIdx.x == 0) {
        schedule_bucket_body(a.next, step_lds);
        // publish the batch. Its tags, offsets and row count went out as
        // device-scope atomic stores (coherent across the L2 caches without a
        // write-back, which would take microseconds under the stream's load);
        // each wavefront waits for its own to complete (a workgroup barrier
        // alone orders them at workgroup scope only), then the mark follows
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __syncthreads();
        if (tid == 0) __hip_atomic_store(a.flag, a.token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();                                  // the stream reuses the schedule's LDS
    } else {
        constexpr uint32_t kWaves = kStreamThreads / kWave;
        row0_items<DT, MODE, VEC, PRE>(a, (blockIdx.x - 1) * kWaves + (threadIdx.x >> 6), (a.grid - 1) * kWaves);
        // one thread waits for the mark; the stream reads the batch with
        // device-scope atomic loads (no cache invalidation, which would stall the
        // streaming compute units around), after the barrier
        if (tid == 0) {
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            while (__hip_atomic_load(a.flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.token) {
                __builtin_amdgcn_s_sleep(2);
                if (__builtin_amdgcn_s_memrealtime() - t0 > kScheduleWaitTicks) {
                    // reported by verify_decide; the stream goes on with what the batch holds
                    __hip_atomic_store(a.flag + 1, a.token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
        __syncthreads();
    }
    stream_slots<DT, MODE, VEC, PRE>(a, stream_lds_at(reinterpret_cast<unsigned char*>(step_lds)));
}

// ---------------------------------------------------------------------------
// inverse-CDF helpers (one wavefront)
// ---------------------------------------------------------------------------

// In-chunk inverse CDF. The chunk of CH logits starting at `beg` of the target
// row (and, for PAIR, of the draft row) is loaded in the stream layout; wt(xt,
// xd) is an element's weight, 0 for a target logit of -inf (exp2 of -inf; the
// elements past V read as -inf). Returns the first element whose running sum from
// `base`, in index order, exceeds thr; else the last element with positive
// weight (beg if none). The chunk is kNV groups of 64 lanes x GW elements in
// index order (lane-major inside a group): the group totals pick the group, a
// scan of the lanes' sums picks the lane, and the lane scans its own elements.
// With `vals`, also the target and (PAIR) draft logits at the returned element,
// from the registers where the chunk was loaded in vector form.
template <int DT, bool VEC, bool PAIR, class Wf>
__device__ __forceinline__ int chunk_pick(const typename Logit<DT>::T* trow, const typename Logit<DT>::T* drow, int beg,
                                          int V, float base, float thr, Wf wt, float2* vals = nullptr) {
    using RW = Raw<DT, VEC>;
    constexpr int GW = RW::kVec;
    const int lane = threadIdx.x & (kWave - 1);
    const bool full = beg + chunk_elems(GW) <= V;
    const int nv = VEC ? V / GW - beg / GW - lane : 0;
    // scalar rows: group u's logits of the lane, -inf past V; loaded group by
    // group (pass 1 keeps only the group sums, the crossing group is reloaded),
    // so that few loads are in flight at once
    auto scalar_group = [&](int u, float (&xt)[GW], float (&xd)[GW]) {
#pragma unroll
        for (int e = 0; e < GW; ++e) {
            const int x = beg + RW::offset(u * GW + e, lane);
            xt[e] = x < V ? RW::LT::load1(trow + x) : -INFINITY;
            if constexpr (PAIR) xd[e] = x < V ? RW::LT::load1(drow + x) : -INFINITY;
        }
    };
    RW rt, rd;
    if constexpr (VEC) {
        rt.load(trow, beg, V, lane, full);
        if constexpr (PAIR) rd.load(drow, beg, V, lane, full);
    }
    // VEC: all weights stay in registers; scalar rows keep none
    float w[VEC ? kNV : 1][GW], ls[kNV], gt[kNV];
#pragma unroll
    for (int u = 0; u < kNV; ++u) {
        float xt[GW], xd[GW];
        if constexpr (VEC) {
            RW::LT::unpack(rt.v[u], xt);
            if constexpr (PAIR) RW::LT::unpack(rd.v[u], xd);
        } else {
            scalar_group(u, xt, xd);
        }
        const bool ok = !VEC || full || u * kWave < nv;
        ls[u] = 0.f;
#pragma unroll
        for (int e = 0; e < GW; ++e) {
            const float we = ok ? wt(xt[e], PAIR ? xd[e] : 0.f) : 0.f;
            if constexpr (VEC) w[u][e] = we;
            ls[u] += we;
        }
        if constexpr (!VEC) __builtin_amdgcn_sched_barrier(0);
    }
    // weights of group u (VEC: kept; scalar rows: reloaded and recomputed, the same values)
    auto group_w = [&](int u, float (&wu)[GW], float (&xt)[GW], float (&xd)[GW]) {
        if constexpr (VEC) {
#pragma unroll
            for (int e = 0; e < GW; ++e) wu[e] = w[u][e];
        } else {
            scalar_group(u, xt, xd);
#pragma unroll
            for (int e = 0; e < GW; ++e) wu[e] = wt(xt[e], PAIR ? xd[e] : 0.f);
        }
    };
#pragma unroll
    for (int u = 0; u < kNV; ++u) gt[u] = wave_sum_dpp(ls[u]);
    float run = base;
#pragma unroll
    for (int u = 0; u < kNV; ++u) {
        if (run + gt[u] > thr) {                        // the crossing is in group u (or, by rounding, later)
            const float incl = wave_incl_scan_f32(ls[u]);
            const uint64_t hit = __ballot(run + incl > thr);
            if (hit) {
                const int l = __builtin_ctzll(hit);
                float wu[GW], xt[GW], xd[GW];
                group_w(u, wu, xt, xd);
                float cum = run + (incl - ls[u]);
                int f = -1, lp = GW - 1;                // first element of the lane past thr
#pragma unroll
                for (int e = 0; e < GW; ++e) {
                    cum += wu[e];
                    if (f < 0 && cum > thr) f = e;
                    if (wu[e] > 0.f) lp = e;
                }
                const int fs = f < 0 ? lp : f;
                const int fe = __builtin_amdgcn_readlane(fs, l);
                const int y = beg + RW::offset(u * GW + fe, l);
                if (vals) {
                    if constexpr (VEC) {
                        float tv[GW], dv[GW];
                        RW::LT::unpack(rt.v[u], tv);
                        if constexpr (PAIR) RW::LT::unpack(rd.v[u], dv);
                        float st = tv[0], sd = PAIR ? dv[0] : 0.f;
#pragma unroll
                        for (int e = 1; e < GW; ++e)
                            if (fs == e) {
                                st = tv[e];
                                if constexpr (PAIR) sd = dv[e];
                            }
                        *vals = make_float2(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(st), l)),
                                            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sd), l)));
                    } else {
                        *vals = make_float2(RW::LT::load1(trow + y), PAIR ? RW::LT::load1(drow + y) : 0.f);
                    }
                }
                return y;
            }
        }
        run += gt[u];
    }
    // no crossing (rounding): the last element with positive weight
    int lastw = -1;
#pragma unroll
    for (int u = 0; u < kNV; ++u) {
        float wu[GW], xt[GW], xd[GW];
        group_w(u, wu, xt, xd);
#pragma unroll
        for (int e = 0; e < GW; ++e)
            if (wu[e] > 0.f) lastw = beg + RW::offset(u * GW + e, lane);
    }
    const int lw = -wave_min_int_dpp(-lastw);
    const int y = lw >= 0 ? lw : beg;
    if (vals) *vals = make_float2(RW::LT::load1(trow + y), PAIR ? RW::LT::load1(drow + y) : 0.f);
    return y;
}

// Chunk holding the draw among C chunk masses, in chunk order: the first chunk
// whose inclusive prefix exceeds thr = u * total, with the prefix before it in
// `base`; without a crossing (rounding), the last chunk with positive mass and
// an in-chunk threshold of +inf.
template <class Mf>
__device__ __forceinline__ int wave_find_chunk(int C, float u, Mf mass_of, float& base, float& cthr) {
    const int lane = threadIdx.x & (kWave - 1);
    float total = 0.f;
    for (int c0 = 0; c0 < C; c0 += kWave) total += wave_sum_dpp(c0 + lane < C ? mass_of(c0 + lane) : 0.f);
    const float thr = u * total;
    float carry = 0.f;
    int last_pos = -1;
    for (int c0 = 0; c0 < C; c0 += kWave) {
        const int cc = c0 + lane;
        const float mc = cc < C ? mass_of(cc) : 0.f;
        const float inc = wave_incl_scan_f32(mc) + carry;
        const uint64_t hit = __ballot(cc < C && inc > thr);
        const uint64_t pos = __ballot(cc < C && mc > 0.f);
        if (pos) last_pos = c0 + 63 - __builtin_clzll(pos);
        if (hit) {
            const int l = __builtin_ctzll(hit);
            base = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inc - mc), l));
            cthr = thr;
            return c0 + l;
        }
        carry = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inc), 63));
    }
    base = 0.f;
    cthr = INFINITY;
    return last_pos < 0 ? 0 : last_pos;
}

// max(0, p - q) of one element. lp = Mp + log2 Zp and lq = Mq + log2 Zq are
// the base-2 log-normalisers of the row pair, so p = exp2(xt * c - lp) with the
// normaliser folded into the exponent. A -inf logit gives probability 0.
__device__ __forceinline__ float residual_weight(float xt, float xd, float c, float lp, float lq) {
    return fmaxf(__builtin_amdgcn_exp2f(fmaf(xt, c, -lp)) - __builtin_amdgcn_exp2f(fmaf(xd, c, -lq)), 0.f);
}

// ---------------------------------------------------------------------------
// verify_decide
// ---------------------------------------------------------------------------

// Residual mass of one chunk of a row pair, one 16-byte vector (or group of
// scalars) at a time so that few values are live at once.
// Scalar rows: the same sum with the chunk read group by group (kVec logits per
// lane of each row at a time), so that few loads are in flight at once.
template <int DT>
__device__ __forceinline__ float scalar_chunk_residual_mass(const typename Logit<DT>::T* trow,
                                                            const typename Logit<DT>::T* drow, int beg, int V,
                                                            int lane, float c, float lp, float lq) {
    using RW = Raw<DT, false>;
    constexpr int GW = RW::kVec;
    float s[2] = {0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kNV; ++u) {
#pragma unroll
        for (int e = 0; e < GW; ++e) {
            const int x = beg + RW::offset(u * GW + e, lane);
            const float xt = x < V ? RW::LT::load1(trow + x) : -INFINITY;
            const float xd = x < V ? RW::LT::load1(drow + x) : -INFINITY;
            s[e & 1] += residual_weight(xt, xd, c, lp, lq);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    return wave_sum_dpp(s[0] + s[1]);
}

template <int DT, bool VEC>
__device__ __forceinline__ float chunk_residual_mass(const Raw<DT, VEC>& rt, const Raw<DT, VEC>& rd, int beg, int V,
                                                     int lane, float c, float lp, float lq) {
    using RW = Raw<DT, VEC>;
    constexpr int GW = RW::kVec;
    const bool full = beg + chunk_elems(GW) <= V;
    const int nv = VEC ? V / GW - beg / GW - lane : 0;
    float s[2] = {0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kNV; ++u) {
        float xt[GW], xd[GW];
        if constexpr (VEC) {
            RW::LT::unpack(rt.v[u], xt);
            RW::LT::unpack(rd.v[u], xd);
        } else {
#pragma unroll
            for (int e = 0; e < GW; ++e) { xt[e] = rt.s[u * GW + e]; xd[e] = rd.s[u * GW + e]; }
        }
        const bool ok = !VEC || full || u * kWave < nv;
        if (ok) {
#pragma unroll
            for (int e = 0; e < GW; ++e)
                s[e & 1] += residual_weight(xt[e], xd[e], c, lp, lq);
        }
    }
    return wave_sum_dpp(s[0] + s[1]);
}

// Softmax state (M, S) of a row from its chunk partials, or (argmax value,
// lowest index) in greedy mode: one wavefront. load_partials issues the first
// kMergePre * 64 partials in one round (lane's partials lane + u * 64, left in
// v); reduce_partials merges them and the rest.
constexpr int kMergePre = 4;

template <bool SAMPLE>
__device__ __forceinline__ void load_partials(const float2* part, int C, int lane, float2 (&v)[kMergePre]) {
#pragma unroll
    for (int u = 0; u < kMergePre; ++u) {
        const int cc = lane + u * kWave;
        v[u] = cc < C ? part[cc] : (SAMPLE ? make_float2(-INFINITY, 0.f) : make_float2(-INFINITY, __int_as_float(INT_MAX)));
    }
}

template <bool SAMPLE>
__device__ __forceinline__ float2 reduce_partials(const float2* part, int C, int lane, const float2 (&v)[kMergePre]) {
    constexpr int kPre = kMergePre;
    float m = -INFINITY, z = 0.f;
    int gi = INT_MAX;
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        if (SAMPLE) lse_merge(m, z, v[u].x, v[u].y);
        else argmax_merge(m, gi, v[u].x, __float_as_int(v[u].y));
    }
    for (int cc = lane + kPre * kWave; cc < C; cc += kWave) {
        const float2 p = part[cc];
        if (SAMPLE) lse_merge(m, z, p.x, p.y);
        else argmax_merge(m, gi, p.x, __float_as_int(p.y));
    }
    if (SAMPLE) {
        const float M = wave_max_dpp(m);
        const float zs = wave_sum_dpp(m == -INFINITY ? 0.f : z * exp2f(m - M));
        return make_float2(M, zs);
    }
    wave_argmax_dpp(m, gi);
    return make_float2(m, __int_as_float(gi));
}

// Chunk holding the draw among C chunks given the inclusive prefix sums `pre`
// of their masses (in LDS): the first chunk whose prefix exceeds
// thr = u * pre[C-1], with the prefix before it in `base`; without one
// (rounding), the last chunk with positive mass and an in-chunk threshold of
// +inf.
__device__ __forceinline__ int wave_find_chunk_prefix(int C, float u, const float* pre, float& base, float& cthr) {
    const int lane = threadIdx.x & (kWave - 1);
    const float thr = u * pre[C - 1];
    for (int c0 = 0; c0 < C; c0 += kWave) {
        const int cc = c0 + lane;
        const uint64_t hit = __ballot(cc < C && pre[min(cc, C - 1)] > thr);
        if (hit) {
            const int ch = c0 + __builtin_ctzll(hit);
            base = ch > 0 ? pre[ch - 1] : 0.f;
            cthr = thr;
            return ch;
        }
    }
    int last_pos = -1;
    for (int c0 = 0; c0 < C; c0 += kWave) {
        const int cc = c0 + lane;
        const uint64_t pos = __ballot(cc < C && pre[min(cc, C - 1)] > (cc > 0 ? pre[max(cc - 1, 0)] : 0.f));
        if (pos) last_pos = c0 + 63 - __builtin_clzll(pos);
    }
    base = 0.f;
    cthr = INFINITY;
    return last_pos < 0 ? 0 : last_pos;
}

// One workgroup per request. Phase 1: wavefront j merges the partials of row
// j of the request, decides it, and the first rejection a_r follows. Phase 2
// (sampling): a request with a_r < L_r draws from the residual of its rejected
// row pair. With counter-based uniforms the wavefronts first run rejection
// trials from p (no re-read of the rows); with caller uniforms, or when every
// trial is rejected, all wavefronts stream the row pair into per-chunk residual
// masses in LDS and wavefront 0 draws by the inverse CDF (chunk, then position
// in the chunk). With every row kept, wavefront 0 draws the bonus token from p
// of the bonus row, chunk masses taken from the partials.
static_assert(kDecideThreads == kSchedThreads, "the next round's schedule runs in a decide workgroup");

// One rejection trial of the residual draw at row a_r (see verify_decide):
// y ~ p by the inverse CDF with u1 (chunk masses of p in pm, plain or as prefix
// sums), kept iff u2 < 1 - q(y) / p(y); returns y, or -1 if it was rejected.
// Only the target chunk is loaded, q's logit at y after the pick: the draft
// chunk along with it (no second round trip) doubled the round's burst of loads
// (16 pairs of 8 KiB per rejecting request at once), 0.7 us slower at 256 requests.
template <int DT, bool VEC>
__device__ __forceinline__ int residual_trial(const typename Logit<DT>::T* trow, const typename Logit<DT>::T* drow,
                                              int C, int CH, int V, bool keep_mass, const float* pm, float4 st, float c,
                                              float u1, float u2) {
    using RW = Raw<DT, VEC>;
    float cb, cth;
    const int cs = keep_mass ? wave_find_chunk_prefix(C, u1, pm, cb, cth)
                             : wave_find_chunk(C, u1, [&](int cc) { return pm[cc]; }, cb, cth);
    float2 xy;
    const int yy = chunk_pick<DT, VEC, false>(trow, drow, cs * CH, V, cb, cth, [&](float xt_, float) {
        return __builtin_amdgcn_exp2f(fmaf(xt_, c, -st.x));
    }, &xy);
    xy.y = RW::LT::load1(drow + yy);
    const float py = exp2f(fmaf(xy.x, c, -st.x)) / st.y;
    const float qy = exp2f(fmaf(xy.y, c, -st.z)) / st.w;
    return py > 0.f && u2 < 1.f - qy / py ? yy : -1;
}

template <int DT, int MODE, bool VEC, int NT, bool NEXT, bool PRE>
// Four wavefronts per SIMD: a 1024-thread workgroup, or two 512-thread ones per
// compute unit (every request resident at once with up to twice as many
// requests as units), so at most 128 VGPRs. NEXT: the launch also runs the next
// round's schedule (a separate instantiation, so that the schedule's register
// pressure stays out of the decisions' code when there is none). PRE: spec_step
// streamed rows of npre > 1 kinds beside the schedule (verify_step_stream).
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void verify_decide(VerifyArgs a) {
    const int nsplit = MODE == SPECV_SAMPLE ? a.nsplit : 1;
    if constexpr (NEXT) {
        static_assert(NT == kSchedThreads, "the next round's schedule runs in a 1024-thread workgroup");
        if (int(blockIdx.x) == nsplit * a.R) {                  // the next round's schedule, beside this round's decisions
            extern __shared__ __align__(16) uint64_t sched_lds[];
            schedule_bucket_body(a.next, sched_lds);
            return;
        }
    }
    using RW = Raw<DT, VEC>;
    using T = typename RW::T;
    constexpr bool SAMPLE = MODE == SPECV_SAMPLE;
    constexpr int kW = NT / kWave;
    __shared__ int keep_s[SPECV_MAX_K + 1];
    __shared__ int g_s[SPECV_MAX_K + 1];
    __shared__ int x_s[SPECV_MAX_K + 1];           // the draft tokens of the request's rows
    __shared__ float4 st_s[SPECV_MAX_K + 1];
    __shared__ float4 prq_s[SAMPLE ? SPECV_MAX_K : 1];   // sampling: p(x), q(x), p(x)/q(x) per verified row
    __shared__ float mass_s[SAMPLE ? kMaxChunks : 1];
    __shared__ int trial_y_s[SAMPLE ? kResidualTrials : 1];
    // counter-based uniforms, computed in phase 1: (u1, u2) of trial t at position i
    // in tu_s[t * kTuStride + i] (trial 0's u1 is also the bonus draw's uniform),
    // the acceptance uniform of row j in ua_s[j]
    constexpr int kTuStride = SPECV_MAX_K + 1;
    __shared__ float2 tu_s[SAMPLE ? kResidualTrials * kTuStride : 1];
    __shared__ float ua_s[SAMPLE ? SPECV_MAX_K : 1];
    __shared__ int bad_s, nonfinite_s, stats_bad_s, rnext_s, last_s, win_s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = int(blockIdx.x) / nsplit, part = int(blockIdx.x) % nsplit;
    const bool writer = part == 0;                 // the workgroup that writes the request's decisions
    const int k = a.k, C = a.C, CH = a.CH, V = a.V;
    const int nrows = min(max(*a.n_rows, 0), a.Bmax);
    const int N = a.cu_rows[a.R];
    const int base = a.cu_rows[r];
    const int L = a.cu_rows[r + 1] - base;
    // sampling: every row's chunk masses of p stay in LDS from phase 1 (as inclusive
    // prefix sums in chunk order) when they fit
    const bool keep_mass = L >= 0 && L <= k && (L + 1) * C <= kMaxChunks;
    const bool gen = SAMPLE && !a.uniforms;        // the library's own uniforms
    int32_t* out = a.out_tokens + long(r) * (k + 1);
    // Chunk partials of this request's row j (batch row t): the rows streamed
    // beside the schedule (spec_step) are in part0, the others in part_p /
    // part_q; ax0 holds those rows' logits at the draft token.
    const int npt = PRE ? 2 : (a.pre0 ? 1 : 0);                 // target rows (r, 0 .. npt - 1)
    const bool pre_d0 = PRE && a.npre > 2;                      // draft row (r, 0)
    auto p_parts = [&](int j, int t) {
        if constexpr (PRE) return j < 2 ? a.part0 + (long(j) * a.R + r) * C : a.part_p + long(t) * C;
        return (a.pre0 && j == 0) ? a.part0 + long(r) * C : a.part_p + long(t) * C;
    };
    auto q_parts = [&](int j, int t) {
        return (PRE && j == 0 && pre_d0) ? a.part0 + (2L * a.R + r) * C : a.part_q + long(t) * C;
    };
    if (a.pre0 && blockIdx.x == 0 && tid == 0) {
        // spec_step: a streaming workgroup that gave up waiting for the schedule
        // voids the call; the mark is cleared for the next call (a replayed graph
        // repeats this call's mark)
        if (a.flag[1] == a.token) atomicOr(&a.hdr->status, SPECV_STATUS_LATE_SCHEDULE);
        a.flag[0] = 0;
    }
    if (tid == 0) {
        bad_s = L < 0 || L > k || base < 0 || base + L > N || N < 0 || N + r >= nrows;
        nonfinite_s = 0;
        stats_bad_s = 0;
        rnext_s = 0;
        win_s = INT_MAX;
    }
    __syncthreads();

    if (!bad_s) {
        // The counter-based uniforms, one Philox block per thread, counted from the
        // workgroup's last thread (wavefronts without rows first): slot s < 16 (L+1)
        // is trial s / (L+1) at position s % (L+1), the next L slots the acceptance
        // uniforms of rows 0..L-1. Computed while the partials are in flight; read
        // after the workgroup barrier.
        auto philox_slots = [&]() {
            if constexpr (SAMPLE) {
                const int npos = L + 1, ntp = kResidualTrials * npos, ns = ntp + L;
                for (int sl = NT - 1 - tid; sl < ns; sl += NT) {
                    const bool trial = sl < ntp;
                    const int t = sl / npos, i = sl % npos, j = sl - ntp;
                    uint64_t w0 = uint64_t(trial ? i : j) + 1u, w1 = uint64_t(r);
                    uint64_t w2 = trial ? kPurposeDraw : kPurposeAccept, w3 = trial ? uint64_t(t) : 0u;
                    philox4x64_10(w0, w1, w2, w3, a.seed, a.step);
                    const float u1 = float(uint32_t(w0 >> 40)) * 0x1p-24f;
                    const float u2 = float(uint32_t(w1 >> 40)) * 0x1p-24f;
                    if (trial) tu_s[t * kTuStride + i] = make_float2(u1, u2);
                    else ua_s[j] = u1;
                }
            }
        };
        bool slots_done = !gen;
        for (int j = wave; j <= L; j += kW) {
            const bool verified = j < L;
            const int t = verified ? base + j : N + r;
            // independent loads first: one round of latency with the partials
            const int tag_r = a.tags[2 * t], tag_j = a.tags[2 * t + 1];
            const int x = verified ? a.tokens[long(r) * k + j] : 0;
            RowRec rc{0.f, 0.f};
            if (SAMPLE && verified) rc = a.rec[t];
            specv_draft_stat ds{};
            if (SAMPLE && verified && a.stats) ds = a.stats[long(r) * k + j];
            if (SAMPLE && verified && j < npt) rc.ax = a.ax0[long(j) * a.R + r];   // streamed beside the schedule
            if (PRE && SAMPLE && verified && j == 0 && pre_d0) rc.bx = a.ax0[2L * a.R + r];
            const float2* pp = p_parts(j, t);
            const float2* pq = q_parts(j, t);
            float2 pv[kMergePre], qv[kMergePre];
            load_partials<SAMPLE>(pp, C, lane, pv);
            if (SAMPLE && verified && !a.stats) load_partials<true>(pq, C, lane, qv);
            float uj = 0.f;
            if (SAMPLE && verified && !gen) uj = a.uniforms[long(r) * (k + 1) + j];
            if (!slots_done) {
                philox_slots();
                slots_done = true;
            }
            const float2 P = reduce_partials<SAMPLE>(pp, C, lane, pv);
            float2 Q = make_float2(-INFINITY, 0.f);
            if (SAMPLE && verified) {
                if (a.stats) {                     // q's state and q(x) from the draft head
                    Q = make_float2(ds.m, ds.z);
                    rc.bx = ds.x_logit;
                } else {
                    Q = reduce_partials<true>(pq, C, lane, qv);
                }
            }
            if (SAMPLE && keep_mass) {
                // the row's chunk masses of p relative to its max as inclusive prefix
                // sums, for a draw from p at this row
                float* mrow = mass_s + j * C;
                float carry = 0.f;
#pragma unroll
                for (int u = 0; u < kMergePre; ++u) {
                    if (u * kWave < C) {
                        const int cc = lane + u * kWave;
                        const float m = cc < C && pv[u].x != -INFINITY ? pv[u].y * exp2f(pv[u].x - P.x) : 0.f;
                        const float inc = wave_incl_scan_f32(m) + carry;
                        if (cc < C) mrow[cc] = inc;
                        carry = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inc), 63));
                    }
                }
                for (int c0 = kMergePre * kWave; c0 < C; c0 += kWave) {
                    const int cc = c0 + lane;
                    float m = 0.f;
                    if (cc < C) {
                        const float2 q = pp[cc];
                        m = q.x == -INFINITY ? 0.f : q.y * exp2f(q.x - P.x);
                    }
                    const float inc = wave_incl_scan_f32(m) + carry;
                    if (cc < C) mrow[cc] = inc;
                    carry = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inc), 63));
                }
            }
            if (lane != 0) continue;               // lane 0 decides the row
            if (tag_r != r || tag_j != j) bad_s = 1;
            if (SAMPLE && verified && a.stats && (__float_as_uint(ds.c) != __float_as_uint(a.c) || ds.token != x))
                stats_bad_s = 1;
            // a row with a NaN or +inf logit: a softmax state (M, S) that is not
            // finite (an all -inf row too: no distribution), or in greedy mode the
            // (+inf, INT_MIN) mark of verify_stream
            const bool nf = SAMPLE ? !(finite_bits(P.x) && finite_bits(P.y) &&
                                       (!verified || (finite_bits(Q.x) && finite_bits(Q.y))))
                                   : __float_as_uint(P.x) == 0x7f800000u;
            if (nf) nonfinite_s = 1;
            const bool xok = x >= 0 && x < V;
            if (writer && verified && !xok) atomicOr(&a.hdr->status, SPECV_STATUS_BAD_TOKEN);
            x_s[j] = x;
            if (!SAMPLE) {
                const int gi = __float_as_int(P.y);
                const int y = gi == INT_MAX ? 0 : gi;
                const bool keep = verified && x == y;
                g_s[j] = y;
                keep_s[j] = keep;
                if (a.diag && writer)
                    reinterpret_cast<float4*>(a.diag)[t] =
                        make_float4(float(y), P.x, 0.f, verified ? (keep ? 1.f : 0.f) : -1.f);
            } else {
                // the keep decision u < min(1, p(x) / q(x)) follows the barrier, when
                // every row's uniform is there (a token outside [0, V): ratio 0, rejected)
                st_s[j] = make_float4(P.x, P.y, Q.x, Q.y);
                float px = 0.f, qx = 0.f, ratio = 0.f;
                if (verified && xok) {
                    px = exp2f(fmaf(rc.ax, a.c, -P.x)) / P.y;
                    qx = exp2f(fmaf(rc.bx, a.c, -Q.x)) / Q.y;
                    ratio = qx > 0.f ? px / qx : INFINITY;
                }
                if (verified) {
                    prq_s[j] = make_float4(px, qx, ratio, 0.f);
                    if (!gen) ua_s[j] = uj;
                }
            }
        }
        if (!slots_done) philox_slots();           // a wavefront without rows
    }
    __syncthreads();
    if (bad_s || nonfinite_s || stats_bad_s) {
        // a data error: the request's results are void (accepted length 0, no tokens)
        if (!writer) return;
        if (tid == 0) {
            atomicOr(&a.hdr->status, bad_s ? SPECV_STATUS_BAD_TAG
                                           : (stats_bad_s ? SPECV_STATUS_BAD_STATS : SPECV_STATUS_NONFINITE));
            a.acc_len[r] = 0;
        }
        if (tid <= k) out[tid] = -1;
        return;
    }
    int acc = L;
    if constexpr (SAMPLE) {
        // every wavefront decides the rows (lane j: row j) and finds a_r itself
        const bool kp = lane < L ? ua_s[lane] < fminf(1.f, prq_s[lane].z) : true;
        const uint64_t rej = __ballot(!kp);
        acc = rej ? __builtin_ctzll(rej) : L;
    } else {
        for (int j = 0; j < L; ++j)
            if (!keep_s[j]) { acc = j; break; }
    }
    // the request's results, by the last wavefront (the first ones start the draw):
    // the accepted length, the kept tokens and -1 after the extra one (the drawn
    // token out[acc] is written by the workgroup that draws it), the rows' records
    if (writer && wave == kW - 1) {
        if (lane <= k && !(SAMPLE && lane == acc)) out[lane] = lane < acc ? x_s[lane] : (lane == acc ? g_s[acc] : -1);
        if (lane == 0) a.acc_len[r] = acc;
        if (SAMPLE && a.diag && lane < L) {
            const float4 q = prq_s[lane];
            reinterpret_cast<float4*>(a.diag)[base + lane] = make_float4(q.x, q.y, q.z, ua_s[lane]);
        }
    }
    if constexpr (SAMPLE) {
        const float4 st = st_s[acc];
        const float c = a.c, lp = st.x + log2f(st.y), lq = st.z + log2f(st.w);
        const T* trow = static_cast<const T*>(a.target) + (long(r) * (k + 1) + acc) * long(V);
        const T* drow = static_cast<const T*>(a.draft) + (long(r) * k + min(acc, k - 1)) * long(V);
        const bool rejected = acc < L;
        if (!rejected && !writer) return;          // the bonus draw needs no re-read: one workgroup
        if (rejected && !a.uniforms) {
            // Counter-based uniforms: the residual by rejection from p. Trial t
            // draws y ~ p of row a_r (chunk masses from the partials) with its
            // first uniform and keeps y iff its second lies below 1 - q(y) / p(y),
            // so a kept y has probability max(0, p(y) - q(y)) per trial: the
            // normalised residual. The trials are independent, so the wavefronts
            // run them side by side, kResidualTrials at a time, and the lowest
            // kept one gives the token; a wavefront stops once a lower trial than
            // its next one was kept. A further round runs only when every trial
            // of the previous ones was rejected (where p and q nearly agree), its
            // uniforms computed by the wavefront that needs them. Every workgroup
            // of the request runs them and reaches the same result; with none of
            // kTrialsMax kept the draw falls back to the residual's inverse CDF
            // (the re-read below) with the uniform of trial kTrialsMax.
            const float* pm = mass_s + (keep_mass ? acc * C : 0);
            if (!keep_mass) {
                const float2* pp = p_parts(acc, base + acc);
                for (int cc = tid; cc < C; cc += NT) {
                    const float2 q = pp[cc];
                    mass_s[cc] = q.x == -INFINITY ? 0.f : q.y * exp2f(q.x - st.x);
                }
                __syncthreads();
            }
            // the kept trial's token (the round that kept it left its token and
            // uniforms at index win % 16) and the bonus row's record: -(kept trial + 1),
            // a_r, the token, the trial's first uniform
            auto emit_kept = [&](int win) {
                if (writer && tid == 0) {
                    const int w16 = win % kResidualTrials;
                    const int y = trial_y_s[w16];
                    out[acc] = y;
                    if (a.diag)
                        reinterpret_cast<float4*>(a.diag)[N + r] =
                            make_float4(-float(win + 1), float(acc), float(y), tu_s[w16 * kTuStride + acc].x);
                }
            };
            for (int t = wave; t < kResidualTrials; t += kW) {                 // the first round
                if (__hip_atomic_load(&win_s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < t) break;
                const float2 uu = tu_s[t * kTuStride + acc];
                const int y = residual_trial<DT, VEC>(trow, drow, C, CH, V, keep_mass, pm, st, c, uu.x, uu.y);
                if (lane == 0 && y >= 0) {
                    trial_y_s[t] = y;
                    atomicMin(&win_s, t);
                }
            }
            __syncthreads();
            const int win = win_s;
            if (win != INT_MAX) {
                emit_kept(win);
                return;
            }
            // Later rounds, only when every earlier trial was rejected (placed after
            // the first round's exit, so that the common path's code keeps its
            // shape). Round t0 runs trials t0 .. t0 + 15 with their uniforms
            // computed into column a_r of the table (the previous round's being
            // spent); a kept trial leaves its token at index t - t0. Every wavefront
            // decides alike whether to run a round: a round keeps only trials >= its
            // first, so the value read after the barrier is at least t0 for all
            // wavefronts or for none.
            for (int t0 = kResidualTrials; t0 < kTrialsMax; t0 += kResidualTrials) {
                if (__hip_atomic_load(&win_s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < t0) break;
                if (tid < kResidualTrials) {
                    float u1, u2;
                    philox_trial(a.seed, a.step, uint32_t(r), uint32_t(acc), uint32_t(t0 + tid), u1, u2);
                    tu_s[tid * kTuStride + acc] = make_float2(u1, u2);
                }
                __syncthreads();
                for (int t = wave; t < kResidualTrials; t += kW) {
                    if (__hip_atomic_load(&win_s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < t0 + t) break;
                    const float2 uu = tu_s[t * kTuStride + acc];
                    const int y = residual_trial<DT, VEC>(trow, drow, C, CH, V, keep_mass, pm, st, c, uu.x, uu.y);
                    if (lane == 0 && y >= 0) {
                        trial_y_s[t] = y;
                        atomicMin(&win_s, t0 + t);
                    }
                }
                __syncthreads();
            }
            if (win_s != INT_MAX) {
                emit_kept(win_s);
                return;
            }
        }
        // a rejected row pair is split between the request's nsplit workgroups: chunks [lo, hi)
        const int Cs = (C + nsplit - 1) / nsplit;
        const int lo = rejected ? min(C, part * Cs) : 0, hi = rejected ? min(C, lo + Cs) : C;
        if (rejected) {
            // the rejected row pair: each wavefront takes the next chunk from an
            // LDS counter (the compute unit serves its waves unevenly) and loads
            // it while it reduces the previous one
            auto issue = [&](RW& rt, RW& rd, int ch) {
                const int beg = ch * CH;
                const bool full = beg + CH <= V;
                rt.load(trow, beg, V, lane, full);
                rd.load(drow, beg, V, lane, full);
            };
            auto grab = [&]() {
                int i = 0;
                if (lane == 0) i = atomicAdd(&rnext_s, 1);
                return lo + __builtin_amdgcn_readfirstlane(i);
            };
            if constexpr (!VEC) {                  // scalar rows: one chunk at a time (registers)
                for (int ch = grab(); ch < hi; ch = grab()) {
                    const float m0 = scalar_chunk_residual_mass<DT>(trow, drow, ch * CH, V, lane, c, lp, lq);
                    if (lane == 0) mass_s[ch] = m0;
                }
            } else {
                RW t0, d0, t1, d1;
                int c0 = grab();
                if (c0 < hi) issue(t0, d0, c0);
                while (c0 < hi) {
                    const int c1 = grab();
                    if (c1 < hi) issue(t1, d1, c1);
                    const float m0 = chunk_residual_mass(t0, d0, c0 * CH, V, lane, c, lp, lq);
                    if (lane == 0) mass_s[c0] = m0;
                    if (c1 >= hi) break;
                    c0 = grab();
                    if (c0 < hi) issue(t0, d0, c0);
                    const float m1 = chunk_residual_mass(t1, d1, c1 * CH, V, lane, c, lp, lq);
                    if (lane == 0) mass_s[c1] = m1;
                }
            }
        } else if (!keep_mass) {
            // bonus row: chunk masses of p relative to Mp, from the partials
            const float2* pp = p_parts(L, N + r);
            for (int cc = tid; cc < C; cc += NT) {
                const float2 q = pp[cc];
                mass_s[cc] = q.x == -INFINITY ? 0.f : q.y * exp2f(q.x - st.x);
            }
        }
        __syncthreads();
        if (rejected && nsplit > 1) {
            // exchange the parts' chunk masses: device-scope stores, then one arrival
            // per part, an acquire-release RMW at agent scope; the part that arrives
            // last reads the others' masses and draws the token. A workgroup barrier
            // orders the other wavefronts' stores at workgroup scope only (it does
            // not wait for them to reach the device), so each wavefront first waits
            // for its own stores to complete.
            float* gm = a.res_mass + long(r) * C;
            for (int cc = lo + tid; cc < hi; cc += NT)
                __hip_atomic_store(gm + cc, mass_s[cc], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_waitcnt(0);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __syncthreads();
            if (tid == 0)
                last_s = __hip_atomic_fetch_add(a.res_cnt + r, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
                         nsplit - 1;
            __syncthreads();
            if (!last_s) return;
            for (int cc = tid; cc < C; cc += NT)
                if (cc < lo || cc >= hi)
                    mass_s[cc] = __hip_atomic_load(gm + cc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (tid == 0) __hip_atomic_store(a.res_cnt + r, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
        }
        if (wave != 0) return;
        float ub;
        if (a.uniforms) {
            ub = a.uniforms[long(r) * (k + 1) + k];
        } else if (rejected) {                     // the fallback after kTrialsMax rejected trials
            float u2;
            philox_trial(a.seed, a.step, uint32_t(r), uint32_t(acc), uint32_t(kTrialsMax), ub, u2);
        } else {
            ub = tu_s[acc].x;                      // U(seed, step, 1, r, a_r): trial 0's first uniform
        }
        float total = 0.f;
        if (rejected)
            for (int c0 = 0; c0 < C; c0 += kWave) total += wave_sum_dpp(c0 + lane < C ? mass_s[c0 + lane] : 0.f);
        float cbase, cthr;
        int y;
        if (rejected && total > 0.f) {             // residual max(0, p - q) of row a_r
            const int cs = wave_find_chunk(C, ub, [&](int cc) { return mass_s[cc]; }, cbase, cthr);
            y = chunk_pick<DT, VEC, true>(trow, drow, cs * CH, V, cbase, cthr, [&](float xt_, float xd_) {
                return residual_weight(xt_, xd_, c, lp, lq);
            });
        } else {                                   // p of row a_r: the bonus row, or a residual without mass
            if (rejected) {
                const float2* pp = p_parts(acc, base + acc);
                for (int cc = lane; cc < C; cc += kWave) {
                    const float2 q = pp[cc];
                    mass_s[cc] = q.x == -INFINITY ? 0.f : q.y * exp2f(q.x - st.x);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
            const int cs = !rejected && keep_mass
                               ? wave_find_chunk_prefix(C, ub, mass_s + L * C, cbase, cthr)
                               : wave_find_chunk(C, ub, [&](int cc) { return mass_s[cc]; }, cbase, cthr);
            y = chunk_pick<DT, VEC, false>(trow, nullptr, cs * CH, V, cbase, cthr, [&](float xt_, float) {
                return __builtin_amdgcn_exp2f(fmaf(xt_, c, -st.x));
            });
        }
        if (lane == 0) {
            out[acc] = y;
            // the bonus row's record: residual mass sum(max(0, p - q)) at row a_r
            // (0 when every row was kept), a_r, the drawn token, its uniform
            if (a.diag) reinterpret_cast<float4*>(a.diag)[N + r] = make_float4(rejected ? total : 0.f, float(acc),
                                                                               float(y), ub);
        }
    }
}

// ---------------------------------------------------------------------------
// host entry
// ---------------------------------------------------------------------------

static int device_cus(int& cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return fail(SPECV_EDEVICE, "spec_verify: cannot query the device");
    return SPECV_OK;
}

// verify_stream: as many kStreamThreads workgroups as are resident at once
// (one per compute unit), no more than there are slots.
template <class K>
static int stream_grid(K kernel, long slots, int cus, int& G) {
    int per = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, kStreamThreads, 0) != hipSuccess || per < 1)
        return fail(SPECV_EDEVICE, "spec_verify: cannot query the occupancy");
    G = int(std::min<long>(long(cus) * per, std::max<long>(1, slots)));
    return SPECV_OK;
}

// verify_decide, with the next round's schedule as one more workgroup when it
// fits one (else launched after it, on the same stream).
template <int DT, int MODE, bool VEC, int NT>
static int launch_decide(VerifyArgs& a, const SchedArgs* next, hipStream_t s) {
    a.has_next = NT == kSchedThreads && next && schedule_is_bucket(*next);
    if constexpr (NT == kSchedThreads) {
        if (a.has_next) {                       // spec_verify_ex: no rows streamed beside a schedule
            auto kernel = verify_decide<DT, MODE, VEC, NT, true, false>;
            a.next = *next;
            const size_t lds = schedule_bucket_lds(next->R, next->k, next->kk);
            if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                    int(lds)) != hipSuccess)
                return fail(SPECV_EDEVICE, "spec_verify: cannot reserve %zu bytes of LDS", lds);
            SPECV_LAUNCH("verify_decide", kernel, a.nsplit * a.R + 1, NT, lds, s, a);
            return SPECV_OK;
        }
    }
    if (a.pre0 && a.npre > 1)
        SPECV_LAUNCH("verify_decide", (verify_decide<DT, MODE, VEC, NT, false, true>), a.nsplit * a.R, NT, 0, s, a);
    else
        SPECV_LAUNCH("verify_decide", (verify_decide<DT, MODE, VEC, NT, false, false>), a.nsplit * a.R, NT, 0, s, a);
    if (next) return schedule_launch(*next, s);
    return SPECV_OK;
}

// spec_step's schedule mark: unique per call in this process (a counter from a
// random start) and never 0, so that neither an earlier call's mark nor
// whatever a new workspace holds passes for this call's.
static uint64_t call_token() {
    static std::atomic<uint64_t> next{[] {
        std::random_device rd;
        return ((uint64_t(rd()) << 32) | rd()) ^ uint64_t(std::chrono::steady_clock::now().time_since_epoch().count());
    }()};
    uint64_t t = 0;
    while (t == 0) t = next.fetch_add(1, std::memory_order_relaxed);
    return t;
}

// Kinds of row streamed beside spec_step's schedule: the target rows (r, 0)
// always (the batch holds them whatever the lengths). When those alone would be
// done well before the schedule (light loads, long blocks: the streaming
// workgroups would wait for it), also the rows that every request with
// L_r >= 1 needs: target (r, 1) and, if the draft rows are read, draft (r, 0);
// as many kinds as it takes to cover the schedule, no more (rows streamed
// beside it go at a lower rate than the batch's own stream). Estimates: the
// schedule takes ~6.3 us + 3.2 ns per (request, position) under the stream's
// load; one kind of row streams at ~6 TB/s.
static int pre_row_kinds(const VerifyArgs& a, const SchedArgs& first, int elem_bytes, bool draft_rows) {
    const double kind_us = double(a.R) * double(a.V) * elem_bytes / 6.0e6;
    const double sched_us = 6.3 + 0.0032 * double(first.R) * double(first.k);
    const int most = draft_rows ? 3 : 2;
    int n = 1;
    while (n < most && n * kind_us < sched_us) ++n;
    return n;
}

// spec_step's streaming launch (verify_step_stream): this round's schedule in
// workgroup 0, the rows of a.npre kinds (pre_row_kinds) in the others, then the
// batch's other rows in all.
template <class K>
static int launch_step_stream(K kernel, VerifyArgs& a, const SchedArgs& first, int cus, hipStream_t s) {
    a.next = first;
    a.pre0 = 1;
    a.token = call_token();
    const size_t lds = std::max(schedule_bucket_lds(first.R, first.k, first.kk), kStreamLdsBytes);
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            int(lds)) != hipSuccess)
        return fail(SPECV_EDEVICE, "spec_step: cannot reserve %zu bytes of LDS", lds);
    a.grid = std::max(2, cus);
    SPECV_LAUNCH("verify_step_stream", kernel, a.grid, kStreamThreads, lds, s, a);
    return SPECV_OK;
}

template <int DT, bool VEC>
static int launch_verify(int mode, VerifyArgs& a, const SchedArgs* next, hipStream_t s,
                         const SchedArgs* first = nullptr) {
    int cus = 0;
    if (int e = device_cus(cus)) return e;
    int G = 0;
    if (mode == SPECV_GREEDY) {
        if (first) {
            a.npre = pre_row_kinds(a, *first, DT == SPECV_BF16 ? 2 : 4, false);
            const int e = a.npre > 1
                              ? launch_step_stream(verify_step_stream<DT, SPECV_GREEDY, VEC, true>, a, *first, cus, s)
                              : launch_step_stream(verify_step_stream<DT, SPECV_GREEDY, VEC, false>, a, *first, cus, s);
            if (e) return e;
        } else {
            auto ks = verify_stream<DT, SPECV_GREEDY, VEC>;
            if (int e = stream_grid(ks, long(a.Bmax) * a.C, cus, G)) return e;
            a.grid = G;
            SPECV_LAUNCH("verify_stream", ks, G, kStreamThreads, 0, s, a);
        }
        return launch_decide<DT, SPECV_GREEDY, VEC, kDecideThreads>(a, next, s);
    }
    // One 1024-thread decide workgroup fits per compute unit. With fewer requests
    // than compute units a rejected row pair is re-read by up to four of them
    // (each with at least a chunk per wavefront); with more requests than compute
    // units (and no next-round schedule in the launch, which needs 1024 threads)
    // the workgroups have 512 threads, two per compute unit, so that all are
    // resident at once instead of running in two rounds. With counter-based
    // uniforms the re-read is the rare fallback after the residual trials, which
    // every workgroup of the request runs in full, so at most two share a request.
    const bool lagged = next && schedule_is_bucket(*next);
    const int threads = (!lagged && a.R > cus) ? kDecideHalf : kDecideThreads;
    a.nsplit = 1;
    if (threads == kDecideThreads) {
        a.nsplit = a.R * 4 <= cus ? 4 : (a.R * 2 <= cus ? 2 : 1);
        if (!a.uniforms && a.nsplit > 2) a.nsplit = 2;
        while (a.nsplit > 1 && a.C < a.nsplit * (kDecideThreads / kWave)) a.nsplit /= 2;
    }
    if (first) {
        a.npre = pre_row_kinds(a, *first, DT == SPECV_BF16 ? 2 : 4, !a.stats);
        const int e = a.npre > 1
                          ? launch_step_stream(verify_step_stream<DT, SPECV_SAMPLE, VEC, true>, a, *first, cus, s)
                          : launch_step_stream(verify_step_stream<DT, SPECV_SAMPLE, VEC, false>, a, *first, cus, s);
        if (e) return e;
    } else {
        auto ks = verify_stream<DT, SPECV_SAMPLE, VEC>;
        if (int e = stream_grid(ks, (a.stats ? 1L : 2L) * a.Bmax * a.C, cus, G)) return e;
        a.grid = G;
        SPECV_LAUNCH("verify_stream", ks, G, kStreamThreads, 0, s, a);
    }
    if (threads == kDecideThreads)
        return launch_decide<DT, SPECV_SAMPLE, VEC, kDecideThreads>(a, next, s);
    return launch_decide<DT, SPECV_SAMPLE, VEC, kDecideHalf>(a, next, s);
}

}  // namespace specv

extern "C" size_t spec_verify_workspace_bytes(int R, int k, int V) {
    if (R < 1 || k < 1 || k > SPECV_MAX_K || V < 1) return 0;
    return specv::ws_layout(R, k, V).total;
}

namespace specv {

// Argument checks and the kernels' arguments; nothing is enqueued.
static int verify_prepare(int mode, int dtype, int R, int k, int V, const void* target_logits,
                          const void* draft_logits, const int32_t* draft_tokens, const int32_t* tags,
                          const int32_t* cu_rows, const int32_t* n_rows, float temperature, uint64_t seed,
                          uint64_t step, const float* uniforms, int32_t* accepted_len_out, int32_t* out_tokens,
                          float* row_diag, void* ws, size_t ws_bytes, uint32_t* status_word,
                          const specv_draft_stat* draft_stats, VerifyArgs& a, bool& vec) {
    if (mode != SPECV_GREEDY && mode != SPECV_SAMPLE)
        return fail(SPECV_EINVAL, "spec_verify: mode %d is neither greedy (0) nor sample (1)", mode);
    if (dtype != SPECV_BF16 && dtype != SPECV_F32)
        return fail(SPECV_EUNSUPPORTED, "spec_verify: dtype %d unsupported (bf16 = 0, f32 = 1)", dtype);
    if (R < 1 || k < 1 || k > SPECV_MAX_K || V < 1)
        return fail(SPECV_EINVAL, "spec_verify: need R >= 1, 1 <= k <= %d, V >= 1 (got R=%d k=%d V=%d)",
                    SPECV_MAX_K, R, k, V);
    if (long(R) * (k + 1) > INT_MAX / 4 || V > INT_MAX - chunk_elems(8))
        return fail(SPECV_EINVAL, "spec_verify: R*(k+1) or V too large");
    if (!target_logits || !draft_tokens || !tags || !cu_rows || !n_rows || !accepted_len_out ||
        !out_tokens || !ws)
        return fail(SPECV_EINVAL, "spec_verify: NULL required pointer");
    if (mode == SPECV_SAMPLE) {
        if (!draft_logits) return fail(SPECV_EINVAL, "spec_verify: sampling needs draft_logits");
        if (!(temperature > 0.f) || !(temperature < INFINITY))
            return fail(SPECV_EINVAL, "spec_verify: temperature must be finite and > 0 (got %g)",
                        double(temperature));
    }
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return fail(SPECV_EINVAL, "spec_verify: workspace must be 256-byte aligned");
    const Layout lay = ws_layout(R, k, V);
    if (ws_bytes < lay.total)
        return fail(SPECV_EINVAL, "spec_verify: workspace of %zu bytes, need %zu", ws_bytes, lay.total);

    if (long(R) * (k + 1) * 2 * ((V + chunk_elems(4) - 1) / chunk_elems(4)) > INT_MAX)
        return fail(SPECV_EUNSUPPORTED, "spec_verify: R*(k+1)*V too large for one call");
    if (mode == SPECV_SAMPLE && (V + chunk_len(dtype) - 1) / chunk_len(dtype) > kMaxChunks)
        return fail(SPECV_EUNSUPPORTED, "spec_verify: sampling supports at most %d chunks of %d logits per row "
                    "(V = %d)", kMaxChunks, chunk_len(dtype), V);
    const int esize = dtype == SPECV_BF16 ? 2 : 4;
    const int vecw = 16 / esize;
    vec = (V % vecw) == 0 && aligned16(target_logits) && (mode == SPECV_GREEDY || aligned16(draft_logits));

    a.R = R; a.k = k; a.V = V;
    a.CH = chunk_len(dtype);
    a.C = (V + a.CH - 1) / a.CH;
    a.Bmax = R * (k + 1);
    a.target = target_logits;
    a.draft = draft_logits;
    a.tokens = draft_tokens;
    a.tags = tags;
    a.cu_rows = cu_rows;
    a.n_rows = n_rows;
    a.uniforms = uniforms;
    a.stats = mode == SPECV_SAMPLE ? draft_stats : nullptr;
    a.seed = seed;
    a.step = step;
    a.c = mode == SPECV_SAMPLE ? float(1.4426950408889634 / double(temperature)) : 1.f;
    a.acc_len = accepted_len_out;
    a.out_tokens = out_tokens;
    a.diag = row_diag;
    char* w = static_cast<char*>(ws);
    // the kernels use only the header's first word, the status
    a.hdr = status_word ? reinterpret_cast<WsHeader*>(status_word) : reinterpret_cast<WsHeader*>(w);
    a.part_p = reinterpret_cast<float2*>(w + lay.part_p);
    a.part_q = reinterpret_cast<float2*>(w + lay.part_q);
    a.rec = reinterpret_cast<RowRec*>(w + lay.rec);
    a.res_mass = reinterpret_cast<float*>(w + lay.res_mass);
    a.res_cnt = reinterpret_cast<int*>(w + lay.res_cnt);
    a.part0 = reinterpret_cast<float2*>(w + lay.part0);
    a.ax0 = reinterpret_cast<float*>(w + lay.ax0);
    a.flag = reinterpret_cast<uint64_t*>(w + lay.flag);
    a.token = 0;
    a.pre0 = 0;
    a.npre = 1;
    a.nsplit = 1;
    a.has_next = 0;
    return SPECV_OK;
}

// Enqueue the kernels of a prepared call; `first`: this round's schedule, run
// beside the rows (r, 0) (spec_step); `next`: the next round's (spec_verify_ex).
static int verify_launch(int mode, int dtype, bool vec, VerifyArgs& a, const SchedArgs* next,
                         const SchedArgs* first, specv_stream stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == SPECV_BF16)
        return vec ? launch_verify<SPECV_BF16, true>(mode, a, next, s, first)
                   : launch_verify<SPECV_BF16, false>(mode, a, next, s, first);
    return vec ? launch_verify<SPECV_F32, true>(mode, a, next, s, first)
               : launch_verify<SPECV_F32, false>(mode, a, next, s, first);
}

static int verify_impl(int mode, int dtype, int R, int k, int V, const void* target_logits, const void* draft_logits,
                       const int32_t* draft_tokens, const int32_t* tags, const int32_t* cu_rows, const int32_t* n_rows,
                       float temperature, uint64_t seed, uint64_t step, const float* uniforms,
                       int32_t* accepted_len_out, int32_t* out_tokens, float* row_diag, void* ws, size_t ws_bytes,
                       const SchedArgs* next, specv_stream stream, uint32_t* status_word = nullptr,
                       const specv_draft_stat* draft_stats = nullptr) {
    VerifyArgs a;
    bool vec = false;
    if (int e = verify_prepare(mode, dtype, R, k, V, target_logits, draft_logits, draft_tokens, tags, cu_rows, n_rows,
                               temperature, seed, step, uniforms, accepted_len_out, out_tokens, row_diag, ws, ws_bytes,
                               status_word, draft_stats, a, vec))
        return e;
    return verify_launch(mode, dtype, vec, a, next, nullptr, stream);
}

}  // namespace specv

extern "C" int spec_verify(int mode, int dtype, int R, int k, int V, const void* target_logits,
                           const void* draft_logits, const int32_t* draft_tokens, const int32_t* tags,
                           const int32_t* cu_rows, const int32_t* n_rows, float temperature, uint64_t seed,
                           uint64_t step, const float* uniforms, int32_t* accepted_len_out, int32_t* out_tokens,
                           float* row_diag, void* ws, size_t ws_bytes, specv_stream stream) {
    specv::clear_error();
    return specv::verify_impl(mode, dtype, R, k, V, target_logits, draft_logits, draft_tokens, tags, cu_rows, n_rows,
                              temperature, seed, step, uniforms, accepted_len_out, out_tokens, row_diag, ws, ws_bytes,
                              nullptr, stream);
}

extern "C" int spec_verify_ex(int mode, int dtype, int R, int k, int V, const void* target_logits,
                              const void* draft_logits, const int32_t* draft_tokens, const int32_t* tags,
                              const int32_t* cu_rows, const int32_t* n_rows, float temperature, uint64_t seed,
                              uint64_t step, const float* uniforms, int32_t* accepted_len_out, int32_t* out_tokens,
                              float* row_diag, void* ws, size_t ws_bytes, const specv_draft_stat* draft_stats,
                              const specv_schedule_job* next, specv_stream stream) {
    using namespace specv;
    clear_error();
    SchedArgs na;
    if (next) {
        if (int e = schedule_prepare(next->R, next->k, next->conf_logit, next->pos_temp, next->tbl_tokens,
                                     next->tbl_thr, next->n_tbl, next->max_len, next->len_out, next->tags_out,
                                     next->cu_rows_out, next->n_rows_out, next->survival_out, next->ws,
                                     next->ws_bytes, "spec_verify_ex (next)", na))
            return e;
        if (next->tags_out == tags || next->cu_rows_out == cu_rows || next->n_rows_out == n_rows)
            return fail(SPECV_EINVAL, "spec_verify_ex: the next schedule must write a batch other than this one");
    }
    return verify_impl(mode, dtype, R, k, V, target_logits, draft_logits, draft_tokens, tags, cu_rows, n_rows,
                       temperature, seed, step, uniforms, accepted_len_out, out_tokens, row_diag, ws, ws_bytes,
                       next ? &na : nullptr, stream, nullptr, draft_stats);
}

// ---------------------------------------------------------------------------
// spec_step: this round's schedule, then its verification
// ---------------------------------------------------------------------------

extern "C" int spec_step(const specv_schedule_job* sched, int mode, int dtype, int V, const void* target_logits,
                         const void* draft_logits, const int32_t* draft_tokens, float temperature, uint64_t seed,
                         uint64_t step, const float* uniforms, int32_t* accepted_len_out, int32_t* out_tokens,
                         float* row_diag, const specv_draft_stat* draft_stats, void* ws, size_t ws_bytes,
                         specv_stream stream) {
    using namespace specv;
    clear_error();
    if (!sched) return fail(SPECV_EINVAL, "spec_step: NULL schedule job");
    SchedArgs sa;
    if (int e = schedule_prepare(sched->R, sched->k, sched->conf_logit, sched->pos_temp, sched->tbl_tokens,
                                 sched->tbl_thr, sched->n_tbl, sched->max_len, sched->len_out, sched->tags_out,
                                 sched->cu_rows_out, sched->n_rows_out, sched->survival_out, sched->ws, sched->ws_bytes,
                                 "spec_step (schedule)", sa))
        return e;
    VerifyArgs a;
    bool vec = false;
    if (int e = verify_prepare(mode, dtype, sched->R, sched->k, V, target_logits, draft_logits, draft_tokens,
                               sched->tags_out, sched->cu_rows_out, sched->n_rows_out, temperature, seed, step,
                               uniforms, accepted_len_out, out_tokens, row_diag, ws, ws_bytes, nullptr, draft_stats, a,
                               vec))
        return e;
    if (!schedule_is_bucket(sa)) {             // fixed lengths, or a schedule beyond one workgroup: in sequence
        if (int e = schedule_launch(sa, static_cast<hipStream_t>(stream))) return e;
        return verify_launch(mode, dtype, vec, a, nullptr, nullptr, stream);
    }
    return verify_launch(mode, dtype, vec, a, nullptr, &sa, stream);
}

// ---------------------------------------------------------------------------
// spec_verify_noalloc: the workspace in a static device array
// ---------------------------------------------------------------------------

namespace specv {

constexpr size_t kNoallocScratchBytes = size_t(SPECV_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

// Every GPU the library runs on holds its own copy of this array until the
// process ends. Host code never uses its name as an address: the per-device
// address comes from hipGetSymbolAddress.
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, looked up on the first call on
// that device (with that device current) and kept.
static int scratch_address(void*& ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return fail(SPECV_EDEVICE, "spec_verify_noalloc: cannot query the current device");
    if (dev >= kMaxDevices)
        return fail(SPECV_EUNSUPPORTED, "spec_verify_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(SPECV_EDEVICE, "spec_verify_noalloc: hipGetSymbolAddress failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    ptr = g_scratch_ptr[dev];
    return SPECV_OK;
}

}  // namespace specv

extern "C" int spec_verify_noalloc(int mode, int dtype, int R, int k, int V, const void* target_logits,
                                   const void* draft_logits, const int32_t* draft_tokens, const int32_t* tags,
                                   const int32_t* cu_rows, const int32_t* n_rows, float temperature, uint64_t seed,
                                   uint64_t step, const float* uniforms, int32_t* accepted_len_out,
                                   int32_t* out_tokens, float* row_diag, uint32_t* status_out, specv_stream stream) {
    using namespace specv;
    clear_error();
    if (R < 1 || k < 1 || k > SPECV_MAX_K || V < 1)
        return fail(SPECV_EINVAL, "spec_verify_noalloc: need R >= 1, 1 <= k <= %d, V >= 1 (got R=%d k=%d V=%d)",
                    SPECV_MAX_K, R, k, V);
    const size_t need = ws_layout(R, k, V).total;
    if (need > kNoallocScratchBytes)
        return fail(SPECV_EUNSUPPORTED,
                    "spec_verify_noalloc: R=%d, k=%d, V=%d needs %zu bytes of scratch, above the static %zu "
                    "(SPECV_NOALLOC_SCRATCH_BYTES); use spec_verify with a workspace",
                    R, k, V, need, kNoallocScratchBytes);
    void* ws = nullptr;
    if (int e = scratch_address(ws)) return e;
    return verify_impl(mode, dtype, R, k, V, target_logits, draft_logits, draft_tokens, tags, cu_rows, n_rows,
                       temperature, seed, step, uniforms, accepted_len_out, out_tokens, row_diag, ws,
                       kNoallocScratchBytes, nullptr, stream, status_out);
}
