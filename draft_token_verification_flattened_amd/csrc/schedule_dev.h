// Device code of the prefix scheduler shared by spec_schedule (its own
// kernels) and spec_verify_ex (which runs the next round's schedule as one
// extra workgroup of its decide launch): keys, the throughput table, the gain,
// the flattening, and the single-workgroup bucket scheduler.
//
// Bit-exactness: survival is float64, quantised to an integer key
// Q = floor(S * 2^32 + 0.5); sums of keys are integers (order-free); the gain
// G(M) uses one fixed float64 formula, with contraction disabled where a
// multiply-add could form, so a host reference computing the same formula gets
// the same bits.
#pragma once

#include <climits>

#include "common.h"

namespace specv {

constexpr int kSchedThreads = 1024;
constexpr int kMaxTbl = 64;

// Sort key: ascending order = Q descending, then position ascending, then
// request ascending. Q <= 2^32 needs 33 bits; position 5 bits; request 14 bits.
__device__ __forceinline__ uint64_t make_key(uint64_t Q, int i, int r) {
    return ((((1ull << 33) - 1ull) - Q) << 19) | (uint64_t(i) << 14) | uint64_t(r);
}
__device__ __forceinline__ uint64_t key_q(uint64_t key) { return ((1ull << 33) - 1ull) - (key >> 19); }

__device__ __forceinline__ double survival_step(float z, float T) {
    const double t = double(z) / double(T);
    return 1.0 / (1.0 + exp(-t));
}

__device__ __forceinline__ uint64_t quantise(double S) {
    // S in [0, 1]: x in [0, 2^32], an integer; only x = 2^32 needs more than 32 bits
    const double x = floor(S * 4294967296.0 + 0.5);
    return x >= 4294967296.0 ? (1ull << 32) : uint64_t(uint32_t(x));
}

// Table lookup: linear interpolation on the segment [B_j, B_j+1) holding bt
// (found by binary search; the batch tokens are strictly increasing).
__device__ __forceinline__ double throughput(int bt, const int* tb, const double* tt, int n) {
#pragma clang fp contract(off)
    if (bt < tb[0]) return (tt[0] * double(bt)) / double(tb[0]);
    if (bt >= tb[n - 1]) return tt[n - 1];
    int lo = 0, hi = n - 1;                 // tb[lo] <= bt < tb[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tb[mid] <= bt) lo = mid; else hi = mid;
    }
    const double frac = double(bt - tb[lo]) / double(tb[hi] - tb[lo]);
    return tt[lo] + (tt[hi] - tt[lo]) * frac;
}

// throughput() at increasing bt: `lo` (start at -1) keeps the segment of the
// previous call, so that only the first in-table lookup searches.
__device__ __forceinline__ double throughput_next(int bt, const int* tb, const double* tt, int n, int& lo) {
#pragma clang fp contract(off)
    if (bt < tb[0]) return (tt[0] * double(bt)) / double(tb[0]);
    if (bt >= tb[n - 1]) return tt[n - 1];
    if (lo < 0) {
        int l = 0, h = n - 1;               // tb[l] <= bt < tb[h]
        while (h - l > 1) {
            const int mid = (l + h) >> 1;
            if (tb[mid] <= bt) l = mid; else h = mid;
        }
        lo = l;
    } else {
        while (tb[lo + 1] <= bt) ++lo;      // bt < tb[n - 1]: stops at n - 2 at most
    }
    const int hi = lo + 1;
    const double frac = double(bt - tb[lo]) / double(tb[hi] - tb[lo]);
    return tt[lo] + (tt[hi] - tt[lo]) * frac;
}

// Block-wide exclusive scan of one 64-bit value per thread; returns the total too.
__device__ __forceinline__ uint64_t block_exclusive_scan_u64(uint64_t v, uint64_t* sh, uint64_t& total) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    uint64_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint64_t t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) sh[w] = incl;
    __syncthreads();
    if (w == 0) {
        const int nw = blockDim.x >> 6;
        uint64_t x = lane < nw ? sh[lane] : 0ull;
        uint64_t xi = x;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            uint64_t t = __shfl_up(xi, o, 64);
            if (lane >= o) xi += t;
        }
        if (lane < nw) sh[lane] = xi - x;
        if (lane == nw - 1) sh[32] = xi;
    }
    __syncthreads();
    const uint64_t res = sh[w] + incl - v;
    total = sh[32];
    __syncthreads();
    return res;
}

// Wave maximum of a double (DPP on both halves), as a scalar.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_d(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(int(b), int(b), CTRL, ROW_MASK, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(int(b >> 32), int(b >> 32), CTRL, ROW_MASK, 0xf, false);
    return __longlong_as_double((long long)(unsigned)lo | ((long long)hi << 32));
}
__device__ __forceinline__ double wave_max_f64(double v) {
    v = fmax(v, dpp_d<0xb1>(v));
    v = fmax(v, dpp_d<0x4e>(v));
    v = fmax(v, dpp_d<0x141>(v));
    v = fmax(v, dpp_d<0x140>(v));
    v = fmax(v, dpp_d<0x142, 0xa>(v));
    v = fmax(v, dpp_d<0x143, 0xc>(v));
    const long long b = __double_as_longlong(v);
    return __longlong_as_double(((long long)__builtin_amdgcn_readlane(int(b >> 32), 63) << 32) |
                                (long long)(unsigned)__builtin_amdgcn_readlane(int(b), 63));
}

// Best prefix over the wave: the largest G, then the smallest M with it.
__device__ __forceinline__ void wave_best_gm(double& g, int& m) {
    const double gm = wave_max_f64(g);
    m = wave_min_int_dpp(g == gm ? m : INT_MAX);
    g = gm;
}

struct SchedArgs {
    int R, k, kk, max_len, n_tbl;
    const float* z;
    const float* T;
    const int32_t* tbl_b;
    const double* tbl_t;
    const int32_t* len_in;          // spec_flatten only
    int32_t* len_out;
    int32_t* tags;
    int32_t* cu_rows;
    int32_t* n_rows;
    double* survival;
    struct SchedWs* ws;
};


// Workspace of spec_schedule's multi-workgroup kernel: an arrival counter
// (cleared by schedule_ws_clear ahead of every launch on the same stream) and
// one best-prefix record per workgroup.
constexpr int kMaxSchedGroups = 256;
struct SchedBest {
    long long g;
    int m;
    int pad;
    uint64_t key;
    uint64_t pad2;
};
struct SchedWs {
    int done;
    int pad[63];
    SchedBest best[kMaxSchedGroups];
};

// Flattened batch for the lengths given by `len_of`, this thread's contiguous
// request range [r0, r1): verified rows first, request-major (request r's at
// cu_rows[r] .. cu_rows[r+1]-1, tags (r, 0) .. (r, L_r - 1)), then one bonus row
// per request at N + r with tag (r, L_r); N = cu_rows[R], n_rows = N + R.
template <typename F>
__device__ __forceinline__ void flatten_block(const SchedArgs& a, int r0, int r1, F len_of, int* sh) {
    constexpr int kKeep = 4;                    // lengths kept in registers; more are recomputed
    int Lk[kKeep];
    int local = 0;
#pragma unroll
    for (int q = 0; q < kKeep; ++q) {
        Lk[q] = r0 + q < r1 ? len_of(r0 + q) : 0;
        local += Lk[q];
    }
    for (int r = r0 + kKeep; r < r1; ++r) local += len_of(r);
    int N;
    int off = block_exclusive_scan_i32(local, sh, N);
    for (int r = r0; r < r1; ++r) {
        int L = 0;
#pragma unroll
        for (int q = 0; q < kKeep; ++q)
            if (r == r0 + q) L = Lk[q];
        if (r >= r0 + kKeep) L = len_of(r);
        a.cu_rows[r] = off;
        if (a.len_out) a.len_out[r] = L;
        for (int j = 0; j < L; ++j) {
            a.tags[2 * (off + j)] = r;
            a.tags[2 * (off + j) + 1] = j;
        }
        a.tags[2 * (N + r)] = r;
        a.tags[2 * (N + r) + 1] = L;
        off += L;
    }
    if (threadIdx.x == 0) {
        a.cu_rows[a.R] = N;
        *a.n_rows = N + a.R;
    }
}

// flatten_block for the bucket scheduler's single workgroup of kSchedThreads
// threads, with LDS to spare: each request marks its rows in `rowmap` (N + R
// entries: request << 6 | position), then one thread per flattened row writes
// its tag, so that a wavefront's tag stores cover one contiguous range (8 bytes
// per row when the tags are 8-byte aligned).
// The batch is written with device-scope atomic stores, which the memory keeps
// coherent across the chip's L2 caches without a cache write-back: spec_step's
// streaming workgroups read it while this workgroup's kernel still runs.
__device__ __forceinline__ void store_dev(int32_t* p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename F>
__device__ __forceinline__ void flatten_rows_lds(const SchedArgs& a, int r0, int r1, F len_of, int* sh,
                                                 int* rowmap) {
    constexpr int kKeep = 4;                    // lengths kept in registers; more are recomputed
    int Lk[kKeep];
    int local = 0;
#pragma unroll
    for (int q = 0; q < kKeep; ++q) {
        Lk[q] = r0 + q < r1 ? len_of(r0 + q) : 0;
        local += Lk[q];
    }
    for (int r = r0 + kKeep; r < r1; ++r) local += len_of(r);
    int N;
    int off = block_exclusive_scan_i32(local, sh, N, kSchedThreads / 64);
    for (int r = r0; r < r1; ++r) {
        int L = 0;
#pragma unroll
        for (int q = 0; q < kKeep; ++q)
            if (r == r0 + q) L = Lk[q];
        if (r >= r0 + kKeep) L = len_of(r);
        store_dev(a.cu_rows + r, off);
        if (a.len_out) a.len_out[r] = L;
        for (int j = 0; j < L; ++j) rowmap[off + j] = (r << 6) | j;
        rowmap[N + r] = (r << 6) | L;
        off += L;
    }
    if (threadIdx.x == 0) {
        store_dev(a.cu_rows + a.R, N);
        store_dev(a.n_rows, N + a.R);
    }
    __syncthreads();
    const int rows = N + a.R;
    if ((reinterpret_cast<uintptr_t>(a.tags) & 7u) == 0) {
        uint64_t* t2 = reinterpret_cast<uint64_t*>(a.tags);     // (request, position): request in the low word
        for (int t = threadIdx.x; t < rows; t += kSchedThreads) {
            const int v = rowmap[t];
            __hip_atomic_store(t2 + t, (uint64_t(uint32_t(v & 63)) << 32) | uint32_t(v >> 6), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    } else {
        for (int t = threadIdx.x; t < rows; t += kSchedThreads) {
            const int v = rowmap[t];
            store_dev(a.tags + 2 * t, v >> 6);
            store_dev(a.tags + 2 * t + 1, v & 63);
        }
    }
}

// ---------------------------------------------------------------------------
// schedule_bucket: the same schedule from one workgroup, for R * k <= 4096.
// The keys are sorted by a bucket pass on their leading bits (bucket order is
// key order) followed by an exact rank inside each bucket; then the prefix
// sums of Q in sorted order give P(M) for every M, and G(M) follows. No
// workgroup waits for another. Inside a bucket every key compares itself with
// every member, so a bucket of s keys costs s steps: many near-equal
// survivals make it slower, never wrong.
// ---------------------------------------------------------------------------

constexpr int kBuckets = 4096;
constexpr int kBucketItems = 4096;          // largest R * k for schedule_bucket

// Bucket of a key, from its Q; ascending bucket = descending Q, so bucket order
// is key order. Survivals S = Q / 2^32 >= 1/4 take steps of 2^-12 in S (buckets
// 0..3072). Smaller ones, which decaying confidences over a long block make
// plentiful, go by octave: the leading one's position and the next bits of Q,
// 128 buckets per octave for S in [1/16, 1/4) (3073..3328), 64 per octave down
// to 2^-10 (3329..3712), 16 per octave below (3713..4064); Q = 0 is bucket 4065.
//
// Below 2^30 the octave bucket is base - (e << nb) - m, with e the leading
// one's position, nb the bits taken after it (7, 6 or 4) and m those bits,
// read from q shifted so that the leading one is bit 31; no branches.
__device__ __forceinline__ int bucket_of_q(uint64_t q) {
    const uint32_t q32 = uint32_t(q);                            // q < 2^30 where used
    const int lz = __builtin_clz(q32 | 1u), e = 31 - lz;         // q32 = 0 is handled below
    const int nb = e >= 28 ? 7 : (e >= 22 ? 6 : 4);
    const int base = e >= 28 ? 3073 + 255 + 28 * 128 : (e >= 22 ? 3329 + 383 + 22 * 64 : 3713 + 351);
    const int m = int(((q32 << lz) >> (31 - nb)) & ((1u << nb) - 1u));
    const int low = q32 == 0 ? 4065 : base - (e << nb) - m;
    return q >= (1ull << 30) ? int(((1ull << 32) - q) >> 20) : low;
}
static_assert(4065 < kBuckets, "bucket range");

// The whole schedule by one workgroup of kSchedThreads threads; `lds` holds
// schedule_bucket_lds(R, k, kk) bytes: keys [R*k] | grouped [n] | sorted [n] |
// bucket counts and offsets [kBuckets] each.
__device__ __forceinline__ void schedule_bucket_body(const SchedArgs& a, uint64_t* lds) {
    __shared__ int tb[kMaxTbl];
    __shared__ double tt[kMaxTbl];
    __shared__ double wg_sh[kSchedThreads / 64];
    __shared__ int wm_sh[kSchedThreads / 64];
    __shared__ int sh[64], sh2[64];
    __shared__ uint64_t kt_sh;
    // kSchedThreads threads (a constant: in a source built with -mno-amdgpu-ieee
    // blockDim is a device-library call that waits on memory)
    const int tid = threadIdx.x, nt = kSchedThreads, lane = tid & 63, wave = tid >> 6, nwav = nt >> 6;
    const int R = a.R, k = a.k, kk = a.kk, n = R * kk, Rk = R * k;
    const bool surv = a.survival != nullptr;
    const int kc = surv ? k : kk;
    uint64_t* keys = lds;
    uint64_t* grp = keys + Rk;
    uint64_t* srt = grp + n;
    int* cnt = reinterpret_cast<int*>(srt + n);
    int* off = cnt + kBuckets;
    double* sg = reinterpret_cast<double*>(keys);

    // The sigmoids and the running products sit at a stride of ks = k | 1
    // doubles per request: the thread that walks one request's positions then
    // reads and writes its own bank pair at every step (an even stride such as
    // 16 doubles would put all 64 lanes on one bank). R * ks doubles fit in the
    // keys and grouped regions (kk >= 1).
    const int ks = k | 1;
    // e / k for e < 4096 and k <= 32 as (e * mk) >> 20, mk = ceil(2^20 / k):
    // exact, since e * (mk * k - 2^20) < 4096 * k < 2^20
    const uint32_t mk = ((1u << 20) + uint32_t(k) - 1u) / uint32_t(k);
    auto div_k = [&](int e) { return int((uint32_t(e) * mk) >> 20); };

    // 1. table, empty histogram, one calibrated sigmoid per (request, position);
    //    every global load is issued before the first use, so they take one
    //    round trip together
    constexpr int kElPer = kBucketItems / kSchedThreads;
    float zv[kElPer], Tv[kElPer];
#pragma unroll
    for (int j = 0; j < kElPer; ++j) {
        const int e = tid + j * nt, i = e - div_k(e) * k;
        zv[j] = 0.f; Tv[j] = 1.f;
        if (e < Rk && i < kc) { zv[j] = a.z[e]; Tv[j] = a.T[i]; }
    }
    int tbv = 0;
    double ttv = 0.0;
    if (tid < a.n_tbl) { tbv = a.tbl_b[tid]; ttv = a.tbl_t[tid]; }          // n_tbl <= kMaxTbl <= nt
    for (int b = tid; b < kBuckets; b += nt) cnt[b] = 0;
    if (tid < a.n_tbl) { tb[tid] = tbv; tt[tid] = ttv; }
#pragma unroll
    for (int j = 0; j < kElPer; ++j) {
        const int e = tid + j * nt;
        if (e < Rk) {
            const int r = div_k(e), i = e - r * k;
            if (i < kc) sg[r * ks + i] = survival_step(zv[j], Tv[j]);
        }
    }
    __syncthreads();

    // this thread's prefix lengths M = p + 1, p in [p0, p1): their throughput
    // does not depend on the keys
    constexpr int kPosPer = kBucketItems / kSchedThreads;
    const int per = (n + nt - 1) / nt;
    const int p0 = min(n, tid * per), p1 = min(n, p0 + per);
    double thr[kPosPer];
    {
        int seg = -1;
#pragma unroll
        for (int q = 0; q < kPosPer; ++q)
            thr[q] = p0 + q < p1 ? throughput_next(R + p0 + q + 1, tb, tt, a.n_tbl, seg) : 0.0;
    }

    // 2. survival: the running products in position order, one thread per
    //    request doing only the chain (its sigmoids read eight at a time) and
    //    writing each product over its sigmoid; then every thread turns its
    //    (request, position) elements into keys and bucket counts and stores the
    //    survival (contiguous). Positions >= kk get a key above every real one.
    constexpr int kSgBatch = 8;
    for (int r = tid; r < R; r += nt) {
        double S = 1.0;
        for (int i0 = 0; i0 < kc; i0 += kSgBatch) {
            double sv[kSgBatch];
#pragma unroll
            for (int q = 0; q < kSgBatch; ++q) sv[q] = i0 + q < kc ? sg[r * ks + i0 + q] : 1.0;
#pragma unroll
            for (int q = 0; q < kSgBatch; ++q)
                if (i0 + q < kc) {
                    S = S * sv[q];
                    sg[r * ks + i0 + q] = S;
                }
        }
    }
    __syncthreads();
    // this thread's keys stay in registers (kv) from here on, with their buckets
    uint64_t kv[kElPer];
    int bk[kElPer];
#pragma unroll
    for (int j = 0; j < kElPer; ++j) {
        const int e = tid + j * nt;
        kv[j] = ~0ull;
        bk[j] = 0;
        if (e < Rk) {
            const int r = div_k(e), i = e - r * k;
            const double S = i < kc ? sg[r * ks + i] : 0.0;
            if (surv && i < kc) a.survival[e] = S;
            if (i < kk) {
                const uint64_t Q = quantise(S);
                kv[j] = make_key(Q, i, r);
                bk[j] = bucket_of_q(Q);
                atomicAdd(&cnt[bk[j]], 1);
            }
        }
    }
    __syncthreads();                           // the keys go over the products
#pragma unroll
    for (int j = 0; j < kElPer; ++j)
        if (tid + j * nt < Rk) keys[tid + j * nt] = kv[j];
    __syncthreads();

    // 3. bucket offsets (exclusive scan), then every key into its bucket
    {
        constexpr int kPer = kBuckets / kSchedThreads;
        int loc[kPer];
        int sum = 0;
#pragma unroll
        for (int q = 0; q < kPer; ++q) { loc[q] = cnt[tid * kPer + q]; sum += loc[q]; }
        int total;
        int base = block_exclusive_scan_i32(sum, sh, total, nwav);
#pragma unroll
        for (int q = 0; q < kPer; ++q) { off[tid * kPer + q] = base; base += loc[q]; }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kElPer; ++j)
        if (kv[j] != ~0ull) grp[atomicAdd(&off[bk[j]], 1)] = kv[j];
    __syncthreads();

    // 4. exact sorted position: bucket start + smaller keys of the same bucket,
    //    compared four at a time
#pragma unroll
    for (int j = 0; j < kElPer; ++j) {
        const uint64_t x = kv[j];
        if (x == ~0ull) continue;
        const int end = off[bk[j]], beg = end - cnt[bk[j]];
        int rank = beg;
        for (int m = beg; m < end; m += 4) {
            const uint64_t g0 = grp[m];
            const uint64_t g1 = m + 1 < end ? grp[m + 1] : ~0ull;
            const uint64_t g2 = m + 2 < end ? grp[m + 2] : ~0ull;
            const uint64_t g3 = m + 3 < end ? grp[m + 3] : ~0ull;
            rank += int(g0 < x) + int(g1 < x) + int(g2 < x) + int(g3 < x);
        }
        srt[rank] = x;
    }
    __syncthreads();

    // 5. P(M) for every prefix length (contiguous positions per thread), G(M),
    //    and the best prefix: largest G, then smallest M
    //    Q <= 2^32 is scanned as two exact 32-bit sums of its 16-bit halves.
    const uint64_t R32 = uint64_t(R) << 32;
    uint64_t qv[kPosPer];
    int lo = 0, hi = 0;
#pragma unroll
    for (int q = 0; q < kPosPer; ++q) {
        qv[q] = p0 + q < p1 ? key_q(srt[p0 + q]) : 0ull;
        lo += int(qv[q] & 0xffffu);
        hi += int(qv[q] >> 16);
    }
    // both exclusive scans at once; sh and sh2 are not written again before the
    // barrier that follows the gains
    int elo, ehi;
    {
        const int ilo = wave_incl_scan_i32(lo), ihi = wave_incl_scan_i32(hi);
        if (lane == 63) { sh[wave] = ilo; sh2[wave] = ihi; }
        __syncthreads();
        int blo = 0, bhi = 0;
        for (int q = 0; q < wave; ++q) { blo += sh[q]; bhi += sh2[q]; }
        elo = blo + ilo - lo;
        ehi = bhi + ihi - hi;
    }
    uint64_t P = (uint64_t(uint32_t(ehi)) << 16) + uint64_t(uint32_t(elo));
    double g = -1.0;                                          // below every gain
    int m = INT_MAX;
#pragma unroll
    for (int q = 0; q < kPosPer; ++q) {
        if (p0 + q < p1) {
            P += qv[q];
            const int M = p0 + q + 1, bt = R + M;
            const double G = (double(R32 + P) * thr[q]) / double(bt);
            if (G > g) { g = G; m = M; }                      // positions ascend: first M wins ties
        }
    }
    if (tid == 0) {                                           // the empty prefix, M = 0
        const double G0 = (double(R32) * throughput(R, tb, tt, a.n_tbl)) / double(R);
        if (G0 >= g) { g = G0; m = 0; }
    }
    wave_best_gm(g, m);
    if (lane == 0) { wg_sh[wave] = g; wm_sh[wave] = m; }
    __syncthreads();
    if (wave == 0) {
        double gw = lane < nwav ? wg_sh[lane] : -1.0;
        int mw = lane < nwav ? wm_sh[lane] : INT_MAX;
        wave_best_gm(gw, mw);
        if (lane == 0) {
            kt_sh = mw > 0 ? srt[mw - 1] : 0ull;          // 0: below every key
        }
    }
    __syncthreads();

    // 6. lengths and the batch. A request's keys increase with the position, so
    //    the keys <= kt are its first L; the element at L - 1 (the last one in)
    //    writes L, or the element at 0 writes 0 when none is in (also when the
    //    best prefix is empty: every key is above 0). The sorted keys are no
    //    longer needed: their space holds the lengths.
    const uint64_t kt = kt_sh;
    int* len_sh = reinterpret_cast<int*>(srt);
#pragma unroll
    for (int j = 0; j < kElPer; ++j) {
        const int e = tid + j * nt;
        if (e < Rk) {
            const int r = div_k(e), i = e - r * k;
            if (i < kk) {
                const bool in = kv[j] <= kt;
                const bool next_in = i + 1 < kk && keys[e + 1] <= kt;
                if (in && !next_in) len_sh[r] = i + 1;
                if (i == 0 && !in) len_sh[r] = 0;
            }
        }
    }
    __syncthreads();
    auto len_of = [&](int r) { return len_sh[r]; };
    const int rper = (R + nt - 1) / nt;
    const int r0 = min(R, tid * rper), r1 = min(R, r0 + rper);
    // grouped keys are no longer needed: their space holds the row map
    flatten_rows_lds(a, r0, r1, len_of, sh, reinterpret_cast<int*>(grp));
}

__host__ __device__ inline size_t schedule_bucket_lds(int R, int k, int kk) {
    return size_t(R) * k * sizeof(uint64_t) + 2 * size_t(R) * kk * sizeof(uint64_t) + 2 * size_t(kBuckets) * sizeof(int);
}

// Host side (schedule.hip): check a schedule request and fill its arguments,
// then launch it on `s` (the multi-workgroup path, or the fixed lengths).
int schedule_prepare(int R, int k, const float* conf_logit, const float* pos_temp, const int32_t* tbl_tokens,
                     const double* tbl_thr, int n_tbl, int max_len, int32_t* len_out, int32_t* tags_out,
                     int32_t* cu_rows_out, int32_t* n_rows_out, double* survival_out, void* ws, size_t ws_bytes,
                     const char* who, SchedArgs& a);
int schedule_launch(const SchedArgs& a, hipStream_t s);
// True when the single-workgroup bucket kernel handles this request.
inline bool schedule_is_bucket(const SchedArgs& a) {
    return a.max_len > 0 && long(a.R) * a.k <= kBucketItems;
}

}  // namespace specv
