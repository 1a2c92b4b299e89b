// spec_schedule / spec_flatten: calibrated survival, the hardware-aware prefix
// scheduler, and the tagged flattening of the chosen rows.
//
// Pages: a confidence head scores each draft token's survival given its prefix
// and a post-hoc temporal temperature scaling corrects its over-confidence; the
// scheduler then sets each request's verification length from the engine's
// measured throughput ("刚融完500亿创始人亲自下场写代码…", section
// "2. 置信度调度验证"); the score is conditional on all earlier tokens being
// accepted, and the length depends on load, confidence and the throughput-vs-
// batch curve ("DSpark 的 661% 提速…", section 3.2); drafts of all requests are
// ranked by confidence and added batch by batch while the extra step time per
// extra correct token pays ("DeepSeek服务器不再卡顿！…", section "DSpark的神奇之处");
// the choice is a global throughput maximisation (aibuzzwire.news article,
// section "置信度计划、负载感知验证").
//
// The scheduler needs, for every prefix length M of the candidates sorted by
// key, the key sum P(M), and then the M with the largest gain. It does not sort:
// candidate x sits at sorted position rank(x) = #{keys < x}, so the prefix that
// ends at x has M = rank(x) + 1 and P(M) = (sum of Q over keys < x) + Q(x).
// schedule_rank spreads those all-pairs counts over up to 256 workgroups (each
// recomputes all keys into its LDS, then counts for its slice of keys), each
// workgroup posts its best (G, M, key), and the last one to finish picks the
// overall best and flattens. On one compute unit a sort of a few thousand
// 64-bit keys costs ~10-20 us; the spread count costs ~1-2 us.
//
// Bit-exactness: survival is float64, quantised to an integer key
// Q = floor(S * 2^32 + 0.5); sums of keys are integers (order-free); the gain
// G(M) uses one fixed float64 formula with contraction disabled, so a host
// reference computing the same formula gets the same bits.
#pragma clang fp contract(off)

#include <climits>

#include "common.h"
#include "host.h"

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
    return uint64_t(floor(S * 4294967296.0 + 0.5));
}

// Table lookup: linear interpolation on the segment [B_j, B_j+1) holding bt
// (found by binary search; the batch tokens are strictly increasing).
__device__ double throughput(int bt, const int* tb, const double* tt, int n) {
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

// Block-wide exclusive scan of one 64-bit value per thread; returns the total too.
__device__ uint64_t block_exclusive_scan_u64(uint64_t v, uint64_t* sh, uint64_t& total) {
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

// Workspace of spec_schedule: a finish counter (zero between calls) and one
// best-prefix record per workgroup.
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
__device__ void flatten_block(const SchedArgs& a, int r0, int r1, F len_of, int* sh) {
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

// Keys of all candidates into LDS, request-major (keys[r * kk + i]); the
// survival of every (r, i < k) to `survival` when it is not NULL.
__device__ void compute_keys(const SchedArgs& a, uint64_t* keys, bool write_survival) {
    for (int r = threadIdx.x; r < a.R; r += blockDim.x) {
        double S = 1.0;
        for (int i = 0; i < a.k; ++i) {
            if (i >= a.kk && !write_survival) break;
            S = S * survival_step(a.z[long(r) * a.k + i], a.T[i]);
            if (write_survival) a.survival[long(r) * a.k + i] = S;
            if (i < a.kk) keys[r * a.kk + i] = make_key(quantise(S), i, r);
        }
    }
}

// All lengths fixed (max_len < 0: all k; max_len == 0: none): survival and flatten.
__global__ __launch_bounds__(kSchedThreads) void schedule_fixed(SchedArgs a) {
    __shared__ int sh[64];
    const int tid = threadIdx.x, nt = blockDim.x;
    if (a.survival) {
        for (int r = tid; r < a.R; r += nt) {
            double S = 1.0;
            for (int i = 0; i < a.k; ++i) {
                S = S * survival_step(a.z[long(r) * a.k + i], a.T[i]);
                a.survival[long(r) * a.k + i] = S;
            }
        }
    }
    const int Lfix = a.max_len < 0 ? a.k : 0;
    const int per = (a.R + nt - 1) / nt;
    const int r0 = min(a.R, tid * per), r1 = min(a.R, r0 + per);
    flatten_block(a, r0, r1, [&](int) { return Lfix; }, sh);
}

__device__ __forceinline__ void put64(unsigned long long* p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long get64(unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup's best prefix, or the winner of a merge: larger G first, then
// smaller M. G >= 0, so its bits order like its value as signed integers; an
// empty candidate carries G bits LLONG_MIN.
struct Best {
    long long g;
    int m;
    uint64_t key;
};

__device__ __forceinline__ void best_merge(Best& x, long long g, int m, uint64_t key) {
    if (g > x.g || (g == x.g && m < x.m)) { x.g = g; x.m = m; x.key = key; }
}

__device__ __forceinline__ void wave_best(Best& b) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const long long g2 = __shfl_xor(b.g, o, 64);
        const int m2 = __shfl_xor(b.m, o, 64);
        const uint64_t k2 = __shfl_xor(b.key, o, 64);
        best_merge(b, g2, m2, k2);
    }
}

__global__ __launch_bounds__(kSchedThreads) void schedule_rank(SchedArgs a, int kw) {
    extern __shared__ __align__(16) uint64_t keys[];          // [R * kk]
    __shared__ int tb[kMaxTbl];
    __shared__ double tt[kMaxTbl];
    __shared__ unsigned long long cnt_sh[64];                  // per local key (kw <= 64)
    __shared__ unsigned long long sum_sh[64];
    __shared__ uint64_t sh[64];
    __shared__ int ish[64];
    __shared__ int last_sh;
    const int tid = threadIdx.x, nt = blockDim.x;
    const int n = a.R * a.kk;

    // 1. table and all keys
    for (int i = tid; i < a.n_tbl; i += nt) { tb[i] = a.tbl_b[i]; tt[i] = a.tbl_t[i]; }
    if (tid < kw) { cnt_sh[tid] = 0ull; sum_sh[tid] = 0ull; }
    compute_keys(a, keys, blockIdx.x == 0 && a.survival != nullptr);
    __syncthreads();

    // 2. rank and prefix sum of this workgroup's keys [j0, j0 + kw): thread
    //    (key a_, segment b_) counts over its share of all n keys
    const int j0 = blockIdx.x * kw;
    const int a_ = tid % kw, b_ = tid / kw, nseg = nt / kw;
    const int j = j0 + a_;
    if (j < n) {
        const uint64_t x = keys[j];
        const int s0 = int(long(n) * b_ / nseg), s1 = int(long(n) * (b_ + 1) / nseg);
        unsigned cnt = 0;
        unsigned long long sum = 0;
        for (int y = s0; y < s1; ++y) {
            const uint64_t ky = keys[y];
            if (ky < x) { ++cnt; sum += key_q(ky); }
        }
        atomicAdd(&cnt_sh[a_], (unsigned long long)cnt);
        atomicAdd(&sum_sh[a_], sum);
    }
    __syncthreads();

    // 3. this workgroup's best prefix; post it; the last workgroup continues
    const uint64_t R32 = uint64_t(a.R) << 32;
    if (tid < 64) {
        Best b{LLONG_MIN, INT_MAX, 0ull};
        for (int q = tid; q < kw && j0 + q < n; q += 64) {
            const uint64_t x = keys[j0 + q];
            const int M = int(cnt_sh[q]) + 1, bt = a.R + M;
            const uint64_t P = sum_sh[q] + key_q(x);
            const double G = (double(R32 + P) * throughput(bt, tb, tt, a.n_tbl)) / double(bt);
            best_merge(b, __double_as_longlong(G), M, x);
        }
        if (blockIdx.x == 0 && tid == 0) {                   // the empty prefix, M = 0
            const double G0 = (double(R32) * throughput(a.R, tb, tt, a.n_tbl)) / double(a.R);
            best_merge(b, __double_as_longlong(G0), 0, 0ull);
        }
        wave_best(b);
        if (tid == 0) {
            SchedWs* w = a.ws;
            put64(reinterpret_cast<unsigned long long*>(&w->best[blockIdx.x].g), (unsigned long long)b.g);
            __hip_atomic_store(&w->best[blockIdx.x].m, b.m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            put64(reinterpret_cast<unsigned long long*>(&w->best[blockIdx.x].key), b.key);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_waitcnt(0);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            last_sh = __hip_atomic_fetch_add(&w->done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                      int(gridDim.x) - 1;
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
        }
    }
    __syncthreads();
    if (!last_sh) return;

    // 4. overall best: the selected candidates are the keys <= its key (none if M = 0)
    if (tid < 64) {
        SchedWs* w = a.ws;
        Best b{LLONG_MIN, INT_MAX, 0ull};
        for (int q = tid; q < int(gridDim.x); q += 64)
            best_merge(b, (long long)get64(reinterpret_cast<unsigned long long*>(&w->best[q].g)),
                       __hip_atomic_load(&w->best[q].m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                       get64(reinterpret_cast<unsigned long long*>(&w->best[q].key)));
        wave_best(b);
        if (tid == 0) {
            sh[62] = b.key;
            sh[63] = uint64_t(b.m);
            __hip_atomic_store(&w->done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    const uint64_t kt = sh[62];
    const bool any = sh[63] > 0;
    __syncthreads();
    // a request's keys increase with the position, so its selection is a prefix:
    // its length is the number of its keys <= kt
    auto len_of = [&](int r) {
        int L = 0;
        if (any)
            for (int i = 0; i < a.kk; ++i) L += keys[r * a.kk + i] <= kt ? 1 : 0;
        return L;
    };
    const int per = (a.R + nt - 1) / nt;
    const int r0 = min(a.R, tid * per), r1 = min(a.R, r0 + per);
    flatten_block(a, r0, r1, len_of, ish);
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

// Bucket of a key: 2^32 - Q in steps of 2^20 (ascending bucket = descending Q).
__device__ __forceinline__ int bucket_of(uint64_t key) {
    const uint64_t d = (1ull << 32) - key_q(key);
    return int(min(d >> 20, uint64_t(kBuckets - 1)));
}

__global__ __launch_bounds__(kSchedThreads) void schedule_bucket(SchedArgs a) {
    extern __shared__ __align__(16) uint64_t lds[];   // keys [R*k] | grouped [n] | sorted [n] | cnt, off [kBuckets]
    __shared__ int tb[kMaxTbl];
    __shared__ double tt[kMaxTbl];
    __shared__ double wg_sh[kSchedThreads / 64];
    __shared__ int wm_sh[kSchedThreads / 64];
    __shared__ int sh[64], sh2[64];
    __shared__ uint64_t kt_sh;
    __shared__ int any_sh;
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6, nwav = nt >> 6;
    const int R = a.R, k = a.k, kk = a.kk, n = R * kk, Rk = R * k;
    const bool surv = a.survival != nullptr;
    const int kc = surv ? k : kk;
    uint64_t* keys = lds;
    uint64_t* grp = keys + Rk;
    uint64_t* srt = grp + n;
    int* cnt = reinterpret_cast<int*>(srt + n);
    int* off = cnt + kBuckets;
    double* sg = reinterpret_cast<double*>(keys);

    // 1. table, empty histogram, one calibrated sigmoid per (request, position)
    for (int i = tid; i < a.n_tbl; i += nt) { tb[i] = a.tbl_b[i]; tt[i] = a.tbl_t[i]; }
    for (int b = tid; b < kBuckets; b += nt) cnt[b] = 0;
    for (int e = tid; e < Rk; e += nt) {
        const int i = e % k;
        if (i < kc) sg[e] = survival_step(a.z[e], a.T[i]);
    }
    __syncthreads();

    // this thread's prefix lengths M = p + 1, p in [p0, p1): their throughput
    // does not depend on the keys
    constexpr int kPosPer = kBucketItems / kSchedThreads;
    const int per = (n + nt - 1) / nt;
    const int p0 = min(n, tid * per), p1 = min(n, p0 + per);
    double thr[kPosPer];
#pragma unroll
    for (int q = 0; q < kPosPer; ++q) thr[q] = p0 + q < p1 ? throughput(R + p0 + q + 1, tb, tt, a.n_tbl) : 0.0;

    // 2. survival (running products in position order) and keys, in place;
    //    positions >= kk get a key above every real one
    for (int r = tid; r < R; r += nt) {
        double S = 1.0;
        for (int i = 0; i < k; ++i) {
            const int e = r * k + i;
            if (i < kc) {
                S = S * sg[e];
                if (surv) a.survival[long(r) * k + i] = S;
            }
            uint64_t key = ~0ull;
            if (i < kk) {
                key = make_key(quantise(S), i, r);
                atomicAdd(&cnt[bucket_of(key)], 1);
            }
            keys[e] = key;
        }
    }
    __syncthreads();

    // 3. bucket offsets (exclusive scan), then every key into its bucket
    {
        constexpr int kPer = kBuckets / kSchedThreads;
        int loc[kPer];
        int sum = 0;
#pragma unroll
        for (int q = 0; q < kPer; ++q) { loc[q] = cnt[tid * kPer + q]; sum += loc[q]; }
        int total;
        int base = block_exclusive_scan_i32(sum, sh, total);
#pragma unroll
        for (int q = 0; q < kPer; ++q) { off[tid * kPer + q] = base; base += loc[q]; }
    }
    __syncthreads();
    for (int e = tid; e < Rk; e += nt) {
        const uint64_t x = keys[e];
        if (x != ~0ull) grp[atomicAdd(&off[bucket_of(x)], 1)] = x;
    }
    __syncthreads();

    // 4. exact sorted position: bucket start + smaller keys of the same bucket
    for (int e = tid; e < Rk; e += nt) {
        const uint64_t x = keys[e];
        if (x == ~0ull) continue;
        const int b = bucket_of(x);
        const int end = off[b], beg = end - cnt[b];
        int rank = beg;
        for (int m = beg; m < end; ++m) rank += grp[m] < x ? 1 : 0;
        srt[rank] = x;
    }
    __syncthreads();

    // 5. P(M) for every prefix length (contiguous positions per thread), G(M),
    //    and the best prefix: largest G, then smallest M
    //    Q <= 2^32 is scanned as two exact 32-bit sums of its 16-bit halves.
    const uint64_t R32 = uint64_t(R) << 32;
    int lo = 0, hi = 0;
    for (int p = p0; p < p1; ++p) {
        const uint64_t q = key_q(srt[p]);
        lo += int(q & 0xffffu);
        hi += int(q >> 16);
    }
    int tlo, thi;
    const int elo = block_exclusive_scan_i32(lo, sh, tlo);
    const int ehi = block_exclusive_scan_i32(hi, sh2, thi);
    uint64_t P = (uint64_t(uint32_t(ehi)) << 16) + uint64_t(uint32_t(elo));
    double g = -1.0;                                          // below every gain
    int m = INT_MAX;
#pragma unroll
    for (int q = 0; q < kPosPer; ++q) {
        if (p0 + q < p1) {
            P += key_q(srt[p0 + q]);
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
            any_sh = mw > 0;
            kt_sh = mw > 0 ? srt[mw - 1] : 0ull;
        }
    }
    __syncthreads();

    // 6. lengths (a request's keys increase with the position) and the batch
    const uint64_t kt = kt_sh;
    const bool any = any_sh != 0;
    auto len_of = [&](int r) {
        int L = 0;
        if (any)
            for (int i = 0; i < kk; ++i) L += keys[r * k + i] <= kt ? 1 : 0;
        return L;
    };
    const int rper = (R + nt - 1) / nt;
    const int r0 = min(R, tid * rper), r1 = min(R, r0 + rper);
    flatten_block(a, r0, r1, len_of, sh);
}

// spec_flatten, part 1: offsets (single workgroup, contiguous request ranges).
__global__ __launch_bounds__(kSchedThreads) void flatten_offsets_kernel(SchedArgs a) {
    __shared__ uint64_t sh[64];
    const int tid = threadIdx.x, nt = blockDim.x;
    const int per = (a.R + nt - 1) / nt;
    const int r0 = min(a.R, tid * per), r1 = min(a.R, r0 + per);
    uint64_t local = 0;
    for (int r = r0; r < r1; ++r) local += uint64_t(min(max(a.len_in[r], 0), a.k));
    uint64_t total;
    uint64_t off = block_exclusive_scan_u64(local, sh, total);
    for (int r = r0; r < r1; ++r) {
        a.cu_rows[r] = int32_t(off);
        off += uint64_t(min(max(a.len_in[r], 0), a.k));
    }
    if (tid == 0) {
        a.cu_rows[a.R] = int32_t(total);
        *a.n_rows = int32_t(total) + a.R;
    }
}

// spec_flatten, part 2: tags, one thread per request.
__global__ __launch_bounds__(256) void flatten_tags_kernel(SchedArgs a) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= a.R) return;
    const int L = min(max(a.len_in[r], 0), a.k);
    const int off = a.cu_rows[r];
    const int N = a.cu_rows[a.R];
    for (int j = 0; j < L; ++j) {
        a.tags[2 * (off + j)] = r;
        a.tags[2 * (off + j) + 1] = j;
    }
    a.tags[2 * (N + r)] = r;
    a.tags[2 * (N + r) + 1] = L;
}

}  // namespace specv

extern "C" size_t spec_schedule_workspace_bytes(int R, int k) {
    if (R < 1 || k < 1 || k > SPECV_MAX_K || long(R) * k > SPECV_MAX_SCHED_ITEMS) return 0;
    return sizeof(specv::SchedWs);
}

extern "C" int spec_schedule(int R, int k, const float* conf_logit, const float* pos_temp,
                             const int32_t* tbl_tokens, const double* tbl_thr, int n_tbl, int max_len,
                             int32_t* len_out, int32_t* tags_out, int32_t* cu_rows_out,
                             int32_t* n_rows_out, double* survival_out, void* ws, size_t ws_bytes,
                             specv_stream stream) {
    using namespace specv;
    clear_error();
    if (R < 1 || k < 1 || k > SPECV_MAX_K || long(R) * k > SPECV_MAX_SCHED_ITEMS)
        return fail(SPECV_EINVAL, "spec_schedule: need R >= 1, 1 <= k <= %d, R*k <= %d (got R=%d k=%d)",
                    SPECV_MAX_K, SPECV_MAX_SCHED_ITEMS, R, k);
    if (max_len < -1 || max_len > k)
        return fail(SPECV_EINVAL, "spec_schedule: max_len must be -1 or in [0, k] (got %d)", max_len);
    if (max_len != -1 && max_len != 0 && (n_tbl < 1 || n_tbl > kMaxTbl))
        return fail(SPECV_EINVAL, "spec_schedule: n_tbl must be in [1, %d] (got %d)", kMaxTbl, n_tbl);
    if (!conf_logit || !pos_temp || !len_out || !tags_out || !cu_rows_out || !n_rows_out || !ws)
        return fail(SPECV_EINVAL, "spec_schedule: NULL required pointer");
    if (max_len > 0 && (!tbl_tokens || !tbl_thr))
        return fail(SPECV_EINVAL, "spec_schedule: NULL throughput table");
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return fail(SPECV_EINVAL, "spec_schedule: workspace must be 256-byte aligned");
    if (ws_bytes < sizeof(SchedWs))
        return fail(SPECV_EINVAL, "spec_schedule: workspace of %zu bytes, need %zu", ws_bytes, sizeof(SchedWs));
    SchedArgs a;
    a.R = R; a.k = k;
    a.max_len = max_len;
    a.kk = max_len < 0 ? k : max_len;
    a.n_tbl = n_tbl;
    a.z = conf_logit; a.T = pos_temp;
    a.tbl_b = tbl_tokens; a.tbl_t = tbl_thr;
    a.len_in = nullptr;
    a.len_out = len_out; a.tags = tags_out; a.cu_rows = cu_rows_out; a.n_rows = n_rows_out;
    a.survival = survival_out;
    a.ws = static_cast<SchedWs*>(ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (max_len < 0 || max_len == 0) {
        SPECV_LAUNCH("schedule", schedule_fixed, 1, kSchedThreads, 0, s, a);
        return SPECV_OK;
    }
    if (long(R) * k <= kBucketItems) {
        const size_t lds = size_t(R) * k * sizeof(uint64_t) + 2 * size_t(R) * a.kk * sizeof(uint64_t) +
                           2 * size_t(kBuckets) * sizeof(int);
        if (lds > 65536 &&
            hipFuncSetAttribute(reinterpret_cast<const void*>(schedule_bucket),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
            return fail(SPECV_EDEVICE, "spec_schedule: cannot reserve %zu bytes of LDS", lds);
        SPECV_LAUNCH("schedule", schedule_bucket, 1, kSchedThreads, lds, s, a);
        return SPECV_OK;
    }
    // keys per workgroup: a power of two >= 16, enough for at most 256 workgroups
    const int n = R * a.kk;
    int kw = 16;
    while (long(kw) * kMaxSchedGroups < n) kw <<= 1;
    const int groups = (n + kw - 1) / kw;
    const size_t lds = size_t(n) * sizeof(uint64_t);
    if (lds > 65536 &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(schedule_rank),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
        return fail(SPECV_EDEVICE, "spec_schedule: cannot reserve %zu bytes of LDS", lds);
    SPECV_LAUNCH("schedule", schedule_rank, groups, kSchedThreads, lds, s, a, kw);
    return SPECV_OK;
}

extern "C" int spec_flatten(int R, int k, const int32_t* len_in, int32_t* tags_out,
                            int32_t* cu_rows_out, int32_t* n_rows_out, specv_stream stream) {
    using namespace specv;
    clear_error();
    if (R < 1 || k < 1 || k > SPECV_MAX_K || long(R) * (k + 1) > INT_MAX / 2)
        return fail(SPECV_EINVAL, "spec_flatten: need R >= 1, 1 <= k <= %d (got R=%d k=%d)", SPECV_MAX_K, R, k);
    if (!len_in || !tags_out || !cu_rows_out || !n_rows_out)
        return fail(SPECV_EINVAL, "spec_flatten: NULL required pointer");
    SchedArgs a{};
    a.R = R; a.k = k;
    a.len_in = len_in; a.tags = tags_out; a.cu_rows = cu_rows_out; a.n_rows = n_rows_out;
    hipStream_t s = static_cast<hipStream_t>(stream);
    SPECV_LAUNCH("flatten_offsets", flatten_offsets_kernel, 1, kSchedThreads, 0, s, a);
    SPECV_LAUNCH("flatten_tags", flatten_tags_kernel, (R + 255) / 256, 256, 0, s, a);
    return SPECV_OK;
}
