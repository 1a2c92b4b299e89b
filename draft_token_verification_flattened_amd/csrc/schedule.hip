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
// overall best and flattens. With R * k <= 4096, schedule_bucket does the
// whole schedule in one workgroup instead (schedule_dev.h), without a handoff
// between workgroups. On one compute unit a comparison sort of a few thousand
// 64-bit keys costs ~10-20 us.
//
// Bit-exactness: see schedule_dev.h.
#pragma clang fp contract(off)

#include <climits>

#include "common.h"
#include "host.h"
#include "schedule_dev.h"

namespace specv {

__global__ __launch_bounds__(kSchedThreads) void schedule_bucket(SchedArgs a) {
    extern __shared__ __align__(16) uint64_t lds[];
    schedule_bucket_body(a, lds);
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

// Clears schedule_rank's arrival counter; launched ahead of it on the same
// stream, so the workspace needs no initialisation and a counter left behind by
// an earlier call (or any other contents) cannot hide the last arrival.
__global__ __launch_bounds__(64) void schedule_ws_clear(SchedWs* ws) {
    if (threadIdx.x == 0) ws->done = 0;
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
            // release: this record is visible before the arrival; acquire: the
            // last to arrive sees every record
            last_sh = __hip_atomic_fetch_add(&w->done, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
                      int(gridDim.x) - 1;
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

namespace specv {

int schedule_prepare(int R, int k, const float* conf_logit, const float* pos_temp, const int32_t* tbl_tokens,
                     const double* tbl_thr, int n_tbl, int max_len, int32_t* len_out, int32_t* tags_out,
                     int32_t* cu_rows_out, int32_t* n_rows_out, double* survival_out, void* ws, size_t ws_bytes,
                     const char* who, SchedArgs& a) {
    if (R < 1 || k < 1 || k > SPECV_MAX_K || long(R) * k > SPECV_MAX_SCHED_ITEMS)
        return fail(SPECV_EINVAL, "%s: need R >= 1, 1 <= k <= %d, R*k <= %d (got R=%d k=%d)", who, SPECV_MAX_K,
                    SPECV_MAX_SCHED_ITEMS, R, k);
    if (max_len < -1 || max_len > k)
        return fail(SPECV_EINVAL, "%s: max_len must be -1 or in [0, k] (got %d)", who, max_len);
    if (max_len != -1 && max_len != 0 && (n_tbl < 1 || n_tbl > kMaxTbl))
        return fail(SPECV_EINVAL, "%s: n_tbl must be in [1, %d] (got %d)", who, kMaxTbl, n_tbl);
    if (!conf_logit || !pos_temp || !len_out || !tags_out || !cu_rows_out || !n_rows_out || !ws)
        return fail(SPECV_EINVAL, "%s: NULL required pointer", who);
    if (max_len > 0 && (!tbl_tokens || !tbl_thr))
        return fail(SPECV_EINVAL, "%s: NULL throughput table", who);
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return fail(SPECV_EINVAL, "%s: workspace must be 256-byte aligned", who);
    if (ws_bytes < sizeof(SchedWs))
        return fail(SPECV_EINVAL, "%s: workspace of %zu bytes, need %zu", who, ws_bytes, sizeof(SchedWs));
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
    return SPECV_OK;
}

int schedule_launch(const SchedArgs& a, hipStream_t s) {
    const int R = a.R, k = a.k;
    if (a.max_len < 0 || a.max_len == 0) {
        SPECV_LAUNCH("schedule", schedule_fixed, 1, kSchedThreads, 0, s, a);
        return SPECV_OK;
    }
    if (schedule_is_bucket(a)) {
        const size_t lds = schedule_bucket_lds(R, k, a.kk);
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
    SPECV_LAUNCH("sched_ws_clear", schedule_ws_clear, 1, 64, 0, s, a.ws);
    SPECV_LAUNCH("schedule", schedule_rank, groups, kSchedThreads, lds, s, a, kw);
    return SPECV_OK;
}

}  // namespace specv

extern "C" int spec_schedule(int R, int k, const float* conf_logit, const float* pos_temp,
                             const int32_t* tbl_tokens, const double* tbl_thr, int n_tbl, int max_len,
                             int32_t* len_out, int32_t* tags_out, int32_t* cu_rows_out,
                             int32_t* n_rows_out, double* survival_out, void* ws, size_t ws_bytes,
                             specv_stream stream) {
    using namespace specv;
    clear_error();
    SchedArgs a;
    if (int e = schedule_prepare(R, k, conf_logit, pos_temp, tbl_tokens, tbl_thr, n_tbl, max_len, len_out, tags_out,
                                 cu_rows_out, n_rows_out, survival_out, ws, ws_bytes, "spec_schedule", a))
        return e;
    return schedule_launch(a, static_cast<hipStream_t>(stream));
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
