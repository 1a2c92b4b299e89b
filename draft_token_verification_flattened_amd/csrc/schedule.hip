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
// One workgroup of 1024 threads does everything: the candidate count is at most
// 16384, small enough for the keys to sit in the local data share, and the
// whole call is a few microseconds of latency-bound work.
//
// Bit-exactness: survival is float64, quantised to an integer key
// Q = floor(S * 2^32 + 0.5); prefix sums of keys are integers (order-free); the
// gain G(M) uses one fixed float64 formula with contraction disabled, so a host
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

__device__ double throughput(int bt, const int* tb, const double* tt, int n) {
    if (bt < tb[0]) return (tt[0] * double(bt)) / double(tb[0]);
    if (bt >= tb[n - 1]) return tt[n - 1];
    for (int j = 0; j + 1 < n; ++j) {
        if (tb[j] <= bt && bt < tb[j + 1]) {
            const double frac = double(bt - tb[j]) / double(tb[j + 1] - tb[j]);
            return tt[j] + (tt[j + 1] - tt[j]) * frac;
        }
    }
    return tt[n - 1];
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
};

// Verification length of request r for selection threshold `kstar` (a key;
// candidates with smaller keys are selected).
__device__ int request_length(const SchedArgs& a, int r, uint64_t kstar) {
    double S = 1.0;
    int L = 0;
    for (int i = 0; i < a.kk; ++i) {
        S = S * survival_step(a.z[long(r) * a.k + i], a.T[i]);
        if (make_key(quantise(S), i, r) < kstar) ++L;
    }
    return L;
}

// Write cu_rows, tags, n_rows (and len_out) for this thread's contiguous
// request range [r0, r1) given lengths computed by `len_of`.
template <typename F>
__device__ void flatten_block(const SchedArgs& a, int r0, int r1, F len_of, uint64_t* sh) {
    uint64_t local = 0;
    for (int r = r0; r < r1; ++r) local += uint64_t(len_of(r) + 1);
    uint64_t total;
    uint64_t off = block_exclusive_scan_u64(local, sh, total);
    for (int r = r0; r < r1; ++r) {
        const int L = len_of(r);
        a.cu_rows[r] = int32_t(off);
        if (a.len_out) a.len_out[r] = L;
        for (int j = 0; j <= L; ++j) {
            a.tags[2 * (off + j)] = r;
            a.tags[2 * (off + j) + 1] = j;
        }
        off += uint64_t(L + 1);
    }
    if (threadIdx.x == 0) {
        a.cu_rows[a.R] = int32_t(total);
        *a.n_rows = int32_t(total);
    }
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(SchedArgs a) {
    __shared__ uint64_t keys[SPECV_MAX_SCHED_ITEMS];
    __shared__ uint64_t sh[64];
    __shared__ int tb[kMaxTbl];
    __shared__ double tt[kMaxTbl];
    __shared__ double red_g[kSchedThreads / 64];
    __shared__ int red_m[kSchedThreads / 64];
    __shared__ uint64_t kstar_sh;

    const int tid = threadIdx.x, nt = blockDim.x;
    const int per = (a.R + nt - 1) / nt;
    const int r0 = min(a.R, tid * per), r1 = min(a.R, r0 + per);

    if (a.max_len < 0 || a.kk == 0) {
        // verify all k (max_len < 0) or nothing (max_len == 0)
        const int Lfix = a.max_len < 0 ? a.k : 0;
        if (a.survival) {
            for (int r = r0; r < r1; ++r) {
                double S = 1.0;
                for (int i = 0; i < a.k; ++i) {
                    S = S * survival_step(a.z[long(r) * a.k + i], a.T[i]);
                    a.survival[long(r) * a.k + i] = S;
                }
            }
        }
        flatten_block(a, r0, r1, [&](int) { return Lfix; }, sh);
        return;
    }

    for (int i = tid; i < a.n_tbl; i += nt) { tb[i] = a.tbl_b[i]; tt[i] = a.tbl_t[i]; }

    // 1. calibrated survival, quantised keys
    const int n = a.R * a.kk;
    int n2 = 1;
    while (n2 < n) n2 <<= 1;
    for (int r = r0; r < r1; ++r) {
        double S = 1.0;
        for (int i = 0; i < a.k; ++i) {
            S = S * survival_step(a.z[long(r) * a.k + i], a.T[i]);
            if (a.survival) a.survival[long(r) * a.k + i] = S;
            if (i < a.kk) keys[r * a.kk + i] = make_key(quantise(S), i, r);
        }
    }
    for (int i = n + tid; i < n2; i += nt) keys[i] = ~0ull;
    __syncthreads();

    // 2. bitonic sort, ascending
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int idx = tid; idx < (n2 >> 1); idx += nt) {
                const int pos = 2 * idx - (idx & (stride - 1));
                const int par = pos + stride;
                const bool asc = (pos & size) == 0;
                const uint64_t x = keys[pos], y = keys[par];
                if ((x > y) == asc) { keys[pos] = y; keys[par] = x; }
            }
            __syncthreads();
        }
    }

    // 3. prefix sums of keys in sorted order; gain of every prefix length M
    const uint64_t R32 = uint64_t(a.R) << 32;
    const int seg = (n + nt - 1) / nt;
    const int m0 = min(n, tid * seg), m1 = min(n, m0 + seg);
    uint64_t local = 0;
    for (int m = m0; m < m1; ++m) local += key_q(keys[m]);
    uint64_t total;
    uint64_t P = block_exclusive_scan_u64(local, sh, total);
    double best = -1.0;
    int bestM = INT_MAX;
    if (tid == 0) {
        const int bt = a.R;
        best = (double(R32) * throughput(bt, tb, tt, a.n_tbl)) / double(bt);
        bestM = 0;
    }
    for (int m = m0; m < m1; ++m) {
        P += key_q(keys[m]);
        const int M = m + 1, bt = a.R + M;
        const double G = (double(R32 + P) * throughput(bt, tb, tt, a.n_tbl)) / double(bt);
        if (G > best) { best = G; bestM = M; }     // increasing M: strict keeps the first
    }
    // block arg-max: larger G, then smaller M
    const int lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const double g2 = __shfl_xor(best, o, 64);
        const int m2 = __shfl_xor(bestM, o, 64);
        if (g2 > best || (g2 == best && m2 < bestM)) { best = g2; bestM = m2; }
    }
    if (lane == 0) { red_g[w] = best; red_m[w] = bestM; }
    __syncthreads();
    if (tid == 0) {
        double bg = red_g[0];
        int bm = red_m[0];
        for (int q = 1; q < (nt >> 6); ++q)
            if (red_g[q] > bg || (red_g[q] == bg && red_m[q] < bm)) { bg = red_g[q]; bm = red_m[q]; }
        kstar_sh = bm < n ? keys[bm] : ~0ull;
    }
    __syncthreads();
    const uint64_t kstar = kstar_sh;

    // 4. lengths and flatten
    flatten_block(a, r0, r1, [&](int r) { return request_length(a, r, kstar); }, sh);
}

// spec_flatten, part 1: offsets (single workgroup, contiguous request ranges).
__global__ __launch_bounds__(kSchedThreads) void flatten_offsets_kernel(SchedArgs a) {
    __shared__ uint64_t sh[64];
    const int tid = threadIdx.x, nt = blockDim.x;
    const int per = (a.R + nt - 1) / nt;
    const int r0 = min(a.R, tid * per), r1 = min(a.R, r0 + per);
    uint64_t local = 0;
    for (int r = r0; r < r1; ++r) local += uint64_t(min(max(a.len_in[r], 0), a.k) + 1);
    uint64_t total;
    uint64_t off = block_exclusive_scan_u64(local, sh, total);
    for (int r = r0; r < r1; ++r) {
        a.cu_rows[r] = int32_t(off);
        off += uint64_t(min(max(a.len_in[r], 0), a.k) + 1);
    }
    if (tid == 0) {
        a.cu_rows[a.R] = int32_t(total);
        *a.n_rows = int32_t(total);
    }
}

// spec_flatten, part 2: tags, one thread per request.
__global__ __launch_bounds__(256) void flatten_tags_kernel(SchedArgs a) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= a.R) return;
    const int L = min(max(a.len_in[r], 0), a.k);
    const int off = a.cu_rows[r];
    for (int j = 0; j <= L; ++j) {
        a.tags[2 * (off + j)] = r;
        a.tags[2 * (off + j) + 1] = j;
    }
}

}  // namespace specv

extern "C" int spec_schedule(int R, int k, const float* conf_logit, const float* pos_temp,
                             const int32_t* tbl_tokens, const double* tbl_thr, int n_tbl, int max_len,
                             int32_t* len_out, int32_t* tags_out, int32_t* cu_rows_out,
                             int32_t* n_rows_out, double* survival_out, specv_stream stream) {
    using namespace specv;
    clear_error();
    if (R < 1 || k < 1 || k > SPECV_MAX_K || long(R) * k > SPECV_MAX_SCHED_ITEMS)
        return fail(SPECV_EINVAL, "spec_schedule: need R >= 1, 1 <= k <= %d, R*k <= %d (got R=%d k=%d)",
                    SPECV_MAX_K, SPECV_MAX_SCHED_ITEMS, R, k);
    if (max_len < -1 || max_len > k)
        return fail(SPECV_EINVAL, "spec_schedule: max_len must be -1 or in [0, k] (got %d)", max_len);
    if (max_len != -1 && max_len != 0 && (n_tbl < 1 || n_tbl > kMaxTbl))
        return fail(SPECV_EINVAL, "spec_schedule: n_tbl must be in [1, %d] (got %d)", kMaxTbl, n_tbl);
    if (!conf_logit || !pos_temp || !len_out || !tags_out || !cu_rows_out || !n_rows_out)
        return fail(SPECV_EINVAL, "spec_schedule: NULL required pointer");
    if (max_len > 0 && (!tbl_tokens || !tbl_thr))
        return fail(SPECV_EINVAL, "spec_schedule: NULL throughput table");
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
    hipStream_t s = static_cast<hipStream_t>(stream);
    SPECV_LAUNCH("schedule", s, schedule_kernel<<<1, kSchedThreads, 0, s>>>(a));
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
    SPECV_LAUNCH("flatten_offsets", s, flatten_offsets_kernel<<<1, kSchedThreads, 0, s>>>(a));
    SPECV_LAUNCH("flatten_tags", s, flatten_tags_kernel<<<(R + 255) / 256, 256, 0, s>>>(a));
    return SPECV_OK;
}
