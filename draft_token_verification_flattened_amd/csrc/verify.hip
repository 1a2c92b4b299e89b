// spec_verify: the exact acceptance rule over a flattened, tagged varlen batch.
//
// Pages: every selected draft token becomes one element of a single batch and a
// tag tensor (request, position) carries the in-sequence dependency ("刚融完500亿
// 创始人亲自下场写代码…", engineering table, row "内核利用率暴跌"); verified tokens
// are kept and the first divergence is resampled ("DSpark 的 661% 提速，是真突破
// 还是数字游戏？", section 一); rejection sampling keeps the target's distribution
// ("DeepSeek服务器不再卡顿！…", section "DSpark的神奇之处").
//
// Four kernels on one stream:
//   verify_partials   one wavefront per (row slot, vocabulary chunk): streams a
//                     2048-logit chunk of a target (or draft) row with 16-byte
//                     loads and writes a partial: (max, index) in greedy mode,
//                     the base-2 online softmax state (m, s) in sampling mode.
//                     All HBM traffic of the step is here.
//   verify_finalize   one wavefront per request: merges chunk partials per row,
//                     decides every verified row, finds the first rejection
//                     a_r, writes accepted lengths and tokens (greedy: final).
//   resample_mass     sampling only; one wavefront per (request, chunk) of the
//                     rejected row: chunk mass of max(0, p - q).
//   resample_pick     sampling only; one wavefront per request: chunk prefix
//                     sums, then an in-chunk scan for the inverse-CDF draw.
#include <climits>

#include "common.h"
#include "host.h"

namespace specv {

constexpr int kChunk = 2048;        // logits per (row, chunk) work item
constexpr int kWavesPerBlock = 4;   // 256-thread workgroups

struct VerifyArgs {
    int R, k, V, C;                 // C = chunks per row
    int Bmax;                       // R * (k + 1)
    const void* target;
    const void* draft;
    const int32_t* tokens;
    const int32_t* tags;
    const int32_t* cu_rows;
    const int32_t* n_rows;
    const float* uniforms;
    float c;                        // log2(e) / tau
    int32_t* acc_len;
    int32_t* out_tokens;
    float* diag;
    WsHeader* hdr;
    float2* part;                   // [slots * C]; slot = t (greedy) or 2t + tensor
    float4* rs_stat;                // [R] {m_p, s_p, m_q, s_q} of the resample row
    int4* rs_row;                   // [R] {row t, a_r, kind (0 residual, 1 bonus), 0}
    float* mass;                    // [R * C]
};

struct Layout {
    size_t part, rs_stat, rs_row, mass, total;
};

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static Layout ws_layout(int mode, int R, int k, int V) {
    Layout l;
    size_t C = (size_t(V) + kChunk - 1) / kChunk;
    size_t slots = size_t(mode == SPECV_SAMPLE ? 2 : 1) * size_t(R) * size_t(k + 1);
    size_t off = align256(sizeof(WsHeader));
    l.part = off;
    off = align256(off + slots * C * sizeof(float2));
    l.rs_stat = off;
    off = align256(off + size_t(R) * sizeof(float4));
    l.rs_row = off;
    off = align256(off + size_t(R) * sizeof(int4));
    l.mass = off;
    off = align256(off + size_t(R) * C * sizeof(float));
    l.total = off;
    return l;
}

// ---------------------------------------------------------------------------
// pass 1: per (row slot, chunk) partials
// ---------------------------------------------------------------------------

template <int DT, int MODE, bool VEC>
__global__ __launch_bounds__(256) void verify_partials(VerifyArgs a) {
    using LT = Logit<DT>;
    using T = typename LT::T;
    constexpr int kV = LT::kVec;
    constexpr int kU = kChunk / (kWave * kV);      // 16-byte loads per lane

    const int lane = threadIdx.x & (kWave - 1);
    const long item = long(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    if (blockIdx.x == 0 && threadIdx.x == 0) a.hdr->status = 0u;   // this kernel sets no bits
    const int chunk = int(item % a.C);
    const long slot = item / a.C;
    const int t = MODE == SPECV_SAMPLE ? int(slot >> 1) : int(slot);
    const int tensor = MODE == SPECV_SAMPLE ? int(slot & 1) : 0;
    if (t >= a.Bmax || t >= *a.n_rows) return;
    const int r = a.tags[2 * t], j = a.tags[2 * t + 1];
    if (r < 0 || r >= a.R || j < 0 || j > a.k) return;            // reported by finalize
    if (tensor == 1) {
        const int L = a.cu_rows[r + 1] - a.cu_rows[r] - 1;
        if (j >= L || j >= a.k) return;                            // bonus rows have no draft
    }
    const T* row = tensor == 0
        ? static_cast<const T*>(a.target) + (long(r) * (a.k + 1) + j) * long(a.V)
        : static_cast<const T*>(a.draft) + (long(r) * a.k + j) * long(a.V);
    const int beg = chunk * kChunk;
    const int end = min(a.V, beg + kChunk);

    float2 res;
    if (MODE == SPECV_GREEDY) {
        float bv = -INFINITY;
        int bi = INT_MAX;
        if (VEC) {
            const uint4* vrow = reinterpret_cast<const uint4*>(row);
            uint4 buf[kU];
            const int v0 = beg / kV, v1 = end / kV;
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                int v = v0 + u * kWave + lane;
                if (v < v1) buf[u] = vrow[v];
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                int v = v0 + u * kWave + lane;
                if (v < v1) {
                    float x[kV];
                    LT::unpack(buf[u], x);
#pragma unroll
                    for (int e = 0; e < kV; ++e)
                        if (bi == INT_MAX || x[e] > bv) { bv = x[e]; bi = v * kV + e; }
                }
            }
        } else {
            for (int e = beg + lane; e < end; e += kWave) {
                float x = LT::load1(row + e);
                if (bi == INT_MAX || x > bv) { bv = x; bi = e; }
            }
        }
        wave_argmax(bv, bi);
        res = make_float2(bv, __int_as_float(bi));
    } else {
        const float c = a.c;
        float m = -INFINITY, s = 0.f;
        if (VEC) {
            const uint4* vrow = reinterpret_cast<const uint4*>(row);
            uint4 buf[kU];
            const int v0 = beg / kV, v1 = end / kV;
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                int v = v0 + u * kWave + lane;
                if (v < v1) buf[u] = vrow[v];
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                int v = v0 + u * kWave + lane;
                if (v < v1) {
                    float x[kV];
                    LT::unpack(buf[u], x);
                    float vm = x[0];
#pragma unroll
                    for (int e = 1; e < kV; ++e) vm = fmaxf(vm, x[e]);
                    const float am = vm * c;
                    if (am > m) { s *= __builtin_amdgcn_exp2f(m - am); m = am; }
#pragma unroll
                    for (int e = 0; e < kV; ++e) s += __builtin_amdgcn_exp2f(fmaf(x[e], c, -m));
                }
            }
        } else {
            for (int e = beg + lane; e < end; e += kWave) {
                float x = LT::load1(row + e);
                const float am = x * c;
                if (am > m) { s *= __builtin_amdgcn_exp2f(m - am); m = am; }
                s += __builtin_amdgcn_exp2f(fmaf(x, c, -m));
            }
        }
        wave_lse(m, s);
        res = make_float2(m, s);
    }
    if (lane == 0) a.part[slot * a.C + chunk] = res;
}

// ---------------------------------------------------------------------------
// per-request decisions
// ---------------------------------------------------------------------------

template <int DT, int MODE>
__global__ __launch_bounds__(256) void verify_finalize(VerifyArgs a) {
    using LT = Logit<DT>;
    using T = typename LT::T;
    const int lane = threadIdx.x & (kWave - 1);
    const int r = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (r >= a.R) return;
    const int k = a.k;
    const int base = a.cu_rows[r];
    const int L = a.cu_rows[r + 1] - base - 1;
    int32_t* out = a.out_tokens + long(r) * (k + 1);

    bool bad = L < 0 || L > k || base < 0 || base + L >= a.Bmax;
    if (!bad && lane <= L) {
        const int t = base + lane;
        bad = a.tags[2 * t] != r || a.tags[2 * t + 1] != lane;
    }
    bad = __any(bad);
    if (bad) {
        if (lane == 0) {
            set_status(a.hdr, SPECV_STATUS_BAD_TAG);
            a.acc_len[r] = 0;
            if (MODE == SPECV_SAMPLE) a.rs_row[r] = make_int4(-1, 0, 2, 0);
        }
        if (lane <= k) out[lane] = -1;
        return;
    }

    int acc = L;              // first rejected position (L if none)
    int y = -1;               // greedy: token emitted at position acc
    float4 stat = make_float4(0.f, 0.f, 0.f, 0.f);
    int rs_t = base + L;

    for (int j = 0; j <= L; ++j) {
        const int t = base + j;
        const bool verified = j < L;
        int x = -1;
        bool xok = true;
        if (verified) {
            x = a.tokens[long(r) * k + j];
            xok = x >= 0 && x < a.V;
        }
        if (MODE == SPECV_GREEDY) {
            float bv = -INFINITY;
            int bi = INT_MAX;
            for (int ch = lane; ch < a.C; ch += kWave) {
                float2 p = a.part[long(t) * a.C + ch];
                argmax_merge(bv, bi, p.x, __float_as_int(p.y));
            }
            wave_argmax(bv, bi);
            bool keep = false;
            if (verified) {
                keep = xok && bi == x;
                if (!keep && acc == L) { acc = j; y = bi; }
            } else if (acc == L) {
                y = bi;
            }
            if (a.diag && lane == 0)
                reinterpret_cast<float4*>(a.diag)[t] =
                    make_float4(float(bi), bv, 0.f, verified ? (keep ? 1.f : 0.f) : -1.f);
        } else {
            float mp = -INFINITY, sp = 0.f, mq = -INFINITY, sq = 0.f;
            for (int ch = lane; ch < a.C; ch += kWave) {
                float2 p = a.part[long(2 * t) * a.C + ch];
                lse_merge(mp, sp, p.x, p.y);
                if (verified) {
                    float2 q = a.part[long(2 * t + 1) * a.C + ch];
                    lse_merge(mq, sq, q.x, q.y);
                }
            }
            wave_lse(mp, sp);
            if (verified) wave_lse(mq, sq);
            if (verified) {
                float px = 0.f, qx = 0.f, ratio = 0.f;
                bool keep = false;
                if (xok) {
                    const T* trow = static_cast<const T*>(a.target) + (long(r) * (k + 1) + j) * long(a.V);
                    const T* drow = static_cast<const T*>(a.draft) + (long(r) * k + j) * long(a.V);
                    const float tx = LT::load1(trow + x);
                    const float dx = LT::load1(drow + x);
                    px = exp2f(fmaf(tx, a.c, -mp)) / sp;
                    qx = exp2f(fmaf(dx, a.c, -mq)) / sq;
                    ratio = qx > 0.f ? px / qx : INFINITY;
                    const float u = a.uniforms[long(r) * (k + 1) + j];
                    keep = u < fminf(1.f, ratio);
                }
                if (!keep && acc == L) {
                    acc = j;
                    stat = make_float4(mp, sp, mq, sq);
                    rs_t = t;
                }
                if (a.diag && lane == 0)
                    reinterpret_cast<float4*>(a.diag)[t] = make_float4(px, qx, ratio, keep ? 1.f : 0.f);
            } else {
                if (acc == L) stat = make_float4(mp, sp, 0.f, 0.f);
                if (a.diag && lane == 0)
                    reinterpret_cast<float4*>(a.diag)[t] = make_float4(0.f, 0.f, 0.f, -1.f);
            }
        }
        if (verified && !xok && lane == 0) set_status(a.hdr, SPECV_STATUS_BAD_TOKEN);
    }

    if (lane <= k) {
        int v = -1;
        if (lane < acc) v = a.tokens[long(r) * k + lane];
        else if (lane == acc && MODE == SPECV_GREEDY) v = y;
        out[lane] = v;
    }
    if (lane == 0) {
        a.acc_len[r] = acc;
        if (MODE == SPECV_SAMPLE) {
            a.rs_stat[r] = stat;
            a.rs_row[r] = make_int4(rs_t, acc, acc < L ? 0 : 1, 0);
        }
    }
}

// ---------------------------------------------------------------------------
// resample: chunk masses of the residual max(0, p - q)
// ---------------------------------------------------------------------------

template <int DT, bool VEC>
__device__ __forceinline__ float residual_weight(float tx, float dx, float c, float4 st,
                                                 float inv_sp, float inv_sq) {
    const float p = exp2f(fmaf(tx, c, -st.x)) * inv_sp;
    const float q = exp2f(fmaf(dx, c, -st.z)) * inv_sq;
    return fmaxf(p - q, 0.f);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(256) void resample_mass(VerifyArgs a) {
    using LT = Logit<DT>;
    using T = typename LT::T;
    constexpr int kV = LT::kVec;
    constexpr int kU = kChunk / (kWave * kV);
    const int lane = threadIdx.x & (kWave - 1);
    const long item = long(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    if (item >= long(a.R) * a.C) return;
    const int r = int(item / a.C), chunk = int(item % a.C);
    const int4 rw = a.rs_row[r];
    if (rw.z != 0) return;                               // bonus / invalid: no residual
    const float4 st = a.rs_stat[r];
    const int j = rw.y;
    const T* trow = static_cast<const T*>(a.target) + (long(r) * (a.k + 1) + j) * long(a.V);
    const T* drow = static_cast<const T*>(a.draft) + (long(r) * a.k + j) * long(a.V);
    const float c = a.c, inv_sp = 1.f / st.y, inv_sq = 1.f / st.w;
    const int beg = chunk * kChunk, end = min(a.V, beg + kChunk);
    float s = 0.f;
    if (VEC) {
        const uint4* vt = reinterpret_cast<const uint4*>(trow);
        const uint4* vd = reinterpret_cast<const uint4*>(drow);
        const int v0 = beg / kV, v1 = end / kV;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            int v = v0 + u * kWave + lane;
            if (v < v1) {
                float xt[kV], xd[kV];
                LT::unpack(vt[v], xt);
                LT::unpack(vd[v], xd);
#pragma unroll
                for (int e = 0; e < kV; ++e) s += residual_weight<DT, VEC>(xt[e], xd[e], c, st, inv_sp, inv_sq);
            }
        }
    } else {
        for (int e = beg + lane; e < end; e += kWave)
            s += residual_weight<DT, VEC>(LT::load1(trow + e), LT::load1(drow + e), c, st, inv_sp, inv_sq);
    }
    s = wave_sum(s);
    if (lane == 0) a.mass[item] = s;
}

// ---------------------------------------------------------------------------
// resample: inverse-CDF pick
// ---------------------------------------------------------------------------

template <int DT, bool VEC>
__global__ __launch_bounds__(256) void resample_pick(VerifyArgs a) {
    using LT = Logit<DT>;
    using T = typename LT::T;
    const int lane = threadIdx.x & (kWave - 1);
    const int r = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (r >= a.R) return;
    const int4 rw = a.rs_row[r];
    if (rw.z == 2) return;
    const float4 st = a.rs_stat[r];
    const int t = rw.x, j = rw.y;
    bool residual = rw.z == 0;
    const int C = a.C;
    const float c = a.c;

    // chunk masses: the residual's, or the target row's own (unnormalised,
    // relative to its maximum) from the pass-1 partials
    auto chunk_mass = [&](int ch, bool res) -> float {
        if (res) return a.mass[long(r) * C + ch];
        float2 p = a.part[long(2 * t) * C + ch];
        return p.x == -INFINITY ? 0.f : p.y * exp2f(p.x - st.x);
    };
    float W = 0.f;
    if (residual) {
        for (int ch0 = 0; ch0 < C; ch0 += kWave) {
            int ch = ch0 + lane;
            W += wave_sum(ch < C ? chunk_mass(ch, true) : 0.f);
        }
        if (!(W > 0.f)) residual = false;                 // empty residual: draw from p
    }
    if (!residual) {
        W = 0.f;
        for (int ch0 = 0; ch0 < C; ch0 += kWave) {
            int ch = ch0 + lane;
            W += wave_sum(ch < C ? chunk_mass(ch, false) : 0.f);
        }
    }
    const float thr = a.uniforms[long(r) * (a.k + 1) + a.k] * W;
    const T* trow = static_cast<const T*>(a.target) + (long(r) * (a.k + 1) + j) * long(a.V);
    const T* drow = residual ? static_cast<const T*>(a.draft) + (long(r) * a.k + j) * long(a.V) : nullptr;
    const float inv_sp = 1.f / st.y, inv_sq = residual ? 1.f / st.w : 0.f;
    auto weight = [&](int e) -> float {
        const float tx = LT::load1(trow + e);
        if (residual) return residual_weight<DT, VEC>(tx, LT::load1(drow + e), c, st, inv_sp, inv_sq);
        return exp2f(fmaf(tx, c, -st.x));
    };
    const int yv = inv_cdf_pick(C, a.V, kChunk, thr, [&](int ch) { return chunk_mass(ch, residual); },
                                weight, lane);
    if (lane == 0) a.out_tokens[long(r) * (a.k + 1) + rw.y] = yv;
}

// ---------------------------------------------------------------------------
// host entry
// ---------------------------------------------------------------------------

template <int DT>
static int launch_verify(int mode, bool vec, const VerifyArgs& a, hipStream_t s) {
    const long slots = long(mode == SPECV_SAMPLE ? 2 : 1) * a.Bmax;
    const long items = slots * a.C;
    const dim3 blk(kWave * kWavesPerBlock);
    const dim3 g1((items + kWavesPerBlock - 1) / kWavesPerBlock);
    const dim3 gR((a.R + kWavesPerBlock - 1) / kWavesPerBlock);
    const dim3 gRC((long(a.R) * a.C + kWavesPerBlock - 1) / kWavesPerBlock);
    if (mode == SPECV_GREEDY) {
        if (vec)
            SPECV_LAUNCH("verify_partials", s, verify_partials<DT, SPECV_GREEDY, true><<<g1, blk, 0, s>>>(a));
        else
            SPECV_LAUNCH("verify_partials", s, verify_partials<DT, SPECV_GREEDY, false><<<g1, blk, 0, s>>>(a));
        SPECV_LAUNCH("verify_finalize", s, verify_finalize<DT, SPECV_GREEDY><<<gR, blk, 0, s>>>(a));
        return SPECV_OK;
    }
    if (vec) {
        SPECV_LAUNCH("verify_partials", s, verify_partials<DT, SPECV_SAMPLE, true><<<g1, blk, 0, s>>>(a));
        SPECV_LAUNCH("verify_finalize", s, verify_finalize<DT, SPECV_SAMPLE><<<gR, blk, 0, s>>>(a));
        SPECV_LAUNCH("resample_mass", s, resample_mass<DT, true><<<gRC, blk, 0, s>>>(a));
        SPECV_LAUNCH("resample_pick", s, resample_pick<DT, true><<<gR, blk, 0, s>>>(a));
    } else {
        SPECV_LAUNCH("verify_partials", s, verify_partials<DT, SPECV_SAMPLE, false><<<g1, blk, 0, s>>>(a));
        SPECV_LAUNCH("verify_finalize", s, verify_finalize<DT, SPECV_SAMPLE><<<gR, blk, 0, s>>>(a));
        SPECV_LAUNCH("resample_mass", s, resample_mass<DT, false><<<gRC, blk, 0, s>>>(a));
        SPECV_LAUNCH("resample_pick", s, resample_pick<DT, false><<<gR, blk, 0, s>>>(a));
    }
    return SPECV_OK;
}

}  // namespace specv

extern "C" size_t spec_verify_workspace_bytes(int mode, int R, int k, int V) {
    if (R < 1 || k < 1 || k > SPECV_MAX_K || V < 1 || (mode != SPECV_GREEDY && mode != SPECV_SAMPLE))
        return 0;
    return specv::ws_layout(mode, R, k, V).total;
}

extern "C" int spec_verify(int mode, int dtype, int R, int k, int V, const void* target_logits,
                           const void* draft_logits, const int32_t* draft_tokens, const int32_t* tags,
                           const int32_t* cu_rows, const int32_t* n_rows, float temperature,
                           const float* uniforms, int32_t* accepted_len_out, int32_t* out_tokens,
                           float* row_diag, void* ws, size_t ws_bytes, specv_stream stream) {
    using namespace specv;
    clear_error();
    if (mode != SPECV_GREEDY && mode != SPECV_SAMPLE)
        return fail(SPECV_EINVAL, "spec_verify: mode %d is neither greedy (0) nor sample (1)", mode);
    if (dtype != SPECV_BF16 && dtype != SPECV_F32)
        return fail(SPECV_EUNSUPPORTED, "spec_verify: dtype %d unsupported (bf16 = 0, f32 = 1)", dtype);
    if (R < 1 || k < 1 || k > SPECV_MAX_K || V < 1)
        return fail(SPECV_EINVAL, "spec_verify: need R >= 1, 1 <= k <= %d, V >= 1 (got R=%d k=%d V=%d)",
                    SPECV_MAX_K, R, k, V);
    if (long(R) * (k + 1) > INT_MAX / 2)
        return fail(SPECV_EINVAL, "spec_verify: R*(k+1) too large");
    if (!target_logits || !draft_tokens || !tags || !cu_rows || !n_rows || !accepted_len_out ||
        !out_tokens || !ws)
        return fail(SPECV_EINVAL, "spec_verify: NULL required pointer");
    if (mode == SPECV_SAMPLE) {
        if (!draft_logits || !uniforms)
            return fail(SPECV_EINVAL, "spec_verify: sampling needs draft_logits and uniforms");
        if (!(temperature > 0.f) || !(temperature < INFINITY))
            return fail(SPECV_EINVAL, "spec_verify: temperature must be finite and > 0 (got %g)",
                        double(temperature));
    }
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return fail(SPECV_EINVAL, "spec_verify: workspace must be 256-byte aligned");
    const Layout lay = ws_layout(mode, R, k, V);
    if (ws_bytes < lay.total)
        return fail(SPECV_EINVAL, "spec_verify: workspace of %zu bytes, need %zu", ws_bytes, lay.total);

    const int esize = dtype == SPECV_BF16 ? 2 : 4;
    const int vecw = 16 / esize;
    bool vec = (V % vecw) == 0 && aligned16(target_logits) &&
               (mode == SPECV_GREEDY || aligned16(draft_logits));

    VerifyArgs a;
    a.R = R; a.k = k; a.V = V;
    a.C = (V + kChunk - 1) / kChunk;
    a.Bmax = R * (k + 1);
    a.target = target_logits;
    a.draft = draft_logits;
    a.tokens = draft_tokens;
    a.tags = tags;
    a.cu_rows = cu_rows;
    a.n_rows = n_rows;
    a.uniforms = uniforms;
    a.c = mode == SPECV_SAMPLE ? float(1.4426950408889634 / double(temperature)) : 1.f;
    a.acc_len = accepted_len_out;
    a.out_tokens = out_tokens;
    a.diag = row_diag;
    char* w = static_cast<char*>(ws);
    a.hdr = reinterpret_cast<WsHeader*>(w);
    a.part = reinterpret_cast<float2*>(w + lay.part);
    a.rs_stat = reinterpret_cast<float4*>(w + lay.rs_stat);
    a.rs_row = reinterpret_cast<int4*>(w + lay.rs_row);
    a.mass = reinterpret_cast<float*>(w + lay.mass);
    hipStream_t s = static_cast<hipStream_t>(stream);
    return dtype == SPECV_BF16 ? launch_verify<SPECV_BF16>(mode, vec, a, s)
                               : launch_verify<SPECV_F32>(mode, vec, a, s);
}
