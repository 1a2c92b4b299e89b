// spec_attention: tag-masked attention of the flattened verification rows over
// a paged KV cache.
//
// Pages: padded decode kernels lose their utilisation on dynamic,
// variable-length verification, so every verified token is flattened into an
// independent element and the per-sequence dependencies travel in a tag tensor
// ("刚融完500亿创始人亲自下场写代码…", engineering table, row "内核利用率暴跌":
// 物理解耦稀疏注意力).
//
// Row t of the flattened batch, tag (r, j), is the query at position ctx_r + j
// of request r and sees request r's cached positions 0 .. ctx_r + j. The rows
// of a request share its pages, so one wavefront takes a request, one KV head
// and one run of key tiles (a split of fixed length, so that long and short
// contexts become equal work items), and streams those keys once for all the
// request's rows and all query heads of that KV head (grouped-query
// attention): up to 16 * MB query vectors per wavefront. Per 32-key tile
// (inside one page):
//   S^T = K Q^T    v_mfma_f32_16x16x32_bf16 with K fragments read straight
//                  from the cache rows; a lane ends up holding 8 keys of one
//                  query vector's column;
//   softmax        online, base 2; the column maximum needs two cross-lane
//                  steps, the column sums stay per lane until the end; keys
//                  after a row's tag position are masked;
//   O^T += V^T P^T the lane's 8 probabilities, rounded to bf16, are its B
//                  fragment as they stand (the key order inside a k-block is
//                  free as long as both operands use the same); V goes
//                  through LDS transposed, in that key order.
// The next tile's K and V are in flight while a tile is computed. A second
// kernel merges the splits, O = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s.
#include <algorithm>
#include <climits>

#include "common.h"
#include "host.h"

namespace specv {

namespace {

constexpr int kD = 128;                    // head dimension
constexpr int kTile = 32;                  // keys per tile
constexpr int kMaxMB = 2;                  // 16-vector query blocks per wavefront (more chunk the request)
constexpr int kLds = 40;                   // bf16 per LDS row of the V^T tile (32 keys + padding)

using bf16x8 = __attribute__((__vector_size__(8 * sizeof(short)))) short;
using f32x4 = __attribute__((__vector_size__(4 * sizeof(float)))) float;

struct AttnArgs {
    int R, k, Hq, Hkv, G, page_size, num_pages, max_pages;
    int head_major;                        // cache layout: 0 [pages, page_size, Hkv, D], 1 [pages, Hkv, page_size, D]
    int C;                                 // query chunks per (request, KV head)
    int split_tiles, Smax;                 // tiles per split; splits per request at most
    int Mmax;                              // (k+1) G: query vectors of a full request
    const uint16_t* q;                     // [R*(k+1), Hq, D]
    const uint16_t* kc;                    // [num_pages, page_size, Hkv, D] or [num_pages, Hkv, page_size, D]
    const uint16_t* vc;
    const int32_t* page_table;             // [R, max_pages]
    const int32_t* ctx_len;                // [R]
    const int32_t* tags;
    const int32_t* cu_rows;
    const int32_t* n_rows;
    float* out;                            // [R*(k+1), Hq, D]
    WsHeader* hdr;
    float* po;                             // [R, Hkv, Smax, Mmax, D] partial outputs
    float2* pml;                           // [R, Hkv, Smax, Mmax] (max, sum), base 2
    uint32_t* err;                         // [R, Hkv, Smax, C] status bits per wavefront
};

struct AttnLayout {
    size_t po, pml, err, total;
};

size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

AttnLayout attn_layout(int R, int Hkv, int Smax, int Mmax, int C) {
    AttnLayout l;
    const size_t n = size_t(R) * Hkv * Smax;
    l.po = a256(sizeof(WsHeader));
    l.pml = a256(l.po + n * Mmax * kD * sizeof(float));
    l.err = a256(l.pml + n * Mmax * sizeof(float2));
    l.total = a256(l.err + n * C * sizeof(uint32_t));
    return l;
}

// The request's rows: verified rows cu_rows[r] + j (j < L), then the bonus row
// N + r; `ok` when cu_rows and n_rows agree with that layout.
struct Req {
    int L, N, base, ctx, nk;
    bool rows_ok, ctx_ok;
};
__device__ __forceinline__ Req request(const AttnArgs& a, int r) {
    Req q;
    const int nrows = *a.n_rows;
    q.N = a.cu_rows[a.R];
    q.base = a.cu_rows[r];
    q.L = a.cu_rows[r + 1] - q.base;
    q.rows_ok = q.L >= 0 && q.L <= a.k && q.base >= 0 && q.base + q.L <= q.N && q.N + a.R == nrows &&
                nrows <= a.R * (a.k + 1);
    q.ctx = a.ctx_len[r];
    q.nk = q.ctx + q.L + 1;                  // keys the bonus row sees
    q.ctx_ok = q.ctx >= 0 && q.ctx <= a.max_pages * a.page_size - (a.k + 1);
    return q;
}
__device__ __forceinline__ int row_of(const Req& q, int r, int jr) { return jr < q.L ? q.base + jr : q.N + r; }
__device__ __forceinline__ int splits_of(const AttnArgs& a, const Req& q) {
    return (q.nk + kTile * a.split_tiles - 1) / (kTile * a.split_tiles);
}
__device__ __forceinline__ bool tag_ok(const AttnArgs& a, int t, int r, int jr) {
    return a.tags[2 * t] == r && a.tags[2 * t + 1] == jr;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {   // nearest, ties to even; lo, hi finite
    const uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
    const uint32_t ra = (a + 0x7FFFu + ((a >> 16) & 1u)) >> 16;
    const uint32_t rb = (b + 0x7FFFu + ((b >> 16) & 1u)) & 0xFFFF0000u;
    return ra | rb;
}

// Grid: (split, request, KV head, chunk) with the split slowest, so that the
// dispatcher hands out every request's first split before any second one and
// the empty tail (splits beyond a request's length) comes last.
// Two wavefronts per SIMD: about 210 registers each, no spills.
template <int MB>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void attn_partial(AttnArgs a) {
    __shared__ __align__(16) uint16_t vt[kD * kLds];     // V^T tile: [d][key slot]
    const int lane = threadIdx.x, g = lane >> 4, l16 = lane & 15;
    int b = blockIdx.x;
    const int c = b % a.C; b /= a.C;
    const int hk = b % a.Hkv; b /= a.Hkv;
    const int r = b % a.R;
    const int s = b / a.R;
    if (blockIdx.x == 0 && lane == 0) a.hdr->status = 0u;
    const long rec = (long(r) * a.Hkv + hk) * a.Smax + s;
    const Req rq = request(a, r);
    uint32_t* errw = a.err + rec * a.C + c;
    if (!rq.rows_ok || !rq.ctx_ok || s >= splits_of(a, rq)) {
        if (lane == 0) *errw = 0u;
        return;
    }
    const int G = a.G, M = (rq.L + 1) * G;
    const int m0 = c * 16 * MB;                       // first query vector of this chunk
    const int Mc = min(M - m0, 16 * MB);              // vectors in this chunk (may be <= 0)
    // keys this chunk needs: up to the last vector's row
    const int nkc = Mc > 0 ? rq.ctx + (m0 + Mc - 1) / G + 1 : 0;
    const int tiles = (nkc + kTile - 1) / kTile;
    const int t0 = s * a.split_tiles, t1 = min(tiles, t0 + a.split_tiles);

    // Q^T fragments (B operand): lane holds Q[m = 16 mb + l16][d = 32 ks + 8 g ..]; last
    // visible position of that column (-1: none, for padding or a bad tag)
    bf16x8 qf[MB][4];
    int lim[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = m0 + 16 * mb + l16;
        lim[mb] = -1;
        const uint16_t* qrow = a.q;
        if (16 * mb + l16 < Mc) {
            const int jr = m / G, t = row_of(rq, r, jr);
            if (tag_ok(a, t, r, jr)) lim[mb] = rq.ctx + jr;
            qrow = a.q + (long(t) * a.Hq + hk * G + m % G) * kD;
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint4 v = lim[mb] >= 0 ? *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g)
                                         : make_uint4(0, 0, 0, 0);
            qf[mb][ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    f32x4 o[8][MB];                                   // O^T[d = 16 db + 4 g + e][m = 16 mb + l16]
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) o[db][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mcol[MB], lsum[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) { mcol[mb] = -INFINITY; lsum[mb] = 0.f; }
    const float cs = 1.4426950408889634f / sqrtf(float(kD));     // log2(e) / sqrt(D)

    // Tile loads, K and V alike: lane holds row [key p0 + 16 kb + l16][d = 32 ks + 8 g ..];
    // keys at or past nkc read as zero (their V must not meet a zero weight as NaN).
    uint32_t err = 0;
    uint4 kr[2][4], vr[2][4];
    auto load_tile = [&](int tile) {
        const int p0 = tile * kTile;
        int page = a.page_table[long(r) * a.max_pages + p0 / a.page_size];
        if (page < 0 || page >= a.num_pages) { err |= SPECV_STATUS_BAD_PAGE; page = 0; }
        // element offset of (page, slot, head hk): position-major or head-major pages
        const long slot0 = p0 % a.page_size;
        const long pstride = a.head_major ? kD : long(a.Hkv) * kD;           // between positions
        const long base = a.head_major ? ((long(page) * a.Hkv + hk) * a.page_size) * kD
                                       : (long(page) * a.page_size * a.Hkv + hk) * kD;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bool ok = p0 + 16 * kb + l16 < nkc;
            const long off = base + (slot0 + 16 * kb + l16) * pstride + 8 * g;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                kr[kb][ks] = ok ? *reinterpret_cast<const uint4*>(a.kc + off + 32 * ks) : make_uint4(0, 0, 0, 0);
                vr[kb][ks] = ok ? *reinterpret_cast<const uint4*>(a.vc + off + 32 * ks) : make_uint4(0, 0, 0, 0);
            }
        }
    };

    // LDS column of key 16 kb + l16: k-slot 8 (l16 >> 2) + 4 kb + (l16 & 3), matching the
    // B fragment below (slot 8 g + 4 kb + e <-> key 16 kb + 4 g + e). Per tile: V to LDS,
    // S from the K registers, then the next tile's loads go into the freed registers and
    // are in flight during the softmax and O += V^T P^T.
    if (t0 < t1) load_tile(t0);
    for (int tile = t0; tile < t1; ++tile) {
        const int p0 = tile * kTile;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int col = 8 * (l16 >> 2) + 4 * kb + (l16 & 3);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const uint32_t w[4] = {vr[kb][ks].x, vr[kb][ks].y, vr[kb][ks].z, vr[kb][ks].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int d = 32 * ks + 8 * g + 2 * e;
                    vt[d * kLds + col] = uint16_t(w[e] & 0xFFFFu);
                    vt[(d + 1) * kLds + col] = uint16_t(w[e] >> 16);
                }
            }
        }
        // S^T[key 16 kb + 4 g + e][m 16 mb + l16]
        f32x4 sc[2][MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[kb][ks]),
                                                                  qf[mb][ks], acc, 0, 0, 0);
                sc[kb][mb] = acc;
            }
        if (tile + 1 < t1) load_tile(tile + 1);

        bf16x8 pf[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            float x[8];
            float tmax = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int p = p0 + 16 * kb + 4 * g + e;
                    x[4 * kb + e] = p <= lim[mb] ? sc[kb][mb][e] * cs : -INFINITY;
                    tmax = fmaxf(tmax, x[4 * kb + e]);
                }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float mn = fmaxf(mcol[mb], tmax);
            const float ms = mn == -INFINITY ? 0.f : mn;          // nothing visible yet: all weights 0
            const float alpha = __builtin_amdgcn_exp2f(mcol[mb] - ms);
            mcol[mb] = mn;
            float pv[8], ps = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) { pv[i] = __builtin_amdgcn_exp2f(x[i] - ms); ps += pv[i]; }
            lsum[mb] = lsum[mb] * alpha + ps;
#pragma unroll
            for (int db = 0; db < 8; ++db)
#pragma unroll
                for (int e = 0; e < 4; ++e) o[db][mb][e] *= alpha;
            const uint4 pk = make_uint4(pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]),
                                        pack_bf16(pv[4], pv[5]), pack_bf16(pv[6], pv[7]));
            pf[mb] = __builtin_bit_cast(bf16x8, pk);
        }
        __syncthreads();
        // O^T += V^T P^T: A = V^T[d 16 db + l16][slots 8 g ..], B = P^T[slots 8 g ..][m l16]
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const bf16x8 vf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&vt[(16 * db + l16) * kLds + 8 * g]));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                o[db][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[mb], o[db][mb], 0, 0, 0);
        }
        __syncthreads();
    }

    // partials: (max, sum) per column, O^T unnormalised
    const long prow = rec * a.Mmax;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        float l = lsum[mb];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        const int mm = 16 * mb + l16;
        if (mm >= Mc) continue;
        const long row = prow + m0 + mm;
        if (g == 0) a.pml[row] = make_float2(mcol[mb], l);
#pragma unroll
        for (int db = 0; db < 8; ++db)
            *reinterpret_cast<float4*>(a.po + row * kD + 16 * db + 4 * g) =
                make_float4(o[db][mb][0], o[db][mb][1], o[db][mb][2], o[db][mb][3]);
    }
    if (lane == 0) *errw = err;                       // wave-uniform: one page per tile
}

// Merge the splits of one (request, KV head) and write its rows; rows with a
// bad tag and requests with a bad page or context are written as zeros.
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
    __shared__ float wmx[64], winv[64];
    const int hk = blockIdx.x % a.Hkv, r = blockIdx.x / a.Hkv;
    const Req rq = request(a, r);
    if (!rq.rows_ok) {                                // rows unknown: nothing written
        if (threadIdx.x == 0 && hk == 0) set_status(a.hdr, SPECV_STATUS_BAD_TAG);
        return;
    }
    const long rec = (long(r) * a.Hkv + hk) * a.Smax;
    const int S = rq.ctx_ok ? splits_of(a, rq) : 0;
    uint32_t bad = rq.ctx_ok ? 0u : SPECV_STATUS_BAD_PAGE;
    for (int i = 0; i < S * a.C; ++i) bad |= a.err[rec * a.C + i];
    const int G = a.G, M = (rq.L + 1) * G;
    bool badtag = false;
    for (int m0 = 0; m0 < M; m0 += 64) {
        __syncthreads();
        if (threadIdx.x < 64 && m0 + int(threadIdx.x) < M) {    // per vector: max over splits, 1 / sum
            const int m = m0 + threadIdx.x;
            float mx = -INFINITY, den = 0.f;
            for (int s = 0; s < S; ++s) mx = fmaxf(mx, a.pml[(rec + s) * a.Mmax + m].x);
            for (int s = 0; s < S; ++s) {
                const float2 ml = a.pml[(rec + s) * a.Mmax + m];
                if (ml.x != -INFINITY) den += __builtin_amdgcn_exp2f(ml.x - mx) * ml.y;
            }
            wmx[threadIdx.x] = mx;
            winv[threadIdx.x] = den > 0.f ? 1.f / den : 0.f;
        }
        __syncthreads();
        const int mend = min(M - m0, 64);
        for (int i = threadIdx.x; i < mend * (kD / 4); i += blockDim.x) {
            const int mi = i / (kD / 4), d4 = i % (kD / 4), m = m0 + mi;
            const int jr = m / G, t = row_of(rq, r, jr);
            const bool tok = tag_ok(a, t, r, jr);
            badtag |= !tok;
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            const float mx = wmx[mi], inv = winv[mi];
            if (tok && !bad && inv > 0.f) {
                for (int s = 0; s < S; ++s) {
                    const float2 ml = a.pml[(rec + s) * a.Mmax + m];
                    if (ml.x == -INFINITY) continue;
                    const float w = __builtin_amdgcn_exp2f(ml.x - mx) * inv;
                    const float4 v = *reinterpret_cast<const float4*>(a.po + ((rec + s) * a.Mmax + m) * kD + 4 * d4);
                    acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
                }
            }
            *reinterpret_cast<float4*>(a.out + (long(t) * a.Hq + hk * G + m % G) * kD + 4 * d4) = acc;
        }
    }
    if (bad && threadIdx.x == 0) set_status(a.hdr, bad);
    if (badtag) set_status(a.hdr, SPECV_STATUS_BAD_TAG);
}

struct AttnPlan {
    int G, Mmax, MB, C, split_tiles, Smax;
};

int attn_plan(int R, int k, int Hq, int Hkv, int page_size, int max_pages, int split_keys, int cus, AttnPlan& p) {
    p.G = Hq / Hkv;
    p.Mmax = (k + 1) * p.G;
    p.MB = std::min(kMaxMB, (p.Mmax + 15) / 16);
    p.C = (p.Mmax + 16 * p.MB - 1) / (16 * p.MB);
    const long max_tiles = (long(max_pages) * page_size + kTile - 1) / kTile;
    if (split_keys > 0) {
        p.split_tiles = split_keys / kTile;
    } else {
        // about one resident round, 8 wavefronts per compute unit (two per SIMD at this
        // kernel's registers), if every request used its whole page-table row: in a
        // sweep of fixed split lengths at 256 requests with 1-3 K contexts, fewer and
        // longer splits ran fastest (no split 444 us per call, 33-tile splits 462 us)
        const long items = long(R) * Hkv * p.C * max_tiles;
        p.split_tiles = int(std::max<long>(4, (items + 8L * cus - 1) / (8L * cus)));
    }
    p.split_tiles = int(std::min<long>(p.split_tiles, max_tiles));
    p.Smax = int((max_tiles + p.split_tiles - 1) / p.split_tiles);
    return SPECV_OK;
}

int attn_check(int R, int k, int Hq, int Hkv, int D, int page_size, int num_pages, int max_pages, int split_keys,
               int kv_layout) {
    if (kv_layout != SPECV_KV_POSITION_MAJOR && kv_layout != SPECV_KV_HEAD_MAJOR)
        return fail(SPECV_EINVAL, "spec_attention: kv_layout %d is neither position-major (0) nor head-major (1)",
                    kv_layout);
    if (R < 1 || k < 1 || k > SPECV_MAX_K || Hkv < 1 || Hq < Hkv || Hq % Hkv || num_pages < 1 || max_pages < 1)
        return fail(SPECV_EINVAL,
                    "spec_attention: need R >= 1, 1 <= k <= %d, H_kv >= 1 dividing H_q, num_pages >= 1, max_pages >= 1",
                    SPECV_MAX_K);
    if (D != kD) return fail(SPECV_EUNSUPPORTED, "spec_attention: head dimension %d unsupported (only %d)", D, kD);
    if (page_size < kTile || page_size % kTile)
        return fail(SPECV_EUNSUPPORTED, "spec_attention: page size %d must be a multiple of %d", page_size, kTile);
    if (split_keys < 0 || split_keys % kTile)
        return fail(SPECV_EINVAL, "spec_attention: split_keys %d must be 0 (automatic) or a positive multiple of %d",
                    split_keys, kTile);
    if (long(max_pages) * page_size < k + 1)
        return fail(SPECV_EINVAL, "spec_attention: a page-table row of %d pages cannot hold k + 1 = %d positions",
                    max_pages, k + 1);
    if (long(max_pages) * page_size > INT_MAX / 2 || long(num_pages) * page_size * Hkv * kD > LONG_MAX / 4 ||
        long(R) * (k + 1) * Hq * kD > INT_MAX)
        return fail(SPECV_EUNSUPPORTED, "spec_attention: sizes overflow the kernel's index range");
    return SPECV_OK;
}

int device_cus(int& cus) {
    int dev = 0;
    cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return fail(SPECV_EDEVICE, "spec_attention: cannot query the device");
    return SPECV_OK;
}

}  // namespace

}  // namespace specv

extern "C" size_t spec_attention_workspace_bytes(int R, int k, int Hq, int Hkv, int page_size, int max_pages,
                                                 int split_keys) {
    using namespace specv;
    if (attn_check(R, k, Hq, Hkv, kD, page_size, 1, max_pages, split_keys, SPECV_KV_POSITION_MAJOR)) return 0;
    int cus = 0;
    if (device_cus(cus)) cus = 256;
    AttnPlan p;
    attn_plan(R, k, Hq, Hkv, page_size, max_pages, split_keys, cus, p);
    return attn_layout(R, Hkv, p.Smax, p.Mmax, p.C).total;
}

extern "C" int spec_attention(int R, int k, int Hq, int Hkv, int D, int page_size, int num_pages, int max_pages,
                              int kv_layout, int split_keys, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* page_table, const int32_t* ctx_len, const int32_t* tags,
                              const int32_t* cu_rows, const int32_t* n_rows, float* out, void* ws, size_t ws_bytes,
                              specv_stream stream) {
    using namespace specv;
    clear_error();
    if (int e = attn_check(R, k, Hq, Hkv, D, page_size, num_pages, max_pages, split_keys, kv_layout)) return e;
    if (!q || !k_cache || !v_cache || !page_table || !ctx_len || !tags || !cu_rows || !n_rows || !out || !ws)
        return fail(SPECV_EINVAL, "spec_attention: NULL required pointer");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return fail(SPECV_EINVAL, "spec_attention: q, the caches and out must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return fail(SPECV_EINVAL, "spec_attention: workspace must be 256-byte aligned");
    int cus = 0;
    if (int e = device_cus(cus)) return e;
    AttnPlan p;
    attn_plan(R, k, Hq, Hkv, page_size, max_pages, split_keys, cus, p);
    const AttnLayout lay = attn_layout(R, Hkv, p.Smax, p.Mmax, p.C);
    if (ws_bytes < lay.total)
        return fail(SPECV_EINVAL, "spec_attention: workspace of %zu bytes, need %zu", ws_bytes, lay.total);
    const long grid = long(p.Smax) * R * Hkv * p.C;
    if (grid > INT_MAX) return fail(SPECV_EUNSUPPORTED, "spec_attention: %ld work items exceed the grid", grid);
    AttnArgs a;
    a.R = R; a.k = k; a.Hq = Hq; a.Hkv = Hkv; a.G = p.G;
    a.page_size = page_size; a.num_pages = num_pages; a.max_pages = max_pages;
    a.head_major = kv_layout == SPECV_KV_HEAD_MAJOR;
    a.C = p.C; a.split_tiles = p.split_tiles; a.Smax = p.Smax; a.Mmax = p.Mmax;
    a.q = static_cast<const uint16_t*>(q);
    a.kc = static_cast<const uint16_t*>(k_cache);
    a.vc = static_cast<const uint16_t*>(v_cache);
    a.page_table = page_table; a.ctx_len = ctx_len;
    a.tags = tags; a.cu_rows = cu_rows; a.n_rows = n_rows;
    a.out = out;
    char* w = static_cast<char*>(ws);
    a.hdr = reinterpret_cast<WsHeader*>(w);
    a.po = reinterpret_cast<float*>(w + lay.po);
    a.pml = reinterpret_cast<float2*>(w + lay.pml);
    a.err = reinterpret_cast<uint32_t*>(w + lay.err);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.MB == 1)
        SPECV_LAUNCH("attn_partial", attn_partial<1>, int(grid), 64, 0, s, a);
    else
        SPECV_LAUNCH("attn_partial", attn_partial<2>, int(grid), 64, 0, s, a);
    SPECV_LAUNCH("attn_combine", attn_combine, R * Hkv, 256, 0, s, a);
    return SPECV_OK;
}
