/*
 * specv.h -- C ABI of the MI355X (gfx950) library for confidence-scheduled,
 * flattened speculative verification (DSpark).
 *
 * The operations follow the DSpark pages, cited by title and section:
 *   [P1] "刚融完500亿创始人亲自下场写代码DeepSeek不卷参数专治AI“嘴慢”"
 *        (mooersco.com), sections "1. 半自回归生成", "2. 置信度调度验证" and the
 *        engineering table under "不止是算法更是“工业级”的系统魔改".
 *   [P2] "DSpark 的 661% 提速，是真突破还是数字游戏？" (new-universe.cn),
 *        sections 一, 3.1 and 3.2.
 *   [P3] "DeepSeek服务器不再卡顿！DSpark加速60% - 80%，推理成本降40%"
 *        (qwbw.cn), sections "DSpark的神奇之处" and "成本与质量的考量".
 *   [P4] aibuzzwire.news, "deepseek-dspark-speculative-decoding-85-percent-
 *        faster-llm-inference", section "置信度计划、负载感知验证".
 *
 * Conventions for every call
 *   - Array arguments are DEVICE pointers owned by the caller; the library
 *     never keeps them after the call returns.
 *   - A call validates its scalar arguments and pointers on the host, then
 *     only enqueues kernels on `stream` (a hipStream_t; NULL is the null
 *     stream) and returns. It never allocates, frees or synchronises.
 *   - Return value: SPECV_OK, or a negative code; on SPECV_EINVAL and
 *     SPECV_EUNSUPPORTED nothing was enqueued. specv_last_error() gives a
 *     message (per host thread).
 *   - Data errors found on the device (a draft token outside [0, V), a tag that
 *     disagrees with cu_rows, a logit that is NaN or +inf) never fault: a bit
 *     is set in the workspace status word, readable with specv_read_status(),
 *     and the offending row or request is handled as each call states.
 *   - Calls that share a workspace must not run concurrently.
 *   - Random numbers: every uniform a call consumes is
 *       U(seed, step, purpose, r, i) = (word 0 of Philox4x64-10 at counter
 *           (i + 1, r, purpose, 0) under key (seed, step)) >> 40, times 2^-24
 *     (Philox: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 *     1, 2, 3", SC'11), a float multiple of 2^-24 in [0, 1), addressed by the
 *     decision it drives (purpose 0: keep or reject the draft token at position i
 *     of request r; 1: the extra token drawn at position i = a_r; 2: the draft
 *     head's token at position i), so results depend on neither the schedule
 *     nor the row order (the residual draw's rejection trials use words 0 and 1
 *     of the blocks at counters (a_r + 1, r, 1, t), t = 0 .. 64; spec_verify
 *     states how). A caller that advances `step` once per decoding step
 *     gets fresh, reproducible randomness without any state in the library.
 *     The pages name Philox-seeded trials only; the rest is this library's
 *     reading. A caller may pass its own uniforms instead (the `uniforms`
 *     arguments; NULL selects the generator).
 *   - No global mutable state, with one opt-in exception: the timing hooks at
 *     the end of this header (off by default, guarded by a mutex, meant for
 *     benchmarks; they change no result).
 *   - Row-major layouts throughout. "bf16" arrays hold IEEE bfloat16 values
 *     (2 bytes each); "f32" arrays hold float.
 */
#ifndef SPECV_H
#define SPECV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* specv_stream; /* a hipStream_t */

enum {
    SPECV_OK = 0,
    SPECV_EINVAL = -1,        /* bad argument; nothing enqueued */
    SPECV_EUNSUPPORTED = -2,  /* valid but not supported (dtype, sizes); nothing enqueued */
    SPECV_EDEVICE = -3        /* a HIP launch or runtime call failed */
};

enum { SPECV_BF16 = 0, SPECV_F32 = 1 };       /* logit storage type */
enum { SPECV_GREEDY = 0, SPECV_SAMPLE = 1 };  /* acceptance mode */
enum { SPECV_KV_POSITION_MAJOR = 0, SPECV_KV_HEAD_MAJOR = 1 };  /* spec_attention cache layout */

/* status-word bits (specv_read_status) */
enum {
    SPECV_STATUS_BAD_TOKEN = 1u, /* a draft token outside [0, V) */
    SPECV_STATUS_BAD_TAG = 2u,   /* tags[] disagrees with cu_rows[] */
    SPECV_STATUS_BAD_PAGE = 4u,  /* spec_attention: a page id outside [0, num_pages), or a
                                    context length that is negative or overruns its page-table row */
    SPECV_STATUS_NONFINITE = 8u, /* a logit row with a NaN or +inf value (sampling: also a row
                                    of -inf only, which has no distribution) */
    SPECV_STATUS_BAD_STATS = 16u, /* spec_verify_ex: a draft statistic made at another temperature
                                     or for another token than the one verified */
    SPECV_STATUS_LATE_SCHEDULE = 32u /* spec_step: the verification pass stopped waiting for the
                                        schedule (one second; only other work holding the device
                                        can delay it so long): every result of the call is void */
};

/* The draft head's statistics of one draft row (r, i), written by markov_draft
 * and rnn_draft in sampling mode, read by spec_verify_ex: the base-2 softmax
 * state of the stored draft logits, so that verification needs no pass over
 * the draft rows. */
typedef struct {
    float m;          /* max over the row of logit * c */
    float z;          /* sum over the row of exp2(logit * c - m) */
    float x_logit;    /* the stored logit of the drawn token */
    float c;          /* log2(e) / temperature, the scale used */
    int32_t token;    /* the drawn token */
    int32_t pad[3];
} specv_draft_stat;

/* Limits of the scheduler: all candidate keys of one call are held in the
 * local data share of each of its workgroups. */
#define SPECV_MAX_K 32
#define SPECV_MAX_SCHED_ITEMS 16384 /* R * k */

/* ------------------------------------------------------------------------ */
/* spec_schedule                                                             */
/* ------------------------------------------------------------------------ */
/*
 * Calibrate confidences, turn them into survival probabilities, choose each
 * request's verification length with the hardware-aware prefix scheduler, and
 * flatten the chosen rows ([P1] "2. 置信度调度验证"; [P2] 3.2; [P3] "DSpark的神奇之处";
 * [P4] "置信度计划、负载感知验证"; flattening: [P1] engineering table, row
 * "内核利用率暴跌").
 *
 *   c[r,i] = 1 / (1 + exp(-z[r,i] / T[i]))          temporal temperature scaling
 *   S[r,i] = c[r,0] * ... * c[r,i]                    survival (float64)
 *   Q[r,i] = floor(S[r,i] * 2^32 + 0.5)               integer key
 *   Candidates (r,i), i < min(k, max_len), sorted by Q descending, then i, then r.
 *   For M = 0 .. #candidates, with P(M) the sum of the first M keys and Bt = R + M:
 *     G(M) = (R * 2^32 + P(M)) * thr(Bt) / Bt        (float64, no fused ops)
 *   thr(Bt) interpolates the table linearly; below tbl_tokens[0] it is
 *   tbl_thr[0] * Bt / tbl_tokens[0]; at or above the last point it is the last
 *   value. M* = the smallest M with the largest G; L_r = the number of request
 *   r's candidates among the first M*. max_len < 0 forces L_r = k.
 *   Flatten (one element per row, tagged (r, j)): the verified rows first,
 *   request-major: request r's rows cu_rows[r] .. cu_rows[r+1]-1 carry
 *   (r, 0) .. (r, L_r - 1), cu_rows = exclusive prefix sum of L, N = cu_rows[R];
 *   then one bonus row per request: row N + r carries (r, L_r).
 *   n_rows = N + R. (The pages fix no order; this one keeps the rows that need
 *   draft logits in one block.)
 *
 * Arguments (device pointers unless noted)
 *   R, k          requests and draft block size (host ints): 1 <= k <= 32,
 *                 R >= 1, R*k <= 16384
 *   conf_logit    f32 [R,k]   raw confidence-head logits z
 *   pos_temp      f32 [k]     temperatures T_i > 0 (not checked on the device)
 *   tbl_tokens    i32 [n_tbl] batch tokens, strictly increasing, > 0
 *   tbl_thr       f64 [n_tbl] throughput at those batch sizes, > 0
 *   n_tbl         host int, 1..64
 *   max_len       host int, -1 (verify all k) or 0..k
 *   len_out       i32 [R]           L_r
 *   tags_out      i32 [R*(k+1),2]   (request, position) per flattened row;
 *                                   rows >= n_rows are left untouched
 *   cu_rows_out   i32 [R+1]         verified-row offsets (see Flatten)
 *   n_rows_out    i32 [1]
 *   survival_out  f64 [R,k] or NULL
 *   ws, ws_bytes  workspace of at least spec_schedule_workspace_bytes(R, k)
 *                 bytes, 256-byte aligned; needs no initialisation
 * Execution (on `stream`; no sort):
 *   - max_len -1 or 0: one workgroup writes the survival and flattens the fixed
 *     lengths.
 *   - R * k <= 4096: one 1024-thread workgroup does everything in
 *     its local data share: the keys go into 4096 buckets ordered like the keys
 *     (linear in S above 1/4, by octave below), each key's sorted position is its
 *     bucket's start plus the smaller keys in its bucket, P(M) comes from exact
 *     integer scans, then G(M) for every M, the best M, the lengths and the
 *     flattened batch.
 *   - larger: a one-wavefront kernel clears the workspace's arrival counter,
 *     then up to 256 workgroups each compute every key, count for their share
 *     of keys how many keys are smaller (and their sum) and post their best
 *     prefix; the last to arrive picks the overall best and flattens.
 * Errors: SPECV_EINVAL for NULL required pointers, out-of-range sizes or a small
 *   workspace; SPECV_EDEVICE if the launch fails.
 */
size_t spec_schedule_workspace_bytes(int R, int k);
int spec_schedule(int R, int k, const float* conf_logit, const float* pos_temp,
                  const int32_t* tbl_tokens, const double* tbl_thr, int n_tbl, int max_len,
                  int32_t* len_out, int32_t* tags_out, int32_t* cu_rows_out,
                  int32_t* n_rows_out, double* survival_out, void* ws, size_t ws_bytes,
                  specv_stream stream);

/* ------------------------------------------------------------------------ */
/* spec_flatten                                                              */
/* ------------------------------------------------------------------------ */
/*
 * Flatten given verification lengths (e.g. decided by the caller one or two
 * rounds ahead) into the tagged varlen batch that spec_verify consumes
 * ([P1] engineering table, row "内核利用率暴跌"). Same outputs as the
 * flattening part of spec_schedule. Lengths outside [0, k] are clamped.
 *   R >= 1, 1 <= k <= 32 (host ints); len_in i32 [R]; tags_out i32 [R*(k+1),2];
 *   cu_rows_out i32 [R+1]; n_rows_out i32 [1].
 */
int spec_flatten(int R, int k, const int32_t* len_in, int32_t* tags_out,
                 int32_t* cu_rows_out, int32_t* n_rows_out, specv_stream stream);

/* ------------------------------------------------------------------------ */
/* spec_verify                                                               */
/* ------------------------------------------------------------------------ */
/*
 * The exact acceptance rule over the flattened batch ([P2] 一: verified tokens
 * are kept and the first divergence is resampled; [P3] "DSpark的神奇之处":
 * rejection sampling keeps the target's distribution; [P4] opening: the longest
 * correct prefix is accepted).
 *
 * The batch is spec_schedule's / spec_flatten's: request r has L_r =
 * cu_rows[r+1] - cu_rows[r] verified rows at cu_rows[r] + j (j < L_r) and its
 * bonus row at cu_rows[R] + r (j = L_r); tags must agree with that layout.
 *   greedy:   g_j = argmax_v target[r,j,v] (lowest index on ties);
 *             keep x_j iff g_j == x_j.
 *   sampling: p_j = softmax(target[r,j,:] / tau), q_j = softmax(draft[r,j,:] / tau);
 *             keep x_j iff u[r,j] < min(1, p_j(x_j) / q_j(x_j)).
 *   a_r = first j < L_r not kept, else L_r.
 *   out_tokens[r,0..a_r-1] = x[r,0..a_r-1]; out_tokens[r,a_r] =
 *     greedy:   g_{a_r};
 *     sampling, a_r = L_r: the bonus token, an inverse-CDF draw from p_{L_r}
 *               with u = U(seed, step, 1, r, a_r) or the caller's u[r,k]: the
 *               smallest v with w_0 + .. + w_v > u * sum(w);
 *     sampling, a_r < L_r: a draw from max(0, p - q) at row a_r (from p when
 *               that residual has no mass). With the caller's uniforms: the
 *               inverse-CDF draw with u[r,k]. With the generator: rejection
 *               from p, trial t = 0, 1, .. 63 taking (u1, u2) = words 0 and 1
 *               of the block at counter (a_r + 1, r, 1, t), each >> 40 times
 *               2^-24: y = the inverse-CDF draw from p with u1, kept iff
 *               u2 < 1 - q(y) / p(y); the first kept y is the token (exactly
 *               residual-distributed). With all 64 rejected: the inverse-CDF
 *               draw from the residual with u1 of trial 64.
 *   out_tokens[r, a_r+1 .. k] = -1; accepted_len[r] = a_r.
 * Uniforms: u[r,j] = U(seed, step, 0, r, j) and the draws' above (see the
 * conventions), or the caller's `uniforms`.
 * Arithmetic is float32 (softmax statistics in base 2 with a pre-scaled
 * log2(e)/tau); greedy decisions are exact comparisons.
 * Logits may be -inf (a token that cannot be drawn). A request with a NaN or
 * +inf logit in any row this call reads for it (sampling: also a row of -inf
 * only) gets accepted_len 0 and out_tokens all -1, and sets
 * SPECV_STATUS_NONFINITE; the other requests are unaffected.
 *
 * Arguments (device pointers unless noted)
 *   mode, dtype     SPECV_GREEDY / SPECV_SAMPLE, SPECV_BF16 / SPECV_F32
 *   R, k, V         host ints: R >= 1, 1 <= k <= 32, V >= 1
 *   target_logits   [R,k+1,V] in dtype
 *   draft_logits    [R,k,V] in dtype (sampling); ignored and may be NULL in greedy
 *   draft_tokens    i32 [R,k]
 *   tags, cu_rows, n_rows   the flattened batch (spec_schedule / spec_flatten)
 *   temperature     host float tau > 0 (sampling); ignored in greedy
 *   seed, step      host uint64: the key of the uniforms (sampling)
 *   uniforms        NULL (the generator), or f32 [R,k+1] in [0,1): column j < k
 *                   decides row j, column k drives the resample / bonus draw
 *   accepted_len_out i32 [R]
 *   out_tokens       i32 [R,k+1]
 *   row_diag         f32 [R*(k+1),4] or NULL. Verified rows: sampling
 *                    {p(x), q(x), p(x)/q(x), u}, greedy {argmax, max logit, 0,
 *                    kept}. Bonus row of request r (row N + r): sampling
 *                    {m, a_r, drawn token, u of the draw (the kept trial's u1)}
 *                    with m = -(t + 1) for a draw kept at trial t, else
 *                    sum(max(0, p - q)) at row a_r (0 when a_r = L_r); greedy
 *                    {argmax, max logit, 0, -1}. Rows of a request with a data
 *                    error: undefined.
 *   ws, ws_bytes     workspace of at least spec_verify_workspace_bytes(R,k,V)
 *                    bytes, 256-byte aligned; its contents need no
 *                    initialisation (chunk partials of the call in flight)
 * Execution: two kernels on `stream`. A persistent grid streams every logit
 * row of the batch once into per-chunk partials; then one workgroup per request
 * decides its rows and, in sampling mode, draws the extra token: the bonus
 * draw and the rejection trials read one chunk of a row per draw; the
 * inverse-CDF residual draw (caller uniforms, or all trials rejected) re-reads
 * the rejected row pair. With fewer requests than compute units (sampling),
 * two or four workgroups share a request's re-read and the last to finish
 * draws; none ever waits for another.
 * Errors: SPECV_EINVAL (NULL pointers, sizes, tau, small workspace),
 *         SPECV_EUNSUPPORTED (dtype; R*(k+1)*V beyond 32-bit item counts;
 *         sampling with more than 4096 chunks per row, i.e. V > 8388608 in
 *         bf16 or V > 4194304 in f32), SPECV_EDEVICE (launch failure).
 */
size_t spec_verify_workspace_bytes(int R, int k, int V);
int spec_verify(int mode, int dtype, int R, int k, int V, const void* target_logits,
                const void* draft_logits, const int32_t* draft_tokens, const int32_t* tags,
                const int32_t* cu_rows, const int32_t* n_rows, float temperature, uint64_t seed,
                uint64_t step, const float* uniforms, int32_t* accepted_len_out, int32_t* out_tokens,
                float* row_diag, void* ws, size_t ws_bytes, specv_stream stream);

/* ------------------------------------------------------------------------ */
/* spec_verify_ex: spec_verify with the next round's schedule riding along   */
/* ------------------------------------------------------------------------ */
/*
 * The asynchronous lagged scheduler ([P1] section "2. 置信度调度验证": lengths
 * for a round come from confidences of two rounds earlier, so the schedule
 * leaves the critical path; fixed-capacity launches can be replayed as a
 * graph). spec_verify_ex verifies this round exactly as spec_verify does and,
 * in the same launch sequence on the same stream, computes the spec_schedule
 * described by `next` (typically the next round's batch, from older
 * confidences). When next->R * next->k <= 4096 and next->max_len >= 1 the
 * schedule runs as one extra workgroup of the decide kernel, beside this
 * round's decisions; otherwise it is launched after them on the same stream.
 * Its results are those of spec_schedule with the same arguments, bit for bit.
 *
 * next: host pointer, or NULL (then spec_verify_ex is spec_verify). Its fields
 *   are spec_schedule's arguments (device pointers as there). Its batch
 *   (tags_out, cu_rows_out, n_rows_out) must be other buffers than this call's
 *   tags, cu_rows and n_rows, and nothing else may use its workspace meanwhile.
 *
 * draft_stats: NULL, or (sampling) the draft head's specv_draft_stat [R,k] for
 *   these draft rows (markov_draft / rnn_draft, same temperature). q's
 *   normaliser and q(x) then come from them and the verification pass reads
 *   no draft row; the draft logits are still read for the rejected rows'
 *   residuals. A statistic whose scale c is not log2(e)/temperature, or whose
 *   token is not draft_tokens[r,i], voids its request and sets
 *   SPECV_STATUS_BAD_STATS. Ignored in greedy mode.
 * Errors: as spec_verify and spec_schedule (with "spec_verify_ex (next)" in the
 *   message for the job); SPECV_EINVAL if the next batch is this one.
 */
typedef struct {
    int R, k;
    const float* conf_logit;        /* f32 [R,k] */
    const float* pos_temp;          /* f32 [k] */
    const int32_t* tbl_tokens;      /* i32 [n_tbl] */
    const double* tbl_thr;          /* f64 [n_tbl] */
    int n_tbl, max_len;
    int32_t* len_out;               /* i32 [R] */
    int32_t* tags_out;              /* i32 [R*(k+1),2] */
    int32_t* cu_rows_out;           /* i32 [R+1] */
    int32_t* n_rows_out;            /* i32 [1] */
    double* survival_out;           /* f64 [R,k] or NULL */
    void* ws;                       /* spec_schedule_workspace_bytes(R, k) bytes */
    size_t ws_bytes;
} specv_schedule_job;

int spec_verify_ex(int mode, int dtype, int R, int k, int V, const void* target_logits,
                   const void* draft_logits, const int32_t* draft_tokens, const int32_t* tags,
                   const int32_t* cu_rows, const int32_t* n_rows, float temperature, uint64_t seed,
                   uint64_t step, const float* uniforms, int32_t* accepted_len_out, int32_t* out_tokens,
                   float* row_diag, void* ws, size_t ws_bytes, const specv_draft_stat* draft_stats,
                   const specv_schedule_job* next, specv_stream stream);

/* ------------------------------------------------------------------------ */
/* spec_step: this round's schedule, then its verification                   */
/* ------------------------------------------------------------------------ */
/*
 * spec_schedule of the job `sched` (this round's confidences) followed by
 * spec_verify of the batch it writes (its tags_out, cu_rows_out, n_rows_out),
 * with the same results bit for bit: the synchronous step of [P2] 3.2 and
 * [P3] "DSpark的神奇之处" (schedule from the current confidences, then verify).
 * When the schedule fits one workgroup (R * k <= 4096, max_len >= 1), one
 * launch holds both the schedule and the verification pass: the schedule runs
 * on one compute unit while the others stream every request's target row
 * (r, 0), which the batch holds whatever lengths the schedule picks (verified
 * row 0, or the bonus row when L_r = 0), and, when those rows alone would be
 * read well before the schedule is done (few requests for their positions),
 * also the target rows (r, 1) and draft rows (r, 0), which every request with
 * L_r > 0 needs (those of requests with L_r = 0 are read for nothing); the
 * schedule writes the batch with
 * device-scope atomic stores and then a completion mark unique to the call,
 * and the other workgroups, once the mark is there, stream the batch's other
 * rows. The latency-bound schedule hides behind reads the step needs anyway,
 * and the grid does not drain between the two. A streaming workgroup that
 * waits a second for the mark (only other work holding the device can delay
 * the schedule so long) goes on and sets SPECV_STATUS_LATE_SCHEDULE: the
 * call's results are then void. Otherwise the schedule and the verification
 * run one after the other.
 * Arguments: sched as spec_verify_ex's `next` (a host pointer; device
 *   pointers inside; its workspace separate from `ws`); the others as
 *   spec_verify_ex, with R and k taken from sched.
 * Errors: as spec_schedule and spec_verify ("spec_step (schedule)" in the
 *   message for the job); all arguments are checked before anything is
 *   enqueued.
 */
int spec_step(const specv_schedule_job* sched, int mode, int dtype, int V, const void* target_logits,
              const void* draft_logits, const int32_t* draft_tokens, float temperature, uint64_t seed,
              uint64_t step, const float* uniforms, int32_t* accepted_len_out, int32_t* out_tokens,
              float* row_diag, const specv_draft_stat* draft_stats, void* ws, size_t ws_bytes,
              specv_stream stream);

/* ------------------------------------------------------------------------ */
/* spec_verify_noalloc: spec_verify without a workspace                      */
/* ------------------------------------------------------------------------ */
/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. It computes
 * exactly what spec_verify computes (same kernels), but its chunk partials
 * live in one static device array of SPECV_NOALLOC_SCRATCH_BYTES inside the
 * library, which each GPU the library runs on holds until the process ends.
 * The call allocates nothing: it looks the array's address up once per device
 * (on its first call there) and then only enqueues kernels.
 *
 * Arguments: as spec_verify, without ws and ws_bytes, plus
 *   status_out  NULL, or a device u32 that receives the status word (0 or
 *               SPECV_STATUS_* bits) when the call's kernels have run; with
 *               NULL the status word stays inside the library.
 * Limit: spec_verify_workspace_bytes(R, k, V) <= SPECV_NOALLOC_SCRATCH_BYTES
 *   (e.g. R = 512, k = 5, V = 151936 needs 7.7 MB); larger batches return
 *   SPECV_EUNSUPPORTED with the sizes in the message.
 * Every call on one GPU uses that GPU's one array and leaves its contents
 * behind (the kernels clear what must start at zero): calls that may overlap
 * on one GPU, on different streams or from different host threads, race and
 * must be serialised by the caller. Not usable with spec_verify_ex's
 * next-round schedule.
 * Errors: as spec_verify.
 */
#define SPECV_NOALLOC_SCRATCH_BYTES (16u << 20)
int spec_verify_noalloc(int mode, int dtype, int R, int k, int V, const void* target_logits,
                        const void* draft_logits, const int32_t* draft_tokens, const int32_t* tags,
                        const int32_t* cu_rows, const int32_t* n_rows, float temperature, uint64_t seed,
                        uint64_t step, const float* uniforms, int32_t* accepted_len_out,
                        int32_t* out_tokens, float* row_diag, uint32_t* status_out, specv_stream stream);

/* ------------------------------------------------------------------------ */
/* markov_draft                                                              */
/* ------------------------------------------------------------------------ */
/*
 * The Markov head of the semi-autoregressive drafter ([P1] "1. 半自回归生成":
 * a parallel backbone plus a light sequential module injecting prefix
 * information token by token, by default a Markov head that depends only on the
 * previous token; [P2] 3.1). For i = 0..k-1, with x_{-1} = prev_token[r]:
 *   dl[r,i,:] = round(backbone[r,i,:] + emb[x_{i-1},:] . proj^T)  (float32
 *               accumulation; one round-to-nearest-even to dtype)
 *   x_i = argmax dl[r,i,:] (greedy, lowest index) or the inverse-CDF draw from
 *         softmax(dl[r,i,:] / tau) with u = U(seed, step, 2, r, i), or
 *         uniforms[r,i] (sampling).
 * The rounded logits are written out: they are the draft distribution the
 * verifier must use. In sampling mode the call can also write each draft row's
 * specv_draft_stat (draft_stats_out), which lets spec_verify_ex skip the pass
 * over the draft rows. A row whose softmax state (sampling) or maximum (greedy:
 * +inf) is not finite sets SPECV_STATUS_NONFINITE; its token is then
 * unspecified (within [0, V)).
 *
 * Arguments (device pointers unless noted)
 *   mode, dtype     as spec_verify
 *   R, k, V, d_m    host ints: R >= 1, 1 <= k <= 32, V >= 1, d_m >= 1
 *                   (bf16: d_m % 32 == 0 and d_m <= 480)
 *   backbone_logits [R,k,V] dtype
 *   emb             [V,d_m] dtype   previous-token embedding
 *   proj            [V,d_m] dtype   projection, one d_m row per vocabulary entry
 *                   (the transpose of a [d_m,V] weight: a 64-entry vocabulary
 *                   slice of it is one contiguous 64 x d_m block, which the
 *                   projection kernel stages into its local data share with
 *                   plain linear loads)
 *   prev_token      i32 [R]          last committed token
 *   temperature     host float > 0 (sampling)
 *   seed, step      host uint64: the key of the uniforms (sampling)
 *   uniforms        NULL (the generator), or f32 [R,k] (sampling)
 *   draft_tokens_out i32 [R,k];  draft_logits_out [R,k,V] dtype
 *   draft_stats_out  NULL, or specv_draft_stat [R,k] (written in sampling mode)
 *   ws, ws_bytes    at least markov_draft_workspace_bytes(R,k,V,d_m)
 * Errors: as spec_verify.
 */
size_t markov_draft_workspace_bytes(int R, int k, int V, int d_m);
int markov_draft(int mode, int dtype, int R, int k, int V, int d_m,
                 const void* backbone_logits, const void* emb, const void* proj,
                 const int32_t* prev_token, float temperature, uint64_t seed, uint64_t step,
                 const float* uniforms, int32_t* draft_tokens_out, void* draft_logits_out,
                 specv_draft_stat* draft_stats_out, void* ws, size_t ws_bytes, specv_stream stream);

/* ------------------------------------------------------------------------ */
/* rnn_draft                                                                 */
/* ------------------------------------------------------------------------ */
/*
 * The RNN head: the pages' other light sequential module, which carries the
 * whole prefix of the block in a recurrent state instead of the previous token
 * alone ([P1] "1. 半自回归生成"; [P2] 3.1: more of the block's history, small
 * gain, more cost). Read as, for i = 0..k-1, with h_{-1} = 0 and
 * x_{-1} = prev_token[r]:
 *   h_i      = round(tanh(emb[x_{i-1},:] + rec . h_{i-1}))   ((rec . h)_j = sum_q rec[j,q] h_q;
 *              float32 accumulation; rounded to dtype: the operand of the products)
 *   dl[r,i,:] = round(backbone[r,i,:] + h_i . proj^T)          (as markov_draft)
 *   x_i       drawn as markov_draft draws.
 *
 * Arguments: as markov_draft, plus
 *   rec       [d_m,d_m] dtype   the recurrence
 *   state_out optional [R,k,d_m] dtype: the states h_i (NULL: kept in the
 *             workspace); 16-byte aligned for bf16
 *   d_m       <= 512 (bf16: a multiple of 32, <= 480)
 *   ws        at least rnn_draft_workspace_bytes(R,k,V,d_m)
 * Errors: as markov_draft.
 */
size_t rnn_draft_workspace_bytes(int R, int k, int V, int d_m);
int rnn_draft(int mode, int dtype, int R, int k, int V, int d_m, const void* backbone_logits,
              const void* emb, const void* rec, const void* proj, const int32_t* prev_token,
              float temperature, uint64_t seed, uint64_t step, const float* uniforms,
              int32_t* draft_tokens_out, void* draft_logits_out, specv_draft_stat* draft_stats_out,
              void* state_out, void* ws, size_t ws_bytes, specv_stream stream);

/* ------------------------------------------------------------------------ */
/* spec_attention                                                            */
/* ------------------------------------------------------------------------ */
/*
 * Attention of the flattened verification batch over a paged KV cache, masked
 * by the tag tensor. [P1], engineering table, row "内核利用率暴跌": padded
 * kernels lose their utilisation on dynamic, variable-length verification, so
 * each token is flattened into an independent element and the sequence
 * dependencies travel in a tag tensor (physically decoupled sparse attention).
 *
 * For every flattened row t < n_rows with tag (r, j) and every query head h:
 *   out[t,h,:] = sum_p w_p V_r[p, h/G, :],  w = softmax_p(q[t,h,:] . K_r[p, h/G, :] / sqrt(D)),
 * over request r's positions p = 0 .. ctx_len[r] + j (G = H_q / H_kv: grouped-
 * query attention). Position p of request r is slot p % page_size of page
 * page_table[r, p / page_size]. The verified tokens' own keys and values are
 * expected in the cache already (positions ctx_len[r] .. ctx_len[r] + L_r).
 * Arithmetic: scores and sums in float32 from exact bf16 products; the
 * softmax weights enter the weighted sum of values rounded to bf16.
 *
 * Arguments (device pointers unless noted)
 *   R, k            host ints: R >= 1, 1 <= k <= 32; the flattened batch has
 *                   R*(k+1) row slots in the spec_flatten layout
 *   Hq, Hkv, D      host ints: H_kv divides H_q; D == 128
 *   page_size       host int, a multiple of 32
 *   num_pages       host int: pages in each cache pool
 *   max_pages       host int: columns of page_table; ctx_len[r] + k + 1 must
 *                   fit in max_pages * page_size
 *   kv_layout       host int: SPECV_KV_POSITION_MAJOR, pages [page_size, Hkv, D]
 *                   (a position's heads side by side), or SPECV_KV_HEAD_MAJOR,
 *                   pages [Hkv, page_size, D] (each head's page_size x D block
 *                   contiguous; the faster one to stream, ~12% at 64-key pages)
 *   split_keys      host int: keys per work item (a multiple of 32), or 0 to
 *                   let the library choose; a tuning knob, results depend on
 *                   it only through the float32 summation order
 *   q               bf16 [R*(k+1), Hq, D] queries of the flattened rows
 *   k_cache, v_cache bf16 [num_pages, page_size, Hkv, D] or [num_pages, Hkv, page_size, D]
 *   page_table      i32 [R, max_pages];  ctx_len i32 [R] (>= 0)
 *   tags, cu_rows, n_rows  as written by spec_schedule / spec_flatten
 *   out             f32 [R*(k+1), Hq, D]; rows >= n_rows are not written
 *   ws, ws_bytes    at least spec_attention_workspace_bytes(...) bytes with the
 *                   same R, k, Hq, Hkv, page_size, max_pages, split_keys;
 *                   256-byte aligned; no initialisation needed
 *   q, caches, out  16-byte aligned
 * Data errors (status word): a row whose tag disagrees with cu_rows is
 * written as zeros (SPECV_STATUS_BAD_TAG; when cu_rows itself is inconsistent
 * the request's rows are not written); a page id outside [0, num_pages) or a
 * context length that is negative or overruns the page-table row makes the
 * request's rows zeros (SPECV_STATUS_BAD_PAGE). No read leaves the pools.
 * Errors: SPECV_EINVAL for bad sizes or layout, NULL or misaligned pointers or a
 * short workspace; SPECV_EUNSUPPORTED for D != 128, page sizes that are not a
 * multiple of 32, or sizes beyond 32-bit grid and index ranges.
 */
size_t spec_attention_workspace_bytes(int R, int k, int Hq, int Hkv, int page_size, int max_pages,
                                      int split_keys);
int spec_attention(int R, int k, int Hq, int Hkv, int D, int page_size, int num_pages, int max_pages,
                   int kv_layout, int split_keys, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* page_table, const int32_t* ctx_len, const int32_t* tags,
                   const int32_t* cu_rows, const int32_t* n_rows, float* out, void* ws, size_t ws_bytes,
                   specv_stream stream);

/* ------------------------------------------------------------------------ */
/* diagnostics                                                               */
/* ------------------------------------------------------------------------ */

/* Message of the last failed call on this host thread ("" if none). */
const char* specv_last_error(void);

/* Read the workspace status word of the last spec_verify / markov_draft /
 * rnn_draft / spec_attention call that used `ws` (synchronises `stream`). */
int specv_read_status(const void* ws, specv_stream stream, uint32_t* status_out);

/* Per-kernel timing with HIP events that the library attaches to each kernel
 * it enqueues (hipExtLaunchKernel). Off by default; meant for benchmarks. This
 * registry is the library's only global mutable state: it is process-wide,
 * guarded by a mutex, and changes no result. A launch made while timing is on
 * from one host thread is recorded with the others. specv_timing_read
 * synchronises the recorded events and returns the number of launches and
 * their summed duration for kernels whose name starts with `prefix`. */
int specv_timing_enable(int on);
int specv_timing_reset(void);
int specv_timing_read(const char* prefix, int* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* SPECV_H */
