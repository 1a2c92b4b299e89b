// Host-side checks of libspecv's C ABI, built together with the library's
// sources under AddressSanitizer and UndefinedBehaviorSanitizer (host code
// only) by draft_token_verification_flattened_amd/build.py
// (build_sanitized_check). No GPU is needed: every call below is refused by
// the host-side validation before anything is enqueued, except the timing and
// error hooks, which are exercised from several threads at once.
//
// Exit status 0 when every expectation holds; the sanitizers abort on the
// first memory or undefined-behaviour error they find.
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "specv.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "FAILED: %s (last error: %s)\n", what, specv_last_error());
        ++failures;
    }
}

void expect_code(int got, int want, const char* needle, const char* what) {
    const std::string msg = specv_last_error();
    if (got != want || msg.find(needle) == std::string::npos) {
        std::fprintf(stderr, "FAILED: %s: code %d (want %d), message \"%s\" (want \"%s\")\n", what, got, want,
                     msg.c_str(), needle);
        ++failures;
    }
}

// A non-NULL, 256-byte aligned address that validation never dereferences.
void* const FAKE = reinterpret_cast<void*>(uintptr_t(1) << 20);
template <class T>
T* fake(size_t off = 0) {
    return reinterpret_cast<T*>(static_cast<char*>(FAKE) + off);
}

int verify(int mode, int dtype, int R, int k, int V, const void* draft, float tau, void* ws, size_t ws_bytes,
           const float* u = nullptr) {
    return spec_verify(mode, dtype, R, k, V, FAKE, draft, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(),
                       fake<int32_t>(), tau, 7, 0, u, fake<int32_t>(), fake<int32_t>(), nullptr, ws, ws_bytes,
                       nullptr);
}

}  // namespace

int main() {
    // workspace sizes, including sizes whose products overflow 32 bits
    expect(spec_verify_workspace_bytes(256, 5, 151936) > 0, "verify workspace c2");
    expect(spec_verify_workspace_bytes(0, 5, 10) == 0, "verify workspace R = 0");
    expect(spec_verify_workspace_bytes(1 << 20, 32, 1 << 30) > (size_t(1) << 32), "verify workspace 64-bit");
    expect(spec_schedule_workspace_bytes(4000, 5) == 0, "schedule workspace beyond R*k");
    expect(markov_draft_workspace_bytes(512, 5, 151936, 256) > 0, "markov workspace c4");
    expect(rnn_draft_workspace_bytes(1, 0, 10, 4) == 0, "rnn workspace k = 0");
    expect(spec_attention_workspace_bytes(256, 5, 32, 8, 64, 49, 0) > 0, "attention workspace");

    // spec_verify's validation
    const size_t big = size_t(1) << 30;
    expect_code(verify(3, SPECV_BF16, 4, 5, 1024, FAKE, 1.f, FAKE, big), SPECV_EINVAL, "mode", "verify mode");
    expect_code(verify(SPECV_SAMPLE, 9, 4, 5, 1024, FAKE, 1.f, FAKE, big), SPECV_EUNSUPPORTED, "dtype", "dtype");
    expect_code(verify(SPECV_SAMPLE, SPECV_BF16, 0, 5, 1024, FAKE, 1.f, FAKE, big), SPECV_EINVAL, "R >= 1", "R");
    expect_code(verify(SPECV_SAMPLE, SPECV_BF16, 4, 33, 1024, FAKE, 1.f, FAKE, big), SPECV_EINVAL, "k <=", "k");
    expect_code(verify(SPECV_SAMPLE, SPECV_BF16, 4, 5, 1024, nullptr, 1.f, FAKE, big), SPECV_EINVAL, "draft_logits",
                "draft");
    expect_code(verify(SPECV_SAMPLE, SPECV_BF16, 4, 5, 1024, FAKE, 0.f, FAKE, big), SPECV_EINVAL, "temperature",
                "tau 0");
    expect_code(verify(SPECV_SAMPLE, SPECV_BF16, 4, 5, 1024, FAKE, -1.f, FAKE, big), SPECV_EINVAL, "temperature",
                "tau < 0");
    expect_code(verify(SPECV_SAMPLE, SPECV_BF16, 4, 5, 1024, FAKE, 1.f, fake<char>(16), big), SPECV_EINVAL,
                "aligned", "ws alignment");
    expect_code(verify(SPECV_SAMPLE, SPECV_BF16, 4, 5, 1024, FAKE, 1.f, FAKE, 512), SPECV_EINVAL, "workspace",
                "ws size");
    expect_code(verify(SPECV_SAMPLE, SPECV_BF16, 4, 5, 4096 * 2048 + 1, FAKE, 1.f, FAKE, big), SPECV_EUNSUPPORTED,
                "at most 4096 chunks", "chunks");
    expect_code(verify(SPECV_GREEDY, SPECV_BF16, 4, 5, 1024, nullptr, 1.f, FAKE, 16), SPECV_EINVAL, "workspace",
                "greedy without draft");
    expect_code(verify(SPECV_SAMPLE, SPECV_BF16, 1 << 29, 32, 1024, FAKE, 1.f, FAKE, big), SPECV_EINVAL,
                "too large", "R*(k+1) overflow");
    expect_code(spec_verify_noalloc(SPECV_SAMPLE, SPECV_BF16, 4096, 8, 151936, FAKE, FAKE, fake<int32_t>(),
                                    fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), 1.f, 0, 0, nullptr,
                                    fake<int32_t>(), fake<int32_t>(), nullptr, nullptr, nullptr),
                SPECV_EUNSUPPORTED, "scratch", "noalloc beyond its scratch");

    // spec_verify_ex: a job that would overwrite this call's batch
    specv_schedule_job job{};
    job.R = 4; job.k = 5;
    job.conf_logit = fake<float>(); job.pos_temp = fake<float>();
    job.tbl_tokens = fake<int32_t>(); job.tbl_thr = fake<double>();
    job.n_tbl = 4; job.max_len = 5;
    job.len_out = fake<int32_t>(); job.tags_out = fake<int32_t>(256); job.cu_rows_out = fake<int32_t>(512);
    job.n_rows_out = fake<int32_t>(768); job.ws = FAKE; job.ws_bytes = size_t(1) << 20;
    expect_code(spec_verify_ex(SPECV_SAMPLE, SPECV_BF16, 4, 5, 1024, FAKE, FAKE, fake<int32_t>(), fake<int32_t>(256),
                               fake<int32_t>(4096), fake<int32_t>(8192), 1.f, 7, 0, nullptr, fake<int32_t>(),
                               fake<int32_t>(), nullptr, FAKE, big, nullptr, &job, nullptr),
                SPECV_EINVAL, "other than this one", "verify_ex same batch");

    // spec_step: the job's checks, then the verification's, before anything is enqueued
    expect_code(spec_step(nullptr, SPECV_SAMPLE, SPECV_BF16, 1024, FAKE, FAKE, fake<int32_t>(), 1.f, 0, 0, nullptr,
                          fake<int32_t>(), fake<int32_t>(), nullptr, nullptr, FAKE, big, nullptr),
                SPECV_EINVAL, "NULL schedule job", "step without a job");
    specv_schedule_job sj = job;
    sj.max_len = 9;
    expect_code(spec_step(&sj, SPECV_SAMPLE, SPECV_BF16, 1024, FAKE, FAKE, fake<int32_t>(), 1.f, 0, 0, nullptr,
                          fake<int32_t>(), fake<int32_t>(), nullptr, nullptr, FAKE, big, nullptr),
                SPECV_EINVAL, "spec_step (schedule)", "step with a bad job");
    sj.max_len = 5;
    expect_code(spec_step(&sj, SPECV_SAMPLE, SPECV_BF16, 1024, FAKE, FAKE, fake<int32_t>(), 0.f, 0, 0, nullptr,
                          fake<int32_t>(), fake<int32_t>(), nullptr, nullptr, FAKE, big, nullptr),
                SPECV_EINVAL, "temperature", "step with a bad temperature");

    // spec_schedule / spec_flatten
    auto sched = [&](int R, int k, int n, int max_len, void* ws, size_t wsb, const float* z) {
        return spec_schedule(R, k, z, fake<float>(), fake<int32_t>(), fake<double>(), n, max_len, fake<int32_t>(),
                             fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), nullptr, ws, wsb, nullptr);
    };
    expect_code(sched(0, 5, 8, 5, FAKE, 1 << 20, fake<float>()), SPECV_EINVAL, "R >= 1", "schedule R");
    expect_code(sched(4000, 5, 8, 5, FAKE, 1 << 20, fake<float>()), SPECV_EINVAL, "R*k", "schedule R*k");
    expect_code(sched(4, 5, 8, 6, FAKE, 1 << 20, fake<float>()), SPECV_EINVAL, "max_len", "schedule max_len");
    expect_code(sched(4, 5, 65, 5, FAKE, 1 << 20, fake<float>()), SPECV_EINVAL, "n_tbl", "schedule n_tbl");
    expect_code(sched(4, 5, 8, 5, FAKE, 1 << 20, nullptr), SPECV_EINVAL, "NULL", "schedule NULL");
    expect_code(sched(4, 5, 8, 5, fake<char>(8), 1 << 20, fake<float>()), SPECV_EINVAL, "aligned", "schedule ws");
    expect_code(sched(4, 5, 8, 5, FAKE, 64, fake<float>()), SPECV_EINVAL, "workspace", "schedule ws size");
    expect_code(spec_flatten(0, 5, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), nullptr),
                SPECV_EINVAL, "R >= 1", "flatten R");

    // the draft heads
    expect_code(markov_draft(SPECV_SAMPLE, SPECV_BF16, 4, 5, 64, 48, FAKE, FAKE, FAKE, fake<int32_t>(), 1.f, 7, 0,
                             nullptr, fake<int32_t>(), FAKE, nullptr, FAKE, big, nullptr),
                SPECV_EUNSUPPORTED, "d_m", "markov d_m");
    expect_code(markov_draft(SPECV_SAMPLE, SPECV_F32, 4, 5, 64, 4, FAKE, FAKE, FAKE, fake<int32_t>(), 0.f, 7, 0,
                             nullptr, fake<int32_t>(), FAKE, nullptr, FAKE, big, nullptr),
                SPECV_EINVAL, "temperature", "markov tau");
    expect_code(rnn_draft(SPECV_SAMPLE, SPECV_F32, 4, 5, 64, 4, FAKE, FAKE, nullptr, FAKE, fake<int32_t>(), 1.f, 7, 0,
                          nullptr, fake<int32_t>(), FAKE, nullptr, nullptr, FAKE, big, nullptr),
                SPECV_EINVAL, "rec", "rnn rec");

    // spec_attention
    expect_code(spec_attention(4, 5, 30, 8, 128, 64, 100, 50, 0, 0, FAKE, FAKE, FAKE, fake<int32_t>(),
                               fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), fake<float>(),
                               FAKE, big, nullptr),
                SPECV_EINVAL, "dividing", "attention heads");

    // the error message is per host thread; the timing registry is shared and locked
    std::vector<std::thread> th;
    int per_thread_fail[8] = {0};
    for (int t = 0; t < 8; ++t) {
        th.emplace_back([t, &per_thread_fail] {
            for (int i = 0; i < 200; ++i) {
                const int R = (t % 2) ? 0 : 4;
                const int rc = spec_flatten(R, (t % 2) ? 5 : 40, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(),
                                            fake<int32_t>(), nullptr);
                const std::string msg = specv_last_error();
                if (rc != SPECV_EINVAL || msg.find("spec_flatten") == std::string::npos) ++per_thread_fail[t];
                specv_timing_enable(i % 2);
                int n = -1;
                double ms = -1.0;
                if (specv_timing_read("verify", &n, &ms) != SPECV_OK || n != 0 || ms != 0.0) ++per_thread_fail[t];
                specv_timing_reset();
            }
        });
    }
    for (auto& x : th) x.join();
    specv_timing_enable(0);
    for (int t = 0; t < 8; ++t) expect(per_thread_fail[t] == 0, "threads: errors and timing");

    uint32_t st = 0;
    expect_code(specv_read_status(nullptr, nullptr, &st), SPECV_EINVAL, "NULL", "read_status NULL");

#ifdef SPECV_PLANTED_OVERFLOW
    {   // the control build: a heap read one past the end, which AddressSanitizer must stop
        volatile int* p = new int[4];
        const int v = p[4];
        delete[] p;
        std::printf("planted read %d\n", v);
    }
#endif
    if (failures) {
        std::fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    std::printf("abi sanitized check: all expectations hold\n");
    return 0;
}
