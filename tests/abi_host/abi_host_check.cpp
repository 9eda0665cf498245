// abi_host_check.cpp -- every status path of the C ABI (include/ds_indexer.h),
// driven on the host: api.cpp is linked against the stand-ins of fake_hip.cpp
// instead of the HIP runtime and the kernels.  For each call the test checks
// the status code the header promises and which launchers ran (none at all
// for a rejected call: argument errors are detected before anything is
// launched).  Built with the address and undefined-behaviour sanitizers by
// tests/test_host_sanitizers.py; prints "abi host checks: N passed" and exits
// 0, or names each failed check and exits 1.
#include <limits.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "ds_indexer.h"
#include "fake_hip.hpp"

namespace {

int failures = 0, passed = 0;

void check(bool ok, const char *what, int line)
{
    if (ok) {
        ++passed;
    } else {
        ++failures;
        printf("FAIL line %d: %s\n", line, what);
    }
}
#define CHECK(cond) check((cond), #cond, __LINE__)

// the launchers called since the last reset, by name
std::vector<std::string> ran()
{
    std::vector<std::string> v;
    for (const auto &l : fake::launches)
        v.push_back(l.what);
    return v;
}

using Names = std::vector<std::string>;

// (stand-in device buffers: host memory the fake launchers never read)
alignas(256) char mem[8][4096];
void *const Q = mem[0], *const K = mem[1];
float *const W = reinterpret_cast<float *>(mem[2]);
int32_t *const POS = reinterpret_cast<int32_t *>(mem[3]);
int32_t *const OUT = reinterpret_cast<int32_t *>(mem[4]);
float *const SC = reinterpret_cast<float *>(mem[5]);
void *const X = mem[6], *const WQ = mem[7];

template <class T>
T *off(T *p, int bytes)
{
    return reinterpret_cast<T *>(reinterpret_cast<char *>(p) + bytes);
}

// a call expected to be rejected with `want` before any launch
#define REJECT(want, call)                                                                        \
    do {                                                                                          \
        fake::launches.clear();                                                                   \
        const int st_ = (call);                                                                   \
        check(st_ == (want), #call " == " #want, __LINE__);                                       \
        check(fake::launches.empty(), #call ": nothing launched", __LINE__);                      \
    } while (0)

// a call expected to succeed with exactly these launchers, in order
#define ACCEPT(names, call)                                                                       \
    do {                                                                                          \
        fake::launches.clear();                                                                   \
        const int st_ = (call);                                                                   \
        check(st_ == DS_OK, #call " == DS_OK", __LINE__);                                         \
        check(ran() == Names names, #call ": launchers " #names, __LINE__);                       \
    } while (0)

void create_checks()
{
    ds_indexer *ix = reinterpret_cast<ds_indexer *>(&ix);
    CHECK(ds_indexer_create(nullptr, 0, 64, 128, DS_F16, 512, 64, 4096) == DS_ERR_INVALID_ARG);
    // arguments
    REJECT(DS_ERR_INVALID_ARG, ds_indexer_create(&ix, -1, 64, 128, DS_F16, 512, 64, 4096));
    CHECK(ix == nullptr); // set to NULL on failure
    REJECT(DS_ERR_INVALID_ARG, ds_indexer_create(&ix, 1, 64, 128, DS_F16, 512, 64, 4096));
    REJECT(DS_ERR_INVALID_ARG, ds_indexer_create(&ix, 0, 64, 128, DS_F16, 0, 64, 4096));
    REJECT(DS_ERR_INVALID_ARG, ds_indexer_create(&ix, 0, 64, 128, DS_F16, 2049, 64, 4096));
    REJECT(DS_ERR_INVALID_ARG, ds_indexer_create(&ix, 0, 64, 128, DS_F16, 512, 0, 4096));
    REJECT(DS_ERR_INVALID_ARG,
           ds_indexer_create(&ix, 0, 64, 128, DS_F16, 512, (int64_t)INT_MAX + 1, 4096));
    REJECT(DS_ERR_INVALID_ARG, ds_indexer_create(&ix, 0, 64, 128, DS_F16, 512, 64, 0));
    REJECT(DS_ERR_INVALID_ARG,
           ds_indexer_create(&ix, 0, 64, 128, DS_F16, 512, 64, (int64_t)INT_MAX - 63));
    // combinations that are not compiled
    REJECT(DS_ERR_UNSUPPORTED, ds_indexer_create(&ix, 0, 48, 128, DS_F16, 512, 64, 4096));
    REJECT(DS_ERR_UNSUPPORTED, ds_indexer_create(&ix, 0, 64, 96, DS_F16, 512, 64, 4096));
    REJECT(DS_ERR_UNSUPPORTED, ds_indexer_create(&ix, 0, 64, 128, 3, 512, 64, 4096));
    // 32-bit byte ranges of the kernels, checked before any HIP call (the
    // device count query would fail here)
    fake::fail_device_count = true;
    REJECT(DS_ERR_UNSUPPORTED, ds_indexer_create(&ix, 0, 64, 128, DS_F16, 512, 1, 8388481));
    REJECT(DS_ERR_UNSUPPORTED, ds_indexer_create(&ix, 0, 4, 32, DS_F16, 512, 1, 8388545));
    REJECT(DS_ERR_UNSUPPORTED, ds_indexer_create(&ix, 0, 64, 32, DS_F16, 512, 1, 33554305));
    REJECT(DS_ERR_UNSUPPORTED, ds_indexer_create(&ix, 0, 8, 128, DS_BF16, 512, 1, 1 << 30));
    REJECT(DS_ERR_HIP, ds_indexer_create(&ix, 0, 64, 128, DS_F16, 512, 64, 4096));
    fake::fail_device_count = false;
    // ... and the largest row counts that fit are accepted
    const int64_t fits[][3] = {{64, 128, 8388480}, {4, 32, 8388544}, {64, 32, 33554304},
                               {4, 128, 8388480}};
    for (const auto &f : fits) {
        const int before = fake::live_allocations;
        CHECK(ds_indexer_create(&ix, 0, (int)f[0], (int)f[1], DS_F16, 512, 1, f[2]) == DS_OK);
        CHECK(ix != nullptr);
        ds_indexer_destroy(ix);
        CHECK(fake::live_allocations == before);
    }
    // device scratch that cannot be allocated: nothing leaks
    const int before = fake::live_allocations;
    fake::alloc_limit = 1 << 16;
    REJECT(DS_ERR_OOM, ds_indexer_create(&ix, 0, 64, 128, DS_F16, 512, 64, 4096));
    CHECK(ix == nullptr);
    CHECK(fake::live_allocations == before);
    fake::alloc_limit = (size_t)1 << 31;
    ds_indexer_destroy(nullptr); // accepted and ignored
}

void score_topk_checks(ds_indexer *ix, ds_indexer *big)
{
    // handle: H 64, D 128, fp16, max_topk 512, max_tokens 64, max_rows 4096
    auto call = [&](ds_indexer *h, const void *q, const void *k, const float *w,
                    const int32_t *pos, int64_t T, int64_t N, int ratio, int topk, int32_t *out) {
        return ds_indexer_score_topk(h, q, k, w, pos, T, N, ratio, topk, out, nullptr);
    };
    REJECT(DS_ERR_INVALID_ARG, call(nullptr, Q, K, W, POS, 4, 4096, 4, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, K, W, POS, -1, 4096, 4, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, K, W, POS, 4, -1, 4, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, K, W, POS, 4, 4096, 0, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, nullptr, K, W, POS, 4, 4096, 4, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, nullptr, W, POS, 4, 4096, 4, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, K, nullptr, POS, 4, 4096, 4, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, K, W, nullptr, 4, 4096, 4, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, K, W, POS, 4, 4096, 4, 512, nullptr));
    REJECT(DS_ERR_INVALID_ARG, call(ix, off(Q, 8), K, W, POS, 4, 4096, 4, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, off(K, 8), W, POS, 4, 4096, 4, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, K, off(W, 2), POS, 4, 4096, 4, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, K, W, off(POS, 2), 4, 4096, 4, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, K, W, POS, 4, 4096, 4, 512, off(OUT, 2)));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, K, W, POS, 4, 4096, 4, 0, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, K, W, POS, 4, 4096, 4, -5, OUT));
    REJECT(DS_ERR_CAPACITY, call(ix, Q, K, W, POS, 65, 4096, 4, 512, OUT));
    REJECT(DS_ERR_CAPACITY, call(ix, Q, K, W, POS, 4, 4097, 4, 512, OUT));
    REJECT(DS_ERR_CAPACITY, call(ix, Q, K, W, POS, 4, 4096, 4, 513, OUT));
    // an argument error is reported before a capacity error
    REJECT(DS_ERR_INVALID_ARG, call(ix, nullptr, K, W, POS, 65, 4096, 4, 512, OUT));
    // nothing to do
    ACCEPT(({}), call(ix, Q, K, W, POS, 0, 4096, 4, 512, OUT));
    ACCEPT(({}), call(ix, nullptr, nullptr, nullptr, nullptr, 0, 0, 4, 512, nullptr));
    // N = 0 (no K needed) and N <= topk: the sequential rows, no scorer
    ACCEPT(({"sequential_rows"}), call(ix, Q, nullptr, W, POS, 4, 0, 4, 512, OUT));
    ACCEPT(({"sequential_rows"}), call(ix, Q, K, W, POS, 4, 512, 4, 512, OUT));
    ACCEPT(({"sequential_rows"}), call(ix, Q, K, W, POS, 1, 7, 1, 7, OUT));
    // one token: the decode kernels; several: the prefill kernels
    ACCEPT(({"decode_scorer", "decode_select"}), call(ix, Q, K, W, POS, 1, 4096, 4, 512, OUT));
    ACCEPT(({"prefill_scorer", "topk_stream"}), call(ix, Q, K, W, POS, 2, 4096, 4, 512, OUT));
    ACCEPT(({"prefill_scorer", "topk_stream"}), call(ix, Q, K, W, POS, 64, 513, 4, 512, OUT));
    CHECK(fake::launches[0].topk == 512); // tokens whose rows all fit are not scored
    // a handle whose rows exceed the decode path's limit scores one token with
    // the prefill kernels
    ACCEPT(({"prefill_scorer", "topk_stream"}),
           call(big, Q, K, W, POS, 1, 2000000, 4, 512, OUT));
    // a failed launch is reported
    fake::fail_launches = true;
    fake::launches.clear();
    CHECK(call(ix, Q, K, W, POS, 2, 4096, 4, 512, OUT) == DS_ERR_HIP);
    fake::fail_launches = false;
}

void batch_checks(ds_indexer *ix, ds_indexer *wide, ds_indexer *big)
{
    auto call = [&](ds_indexer *h, const void *q, const void *k, int64_t B, int64_t N, int topk,
                    int32_t *out) {
        return ds_indexer_score_topk_batch(h, q, k, W, POS, B, N, 4, topk, out, nullptr);
    };
    REJECT(DS_ERR_INVALID_ARG, call(nullptr, Q, K, 2, 4096, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, nullptr, K, 2, 4096, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, K, 2, 4096, 512, nullptr));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, off(K, 4), 2, 4096, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, K, -1, 4096, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, K, 2, 4096, 0, OUT));
    REJECT(DS_ERR_CAPACITY, call(ix, Q, K, 65, 4096, 512, OUT));   // above max_tokens
    REJECT(DS_ERR_CAPACITY, call(wide, Q, K, 65, 4096, 512, OUT)); // above 64 sequences
    REJECT(DS_ERR_CAPACITY, call(ix, Q, K, 2, 4097, 512, OUT));
    REJECT(DS_ERR_CAPACITY, call(ix, Q, K, 2, 4096, 513, OUT));
    REJECT(DS_ERR_UNSUPPORTED, call(big, Q, K, 2, 4096, 512, OUT)); // no decode path
    ACCEPT(({}), call(ix, Q, K, 0, 4096, 512, OUT));
    ACCEPT(({"sequential_rows"}), call(ix, Q, K, 5, 300, 512, OUT));
    ACCEPT(({"decode_scorer", "decode_select"}), call(wide, Q, K, 64, 4096, 512, OUT));
    CHECK(fake::launches.size() == 2 && fake::launches[0].B == 64 && fake::launches[1].B == 64);
}

void scores_checks(ds_indexer *ix, ds_indexer *big)
{
    auto call = [&](ds_indexer *h, const void *q, int64_t T, int64_t N, float *sc) {
        return ds_indexer_scores(h, q, K, W, POS, T, N, 4, sc, nullptr);
    };
    REJECT(DS_ERR_INVALID_ARG, call(nullptr, Q, 4, 4096, SC));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, 4, 4096, nullptr));
    REJECT(DS_ERR_INVALID_ARG, call(ix, Q, 4, 4096, off(SC, 2)));
    REJECT(DS_ERR_INVALID_ARG, call(ix, off(Q, 2), 4, 4096, SC));
    REJECT(DS_ERR_CAPACITY, call(ix, Q, 65, 4096, SC));
    REJECT(DS_ERR_CAPACITY, call(ix, Q, 4, 4097, SC));
    ACCEPT(({}), call(ix, Q, 0, 4096, SC));
    ACCEPT(({}), call(ix, Q, 4, 0, SC));
    ACCEPT(({"fill", "decode_scorer"}), call(ix, Q, 1, 4096, SC));
    CHECK(fake::launches[1].topk == 0); // every visible row scored
    ACCEPT(({"fill", "prefill_scorer"}), call(ix, Q, 4, 100, SC));
    CHECK(fake::launches[1].topk == 0);
    ACCEPT(({"fill", "prefill_scorer"}), call(big, Q, 1, 2000000, SC));
}

void projection_checks(ds_indexer *ix)
{
    auto proj = [&](ds_indexer *h, const void *x, const void *wq, int64_t T, int64_t din,
                    void *q) { return ds_indexer_project_q(h, x, wq, T, din, q, nullptr); };
    REJECT(DS_ERR_INVALID_ARG, proj(nullptr, X, WQ, 4, 1536, Q));
    REJECT(DS_ERR_INVALID_ARG, proj(ix, X, WQ, -1, 1536, Q));
    REJECT(DS_ERR_INVALID_ARG, proj(ix, X, WQ, 4, 0, Q));
    REJECT(DS_ERR_INVALID_ARG, proj(ix, nullptr, WQ, 4, 1536, Q));
    REJECT(DS_ERR_INVALID_ARG, proj(ix, X, nullptr, 4, 1536, Q));
    REJECT(DS_ERR_INVALID_ARG, proj(ix, X, WQ, 4, 1536, nullptr));
    REJECT(DS_ERR_INVALID_ARG, proj(ix, off(X, 8), WQ, 4, 1536, Q));
    REJECT(DS_ERR_INVALID_ARG, proj(ix, X, WQ, 4, 1536, off(Q, 4)));
    REJECT(DS_ERR_UNSUPPORTED, proj(ix, X, WQ, 4, 12, Q));          // d_in not a multiple of 8
    REJECT(DS_ERR_UNSUPPORTED, proj(ix, X, WQ, 64, 1 << 24, Q));    // T * d_in * 2 = 2^31
    REJECT(DS_ERR_UNSUPPORTED, proj(ix, X, WQ, 4, 1 << 17, Q));     // H*D * d_in * 2 = 2^31
    REJECT(DS_ERR_CAPACITY, proj(ix, X, WQ, 65, 1536, Q));
    ACCEPT(({}), proj(ix, X, WQ, 0, 1536, Q));
    ACCEPT(({"qproj"}), proj(ix, X, WQ, 64, 1536, Q));
    CHECK(fake::launches[0].N == 1536 && fake::launches[0].topk == 64 * 128);

    auto fused = [&](const void *x, int64_t T, int64_t N, int64_t din, int topk, int32_t *out) {
        return ds_indexer_project_score_topk(ix, x, WQ, K, W, POS, T, N, din, 4, topk, out,
                                             nullptr);
    };
    REJECT(DS_ERR_INVALID_ARG, ds_indexer_project_score_topk(nullptr, X, WQ, K, W, POS, 4, 4096,
                                                             1536, 4, 512, OUT, nullptr));
    REJECT(DS_ERR_INVALID_ARG, fused(X, 4, 4096, 1536, 512, nullptr));
    REJECT(DS_ERR_INVALID_ARG, fused(X, 4, 4096, 1536, 0, OUT));
    REJECT(DS_ERR_INVALID_ARG, fused(nullptr, 4, 4096, 1536, 512, OUT));
    REJECT(DS_ERR_UNSUPPORTED, fused(X, 4, 4096, 20, 512, OUT));
    REJECT(DS_ERR_CAPACITY, fused(X, 65, 4096, 1536, 512, OUT));
    REJECT(DS_ERR_CAPACITY, fused(X, 4, 4096, 1536, 513, OUT));
    ACCEPT(({"qproj", "prefill_scorer", "topk_stream"}), fused(X, 4, 4096, 1536, 512, OUT));
    // every row fits: neither projected nor scored
    ACCEPT(({"sequential_rows"}), fused(X, 4, 512, 1536, 512, OUT));
}

void timing_checks(ds_indexer *ix)
{
    double ms[DS_KERNEL_CLASSES];
    int64_t n[DS_KERNEL_CLASSES];
    CHECK(ds_indexer_timing(nullptr, 1) == DS_ERR_INVALID_ARG);
    CHECK(ds_indexer_timing_read(nullptr, ms, n) == DS_ERR_INVALID_ARG);
    CHECK(ds_indexer_timing_read(ix, nullptr, n) == DS_ERR_INVALID_ARG);
    CHECK(ds_indexer_timing_read(ix, ms, nullptr) == DS_ERR_INVALID_ARG);
    CHECK(ds_indexer_timing(ix, 1) == DS_OK);
    CHECK(ds_indexer_timing_read(ix, ms, n) == DS_OK);
    fake::launches.clear();
    CHECK(ds_indexer_score_topk(ix, Q, K, W, POS, 4, 4096, 4, 512, OUT, nullptr) == DS_OK);
    CHECK(ds_indexer_score_topk(ix, Q, K, W, POS, 1, 4096, 4, 512, OUT, nullptr) == DS_OK);
    CHECK(ds_indexer_score_topk(ix, Q, K, W, POS, 1, 4096, 4, 512, OUT, nullptr) == DS_OK);
    CHECK(ds_indexer_project_q(ix, X, WQ, 4, 64, Q, nullptr) == DS_OK);
    CHECK(fake::launches.size() == 7);
    bool all_timed = true;
    for (const auto &l : fake::launches)
        all_timed &= l.timed;
    CHECK(all_timed);
    CHECK(ds_indexer_timing_read(ix, ms, n) == DS_OK);
    CHECK(n[DS_KERNEL_SCORE] == 1 && n[DS_KERNEL_SELECT] == 1 && n[DS_KERNEL_DECODE_SCORE] == 2 &&
          n[DS_KERNEL_DECODE_SELECT] == 2 && n[DS_KERNEL_PROJECT] == 1);
    CHECK(ms[DS_KERNEL_DECODE_SCORE] == 1.0);
    CHECK(ds_indexer_timing_read(ix, ms, n) == DS_OK); // the record was cleared
    CHECK(n[DS_KERNEL_SCORE] == 0 && n[DS_KERNEL_DECODE_SCORE] == 0);
    CHECK(ds_indexer_timing(ix, 0) == DS_OK);
    fake::launches.clear();
    CHECK(ds_indexer_score_topk(ix, Q, K, W, POS, 4, 4096, 4, 512, OUT, nullptr) == DS_OK);
    CHECK(fake::launches.size() == 2 && !fake::launches[0].timed && !fake::launches[1].timed);
}

void noalloc_checks()
{
    // no handle: the heads, dim and dtype are arguments; scratch is the fixed array
    auto call = [&](const void *q, const void *k, int64_t T, int64_t N, int H, int D, int dt,
                    int topk, int32_t *out) {
        return ds_indexer_score_topk_noalloc(q, k, W, POS, T, N, H, D, dt, 4, topk, out, nullptr);
    };
    const int allocs = fake::live_allocations;
    REJECT(DS_ERR_INVALID_ARG, call(Q, K, -1, 4096, 64, 128, DS_F16, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(Q, K, 4, -1, 64, 128, DS_F16, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(Q, K, 4, 4096, 64, 128, DS_F16, 0, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(nullptr, K, 4, 4096, 64, 128, DS_F16, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(Q, nullptr, 4, 4096, 64, 128, DS_F16, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(Q, K, 4, 4096, 64, 128, DS_F16, 512, nullptr));
    REJECT(DS_ERR_INVALID_ARG, call(off(Q, 8), K, 4, 4096, 64, 128, DS_F16, 512, OUT));
    REJECT(DS_ERR_INVALID_ARG, call(Q, K, 4, 4096, 64, 128, DS_F16, 512, off(OUT, 2)));
    REJECT(DS_ERR_UNSUPPORTED, call(Q, K, 4, 4096, 48, 128, DS_F16, 512, OUT));
    REJECT(DS_ERR_UNSUPPORTED, call(Q, K, 4, 4096, 64, 128, 9, 512, OUT));
    REJECT(DS_ERR_UNSUPPORTED, call(Q, K, 4, 8388481, 64, 128, DS_F16, 512, OUT));
    REJECT(DS_ERR_CAPACITY, call(Q, K, 4, 4096, 64, 128, DS_F16, 2049, OUT));
    // score rows beyond the fixed 2^24 entries
    REJECT(DS_ERR_CAPACITY, call(Q, K, 2048, 8193, 64, 128, DS_F16, 512, OUT));
    REJECT(DS_ERR_CAPACITY, call(Q, K, 2049, 8192, 64, 128, DS_F16, 512, OUT));
    REJECT(DS_ERR_CAPACITY, call(Q, K, 1, 16777217, 64, 32, DS_F16, 512, OUT));
    ACCEPT(({}), call(Q, K, 0, 4096, 64, 128, DS_F16, 512, OUT));
    ACCEPT(({"prefill_scorer", "topk_stream"}), call(Q, K, 2048, 8192, 64, 128, DS_F16, 512, OUT));
    ACCEPT(({"prefill_scorer", "topk_stream"}), call(Q, K, 4, 4096, 4, 32, DS_BF16, 100, OUT));
    // one token: the decode kernels up to their row limit, the prefill ones beyond
    ACCEPT(({"decode_scorer", "decode_select"}), call(Q, K, 1, 1 << 20, 64, 128, DS_F16, 512, OUT));
    ACCEPT(({"prefill_scorer", "topk_stream"}),
           call(Q, K, 1, (1 << 20) + 1, 64, 128, DS_F16, 512, OUT));
    // every row fits: no scratch needed beyond the limits
    ACCEPT(({"sequential_rows"}), call(Q, K, 100000, 300, 64, 128, DS_F16, 512, OUT));
    CHECK(fake::live_allocations == allocs); // nothing allocated
    CHECK(fake::scratch_lookups > 0);
}

void attention_checks()
{
    auto call = [&](int64_t T, const int32_t *idx, int topk, float scale, float *out) {
        return ds_sparse_attention(Q, K, K, X, X, idx, POS, T, 100, 200, 64, 128, DS_BF16, topk,
                                   16, scale, out, nullptr);
    };
    REJECT(DS_ERR_INVALID_ARG, call(4, OUT, 8, 0.0f, SC));
    REJECT(DS_ERR_INVALID_ARG, call(4, nullptr, 8, 0.1f, SC));
    REJECT(DS_ERR_INVALID_ARG, call(4, OUT, 8, 0.1f, off(SC, 4)));
    REJECT(DS_ERR_UNSUPPORTED, call(4, OUT, 2049, 0.1f, SC));
    ACCEPT(({}), call(0, OUT, 8, 0.1f, SC));
    ACCEPT(({"sparse_attention"}), call(4, OUT, 8, 0.1f, SC));
    REJECT(DS_ERR_INVALID_ARG, ds_sparse_attention_all(Q, K, K, X, X, POS, 4, 100, 200, 64, 128,
                                                       DS_BF16, 0, 16, 0.1f, SC, nullptr));
    REJECT(DS_ERR_UNSUPPORTED, ds_sparse_attention_all(Q, K, K, X, X, POS, 4, 2049, 200, 64, 128,
                                                       DS_BF16, 128, 16, 0.1f, SC, nullptr));
    ACCEPT(({"sparse_attention_all"}),
           ds_sparse_attention_all(Q, K, K, X, X, POS, 4, 100, 200, 64, 128, DS_BF16, 128, 16,
                                   0.1f, SC, nullptr));
}

// the selection plus the attention in one call: the two pooled-row counts
// must agree, and every argument of both steps is checked before the first
// launch
void indexed_attention_checks(ds_indexer *ix)
{
    auto call = [&](int64_t T, int64_t n_index, int64_t n_pool, int topk, int heads, float scale,
                    int32_t *idx, float *out) {
        return ds_indexed_sparse_attention(ix, Q, K, W, POS, T, n_index, 4, topk, idx, X, K, K,
                                           n_pool, X, X, 200, heads, 128, 16, scale, out, nullptr);
    };
    REJECT(DS_ERR_INVALID_ARG, ds_indexed_sparse_attention(nullptr, Q, K, W, POS, 4, 1000, 4, 512,
                                                           OUT, X, K, K, 1000, X, X, 200, 64, 128,
                                                           16, 0.1f, SC, nullptr));
    // diverged pooled-row counts, either way round
    REJECT(DS_ERR_INVALID_ARG, call(4, 1000, 999, 512, 64, 0.1f, OUT, SC));
    REJECT(DS_ERR_INVALID_ARG, call(4, 300, 301, 512, 64, 0.1f, OUT, SC));
    // the indexer's checks
    REJECT(DS_ERR_INVALID_ARG, call(4, 1000, 1000, 0, 64, 0.1f, OUT, SC));
    REJECT(DS_ERR_CAPACITY, call(65, 1000, 1000, 512, 64, 0.1f, OUT, SC));
    REJECT(DS_ERR_CAPACITY, call(4, 4097, 4097, 512, 64, 0.1f, OUT, SC));
    REJECT(DS_ERR_CAPACITY, call(4, 1000, 1000, 513, 64, 0.1f, OUT, SC));
    REJECT(DS_ERR_INVALID_ARG, call(4, 1000, 1000, 512, 64, 0.1f, off(OUT, 2), SC));
    // the attention's checks
    REJECT(DS_ERR_INVALID_ARG, call(4, 1000, 1000, 512, 64, 0.0f, OUT, SC));
    REJECT(DS_ERR_INVALID_ARG, call(4, 1000, 1000, 512, 64, 0.1f, OUT, off(SC, 4)));
    REJECT(DS_ERR_INVALID_ARG, call(4, 1000, 1000, 512, 64, 0.1f, OUT, nullptr));
    REJECT(DS_ERR_UNSUPPORTED, call(4, 1000, 1000, 512, 48, 0.1f, OUT, SC));
    ACCEPT(({}), call(0, 1000, 1000, 512, 64, 0.1f, OUT, SC));
    ACCEPT(({"prefill_scorer", "topk_stream", "sparse_attention"}),
           call(4, 1000, 1000, 512, 64, 0.1f, OUT, SC));
    // every pooled row fits: sequential rows, no scoring, then the attention
    ACCEPT(({"sequential_rows", "sparse_attention"}), call(4, 300, 300, 512, 64, 0.1f, OUT, SC));
    ACCEPT(({"decode_scorer", "decode_select", "sparse_attention"}),
           call(1, 4000, 4000, 512, 64, 0.1f, OUT, SC));
}

} // namespace

int main()
{
    fake::reset();
    create_checks();

    ds_indexer *ix = nullptr, *wide = nullptr, *big = nullptr;
    const int base = fake::live_allocations;
    CHECK(ds_indexer_create(&ix, 0, 64, 128, DS_F16, 512, 64, 4096) == DS_OK);
    CHECK(ds_indexer_create(&wide, 0, 64, 128, DS_F16, 512, 100, 4096) == DS_OK);
    // more rows than the single-token path takes (2048 partitions of 512)
    CHECK(ds_indexer_create(&big, 0, 64, 128, DS_F16, 512, 2, 2000000) == DS_OK);
    if (!ix || !wide || !big) {
        printf("FAIL: handles not created\n");
        return 1;
    }
    score_topk_checks(ix, big);
    batch_checks(ix, wide, big);
    scores_checks(ix, big);
    projection_checks(ix);
    timing_checks(ix);
    noalloc_checks();
    attention_checks();
    indexed_attention_checks(ix);
    ds_indexer_destroy(ix);
    ds_indexer_destroy(wide);
    ds_indexer_destroy(big);
    CHECK(fake::live_allocations == base); // destroy frees all device scratch

    printf("abi host checks: %d passed, %d failed\n", passed, failures);
    return failures ? 1 : 0;
}
