// api.cpp -- the C ABI of libds_indexer.so: argument checks, device scratch,
// and the choice between the prefill and the single-token decode kernels.
// Every step of the computation runs in the HIP kernels of scorer.hip and
// topk.hip; this file only validates and launches.
#include "ds_indexer.h"
#include "internal.hpp"

#include <hip/hip_runtime_api.h>
#include <limits.h>
#include <new>
#include <stdint.h>
#include <vector>

struct ds_indexer {
    int device;
    int H, D, dtype, max_topk;
    int64_t max_tokens, max_rows;
    long long ldS;     // row stride of the score scratch (floats)
    float *S;          // [max_tokens][ldS] scores
    void *qbuf;        // [max_tokens][H][D] projected queries (ds_indexer_project_score_topk)
    uint64_t *cand;    // [decode_batch][kDecodeUnion] decode partition candidates
    int *pcount;       // [decode_batch][kDecodeMaxParts]
    uint64_t *pmin;    // [decode_batch][kDecodeMaxParts]
    bool decode_ok;    // single-token path available (max_rows small enough)
    int decode_batch;  // sequences per batched decode call: min(max_tokens, kDecodeMaxBatch)
    // per-kernel timing (ds_indexer_timing)
    struct Mark {
        int cls;
        hipEvent_t a, b;
    };
    bool timing = false;
    std::vector<hipEvent_t> spare;
    std::vector<Mark> marks;
};

namespace {

constexpr int kMaxTopk = 2048;
// single-token path: partitions of kDecodePart rows, at least 8 candidates each
constexpr int64_t kDecodeMaxRows = (int64_t)dsi::kDecodeMaxParts * dsi::kDecodePart;

struct DeviceGuard {
    int prev = -1;
    bool ok = false;
    explicit DeviceGuard(int dev)
    {
        if (hipGetDevice(&prev) != hipSuccess)
            return;
        ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard()
    {
        if (ok && prev >= 0)
            (void)hipSetDevice(prev);
    }
};

bool aligned(const void *p, uintptr_t a)
{
    return ((uintptr_t)p % a) == 0;
}

// candidates kept per decode partition (a power of two): at least twice the
// k best spread evenly over the partitions and at least 8, while the union of
// all lists still fits the merge
int decode_kp(int64_t N, int topk)
{
    const int64_t P = (N + dsi::kDecodePart - 1) / dsi::kDecodePart;
    int64_t kp = 8;
    while (kp * P < 2 * (int64_t)topk && kp < dsi::kDecodePart)
        kp *= 2;
    while (kp > 1 && P * kp > dsi::kDecodeUnion)
        kp /= 2;
    return (int)kp;
}

int check_call(const ds_indexer *ix, const void *q, const void *k, const float *w,
               const int32_t *pos, int64_t T, int64_t N, int ratio, const void *out)
{
    if (!ix || T < 0 || N < 0 || ratio < 1)
        return DS_ERR_INVALID_ARG;
    if (T > 0 && (!q || !w || !pos || !out))
        return DS_ERR_INVALID_ARG;
    if (T > 0 && N > 0 && !k)
        return DS_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, 4) || !aligned(pos, 4) ||
        !aligned(out, 4))
        return DS_ERR_INVALID_ARG;
    if (T > ix->max_tokens || N > ix->max_rows)
        return DS_ERR_CAPACITY;
    return DS_OK;
}

hipEvent_t take_event(ds_indexer *ix)
{
    if (!ix->spare.empty()) {
        hipEvent_t e = ix->spare.back();
        ix->spare.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    return hipEventCreate(&e) == hipSuccess ? e : nullptr;
}

// Runs one launch step; while timing is on, its kernels record a pair of
// events of class `cls` from their own dispatch (start of the first kernel,
// end of the last).
template <class F>
hipError_t timed(ds_indexer *ix, int cls, F &&launch)
{
    if (!ix || !ix->timing)
        return launch(nullptr);
    dsi::Timing tm;
    tm.start = take_event(ix);
    tm.stop = take_event(ix);
    if (!tm.start || !tm.stop) {
        if (tm.start)
            ix->spare.push_back(tm.start);
        if (tm.stop)
            ix->spare.push_back(tm.stop);
        return hipErrorOutOfMemory;
    }
    const hipError_t e = launch(&tm);
    if (e == hipSuccess && tm.started && tm.stopped) {
        ix->marks.push_back({cls, tm.start, tm.stop});
    } else { // nothing launched (or a failure): the events were not used
        ix->spare.push_back(tm.start);
        ix->spare.push_back(tm.stop);
    }
    return e;
}

dsi::Problem problem(const ds_indexer *ix, const void *q, const void *k, const float *w,
                     const int32_t *pos, int64_t T, int64_t N, int ratio)
{
    dsi::Problem p;
    p.q = q;
    p.k = k;
    p.w = w;
    p.pos = pos;
    p.T = (int)T;
    p.N = (int)N;
    p.ratio = ratio;
    p.H = ix->H;
    p.D = ix->D;
    p.dtype = ix->dtype;
    return p;
}

// The device scratch one score + top-k call works in: score rows (ldS floats
// per token) and the single-token path's partition lists.
struct Work {
    float *S;
    long long ldS;
    uint64_t *cand;
    int *pcount;
    uint64_t *pmin;
    bool decode_ok; // the single-token kernels may be used (N small enough)
};

// The launches of one score + top-k call whose arguments have been checked
// (T > 0).  ix only carries the per-kernel timing switch (NULL: no timing).
hipError_t launch_score_topk(ds_indexer *ix, const Work &wk, const dsi::Problem &p, int topk,
                             int32_t *out, hipStream_t s)
{
    const int T = p.T, N = p.N;
    if (N <= topk) {
        // every row of K fits in topk, so every token's visible rows do: the
        // sequential rows, with no scorer and no selection launched
        return timed(ix, T == 1 ? DS_KERNEL_DECODE_SELECT : DS_KERNEL_SELECT, [&](dsi::Timing *tm) {
            return dsi::launch_sequential_rows(p.pos, T, N, p.ratio, topk, out, s, tm);
        });
    }
    hipError_t e;
    if (T == 1 && wk.decode_ok) {
        dsi::DecodeLists dl;
        dl.kp = decode_kp(N, topk);
        dl.cand = wk.cand;
        dl.pcount = wk.pcount;
        dl.pmin = wk.pmin;
        e = timed(ix, DS_KERNEL_DECODE_SCORE, [&](dsi::Timing *tm) {
            return dsi::launch_decode_scorer(p, topk, wk.S, dl, s, tm);
        });
        if (e == hipSuccess)
            e = timed(ix, DS_KERNEL_DECODE_SELECT, [&](dsi::Timing *tm) {
                return dsi::launch_decode_select(wk.S, p.pos, N, p.ratio, topk, dl, out, s, tm);
            });
    } else {
        e = timed(ix, DS_KERNEL_SCORE, [&](dsi::Timing *tm) {
            return dsi::launch_prefill_scorer(p, topk, wk.S, wk.ldS, true, s, tm);
        });
        if (e == hipSuccess)
            e = timed(ix, DS_KERNEL_SELECT, [&](dsi::Timing *tm) {
                return dsi::launch_topk_stream(reinterpret_cast<const uint16_t *>(wk.S), wk.ldS,
                                               p.pos, T, N, p.ratio, topk, out, s, tm);
            });
    }
    return e;
}

} // namespace

extern "C" {

int ds_indexer_create(ds_indexer **out, int device, int n_heads, int head_dim, int dtype,
                      int max_topk, int64_t max_tokens, int64_t max_rows)
{
    if (!out)
        return DS_ERR_INVALID_ARG;
    *out = nullptr;
    if (device < 0 || max_topk < 1 || max_topk > kMaxTopk || max_tokens < 1 || max_rows < 1 ||
        max_tokens > INT_MAX || max_rows > INT_MAX - 64)
        return DS_ERR_INVALID_ARG;
    if (!dsi::scorer_supported(n_heads, head_dim, dtype))
        return DS_ERR_UNSUPPORTED;
    // every call's N is at most max_rows, so this bounds the byte ranges of
    // every later call too
    if (!dsi::scorer_rows_supported(n_heads, head_dim, max_rows))
        return DS_ERR_UNSUPPORTED;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess)
        return DS_ERR_HIP;
    if (device >= ndev)
        return DS_ERR_INVALID_ARG;

    DeviceGuard g(device);
    if (!g.ok)
        return DS_ERR_HIP;
    ds_indexer *ix = new (std::nothrow) ds_indexer();
    if (!ix)
        return DS_ERR_OOM;
    ix->device = device;
    ix->H = n_heads;
    ix->D = head_dim;
    ix->dtype = dtype;
    ix->max_topk = max_topk;
    ix->max_tokens = max_tokens;
    ix->max_rows = max_rows;
    ix->ldS = (max_rows + 63) / 64 * 64;
    ix->decode_ok = max_rows <= kDecodeMaxRows;

    const size_t s_bytes = (size_t)max_tokens * (size_t)ix->ldS * sizeof(float);
    ix->decode_batch = (int)(max_tokens < dsi::kDecodeMaxBatch ? max_tokens : dsi::kDecodeMaxBatch);
    const size_t nb = (size_t)ix->decode_batch;
    bool ok = hipMalloc((void **)&ix->S, s_bytes) == hipSuccess &&
              hipMalloc(&ix->qbuf, (size_t)max_tokens * ix->H * ix->D * 2) == hipSuccess;
    if (ok && ix->decode_ok) {
        ok = hipMalloc((void **)&ix->cand, sizeof(uint64_t) * dsi::kDecodeUnion * nb) == hipSuccess &&
             hipMalloc((void **)&ix->pcount, sizeof(int) * dsi::kDecodeMaxParts * nb) == hipSuccess &&
             hipMalloc((void **)&ix->pmin, sizeof(uint64_t) * dsi::kDecodeMaxParts * nb) == hipSuccess;
    }
    if (!ok) {
        // (freeing what was allocated; hipFree(nullptr) is a no-op)
        (void)hipFree(ix->S);
        (void)hipFree(ix->qbuf);
        (void)hipFree(ix->cand);
        (void)hipFree(ix->pcount);
        (void)hipFree(ix->pmin);
        (void)hipGetLastError(); // clear the failed allocation's status
        delete ix;
        return DS_ERR_OOM;
    }
    *out = ix;
    return DS_OK;
}

int ds_indexer_score_topk(ds_indexer *ix, const void *q, const void *k, const float *w,
                          const int32_t *pos, int64_t T, int64_t N, int ratio, int topk,
                          int32_t *out, void *stream)
{
    int st = check_call(ix, q, k, w, pos, T, N, ratio, out);
    if (st != DS_OK)
        return st;
    if (topk < 1)
        return DS_ERR_INVALID_ARG;
    if (topk > ix->max_topk)
        return DS_ERR_CAPACITY;
    if (T == 0)
        return DS_OK;
    DeviceGuard g(ix->device);
    if (!g.ok)
        return DS_ERR_HIP;
    const Work wk{ix->S, ix->ldS, ix->cand, ix->pcount, ix->pmin, ix->decode_ok};
    const hipError_t e = launch_score_topk(ix, wk, problem(ix, q, k, w, pos, T, N, ratio), topk,
                                           out, (hipStream_t)stream);
    return e == hipSuccess ? DS_OK : DS_ERR_HIP;
}

int ds_indexer_score_topk_noalloc(const void *q, const void *k, const float *w,
                                  const int32_t *pos, int64_t T, int64_t N, int n_heads,
                                  int head_dim, int dtype, int ratio, int topk, int32_t *out,
                                  void *stream)
{
    if (T < 0 || N < 0 || ratio < 1 || topk < 1)
        return DS_ERR_INVALID_ARG;
    if (T > 0 && (!q || !w || !pos || !out))
        return DS_ERR_INVALID_ARG;
    if (T > 0 && N > 0 && !k)
        return DS_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, 4) || !aligned(pos, 4) ||
        !aligned(out, 4))
        return DS_ERR_INVALID_ARG;
    if (!dsi::scorer_supported(n_heads, head_dim, dtype))
        return DS_ERR_UNSUPPORTED;
    if (N > INT_MAX - 64 || !dsi::scorer_rows_supported(n_heads, head_dim, N))
        return DS_ERR_UNSUPPORTED;
    // the fixed scratch: score rows for T * round_up(N, 64) <= kStaticScores
    // (the single-token path needs N of them), then the partition lists
    const long long ldS = (N + 63) / 64 * 64;
    const bool decode = T == 1 && N <= kDecodeMaxRows;
    if (topk > kMaxTopk || T > INT_MAX ||
        (N > topk && !decode && T * ldS > dsi::kStaticScores))
        return DS_ERR_CAPACITY;
    if (T == 0)
        return DS_OK;
    int dev = 0;
    void *base = nullptr;
    if (hipGetDevice(&dev) != hipSuccess || dsi::static_scratch(dev, &base) != hipSuccess)
        return DS_ERR_HIP;
    unsigned char *b = static_cast<unsigned char *>(base);
    Work wk;
    wk.S = reinterpret_cast<float *>(b);
    wk.ldS = ldS;
    wk.cand = reinterpret_cast<uint64_t *>(b + dsi::kStaticScores * 4);
    wk.pmin = wk.cand + dsi::kDecodeUnion;
    wk.pcount = reinterpret_cast<int *>(wk.pmin + dsi::kDecodeMaxParts);
    wk.decode_ok = N <= kDecodeMaxRows;
    dsi::Problem p;
    p.q = q;
    p.k = k;
    p.w = w;
    p.pos = pos;
    p.T = (int)T;
    p.N = (int)N;
    p.ratio = ratio;
    p.H = n_heads;
    p.D = head_dim;
    p.dtype = dtype;
    const hipError_t e = launch_score_topk(nullptr, wk, p, topk, out, (hipStream_t)stream);
    return e == hipSuccess ? DS_OK : DS_ERR_HIP;
}

namespace {

// argument checks of the query projection (host only)
int check_project(const ds_indexer *ix, const void *x, const void *wq, int64_t T, int64_t d_in,
                  const void *q)
{
    if (!ix || T < 0 || d_in < 1)
        return DS_ERR_INVALID_ARG;
    if (T > 0 && (!x || !wq || !q))
        return DS_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(q, 16))
        return DS_ERR_INVALID_ARG;
    const int64_t O = (int64_t)ix->H * ix->D;
    if (d_in >= INT_MAX || !dsi::qproj_supported((int)d_in, (int)O, ix->dtype) ||
        T * d_in * 2 >= ((int64_t)1 << 31) || O * d_in * 2 >= ((int64_t)1 << 31) ||
        T * O * 2 >= ((int64_t)1 << 31))
        return DS_ERR_UNSUPPORTED;
    if (T > ix->max_tokens)
        return DS_ERR_CAPACITY;
    return DS_OK;
}

} // namespace

int ds_indexer_project_q(ds_indexer *ix, const void *x, const void *wq, int64_t T, int64_t d_in,
                         void *q, void *stream)
{
    const int st = check_project(ix, x, wq, T, d_in, q);
    if (st != DS_OK)
        return st;
    if (T == 0)
        return DS_OK;
    const int64_t O = (int64_t)ix->H * ix->D;
    DeviceGuard g(ix->device);
    if (!g.ok)
        return DS_ERR_HIP;
    const hipError_t e = timed(ix, DS_KERNEL_PROJECT, [&](dsi::Timing *tm) {
        return dsi::launch_qproj(x, wq, (int)T, (int)d_in, (int)O, ix->dtype, q,
                                 (hipStream_t)stream, tm);
    });
    return e == hipSuccess ? DS_OK : DS_ERR_HIP;
}

int ds_indexer_project_score_topk(ds_indexer *ix, const void *x, const void *wq, const void *k,
                                  const float *w, const int32_t *pos, int64_t T, int64_t N,
                                  int64_t d_in, int ratio, int topk, int32_t *out, void *stream)
{
    if (!ix)
        return DS_ERR_INVALID_ARG;
    // the checks of the scoring call, with the handle's q buffer standing in
    int st = check_call(ix, T > 0 ? ix->qbuf : nullptr, k, w, pos, T, N, ratio, out);
    if (st != DS_OK)
        return st;
    if (topk < 1)
        return DS_ERR_INVALID_ARG;
    if (topk > ix->max_topk)
        return DS_ERR_CAPACITY;
    st = check_project(ix, x, wq, T, d_in, ix->qbuf);
    if (st != DS_OK)
        return st;
    if (N > topk) { // otherwise every visible row is selected: no projection
        st = ds_indexer_project_q(ix, x, wq, T, d_in, ix->qbuf, stream);
        if (st != DS_OK)
            return st;
    }
    return ds_indexer_score_topk(ix, ix->qbuf, k, w, pos, T, N, ratio, topk, out, stream);
}

int ds_indexer_score_topk_batch(ds_indexer *ix, const void *q, const void *k, const float *w,
                                const int32_t *pos, int64_t B, int64_t N, int ratio, int topk,
                                int32_t *out, void *stream)
{
    // B sequences of one query token each: the checks of a call with T = B
    int st = check_call(ix, q, k, w, pos, B, N, ratio, out);
    if (st != DS_OK)
        return st;
    if (topk < 1)
        return DS_ERR_INVALID_ARG;
    if (topk > ix->max_topk || B > ix->decode_batch)
        return DS_ERR_CAPACITY;
    if (!ix->decode_ok)
        return DS_ERR_UNSUPPORTED;
    if (B == 0)
        return DS_OK;
    DeviceGuard g(ix->device);
    if (!g.ok)
        return DS_ERR_HIP;
    hipStream_t s = (hipStream_t)stream;
    const dsi::Problem p = problem(ix, q, k, w, pos, 1, N, ratio);
    hipError_t e;
    if (N <= topk) {
        e = timed(ix, DS_KERNEL_DECODE_SELECT, [&](dsi::Timing *tm) {
            return dsi::launch_sequential_rows(pos, (int)B, (int)N, ratio, topk, out, s, tm);
        });
    } else {
        dsi::DecodeLists dl;
        dl.kp = decode_kp(N, topk);
        dl.cand = ix->cand;
        dl.pcount = ix->pcount;
        dl.pmin = ix->pmin;
        e = timed(ix, DS_KERNEL_DECODE_SCORE, [&](dsi::Timing *tm) {
            return dsi::launch_decode_scorer(p, topk, ix->S, dl, s, tm, (int)B, ix->ldS);
        });
        if (e == hipSuccess)
            e = timed(ix, DS_KERNEL_DECODE_SELECT, [&](dsi::Timing *tm) {
                return dsi::launch_decode_select(ix->S, pos, (int)N, ratio, topk, dl, out, s, tm,
                                                 (int)B, ix->ldS);
            });
    }
    return e == hipSuccess ? DS_OK : DS_ERR_HIP;
}

int ds_indexer_scores(ds_indexer *ix, const void *q, const void *k, const float *w,
                      const int32_t *pos, int64_t T, int64_t N, int ratio, float *scores,
                      void *stream)
{
    int st = check_call(ix, q, k, w, pos, T, N, ratio, scores);
    if (st != DS_OK)
        return st;
    if (T == 0 || N == 0)
        return DS_OK;
    DeviceGuard g(ix->device);
    if (!g.ok)
        return DS_ERR_HIP;
    hipStream_t s = (hipStream_t)stream;
    const dsi::Problem p = problem(ix, q, k, w, pos, T, N, ratio);
    hipError_t e = dsi::launch_fill(scores, T * N, -__builtin_huge_valf(), s);
    if (e == hipSuccess) {
        // (timed like the scorers of a score + top-k call: the decode stream
        // alone, without its partition lists, is measured this way)
        if (T == 1 && ix->decode_ok)
            e = timed(ix, DS_KERNEL_DECODE_SCORE, [&](dsi::Timing *tm) {
                return dsi::launch_decode_scorer(p, 0, scores, dsi::DecodeLists{}, s, tm);
            });
        else
            e = timed(ix, DS_KERNEL_SCORE, [&](dsi::Timing *tm) {
                return dsi::launch_prefill_scorer(p, 0, scores, (long long)N, false, s, tm);
            });
    }
    return e == hipSuccess ? DS_OK : DS_ERR_HIP;
}

int ds_indexer_timing(ds_indexer *ix, int enable)
{
    if (!ix)
        return DS_ERR_INVALID_ARG;
    ix->timing = enable != 0;
    return DS_OK;
}

int ds_indexer_timing_read(ds_indexer *ix, double *ms, int64_t *launches)
{
    if (!ix || !ms || !launches)
        return DS_ERR_INVALID_ARG;
    DeviceGuard g(ix->device);
    if (!g.ok)
        return DS_ERR_HIP;
    for (int c = 0; c < DS_KERNEL_CLASSES; ++c) {
        ms[c] = 0.0;
        launches[c] = 0;
    }
    int st = DS_OK;
    for (const auto &m : ix->marks) {
        float t = 0.f;
        if (hipEventSynchronize(m.b) != hipSuccess || hipEventElapsedTime(&t, m.a, m.b) != hipSuccess)
            st = DS_ERR_HIP;
        ms[m.cls] += t;
        launches[m.cls] += 1;
        ix->spare.push_back(m.a);
        ix->spare.push_back(m.b);
    }
    ix->marks.clear();
    return st;
}

void ds_indexer_destroy(ds_indexer *ix)
{
    if (!ix)
        return;
    {
        DeviceGuard g(ix->device);
        (void)hipDeviceSynchronize();
        for (const auto &m : ix->marks) {
            (void)hipEventDestroy(m.a);
            (void)hipEventDestroy(m.b);
        }
        for (hipEvent_t e : ix->spare)
            (void)hipEventDestroy(e);
        (void)hipFree(ix->S);
        (void)hipFree(ix->qbuf);
        (void)hipFree(ix->cand);
        (void)hipFree(ix->pcount);
        (void)hipFree(ix->pmin);
    }
    delete ix;
}

namespace {

// the argument checks shared by every attention entry point, and the problem
// they describe: ratio == 0 takes the index list idx[T][topk]; ratio > 0
// attends to every visible pooled row (topk == N).  DS_OK with a.T == 0 means
// there is nothing to launch.
int attention_check(const void *q, const void *k_pool, const void *v_pool, const void *k_local,
                    const void *v_local, const int32_t *idx, const int32_t *pos, int64_t T,
                    int64_t N, int64_t L, int n_heads, int head_dim, int dtype, int64_t topk,
                    int ratio, int window, float scale, float *out, dsi::AttnProblem &a)
{
    a.T = 0;
    // the softmax temperature is a positive finite number (the kernel takes
    // each head's maximum on the unscaled scores)
    if (T < 0 || N < 0 || L < 0 || topk < 0 || window < 0 || !(scale > 0.f) || scale > 3.0e38f)
        return DS_ERR_INVALID_ARG;
    if (!dsi::attention_supported(n_heads, head_dim, dtype) || topk > dsi::kAttnMaxTopk)
        return DS_ERR_UNSUPPORTED;
    const int64_t lim = (int64_t)1 << 30;
    if (T > INT_MAX || N * head_dim >= lim || L * head_dim >= lim ||
        T * (int64_t)n_heads * head_dim >= ((int64_t)1 << 40))
        return DS_ERR_UNSUPPORTED;
    if (T == 0)
        return DS_OK; // (a.T == 0: nothing to launch)
    if (!q || !pos || !out || (ratio == 0 && topk > 0 && !idx) ||
        (N > 0 && (!k_pool || !v_pool)) || (L > 0 && (!k_local || !v_local)))
        return DS_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
        !aligned(k_local, 16) || !aligned(v_local, 16) || !aligned(out, 16) ||
        !aligned(idx, 4) || !aligned(pos, 4))
        return DS_ERR_INVALID_ARG;
    a.q = q;
    a.kp = k_pool;
    a.vp = v_pool;
    a.kl = k_local;
    a.vl = v_local;
    a.idx = ratio > 0 ? nullptr : idx;
    a.pos = pos;
    a.T = (int)T;
    a.N = (int)N;
    a.L = (int)L;
    a.HA = n_heads;
    a.D = head_dim;
    a.topk = (int)topk;
    a.ratio = ratio;
    a.window = window;
    a.dtype = dtype;
    a.scale = scale;
    a.out = out;
    return DS_OK;
}

int attention_call(const void *q, const void *k_pool, const void *v_pool, const void *k_local,
                   const void *v_local, const int32_t *idx, const int32_t *pos, int64_t T,
                   int64_t N, int64_t L, int n_heads, int head_dim, int dtype, int64_t topk,
                   int ratio, int window, float scale, float *out, void *stream)
{
    dsi::AttnProblem a;
    const int st = attention_check(q, k_pool, v_pool, k_local, v_local, idx, pos, T, N, L,
                                   n_heads, head_dim, dtype, topk, ratio, window, scale, out, a);
    if (st != DS_OK || a.T == 0)
        return st;
    return dsi::launch_sparse_attention(a, (hipStream_t)stream) == hipSuccess ? DS_OK : DS_ERR_HIP;
}

} // namespace

int ds_sparse_attention(const void *q, const void *k_pool, const void *v_pool,
                        const void *k_local, const void *v_local, const int32_t *idx,
                        const int32_t *pos, int64_t T, int64_t N, int64_t L, int n_heads,
                        int head_dim, int dtype, int topk, int window, float scale, float *out,
                        void *stream)
{
    return attention_call(q, k_pool, v_pool, k_local, v_local, idx, pos, T, N, L, n_heads,
                          head_dim, dtype, topk, 0, window, scale, out, stream);
}

int ds_sparse_attention_all(const void *q, const void *k_pool, const void *v_pool,
                            const void *k_local, const void *v_local, const int32_t *pos,
                            int64_t T, int64_t N, int64_t L, int n_heads, int head_dim, int dtype,
                            int ratio, int window, float scale, float *out, void *stream)
{
    if (ratio < 1)
        return DS_ERR_INVALID_ARG;
    return attention_call(q, k_pool, v_pool, k_local, v_local, nullptr, pos, T, N, L, n_heads,
                          head_dim, dtype, N, ratio, window, scale, out, stream);
}

int ds_indexed_sparse_attention(ds_indexer *ix, const void *q_index, const void *k_index,
                                const float *w, const int32_t *pos, int64_t T,
                                int64_t n_index_rows, int ratio, int topk, int32_t *idx,
                                const void *q, const void *k_pool, const void *v_pool,
                                int64_t n_pool_rows, const void *k_local, const void *v_local,
                                int64_t L, int n_heads, int head_dim, int window, float scale,
                                float *out, void *stream)
{
    if (!ix)
        return DS_ERR_INVALID_ARG;
    // the indexer's compressed rows and the attention's pooled rows are the
    // same rows: counts that differ mean the two caches have diverged
    if (n_index_rows != n_pool_rows)
        return DS_ERR_INVALID_ARG;
    // every check of both steps before anything is launched
    int st = check_call(ix, q_index, k_index, w, pos, T, n_index_rows, ratio, idx);
    if (st != DS_OK)
        return st;
    if (topk < 1)
        return DS_ERR_INVALID_ARG;
    if (topk > ix->max_topk)
        return DS_ERR_CAPACITY;
    dsi::AttnProblem a;
    st = attention_check(q, k_pool, v_pool, k_local, v_local, idx, pos, T, n_pool_rows, L,
                         n_heads, head_dim, ix->dtype, topk, 0, window, scale, out, a);
    if (st != DS_OK)
        return st;
    // the selection (the sequential rows when every pooled row fits), then
    // the attention over it, in stream order
    st = ds_indexer_score_topk(ix, q_index, k_index, w, pos, T, n_index_rows, ratio, topk, idx,
                               stream);
    if (st != DS_OK || a.T == 0)
        return st;
    DeviceGuard g(ix->device);
    if (!g.ok)
        return DS_ERR_HIP;
    return dsi::launch_sparse_attention(a, (hipStream_t)stream) == hipSuccess ? DS_OK : DS_ERR_HIP;
}

int ds_indexer_stamps_read(int unit, void *host, int64_t bytes)
{
#ifdef DSI_STAMPS
    if (unit < 0 || unit >= dsi::kStampUnits || !host || bytes < 0 ||
        bytes > (int64_t)dsi::kStampRecords * 64)
        return DS_ERR_INVALID_ARG;
    if (hipDeviceSynchronize() != hipSuccess)
        return DS_ERR_HIP;
    hipError_t e = hipSuccess;
    switch (unit) {
    case dsi::kStampDecodeScore: e = dsi::stamps_read_decode(host, (size_t)bytes); break;
    case dsi::kStampTopk: e = dsi::stamps_read_topk(host, (size_t)bytes); break;
    case dsi::kStampMerge: e = dsi::stamps_read_merge(host, (size_t)bytes); break;
    default: e = dsi::stamps_read_attention(host, (size_t)bytes); break;
    }
    return e == hipSuccess ? DS_OK : DS_ERR_HIP;
#else
    (void)unit;
    (void)host;
    (void)bytes;
    return DS_ERR_UNSUPPORTED;
#endif
}

const char *ds_indexer_status_str(int status)
{
    switch (status) {
    case DS_OK: return "ok";
    case DS_ERR_INVALID_ARG: return "invalid argument";
    case DS_ERR_UNSUPPORTED: return "unsupported head count / head dim / dtype";
    case DS_ERR_CAPACITY: return "problem larger than the handle's capacity";
    case DS_ERR_HIP: return "HIP runtime error";
    case DS_ERR_OOM: return "out of device memory";
    default: return "unknown status";
    }
}

} // extern "C"
