// fake_hip.cpp -- host stand-ins for the HIP runtime calls and the kernel
// launchers that api.cpp uses (see fake_hip.hpp).  Device memory is host
// memory that nothing dereferences; launchers only record that they were
// called and with what sizes.
#include "fake_hip.hpp"

#include <hip/hip_runtime_api.h>
#include <stdlib.h>

#include "internal.hpp"

namespace fake {

std::vector<Launch> launches;
size_t alloc_limit = (size_t)1 << 31;
int live_allocations = 0;
int device_count = 1;
bool fail_device_count = false;
bool fail_launches = false;
int scratch_lookups = 0;

void reset()
{
    launches.clear();
    alloc_limit = (size_t)1 << 31;
    device_count = 1;
    fail_device_count = false;
    fail_launches = false;
}

namespace {

int current_device = 0;

hipError_t record(const char *what, long long T, long long N, long long topk, long long B,
                  dsi::Timing *tm)
{
    if (fail_launches)
        return hipErrorLaunchFailure;
    launches.push_back({what, T, N, topk, B, tm != nullptr});
    if (tm) {
        tm->started = tm->start != nullptr;
        tm->stopped = tm->stop != nullptr;
    }
    return hipSuccess;
}

} // namespace
} // namespace fake

extern "C" {

hipError_t hipGetDevice(int *d)
{
    *d = fake::current_device;
    return hipSuccess;
}

hipError_t hipSetDevice(int d)
{
    if (d < 0 || d >= fake::device_count)
        return hipErrorInvalidDevice;
    fake::current_device = d;
    return hipSuccess;
}

hipError_t hipGetDeviceCount(int *n)
{
    if (fake::fail_device_count)
        return hipErrorNoDevice;
    *n = fake::device_count;
    return hipSuccess;
}

hipError_t hipMalloc(void **p, size_t bytes)
{
    *p = nullptr;
    if (bytes > fake::alloc_limit)
        return hipErrorOutOfMemory;
    // (the memory is never touched: reserve address space only)
    *p = aligned_alloc(256, bytes < 256 ? 256 : (bytes + 255) / 256 * 256);
    if (!*p)
        return hipErrorOutOfMemory;
    ++fake::live_allocations;
    return hipSuccess;
}

hipError_t hipFree(void *p)
{
    if (p) {
        free(p);
        --fake::live_allocations;
    }
    return hipSuccess;
}

hipError_t hipGetLastError(void)
{
    return hipSuccess;
}

hipError_t hipDeviceSynchronize(void)
{
    return hipSuccess;
}

hipError_t hipEventCreate(hipEvent_t *e)
{
    *e = reinterpret_cast<hipEvent_t>(new char[16]);
    return hipSuccess;
}

hipError_t hipEventDestroy(hipEvent_t e)
{
    delete[] reinterpret_cast<char *>(e);
    return hipSuccess;
}

hipError_t hipEventSynchronize(hipEvent_t)
{
    return hipSuccess;
}

hipError_t hipEventElapsedTime(float *ms, hipEvent_t, hipEvent_t)
{
    *ms = 0.5f;
    return hipSuccess;
}

} // extern "C"

namespace dsi {

hipError_t launch_prefill_scorer(const Problem &p, int min_rows, float *, long long, bool,
                                 hipStream_t, Timing *tm)
{
    return fake::record("prefill_scorer", p.T, p.N, min_rows, 1, tm);
}

hipError_t launch_decode_scorer(const Problem &p, int min_rows, float *, const DecodeLists &,
                                hipStream_t, Timing *tm, int B, long long)
{
    return fake::record("decode_scorer", p.T, p.N, min_rows, B, tm);
}

hipError_t launch_topk_stream(const uint16_t *, long long, const int32_t *, int T, int N, int,
                              int topk, int32_t *, hipStream_t, Timing *tm)
{
    return fake::record("topk_stream", T, N, topk, 1, tm);
}

hipError_t launch_decode_select(const float *, const int32_t *, int N, int, int topk,
                                const DecodeLists &, int32_t *, hipStream_t, Timing *tm, int B,
                                long long)
{
    return fake::record("decode_select", 1, N, topk, B, tm);
}

hipError_t launch_sequential_rows(const int32_t *, int T, int N, int, int topk, int32_t *,
                                  hipStream_t, Timing *tm)
{
    return fake::record("sequential_rows", T, N, topk, 1, tm);
}

hipError_t launch_qproj(const void *, const void *, int T, int K, int O, int, void *, hipStream_t,
                        Timing *tm)
{
    return fake::record("qproj", T, K, O, 1, tm);
}

hipError_t launch_fill(float *, long long n, float, hipStream_t)
{
    return fake::record("fill", n, 0, 0, 1, nullptr);
}

hipError_t static_scratch(int device, void **ptr)
{
    // (one block the size of the library's array, reserved once)
    static void *block = aligned_alloc(256, (kStaticScratchBytes + 255) / 256 * 256);
    *ptr = nullptr;
    if (device < 0 || device >= fake::device_count || !block)
        return hipErrorInvalidDevice;
    fake::scratch_lookups++;
    *ptr = block;
    return hipSuccess;
}

hipError_t launch_sparse_attention(const AttnProblem &a, hipStream_t, Timing *tm)
{
    return fake::record(a.ratio > 0 ? "sparse_attention_all" : "sparse_attention", a.T, a.N,
                        a.topk, 1, tm);
}

} // namespace dsi
