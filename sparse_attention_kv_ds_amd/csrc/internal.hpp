// internal.hpp -- host-side launchers of the indexer kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsi {

struct Problem {
    const void *q;       // [T][H][D] raw fp16/bf16 bits
    const void *k;       // [N][D]
    const float *w;      // [T][H]
    const int32_t *pos;  // [T]
    int T, N, ratio, H, D, dtype;
};

// rows per decode-selection partition
constexpr int kDecodePart = 1024;
// largest candidate union the decode merge holds in registers (16 per thread)
constexpr int kDecodeUnion = 16384;

bool scorer_supported(int H, int D, int dtype);

// Scores of every token with more than min_rows visible rows, written to
// S[t * ldS + j] for j < n_t (other entries untouched).
hipError_t launch_prefill_scorer(const Problem &p, int min_rows, float *S, long long ldS,
                                 hipStream_t st);

// Same for a single token (T == 1): K streamed across the whole GPU.
hipError_t launch_decode_scorer(const Problem &p, int min_rows, float *S, hipStream_t st);

// Per-token streaming top-k over S rows (one wave per token); skip path for
// tokens whose visible rows all fit.
hipError_t launch_topk_stream(const float *S, long long ldS, const int32_t *pos, int T, int N,
                              int ratio, int topk, int32_t *out, hipStream_t st);

// Single-token selection over S[0..n): per-partition candidates, then one merge.
hipError_t launch_decode_select(const float *S, const int32_t *pos, int N, int ratio, int topk,
                                int kp, uint64_t *cand, int *pcount, uint64_t *pmin,
                                int32_t *out, hipStream_t st);

// p[0..n) = v
hipError_t launch_fill(float *p, long long n, float v, hipStream_t st);

} // namespace dsi
