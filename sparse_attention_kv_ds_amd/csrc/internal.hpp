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
// largest candidate union the decode merge holds in registers (64 per thread)
constexpr int kDecodeUnion = 16384;
// most decode partitions: each lists at least 16 candidates
constexpr int kDecodeMaxParts = kDecodeUnion / 16;

bool scorer_supported(int H, int D, int dtype);

// Scores of every token with more than min_rows visible rows, written to
// S[t * ldS + j] for j < n_t (other entries untouched).
hipError_t launch_prefill_scorer(const Problem &p, int min_rows, float *S, long long ldS,
                                 hipStream_t st);

// Same for a single token (T == 1): one work-group per kDecodePart-row
// partition streams K; writes S[j] for j < n.
hipError_t launch_decode_scorer(const Problem &p, int min_rows, float *S, hipStream_t st);

// Per-token streaming top-k over S rows (one wave per token); skip path for
// tokens whose visible rows all fit.
hipError_t launch_topk_stream(const float *S, long long ldS, const int32_t *pos, int T, int N,
                              int ratio, int topk, int32_t *out, hipStream_t st);

// Single-token selection over S[0..n): each kDecodePart-row partition lists
// its exact best kp keys (in row order) in cand[p*kp ..], their number in
// pcount[p] and the smallest of them in pmin[p] (0 when the partition's rows
// all fit); one work-group then merges the lists into the exact top-k (with an
// exact re-stream of S for partitions whose list may be short).  kp is a power
// of two, ceil(N / kDecodePart) * kp <= kDecodeUnion.
hipError_t launch_decode_select(const float *S, const int32_t *pos, int N, int ratio, int topk,
                                int kp, uint64_t *cand, int *pcount, uint64_t *pmin, int32_t *out,
                                hipStream_t st);

// p[0..n) = v
hipError_t launch_fill(float *p, long long n, float v, hipStream_t st);

} // namespace dsi
