// internal.hpp -- host-side launchers of the indexer kernels (not part of the C ABI).
// Declarations only, on the HIP runtime API types, so that the argument
// checks of api.cpp also build with a plain host C++ compiler.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace dsi {

// element types of q and k (the DS_F16 / DS_BF16 codes of the C ABI)
constexpr int kF16 = 1;
constexpr int kBF16 = 2;

constexpr int kPrefillWaves = 4; // waves per prefill scorer work-group

// The (head count, head dim, dtype) combinations the scorer kernels are built for.
inline bool scorer_supported(int H, int D, int dtype)
{
    const bool h = H == 4 || H == 8 || H == 16 || H == 32 || H == 64;
    const bool d = D == 32 || D == 64 || D == 128;
    return h && d && (dtype == kF16 || dtype == kBF16);
}

// Row counts whose byte ranges fit the 32-bit buffer resources of the scorer
// and the per-token top-k: the whole of K (rows * D * 2 bytes, plus the
// 64-row stage past the end that reads as 0), and one work-group's tile of
// score rows ((64 / H) * kPrefillWaves tokens of round_up(rows, 64) floats),
// which must stay below 2^31 bytes so that the masked-store offset 2^31 lies
// outside every such range.
inline bool scorer_rows_supported(int H, int D, int64_t rows)
{
    const int64_t lim = (int64_t)1 << 31;
    if (H < 1 || D < 1 || rows < 0 || rows > lim)
        return false;
    const int64_t ld = (rows + 63) / 64 * 64;
    const int64_t tile_tokens = (int64_t)(64 / H) * kPrefillWaves;
    return (ld + 64) * D * 2 < lim && tile_tokens * ld * 4 < lim;
}

// q[T][O] = round(x[T][K] . wq[O][K]^T): the shapes the projection kernel takes.
inline bool qproj_supported(int K, int O, int dtype)
{
    return K >= 8 && K % 8 == 0 && O % 128 == 0 && (dtype == kF16 || dtype == kBF16);
}

// Optional kernel timing.  When `start` / `stop` are set, the first kernel of
// a launcher call records `start` as it begins and the last records `stop` as
// it ends, from the kernels' own dispatch (no extra marker on the stream);
// `started` / `stopped` tell whether that happened (no kernel may run).
struct Timing {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
    bool started = false;
    bool stopped = false;
};

struct Problem {
    const void *q;       // [T][H][D] raw fp16/bf16 bits
    const void *k;       // [N][D]
    const float *w;      // [T][H]
    const int32_t *pos;  // [T]
    int T, N, ratio, H, D, dtype;
};

// Phase timestamps (builds with DSI_STAMPS only): records of 8 entries of the
// 100 MHz real-time counter, one array per kernel family, kStampRecords
// records each (record = work-group, token or sequence, as the kernel states).
constexpr int kStampRecords = 4096;
enum { kStampDecodeScore = 0, kStampTopk = 1, kStampMerge = 2, kStampAttention = 3, kStampUnits = 4 };
#ifdef DSI_STAMPS
// copy the first `bytes` of one family's array to host memory (synchronous)
hipError_t stamps_read_decode(void *host, size_t bytes);    // scorer.hip
hipError_t stamps_read_topk(void *host, size_t bytes);      // topk.hip
hipError_t stamps_read_merge(void *host, size_t bytes);     // topk.hip
hipError_t stamps_read_attention(void *host, size_t bytes); // attention.hip
#endif

// rows per decode-selection partition (one decode work-group)
constexpr int kDecodePart = 512;
// largest candidate union the decode merge holds in registers (64 per thread)
constexpr int kDecodeUnion = 16384;
// most decode partitions: each lists at least 8 candidates
constexpr int kDecodeMaxParts = kDecodeUnion / 8;
// most sequences of one batched decode call (each owns kDecodeUnion candidate
// slots and kDecodeMaxParts partition entries of the workspace)
constexpr int kDecodeMaxBatch = 64;

// The allocation-free entry point's scratch (static_scratch.hip): one device
// array per GPU holding kStaticScores fp32 score entries (64 MiB), then one
// sequence's partition lists (kDecodeUnion keys, kDecodeMaxParts smallest
// keys and counts).
constexpr long long kStaticScores = 1LL << 24;
constexpr size_t kStaticScratchBytes =
    (size_t)kStaticScores * 4 + (size_t)kDecodeUnion * 8 + (size_t)kDecodeMaxParts * (8 + 4);

// The address of that array on `device`, which must be the current device;
// looked up once per device and kept until the process ends.
hipError_t static_scratch(int device, void **ptr);

// Scores of every token with more than min_rows visible rows, for j < n_t
// (other entries untouched): split == false, fp32 at S[t * ldS + j]; split,
// the split scores of launch_topk_stream in token t's 4 ldS bytes at
// S + t * ldS: row j's high 16 bits of ordered_score(s[t][j]) at byte
// split_hi_off(j), its low 16 bits kSplitLow bytes further on (common.hpp).
hipError_t launch_prefill_scorer(const Problem &p, int min_rows, float *S, long long ldS,
                                 bool split, hipStream_t st, Timing *tm = nullptr);

// Per-partition candidate lists of the single-token selection: partition p
// (rows p * kDecodePart ..) lists its exact best kp keys in row order in
// cand[p * kp ..] (all its rows when they are <= kp, key 0 in unused slots),
// their number in pcount[p] and the smallest listed key in pmin[p] (0 when
// the list holds every row).  kp is a power of two,
// ceil(N / kDecodePart) * kp <= kDecodeUnion.  cand == nullptr: no lists.
struct DecodeLists {
    int kp = 0;
    uint64_t *cand = nullptr;
    int *pcount = nullptr;
    uint64_t *pmin = nullptr;
};

// Batched decode: B sequences of one query token each, sequence b with its
// own q[b] (H x D), K rows k + b * N * D, weights w[b], position pos[b], score
// row S + b * ldS, candidate slots cand + b * kDecodeUnion, partition entries
// pcount/pmin + b * kDecodeMaxParts and output out + b * topk.  B = 1 is the
// single-token call.

// Same for a single token (T == 1): one work-group per kDecodePart-row
// partition streams K; writes S[j] for j < n and, with dl.cand, the
// partition's candidate list.
hipError_t launch_decode_scorer(const Problem &p, int min_rows, float *S, const DecodeLists &dl,
                                hipStream_t st, Timing *tm = nullptr, int B = 1,
                                long long ldS = 0);

// Per-token streaming top-k over the split scores the prefill scorer writes
// (token t's at S16 + 2 t ldS, laid out as launch_prefill_scorer says); one
// wave per token; skip path for tokens whose visible rows all fit.
hipError_t launch_topk_stream(const uint16_t *S16, long long ldS, const int32_t *pos, int T,
                              int N, int ratio, int topk, int32_t *out, hipStream_t st,
                              Timing *tm = nullptr);

// Single-token selection over S[0..n) from the partitions' candidate lists
// (written by launch_decode_scorer): one work-group merges the lists into the
// exact top-k, with an exact re-stream of S for partitions whose list may be
// short.
hipError_t launch_decode_select(const float *S, const int32_t *pos, int N, int ratio, int topk,
                                const DecodeLists &dl, int32_t *out, hipStream_t st,
                                Timing *tm = nullptr, int B = 1, long long ldS = 0);

// Every token's rows 0 .. n_t-1, then -1, in out[T][topk] (for N <= topk,
// where every visible row is selected and nothing needs scoring).
hipError_t launch_sequential_rows(const int32_t *pos, int T, int N, int ratio, int topk,
                                  int32_t *out, hipStream_t st, Timing *tm = nullptr);

// q[T][O] = round(x[T][K] . wq[O][K]^T) in dtype (qproj.hip)
hipError_t launch_qproj(const void *x, const void *wq, int T, int K, int O, int dtype, void *q,
                        hipStream_t st, Timing *tm = nullptr);

// p[0..n) = v
hipError_t launch_fill(float *p, long long n, float v, hipStream_t st);

// sparse attention over the selected rows (attention.hip)
constexpr int kAttnMaxTopk = 2048; // index-list entries per token held in LDS

struct AttnProblem {
    const void *q;        // [T][HA][D] raw fp16/bf16 bits
    const void *kp, *vp;  // [N][D] pooled rows
    const void *kl, *vl;  // [L][D] raw rows by absolute position
    const int32_t *idx;   // [T][topk]; unused when ratio > 0
    const int32_t *pos;   // [T]
    int T, N, L, HA, D, topk, window, dtype;
    int ratio;            // > 0: every visible pooled row (list of N entries), idx unused
    float scale;
    float *out;           // [T][HA][D] fp32
};

inline bool attention_supported(int HA, int D, int dtype)
{
    return (HA == 32 || HA == 64 || HA == 128) && (D == 64 || D == 128) &&
           (dtype == kF16 || dtype == kBF16);
}

hipError_t launch_sparse_attention(const AttnProblem &a, hipStream_t st, Timing *tm = nullptr);

} // namespace dsi
