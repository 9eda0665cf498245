/*
 * ds_indexer.h -- C ABI of the MI355X (gfx950) lightning indexer.
 *
 * The lightning indexer of DeepSeek V4 sparse attention scores every query
 * token against the compressed KV rows it can see and keeps the best rows per
 * token (top 512 in the model) for the sparse attention that follows ("How I
 * made DeepSeek 12x faster on a Mac Studio", section "1: the kernels").
 *
 * For a query token t at absolute position pos[t], with compression ratio r:
 *
 *   n_t     = clamp(floor((pos[t] + 1) / r), 0, N)      rows 0..n_t-1 are visible
 *                                                       (row j covers raw tokens
 *                                                       r*j .. r*j+r-1)
 *   s[t,j]  = sum_h  w[t,h] * max(0, q[t,h,:] . k[j,:])  for j < n_t
 *   out[t]  = the min(n_t, topk) rows with the largest s[t,j] (among equal
 *             scores the lower row wins), listed in ascending row order and
 *             padded with -1 up to topk entries.
 *
 * A token whose visible rows all fit (n_t <= topk) gets 0 .. n_t-1 without any
 * scoring ("How I turned one oversized DeepSeek optimization into three merged
 * oMLX PRs", section "3. Do not rank candidates when every candidate wins").
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers on the handle's device, dense and
 *     row-major, owned by the caller; the library never frees or retains them
 *     beyond the call.  q and k must be 16-byte aligned; w, pos, out, scores
 *     4-byte aligned.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting: the caller keeps every buffer alive and
 *     unmodified until the stream reaches that point.  No host synchronisation
 *     happens inside a call.  A call enqueues kernel launches only (no
 *     allocation, copy or memset on the stream), so the compute calls can be
 *     captured into a HIP graph and replayed (with kernel timing off).
 *   - A handle owns device scratch (the score matrix and selection candidates);
 *     two calls on one handle must not run concurrently (use one handle per
 *     concurrently used stream).
 *   - Errors are returned as status codes (no exceptions, no abort).  Argument
 *     errors are detected on the host before anything is launched, and leave
 *     the outputs untouched.  Positions are device data and are not checked:
 *     the clamp above defines every value (negative => nothing visible).
 *   - Inputs are assumed finite; for non-finite q, k or w the output is
 *     unspecified (but the call stays in bounds and terminates).
 *   - Debugging: with DS_INDEXER_DEBUG set in the environment (to anything
 *     but "" or "0"; read at every launch), each kernel launch is followed by
 *     a synchronisation of the call's stream, so that a failing kernel makes
 *     the call that launched it return DS_ERR_HIP.  That blocks the host
 *     inside the call and is not allowed under stream capture: tests and
 *     debugging only.
 */
#ifndef DS_INDEXER_H
#define DS_INDEXER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ds_indexer ds_indexer;

/* element types of q and k */
enum { DS_F16 = 1, DS_BF16 = 2 };

/* status codes */
enum {
    DS_OK = 0,
    DS_ERR_INVALID_ARG = -1, /* null / misaligned pointer, negative size, topk < 1, ... */
    DS_ERR_UNSUPPORTED = -2, /* head count / head dim / dtype combination not compiled  */
    DS_ERR_CAPACITY = -3,    /* T, N or topk above what the handle was created for      */
    DS_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed              */
    DS_ERR_OOM = -5          /* device scratch could not be allocated                   */
};

/*
 * Create a handle for one device and one problem family.
 *
 *   out        receives the handle (set to NULL on failure)
 *   device     HIP device ordinal
 *   n_heads    index heads H: 4, 8, 16, 32 or 64
 *   head_dim   D: 32, 64 or 128
 *   dtype      DS_F16 or DS_BF16 (type of q and k)
 *   max_topk   largest topk any call will ask for (1 .. 2048)
 *   max_tokens largest T of any call (>= 1)
 *   max_rows   largest N of any call (>= 1)
 *
 * The kernels address K and one work-group's tile of scores through 32-bit
 * byte ranges, so max_rows must satisfy
 *   (round_up(max_rows, 64) + 64) * head_dim * 2          < 2^31  and
 *   (64 / n_heads) * 4 * round_up(max_rows, 64) * 4       < 2^31
 * (at most 8,388,480 rows at head_dim 128), else DS_ERR_UNSUPPORTED;
 * argument, support and range checks all happen before any HIP call.
 * Allocates max_tokens * round_up(max_rows, 64) * 4 bytes of score scratch
 * plus a few MiB of selection scratch on `device`.  Returns DS_OK,
 * DS_ERR_INVALID_ARG, DS_ERR_UNSUPPORTED, DS_ERR_OOM or DS_ERR_HIP.
 */
int ds_indexer_create(ds_indexer **out, int device, int n_heads, int head_dim, int dtype,
                      int max_topk, int64_t max_tokens, int64_t max_rows);

/*
 * Score and select (the operation defined at the top of this file).
 *
 *   q      [T][H][D]  dtype   query of every index head of every token
 *   k      [N][D]     dtype   compressed KV rows, shared by all index heads
 *   w      [T][H]     float32 per-token head weights
 *   pos    [T]        int32   absolute position of each query token
 *   T, N              number of tokens / rows (0 allowed; N = 0 => all -1)
 *   ratio             compression ratio r >= 1
 *   topk              rows kept per token, 1 <= topk <= max_topk
 *   out    [T][topk]  int32   result: ascending selected rows, then -1
 *   stream            hipStream_t to enqueue on (NULL = null stream)
 *
 * T == 1 uses the single-token decode kernels (K streamed once across the
 * whole GPU, multi-work-group selection); T > 1 uses the prefill kernels.
 * When N <= topk every visible row of every token is selected: the call then
 * writes each token's rows 0 .. n_t-1 (then -1) and launches no scorer ("How
 * I turned one oversized DeepSeek optimization into three merged oMLX PRs",
 * section "3. Do not rank candidates when every candidate wins", decided here
 * from N alone, on the host, with no synchronisation).
 * Returns DS_OK, DS_ERR_INVALID_ARG, DS_ERR_CAPACITY or DS_ERR_HIP.
 */
int ds_indexer_score_topk(ds_indexer *ix, const void *q, const void *k, const float *w,
                          const int32_t *pos, int64_t T, int64_t N, int ratio, int topk,
                          int32_t *out, void *stream);

/*
 * ds_indexer_score_topk without a handle and without allocating anything, for
 * callers that cannot allocate device memory: work captured into a HIP graph,
 * tight serving loops, harnesses that forbid hipMalloc.  Same operation,
 * arguments, layout, kernels and results as ds_indexer_score_topk; the head
 * count, head dim and dtype come as arguments (n_heads, head_dim, dtype as in
 * ds_indexer_create) and the call runs on the CURRENT HIP device, where every
 * pointer must live.
 *
 * Its scratch is one fixed device array per GPU (in the library, held from the
 * first call on that GPU until the process ends): 16,777,216 fp32 score
 * entries (64 MiB) plus one sequence's selection lists (152 KiB).  Limits:
 *   topk <= 2048, T <= INT_MAX, and, unless N <= topk or the single-token
 *   path applies (T == 1 and N <= 1048576), T * round_up(N, 64) <= 16777216
 *   (e.g. 2048 tokens x 8192 rows); beyond them DS_ERR_CAPACITY.
 * Every call on one GPU uses that GPU's one array: calls that overlap on one
 * GPU (two streams, two host threads) race and give wrong results; serialise
 * them.  No kernel reads scratch that the same call did not write first, so
 * nothing is cleared between calls.  No device memory is allocated or freed,
 * and no host synchronisation happens.
 * Returns DS_OK, DS_ERR_INVALID_ARG, DS_ERR_UNSUPPORTED (heads, dim, dtype or
 * rows outside the ranges ds_indexer_create accepts), DS_ERR_CAPACITY or
 * DS_ERR_HIP.
 */
int ds_indexer_score_topk_noalloc(const void *q, const void *k, const float *w,
                                  const int32_t *pos, int64_t T, int64_t N, int n_heads,
                                  int head_dim, int dtype, int ratio, int topk, int32_t *out,
                                  void *stream);

/*
 * Batched decode: B independent sequences of one query token each, in one
 * call -- the single-token path (T == 1) for every sequence at once, so that
 * several sequences share one K stream across the GPU.  Each sequence's result
 * is exactly what ds_indexer_score_topk gives it alone (same rule as "How I
 * made DeepSeek 12x faster on a Mac Studio", section "1: the kernels").
 *
 *   q      [B][H][D]  dtype     one query token per sequence
 *   k      [B][N][D]  dtype     sequence b's compressed rows at k + b*N*D
 *   w      [B][H]     float32
 *   pos    [B]        int32     each sequence's token position
 *   out    [B][topk]  int32     result per sequence (ascending rows, then -1)
 *   B      0 <= B <= min(max_tokens, 64); N <= max_rows; other arguments,
 *          alignment, ownership and asynchrony as ds_indexer_score_topk
 * The handle must allow the single-token path (max_rows <= 1048576), else
 * DS_ERR_UNSUPPORTED.  Uses the handle's workspace, so calls on one handle
 * must not overlap (as for every call).  Returns DS_OK, DS_ERR_INVALID_ARG,
 * DS_ERR_CAPACITY (B, N or topk above the handle's limits),
 * DS_ERR_UNSUPPORTED or DS_ERR_HIP.
 */
int ds_indexer_score_topk_batch(ds_indexer *ix, const void *q, const void *k, const float *w,
                                const int32_t *pos, int64_t B, int64_t N, int ratio, int topk,
                                int32_t *out, void *stream);

/*
 * The indexer's query projection, the step just before the scorer ("How I
 * made DeepSeek 12x faster on a Mac Studio" names the big Q projection ahead
 * of the indexer; its weights are a model parameter):
 *   q[t][h*D + d] = round( sum_i x[t][i] * wq[h*D + d][i] )
 * fp32 sums on the matrix cores, rounded once to nearest even into the
 * handle's dtype, i.e. q in the [T][H][D] layout ds_indexer_score_topk reads.
 *
 *   x   [T][d_in]       dtype   each token's query input, device
 *   wq  [H*D][d_in]     dtype   weights, the usual [out][in] layout, device
 *   q   [T][H][D]       dtype   result (ds_indexer_project_q), device
 *   d_in a positive multiple of 8; H*D a multiple of 128; T*d_in*2 and
 *   H*D*d_in*2 below 2^31 bytes; x, wq, q 16-byte aligned.
 * Returns DS_OK, DS_ERR_INVALID_ARG, DS_ERR_CAPACITY (T above max_tokens),
 * DS_ERR_UNSUPPORTED (d_in or H*D outside the list) or DS_ERR_HIP.
 */
int ds_indexer_project_q(ds_indexer *ix, const void *x, const void *wq, int64_t T, int64_t d_in,
                         void *q, void *stream);

/*
 * The projection fused ahead of the indexer: ds_indexer_project_q into the
 * handle's own q buffer, then ds_indexer_score_topk on it, in one call (k, w,
 * pos, N, ratio, topk, out as there).  When N <= topk nothing is projected or
 * scored: every visible row is selected ("How I turned one oversized DeepSeek
 * optimization into three merged oMLX PRs", section "3. Do not rank
 * candidates when every candidate wins": the query projection is skipped
 * too).  Errors as the two calls.
 */
int ds_indexer_project_score_topk(ds_indexer *ix, const void *x, const void *wq, const void *k,
                                  const float *w, const int32_t *pos, int64_t T, int64_t N,
                                  int64_t d_in, int ratio, int topk, int32_t *out, void *stream);

/*
 * Release the handle and its device scratch.  NULL is accepted and ignored.
 * Waits for the handle's device to finish outstanding work first.
 */
void ds_indexer_destroy(ds_indexer *ix);

/*
 * Test and inspection helper: the scores s[t,j] themselves, as computed by the
 * same scorer kernels the selection uses.
 *
 *   scores [T][N] float32 (device): s[t,j] for every visible row, -inf for
 *          every row token t cannot see.
 * Other arguments as in ds_indexer_score_topk.  Returns DS_OK,
 * DS_ERR_INVALID_ARG, DS_ERR_CAPACITY or DS_ERR_HIP.
 */
int ds_indexer_scores(ds_indexer *ix, const void *q, const void *k, const float *w,
                      const int32_t *pos, int64_t T, int64_t N, int ratio, float *scores,
                      void *stream);

/*
 * Per-kernel timing, for benchmarks and profiling.  While enabled, every kernel
 * launch a call makes is bracketed by a pair of HIP events recorded on that
 * call's stream, per class:
 *   DS_KERNEL_SCORE          prefill scorer           (T > 1)
 *   DS_KERNEL_SELECT         prefill per-token top-k  (T > 1)
 *   DS_KERNEL_DECODE_SCORE   single-token scorer      (T == 1; it also lists each
 *                            512-row partition's best keys)
 *   DS_KERNEL_DECODE_SELECT  single-token selection   (T == 1; the merge of those lists)
 *   DS_KERNEL_PROJECT        query projection         (ds_indexer_project_*)
 * The pages' own evidence is end-to-end prompt throughput with bracketing
 * controls ("How I turned one oversized DeepSeek optimization into three
 * merged oMLX PRs", section "Turn review feedback into an experiment"); this
 * splits a call's time into its kernels.
 *
 * ds_indexer_timing(ix, enable): enable != 0 starts recording, 0 stops.
 *   Returns DS_OK or DS_ERR_INVALID_ARG (NULL handle).
 * ds_indexer_timing_read(ix, ms, launches): waits for every recorded event,
 *   writes the summed milliseconds and launch counts of each class into
 *   ms[DS_KERNEL_CLASSES] and launches[DS_KERNEL_CLASSES] (host arrays), and
 *   clears the record.  Returns DS_OK, DS_ERR_INVALID_ARG or DS_ERR_HIP.
 */
enum {
    DS_KERNEL_SCORE = 0,
    DS_KERNEL_SELECT = 1,
    DS_KERNEL_DECODE_SCORE = 2,
    DS_KERNEL_DECODE_SELECT = 3,
    DS_KERNEL_PROJECT = 4,
    DS_KERNEL_CLASSES = 5
};

int ds_indexer_timing(ds_indexer *ix, int enable);
int ds_indexer_timing_read(ds_indexer *ix, double *ms, int64_t *launches);

/* Static, human-readable text for a status code (never NULL). */
const char *ds_indexer_status_str(int status);

/*
 * Phase timestamps of the kernels' last launches, for profiling (how long each
 * stage of a kernel takes, per work-group or token).  Only the separate stamps
 * build of the library (libds_indexer_stamps.so, the same sources compiled
 * with DSI_STAMPS) records them; every other build returns DS_ERR_UNSUPPORTED
 * and touches nothing.
 *
 *   unit   which kernel's records:
 *            DS_STAMPS_DECODE_SCORE  decode scorer, record = work-group of 512
 *                                    rows (sequence b's at b * ceil(N / 512)):
 *                                    0 start, 1 query and first K blocks in
 *                                    LDS, 2..5 each wave's last block scored,
 *                                    6 partition list written
 *            DS_STAMPS_TOPK          prefill top-k, record = token: 0 start,
 *                                    1 starting threshold, 2 row streamed,
 *                                    3 final selection, 4 rows written;
 *                                    counts, not times: 5 keys buffered after
 *                                    the stream, 6 streams of the row * 65536
 *                                    + searches run while streaming
 *            DS_STAMPS_MERGE         decode merge, record = sequence: 0 start,
 *                                    1 lists loaded, 2 k-th key of the union,
 *                                    3 exactness checked, 4 rows written
 *                                    (5 instead after an exact re-stream)
 *            DS_STAMPS_ATTENTION     sparse attention, record = token: 0 start,
 *                                    1 first block and query landed, 2 last
 *                                    block done, 3 output stores issued
 *   host   host memory receiving `bytes` bytes: records of 8 uint64 entries,
 *          each a reading of the GPU's 100 MHz real-time counter (entries a
 *          launch did not write keep older values); at most 4096 records
 *   bytes  at most 4096 * 64
 *
 * Synchronous: waits for the device's work to finish, then copies.  Returns
 * DS_ERR_INVALID_ARG for an unknown unit, NULL host or bytes out of range,
 * DS_ERR_HIP if the copy fails.
 */
enum { DS_STAMPS_DECODE_SCORE = 0, DS_STAMPS_TOPK = 1, DS_STAMPS_MERGE = 2,
       DS_STAMPS_ATTENTION = 3 };
int ds_indexer_stamps_read(int unit, void *host, int64_t bytes);

/*
 * Sparse attention over the selected rows: the consumer of the indices.
 *
 * The pages describe it as compressed attention over local key/value state
 * together with pooled (compressed) key/value state, the pooled rows given by
 * indices ("How I turned one oversized DeepSeek optimization into three merged
 * oMLX PRs", section "1. Route ratio-128 prefill through native attention"),
 * and the pooled rows a token attends to are the ones the lightning indexer
 * selected for it ("How I made DeepSeek 12x faster on a Mac Studio", opening
 * of section "1: the kernels").  For token t at position pos[t] and head h:
 *
 *   R(t)     = local rows  max(0, pos[t] - window + 1) .. min(pos[t], L - 1)
 *              (none when pos[t] < 0 or window == 0)
 *            + pooled rows idx[t][e] for every entry with 0 <= idx[t][e] < N
 *   o[t,h,:] = sum over r in R(t) of softmax_r(scale * q[t,h,:] . key_r) * value_r
 *            = 0 when R(t) is empty.
 * Keys and values are shared by all heads.  Entries outside [0, N) are padding
 * (ds_indexer_score_topk writes -1 there); a row listed twice counts twice.
 *
 *   q       [T][n_heads][head_dim]  fp16/bf16 bits (dtype), device
 *   k_pool  [N][head_dim], v_pool [N][head_dim]   pooled rows, device
 *   k_local [L][head_dim], v_local [L][head_dim]  raw rows by absolute position, device
 *   idx     [T][topk] int32, device (e.g. the output of ds_indexer_score_topk)
 *   pos     [T] int32 absolute positions, device
 *   out     [T][n_heads][head_dim] float32, device (written in full)
 *   stream  hipStream_t, NULL = null stream; the call only enqueues work
 * Supported: n_heads in {32, 64, 128}, head_dim in {64, 128}, dtype DS_F16 or
 * DS_BF16, 0 <= topk <= 2048, window >= 0, N * head_dim and L * head_dim below
 * 2^30 elements.  q, k_*, v_* and out 16-byte aligned; idx and pos 4-byte
 * aligned.  The caller owns every buffer and keeps it alive until the stream
 * has run the call; the library keeps no state and allocates nothing.
 *
 * Arithmetic: scores and softmax in float32 (base-2 exponentials), the weights
 * rounded to the value type for the value product (relative rounding of each
 * weight at most 2^-8 for bf16, 2^-11 for fp16), accumulation in float32, so
 * each output differs from exact attention by at most about that fraction of
 * the largest |value| in the token's rows.
 *
 * Returns DS_OK, DS_ERR_INVALID_ARG (a null pointer where one is needed,
 * misalignment, negative sizes, a scale that is not positive and finite),
 * DS_ERR_UNSUPPORTED (head count, head dim, dtype or topk outside the list
 * above) or DS_ERR_HIP (launch failure).  Arguments are checked on the host before any launch;
 * positions and index values are not read on the host.
 */
int ds_sparse_attention(const void *q, const void *k_pool, const void *v_pool,
                        const void *k_local, const void *v_local, const int32_t *idx,
                        const int32_t *pos, int64_t T, int64_t N, int64_t L, int n_heads,
                        int head_dim, int dtype, int topk, int window, float scale, float *out,
                        void *stream);

/*
 * Sparse attention in its all-visible form: every token attends to its local
 * rows (as above) plus every pooled row it can see -- rows 0 .. n_t - 1 with
 * n_t = clamp(floor((pos[t] + 1) / ratio), 0, N), the same causal rule as the
 * indexer -- with no index list.  These are the sequential pooled indices that
 * layers with a large compression ratio (128) attend to without an indexer
 * ("How I turned one oversized DeepSeek optimization into three merged oMLX
 * PRs", section "1. Route ratio-128 prefill through native attention"), and
 * what the indexer's selection reduces to when every row fits (section "3. Do
 * not rank candidates when every candidate wins").
 *
 * Arguments, layout, ownership, arithmetic and errors as ds_sparse_attention,
 * without idx and topk; ratio >= 1 (else DS_ERR_INVALID_ARG) and N <= 2048
 * (else DS_ERR_UNSUPPORTED).
 */
int ds_sparse_attention_all(const void *q, const void *k_pool, const void *v_pool,
                            const void *k_local, const void *v_local, const int32_t *pos,
                            int64_t T, int64_t N, int64_t L, int n_heads, int head_dim, int dtype,
                            int ratio, int window, float scale, float *out, void *stream);

/*
 * One attention step with its selection: ds_indexer_score_topk on the
 * handle (q_index, k_index, w, pos, T, n_index_rows, ratio, topk, writing the
 * token's rows into idx), then ds_sparse_attention over the local rows plus
 * the rows in idx (q, k_pool, v_pool, n_pool_rows, k_local, v_local, L,
 * n_heads, head_dim, window, scale, out), in stream order on `stream`.
 *
 * The indexer's compressed rows and the attention's pooled rows are the same
 * rows of the sequence, kept in two caches.  The call checks that their
 * counts agree (n_index_rows == n_pool_rows) before anything runs, and
 * returns DS_ERR_INVALID_ARG when they have diverged ("How I turned one
 * oversized DeepSeek optimization into three merged oMLX PRs", section "3. Do
 * not rank candidates when every candidate wins": the change that skips the
 * scoring when every pooled row fits in the top-k also checks that the
 * attention's and the indexer's pooled-row counts have not diverged).  When
 * every pooled row fits (n_index_rows <= topk) no query is scored: idx gets
 * each token's sequential rows 0 .. n_t - 1 (-1 padded), as from
 * ds_indexer_score_topk, and the attention reads them.
 *
 *   idx     [T][topk] int32, device: written in full (the selection), then read
 *   out     [T][n_heads][head_dim] float32, device: written in full
 * The attention's q, k_pool, v_pool, k_local and v_local hold elements of the
 * handle's dtype.  Layouts, alignment and ownership of every buffer as in the
 * two calls; the attention's launch is not timed by ds_indexer_timing.
 *
 * Returns DS_OK, DS_ERR_INVALID_ARG (NULL handle, diverged row counts, or any
 * argument either call rejects), DS_ERR_CAPACITY (T, n_index_rows or topk above
 * the handle's capacities), DS_ERR_UNSUPPORTED (an attention shape outside
 * ds_sparse_attention's list) or DS_ERR_HIP.  Every check of both steps is made
 * on the host before the first launch, so a rejected call launches nothing
 * and writes neither idx nor out.
 */
int ds_indexed_sparse_attention(ds_indexer *ix, const void *q_index, const void *k_index,
                                const float *w, const int32_t *pos, int64_t T,
                                int64_t n_index_rows, int ratio, int topk, int32_t *idx,
                                const void *q, const void *k_pool, const void *v_pool,
                                int64_t n_pool_rows, const void *k_local, const void *v_local,
                                int64_t L, int n_heads, int head_dim, int window, float scale,
                                float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DS_INDEXER_H */
