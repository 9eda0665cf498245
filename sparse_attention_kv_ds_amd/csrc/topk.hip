// topk.hip -- per-token top-k selection kernels for gfx950.
//
// Keeps the topk best rows of each token by (score desc, row asc) and writes
// them in ascending row order, padded with -1 ("How I made DeepSeek 12x faster
// on a Mac Studio", section "1: the kernels": a single streaming pass with a
// running 512th-best threshold and atomic-free ballot compaction replaces the
// sort; tokens whose rows all fit get the sequential rows directly as in "How
// I turned one oversized DeepSeek optimization into three merged oMLX PRs",
// section "3. Do not rank candidates when every candidate wins").
//
// Every (score, row) is mapped to a unique 64-bit key (common.hpp), so the
// selected set is unique and no tie handling is needed anywhere.  Candidates
// are appended to an LDS buffer in row order (ballot + mbcnt, no atomics), and
// every compaction preserves that order, so the survivors come out ascending
// without a final sort.  When the buffer fills, a threshold search shrinks it
// and raises the running threshold; the final selection finds the exact k-th
// key: bisection over the score bits until at most 64 candidates remain in the
// boundary band, then one bitonic sort of that band across the lanes of a wave.
#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

#include <type_traits>

namespace dsi {

namespace {

// smallest per-wave buffer (in 64-key slots) for selecting topk from batches
// of `batch` keys: room for topk, a quarter more, and a batch after a shrink
int select_slots(int topk, int batch)
{
    for (int s : {4, 8, 16, 32})
        if (s * 64 >= topk + topk / 4 + batch + 64)
            return s;
    return 64;
}

// scores per lane in flight in the prefill stream, and the keys per batch
// (one room check per batch keeps the appends free of the shrink)
constexpr int kStreamU = 16;
constexpr int kStreamBatch = kStreamU * 64;

// phase timestamps (stamps build only).  Prefill top-k, record = token: 0
// start, 1 starting threshold found, 2 row streamed, 3 final selection done,
// 4 rows written; values: 5 keys buffered at the end of the stream, 6 the
// number of streams of the row (1, or 2 after a restart) times 65536 plus the
// searches run while streaming.  Decode merge, record = sequence: 0 start, 1 lists loaded
// and counted, 2 k-th key of the union found, 3 exactness checked, 4 rows
// written (or 5 after the exact re-stream).
DSI_STAMP_ARRAY(topk_stamps);
DSI_STAMP_ARRAY(merge_stamps);

// ---------------------------------------------------------------------------
// prefill: one wave per token over the high halves of its ordered scores (the
// split scores at S16 + 2 t ldS, rows j < n_t), in batches of 1024 rows; the
// next two batches are always in flight while one is appended.  The keys are
// coarse: (high 16 bits of the ordered score, row).  A coarse key order is
// the score order wherever
// the high halves differ, so the streaming shrinks keep whole high halves and
// only the rows that share the boundary's high half need their low halves
// (WaveSelect::finish_coarse).  A row where that boundary holds more keys
// than the buffer's slack (many equal or nearly equal scores) is streamed
// again with exact keys from both halves.
// ---------------------------------------------------------------------------
// the selection key of (the 32-bit ordered score or its high half, row)
__device__ __forceinline__ uint64_t key_of(uint32_t ord, uint32_t row)
{
    return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - row);
}

template <int MAXS>
__global__ __launch_bounds__(256) void topk_stream_kernel(const uint16_t *__restrict__ S16,
                                                          long long ldS,
                                                          const int32_t *__restrict__ pos, int T,
                                                          int N, int ratio, int topk,
                                                          int32_t *__restrict__ out)
{
    extern __shared__ uint64_t keys_lds[];
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int wpb = blockDim.x >> 6;
    const int t = blockIdx.x * wpb + wave;
    if (t >= T)
        return;
    DSI_STAMP(topk_stamps, t, 0, lane == 0);
    const int n = visible_rows(pos[t], ratio, N);
    int32_t *o = out + (long long)t * topk;
    if (n <= topk) { // all rows fit: the sequential rows, no scoring needed
        for (int i = lane; i < topk; i += 64)
            o[i] = i < n ? i : -1;
        return;
    }
    // the token's split scores (common.hpp)
    const auto rs = make_rsrc(S16 + (long long)t * 2 * ldS,
                              (uint32_t)((n + kSplitRows - 1) / kSplitRows) * 4 * kSplitRows);
    auto hi_off = [](int j) { return split_hi_off((uint32_t)j); };
    auto low_of = [&](uint32_t j) { return buf_load_u16(rs, split_hi_off(j) + kSplitLow); };
    // Starting threshold from a sample of the row (runs of 64 consecutive
    // rows, evenly spaced: 16 runs for rows of 4096 and more, 4 for rows of
    // 1024..4095, none below): a bound L that about r sampled keys reach, r
    // chosen so that about 1.5 k keys of the whole row are expected to reach L
    // -- most of the row is then dropped at the first compare, the buffer
    // rarely fills, and the final search has about 1.5 k keys to look at
    // rather than the whole row.  L is rounded down to a whole high half.  The
    // result does not depend on the estimate: when fewer than k keys of the
    // row reach L, the row is streamed again from threshold 0.
    // The sample's loads go out first, then the row's first U entries per
    // lane, so that the search waits only for the sample.  (The run count is
    // a template constant, so that the loads issue back to back and the
    // search's counts have no bound checks.)
    constexpr int kRunsMax = 16;
    uint32_t shi[kRunsMax];
    auto sample_loads = [&](auto runs_c) {
        constexpr int R = decltype(runs_c)::value;
#pragma unroll
        for (int s = 0; s < R; ++s)
            shi[s] = buf_load_u16(rs, hi_off((int)((long long)s * (n - 64) / (R - 1)) + lane));
    };
    auto sample_bound = [&](auto runs_c) -> uint64_t {
        constexpr int R = decltype(runs_c)::value;
        constexpr int NS = R * 64; // sample size
        uint32_t hi[R], lo[R];
#pragma unroll
        for (int s = 0; s < R; ++s) {
            hi[s] = shi[s];
            lo[s] = 0xFFFFFFFFu - (uint32_t)((int)((long long)s * (n - 64) / (R - 1)) + lane);
        }
        const int r = min(NS, (int)((long long)topk * NS * 3 / (2LL * n)) + 8);
        WaveReduce red;
        const uint64_t L = uniform64(select_bound<R>(hi, lo, R, NS, r, r / 4 + 1, red));
        return L == 1ull ? L : L & 0xFFFFFFFF00000000ull;
    };
    const int runs = n >= 4 * 1024 ? 16 : (n >= 4 * 256 ? 4 : 0);
    if (runs == 16)
        sample_loads(std::integral_constant<int, 16>{});
    else if (runs == 4)
        sample_loads(std::integral_constant<int, 4>{});
    // Each lane loads four consecutive rows' high halves (8 bytes) per load:
    // load u of a batch covers rows 256 u .. 256 u + 255, lane l rows
    // 256 u + 4 l .. + 3.  Two batches are in flight while one is appended
    // (measured against one batch of one row per lane per load: 27.4 -> 25.0
    // us at 32k, 37.7 -> 36.3 at 64k; two rows per lane: 25.4 and 36.6; three
    // batches in flight: slower).
    constexpr int U2 = kStreamU / 4;
    static_assert(kSplitRows == 32, "a lane's four rows share one group");
    const uint32_t lane_off = (uint32_t)(lane >> 3) * 128 + (uint32_t)(lane & 7) * 8;
    auto load_quads = [&](int b0, uint64_t (&dst)[U2]) {
#pragma unroll
        for (int u = 0; u < U2; ++u) {
            const int j = b0 + u * 256 + 4 * lane;
            dst[u] = buf_load_u64(rs, j < n ? (uint32_t)(b0 + u * 256) * 4 + lane_off : kOffNone);
        }
    };
    uint64_t cur[U2], nxt[U2], nx2[U2];
    load_quads(0, cur);
    uint64_t lower = 0;
    if (runs == 16)
        lower = sample_bound(std::integral_constant<int, 16>{});
    else if (runs == 4)
        lower = sample_bound(std::integral_constant<int, 4>{});
    DSI_STAMP(topk_stamps, t, 1, lane == 0);
    WaveSelect<MAXS> sel;
    uint64_t *const kbuf = keys_lds + (size_t)wave * WaveSelect<MAXS>::CAP;
#ifdef DSI_STAMPS
    int streams = 0;
#endif
#pragma unroll 1
    for (;;) {
#ifdef DSI_STAMPS
        ++streams;
#endif
        sel.init(kbuf, topk, lower, kStreamBatch, true);
        load_quads(kStreamBatch, nxt);
#pragma unroll 1
        for (int base = 0; base < n; base += kStreamBatch) {
            load_quads(base + 2 * kStreamBatch, nx2);
            sel.make_room(kStreamBatch);
            if (sel.failed)
                break;
            if (base + kStreamBatch <= n) { // a whole batch of visible rows
#pragma unroll
                for (int u = 0; u < U2; ++u) {
                    const uint32_t j = (uint32_t)(base + u * 256 + 4 * lane);
                    const uint64_t h = cur[u];
                    sel.append4(key_of((uint32_t)h & 0xFFFFu, j), true,
                                key_of((uint32_t)(h >> 16) & 0xFFFFu, j + 1), true,
                                key_of((uint32_t)(h >> 32) & 0xFFFFu, j + 2), true,
                                key_of((uint32_t)(h >> 48), j + 3), true);
                }
            } else {
#pragma unroll
                for (int u = 0; u < U2; ++u) {
                    const int j = base + u * 256 + 4 * lane;
                    const uint64_t h = cur[u];
                    sel.append4(key_of((uint32_t)h & 0xFFFFu, (uint32_t)j), j < n,
                                key_of((uint32_t)(h >> 16) & 0xFFFFu, (uint32_t)j + 1), j + 1 < n,
                                key_of((uint32_t)(h >> 32) & 0xFFFFu, (uint32_t)j + 2), j + 2 < n,
                                key_of((uint32_t)(h >> 48), (uint32_t)j + 3), j + 3 < n);
                }
            }
#pragma unroll
            for (int u = 0; u < U2; ++u) {
                cur[u] = nxt[u];
                nxt[u] = nx2[u];
            }
        }
        // (after a shrink the buffer holds >= k keys; without one it holds
        // every key that reached the starting threshold)
        if (sel.failed || sel.cnt >= topk || lower == 0)
            break;
        lower = 0;
        load_quads(0, cur);
    }
    DSI_STAMP(topk_stamps, t, 2, lane == 0);
    DSI_STAMP_VALUE(topk_stamps, t, 5, lane == 0, sel.cnt);
#ifdef DSI_STAMPS
    DSI_STAMP_VALUE(topk_stamps, t, 6, lane == 0,
                    (long long)(streams + sel.failed) * 65536 + sel.shrinks);
#endif
    if (sel.failed) {
        // too many keys share the boundary's high half: the row again, with
        // exact keys (both halves of every ordered score)
        wave_lds_sync();
        sel.init(kbuf, topk, 0, 64);
#pragma unroll 1
        for (int base = 0; base < n; base += 64) {
            const uint32_t j = (uint32_t)(base + lane);
            const uint32_t off = (int)j < n ? hi_off((int)j) : kOffNone;
            const uint32_t ord = (buf_load_u16(rs, off) << 16) | buf_load_u16(rs, off + kSplitLow);
            sel.push(key_of(ord, j), (int)j < n);
        }
        sel.finish();
        DSI_STAMP(topk_stamps, t, 3, lane == 0);
        for (int i = lane; i < topk; i += 64)
            o[i] = key_row(sel.buf[i]);
    } else {
        sel.finish_coarse(low_of, keys_lds + (size_t)wpb * WaveSelect<MAXS>::CAP + wave * 64, o);
        DSI_STAMP(topk_stamps, t, 3, lane == 0);
    }
    DSI_STAMP(topk_stamps, t, 4, lane == 0);
}

// ---------------------------------------------------------------------------
// decode selection: one work-group merges the partition lists (written by
// the decode scorer, one list per work-group of rows).  With tU the
// k-th best key of their union, the union's top k is the exact answer unless
// some partition listed only part of its rows and its smallest listed key is
// above tU (it may hold unlisted rows above tU).  That case falls back to an
// exact re-stream of those partitions' rows by one wave.
// Union element e sits in slot e / NT of thread e % NT: every load reads
// consecutive keys, and element order is row order.  kp is a power of two.
// ---------------------------------------------------------------------------
// The k-th largest key of the union (MS keys per thread, hi == 0: no key;
// at least k keys) through one histogram of the scores instead of a bisection
// with a barrier per bit: kHistBins bins spread over [min, max] of the high
// words (bin = a monotone function of the score, so higher bins hold larger
// keys), counted with LDS adds; one wave finds the bin that holds the k-th key
// and how many keys lie above it; the keys of that bin (at most 64 of them)
// are ranked one per lane.  Returns 0 when that bin holds more than 64 keys
// (many equal or near-equal scores): the caller then bisects.
constexpr int kHistBins = 2048;

template <int MS, int NW>
__device__ __forceinline__ uint64_t union_kth_hist(const uint32_t (&hi)[MS], const uint32_t (&lo)[MS], int k,
                                   BlockReduce<NW> &br, uint32_t *hist, uint64_t *bc, int *info)
{
    constexpr int NT = NW * 64;
    constexpr int BPL = kHistBins / 64; // bins per lane of the scanning wave
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    for (int i = tid; i < kHistBins; i += NT)
        hist[i] = 0u;
    if (tid == 0)
        info[3] = 0; // keys collected from the boundary bin
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
    for (int s = 0; s < MS; ++s)
        if (hi[s] != 0u) {
            mn = min(mn, hi[s]);
            mx = max(mx, hi[s]);
        }
    br.minmax(mn, mx); // (its barrier also orders the clearing before the adds)
    if (mn >= mx)
        return 0ull;
    const float scale = (float)kHistBins / ((float)(mx - mn) + 1.0f);
    auto bin = [&](uint32_t h) { return min(kHistBins - 1, (int)((float)(h - mn) * scale)); };
#pragma unroll
    for (int s = 0; s < MS; ++s)
        if (hi[s] != 0u)
            atomicAdd(&hist[bin(hi[s])], 1u);
    __syncthreads();
    if (wave == 0) {
        uint32_t cnt[BPL];
        uint32_t sum = 0;
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
            cnt[b] = hist[lane * BPL + b];
            sum += cnt[b];
        }
        // inc = keys in the bins of this lane and all higher lanes
        uint32_t inc = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_down(inc, o);
            if (lane + o < 64)
                inc += y;
        }
        const uint32_t above_lane = inc - sum;
        if (above_lane < (uint32_t)k && (uint32_t)k <= inc) { // exactly one lane
            uint32_t above = above_lane;
            bool found = false;
#pragma unroll
            for (int b = BPL - 1; b >= 0; --b) {
                if (!found && above + cnt[b] >= (uint32_t)k) {
                    info[0] = lane * BPL + b;
                    info[1] = (int)above;
                    info[2] = (int)cnt[b];
                    found = true;
                }
                above += found ? 0u : cnt[b];
            }
        }
    }
    __syncthreads();
    const int bb = info[0], above = info[1], cb = info[2];
    if (cb > 64)
        return 0ull; // (same in every thread)
#pragma unroll
    for (int s = 0; s < MS; ++s)
        if (hi[s] != 0u && bin(hi[s]) == bb)
            bc[atomicAdd(&info[3], 1)] = ((uint64_t)hi[s] << 32) | lo[s];
    __syncthreads();
    if (wave == 0) {
        // the boundary bin's keys in any order; the answer has k - above - 1
        // larger ones among them
        const uint64_t x = lane < cb ? bc[lane] : 0ull;
        const int r = rank_among(bc, cb, x);
        const uint64_t hit = ballot(lane < cb && r == k - above - 1);
        const uint64_t t = readlane64(x, (int)__builtin_ctzll(hit));
        if (lane == 0)
            bc[64] = t;
    }
    __syncthreads();
    return bc[64];
}

template <int MAXS, int MS, int NT>
__global__ __launch_bounds__(NT) void decode_merge_kernel(
    const float *__restrict__ S, const int32_t *__restrict__ pos, int N, int ratio, int topk,
    int kp, const uint64_t *__restrict__ cand, const int *__restrict__ pcount,
    const uint64_t *__restrict__ pmin, int32_t *__restrict__ out, long long ldS)
{
    // sequence blockIdx.x of a batched call (0 for a single token)
    {
        const int sb = blockIdx.x;
        S += sb * ldS;
        pos += sb;
        cand += (size_t)sb * kDecodeUnion;
        pcount += sb * kDecodeMaxParts;
        pmin += sb * kDecodeMaxParts;
        out += (size_t)sb * topk;
    }
    constexpr int NW = NT / 64;
    constexpr int PPT = (kDecodeMaxParts + NT - 1) / NT;
    extern __shared__ uint64_t fb_buf[];
    __shared__ int red[BlockReduce<NW>::kWords];
    __shared__ int tab[MS][NW]; // kept keys per slot and wave
    __shared__ uint32_t hist[kHistBins];
    __shared__ uint64_t bcand[65];
    __shared__ int hinfo[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = wave_id();
    DSI_STAMP(merge_stamps, blockIdx.x, 0, tid == 0);
    const int32_t p0 = pos[0];
    const int Pmax = (N + kDecodePart - 1) / kDecodePart;
    const int Umax = Pmax * kp; // <= MS * NT

    // every load is issued before the visible count is known (one round trip)
    uint64_t key[MS];
#pragma unroll
    for (int s = 0; s < MS; ++s)
        key[s] = s * NT + tid < Umax ? cand[s * NT + tid] : 0ull;
    int my_pc[PPT];
    uint64_t my_pm[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int p = tid + i * NT;
        my_pc[i] = p < Pmax ? pcount[p] : 0;
        my_pm[i] = p < Pmax ? pmin[p] : 0ull;
    }
    const int n = visible_rows(p0, ratio, N);
    if (n <= topk) {
        for (int i = tid; i < topk; i += NT)
            out[i] = i < n ? i : -1;
        return;
    }
    const int P = (n + kDecodePart - 1) / kDecodePart;
    const int U = P * kp;
    uint32_t hi[MS], lo[MS];
    int have = 0;
#pragma unroll
    for (int s = 0; s < MS; ++s) {
        const bool in = s * NT + tid < U && key[s] != 0ull; // (unused list slots hold 0)
        hi[s] = in ? (uint32_t)(key[s] >> 32) : 0u;
        lo[s] = in ? (uint32_t)key[s] : 0u;
        have += in;
    }
    BlockReduce<NW> br{red, &tab[0][0], 0};
    const int total = br.sum(wave_sum(have));
    DSI_STAMP(merge_stamps, blockIdx.x, 1, tid == 0);
    bool fallback = total < topk;
    uint64_t tU = 0;
    if (!fallback) {
        // the k-th key of the union
        tU = union_kth_hist<MS, NW>(hi, lo, topk, br, hist, bcand, hinfo);
        if (tU == 0ull)
            tU = select_bound<MS>(hi, lo, MS, total, topk, 0, br);
        DSI_STAMP(merge_stamps, blockIdx.x, 2, tid == 0);
        bool fail = false;
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = tid + i * NT;
            if (p < P) {
                const int rows = min(kDecodePart, n - p * kDecodePart);
                fail |= my_pc[i] == kp && rows > kp && my_pm[i] > tU;
            }
        }
        fallback = br.sum(popc(ballot(fail))) > 0;
    }
    DSI_STAMP(merge_stamps, blockIdx.x, 3, tid == 0);
    if (!fallback) {
        // output position of a kept key: kept keys of earlier slots, then of
        // earlier waves in its slot, then of lower lanes.  Lane s of each wave
        // handles slot s's counts (one LDS write per wave, one read of the
        // four waves' counts, a scan across the slots), then every lane takes
        // its slots' bases from those lanes.
        static_assert(MS <= 64, "one slot per lane");
        uint64_t m[MS];
        int cnt = 0; // lane s: this wave's kept keys in slot s
#pragma unroll
        for (int s = 0; s < MS; ++s) {
            m[s] = ballot(hi[s] != 0u && (((uint64_t)hi[s] << 32) | lo[s]) >= tU);
            cnt = lane == s ? popc(m[s]) : cnt;
        }
        if (lane < MS)
            tab[lane][wave] = cnt;
        lds_barrier();
        int all = 0, before = 0;
        if (lane < MS) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const int c = tab[lane][w];
                all += c;
                before += w < wave ? c : 0;
            }
        }
        int inc = all; // kept keys of slots 0..lane, all waves
#pragma unroll
        for (int o = 1; o < MS; o <<= 1) {
            const int y = __shfl_up(inc, o);
            if (lane >= o)
                inc += y;
        }
        const int base = inc - all + before; // lane s: first position of slot s in this wave
#pragma unroll
        for (int s = 0; s < MS; ++s)
            if ((m[s] >> lane) & 1)
                out[__builtin_amdgcn_readlane(base, s) + mbcnt(m[s])] =
                    key_row(((uint64_t)hi[s] << 32) | lo[s]);
        DSI_STAMP(merge_stamps, blockIdx.x, 4, tid == 0);
        return;
    }
    // exact fallback: one wave re-streams every partition in row order, the
    // listed keys of partitions whose list is known to be enough and all rows
    // of the others, keeping only keys that can still reach the top k
    if (wave != 0)
        return;
    WaveSelect<MAXS> sel;
    sel.init(fb_buf, topk, tU, 64);
    // one 64-key chunk per step (a single push site keeps the kernel small)
    int p = 0, i = 0;
#pragma unroll 1
    while (p < P) {
        const int r0 = p * kDecodePart;
        const int rows = min(kDecodePart, n - r0);
        const int pc = pcount[p];
        const bool raw = pc == kp && rows > kp && pmin[p] > tU;
        const int len = raw ? rows : pc;
        const bool valid = i + lane < len;
        uint64_t k = 0;
        if (valid)
            k = raw ? make_key(S[r0 + i + lane], (uint32_t)(r0 + i + lane))
                    : cand[(size_t)p * kp + i + lane];
        sel.push(k, valid);
        i += 64;
        if (i >= len) {
            ++p;
            i = 0;
        }
    }
    sel.finish();
    for (int i = lane; i < topk; i += 64)
        out[i] = key_row(sel.buf[i]);
    DSI_STAMP(merge_stamps, blockIdx.x, 5, lane == 0);
}

template <int MAXS>
hipError_t topk_stream_one(const uint16_t *S, long long ldS, const int32_t *pos, int T, int N,
                           int ratio, int topk, int32_t *out, hipStream_t st, Timing *tm)
{
    // waves (tokens) per work-group: 64 KiB of LDS at most
    const int wpb = MAXS >= 64 ? 2 : 4;
    // each wave's key buffer, then 64 keys of scratch per wave
    const size_t lds = (size_t)wpb * (MAXS + 1) * 64 * sizeof(uint64_t);
    return launch_kernel(topk_stream_kernel<MAXS>, dim3((T + wpb - 1) / wpb), dim3(wpb * 64), lds,
                         st, tm, true, true, S, ldS, pos, T, N, ratio, topk, out);
}

template <int MAXS>
hipError_t merge_one(const float *S, const int32_t *pos, int N, int ratio, int topk, int kp,
                     const uint64_t *cand, const int *pcount, const uint64_t *pmin, int32_t *out,
                     hipStream_t st, Timing *tm, int B, long long ldS)
{
    const size_t lds = (size_t)MAXS * 64 * sizeof(uint64_t);
    const long long U = (long long)((N + kDecodePart - 1) / kDecodePart) * kp;
    // four waves: a search step's count and its barrier cost about the same
    // (sixteen waves, or three pivots per barrier, measured slower)
    constexpr int NT = 256;
    if (U <= 16 * NT)
        return launch_kernel(decode_merge_kernel<MAXS, 16, NT>, dim3(B), dim3(NT), lds, st, tm,
                             true, true, S, pos, N, ratio, topk, kp, cand, pcount, pmin, out, ldS);
    return launch_kernel(decode_merge_kernel<MAXS, kDecodeUnion / NT, NT>, dim3(B), dim3(NT), lds,
                         st, tm, true, true, S, pos, N, ratio, topk, kp, cand, pcount, pmin, out,
                         ldS);
}

// ---------------------------------------------------------------------------
// Whole-call skip: when every row of K fits in topk, every token's visible rows
// fit, and the answer is each token's rows 0 .. n_t-1, then -1, with nothing
// scored ("How I turned one oversized DeepSeek optimization into three merged
// oMLX PRs", section "3. Do not rank candidates when every candidate wins").
// One work-group per token.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void sequential_rows_kernel(const int32_t *__restrict__ pos, int T,
                                                              int N, int ratio, int topk,
                                                              int32_t *__restrict__ out)
{
    // one token per work-group: its visible count once, then its row of out,
    // four entries per 16-byte store where the row allows it
    const int t = blockIdx.x;
    if (t >= T)
        return; // (never: the grid is T work-groups)
    const int n = visible_rows(pos[t], ratio, N);
    int32_t *o = out + (long long)t * topk;
    if (topk % 4 == 0 && ((uintptr_t)o & 15) == 0) {
        for (int q4 = threadIdx.x; q4 < topk / 4; q4 += 256) {
            const int e = 4 * q4;
            int4 v;
            v.x = e < n ? e : -1;
            v.y = e + 1 < n ? e + 1 : -1;
            v.z = e + 2 < n ? e + 2 : -1;
            v.w = e + 3 < n ? e + 3 : -1;
            *reinterpret_cast<int4 *>(o + e) = v;
        }
    } else {
        for (int e = threadIdx.x; e < topk; e += 256)
            o[e] = e < n ? e : -1;
    }
}

} // namespace

#ifdef DSI_STAMPS
hipError_t stamps_read_topk(void *host, size_t bytes)
{
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(topk_stamps), bytes, 0, hipMemcpyDeviceToHost);
}

hipError_t stamps_read_merge(void *host, size_t bytes)
{
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(merge_stamps), bytes, 0, hipMemcpyDeviceToHost);
}
#endif

hipError_t launch_sequential_rows(const int32_t *pos, int T, int N, int ratio, int topk,
                                  int32_t *out, hipStream_t st, Timing *tm)
{
    if (T <= 0 || topk <= 0)
        return hipSuccess;
    return launch_kernel(sequential_rows_kernel, dim3((unsigned)T), dim3(256), 0, st, tm, true,
                         true, pos, T, N, ratio, topk, out);
}

hipError_t launch_topk_stream(const uint16_t *S, long long ldS, const int32_t *pos, int T,
                              int N, int ratio, int topk, int32_t *out, hipStream_t st, Timing *tm)
{
    if (T <= 0)
        return hipSuccess;
    switch (select_slots(topk, kStreamBatch)) {
    case 4: return topk_stream_one<4>(S, ldS, pos, T, N, ratio, topk, out, st, tm);
    case 8: return topk_stream_one<8>(S, ldS, pos, T, N, ratio, topk, out, st, tm);
    case 16: return topk_stream_one<16>(S, ldS, pos, T, N, ratio, topk, out, st, tm);
    case 32: return topk_stream_one<32>(S, ldS, pos, T, N, ratio, topk, out, st, tm);
    default: return topk_stream_one<64>(S, ldS, pos, T, N, ratio, topk, out, st, tm);
    }
}

hipError_t launch_decode_select(const float *S, const int32_t *pos, int N, int ratio, int topk,
                                const DecodeLists &dl, int32_t *out, hipStream_t st, Timing *tm,
                                int B, long long ldS)
{
    if (B <= 0)
        return hipSuccess;
    const int kp = dl.kp;
    auto *c = dl.cand;
    auto *pc = dl.pcount;
    auto *pm = dl.pmin;
    switch (select_slots(topk, 64)) {
    case 4: return merge_one<4>(S, pos, N, ratio, topk, kp, c, pc, pm, out, st, tm, B, ldS);
    case 8: return merge_one<8>(S, pos, N, ratio, topk, kp, c, pc, pm, out, st, tm, B, ldS);
    case 16: return merge_one<16>(S, pos, N, ratio, topk, kp, c, pc, pm, out, st, tm, B, ldS);
    case 32: return merge_one<32>(S, pos, N, ratio, topk, kp, c, pc, pm, out, st, tm, B, ldS);
    default: return merge_one<64>(S, pos, N, ratio, topk, kp, c, pc, pm, out, st, tm, B, ldS);
    }
}

} // namespace dsi
