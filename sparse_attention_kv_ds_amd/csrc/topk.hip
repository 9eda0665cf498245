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
#include "internal.hpp"

namespace dsi {

namespace {

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = min(v, (uint32_t)__shfl_xor((int)v, o));
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = max(v, (uint32_t)__shfl_xor((int)v, o));
    return v;
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m)
{
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// (the readlane builtins return int: convert through uint32_t so that the low
// word is never sign-extended into the high one)
__device__ __forceinline__ uint64_t uniform64(uint64_t v)
{
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    return ((uint64_t)hi << 32) | lo;
}

// One key per lane, sorted descending across the wave (bitonic network).
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t key)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint64_t other = shfl_xor64(key, stride);
            const bool lower = (lane & stride) == 0;
            const bool desc = (lane & size) == 0; // direction of this lane's run
            const bool take_max = lower == desc;
            const uint64_t mx = other > key ? other : key;
            const uint64_t mn = other > key ? key : other;
            key = take_max ? mx : mn;
        }
    }
    return key;
}

// ---------------------------------------------------------------------------
// Counting over keys held in registers, split in high/low words; slots at or
// past `nsl` (a uniform bound) are not looked at, and key 0 never counts
// because every candidate value tested is >= 1.
// ---------------------------------------------------------------------------
template <int E>
__device__ __forceinline__ int count_hi_ge(const uint32_t (&hi)[E], int nsl, uint32_t c)
{
    int r = 0;
#pragma unroll
    for (int s = 0; s < E; ++s)
        if (s < nsl)
            r += popc(ballot(hi[s] >= c));
    return r;
}

template <int E>
__device__ __forceinline__ int count_lo_ge(const uint32_t (&hi)[E], const uint32_t (&lo)[E],
                                           int nsl, uint32_t v, uint32_t c)
{
    int r = 0;
#pragma unroll
    for (int s = 0; s < E; ++s)
        if (s < nsl)
            r += popc(ballot(hi[s] == v && lo[s] >= c));
    return r;
}

// ---------------------------------------------------------------------------
// Reductions over the participants of a selection: one wave, or a whole
// work-group.  `band_kth` returns the r-th largest (1-based) of the <= 64 keys
// whose high word lies in [v, u) -- gathered into LDS scratch, sorted by one
// wave, and the answer made visible to every participant.
// ---------------------------------------------------------------------------
struct WaveReduce {
    uint64_t *scratch; // 64 keys of LDS
    __device__ int sum(int wave_count) { return wave_count; }
    __device__ uint32_t umin(uint32_t v) { return wave_min_u32(v); }
    __device__ uint32_t umax(uint32_t v) { return wave_max_u32(v); }

    template <int E>
    __device__ uint64_t band_kth(const uint32_t (&hi)[E], const uint32_t (&lo)[E], int nsl,
                                 uint32_t v, uint64_t u, int r)
    {
        const int lane = threadIdx.x & 63;
        wave_lds_sync();
        int nb = 0;
#pragma unroll
        for (int s = 0; s < E; ++s) {
            if (s < nsl) {
                const bool in = hi[s] >= v && (uint64_t)hi[s] < u;
                const uint64_t m = ballot(in);
                if (in)
                    scratch[nb + mbcnt(m)] = ((uint64_t)hi[s] << 32) | lo[s];
                nb += popc(m);
            }
        }
        wave_lds_sync();
        const uint64_t key = lane < nb ? scratch[lane] : 0ull;
        const uint64_t t = readlane64(wave_sort_desc(key), r - 1);
        wave_lds_sync();
        return t;
    }
};

template <int NW>
struct BlockReduce {
    int *red;          // LDS [2][NW]
    uint32_t *redu;    // LDS [2][NW]
    uint64_t *scratch; // LDS, 65 keys
    int phase;
    // Double-buffered slots: one barrier per reduction is enough, because a
    // wave can only overwrite a slot after every wave has passed the barrier
    // of the next reduction, i.e. after every wave finished reading it.
    __device__ int sum(int wave_count)
    {
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0)
            red[phase * NW + wave] = wave_count;
        __syncthreads();
        int s = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            s += red[phase * NW + w];
        phase ^= 1;
        return s;
    }
    template <bool MIN>
    __device__ uint32_t ured(uint32_t v)
    {
        v = MIN ? wave_min_u32(v) : wave_max_u32(v);
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0)
            redu[phase * NW + wave] = v;
        __syncthreads();
        uint32_t r = redu[phase * NW];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            r = MIN ? min(r, redu[phase * NW + w]) : max(r, redu[phase * NW + w]);
        phase ^= 1;
        return r;
    }
    __device__ uint32_t umin(uint32_t v) { return ured<true>(v); }
    __device__ uint32_t umax(uint32_t v) { return ured<false>(v); }

    template <int E>
    __device__ uint64_t band_kth(const uint32_t (&hi)[E], const uint32_t (&lo)[E], int nsl,
                                 uint32_t v, uint64_t u, int r)
    {
        const int lane = threadIdx.x & 63;
        const int wave = threadIdx.x >> 6;
        int wc = 0;
#pragma unroll
        for (int s = 0; s < E; ++s)
            if (s < nsl)
                wc += popc(ballot(hi[s] >= v && (uint64_t)hi[s] < u));
        if (lane == 0)
            red[phase * NW + wave] = wc;
        __syncthreads();
        int nb = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int c = red[phase * NW + w];
            nb += w < wave ? c : 0;
            tot += c;
        }
        phase ^= 1;
#pragma unroll
        for (int s = 0; s < E; ++s) {
            if (s < nsl) {
                const bool in = hi[s] >= v && (uint64_t)hi[s] < u;
                const uint64_t m = ballot(in);
                if (in)
                    scratch[nb + mbcnt(m)] = ((uint64_t)hi[s] << 32) | lo[s];
                nb += popc(m);
            }
        }
        __syncthreads();
        if (wave == 0) {
            const uint64_t key = lane < tot ? scratch[lane] : 0ull;
            const uint64_t t = readlane64(wave_sort_desc(key), r - 1);
            if (lane == 0)
                scratch[64] = t;
        }
        __syncthreads();
        const uint64_t t = scratch[64];
        __syncthreads(); // scratch may be reused right after
        return t;
    }
};

// Threshold search over the keys held by the participants (`tot` valid keys,
// k <= tot).  With slack > 0: returns L with k <= #{keys >= L} <= k + slack
// (a bound, not necessarily a key).  With slack == 0: returns the k-th
// largest key itself.
//
// Bisection on the high word (the score) keeps [v, u) with at least k keys at
// or above v and fewer than k at or above u.  It stops early within the slack,
// or (exact case) once the band [v, u) holds at most 64 keys, which are then
// sorted.  Only a run of more than 64 equal scores across the boundary needs
// the low word (the row), bisected from the bits those keys share.
template <int E, class R>
__device__ uint64_t select_bound(const uint32_t (&hi)[E], const uint32_t (&lo)[E], int nsl,
                                 int tot, int k, int slack, R &red)
{
    uint32_t v = 0;
    uint64_t u = 1ull << 32;
    int cv = tot; // #{keys with high word >= v}
    int cu = 0;   // #{keys with high word >= u}
    for (int b = 31; b >= 0; --b) {
        if (slack > 0 ? cv <= k + slack : cv - cu <= 64)
            break;
        const uint32_t c = v | (1u << b);
        const int cc = red.sum(count_hi_ge<E>(hi, nsl, c));
        if (cc >= k) {
            v = c;
            cv = cc;
        } else {
            u = c;
            cu = cc;
        }
    }
    if (slack > 0 && cv <= k + slack)
        return v ? ((uint64_t)v << 32) : 1ull;
    if (cv - cu <= 64) // (valid keys have a nonzero high word: empty slots stay out of the band)
        return red.template band_kth<E>(hi, lo, nsl, v ? v : 1u, u, k - cu);
    // more than 64 equal scores straddle the boundary: rank them by row
    const int need = k - cu; // here u == v + 1, and >= 2 keys share the high word v
    uint32_t lmin = 0xFFFFFFFFu, lmax = 0u;
#pragma unroll
    for (int s = 0; s < E; ++s)
        if (s < nsl && hi[s] == v) {
            lmin = min(lmin, lo[s]);
            lmax = max(lmax, lo[s]);
        }
    lmin = red.umin(lmin);
    lmax = red.umax(lmax);
    const int top = 31 - __builtin_clz(lmin ^ lmax);
    uint32_t w = lmax & ~((2u << top) - 1u);
    for (int b = top; b >= 0; --b) {
        const uint32_t c = w | (1u << b);
        if (red.sum(count_lo_ge<E>(hi, lo, nsl, v, c)) >= need)
            w = c;
    }
    return ((uint64_t)v << 32) | w;
}

// ---------------------------------------------------------------------------
// One wave's streaming selection state.  Keys enter the LDS buffer when they
// beat the threshold; the buffer always holds every key of the wave's stream
// that can still be among the k best, in the order they arrived.
// ---------------------------------------------------------------------------
template <int MAXS>
struct WaveSelect {
    static constexpr int CAP = MAXS * 64;
    uint64_t *buf; // LDS, CAP keys
    int k;
    int slack;    // a streaming shrink keeps between k and k + slack keys
    int cnt;      // keys in buf (wave-uniform)
    uint64_t tau; // keys <= tau cannot be among the k best (wave-uniform)

    // requires CAP >= k + 128 (select_slots guarantees more)
    __device__ void init(uint64_t *b, int kk, uint64_t lower)
    {
        buf = b;
        k = kk;
        // leave >= 128 free slots after every shrink, so each shrink makes room
        slack = min(CAP / 4, CAP - 128 - kk);
        slack = slack > 0 ? slack : 0;
        cnt = 0;
        tau = lower ? lower - 1 : 0;
    }

    // one key per lane (lanes with valid == false offer nothing)
    __device__ __forceinline__ void push(uint64_t key, bool valid)
    {
        const bool pass = valid && key > tau;
        const uint64_t m = ballot(pass);
        if (m == 0)
            return;
        if (pass)
            buf[cnt + mbcnt(m)] = key;
        cnt += popc(m);
        if (cnt > CAP - 64)
            shrink(slack);
    }

    // keep only the keys >= a bound leaving between k and k + slack of them
    // (exactly k when slack == 0), in order; the buffer's first 64 slots double
    // as scratch for the band sort
    __device__ void shrink(int sl)
    {
        wave_lds_sync();
        const int lane = threadIdx.x & 63;
        const int nsl = (cnt + 63) >> 6;
        uint32_t hi[MAXS], lo[MAXS];
#pragma unroll
        for (int s = 0; s < MAXS; ++s) {
            const int idx = s * 64 + lane;
            uint64_t key = 0;
            if (s < nsl && idx < cnt)
                key = buf[idx];
            hi[s] = (uint32_t)(key >> 32);
            lo[s] = (uint32_t)key;
        }
        WaveReduce red{buf};
        const uint64_t L = uniform64(select_bound<MAXS>(hi, lo, nsl, cnt, k, sl, red));
        int nc = 0;
#pragma unroll
        for (int s = 0; s < MAXS; ++s) {
            if (s < nsl) {
                const uint64_t key = ((uint64_t)hi[s] << 32) | lo[s];
                const bool keep = key >= L;
                const uint64_t m = ballot(keep);
                if (keep)
                    buf[nc + mbcnt(m)] = key;
                nc += popc(m);
            }
        }
        wave_lds_sync();
        cnt = nc;
        tau = L - 1;
    }

    // exactly the k best (requires at least k keys), in order
    __device__ void finish()
    {
        if (cnt > k)
            shrink(0);
        wave_lds_sync();
    }
};

// smallest per-wave buffer (in 64-key slots) for selecting topk: room for topk,
// a quarter more, and 128 free slots after a shrink
int select_slots(int topk)
{
    for (int s : {4, 8, 16, 32})
        if (s * 64 >= topk + topk / 4 + 128)
            return s;
    return 64;
}

// ---------------------------------------------------------------------------
// prefill: one wave per token over its row S[t][0..n_t); the next 512 scores
// are always in flight while the current 512 are pushed.
// ---------------------------------------------------------------------------
template <int MAXS>
__global__ __launch_bounds__(256) void topk_stream_kernel(const float *__restrict__ S, long long ldS,
                                                          const int32_t *__restrict__ pos, int T,
                                                          int N, int ratio, int topk,
                                                          int32_t *__restrict__ out)
{
    extern __shared__ uint64_t keys_lds[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wpb = blockDim.x >> 6;
    const int t = blockIdx.x * wpb + wave;
    if (t >= T)
        return;
    const int n = visible_rows(pos[t], ratio, N);
    int32_t *o = out + (long long)t * topk;
    if (n <= topk) { // all rows fit: the sequential rows, no scoring needed
        for (int i = lane; i < topk; i += 64)
            o[i] = i < n ? i : -1;
        return;
    }
    WaveSelect<MAXS> sel;
    sel.init(keys_lds + (size_t)wave * WaveSelect<MAXS>::CAP, topk, 0);
    const float *row = S + (long long)t * ldS;
    constexpr int U = 8;
    float cur[U], nxt[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = u * 64 + lane;
        cur[u] = j < n ? row[j] : 0.f;
    }
    for (int base = 0; base < n; base += U * 64) {
        const int nb = base + U * 64;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = nb + u * 64 + lane;
            nxt[u] = j < n ? row[j] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + u * 64 + lane;
            sel.push(make_key(cur[u], (uint32_t)j), j < n);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            cur[u] = nxt[u];
    }
    sel.finish();
    for (int i = lane; i < topk; i += 64)
        o[i] = key_row(sel.buf[i]);
}

// ---------------------------------------------------------------------------
// decode, stage 1: partition p = rows [p*1024, min(n, p*1024 + 1024)).  Each
// partition lists its exact best kp keys in row order, with the smallest of
// them (or 0 when the partition has no more than kp rows and lists them all).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int block_exclusive_scan(int c, int *scan)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int inc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o);
        if (lane >= o)
            inc += y;
    }
    if (lane == 63)
        scan[wave] = inc;
    __syncthreads();
    int off = inc - c;
    for (int w = 0; w < wave; ++w)
        off += scan[w];
    return off;
}

__global__ __launch_bounds__(256) void decode_partial_kernel(
    const float *__restrict__ S, const int32_t *__restrict__ pos, int N, int ratio, int topk,
    int kp, uint64_t *__restrict__ cand, int *__restrict__ pcount, uint64_t *__restrict__ pmin)
{
    __shared__ int red[2 * 4];
    __shared__ uint32_t redu[2 * 4];
    __shared__ uint64_t scratch[65];
    __shared__ int scan[4];
    const int n = visible_rows(pos[0], ratio, N);
    if (n <= topk)
        return;
    const int p = blockIdx.x;
    const int r0 = p * kDecodePart;
    if (r0 >= n)
        return;
    const int rows = min(kDecodePart, n - r0);
    const int tid = threadIdx.x;

    uint32_t hi[4], lo[4];
    float v[4];
    if (4 * tid + 3 < rows) {
        const float4 f = *reinterpret_cast<const float4 *>(S + r0 + 4 * tid);
        v[0] = f.x;
        v[1] = f.y;
        v[2] = f.z;
        v[3] = f.w;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = 4 * tid + e < rows ? S[r0 + 4 * tid + e] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint64_t key = 4 * tid + e < rows ? make_key(v[e], (uint32_t)(r0 + 4 * tid + e)) : 0;
        hi[e] = (uint32_t)(key >> 32);
        lo[e] = (uint32_t)key;
    }
    uint64_t *dst = cand + (size_t)p * kp;
    if (rows <= kp) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * tid + e < rows)
                dst[4 * tid + e] = ((uint64_t)hi[e] << 32) | lo[e];
        if (tid == 0) {
            pcount[p] = rows;
            pmin[p] = 0;
        }
        return;
    }
    BlockReduce<4> br{red, redu, scratch, 0};
    const uint64_t L = select_bound<4>(hi, lo, 4, rows, kp, 0, br); // exactly the kp-th key
    int c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        c += (((uint64_t)hi[e] << 32) | lo[e]) >= L;
    int off = block_exclusive_scan(c, scan);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint64_t key = ((uint64_t)hi[e] << 32) | lo[e];
        if (key >= L)
            dst[off++] = key;
    }
    if (tid == 0) {
        pcount[p] = kp;
        pmin[p] = L;
    }
}

// ---------------------------------------------------------------------------
// decode, stage 2: one work-group merges the partition lists.  With tU the
// k-th best key of their union, the union's top k is the exact answer unless
// some partition listed only part of its rows and its smallest listed key is
// above tU (it may hold unlisted rows above tU).  That case falls back to an
// exact re-stream of those partitions' rows by one wave.
// kp is a power of two.
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 1024;
constexpr int kMergeSlots = kDecodeUnion / kMergeThreads; // 16

template <int MAXS>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(
    const float *__restrict__ S, const int32_t *__restrict__ pos, int N, int ratio, int topk,
    int kp, const uint64_t *__restrict__ cand, const int *__restrict__ pcount,
    const uint64_t *__restrict__ pmin, int32_t *__restrict__ out)
{
    constexpr int NW = kMergeThreads / 64;
    extern __shared__ uint64_t fb_buf[];
    __shared__ int red[2 * NW];
    __shared__ uint32_t redu[2 * NW];
    __shared__ uint64_t scratch[65];
    __shared__ int scan[NW];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = visible_rows(pos[0], ratio, N);
    if (n <= topk) {
        for (int i = tid; i < topk; i += kMergeThreads)
            out[i] = i < n ? i : -1;
        return;
    }
    const int P = (n + kDecodePart - 1) / kDecodePart;
    const int U = P * kp;
    const int E = (U + kMergeThreads - 1) / kMergeThreads; // <= kMergeSlots
    const int lgkp = 31 - __builtin_clz(kp);

    // thread i holds union elements [i*E, i*E + E): row order is element order
    uint32_t hi[kMergeSlots], lo[kMergeSlots];
    int have = 0;
#pragma unroll
    for (int s = 0; s < kMergeSlots; ++s) {
        const int e = tid * E + s;
        uint64_t key = 0;
        if (s < E && e < U && (e & (kp - 1)) < pcount[e >> lgkp])
            key = cand[e];
        hi[s] = (uint32_t)(key >> 32);
        lo[s] = (uint32_t)key;
        have += key != 0;
    }
    BlockReduce<NW> br{red, redu, scratch, 0};
    int wc = have;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        wc += __shfl_xor(wc, o);
    const int total = br.sum(wc);
    bool fallback = total < topk;
    uint64_t tU = 0;
    if (!fallback) {
        tU = select_bound<kMergeSlots>(hi, lo, E, total, topk, 0, br); // the k-th key of the union
        bool fail = false;
        for (int p = tid; p < P; p += kMergeThreads) {
            const int rows = min(kDecodePart, n - p * kDecodePart);
            fail |= pcount[p] == kp && rows > kp && pmin[p] > tU;
        }
        fallback = br.sum(popc(ballot(fail))) > 0;
    }
    if (!fallback) {
        int c = 0;
#pragma unroll
        for (int s = 0; s < kMergeSlots; ++s)
            if (s < E)
                c += (((uint64_t)hi[s] << 32) | lo[s]) >= tU;
        int off = block_exclusive_scan(c, scan);
#pragma unroll
        for (int s = 0; s < kMergeSlots; ++s) {
            if (s < E) {
                const uint64_t key = ((uint64_t)hi[s] << 32) | lo[s];
                if (key >= tU)
                    out[off++] = key_row(key);
            }
        }
        return;
    }
    // exact fallback: one wave re-streams every partition in row order, the
    // listed keys of partitions whose list is known to be enough and all rows
    // of the others, keeping only keys that can still reach the top k
    if (wave != 0)
        return;
    WaveSelect<MAXS> sel;
    sel.init(fb_buf, topk, tU);
    for (int p = 0; p < P; ++p) {
        const int r0 = p * kDecodePart;
        const int rows = min(kDecodePart, n - r0);
        const int pc = pcount[p];
        const bool raw = pc == kp && rows > kp && pmin[p] > tU;
        if (raw) {
            for (int i = 0; i < rows; i += 64) {
                const int r = r0 + i + lane;
                const bool valid = i + lane < rows;
                const float sv = valid ? S[r] : 0.f;
                sel.push(make_key(sv, (uint32_t)r), valid);
            }
        } else {
            for (int i = 0; i < pc; i += 64) {
                const bool valid = i + lane < pc;
                const uint64_t key = valid ? cand[(size_t)p * kp + i + lane] : 0;
                sel.push(key, valid);
            }
        }
    }
    sel.finish();
    for (int i = lane; i < topk; i += 64)
        out[i] = key_row(sel.buf[i]);
}

template <int MAXS>
hipError_t topk_stream_one(const float *S, long long ldS, const int32_t *pos, int T, int N,
                           int ratio, int topk, int32_t *out, hipStream_t st)
{
    // waves (tokens) per work-group: 64 KiB of LDS at most
    const int wpb = MAXS >= 64 ? 2 : 4;
    const size_t lds = (size_t)wpb * MAXS * 64 * sizeof(uint64_t);
    hipLaunchKernelGGL((topk_stream_kernel<MAXS>), dim3((T + wpb - 1) / wpb), dim3(wpb * 64), lds,
                       st, S, ldS, pos, T, N, ratio, topk, out);
    return hipGetLastError();
}

template <int MAXS>
hipError_t merge_one(const float *S, const int32_t *pos, int N, int ratio, int topk, int kp,
                     const uint64_t *cand, const int *pcount, const uint64_t *pmin, int32_t *out,
                     hipStream_t st)
{
    const size_t lds = (size_t)MAXS * 64 * sizeof(uint64_t);
    hipLaunchKernelGGL((decode_merge_kernel<MAXS>), dim3(1), dim3(kMergeThreads), lds, st, S, pos,
                       N, ratio, topk, kp, cand, pcount, pmin, out);
    return hipGetLastError();
}

} // namespace

hipError_t launch_topk_stream(const float *S, long long ldS, const int32_t *pos, int T, int N,
                              int ratio, int topk, int32_t *out, hipStream_t st)
{
    if (T <= 0)
        return hipSuccess;
    switch (select_slots(topk)) {
    case 4: return topk_stream_one<4>(S, ldS, pos, T, N, ratio, topk, out, st);
    case 8: return topk_stream_one<8>(S, ldS, pos, T, N, ratio, topk, out, st);
    case 16: return topk_stream_one<16>(S, ldS, pos, T, N, ratio, topk, out, st);
    case 32: return topk_stream_one<32>(S, ldS, pos, T, N, ratio, topk, out, st);
    default: return topk_stream_one<64>(S, ldS, pos, T, N, ratio, topk, out, st);
    }
}

hipError_t launch_decode_select(const float *S, const int32_t *pos, int N, int ratio, int topk,
                                int kp, uint64_t *cand, int *pcount, uint64_t *pmin,
                                int32_t *out, hipStream_t st)
{
    const int P = (N + kDecodePart - 1) / kDecodePart;
    if (P > 0) {
        hipLaunchKernelGGL(decode_partial_kernel, dim3(P), dim3(256), 0, st, S, pos, N, ratio, topk,
                           kp, cand, pcount, pmin);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    switch (select_slots(topk)) {
    case 4: return merge_one<4>(S, pos, N, ratio, topk, kp, cand, pcount, pmin, out, st);
    case 8: return merge_one<8>(S, pos, N, ratio, topk, kp, cand, pcount, pmin, out, st);
    case 16: return merge_one<16>(S, pos, N, ratio, topk, kp, cand, pcount, pmin, out, st);
    case 32: return merge_one<32>(S, pos, N, ratio, topk, kp, cand, pcount, pmin, out, st);
    default: return merge_one<64>(S, pos, N, ratio, topk, kp, cand, pcount, pmin, out, st);
    }
}

} // namespace dsi
