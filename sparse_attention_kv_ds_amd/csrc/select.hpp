// select.hpp -- selection primitives shared by the top-k kernels (gfx950).
//
// Keys are the unique 64-bit (score, row) keys of common.hpp.  The primitives
// count keys held in registers with ballots (no atomics), find a threshold by
// bisection over the score bits, finish the exact k-th key by ranking the
// <= 64 keys left in the boundary band, and keep a wave's streaming candidate
// buffer in LDS in arrival (row) order.
#pragma once

#include "common.hpp"

namespace dsi {
namespace {

// Wave-wide reductions on the VALU alone (DPP row shuffles, then the gfx950
// row and half swaps): every lane ends with the result.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op)
{
    v = op(v, dpp<0xB1>(v));  // quad_perm [1,0,3,2]: lane ^ 1
    v = op(v, dpp<0x4E>(v));  // quad_perm [2,3,0,1]: lane ^ 2
    v = op(v, dpp<0x141>(v)); // row_half_mirror: the other quad of each 8
    v = op(v, dpp<0x140>(v)); // row_mirror: the other 8 of each row of 16
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = op(r[0], r[1]);       // rows 0/1 and 2/3 combined
    const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return op(h[0], h[1]);    // the two halves combined
}

struct OpMin {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; }
};
struct OpMax {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};
struct OpAdd {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
    return readfirstlane(wave_reduce(v, OpMin{}));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    return readfirstlane(wave_reduce(v, OpMax{}));
}

__device__ __forceinline__ int wave_sum(int v)
{
    return (int)readfirstlane(wave_reduce((uint32_t)v, OpAdd{}));
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

// ---------------------------------------------------------------------------
// Counting over keys held in registers, split in high/low words.  Empty slots
// hold key 0, which never counts because every value tested is >= 1.
// ---------------------------------------------------------------------------
// Lane masks of x[s] >= c for four slots, computed back to back into four
// scalar register pairs (written as one block so that the compares are not
// serialised through a single mask register by the scalar counts after them).
__device__ __forceinline__ void ge_masks4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                          uint32_t c, uint64_t &m0, uint64_t &m1, uint64_t &m2,
                                          uint64_t &m3)
{
    asm volatile("v_cmp_ge_u32_e64 %0, %4, %8\n\t"
                 "v_cmp_ge_u32_e64 %1, %5, %8\n\t"
                 "v_cmp_ge_u32_e64 %2, %6, %8\n\t"
                 "v_cmp_ge_u32_e64 %3, %7, %8"
                 : "=&s"(m0), "=&s"(m1), "=&s"(m2), "=&s"(m3) // (written before c is last read)
                 : "v"(x0), "v"(x1), "v"(x2), "v"(x3), "s"(c));
}

// #{keys with high word >= c} over the wave's slots; slots at or past nsl (a
// uniform bound, in steps of 4) are skipped, and empty slots hold 0 while
// c >= 1, so they never count
template <int E>
__device__ __forceinline__ int count_hi_ge(const uint32_t (&hi)[E], int nsl, uint32_t c)
{
    int r = 0;
    // (a guard rather than a break, so that the loop always unrolls and hi[]
    // is only ever indexed by constants)
#pragma unroll
    for (int s = 0; s < E; s += 4) {
        if (s < nsl) {
            if (s + 4 <= E) {
                uint64_t m0, m1, m2, m3;
                ge_masks4(hi[s], hi[s + 1], hi[s + 2], hi[s + 3], c, m0, m1, m2, m3);
                r += popc(m0) + popc(m1) + popc(m2) + popc(m3);
            } else {
#pragma unroll
                for (int t = s; t < E; ++t)
                    r += popc(ballot(hi[t] >= c));
            }
        }
    }
    return r;
}

// ---------------------------------------------------------------------------
// Reductions over the participants of a selection: one wave, or a whole
// work-group.  Every result is the same in all lanes (scalar registers).
// ---------------------------------------------------------------------------
struct WaveReduce {
    __device__ __forceinline__ int sum(int wave_count) { return wave_count; }
    // Low word of the r-th (1-based) key with high word v in participant order:
    // slot 0 of lanes 0..63, then slot 1, ... (r is at most the number of such keys)
    template <int E, class LO>
    __device__ __forceinline__ uint32_t nth(const uint32_t (&hi)[E], const LO &lo, uint32_t v,
                                            int r)
    {
        const int lane = threadIdx.x & 63;
        uint32_t res = 0;
        int before = 0;
#pragma unroll
        for (int s = 0; s < E; ++s) {
            const uint64_t m = ballot(hi[s] == v);
            const int c = popc(m);
            const int q = r - before; // rank within this slot
            if (q >= 1 && q <= c) {
                const uint64_t hit = ballot(((m >> lane) & 1) && mbcnt(m) == q - 1);
                res = __builtin_amdgcn_readlane((uint32_t)lo[s], (int)__builtin_ctzll(hit));
            }
            before += c;
        }
        return res;
    }
    __device__ __forceinline__ void minmax(uint32_t &mn, uint32_t &mx)
    {
        mn = wave_min_u32(mn);
        mx = wave_max_u32(mx);
    }
    __device__ __forceinline__ uint32_t umin(uint32_t v) { return wave_min_u32(v); }
    __device__ __forceinline__ uint32_t umax(uint32_t v) { return wave_max_u32(v); }
};

template <int NW>
struct BlockReduce {
    static constexpr int kWords = 2 * NW * 2; // LDS ints the caller provides
    int *red;  // LDS [2][NW][2]
    int *tab;  // LDS [E][NW] for nth<E>
    int phase; // double-buffered slots: one barrier per reduction is enough,
               // because a wave can only overwrite a slot after every wave has
               // passed the barrier of the next reduction, i.e. after every wave
               // finished reading it
    __device__ __forceinline__ int *mine() { return red + (phase * NW + wave_id()) * 2; }
    __device__ __forceinline__ const int *col(int w) const { return red + (phase * NW + w) * 2; }

    __device__ __forceinline__ int sum(int wave_count)
    {
        if ((threadIdx.x & 63) == 0)
            mine()[0] = wave_count;
        lds_barrier();
        int s = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            s += col(w)[0];
        phase ^= 1;
        return (int)readfirstlane(s);
    }
    __device__ __forceinline__ void minmax(uint32_t &mn, uint32_t &mx)
    {
        mn = wave_min_u32(mn);
        mx = wave_max_u32(mx);
        if ((threadIdx.x & 63) == 0) {
            mine()[0] = (int)mn;
            mine()[1] = (int)mx;
        }
        lds_barrier();
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            mn = min(mn, (uint32_t)col(w)[0]);
            mx = max(mx, (uint32_t)col(w)[1]);
        }
        mn = readfirstlane(mn);
        mx = readfirstlane(mx);
        phase ^= 1;
    }
    template <bool MIN>
    __device__ __forceinline__ uint32_t ured(uint32_t v)
    {
        v = MIN ? wave_min_u32(v) : wave_max_u32(v);
        if ((threadIdx.x & 63) == 0)
            mine()[0] = (int)v;
        lds_barrier();
        uint32_t r = (uint32_t)col(0)[0];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            r = MIN ? min(r, (uint32_t)col(w)[0]) : max(r, (uint32_t)col(w)[0]);
        phase ^= 1;
        return readfirstlane(r);
    }
    __device__ __forceinline__ uint32_t umin(uint32_t v) { return ured<true>(v); }
    __device__ __forceinline__ uint32_t umax(uint32_t v) { return ured<false>(v); }

    // As WaveReduce::nth, in the order slot, then wave, then lane.
    template <int E, class LO>
    __device__ __forceinline__ uint32_t nth(const uint32_t (&hi)[E], const LO &lo, uint32_t v,
                                            int r)
    {
        const int lane = threadIdx.x & 63;
        const int wave = wave_id();
        uint64_t m[E];
#pragma unroll
        for (int s = 0; s < E; ++s) {
            m[s] = ballot(hi[s] == v);
            if (lane == 0)
                tab[s * NW + wave] = popc(m[s]);
        }
        lds_barrier();
        int base = 0;
#pragma unroll
        for (int s = 0; s < E; ++s) {
            int before = 0, all = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const int c = tab[s * NW + w];
                before += w < wave ? c : 0;
                all += c;
            }
            const int q = (int)readfirstlane(r - base - before); // rank within this wave's slot
            if (q >= 1 && q <= popc(m[s])) {
                const uint64_t hit = ballot(((m[s] >> lane) & 1) && mbcnt(m[s]) == q - 1);
                const uint32_t x =
                    __builtin_amdgcn_readlane((uint32_t)lo[s], (int)__builtin_ctzll(hit));
                if (lane == 0)
                    red[phase * NW * 2] = (int)x; // one writer in the whole group
            }
            base += all;
        }
        lds_barrier();
        const uint32_t res = readfirstlane((uint32_t)red[phase * NW * 2]);
        phase ^= 1;
        return res;
    }
};

// The largest (MAX) or smallest key whose high word lies in [v, u), v >= 1.
template <bool MAX, int E, class LO, class R>
__device__ __forceinline__ uint64_t band_extreme(const uint32_t (&hi)[E], const LO &lo, uint32_t v,
                                                 uint64_t u, R &red)
{
    uint32_t h = MAX ? 0u : 0xFFFFFFFFu;
#pragma unroll
    for (int s = 0; s < E; ++s)
        if (hi[s] >= v && (uint64_t)hi[s] < u)
            h = MAX ? max(h, hi[s]) : min(h, hi[s]);
    h = MAX ? red.umax(h) : red.umin(h);
    uint32_t l = MAX ? 0u : 0xFFFFFFFFu;
#pragma unroll
    for (int s = 0; s < E; ++s)
        if (hi[s] == h)
            l = MAX ? max(l, (uint32_t)lo[s]) : min(l, (uint32_t)lo[s]);
    l = MAX ? red.umax(l) : red.umin(l);
    return ((uint64_t)h << 32) | l;
}

// Threshold search over the keys held by the participants (`tot` valid keys,
// k <= tot; empty slots hold key 0; slots at or past nsl are all empty).  With slack > 0: returns L with
// k <= #{keys >= L} <= k + slack (a bound, not necessarily a key).  With
// slack == 0: returns the k-th largest key itself.
//
// The search bisects the high word (the score) between the smallest and the
// largest one, keeping [v, u) with at least k keys at or above v and fewer
// than k at or above u (a band started at the keys' own range needs fewer
// steps than one aligned to a power of two around it).  It stops early within
// the slack, or (exact case) as soon as the k-th key is the largest or the
// smallest of the band [v, u), which one reduction then finds.  Only equal
// scores across the boundary need the low word (the row), bisected from the
// bits those keys share.
template <int E, class LO, class R>
__device__ __forceinline__ uint64_t select_bound(const uint32_t (&hi)[E], const LO &lo, int nsl,
                                                int tot, int k, int slack, R &red)
{
    if (slack > 0 && tot <= k + slack)
        return 1ull;
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
    for (int s = 0; s < E; ++s)
        if (hi[s] != 0u) {
            mn = min(mn, hi[s]);
            mx = max(mx, hi[s]);
        }
    red.minmax(mn, mx);
    // no key with a nonzero high word (only NaN scores map to 0): nothing to
    // separate, keep every key (without this the band below would start
    // inverted and the search would not end)
    if (mn > mx)
        return 1ull;
    // every key's high word is in [v, u): the band starts as [mn, mx] itself
    uint32_t v = mn;
    uint64_t u = (uint64_t)mx + 1;
    int cv = tot; // #{keys with high word >= v}
    int cu = 0;   // #{keys with high word >= u}
#pragma unroll 1
    while (u - v > 1) {
        if (slack > 0 ? cv <= k + slack : (k - cu == 1 || k == cv))
            break;
        const uint32_t c = (uint32_t)(v + ((u - v) >> 1)); // v < c < u
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
        return (uint64_t)v << 32; // v >= mn >= 1
    const uint32_t vb = v ? v : 1u; // (empty slots stay out of the band)
    if (k - cu == 1) // the k-th key is the largest in the band
        return band_extreme<true>(hi, lo, vb, u, red);
    if (k == cv) // ... or the smallest
        return band_extreme<false>(hi, lo, vb, u, red);
    // equal scores straddle the boundary: among the keys with score v, the one
    // with the need-th lowest row -- the participants hold their keys in row
    // order, so it is the need-th such key in that order
    const int need = k - cu; // here u == v + 1, and >= 3 keys share the high word v
    return ((uint64_t)v << 32) | red.template nth<E, LO>(hi, lo, v, need);
}

// #{keys greater than x among arr[0 .. cnt)} (cnt <= 64, uniform; arr holds 64 keys)
__device__ __forceinline__ int rank_among(const uint64_t *arr, int cnt, uint64_t x)
{
    int r = 0;
#pragma unroll 8
    for (int j = 0; j < cnt; j += 2) {
        const uint64_t a = arr[j], b = arr[j + 1]; // (arr[j + 1] may be stale when j + 1 == cnt)
        r += (a > x) + (j + 1 < cnt && b > x);
    }
    return r;
}

// Low words of a wave's LDS key buffer, read on demand: slot s of this lane,
// at a constant offset from the lane's first key.
struct LdsLow {
    const uint64_t *mine; // buf + lane
    __device__ uint32_t operator[](int s) const { return (uint32_t)mine[s * 64]; }
};

template <int MAXS>
struct WaveSelect {
    static constexpr int CAP = MAXS * 64;
    // the largest buffers keep only the high words in registers during a
    // shrink and read the low words from LDS where a decision needs them
    static constexpr bool kLowInLds = MAXS > 32;
    uint64_t *buf; // LDS, CAP keys
    int k;
    int slack;    // a streaming shrink keeps between k and k + slack keys
    int cnt;      // keys in buf (wave-uniform)
    uint64_t tau; // keys <= tau cannot be among the k best (wave-uniform)
    // Coarse keys: the high word holds only the top 16 bits of the ordered
    // score, so keys with the same high word are not in score order.  A
    // streaming shrink then keeps whole high words (a bound with low word 0);
    // when that is impossible within the slack (a single high word straddles
    // the boundary with more than the slack's worth of keys) it sets `failed`
    // and leaves the buffer as it was, and the caller starts again with exact
    // keys.
    bool coarse;
    bool failed;
#ifdef DSI_STAMPS
    int shrinks = 0; // (stamps build: searches run while streaming)
#endif

    // Keys arrive in batches of at most `batch` (a multiple of 64) between
    // make_room() calls; requires CAP >= k + batch + 64.
    __device__ __forceinline__ void init(uint64_t *b, int kk, uint64_t lower, int batch,
                                         bool coarse_keys = false)
    {
        buf = b;
        k = kk;
        // every shrink leaves room for a whole batch
        slack = min(CAP / 4, CAP - batch - kk);
        slack = slack > 0 ? slack : 0;
        cnt = 0;
        tau = lower ? lower - 1 : 0;
        coarse = coarse_keys;
        failed = false;
    }

    // before a batch of up to `incoming` keys
    __device__ __forceinline__ void make_room(int incoming)
    {
        if (cnt > CAP - incoming)
            shrink(slack);
    }

    // one key per lane (lanes with valid == false offer nothing); appends the
    // keys above the threshold, in lane order, without checking for room
    __device__ __forceinline__ void append(uint64_t key, bool valid)
    {
        const bool pass = valid && key > tau;
        const uint64_t m = ballot(pass);
        if (pass)
            buf[cnt + mbcnt(m)] = key;
        cnt += popc(m);
    }

    // four keys per lane, in the order k0 .. k3 within a lane (lane order,
    // then k0 .. k3: consecutive rows held by one lane stay in row order)
    __device__ __forceinline__ void append4(uint64_t k0, bool v0, uint64_t k1, bool v1,
                                            uint64_t k2, bool v2, uint64_t k3, bool v3)
    {
        const bool p0 = v0 && k0 > tau, p1 = v1 && k1 > tau;
        const bool p2 = v2 && k2 > tau, p3 = v3 && k3 > tau;
        const uint64_t m0 = ballot(p0), m1 = ballot(p1), m2 = ballot(p2), m3 = ballot(p3);
        const int at0 = cnt + mbcnt(m0) + mbcnt(m1) + mbcnt(m2) + mbcnt(m3);
        const int at1 = at0 + (p0 ? 1 : 0), at2 = at1 + (p1 ? 1 : 0), at3 = at2 + (p2 ? 1 : 0);
        if (p0)
            buf[at0] = k0;
        if (p1)
            buf[at1] = k1;
        if (p2)
            buf[at2] = k2;
        if (p3)
            buf[at3] = k3;
        cnt += popc(m0) + popc(m1) + popc(m2) + popc(m3);
    }

    // a batch of one key per lane
    __device__ __forceinline__ void push(uint64_t key, bool valid)
    {
        make_room(64);
        append(key, valid);
    }

    // keep only the keys >= a bound leaving between k and k + slack of them
    // (exactly k when slack == 0), in order.  The compaction is in place: a
    // kept key moves to an index no larger than its own, and one wave's LDS
    // accesses stay in program order.
    __device__ __forceinline__ void shrink(int sl)
    {
#ifdef DSI_STAMPS
        shrinks += sl > 0;
#endif
        wave_lds_sync();
        const int lane = threadIdx.x & 63;
        const int nsl = (cnt + 63) >> 6;
        uint32_t hi[MAXS];
        uint32_t lo_r[kLowInLds ? 1 : MAXS];
        const uint64_t *mine = buf + lane; // slot s at constant offset s * 64
        const int rem = cnt - lane;        // slot s holds a key iff s * 64 < rem
#pragma unroll
        for (int s = 0; s < MAXS; ++s) {
            uint64_t key = 0;
            if (s * 64 < rem)
                key = mine[s * 64];
            hi[s] = (uint32_t)(key >> 32);
            if constexpr (!kLowInLds)
                lo_r[s] = (uint32_t)key;
        }
        WaveReduce red;
        uint64_t L;
        // (every slot is looked at: empty ones hold key 0, which never counts)
        if constexpr (kLowInLds)
            L = uniform64(select_bound<MAXS>(hi, LdsLow{mine}, nsl, cnt, k, sl, red));
        else
            L = uniform64(select_bound<MAXS>(hi, lo_r, nsl, cnt, k, sl, red));
        // (a bound within the slack is a whole high word, low word 0, or 1:
        // keep everything; any other bound is a key, which splits a high word)
        if (coarse && sl > 0 && (uint32_t)L != 0u && L != 1ull) {
            failed = true;
            return;
        }
        int nc = 0;
#pragma unroll
        for (int s = 0; s < MAXS; ++s) {
            if (s < nsl) {
                uint32_t lw;
                if constexpr (kLowInLds)
                    lw = (uint32_t)mine[s * 64];
                else
                    lw = lo_r[s];
                const uint64_t key = ((uint64_t)hi[s] << 32) | lw;
                const bool keep = hi[s] != 0u && key >= L; // (hi == 0: no key)
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
    __device__ __forceinline__ void finish()
    {
        if (cnt > k)
            shrink(0);
        wave_lds_sync();
    }

    // The same for coarse keys (at least k, whole high words kept by every
    // shrink), ending with the k best rows, ascending, in out[0 .. k).  The
    // high word h holding the k-th key is found by bisection; the keys above
    // h are in, those below out.  Only the keys of h itself need their exact
    // order: their ordered scores are completed with the low 16 bits,
    // low_of(row).  With at most 64 such keys they are ranked one per lane
    // (scratch: 64 keys of LDS private to the wave) and the rows are written
    // straight from the slots in order, each key of h asking the lane that
    // ranked it whether it is in.  With more, the keys above h are lifted to
    // (h + 1) << 16, above every completed one, the exact search keeps k in
    // the buffer, and the rows are written from there.
    template <class LOW>
    __device__ __forceinline__ void finish_coarse(const LOW &low_of, uint64_t *scratch,
                                                  int32_t *out)
    {
        wave_lds_sync();
        const int lane = threadIdx.x & 63;
        if (cnt <= k) {
            for (int i = lane; i < cnt; i += 64)
                out[i] = key_row(buf[i]);
            return;
        }
        const int nsl = (cnt + 63) >> 6;
        const uint64_t *mine = buf + lane;
        const int rem = cnt - lane;
        uint32_t hi[MAXS];
        uint32_t lo_r[kLowInLds ? 1 : MAXS];
#pragma unroll
        for (int s = 0; s < MAXS; ++s) {
            const uint64_t key = s * 64 < rem ? mine[s * 64] : 0ull;
            hi[s] = (uint32_t)(key >> 32);
            if constexpr (!kLowInLds)
                lo_r[s] = (uint32_t)key;
        }
        auto row_of = [&](int s) -> int {
            if constexpr (kLowInLds)
                return key_row(mine[s * 64]);
            else
                return key_row(lo_r[s]);
        };
        WaveReduce red;
        uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
        for (int s = 0; s < MAXS; ++s)
            if (hi[s] != 0u) {
                mn = min(mn, hi[s]);
                mx = max(mx, hi[s]);
            }
        red.minmax(mn, mx);
        if (mn > mx) {
            // no key with a nonzero high word (only NaN scores map to 0):
            // the first k rows, so that the search below always has a band
            for (int i = lane; i < k; i += 64)
                out[i] = key_row(buf[i]);
            return;
        }
        // #{high >= v} = cv >= k > cu = #{high >= u}
        uint32_t v = mn, u = mx + 1;
        int cv = cnt, cu = 0;
#pragma unroll 1
        while (u - v > 1 && cv != k) {
            const uint32_t c = v + ((u - v) >> 1);
            const int cc = count_hi_ge<MAXS>(hi, nsl, c);
            if (cc >= k) {
                v = c;
                cv = cc;
            } else {
                u = c;
                cu = cc;
            }
        }
        const uint32_t h = v; // unless cv == k, u == v + 1 and h holds the k-th key
        if (cv == k || cv - cu <= 64) {
            // in[B index] for the keys of h, B index = order among them (one per lane)
            bool in_b = false;
            if (cv != k) {
                const int nb = cv - cu, need = k - cu; // 1 <= need < nb
                uint32_t *bidx = reinterpret_cast<uint32_t *>(scratch);
                int c = 0;
#pragma unroll
                for (int s = 0; s < MAXS; ++s) {
                    if (s < nsl) {
                        const bool b = hi[s] == h;
                        const uint64_t m = ballot(b);
                        if (b)
                            bidx[c + mbcnt(m)] = (uint32_t)(s * 64 + lane);
                        c += popc(m);
                    }
                }
                wave_lds_sync();
                const bool has = lane < nb;
                const uint32_t ix = has ? bidx[lane] : 0u;
                const uint32_t lw = has ? (uint32_t)buf[ix] : 0u;
                const uint32_t lo16 = has ? low_of(0xFFFFFFFFu - lw) : 0u;
                const uint64_t ex = has ? ((uint64_t)((h << 16) | lo16) << 32) | lw : 0ull;
                wave_lds_sync(); // (the slots are read before the scratch is reused)
                scratch[lane] = ex;
                wave_lds_sync();
                in_b = has && rank_among(scratch, nb, ex) < need;
            }
            // the rows, in order: high word above h, or h and ranked in (cv == k: every
            // key of h is in)
            const int in_bits = in_b ? 1 : 0;
            int nc = 0, bb = 0;
#pragma unroll
            for (int s = 0; s < MAXS; ++s) {
                if (s < nsl) {
                    const bool b = hi[s] == h;
                    const uint64_t mb = ballot(b);
                    bool keep = hi[s] > h;
                    if (cv == k) {
                        keep = keep || b;
                    } else if (mb) {
                        // (every lane takes part: a lane that is switched off
                        // would read as 0 to the lanes asking it)
                        const int from = bb + mbcnt(mb);
                        const int asked = __builtin_amdgcn_ds_bpermute(from * 4, in_bits);
                        keep = keep || (b && asked != 0);
                    }
                    bb += popc(mb);
                    const uint64_t m = ballot(keep);
                    if (keep)
                        out[nc + mbcnt(m)] = row_of(s);
                    nc += popc(m);
                }
            }
            return;
        }
        uint32_t low16[MAXS];
#pragma unroll
        for (int s = 0; s < MAXS; ++s) {
            low16[s] = 0u;
            if (s < nsl && ballot(hi[s] == h))
                low16[s] = hi[s] == h ? low_of((uint32_t)row_of(s)) : 0u;
        }
        int nc = 0;
#pragma unroll
        for (int s = 0; s < MAXS; ++s) {
            if (s < nsl) {
                const uint32_t lw = 0xFFFFFFFFu - (uint32_t)row_of(s);
                const bool keep = hi[s] != 0u && hi[s] >= h;
                const uint32_t nh = hi[s] == h ? (h << 16) | low16[s] : (h + 1) << 16;
                const uint64_t m = ballot(keep);
                if (keep)
                    buf[nc + mbcnt(m)] = ((uint64_t)nh << 32) | lw;
                nc += popc(m);
            }
        }
        wave_lds_sync();
        cnt = nc;
        coarse = false; // every key left is exact, or above every one that is
        shrink(0);
        wave_lds_sync();
        for (int i = lane; i < k; i += 64)
            out[i] = key_row(buf[i]);
    }
};

// ---------------------------------------------------------------------------
// Small k on one wave, without a search loop.  The k-th largest (k * E <= 64)
// of the keys a wave holds in hi/lo (E per lane, key 0 in empty slots; keys
// only in lanes below LANES; at least k lanes hold a key).  With L the k-th
// largest of the lane maxima,
// at least k keys are >= L, so the answer is >= L; and keys >= L sit only in
// the k lanes whose maximum is >= L, so there are at most k * E of them.  Both
// steps rank at most 64 keys, one per lane, by counting the larger ones among
// all of them (read back from LDS as broadcasts): a fixed number of compares,
// where a bisection would take one dependent count step per score bit.
// scratch: 128 keys of LDS private to the wave.
// ---------------------------------------------------------------------------
template <int E, int LANES = 64>
__device__ __forceinline__ uint64_t wave_kth_small(const uint32_t (&hi)[E], const uint32_t (&lo)[E],
                                                   int k, uint64_t *scratch)
{
    static_assert(E <= 64 && LANES % 2 == 0 && LANES <= 64, "keys per lane, lanes");
    const int lane = threadIdx.x & 63;
    uint64_t key[E];
    uint64_t m = 0;
#pragma unroll
    for (int s = 0; s < E; ++s) {
        key[s] = ((uint64_t)hi[s] << 32) | lo[s];
        m = key[s] > m ? key[s] : m;
    }
    scratch[lane] = m;
    wave_lds_sync();
    // the lane maxima that are keys are distinct, and more than k - 1 of them
    // are nonzero, so exactly one lane has k - 1 larger maxima
    const int r1 = rank_among(scratch, LANES, m);
    const uint64_t L = readlane64(m, (int)__builtin_ctzll(ballot(lane < LANES && r1 == k - 1)));
    // the keys >= L (L >= 1: no empty slot), in slot-then-lane order
    uint64_t *cs = scratch + 64;
    int c = 0;
#pragma unroll
    for (int s = 0; s < E; ++s) {
        const bool in = key[s] >= L;
        const uint64_t b = ballot(in);
        if (in)
            cs[c + mbcnt(b)] = key[s];
        c += popc(b);
    }
    wave_lds_sync();
    const uint64_t x = lane < c ? cs[lane] : 0ull;
    const int r2 = rank_among(cs, c, x);
    const uint64_t t = readlane64(x, (int)__builtin_ctzll(ballot(lane < c && r2 == k - 1)));
    wave_lds_sync(); // (the scratch may be reused after return)
    return t;
}

__device__ __forceinline__ int block_exclusive_scan(int c, int *scan)
{
    const int lane = threadIdx.x & 63, wave = wave_id();
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

} // namespace
} // namespace dsi
