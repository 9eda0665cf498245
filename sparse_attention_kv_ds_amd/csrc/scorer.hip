// scorer.hip -- lightning-indexer scorer kernels for gfx950.
//
// s[t,j] = sum_h w[t,h] * max(0, q[t,h,:] . k[j,:]) for every visible row j
// (the scorer of "How I made DeepSeek 12x faster on a Mac Studio", section
// "1: the kernels": Q and K are packed to half precision once and K tiles are
// read from on-chip memory instead of being re-read from device memory for
// every scored pair).
//
// The contraction Q . K^T is a dense GEMM with M = (token, head) rows of the
// flattened Q [T*H][D], N = compressed rows, K-dim = D; it runs on the
// 32x32x16 fp16/bf16 MFMA.  Each wave keeps 64 (token, head) rows of Q as A
// fragments in registers for its whole lifetime (the register-resident
// operand); 32-row tiles of K are staged once per work-group through LDS and
// shared by all of its waves.  The epilogue works straight on the MFMA
// accumulators: ReLU, multiply by the head weight, and the sum over the heads
// of a token, which is mostly in-lane (a lane's 16 accumulators of one 32-row
// tile are 16 different heads of one row j) plus one exchange between the two
// half-waves.
#include "common.hpp"
#include "internal.hpp"

namespace dsi {

namespace {

constexpr int kPrefillWaves = 8;    // waves per prefill work-group
constexpr int kChunkRows = 1024;    // compressed rows per prefill work-group

// ---------------------------------------------------------------------------
// prefill: blockIdx.x = tile of 64*WAVES (token, head) rows, blockIdx.y = chunk
// of chunk_rows compressed rows.
// ---------------------------------------------------------------------------
template <int H, int D, int DT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void prefill_scorer_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ w,
    const int32_t *__restrict__ pos, int T, int N, int ratio, int min_rows, int chunk_rows,
    float *__restrict__ S, long long ldS)
{
    constexpr int TPW = 64 / H;           // tokens per wave
    constexpr int TPB = TPW * WAVES;      // tokens per work-group
    constexpr int KS = D / 16;            // MFMA steps along D
    constexpr int ROWB = D * 2 + 16;      // LDS bytes per K row (16-byte pad against bank conflicts)
    constexpr int CPR = D / 8;            // 16-byte chunks per K row
    constexpr int NCH = 32 * CPR;         // 16-byte chunks per 32-row tile
    constexpr int NTHR = WAVES * 64;
    constexpr int CPT = (NCH + NTHR - 1) / NTHR;

    __shared__ __attribute__((aligned(16))) unsigned char kt[2][32 * ROWB];
    __shared__ int s_n[TPB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int hf = lane >> 5;
    const int tok_base = blockIdx.x * TPB;
    const int j_chunk = blockIdx.y * chunk_rows;

    // visible rows of the tile's tokens; 0 for tokens past T and for tokens
    // that need no scoring (all their rows fit)
    for (int i = tid; i < TPB; i += NTHR) {
        const int t = tok_base + i;
        const int n = t < T ? visible_rows(pos[t], ratio, N) : 0;
        s_n[i] = n > min_rows ? n : 0;
    }
    __syncthreads();
    int nmax = 0;
    for (int i = 0; i < TPB; ++i)
        nmax = max(nmax, s_n[i]);
    const int j_end = min(j_chunk + chunk_rows, nmax);
    if (j_chunk >= j_end)
        return; // the same decision in every thread of the work-group

    int wn[TPW];
    int wnmax = 0;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        wn[i] = s_n[wave * TPW + i];
        wnmax = max(wnmax, wn[i]);
    }

    // A fragments and head weights of this wave's 64 rows of the flattened Q
    const long long row0 = (long long)(tok_base + wave * TPW) * H;
    const long long rows_total = (long long)T * H;
    u32x4 a[2][KS];
    float wr[2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const long long r = row0 + mt * 32 + col;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            if (wnmax > 0 && r < rows_total)
                a[mt][kk] = *reinterpret_cast<const u32x4 *>(q + r * D + kk * 16 + 8 * hf);
            else
                a[mt][kk] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const long long rr = row0 + mt * 32 + acc_row(i, lane);
            wr[mt][i] = (wnmax > 0 && rr < rows_total) ? w[rr] : 0.f;
        }
    }

    u32x4 stage[CPT];
    auto load_tile = [&](int j0) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int ch = tid + c * NTHR;
            const int j = j0 + ch / CPR;
            if (ch < NCH && j < N)
                stage[c] = *reinterpret_cast<const u32x4 *>(k + (long long)j * D + (ch % CPR) * 8);
            else
                stage[c] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_tile = [&](int b) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int ch = tid + c * NTHR;
            if (ch < NCH)
                *reinterpret_cast<u32x4 *>(&kt[b][(ch / CPR) * ROWB + (ch % CPR) * 16]) = stage[c];
        }
    };

    load_tile(j_chunk);
    store_tile(0);
    __syncthreads();

    int buf = 0;
    for (int j0 = j_chunk; j0 < j_end; j0 += 32) {
        const bool more = j0 + 32 < j_end;
        if (more)
            load_tile(j0 + 32);
        if (j0 < wnmax) {
            f32x16 acc0 = {}, acc1 = {};
            const unsigned char *bp = &kt[buf][col * ROWB + hf * 16];
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const u32x4 b = *reinterpret_cast<const u32x4 *>(bp + kk * 32);
                acc0 = mfma32<DT>(a[0][kk], b, acc0);
                acc1 = mfma32<DT>(a[1][kk], b, acc1);
            }
            const int j = j0 + col;
            if constexpr (H >= 8) {
                // the token of accumulator (mt, i) does not depend on the lane here
                float part[TPW];
#pragma unroll
                for (int tk = 0; tk < TPW; ++tk)
                    part[tk] = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int tk0 = (8 * (i >> 2)) / H;
                    const int tk1 = (32 + 8 * (i >> 2)) / H;
                    part[tk0] = fmaf(wr[0][i], fmaxf(acc0[i], 0.f), part[tk0]);
                    part[tk1] = fmaf(wr[1][i], fmaxf(acc1[i], 0.f), part[tk1]);
                }
#pragma unroll
                for (int tk = 0; tk < TPW; ++tk)
                    part[tk] += __shfl_xor(part[tk], 32);
                // half-wave 0 stores even tokens, half-wave 1 odd ones
#pragma unroll
                for (int tk = 0; tk < TPW; tk += 2) {
                    float v = part[tk];
                    int nn = wn[tk];
                    if constexpr (TPW > 1) {
                        if (hf) {
                            v = part[tk + 1];
                            nn = wn[tk + 1];
                        }
                    } else {
                        if (hf)
                            nn = 0;
                    }
                    if (j < nn)
                        S[(long long)(tok_base + wave * TPW + tk + hf) * ldS + j] = v;
                }
            } else {
                // H == 4: token of (mt, i) = mt*8 + 2*(i/4) + half-wave; its 4
                // heads sit in 4 consecutive registers of one lane
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float v = 0.f;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float x = mt ? acc1[4 * g + e] : acc0[4 * g + e];
                            v = fmaf(wr[mt][4 * g + e], fmaxf(x, 0.f), v);
                        }
                        const int tk = mt * 8 + 2 * g + hf;
                        if (j < s_n[wave * TPW + tk])
                            S[(long long)(tok_base + wave * TPW + tk) * ldS + j] = v;
                    }
                }
            }
        }
        if (more)
            store_tile(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
}

// ---------------------------------------------------------------------------
// decode (T == 1): every wave owns the token's H heads (as 64 rows, zero
// padded) and walks the 32-row blocks of K with a grid-wide stride, loading B
// fragments straight from global memory one block ahead.
// ---------------------------------------------------------------------------
template <int H, int D, int DT>
__global__ __launch_bounds__(256) void decode_scorer_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ w,
    const int32_t *__restrict__ pos, int N, int ratio, int min_rows, float *__restrict__ S)
{
    constexpr int KS = D / 16;
    constexpr int MT = H > 32 ? 2 : 1;
    const int lane = threadIdx.x & 63;
    const int col = lane & 31;
    const int hf = lane >> 5;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nw = gridDim.x * 4;

    const int n = visible_rows(pos[0], ratio, N);
    if (n <= min_rows)
        return;
    const int nblk = (n + 31) / 32;
    if (gw >= nblk)
        return;

    u32x4 a[MT][KS];
    float wr[MT][16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int h = mt * 32 + col;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            a[mt][kk] = h < H ? *reinterpret_cast<const u32x4 *>(q + h * D + kk * 16 + 8 * hf)
                              : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int hh = mt * 32 + acc_row(i, lane);
            wr[mt][i] = hh < H ? w[hh] : 0.f;
        }
    }

    u32x4 b[KS], bn[KS];
    auto load_b = [&](int blk, u32x4(&dst)[KS]) {
        const int j = blk * 32 + col;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            dst[kk] = j < N ? *reinterpret_cast<const u32x4 *>(k + (long long)j * D + kk * 16 + 8 * hf)
                            : u32x4{0u, 0u, 0u, 0u};
    };
    load_b(gw, b);
    for (int blk = gw; blk < nblk; blk += nw) {
        const int nxt = blk + nw;
        if (nxt < nblk)
            load_b(nxt, bn);
        f32x16 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            acc[mt] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                acc[mt] = mfma32<DT>(a[mt][kk], b[kk], acc[mt]);
        }
        float s = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                s = fmaf(wr[mt][i], fmaxf(acc[mt][i], 0.f), s);
        s += __shfl_xor(s, 32);
        const int j = blk * 32 + col;
        if (hf == 0 && j < n)
            S[j] = s;
        if (nxt < nblk) {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                b[kk] = bn[kk];
        }
    }
}

__global__ void fill_kernel(float *__restrict__ p, long long n, float v)
{
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x)
        p[i] = v;
}

template <int H, int D, int DT>
hipError_t prefill_one(const Problem &p, int min_rows, float *S, long long ldS, hipStream_t st)
{
    constexpr int TPB = (64 / H) * kPrefillWaves;
    const dim3 grid((p.T + TPB - 1) / TPB, (p.N + kChunkRows - 1) / kChunkRows);
    hipLaunchKernelGGL((prefill_scorer_kernel<H, D, DT, kPrefillWaves>), grid,
                       dim3(kPrefillWaves * 64), 0, st, (const uint16_t *)p.q,
                       (const uint16_t *)p.k, p.w, p.pos, p.T, p.N, p.ratio, min_rows,
                       kChunkRows, S, ldS);
    return hipGetLastError();
}

template <int H, int D, int DT>
hipError_t decode_one(const Problem &p, int min_rows, float *S, hipStream_t st)
{
    const int nblk = (p.N + 31) / 32;
    int blocks = (nblk + 3) / 4;
    if (blocks > 512)
        blocks = 512;
    hipLaunchKernelGGL((decode_scorer_kernel<H, D, DT>), dim3(blocks), dim3(256), 0, st,
                       (const uint16_t *)p.q, (const uint16_t *)p.k, p.w, p.pos, p.N, p.ratio,
                       min_rows, S);
    return hipGetLastError();
}

// (H, D, dtype) -> instantiation
template <template <int, int, int> class F, typename... A>
hipError_t dispatch(int H, int D, int dt, A... args)
{
#define DSI_CASE(h, d)                                                                    \
    if (H == h && D == d)                                                                 \
        return dt == kF16 ? F<h, d, kF16>::run(args...) : F<h, d, kBF16>::run(args...);
#define DSI_ROW(h) DSI_CASE(h, 32) DSI_CASE(h, 64) DSI_CASE(h, 128)
    DSI_ROW(4) DSI_ROW(8) DSI_ROW(16) DSI_ROW(32) DSI_ROW(64)
#undef DSI_ROW
#undef DSI_CASE
    return hipErrorInvalidValue;
}

template <int H, int D, int DT> struct PrefillF {
    static hipError_t run(const Problem &p, int m, float *S, long long ld, hipStream_t st)
    {
        return prefill_one<H, D, DT>(p, m, S, ld, st);
    }
};
template <int H, int D, int DT> struct DecodeF {
    static hipError_t run(const Problem &p, int m, float *S, hipStream_t st)
    {
        return decode_one<H, D, DT>(p, m, S, st);
    }
};

} // namespace

bool scorer_supported(int H, int D, int dtype)
{
    const bool h = H == 4 || H == 8 || H == 16 || H == 32 || H == 64;
    const bool d = D == 32 || D == 64 || D == 128;
    return h && d && (dtype == kF16 || dtype == kBF16);
}

hipError_t launch_prefill_scorer(const Problem &p, int min_rows, float *S, long long ldS,
                                 hipStream_t st)
{
    if (p.T <= 0 || p.N <= 0)
        return hipSuccess;
    return dispatch<PrefillF>(p.H, p.D, p.dtype, p, min_rows, S, ldS, st);
}

hipError_t launch_decode_scorer(const Problem &p, int min_rows, float *S, hipStream_t st)
{
    if (p.T <= 0 || p.N <= 0)
        return hipSuccess;
    return dispatch<DecodeF>(p.H, p.D, p.dtype, p, min_rows, S, st);
}

hipError_t launch_fill(float *p, long long n, float v, hipStream_t st)
{
    if (n <= 0)
        return hipSuccess;
    long long blocks = (n + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

} // namespace dsi
