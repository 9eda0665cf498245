// qproj.hip -- the indexer's query projection on gfx950:
//   q[t][o] = round_DT( sum_i x[t][i] * wq[o][i] ),  o = h * D + d,
// the step just before the scorer ("How I made DeepSeek 12x faster on a Mac
// Studio" names the big Q projection ahead of the indexer; its weights are a
// model parameter).  x [T][K] and wq [O][K] are raw fp16/bf16 bits (both
// K-contiguous, wq in the usual [out][in] layout); q [T][O] is written in the
// same type, which is the [T][H][D] layout the scorer reads.
//
// A plain GEMM on the matrix cores.  A work-group of eight waves computes a
// tile of 256 tokens x 256 features (256 x 128 when O is not a multiple of
// 256); each wave holds 128 x 64 (or 64 x 64) of it as 32 x 32 accumulator
// tiles of v_mfma_f32_32x32x16.  Large tiles keep the operand bytes per flop
// low at both ends: what the work-group pulls from L2 per stage and what each
// wave reads from LDS per MFMA.  K goes in stages of 64 straight from memory
// into LDS (buffer loads with the LDS bit, two stages, 16-byte chunks
// XOR-swizzled so that the fragment reads are free of bank conflicts); within
// a stage the fragments of the 16-wide step two ahead are read while the
// MFMAs of the current one run.  fp32 accumulation, one rounding (to nearest even) at
// the end, and the tile written through LDS as 16-byte row pieces.
// Work-groups are ordered so that the tiles of one XCD share an eighth of the
// weight rows, which then stay in that XCD's L2.
#include "common.hpp"
#include "launch.hpp"

namespace dsi {

namespace {

constexpr int kQpWaves = 8;
constexpr int kQpStage = 64; // K elements per stage
constexpr int kQpTileM = 256; // tokens per work-group (both configurations)

template <int DT>
__device__ __forceinline__ uint16_t to_storage(float v)
{
    if constexpr (DT == kF16)
        return __builtin_bit_cast(uint16_t, (_Float16)v);
    else
        return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// WM x WN waves, each TM x TN accumulator tiles of 32 x 32
template <int DT, int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(kQpWaves * 64) void qproj_kernel(const uint16_t *__restrict__ x,
                                                             const uint16_t *__restrict__ wq,
                                                             int T, int K, int O,
                                                             uint16_t *__restrict__ q)
{
    constexpr int TILEM = WM * TM * 32, TILEN = WN * TN * 32;
    static_assert(WM * WN == kQpWaves && TILEM == kQpTileM, "tile shape");
    constexpr int CPR = kQpStage / 8;            // 16-byte chunks per staged row
    constexpr int A_B = TILEM * kQpStage * 2;    // bytes of one stage of x rows
    constexpr int B_B = TILEN * kQpStage * 2;    // ... of wq rows
    constexpr int LA = A_B / 1024 / kQpWaves;    // 1 KiB loads per wave and stage
    constexpr int LB = B_B / 1024 / kQpWaves;
    constexpr int KS = kQpStage / 16;            // MFMA steps per stage
    constexpr int ROW_B = 32 * CPR * 16;         // bytes of 32 staged rows
    constexpr int SW = TN * 32;                  // width of a wave's output strip
    constexpr int EPW = A_B / (16 * SW * 2);     // output strips per x stage
    static_assert(LA >= 1 && LB >= 1 && LA + LB < 64, "stage loads split over the waves");
    static_assert(kQpWaves <= 2 * EPW, "output strips fit the two x stages");
    // one array per stage and operand, so that the compiler can tell that the
    // loads into one do not touch the fragment reads of another
    __shared__ __attribute__((aligned(1024))) unsigned char sa0[A_B];
    __shared__ __attribute__((aligned(1024))) unsigned char sa1[A_B];
    __shared__ __attribute__((aligned(1024))) unsigned char sb0[B_B];
    __shared__ __attribute__((aligned(1024))) unsigned char sb1[B_B];

    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int col = lane & 31;
    const int hf = lane >> 5;

    // tile of this work-group: consecutive work-groups go to different XCDs,
    // so XCD x = id % 8 takes the feature blocks of its eighth of the weights
    const int nbm = (T + TILEM - 1) / TILEM, nbn = O / TILEN;
    const int id = blockIdx.x;
    int bm, bn;
    if (nbn % 8 == 0) {
        const int per = nbn / 8, i = id / 8;
        bn = (id % 8) * per + i % per;
        bm = i / per;
    } else {
        bn = id % nbn;
        bm = id / nbn;
    }
    if (bm >= nbm)
        return; // (never: the grid is nbm * nbn work-groups)
    const int m0 = bm * TILEM, n0 = bn * TILEN;

    // stage loads: load i of this wave fills 16-byte slots [64 (wave*L+i), +64)
    // of an operand's stage, lane by lane; the lane fetches the chunk that
    // belongs in its slot; chunks past K and rows past T read as 0
    const auto rx = make_rsrc(x, (uint32_t)T * K * 2);
    const auto rw = make_rsrc(wq, (uint32_t)O * K * 2);
    uint32_t xoff[LA], woff[LB];
    int xch[LA], wch[LB]; // first element of the lane's chunk within the stage
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int sl = (wave * LA + i) * 64 + lane;
        const int r = sl / CPR;
        const int c = (sl % CPR) ^ ((r / (16 / CPR)) % CPR);
        xch[i] = c * 8;
        xoff[i] = ((uint32_t)(m0 + r) * K + c * 8) * 2;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int sl = (wave * LB + i) * 64 + lane;
        const int r = sl / CPR;
        const int c = (sl % CPR) ^ ((r / (16 / CPR)) % CPR);
        wch[i] = c * 8;
        woff[i] = ((uint32_t)(n0 + r) * K + c * 8) * 2;
    }
    auto load_stage = [&](int k0, unsigned char *sa, unsigned char *sb) {
#pragma unroll
        for (int i = 0; i < LA; ++i)
            buf_load16_lds(rx, sa + (wave * LA + i) * 1024,
                           k0 + xch[i] < K ? xoff[i] + k0 * 2 : kOffNone);
#pragma unroll
        for (int i = 0; i < LB; ++i)
            buf_load16_lds(rw, sb + (wave * LB + i) * 1024,
                           k0 + wch[i] < K ? woff[i] + k0 * 2 : kOffNone);
    };

    // fragment (t, kk) of this wave: staged row base + t * 32 + col, chunk
    // 2 kk + hf.  The swizzle depends on the row modulo 32 only, so t adds
    // the constant t * ROW_B.
    const int wm = wave / WN, wn = wave % WN;
    uint32_t ak[KS], bk[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        ak[kk] = (uint32_t)stage_slot<CPR>(wm * TM * 32 + col, 2 * kk + hf) * 16;
        bk[kk] = (uint32_t)stage_slot<CPR>(wn * TN * 32 + col, 2 * kk + hf) * 16;
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int mt = 0; mt < TM; ++mt)
#pragma unroll
        for (int nt = 0; nt < TN; ++nt)
            acc[mt][nt] = f32x16{};
    // the fragments of step kk + PF are read before the MFMAs of step kk; the
    // scheduling fences keep that order (left to itself the compiler reads
    // each step's fragments just before its MFMAs, which then wait for them:
    // measured 8-9 % slower)
    auto compute = [&](const unsigned char *sa, const unsigned char *sb) {
        constexpr int PF = 2;
        u32x4 a[PF + 1][TM], b[PF + 1][TN];
        auto rd = [&](int kk, int slot) {
#pragma unroll
            for (int t = 0; t < TM; ++t)
                a[slot][t] = *reinterpret_cast<const u32x4 *>(sa + ak[kk] + t * ROW_B);
#pragma unroll
            for (int t = 0; t < TN; ++t)
                b[slot][t] = *reinterpret_cast<const u32x4 *>(sb + bk[kk] + t * ROW_B);
        };
#pragma unroll
        for (int kk = 0; kk < PF && kk < KS; ++kk)
            rd(kk, kk);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            if (kk + PF < KS)
                rd(kk + PF, (kk + PF) % (PF + 1));
            __builtin_amdgcn_sched_barrier(0);
            const int cur = kk % (PF + 1);
#pragma unroll
            for (int mt = 0; mt < TM; ++mt)
#pragma unroll
                for (int nt = 0; nt < TN; ++nt)
                    acc[mt][nt] = mfma32<DT>(a[cur][mt], b[cur][nt], acc[mt][nt]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // stage s sits in buffer s % 2; stage s + 1 is loaded while stage s is
    // computed, then each wave waits for its own loads and the barrier
    // publishes every wave's (and frees buffer s % 2 for stage s + 2)
    const int nst = (K + kQpStage - 1) / kQpStage;
    load_stage(0, sa0, sb0);
    wait_vmcnt<0>();
    __syncthreads();
    for (int s = 0;; s += 2) {
        if (s + 1 < nst)
            load_stage((s + 1) * kQpStage, sa1, sb1);
        compute(sa0, sb0);
        if (s + 1 >= nst)
            break;
        wait_vmcnt<0>();
        lds_barrier();
        if (s + 2 < nst)
            load_stage((s + 2) * kQpStage, sa0, sb0);
        compute(sa1, sb1);
        if (s + 2 >= nst)
            break;
        wait_vmcnt<0>();
        lds_barrier();
    }
    __syncthreads(); // every wave is done with the stages

    // round and write, per 16-row half of each 32-row strip of the wave's
    // tile: rows into a wave-private LDS region (16 x SW), then out as
    // 16-byte row pieces.  Accumulator entries i = 0..7 hold rows 0..15 of
    // the 32 x 32 tile, i = 8..15 rows 16..31.
    uint16_t *strip = reinterpret_cast<uint16_t *>(wave < EPW ? sa0 : sa1) + (wave % EPW) * 16 * SW;
    const auto rq = make_rsrc(q, (uint32_t)T * O * 2);
#pragma unroll
    for (int mt = 0; mt < TM; ++mt) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int nt = 0; nt < TN; ++nt)
#pragma unroll
                for (int i = 8 * h; i < 8 * h + 8; ++i)
                    strip[(acc_row(i, lane) - 16 * h) * SW + nt * 32 + col] =
                        to_storage<DT>(acc[mt][nt][i]);
            wave_lds_sync();
#pragma unroll
            for (int e = 0; e < TN; ++e) {
                const int c = e * 64 + lane; // piece: row c / (4 TN), columns 8 (c % 4 TN) ..
                const int r = c / (4 * TN), cc = (c % (4 * TN)) * 8;
                const u32x4 v = *reinterpret_cast<const u32x4 *>(strip + r * SW + cc);
                const int row = m0 + wm * TM * 32 + mt * 32 + 16 * h + r;
                const uint32_t off =
                    row < T ? ((uint32_t)row * O + n0 + wn * SW + cc) * 2 : kOffNone;
                __builtin_amdgcn_raw_buffer_store_b128(v, rq, off, 0, 0);
            }
            wave_lds_sync();
        }
    }
}

template <int DT>
hipError_t launch_qproj_dt(const uint16_t *x, const uint16_t *wq, int T, int K, int O, uint16_t *q,
                           hipStream_t st, Timing *tm)
{
    const int nbm = (T + kQpTileM - 1) / kQpTileM;
    if (O % 256 == 0) // 2 x 4 waves of 128 x 64
        return launch_kernel(qproj_kernel<DT, 2, 4, 4, 2>, dim3(nbm * (O / 256)),
                             dim3(kQpWaves * 64), 0, st, tm, true, true, x, wq, T, K, O, q);
    // 4 x 2 waves of 64 x 64
    return launch_kernel(qproj_kernel<DT, 4, 2, 2, 2>, dim3(nbm * (O / 128)), dim3(kQpWaves * 64),
                         0, st, tm, true, true, x, wq, T, K, O, q);
}

} // namespace

hipError_t launch_qproj(const void *x, const void *wq, int T, int K, int O, int dtype, void *q,
                        hipStream_t st, Timing *tm)
{
    if (T <= 0)
        return hipSuccess;
    const auto *xs = static_cast<const uint16_t *>(x);
    const auto *ws = static_cast<const uint16_t *>(wq);
    auto *qs = static_cast<uint16_t *>(q);
    if (dtype == kF16)
        return launch_qproj_dt<kF16>(xs, ws, T, K, O, qs, st, tm);
    return launch_qproj_dt<kBF16>(xs, ws, T, K, O, qs, st, tm);
}

} // namespace dsi
