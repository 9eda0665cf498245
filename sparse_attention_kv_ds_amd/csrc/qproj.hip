// qproj.hip -- the indexer's query projection on gfx950:
//   q[t][o] = round_DT( sum_i x[t][i] * wq[o][i] ),  o = h * D + d,
// the step just before the scorer ("How I made DeepSeek 12x faster on a Mac
// Studio" names the big Q projection ahead of the indexer; its weights are a
// model parameter).  x [T][K] and wq [O][K] are raw fp16/bf16 bits (both
// K-contiguous, wq in the usual [out][in] layout); q [T][O] is written in the
// same type, which is the [T][H][D] layout the scorer reads.
//
// A plain GEMM on the matrix cores: work-group tiles of 128 tokens x 128
// features, four waves of 64 x 64 (2 x 2 tiles of v_mfma_f32_32x32x16), K in
// stages of 64 that go straight from memory into LDS (buffer loads with the
// LDS bit, two stages, 16-byte chunks XOR-swizzled so that the fragment reads
// are free of bank conflicts), fp32 accumulation, one rounding (to nearest
// even) at the end, and the tile written through LDS as 16-byte stores.
// Work-groups are ordered so that the tiles of one XCD share an eighth of the
// weight rows, which then stay in that XCD's L2.
#include "common.hpp"
#include "internal.hpp"

namespace dsi {

namespace {

constexpr int kQpTile = 128;   // tokens and features per work-group
constexpr int kQpStage = 64;   // K elements per stage
constexpr int kQpWaves = 4;

template <int DT>
__device__ __forceinline__ uint16_t to_storage(float v)
{
    if constexpr (DT == kF16)
        return __builtin_bit_cast(uint16_t, (_Float16)v);
    else
        return __builtin_bit_cast(uint16_t, (__bf16)v);
}

template <int DT>
__global__ __launch_bounds__(kQpWaves * 64) void qproj_kernel(const uint16_t *__restrict__ x,
                                                             const uint16_t *__restrict__ wq,
                                                             int T, int K, int O,
                                                             uint16_t *__restrict__ q)
{
    constexpr int CPR = kQpStage / 8;                 // 16-byte chunks per staged row
    constexpr int TILE_B = kQpTile * kQpStage * 2;    // bytes of one operand's stage
    constexpr int LPW = TILE_B / 1024 / kQpWaves;     // 1 KiB loads per wave and operand
    constexpr int KS = kQpStage / 16;                 // MFMA steps per stage
    // separate arrays per stage and operand, so that the compiler can tell that
    // the loads into one do not touch the fragment reads of another
    __shared__ __attribute__((aligned(1024))) unsigned char sa0[TILE_B];
    __shared__ __attribute__((aligned(1024))) unsigned char sb0[TILE_B];
    __shared__ __attribute__((aligned(1024))) unsigned char sa1[TILE_B];
    __shared__ __attribute__((aligned(1024))) unsigned char sb1[TILE_B];

    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int col = lane & 31;
    const int hf = lane >> 5;

    // tile of this work-group: consecutive work-groups go to different XCDs,
    // so XCD x = id % 8 takes the feature blocks of its eighth of the weights
    const int nbm = (T + kQpTile - 1) / kQpTile, nbn = O / kQpTile;
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
    const int m0 = bm * kQpTile, n0 = bn * kQpTile;

    // stage loads: load i of this wave fills 16-byte slots [64 (wave*LPW+i), +64)
    // of each operand's stage, lane by lane; the lane fetches the chunk that
    // belongs in its slot; chunks past K and rows past T read as 0
    const auto rx = make_rsrc(x, (uint32_t)T * K * 2);
    const auto rw = make_rsrc(wq, (uint32_t)O * K * 2);
    uint32_t xoff[LPW], woff[LPW];
    int kch[LPW]; // first element of the lane's chunk within the stage
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int s = (wave * LPW + i) * 64 + lane;
        const int r = s / CPR;
        const int c = (s % CPR) ^ ((r / (16 / CPR)) % CPR);
        kch[i] = c * 8;
        xoff[i] = ((uint32_t)(m0 + r) * K + c * 8) * 2;
        woff[i] = ((uint32_t)(n0 + r) * K + c * 8) * 2;
    }
    auto load_stage = [&](int k0, unsigned char *sa, unsigned char *sb) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const bool in = k0 + kch[i] < K;
            buf_load16_lds(rx, sa + (wave * LPW + i) * 1024, in ? xoff[i] + k0 * 2 : kOffNone);
            buf_load16_lds(rw, sb + (wave * LPW + i) * 1024, in ? woff[i] + k0 * 2 : kOffNone);
        }
    };

    // fragment offsets: this wave's 64 x 64 sub-tile is rows wm*64.. of x,
    // rows wn*64.. of wq; fragment (t, kk) is row t*32 + col, chunk 2 kk + hf
    const int wm = wave >> 1, wn = wave & 1;
    uint32_t aoff[2][KS], boff[2][KS];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            aoff[t][kk] = (uint32_t)stage_slot<CPR>(wm * 64 + t * 32 + col, 2 * kk + hf) * 16;
            boff[t][kk] = (uint32_t)stage_slot<CPR>(wn * 64 + t * 32 + col, 2 * kk + hf) * 16;
        }

    f32x16 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = f32x16{};
    auto compute = [&](const unsigned char *sa, const unsigned char *sb) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            u32x4 a[2], b[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                a[t] = *reinterpret_cast<const u32x4 *>(sa + aoff[t][kk]);
                b[t] = *reinterpret_cast<const u32x4 *>(sb + boff[t][kk]);
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    acc[mt][nt] = mfma32<DT>(a[mt], b[nt], acc[mt][nt]);
        }
    };

    const int nst = (K + kQpStage - 1) / kQpStage;
    load_stage(0, sa0, sb0);
    wait_vmcnt<0>();
    __syncthreads();
    // two stages per iteration, so that every LDS offset is a constant
    for (int s = 0;;) {
        if (s + 1 < nst)
            load_stage((s + 1) * kQpStage, sa1, sb1);
        compute(sa0, sb0);
        wait_vmcnt<0>();
        lds_barrier();
        if (++s >= nst)
            break;
        if (s + 1 < nst)
            load_stage((s + 1) * kQpStage, sa0, sb0);
        compute(sa1, sb1);
        wait_vmcnt<0>();
        lds_barrier();
        if (++s >= nst)
            break;
    }

    // round and write: each wave's 64 x 64 sub-tile goes row-major into LDS
    // (waves 0, 1 in the first stage's x array, 2, 3 in its wq array), then out
    // as 16-byte rows pieces
    uint16_t *tile = reinterpret_cast<uint16_t *>((wave < 2 ? sa0 : sb0) + (wave & 1) * 8192);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                tile[(mt * 32 + acc_row(i, lane)) * 64 + nt * 32 + col] =
                    to_storage<DT>(acc[mt][nt][i]);
    wave_lds_sync();
    const auto rq = make_rsrc(q, (uint32_t)T * O * 2);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int c = e * 64 + lane; // 16-byte piece: row c / 8, columns 8 (c % 8) ..
        const int r = c >> 3, cc = (c & 7) * 8;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(tile + r * 64 + cc);
        const int row = m0 + wm * 64 + r;
        const uint32_t off =
            row < T ? ((uint32_t)row * O + n0 + wn * 64 + cc) * 2 : kOffNone;
        __builtin_amdgcn_raw_buffer_store_b128(v, rq, off, 0, 0);
    }
}

} // namespace

bool qproj_supported(int K, int O, int dtype)
{
    return K >= 8 && K % 8 == 0 && O % kQpTile == 0 && (dtype == kF16 || dtype == kBF16);
}

hipError_t launch_qproj(const void *x, const void *wq, int T, int K, int O, int dtype, void *q,
                        hipStream_t st, Timing *tm)
{
    if (T <= 0)
        return hipSuccess;
    const int blocks = (T + kQpTile - 1) / kQpTile * (O / kQpTile);
    const auto *xs = static_cast<const uint16_t *>(x);
    const auto *ws = static_cast<const uint16_t *>(wq);
    auto *qs = static_cast<uint16_t *>(q);
    if (dtype == kF16)
        return launch_kernel(qproj_kernel<kF16>, dim3(blocks), dim3(kQpWaves * 64), 0, st, tm, true,
                             true, xs, ws, T, K, O, qs);
    return launch_kernel(qproj_kernel<kBF16>, dim3(blocks), dim3(kQpWaves * 64), 0, st, tm, true,
                         true, xs, ws, T, K, O, qs);
}

} // namespace dsi
