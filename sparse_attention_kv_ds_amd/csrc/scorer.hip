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
#include "launch.hpp"
#include "select.hpp"

namespace dsi {

namespace {

constexpr int kChunkRows = 2048;    // compressed rows per prefill work-group (multiple of 64)
constexpr int kStageRows = 64;      // K rows per LDS stage (two 32-row blocks)

// ---------------------------------------------------------------------------
// prefill: blockIdx.x = tile of 64*WAVES (token, head) rows, blockIdx.y = chunk
// of chunk_rows compressed rows (a multiple of the 64-row LDS stage).
//
// K moves through two LDS stages of 64 rows.  The loads go straight from
// memory into LDS (buffer loads with the LDS bit: no registers, no LDS write
// instructions), unpadded, with the 16-byte chunks of each row swizzled so that
// the MFMA fragment reads are free of bank conflicts; every lane's fragment
// addresses are computed once.  The loads of stage s+1 are issued as stage s
// starts; at its end each wave waits for its own loads (vmcnt, not counting the
// score stores issued since) and one barrier publishes them to the group.
//
// Per 64-row stage: 2 blocks of 32 rows, each its 16 MFMAs then its epilogue
// (one accumulator pair per wave keeps the kernel at three waves per SIMD, so
// that other waves' MFMAs cover each wave's epilogue).  Rows past N read as 0
// and masked score stores are dropped (buffer-resource ranges).
//
// Output: with SPLIT == false, token t's scores as fp32 at S + t ldS.  With
// SPLIT, the split scores of the streaming top-k (common.hpp: per 32-row
// block, the rows' high halves, then their low halves), so that the
// selection loads the high halves and the low halves only for the rows it
// cannot order by the high ones.  The same bytes are written either way, one
// 128-byte line per block; with one token per wave the two half-waves store
// the two halves of a block (one store instruction per block, as for fp32).
// ---------------------------------------------------------------------------
template <int H, int D, int DT, int WAVES, int SR, bool SPLIT>
__global__ __launch_bounds__(WAVES * 64) void prefill_scorer_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ w,
    const int32_t *__restrict__ pos, int T, int N, int ratio, int min_rows, int chunk_rows,
    float *__restrict__ S, long long ldS)
{
    constexpr int TPW = 64 / H;       // tokens per wave
    constexpr int TPB = TPW * WAVES;  // tokens per work-group
    constexpr int KS = D / 16;        // MFMA steps along D
    constexpr int CPR = D / 8;        // 16-byte chunks per K row
    static_assert(SR % 64 == 0, "stages of whole pairs of 32-row blocks");
    constexpr int STAGE_B = SR * D * 2;            // bytes of one stage
    constexpr int LPW = SR * CPR / 64 / WAVES;     // 1 KiB LDS loads per wave per stage
    static_assert(SR * CPR % (64 * WAVES) == 0, "stage must split evenly over the waves");

    // the two stages are separate arrays so that the compiler can tell that
    // the loads into one do not touch the fragment reads of the other
    __shared__ __attribute__((aligned(1024))) unsigned char kt0[STAGE_B];
    __shared__ __attribute__((aligned(1024))) unsigned char kt1[STAGE_B];
    __shared__ int s_n[TPB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = wave_id();
    const int col = lane & 31;
    const int hf = lane >> 5;
    const int tok_base = blockIdx.x * TPB;
    const int j_chunk = blockIdx.y * chunk_rows;

    // visible rows of the tile's tokens; 0 for tokens past T and for tokens
    // that need no scoring (all their rows fit)
    for (int i = tid; i < TPB; i += WAVES * 64) {
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

    // K stage loads: load i of this wave fills LDS slots [64 (wave*LPW + i), +64)
    // lane by lane; the lane fetches the chunk that belongs in its slot
    const auto rk = make_rsrc(k, (uint32_t)N * D * 2);
    uint32_t kvoff[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int s = (wave * LPW + i) * 64 + lane;
        const int r = s / CPR;
        const int c = (s % CPR) ^ ((r / (16 / CPR)) % CPR);
        kvoff[i] = (uint32_t)(r * CPR + c) * 16;
    }
    auto load_stage = [&](int j0, unsigned char *kt) {
        const uint32_t base = (uint32_t)j0 * D * 2;
#pragma unroll
        for (int i = 0; i < LPW; ++i)
            buf_load16_lds(rk, kt + (wave * LPW + i) * 1024, base + kvoff[i]);
    };
    load_stage(j_chunk, kt0);

    // tokens this lane stores: half-wave hf stores tokens hf, hf+2, ... of the
    // wave (H >= 8) or tokens 2g + hf of each 8-token tile (H == 4)
    constexpr int NST = H == 4 ? 8 : (TPW + 1) / 2;
    // store instructions per block: one per token slot, two (one per half)
    // for split scores when a lane holds a whole token's score
    constexpr int NSTORE = SPLIT && TPW > 1 ? 2 * NST : NST;
    int st_n[NST], st_tok[NST];
#pragma unroll
    for (int e = 0; e < NST; ++e) {
        int tk;
        if constexpr (H == 4)
            tk = (e >> 2) * 8 + 2 * (e & 3) + hf;
        else if constexpr (SPLIT && TPW == 1)
            tk = 0; // both half-waves store the wave's one token (one half each)
        else
            tk = 2 * e + hf;
        st_tok[e] = wave * TPW + tk;
        st_n[e] = tk < TPW ? s_n[wave * TPW + tk] : 0;
    }

    const int t_here = min(TPB, T - tok_base);
    const auto rq = make_rsrc(q + (long long)tok_base * H * D, (uint32_t)t_here * H * D * 2);
    const auto rw = make_rsrc(w + (long long)tok_base * H, (uint32_t)t_here * H * 4);
    const auto rs = make_rsrc(S + (long long)tok_base * ldS, (uint32_t)(t_here * ldS * 4));

    // A fragments (this wave's 64 rows of the flattened Q) and head weights
    u32x4 a[2][KS];
    float wr[2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const uint32_t r = wave * 64 + mt * 32 + col;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            a[mt][kk] = buf_load16(rq, (r * D + kk * 16 + 8 * hf) * 2);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            wr[mt][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rw, (uint32_t)(wave * 64 + mt * 32 + acc_row(i, lane)) * 4, 0, 0));
    }

    // this lane's B fragment byte offsets within a 32-row block: row col,
    // chunk 2 kk + hf (elements 16 kk + 8 hf ..)
    uint32_t boff[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
        boff[kk] = (uint32_t)stage_slot<CPR>(col, 2 * kk + hf) * 16;

    // (split scores, one token per wave: the shift that leaves this half-wave's
    // 16 bits of an ordered score at the bottom)
    const uint32_t lo_shift = hf ? 0u : 16u;
    (void)lo_shift;

    // Lane-local partial sums of the epilogue: slot = token of the lane (see
    // st_tok), two interleaved sums per slot for instruction-level parallelism.
    constexpr int NSLOT = H == 4 ? 8 : TPW;
    // accumulator (mt, i) -> slot
    auto slot_of = [](int mt, int i) constexpr {
        return H == 4 ? mt * 4 + (i >> 2) : (32 * mt + 8 * (i >> 2)) / H;
    };

    // One 32-row block of K (LDS rows at kb, compressed rows jb..jb+31): the
    // MFMAs into c0/c1, then ReLU, head weight and the sum over each token's
    // heads, and the store of s[t][jb + col].  The VALU work of one wave's
    // epilogue runs while the other waves of its SIMD keep the matrix core
    // busy (three waves fit: one accumulator pair per wave).
    auto block = [&](const unsigned char *kb, int jb) __attribute__((always_inline)) {
        f32x16 c0 = f32x16{}, c1 = f32x16{};
        // the K fragments are read PF steps ahead of their MFMAs; the
        // scheduling fences keep that order (left to itself the compiler reads
        // one step ahead, and each MFMA pair then waits for its LDS read:
        // measured 2-8 % slower)
        constexpr int PF = 2;
        u32x4 bq[PF + 1];
#pragma unroll
        for (int kk = 0; kk < PF && kk < KS; ++kk)
            bq[kk] = *reinterpret_cast<const u32x4 *>(kb + boff[kk]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            if (kk + PF < KS)
                bq[(kk + PF) % (PF + 1)] = *reinterpret_cast<const u32x4 *>(kb + boff[kk + PF]);
            __builtin_amdgcn_sched_barrier(0);
            c0 = mfma32<DT>(a[0][kk], bq[kk % (PF + 1)], c0);
            c1 = mfma32<DT>(a[1][kk], bq[kk % (PF + 1)], c1);
            __builtin_amdgcn_sched_barrier(0);
        }
        float part[NSLOT][2];
#pragma unroll
        for (int sl = 0; sl < NSLOT; ++sl)
            part[sl][0] = part[sl][1] = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            part[slot_of(0, i)][i & 1] = fmaf(wr[0][i], fmaxf(c0[i], 0.f), part[slot_of(0, i)][i & 1]);
            part[slot_of(1, i)][i & 1] = fmaf(wr[1][i], fmaxf(c1[i], 0.f), part[slot_of(1, i)][i & 1]);
        }
        const int j = jb + col;
#pragma unroll
        for (int e = 0; e < NST; ++e) {
            float v;
            if constexpr (H == 4) {
                v = part[e][0] + part[e][1]; // all 4 heads of the token are in this lane
            } else {
                // both half-waves hold a part of every token: add the halves
                const float v0 = add_other_half(part[2 * e][0] + part[2 * e][1]);
                v = v0;
                if constexpr (TPW > 1) {
                    const float v1 = add_other_half(part[2 * e + 1][0] + part[2 * e + 1][1]);
                    v = hf ? v1 : v0;
                }
            }
            const bool ok = (unsigned)j < (unsigned)st_n[e];
            if constexpr (!SPLIT) {
                buf_store_f32(rs, ok ? (uint32_t)((st_tok[e] * ldS + j) * 4) : kOffNone, v);
            } else {
                // ordered_score(v) without its -0 fold: v is never -0 (every
                // sum here starts from +0, and a round-to-nearest sum or
                // fused multiply-add reaches -0 only from -0 operands)
                const uint32_t b = __float_as_uint(v);
                const uint32_t ov = b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
                // (the block is one group of split scores: jb is a multiple of 32)
                static_assert(kSplitRows == 32, "one 32-row block per group");
                const uint32_t hi_off = (uint32_t)(st_tok[e] * ldS * 4) +
                                        split_hi_off((uint32_t)jb) + split_hi_off((uint32_t)col);
                if constexpr (TPW == 1) {
                    // (both halves hold v: the lower stores the high bits)
                    buf_store_u16(rs, ok ? hi_off + kSplitLow * hf : kOffNone, ov >> lo_shift);
                } else {
                    buf_store_u16(rs, ok ? hi_off : kOffNone, ov >> 16);
                    buf_store_u16(rs, ok ? hi_off + kSplitLow : kOffNone, ov);
                }
            }
        }
    };

    // the blocks of one stage (rows js.. in LDS at kt)
    auto run_stage = [&](const unsigned char *kt, int js) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < SR / 32; ++b) {
            if (b > 0 && js + 32 * b >= j_end)
                break; // the rest of the last stage is past every token's rows
            block(kt + 32 * b * D * 2, js + 32 * b);
        }
    };
    // end of a stage: this wave's loads of the next stage have landed (the
    // score stores issued after them, NST per block, may still be in flight),
    // then every wave's have
    auto stage_done = [&]() {
        wait_vmcnt<SR / 32 * NSTORE>();
        lds_barrier();
    };

    wait_vmcnt<0>(); // stage 0, the query rows and the weights
    __syncthreads();
    // two stages per iteration, so that every LDS offset is a constant
    for (int js = j_chunk;;) {
        if (js + SR < j_end)
            load_stage(js + SR, kt1);
        run_stage(kt0, js);
        stage_done();
        js += SR;
        if (js >= j_end)
            break;
        if (js + SR < j_end)
            load_stage(js + SR, kt0);
        run_stage(kt1, js);
        stage_done();
        js += SR;
        if (js >= j_end)
            break;
    }
}

// ---------------------------------------------------------------------------
// decode (T == 1): work-groups of WAVES waves; each wave scores NB consecutive
// 32-row blocks of K.  Decode is bound by the K stream, so the kernel keeps as
// many K bytes in flight per CU as LDS allows, all the time: every K block
// goes straight from memory into one of two LDS slots of its wave (buffer
// loads with the LDS bit, non-temporal: each byte is read once per call); as
// soon as block b has landed, the wave copies its MFMA fragments into
// registers and reuses the slot for block b+2, then computes block b while
// b+1 and b+2 are in flight.  The query rows are staged once per work-group
// in LDS.  The 16-byte chunks of every staged row are swizzled so that the
// fragment reads are free of bank conflicts.  (Loading MFMA fragments straight
// into registers would read 32 bytes from each of 32 rows per instruction,
// which the memory system serves markedly slower.)  No load waits for pos: K
// rows past the visible count are fetched and dropped (the caller passes the
// rows that exist, so at decode nearly all are visible).
// ---------------------------------------------------------------------------
// K loads marked non-temporal: every byte of K is read once per call
constexpr int kStreamAux = 2;

// phase timestamps of the decode scorer (stamps build only), record = work-group
// (blockIdx.y * gridDim.x + blockIdx.x): 0 start, 1 query and first blocks in
// LDS, 2 + w wave w's last block scored, 6 partition list written
DSI_STAMP_ARRAY(decode_stamps);

template <int H, int D, int DT, int WAVES, int NB>
__global__ __launch_bounds__(WAVES * 64) void decode_scorer_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ w,
    const int32_t *__restrict__ pos, int N, int ratio, int min_rows, float *__restrict__ S, int kp,
    uint64_t *__restrict__ cand, int *__restrict__ pcount, uint64_t *__restrict__ pmin,
    long long ldS)
{
    const long long stamp_rec = (long long)blockIdx.y * gridDim.x + blockIdx.x;
    (void)stamp_rec; // (only the stamps build records)
    DSI_STAMP(decode_stamps, stamp_rec, 0, threadIdx.x == 0);
    // sequence blockIdx.y of a batched call (0 for a single token)
    {
        const int sb = blockIdx.y;
        q += (size_t)sb * H * D;
        k += (size_t)sb * N * D;
        w += sb * H;
        pos += sb;
        S += sb * ldS;
        if (cand) {
            cand += (size_t)sb * kDecodeUnion;
            pcount += sb * kDecodeMaxParts;
            pmin += sb * kDecodeMaxParts;
        }
    }
    constexpr int KS = D / 16;
    constexpr int MT = H > 32 ? 2 : 1;       // 32-head tiles of the query
    constexpr int CPR = D / 8;               // 16-byte chunks per row
    constexpr int BLK_B = 32 * D * 2;        // bytes of one 32-row block
    constexpr int KPB = BLK_B / 1024;        // 1 KiB loads per K block
    constexpr int QL = MT * 32 * CPR / 64;   // 1 KiB loads of the query, whole group
    constexpr int QLW = (QL + WAVES - 1) / WAVES;
    static_assert(BLK_B % 1024 == 0, "whole 1 KiB loads per block");
    static_assert(NB >= 1 && KPB + 2 < 64, "vmcnt has 6 bits");
    // the two slots are separate arrays so that the compiler can tell that the
    // loads into one do not touch the fragment reads of the other
    __shared__ __attribute__((aligned(1024))) unsigned char qs[QLW * WAVES * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char kst0[WAVES * BLK_B];
    __shared__ __attribute__((aligned(1024))) unsigned char kst1[WAVES * BLK_B];

    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int col = lane & 31;
    const int hf = lane >> 5;
    const int32_t p0 = pos[0];
    const int r0 = blockIdx.x * (WAVES * NB * 32);
    const int wrow = r0 + wave * NB * 32;
    unsigned char *const ks[2] = {kst0 + wave * BLK_B, kst1 + wave * BLK_B};

    // head weights of this lane's accumulator rows (4 consecutive heads per
    // load; heads past H read as 0)
    const auto rw = make_rsrc(w, (uint32_t)(H * 4));
    u32x4 wv[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            wv[mt][g] = buf_load16(rw, (uint32_t)(mt * 32 + acc_row(4 * g, lane)) * 4);
    // the query rows, swizzled (heads past H read as 0)
    const auto rq = make_rsrc(q, (uint32_t)(H * D * 2));
#pragma unroll
    for (int i = 0; i < QLW; ++i) {
        const int li = wave * QLW + i;
        const int sl = li * 64 + lane, r = sl / CPR;
        const int c = (sl % CPR) ^ ((r / (16 / CPR)) % CPR);
        if (li < QL)
            buf_load16_lds(rq, qs + li * 1024, (uint32_t)(r * CPR + c) * 16);
    }
    // K block b of this wave into slot b % 2: load i fills the slot's 16-byte
    // units [64 i, 64 i + 64) lane by lane, each lane fetching the chunk that
    // belongs in its unit (rows past N read as 0)
    const auto rk = make_rsrc(k, (uint32_t)N * D * 2);
    uint32_t koff[KPB];
#pragma unroll
    for (int i = 0; i < KPB; ++i) {
        const int sl = i * 64 + lane, r = sl / CPR;
        const int c = (sl % CPR) ^ ((r / (16 / CPR)) % CPR);
        koff[i] = ((uint32_t)(wrow + r) * CPR + c) * 16;
    }
    auto load_block = [&](int b) {
#pragma unroll
        for (int i = 0; i < KPB; ++i)
            buf_load16_lds<kStreamAux>(rk, ks[b & 1] + i * 1024, koff[i] + (uint32_t)b * BLK_B);
    };
    load_block(0);
    if (NB > 1)
        load_block(1);

    const int n = visible_rows(p0, ratio, N);
    if (n <= min_rows || r0 >= n) {
        wait_vmcnt<0>(); // no load into this group's LDS outlives it
        return;          // same for the whole work-group
    }
    // the weights and the query (issued before every K load) have landed
    // here and in every wave
    wait_vmcnt<(NB > 1 ? 2 : 1) * KPB>();
    lds_barrier();
    DSI_STAMP(decode_stamps, stamp_rec, 1, threadIdx.x == 0);
    u32x4 a[MT][KS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            a[mt][kk] = *reinterpret_cast<const u32x4 *>(
                qs + (mt * 32 * CPR + stage_slot<CPR>(col, 2 * kk + hf)) * 16);
    float wr[MT][16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            wr[mt][i] = __uint_as_float(wv[mt][i >> 2][i & 3]);
    uint32_t boff[KS]; // row col, elements 16 kk + 8 hf ..
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
        boff[kk] = (uint32_t)stage_slot<CPR>(col, 2 * kk + hf) * 16;
    const auto rs = make_rsrc(S, (uint32_t)n * 4);
    // wait until block b has landed: issued after it are block b+1 (if any)
    // and the score stores of blocks b-2 and b-1 (those that exist)
    auto wait_block = [&](int b) {
        const int st = b < 2 ? b : 2;
        if (b + 1 < NB) {
            if (st == 0)
                wait_vmcnt<KPB>();
            else if (st == 1)
                wait_vmcnt<KPB + 1>();
            else
                wait_vmcnt<KPB + 2>();
        } else {
            if (st == 0)
                wait_vmcnt<0>();
            else if (st == 1)
                wait_vmcnt<1>();
            else
                wait_vmcnt<2>();
        }
    };
    float scb[NB]; // this lane's score of row col of each block
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        wait_block(b);
        wave_lds_sync();
        u32x4 bk[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            bk[kk] = *reinterpret_cast<const u32x4 *>(ks[b & 1] + boff[kk]);
        if (b + 2 < NB) {
            // the slot's fragments are in registers: reuse it for block b+2
            wait_lgkmcnt0();
            wave_lds_sync();
            load_block(b + 2);
        }
        f32x16 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            acc[mt] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = mfma32<DT>(a[mt][kk], bk[kk], acc[mt]);
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                s0 = fmaf(wr[mt][i], fmaxf(acc[mt][i], 0.f), s0);
                s1 = fmaf(wr[mt][i + 1], fmaxf(acc[mt][i + 1], 0.f), s1);
            }
        const float sc = add_other_half(s0 + s1);
        scb[b] = sc;
        // rows >= n dropped
        buf_store_f32(rs, hf == 0 ? (uint32_t)(wrow + b * 32 + col) * 4 : kOffNone, sc);
    }
    DSI_STAMP(decode_stamps, stamp_rec, 2 + wave, lane == 0 && wave < 4);
    if (cand == nullptr)
        return;

    // The work-group's rows are one selection partition: list its kp best keys
    // in row order (all its rows when they are <= kp, key 0 in unused slots),
    // their number in pcount and the smallest listed key in pmin (0 when the
    // list holds every row).
    constexpr int ROWS = WAVES * NB * 32;
    static_assert(ROWS == kDecodePart, "a decode work-group covers one selection partition");
    const int rows = min(ROWS, n - r0);
    uint64_t *list = cand + (size_t)blockIdx.x * kp;
    if (kp <= 8) {
        // Small lists (many partitions): each wave first keeps the best kp of
        // its own NB * 32 rows (the partition's best kp are among them), by
        // ranking, in parallel and without a barrier; then one wave ranks the
        // WAVES * kp survivors.  The survivors go through each wave's first
        // slot (its loads have all landed and been read), the ranking scratch
        // is its second.
        static_assert(WAVES * 8 <= 64, "one survivor per lane");
        uint32_t hi[NB], lo[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int row = wrow + b * 32 + col; // lanes 32..63 hold the same scores: no key
            const uint64_t key = hf == 0 && row < n ? make_key(scb[b], (uint32_t)row) : 0ull;
            hi[b] = (uint32_t)(key >> 32);
            lo[b] = (uint32_t)key;
        }
        const int nv = min(max(n - wrow, 0), NB * 32); // rows of this wave
        uint64_t tw = 1ull;
        if (nv > kp) // (then more than kp lanes hold a key)
            tw = wave_kth_small<NB, 32>(hi, lo, kp,
                                        reinterpret_cast<uint64_t *>(kst1 + wave * BLK_B));
        uint64_t *wl = reinterpret_cast<uint64_t *>(kst0 + wave * BLK_B);
        int c = 0;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint64_t key = ((uint64_t)hi[b] << 32) | lo[b];
            const bool keep = key >= tw; // (tw >= 1: no empty slot)
            const uint64_t m = ballot(keep);
            if (keep)
                wl[c + mbcnt(m)] = key;
            c += popc(m);
        }
        if (lane >= c && lane < 8)
            wl[lane] = 0ull;
        __syncthreads();
        if (wave != 0)
            return;
        // survivor j = entry j % 8 of wave j / 8's list, in row order
        const uint64_t x =
            lane < WAVES * 8 ? reinterpret_cast<const uint64_t *>(kst0 + (lane >> 3) * BLK_B)[lane & 7]
                             : 0ull;
        uint64_t t = 1ull;
        if (rows > kp) {
            // more than kp rows: the survivors hold at least kp keys, so
            // exactly one has kp - 1 larger ones
            int r = 0;
#pragma unroll
            for (int w = 0; w < WAVES; ++w)
                r += rank_among(reinterpret_cast<const uint64_t *>(kst0 + w * BLK_B), 8, x);
            t = readlane64(x, (int)__builtin_ctzll(ballot(x != 0ull && r == kp - 1)));
        }
        const bool keep = x != 0ull && x >= t;
        const uint64_t m = ballot(keep);
        if (keep)
            list[mbcnt(m)] = x;
        const int nc = popc(m);
        if (lane >= nc && lane < kp)
            list[lane] = 0ull;
        if (lane == 0) {
            pcount[blockIdx.x] = nc;
            pmin[blockIdx.x] = rows > kp ? t : 0ull;
        }
        DSI_STAMP(decode_stamps, stamp_rec, 6, lane == 0);
        return;
    }

    // Longer lists: the scores go through LDS (each wave's first slot) to one
    // wave, which finds the kp-th best key by the threshold search.  (Taking
    // the best keys by rounds of wave maxima measured slower.)
    constexpr int E = ROWS / 64; // keys per lane
    float *const mine = reinterpret_cast<float *>(kst0 + wave * BLK_B);
    if (hf == 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
            mine[b * 32 + col] = scb[b];
    }
    __syncthreads();
    if (wave != 0)
        return;
    uint32_t hi[E], lo[E];
#pragma unroll
    for (int s = 0; s < E; ++s) {
        const int i = s * 64 + lane; // row r0 + i, held by wave i / (NB * 32)
        const float v = reinterpret_cast<const float *>(kst0 + (i / (NB * 32)) * BLK_B)[i % (NB * 32)];
        const uint64_t key = i < rows ? make_key(v, (uint32_t)(r0 + i)) : 0ull;
        hi[s] = (uint32_t)(key >> 32);
        lo[s] = (uint32_t)key;
    }
    uint64_t t = 1ull; // every valid key is >= 1
    if (rows > kp) {
        WaveReduce red;
        t = select_bound<E>(hi, lo, E, rows, kp, 0, red); // the kp-th best key
    }
    int nc = 0;
#pragma unroll
    for (int s = 0; s < E; ++s) {
        const uint64_t key = ((uint64_t)hi[s] << 32) | lo[s];
        const bool keep = key >= t;
        const uint64_t m = ballot(keep);
        if (keep)
            list[nc + mbcnt(m)] = key;
        nc += popc(m);
    }
    for (int i = nc + lane; i < kp; i += 64)
        list[i] = 0ull;
    if (lane == 0) {
        pcount[blockIdx.x] = nc;
        pmin[blockIdx.x] = rows > kp ? t : 0ull;
    }
    DSI_STAMP(decode_stamps, stamp_rec, 6, lane == 0);
}

__global__ void fill_kernel(float *__restrict__ p, long long n, float v)
{
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x)
        p[i] = v;
}

template <int H, int D, int DT>
hipError_t prefill_one(const Problem &p, int min_rows, float *S, long long ldS, bool split,
                       hipStream_t st, Timing *tm)
{
    constexpr int TPB = (64 / H) * kPrefillWaves;
    const dim3 grid((p.T + TPB - 1) / TPB, (p.N + kChunkRows - 1) / kChunkRows);
    if (split)
        return launch_kernel(prefill_scorer_kernel<H, D, DT, kPrefillWaves, kStageRows, true>,
                             grid, dim3(kPrefillWaves * 64), 0, st, tm, true, true, p.q, p.k, p.w,
                             p.pos, p.T, p.N, p.ratio, min_rows, kChunkRows, S, ldS);
    return launch_kernel(prefill_scorer_kernel<H, D, DT, kPrefillWaves, kStageRows, false>, grid,
                         dim3(kPrefillWaves * 64), 0, st, tm, true, true, p.q, p.k, p.w, p.pos,
                         p.T, p.N, p.ratio, min_rows, kChunkRows, S, ldS);
}

constexpr int kDecWaves = 4;  // waves per decode work-group
constexpr int kDecBlocks = 4; // 32-row K blocks per decode wave

template <int H, int D, int DT>
hipError_t decode_one(const Problem &p, int min_rows, float *S, const DecodeLists &dl,
                      hipStream_t st, Timing *tm, int B, long long ldS)
{
    constexpr int ROWS = kDecWaves * kDecBlocks * 32; // per work-group
    return launch_kernel(decode_scorer_kernel<H, D, DT, kDecWaves, kDecBlocks>,
                         dim3((p.N + ROWS - 1) / ROWS, B), dim3(kDecWaves * 64), 0, st, tm, true,
                         true, p.q, p.k, p.w, p.pos, p.N, p.ratio, min_rows, S, dl.kp, dl.cand,
                         dl.pcount, dl.pmin, ldS);
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
    static hipError_t run(const Problem &p, int m, float *S, long long ld, bool split,
                          hipStream_t st, Timing *tm)
    {
        return prefill_one<H, D, DT>(p, m, S, ld, split, st, tm);
    }
};
template <int H, int D, int DT> struct DecodeF {
    static hipError_t run(const Problem &p, int m, float *S, const DecodeLists *dl, hipStream_t st,
                          Timing *tm, int B, long long ldS)
    {
        return decode_one<H, D, DT>(p, m, S, *dl, st, tm, B, ldS);
    }
};

} // namespace

hipError_t launch_prefill_scorer(const Problem &p, int min_rows, float *S, long long ldS,
                                 bool split, hipStream_t st, Timing *tm)
{
    if (p.T <= 0 || p.N <= 0)
        return hipSuccess;
    return dispatch<PrefillF>(p.H, p.D, p.dtype, p, min_rows, S, ldS, split, st, tm);
}

hipError_t launch_decode_scorer(const Problem &p, int min_rows, float *S, const DecodeLists &dl,
                                hipStream_t st, Timing *tm, int B, long long ldS)
{
    if (p.T <= 0 || p.N <= 0 || B <= 0)
        return hipSuccess;
    return dispatch<DecodeF>(p.H, p.D, p.dtype, p, min_rows, S, &dl, st, tm, B, ldS);
}

#ifdef DSI_STAMPS
hipError_t stamps_read_decode(void *host, size_t bytes)
{
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(decode_stamps), bytes, 0, hipMemcpyDeviceToHost);
}
#endif

hipError_t launch_fill(float *p, long long n, float v, hipStream_t st)
{
    if (n <= 0)
        return hipSuccess;
    long long blocks = (n + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    (void)hipGetLastError(); // (see launch_kernel)
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
    return after_launch(hipGetLastError(), st);
}

} // namespace dsi
