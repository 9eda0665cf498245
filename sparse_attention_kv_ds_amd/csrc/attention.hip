// attention.hip -- sparse attention over the selected rows, for gfx950.
//
// For token t at position p and attention head h, one softmax over the rows
// R(t) = the local raw rows max(0, p - window + 1) .. min(p, L-1) plus the
// pooled rows listed in idx[t] (entries outside [0, N) are padding):
//   o[t,h,:] = sum_r softmax_r(scale * q[t,h,:] . key_r) value_r
// with keys and values shared by all heads ("How I turned one oversized
// DeepSeek optimization into three merged oMLX PRs", section "1. Route
// ratio-128 prefill through native attention": local and pooled key/value
// state attended together, the pooled rows given by indices; the indices are
// the lightning indexer's selection, "How I made DeepSeek 12x faster on a Mac
// Studio", section "1: the kernels").
//
// The all-visible form (ratio > 0, no index list) attends to every pooled row
// the token can see, rows 0 .. n-1 with n = floor((p + 1) / ratio) clamped
// to [0, N]: the sequential pooled indices of ratio-128 layers (same section
// of the oMLX page).
//
// One work-group per token, one wave per 32 heads.  The token's rows are taken
// in blocks of 32: the local rows first (their last block padded), then the
// index list in order, so that every block reads one tensor pair.  Each
// block's K and V rows go straight from memory into LDS (buffer loads with the
// LDS bit): V of the next block during the whole of the current one, K of the
// next block once every wave holds the current block's K fragments.  One K
// stage and two V stages (24 KiB at D = 128) plus the index list leave room
// for six work-groups, three waves per SIMD, per CU.
//   * S^T = K_blk . Q^T on the 32x32x16 MFMA: each lane then holds 16 keys of
//     one head, so the softmax statistics of a head live in one lane pair.
//   * Online softmax in base 2 with a lazy rescale: the running exponent base
//     of a head moves only when a block's maximum exceeds it by more than 8,
//     so p <= 2^8 and the accumulators are rescaled rarely.
//   * O^T += V_blk^T . P^T on the MFMA: P comes straight from the S^T
//     accumulators (converted to the value type), V^T fragments from the
//     row-major V block by LDS transpose reads (ds_read_b64_tr_b16).
// Output fp32, o = O / (sum of p), 0 for a token with no row, written a
// 32-wide value tile at a time through the free stage arrays as whole
// 128-byte pieces.
#include "common.hpp"
#include "launch.hpp"

namespace dsi {

namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));

// phase timestamps (stamps build only), record = token: 0 start, 1 first block
// and the query fragments landed, 2 last block done, 3 output stores issued
DSI_STAMP_ARRAY(attn_stamps);

// 4 x 16-bit of the transposed LDS read: within each group of 16 lanes, lane
// i receives element i % 4 of the 8-byte chunk addressed by lane 4 e + i / 4,
// for e = 0..3.
__device__ __forceinline__ uint64_t lds_read_tr16(const void *p)
{
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)const_cast<void *>(p));
    return __builtin_bit_cast(uint64_t, r);
}

// Swizzle of V row r in LDS: its 16-byte chunks are XORed with 4 vswz(r), so
// that rows r, r+1, r+2, r+3 (D = 128: 256-byte rows) or r .. r+7 (D = 64)
// put the same 32 columns on four different 64-byte quarters of the banks.
template <int D>
__device__ __forceinline__ int vswz(int r)
{
    return D == 128 ? (r & 3) : ((r >> 1) & 1);
}

// c ? a : b between two values.  Inside a lambda that captures by reference,
// a conditional expression over captured names becomes a choice between
// their addresses, which keeps the captured variables in scratch memory; as
// function arguments they are read first and only the values are chosen.
template <class T>
__device__ __forceinline__ T pick(bool c, T a, T b)
{
    return c ? a : b;
}

// 2^x by the hardware instruction alone (no rescaling of results below
// 2^-126: every p here is at most 2^8 and the largest is at least 1, so such
// terms are far below the rounding of the sum)
__device__ __forceinline__ float exp2_fast(float x)
{
    return __builtin_amdgcn_exp2f(x);
}

// two floats -> two 16-bit values of type DT (round to nearest even)
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    if constexpr (DT == kF16) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const h2 v = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        const b2 v = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, v);
    }
}

// IDS: capacity of the index list in LDS (entries; at least 32 ceil(topk / 32))
template <int WAVES, int D, int DT, int IDS>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(3, 3))) void sparse_attention_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kp,
    const uint16_t *__restrict__ vp, const uint16_t *__restrict__ kl,
    const uint16_t *__restrict__ vl, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ pos, int N, int L, int topk, int ratio, int window,
    float scale_log2, float *__restrict__ out)
{
    constexpr int HA = WAVES * 32;
    constexpr int KS = D / 16;            // MFMA steps along D for S
    constexpr int DTL = D / 32;           // 32-wide value tiles
    constexpr int CPR = D / 8;            // 16-byte chunks per row
    constexpr int RPL = 64 / CPR;         // rows per 1 KiB load
    constexpr int BLK_B = 32 * D * 2;     // bytes of 32 rows
    constexpr int LPB = BLK_B / 1024;     // 1 KiB loads per block and tensor
    // the row stored for an empty slot: its rows start at byte 2^31, past
    // every tensor (each holds fewer than 2^30 / D rows, under 2^31 bytes),
    // and its 16-byte loads end well below 2^32
    constexpr uint32_t kNoRow = 0x80000000u / (2 * D);

    __shared__ int32_t ids[IDS];
    // one array per stage and tensor, so that the compiler can tell that the
    // loads into one stage do not touch the fragment reads of the other
    __shared__ __attribute__((aligned(1024))) unsigned char ks0[BLK_B];
    __shared__ __attribute__((aligned(1024))) unsigned char vs0[BLK_B];
    __shared__ __attribute__((aligned(1024))) unsigned char vs1[BLK_B];

    // work-groups go to the 8 XCDs in turn: give each XCD one contiguous run
    // of tokens, so that the overlapping local windows of neighbouring tokens
    // meet in the same L2
    int t;
    {
        const int T = gridDim.x, w = blockIdx.x, x = w & 7, q8 = T >> 3, r8 = T & 7;
        t = x * q8 + min(x, r8) + (w >> 3);
    }
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int col = lane & 31;
    const int hf = lane >> 5;
    DSI_STAMP(attn_stamps, t, 0, threadIdx.x == 0);
    const int p = pos[t];
    int lo = 0, n_loc = 0;
    if (p >= 0 && window > 0) {
        lo = max(0, p - window + 1);
        n_loc = max(0, min(p, L - 1) - lo + 1);
    }
    const int nb_loc = (n_loc + 31) >> 5;
    const int nb_pool = (topk + 31) >> 5;
    const int nb = nb_loc + nb_pool;

    u32x4 qf[KS]; // this wave's 32 heads as MFMA B fragments (loaded below)
    const uint32_t bytes_p = (uint32_t)N * D * 2, bytes_l = (uint32_t)L * D * 2;

    // Loads of a block: 1 KiB load i (0 <= i < LPB) of a tensor covers rows
    // RPL i .. RPL i + RPL-1, lane by lane (row RPL i + lane / CPR, 16-byte
    // chunk lane % CPR; K chunks swizzled, V rows plain, as the transpose reads
    // want whole 8-byte runs of a row).  Wave w issues loads i0 .. i0 + NI - 1
    // of both tensors: the rows, not the tensors, are split over the waves
    // (measured: with one wave per tensor the same gather takes about twice
    // as long).
    constexpr int NI = LPB / WAVES;
    static_assert(NI >= 1 && NI * WAVES == LPB, "block loads split evenly over the waves");
    const int i0 = wave * NI;
    const int pc = lane % CPR;

    // this lane's row of each of its loads of block b, kNoRow for an empty
    // slot (the pooled rows come from the index list in one round of LDS
    // reads).  kNoRow * CPR * 16 lies past every tensor's range, so an empty
    // slot's load is dropped by the range check with no compare of its own.
    auto block_rows = [&](int b, uint32_t (&row)[NI]) {
        if (b < nb_loc) {
#pragma unroll
            for (int n = 0; n < NI; ++n) {
                const int k = 32 * b + (i0 + n) * RPL + lane / CPR;
                row[n] = k < n_loc ? (uint32_t)(lo + k) : kNoRow;
            }
        } else {
            const uint32_t *e =
                reinterpret_cast<const uint32_t *>(ids) + 32 * (b - nb_loc) + i0 * RPL + lane / CPR;
#pragma unroll
            for (int n = 0; n < NI; ++n)
                row[n] = e[n * RPL];
        }
    };
    // this wave's loads of block b of K (isk) or V, rows `row`, into stage st
    auto issue = [&](int b, const uint32_t (&row)[NI], unsigned char *st, bool isk) {
        const bool local = b < nb_loc;
        const uint16_t *base = pick(isk, pick(local, kl, kp), pick(local, vl, vp));
        const auto r = make_rsrc(base, local ? bytes_l : bytes_p);
#pragma unroll
        for (int n = 0; n < NI; ++n) {
            const int rr = (i0 + n) * RPL + lane / CPR; // row slot in the block
            const int c = isk ? pc ^ ((rr / (16 / CPR)) % CPR) : pc ^ (4 * vswz<D>(rr));
            buf_load16_lds(r, st + (i0 + n) * 1024, row[n] * (CPR * 16) + (uint32_t)c * 16);
        }
    };
    auto load_block = [&](int b, unsigned char *kst, unsigned char *vst) {
        uint32_t row[NI];
        block_rows(b, row);
        issue(b, row, kst, true);
        issue(b, row, vst, false);
    };

    // per lane: head col of this wave's tile; the two half-waves hold
    // different keys of the same head and keep the same exponent base
    float m_base = -__builtin_huge_valf(); // exponent base (log2 domain)
    float l_part = 0.f;                    // this lane's part of the sum of p
    f32x16 o[DTL];
#pragma unroll
    for (int d = 0; d < DTL; ++d)
        o[d] = f32x16{};

    // K fragment offsets within a stage: key col, elements 16 kk + 8 hf ..
    uint32_t koff[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
        koff[kk] = (uint32_t)stage_slot<CPR>(col, 2 * kk + hf) * 16;
    // V^T fragment offsets (transpose reads): group g = lane / 16 covers value
    // columns 16 (g % 2) .. + 15 of a 32-wide tile and keys 4 (g / 2) + 0..3 of
    // each 8-key run; lane L of the group addresses key 4 (g / 2) + L / 4,
    // columns 4 (L % 4) .. + 3.  V rows are swizzled in 64-byte groups (chunk
    // c of row r sits at c ^ 4 vswz(r)), so that the eight rows one read
    // touches fall on all the LDS banks rather than on the same quarter; every
    // row this lane addresses has the same vswz.
    const int g = lane >> 4, Lg = lane & 15;
    const int vsw_lane = vswz<D>(4 * (g >> 1) + (Lg >> 2));
    uint32_t voffd[DTL];
#pragma unroll
    for (int d = 0; d < DTL; ++d)
        voffd[d] = ((uint32_t)(4 * (g >> 1) + (Lg >> 2)) * D + 32 * (d ^ vsw_lane) + 16 * (g & 1) +
                    4 * (Lg & 3)) * 2;

    // block b from K stage kst and V stage vst; k_done() runs once this
    // wave's K fragments are in registers
    auto compute_block = [&](int b, const unsigned char *kst, const unsigned char *vst,
                             auto &&pre, auto &&k_done) {
        // this lane's key slot of the block is valid (read here, used after
        // the score MFMAs); a block with no valid key goes through with every
        // score -inf (its p are all 0): an early exit here would give the
        // accumulators a second home across the loop and cost registers
        bool valid;
        if (b < nb_loc)
            valid = 32 * b + col < n_loc;
        else
            valid = (uint32_t)ids[32 * (b - nb_loc) + col] != kNoRow;
        // S^T: lane holds head col, keys 8 (i / 4) + 4 hf + i % 4
        f32x16 s = f32x16{};
        {
            // K fragments read PF steps ahead of their MFMAs; the scheduling
            // fences keep that order (left to itself the compiler reads one
            // step ahead, and each MFMA waits for its LDS read).  pre() (the
            // next block's V loads) goes out once the first reads are issued.
            constexpr int PF = 2;
            u32x4 kf[PF + 1];
#pragma unroll
            for (int kk = 0; kk < PF && kk < KS; ++kk)
                kf[kk] = *reinterpret_cast<const u32x4 *>(kst + koff[kk]);
            __builtin_amdgcn_sched_barrier(0);
            pre();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                if (kk + PF < KS)
                    kf[(kk + PF) % (PF + 1)] = *reinterpret_cast<const u32x4 *>(kst + koff[kk + PF]);
                __builtin_amdgcn_sched_barrier(0);
                s = mfma32<DT>(kf[kk % (PF + 1)], qf[kk], s);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        k_done();
        const uint64_t vm = ballot(lane < 32 && valid);
        // empty key slots (partial blocks only) score -inf
        if ((uint32_t)vm != 0xFFFFFFFFu) {
            const uint32_t mh = (uint32_t)(vm >> (4 * hf));
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = 8 * (i >> 2) + (i & 3);
                s[i] = (mh >> key) & 1u ? s[i] : -__builtin_huge_valf();
            }
        }
        // the block's maximum of the head in the log2 domain (the scale is
        // positive, so it is the scaled maximum of the raw scores)
        float mx = -__builtin_huge_valf();
#pragma unroll
        for (int i = 0; i < 16; ++i)
            mx = fmaxf(mx, s[i]);
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                             __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
        }
        // lazy rescale: move the base only when the block's maximum is more
        // than 2^8 above it
        if (ballot(mx > m_base + 8.f)) {
            const bool move = mx > m_base + 8.f;
            const float nbase = move ? mx : m_base;
            // 0 when the old base is -inf; 1 for a head whose base stays
            const float alpha = move ? exp2_fast(m_base - nbase) : 1.f;
            m_base = nbase;
            l_part *= alpha;
#pragma unroll
            for (int d = 0; d < DTL; ++d)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    o[d][i] *= alpha;
        }
        const float nb2 = m_base == -__builtin_huge_valf() ? 0.f : -m_base;
        // V^T fragments one MFMA ahead, the first one's reads before the
        // exponentials, so that no value MFMA waits for its LDS reads
        // (measured: 3-4 % faster than reading each just before its MFMA)
        auto vread = [&](int st, int d) -> u32x4 {
            const unsigned char *vb = vst + voffd[d] + (uint32_t)(16 * st * D) * 2;
            const uint64_t lo4 = lds_read_tr16(vb);
            const uint64_t hi4 = lds_read_tr16(vb + 8 * D * 2);
            return u32x4{(uint32_t)lo4, (uint32_t)(lo4 >> 32), (uint32_t)hi4, (uint32_t)(hi4 >> 32)};
        };
        u32x4 vf[2];
        vf[0] = vread(0, 0);
        __builtin_amdgcn_sched_barrier(0);
        uint32_t pk[8];
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const float p0 = exp2_fast(fmaf(s[i], scale_log2, nb2));
            const float p1 = exp2_fast(fmaf(s[i + 1], scale_log2, nb2));
            l_part += p0 + p1;
            pk[i >> 1] = pack2<DT>(p0, p1);
        }
        __builtin_amdgcn_sched_barrier(0);
        // O^T += V^T . P^T over the block's two 16-key steps
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const u32x4 pf = {pk[4 * st], pk[4 * st + 1], pk[4 * st + 2], pk[4 * st + 3]};
#pragma unroll
            for (int d = 0; d < DTL; ++d) {
                const int i = st * DTL + d;
                if (i + 1 < 2 * DTL)
                    vf[(i + 1) & 1] = vread((i + 1) / DTL, (i + 1) % DTL);
                __builtin_amdgcn_sched_barrier(0);
                o[d] = mfma32<DT>(vf[i & 1], pf, o[d]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // Block 0 is issued first when it holds local rows (it needs no index
    // list), then the query fragments and the index list, so that the three
    // are in flight together.
    if (nb_loc > 0)
        load_block(0, ks0, vs0);
    // this wave's 32 heads as MFMA B fragments: head col, elements 16 kk + 8 hf ..
    const auto rq = make_rsrc(q + ((long long)t * HA + wave * 32) * D, 32u * D * 2);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
        qf[kk] = buf_load16(rq, ((uint32_t)col * D + kk * 16 + hf * 8) * 2);
    // entries outside [0, N) and the padding become kNoRow (empty slots); with
    // ratio > 0 the list is every pooled row the token can see, 0 .. n-1
    const int n_all = ratio > 0 ? visible_rows(p, ratio, N) : 0;
    for (int e = threadIdx.x; e < 32 * nb_pool; e += WAVES * 64) {
        int j;
        if (ratio > 0)
            j = e < n_all ? e : -1;
        else
            j = e < topk ? idx[(long long)t * topk + e] : -1;
        ids[e] = (uint32_t)j < (uint32_t)N ? j : (int32_t)kNoRow;
    }


    lds_barrier(); // the index list, written by every wave
    if (nb > 0) {
        if (nb_loc == 0)
            load_block(0, ks0, vs0);
        wait_vmcnt<0>(); // block 0 and the query fragments
        __syncthreads();
        DSI_STAMP(attn_stamps, t, 1, threadIdx.x == 0);
        // block b: V of block b + 1 loads into the other V stage from the
        // start; K of block b + 1 into the one K stage once every wave holds
        // the K fragments of block b (the barrier in the hook)
        auto step = [&](int b, const unsigned char *vc, unsigned char *vn) {
            const bool more = b + 1 < nb;
            uint32_t row[NI];
            if (more)
                block_rows(b + 1, row);
            compute_block(b, ks0, vc, [&] {
                if (more)
                    issue(b + 1, row, vn, false);
            }, [&] {
                lds_barrier();
                if (more)
                    issue(b + 1, row, ks0, true);
            });
            wait_vmcnt<0>();
            lds_barrier();
        };
        // two blocks per iteration, so that both V stages are named arrays
        // and the compiler can tell the loads into one from the reads of the
        // other
        for (int b = 0;;) {
            step(b, vs0, vs1);
            if (++b >= nb)
                break;
            step(b, vs1, vs0);
            if (++b >= nb)
                break;
        }
    }

    DSI_STAMP(attn_stamps, t, 2, threadIdx.x == 0);
    // o = O / l for head col (the two halves' parts of l added)
    float l = add_other_half(l_part);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if constexpr (WAVES <= 3) {
        // One 32-wide value tile at a time goes through this wave's own LDS
        // region (a stage array, free after the last block: 32 heads x 32
        // floats, the eight 16-byte chunks of head h's row at chunk ^ (h % 8))
        // and out as whole 128-byte pieces, eight heads per store.  (A lane
        // holds four 16-byte pieces of one head per tile, 512 bytes apart from
        // its neighbours': stored directly, every store writes 32 partial
        // lines.)  Every stage array holds 4 KiB at D = 64 and 128.
        static_assert(BLK_B >= 32 * 32 * 4, "a stage array holds one 32 x 32 float tile");
        float *const stg = reinterpret_cast<float *>(wave == 0 ? ks0 : (wave == 1 ? vs0 : vs1));
        const auto ro = make_rsrc(out + ((long long)t * HA + wave * 32) * D, 32u * D * 4);
#pragma unroll
        for (int d = 0; d < DTL; ++d) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float4 v;
                v.x = o[d][4 * r] * inv;
                v.y = o[d][4 * r + 1] * inv;
                v.z = o[d][4 * r + 2] * inv;
                v.w = o[d][4 * r + 3] * inv;
                // value columns 8 r + 4 hf .. + 3 of the tile: chunk 2 r + hf
                *reinterpret_cast<float4 *>(stg + col * 32 + 4 * ((2 * r + hf) ^ (col & 7))) = v;
            }
            wave_lds_sync();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int h = 8 * j + (lane >> 3), c = lane & 7;
                const float4 v = *reinterpret_cast<const float4 *>(stg + h * 32 + 4 * (c ^ (h & 7)));
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro,
                                                       (uint32_t)(h * D + 32 * d + 4 * c) * 4, 0, 0);
            }
            wave_lds_sync();
        }
    } else {
        // four waves (128 heads): no stage array of its own for the fourth,
        // so every lane stores its pieces directly
        float *ot = out + ((long long)t * HA + wave * 32 + col) * D;
#pragma unroll
        for (int d = 0; d < DTL; ++d)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float4 v;
                v.x = o[d][4 * r] * inv;
                v.y = o[d][4 * r + 1] * inv;
                v.z = o[d][4 * r + 2] * inv;
                v.w = o[d][4 * r + 3] * inv;
                *reinterpret_cast<float4 *>(ot + 32 * d + 8 * r + 4 * hf) = v;
            }
    }
    DSI_STAMP(attn_stamps, t, 3, threadIdx.x == 0);
}

template <int WAVES, int D, int DT, int IDS>
hipError_t attn_launch(const AttnProblem &a, float scale_log2, hipStream_t st, Timing *tm)
{
    return launch_kernel(sparse_attention_kernel<WAVES, D, DT, IDS>, dim3(a.T), dim3(WAVES * 64),
                         0, st, tm, true, true, a.q, a.kp, a.vp, a.kl, a.vl, a.idx, a.pos, a.N,
                         a.L, a.topk, a.ratio, a.window, scale_log2, a.out);
}

template <int WAVES, int D>
hipError_t attn_one(const AttnProblem &a, hipStream_t st, Timing *tm)
{
    const float scale_log2 = a.scale * 1.4426950408889634f;
    // the index list, padded to whole blocks of 32: a short list keeps the
    // LDS of a work-group at 26 KiB (D = 128), six per CU
    const bool small = a.topk <= 512;
    if (a.dtype == kF16)
        return small ? attn_launch<WAVES, D, kF16, 512>(a, scale_log2, st, tm)
                     : attn_launch<WAVES, D, kF16, kAttnMaxTopk>(a, scale_log2, st, tm);
    return small ? attn_launch<WAVES, D, kBF16, 512>(a, scale_log2, st, tm)
                 : attn_launch<WAVES, D, kBF16, kAttnMaxTopk>(a, scale_log2, st, tm);
}

} // namespace

#ifdef DSI_STAMPS
hipError_t stamps_read_attention(void *host, size_t bytes)
{
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(attn_stamps), bytes, 0, hipMemcpyDeviceToHost);
}
#endif

hipError_t launch_sparse_attention(const AttnProblem &a, hipStream_t st, Timing *tm)
{
    if (a.T <= 0)
        return hipSuccess;
#define DSI_ATTN(w, d)                                                                    \
    if (a.HA == 32 * w && a.D == d)                                                       \
        return attn_one<w, d>(a, st, tm);
    DSI_ATTN(1, 64) DSI_ATTN(1, 128) DSI_ATTN(2, 64) DSI_ATTN(2, 128) DSI_ATTN(4, 64)
    DSI_ATTN(4, 128)
#undef DSI_ATTN
    return hipErrorInvalidValue;
}

} // namespace dsi
