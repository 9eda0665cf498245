// common.hpp -- device helpers shared by the indexer kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"

namespace dsi {

constexpr int kWave = 64;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One 32x32x16 MFMA step, C += A * B, where lane l supplies A row (l % 32)
// and B column (l % 32), each as 8 consecutive elements of the contraction
// dimension (16 bytes of raw fp16/bf16 bits).  Both operands use the same
// lane -> contraction-index assignment, so the sum over the 16 contraction
// indices is what it should be whatever order the matrix core uses inside.
template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c)
{
    if constexpr (DT == kF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                      __builtin_bit_cast(half8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Accumulator layout of a 32x32 MFMA: lane l, register i holds
// C[row][col] with col = l % 32 and row = 8*(i/4) + 4*(l/32) + i%4.
__device__ __forceinline__ int acc_row(int i, int lane)
{
    return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// Number of compressed rows visible from absolute position pos: row j covers
// raw tokens ratio*j .. ratio*j+ratio-1 and is visible once all of them are.
__device__ __forceinline__ int visible_rows(int32_t pos, int ratio, int n_rows)
{
    if (pos < 0)
        return 0;
    const uint32_t n = ((uint32_t)pos + 1u) / (uint32_t)ratio; // pos + 1 <= 2^31: no overflow
    return n < (uint32_t)n_rows ? (int)n : n_rows;
}

// Unique, totally ordered selection key of (score, row): a larger key is a
// better row.  High word: the score's bits mapped so that unsigned order is
// float order (-0 folded onto +0 so equal scores compare equal); low word:
// ~row, so among equal scores the lower row has the larger key.  Every key of
// a finite (or -inf) score is > 0, so 0 can stand for "no key".
__device__ __forceinline__ uint32_t ordered_score(float s)
{
    uint32_t b = __float_as_uint(s);
    if (b == 0x80000000u)
        b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(float s, uint32_t row)
{
    return ((uint64_t)ordered_score(s) << 32) | (uint64_t)(0xFFFFFFFFu - row);
}

__device__ __forceinline__ int key_row(uint64_t key)
{
    return (int)(0xFFFFFFFFu - (uint32_t)key);
}

__device__ __forceinline__ uint64_t ballot(bool p)
{
    return __ballot(p);
}

__device__ __forceinline__ int popc(uint64_t m)
{
    return __popcll(m);
}

// lanes below this one in a mask
__device__ __forceinline__ int mbcnt(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Order this wave's LDS accesses before/after the point (lanes of one wave
// read what other lanes of the same wave wrote).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Work-group barrier that orders LDS only: waits for this wave's LDS accesses,
// then s_barrier.  Unlike __syncthreads it does not also wait for outstanding
// global stores, which no other wave of the group reads.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ int wave_max(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = max(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ uint32_t readfirstlane(uint32_t v)
{
    return __builtin_amdgcn_readfirstlane(v);
}

// This wave's index in the work-group, as a value the compiler knows to be
// the same in every lane (scalar registers, scalar control flow).
__device__ __forceinline__ int wave_id()
{
    return (int)readfirstlane(threadIdx.x >> 6);
}

// Buffer resource over [base, base + bytes): loads past the end return 0 and
// stores past the end are dropped by the hardware, so bounds become offsets
// rather than branches.  (gfx9 descriptor word 3.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// an offset past the end of every resource built here (all are < 2 GiB), with
// headroom so that offset + access size cannot wrap
constexpr uint32_t kOffNone = 0x80000000u;

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ void buf_store_f32(__amdgpu_buffer_rsrc_t r, uint32_t off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

// Split scores of the prefill path (the scorer writes them, the streaming
// top-k reads them): token t's row of 4 ldS bytes holds, per group of
// kSplitRows rows, the high 16 bits of the rows' ordered scores
// (ordered_score), then their low 16 bits.  A group of 32 is one scorer
// block stored as one whole 128-byte line.  (Groups of 64, whose high halves
// fill lines of their own, halve what the selection fetches from HBM, but
// the scorer then writes every line in two halves from two blocks, which
// costs it more than the selection gains.)
constexpr int kSplitRows = 32;
constexpr uint32_t kSplitLow = 2 * kSplitRows; // bytes from a row's high half to its low half

// byte offset of row j's high half within a token's split scores
__device__ __forceinline__ uint32_t split_hi_off(uint32_t j)
{
    return j / kSplitRows * (4 * kSplitRows) + j % kSplitRows * 2;
}

// the low 16 bits of v
__device__ __forceinline__ void buf_store_u16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, off, 0, 0);
}

// 64 bits (0 past the end of the resource)
__device__ __forceinline__ uint64_t buf_load_u64(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    return ((uint64_t)v[1] << 32) | v[0];
}

// 16 bits, zero-extended (0 past the end of the resource)
__device__ __forceinline__ uint32_t buf_load_u16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// 16 bytes per lane from r at byte offset off straight into LDS: lane l's
// bytes land at lds + 16 l (lds must be the same in every lane).  The load is
// counted by vmcnt and its data is in LDS once that count says it completed.
// AUX: cache policy bits of the load (e.g. 2 = non-temporal).
template <int AUX = 0>
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                             off, 0, 0, AUX);
}

// s_waitcnt with only vmcnt <= n (n < 64): waits until at most n vector
// memory instructions of this wave are outstanding (they complete in order)
template <int n>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(n >= 0 && n < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// s_waitcnt with only lgkmcnt(0): this wave's LDS accesses have completed
__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));
}

// LDS slot (16-byte units) of chunk c of row r in a staging area of rows of
// CPR 16-byte chunks (CPR = 4, 8 or 16), no padding: the chunk index is XORed
// with a function of the row so that the 16 rows read by 16 consecutive lanes
// of one MFMA fragment load fall in 16 different bank groups.  The map is its
// own inverse within a row, so the chunk held by slot position p of row r is
// p ^ (the same function of r).
template <int CPR>
__device__ __forceinline__ int stage_slot(int r, int c)
{
    return r * CPR + (c ^ ((r / (16 / CPR)) % CPR));
}

// v + (the same register of lane l ^ 32): one cross-half swap, no LDS traffic
__device__ __forceinline__ float add_other_half(float v)
{
    const uint32_t u = __float_as_uint(v);
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Phase timestamps, compiled in only with DSI_STAMPS (the separate stamps
// build behind the phase breakdowns): DSI_STAMP_ARRAY(a) defines the device
// array `a` of kStampRecords records of 8 entries in the source file that uses
// it, and DSI_STAMP(a, i, ph, cond) writes the 100 MHz real-time counter to
// entry ph of record i from the lanes where cond holds (records past the end
// are dropped).  Without DSI_STAMPS both expand to nothing.
#ifdef DSI_STAMPS
#define DSI_STAMP_ARRAY(a) __device__ unsigned long long a[kStampRecords * 8]
#define DSI_STAMP(a, i, ph, cond)                                                 \
    do {                                                                          \
        const long long i_ = (i);                                                 \
        if ((cond) && i_ < kStampRecords)                                         \
            a[i_ * 8 + (ph)] = __builtin_amdgcn_s_memrealtime();                  \
    } while (0)
// DSI_STAMP_VALUE(a, i, ph, cond, v): the same, recording the value v (a
// count, not a time)
#define DSI_STAMP_VALUE(a, i, ph, cond, v)                                        \
    do {                                                                          \
        const long long i_ = (i);                                                 \
        if ((cond) && i_ < kStampRecords)                                         \
            a[i_ * 8 + (ph)] = (unsigned long long)(v);                           \
    } while (0)
#else
#define DSI_STAMP_ARRAY(a) static_assert(true, "")
#define DSI_STAMP_VALUE(a, i, ph, cond, v) \
    do {                                   \
    } while (0)
#define DSI_STAMP(a, i, ph, cond) \
    do {                          \
    } while (0)
#endif

} // namespace dsi
