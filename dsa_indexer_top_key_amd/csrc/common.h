// Shared device helpers of the gfx950 DSA kernels: bf16 conversion, MFMA vector types and
// wave-level reductions.  Internal to the library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kIndexHeads = 32;   // indexer query heads
constexpr int kIndexDim = 128;    // width of index queries and keys
constexpr int kTopK = 2048;       // selection budget
constexpr int kMlaHeads = 96;     // main-attention heads
constexpr int kLatent = 512;      // KV latent rank (values)
constexpr int kCompanion = 64;    // companion key width
constexpr int kQK = kLatent + kCompanion;  // 576-wide absorbed logits

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(4))) int32_t i32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 bits (NaN -> canonical quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Request of query t: q_req[t] when it lies in [0, B), else -1.  A query outside the batch
// has no admissible position (its scores are not written, its ID row is all -1, its read is
// zero), so no request-indexed array is ever read out of bounds.
__device__ __forceinline__ int query_request(const int32_t* q_req, int64_t t, int32_t B) {
    const int b = q_req[t];
    return (b >= 0 && b < B) ? b : -1;
}

// Admissible count n_t = min(pos + 1, S_b) (causal, the diagonal included), clamped to
// [0, max_s]; 0 for a query outside the batch (b < 0).
__device__ __forceinline__ int64_t admissible_count(const int64_t* kv_off, int b, int32_t pos,
                                                    int64_t max_s) {
    if (b < 0) return 0;
    const int64_t s_b = kv_off[b + 1] - kv_off[b];
    int64_t n = static_cast<int64_t>(pos) + 1;
    n = n < s_b ? n : s_b;
    n = n < max_s ? n : max_s;
    return n > 0 ? n : 0;
}

// Workgroup barrier that orders LDS only: LDS writes issued before it are visible to LDS
// reads after it, while global-memory loads (and global->LDS copies) stay in flight; where
// a kernel hands such data across the barrier it waits on vmcnt explicitly.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

typedef __attribute__((address_space(3))) void lds_void;

// Byte offset of an LDS location, as the LDS instructions and M0 take it.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)p));
}

// One direct global->LDS copy (gfx950 global_load_lds_dwordx4): lane l moves 16 bytes from its
// own address src to LDS bytes [lds_base + 16 l, +16); nothing passes through registers.  It is
// issued through inline assembly so the compiler does not track it -- the compiler would
// otherwise assume the copy may alias every later LDS read and drain the LDS queue before each
// of them, defeating operand prefetch.  Every wait for these copies is an explicit vmcnt wait
// (vector-memory loads complete in issue order, so waiting until at most N operations are
// outstanding, where N counts the loads issued after a copy, covers that copy; stores issued
// in between only make such a wait stricter).  M0 holds the wave-uniform LDS base; one wait
// state separates writing M0 from the copy.  With NT the copy carries the non-temporal hint:
// data read once should not displace cached lines (a pure copy stream measured 7.2 TB/s with
// the hint and 6.2 TB/s without it).
template <bool NT = false>
__device__ __forceinline__ void copy_to_lds(const void* src, uint32_t lds_base) {
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                     :
                     : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "memory");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     :
                     : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "memory");
}

// Wait until at most N of this wave's vector-memory operations are outstanding
// (s_waitcnt vmcnt(N) with expcnt/lgkmcnt left at their maxima; N <= 63).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit counter");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Cross-lane moves through DPP (data-parallel primitives on the VALU, no LDS round trip).
// Controls: quad_perm [1,0,3,2] and [2,3,0,1] swap lanes at distance 1 and 2, row_half_mirror
// reverses each group of 8 lanes, row_mirror each row of 16, row_shr:n shifts a row right by
// n, row_bcast:15 / row_bcast:31 broadcast lane 15 / 31 of a row into the following rows
// (the rows written are chosen by row_mask).  Lanes that are not written keep `old`.
constexpr int dpp_row_shr(int n) { return 0x110 + n; }
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        static_cast<int>(old), static_cast<int>(v), Ctrl, RowMask, 0xF, false));
}

// Reduction over the 64 lanes of a wave; the result is wave-uniform.  Four DPP steps reduce
// each row of 16 lanes, then the four row results are combined through scalar registers.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
    v = op(v, dpp_u32<kDppQuadXor1>(v, v));
    v = op(v, dpp_u32<kDppQuadXor2>(v, v));
    v = op(v, dpp_u32<kDppRowHalfMirror>(v, v));
    v = op(v, dpp_u32<kDppRowMirror>(v, v));
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return op(op(r0, r1), op(r2, r3));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    return wave_reduce_u32(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    return wave_reduce_u32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    return wave_reduce_u32(v, [](uint32_t a, uint32_t b) { return a + b; });
}

// Inclusive prefix sum over the 64 lanes of a wave (lane order): shifts by 1, 2, 4, 8 within
// each row of 16, then the running totals of rows 0 and 0..1 are carried into later rows.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
    v += dpp_u32<dpp_row_shr(1)>(0u, v);
    v += dpp_u32<dpp_row_shr(2)>(0u, v);
    v += dpp_u32<dpp_row_shr(4)>(0u, v);
    v += dpp_u32<dpp_row_shr(8)>(0u, v);
    v += dpp_u32<kDppRowBcast15, 0xA>(0u, v);
    v += dpp_u32<kDppRowBcast31, 0xC>(0u, v);
    return v;
}

// Store one 32 x 32 accumulator tile of v_mfma_f32_32x32x*: rows row0 + 8(r/4) + 4hh + r%4
// for r = 0..15 (hh = lane / 32), column col0 + lane % 32, into a row-major bf16 matrix with
// leading dimension ld; rows >= n_rows are skipped.  Lanes 2j and 2j+1 trade one value (DPP
// swap of adjacent lanes) so that each lane stores two adjacent columns of one row in 4 bytes
// -- the even lane row R, the odd lane row R + 1 -- half as many store instructions, each
// writing 64-byte runs.
__device__ __forceinline__ void store_tile_bf16(uint16_t* dst, int64_t ld, int row0, int col0,
                                                const float (&v)[16], int lane,
                                                int n_rows = 0x7fffffff) {
    const bool odd = lane & 1;
    const int hh = (lane >> 5) & 1;
    const int col = col0 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
        const int row = row0 + 8 * (r >> 2) + 4 * hh + (r & 3);  // r % 4 is 0 or 2
        const float send = odd ? v[r] : v[r + 1];
        const float recv = __uint_as_float(dpp_u32<kDppQuadXor1>(0u, __float_as_uint(send)));
        const uint32_t packed = odd ? pack_bf16x2(recv, v[r + 1]) : pack_bf16x2(v[r], recv);
        const int my_row = row + (odd ? 1 : 0);
        if (my_row < n_rows)
            *reinterpret_cast<uint32_t*>(dst + static_cast<int64_t>(my_row) * ld + col - (odd ? 1 : 0)) = packed;
    }
}

// Compute units of the current device, looked up once per device (defined in topk.hip).
int device_cus();

}  // namespace dsa
