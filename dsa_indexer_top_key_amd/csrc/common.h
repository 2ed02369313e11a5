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
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

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

// Workgroup barrier that orders LDS only: LDS writes issued before it are visible to LDS
// reads after it, while global-memory loads (and global->LDS copies) stay in flight; where
// a kernel hands such data across the barrier it waits on vmcnt explicitly.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = min(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), m)));
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), m)));
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
    const int l = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t o = static_cast<uint32_t>(__shfl_up(static_cast<int>(v), d));
        if (l >= d) v += o;
    }
    return v;
}

}  // namespace dsa
