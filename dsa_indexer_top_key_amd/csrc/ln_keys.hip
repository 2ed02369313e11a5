// Stage 1: LayerNorm of the 128-wide index keys, fp32 in, bf16 (RNE) out.
//
// Page "Kimi K3.1 Pro: Sparse-Zugriffe, keine kleinere Historie", section "Eine Query durch
// den Indexer verfolgen": keys [S,128] are produced by a projection followed by LayerNorm;
// the adapter paragraph fixes LayerNorm (not RMSNorm), FP32 normalisation, no Hadamard
// transform and no rotation of index keys.
//
// HBM-bound streaming (512 B read + 256 B written per row).  Half a wave (32 lanes) owns
// one row: each lane holds four consecutive floats (one 16-byte load), the mean and the
// biased variance are reduced across the 32 lanes with xor-shuffles, and each lane stores
// four bf16 (8 bytes).  Every load and store is fully coalesced; a grid-stride loop over four
// blocks per CU keeps enough rows in flight to cover HBM latency.
#include "common.h"

namespace dsa {

// The keys are written once and not read back by this call: non-temporal stores (2 M keys,
// cold: 361 -> 345 us), like the non-temporal loads of the raw rows.
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float half_wave_sum(float v) {
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) v += __shfl_xor(v, m, 32);
    return v;
}

__global__ __launch_bounds__(256) void ln_keys_kernel(const float* __restrict__ raw,
                                                      const float* __restrict__ gamma,
                                                      const float* __restrict__ beta, float eps,
                                                      uint16_t* __restrict__ keys,
                                                      int64_t n_rows) {
    const int sub = threadIdx.x & 31;
    const int64_t group = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 5;
    const int64_t n_groups = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 5;
    const float4 g = reinterpret_cast<const float4*>(gamma)[sub];
    const float4 b = reinterpret_cast<const float4*>(beta)[sub];
    constexpr float inv_d = 1.0f / kIndexDim;
    // two rows per group per iteration keep two independent loads in flight
    for (int64_t row = group; row < n_rows; row += 2 * n_groups) {
        const int64_t row2 = row + n_groups;
        const bool has2 = row2 < n_rows;
        const f32x4 xv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(raw + row * kIndexDim) + sub);
        f32x4 yv = {0.f, 0.f, 0.f, 0.f};
        if (has2) yv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(raw + row2 * kIndexDim) + sub);
        const float4 x = make_float4(xv[0], xv[1], xv[2], xv[3]);
        const float4 y = make_float4(yv[0], yv[1], yv[2], yv[3]);
        const float mx = half_wave_sum((x.x + x.y) + (x.z + x.w)) * inv_d;
        const float my = half_wave_sum((y.x + y.y) + (y.z + y.w)) * inv_d;
        const float4 dx = make_float4(x.x - mx, x.y - mx, x.z - mx, x.w - mx);
        const float4 dy = make_float4(y.x - my, y.y - my, y.z - my, y.w - my);
        const float vx = half_wave_sum((dx.x * dx.x + dx.y * dx.y) + (dx.z * dx.z + dx.w * dx.w)) * inv_d;
        const float vy = half_wave_sum((dy.x * dy.x + dy.y * dy.y) + (dy.z * dy.z + dy.w * dy.w)) * inv_d;
        const float rx = 1.0f / sqrtf(vx + eps);
        const float ry = 1.0f / sqrtf(vy + eps);
        uint2 ox, oy;
        ox.x = pack_bf16x2(dx.x * rx * g.x + b.x, dx.y * rx * g.y + b.y);
        ox.y = pack_bf16x2(dx.z * rx * g.z + b.z, dx.w * rx * g.w + b.w);
        __builtin_nontemporal_store(u32x2v{ox.x, ox.y}, reinterpret_cast<u32x2v*>(keys + row * kIndexDim) + sub);
        if (has2) {
            oy.x = pack_bf16x2(dy.x * ry * g.x + b.x, dy.y * ry * g.y + b.y);
            oy.y = pack_bf16x2(dy.z * ry * g.z + b.z, dy.w * ry * g.w + b.w);
            __builtin_nontemporal_store(u32x2v{oy.x, oy.y}, reinterpret_cast<u32x2v*>(keys + row2 * kIndexDim) + sub);
        }
    }
}

hipError_t launch_ln_keys(const float* raw, const float* gamma, const float* beta, float eps,
                          uint16_t* keys, int64_t n_rows, hipStream_t stream) {
    // 8 rows per 256-thread block per pass, two passes per iteration; at most 4 blocks per CU
    // (grid-stride): on 2 M keys, cold, 4 per CU took 285 us, 3 per CU 323, 2 per CU 392, 6
    // per CU 295, 8 per CU 333 and 16 per CU 349 (more resident waves than needed to cover
    // the latency only slowed the mixed read/write stream)
    const int64_t want = (n_rows + 15) / 16;
    const int64_t cap = 4 * static_cast<int64_t>(device_cus());
    const int blocks = static_cast<int>(want < cap ? (want < 1 ? 1 : want) : cap);
    hipLaunchKernelGGL(ln_keys_kernel, dim3(blocks), dim3(256), 0, stream, raw, gamma, beta,
                       eps, keys, n_rows);
    return hipGetLastError();
}

}  // namespace dsa
