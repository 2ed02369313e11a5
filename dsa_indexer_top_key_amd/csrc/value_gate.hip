// Post-read epilogue: per-head value up-projection and the sigmoid output gate.
//
// Page "Kimi K3.1 Pro: Sparse-Zugriffe, keine kleinere Historie", section "Was ändert sich
// – und was nicht?": 96 main-attention heads with 128-wide value heads.  The sparse read stays
// in the shared 512-wide latent (absorbed MLA), so each head's value is its own
// up-projection of that read.  The paragraph after the Gated-MLA one: a learned,
// coordinatewise sigmoid output gate follows the sparse attention, before the output
// projection (input-dependent, per the K3 guide's MLA section).
//
//   u_th = (W_UV[h] o_th) * sigmoid(g_th)      o_th in R^512, W_UV[h] in R^{128 x 512}
//
// Bytes per call: T x (96 x 512 + 2 x 96 x 128) bf16 plus the 12.6 MB of W_UV; 128 MACs per
// byte of W_UV when T is large, 1 MAC per byte of o -- HBM-bound at every batch size.
//
// One block per (32 queries, head h); block index = query tile x 96 + h, so every block of a
// head lands on the same XCD (96 is a multiple of 8) and W_UV[h] (128 KB) stays in that
// XCD's L2 across query tiles.  Eight waves: wave w computes value columns 32 (w % 4) ..
// +31 over latent half w / 4 (256 dims) with v_mfma_f32_32x32x16_bf16 (A = 32 query rows of
// o, B = 32 rows of W_UV[h], K = latent dims), issuing all of its 32 loads before the first
// MFMA -- the call is small and latency-bound at decode sizes, so every byte a wave needs is
// requested at once.  The upper-half waves hand their partial sums to the lower-half waves
// through LDS.  K order: in each 64-dim slab a lane (row r, half hh) loads 64 contiguous
// bytes, dims 32 hh .. 32 hh + 31 of the slab, and K-step j of the slab takes its j-th 16
// bytes; A and B use the same order, so the contraction is unchanged.  The gate is applied to
// the fp32 sums (sigmoid in fp32) and the result is stored as bf16 (round to nearest even).
#include "common.h"

namespace dsa {

constexpr int kValueDim = 128;        // value head width
constexpr int kVgRows = 32;           // queries per block
constexpr int kVgSlabs = kLatent / 64 / 2;  // 64-dim slabs per latent half

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

__global__ __launch_bounds__(512) void value_gate_kernel(const uint16_t* __restrict__ o,
                                                         const uint16_t* __restrict__ w_uv,
                                                         const uint16_t* __restrict__ gate,
                                                         int32_t T, uint16_t* __restrict__ out) {
    __shared__ f32x16 part[4][64];  // upper-half partial sums, per column group and lane
    const int h = static_cast<int>(blockIdx.x) % kMlaHeads;
    const int t0 = (static_cast<int>(blockIdx.x) / kMlaHeads) * kVgRows;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int cg = wave & 3;   // value columns 32 cg .. 32 cg + 31
    const int kh = wave >> 2;  // latent dims 256 kh .. 256 kh + 255
    const int r = lane & 31;
    const int hh = lane >> 5;
    // A row: query t0 + r (rows past T read the last query; their results are not stored)
    const int tq = t0 + r < T ? t0 + r : T - 1;
    const u32x4* arow = reinterpret_cast<const u32x4*>(o + (static_cast<int64_t>(tq) * kMlaHeads + h) * kLatent + 256 * kh + 32 * hh);
    const u32x4* brow = reinterpret_cast<const u32x4*>(w_uv + (static_cast<int64_t>(h) * kValueDim + 32 * cg + r) * kLatent + 256 * kh + 32 * hh);
    u32x4 a[kVgSlabs][4], b[kVgSlabs][4];
#pragma unroll
    for (int s2 = 0; s2 < kVgSlabs; ++s2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // a slab is 64 dims = 8 u32x4 further along the row
            a[s2][j] = arow[8 * s2 + j];
            b[s2][j] = brow[8 * s2 + j];
        }
    // keep every load ahead of the MFMAs (left alone, the scheduler sinks each load next to
    // its MFMA and leaves about three in flight)
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc = {};
#pragma unroll
    for (int s2 = 0; s2 < kVgSlabs; ++s2)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[s2][j]), as_bf16x8(b[s2][j]), acc, 0, 0, 0);
    if (kh == 1) part[cg][lane] = acc;
    __syncthreads();
    if (kh == 1) return;  // block-uniform per wave; no barrier follows
    acc += part[cg][lane];
    // epilogue: acc[i] is query row 8(i/4) + 4hh + i%4, value column 32 cg + r
    const int col = 32 * cg + r;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = t0 + 8 * (i >> 2) + 4 * hh + (i & 3);
        const int rr = row < T ? row : T - 1;
        const float g = bf16_to_f32(gate[(static_cast<int64_t>(rr) * kMlaHeads + h) * kValueDim + col]);
        v[i] = acc[i] * sigmoidf_(g);
    }
    store_tile_bf16(out + (static_cast<int64_t>(t0) * kMlaHeads + h) * kValueDim, kMlaHeads * kValueDim,
                    0, 32 * cg, v, lane, T - t0);
}

hipError_t launch_value_gate(const uint16_t* o, const uint16_t* w_uv, const uint16_t* gate,
                             int32_t T, uint16_t* out, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    const int64_t blocks = static_cast<int64_t>((T + kVgRows - 1) / kVgRows) * kMlaHeads;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(value_gate_kernel, dim3(static_cast<unsigned>(blocks)), dim3(512), 0,
                       stream, o, w_uv, gate, T, out);
    return hipGetLastError();
}

}  // namespace dsa
