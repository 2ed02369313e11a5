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
// One block per (head h, range of 32-query tiles); the four waves own the four groups of 32
// value columns.  Each wave keeps its 32 rows of W_UV[h] -- all 512 latent dims, as the B
// operands of the 32 K-steps -- in registers for the whole block, so the weights are read
// once per block.  Half of them arrive through LDS by whole-line copies (the other half is
// loaded straight into registers, so that all of W_UV[h] is in flight at once; see the
// staging below).  The query tiles stream through a two-slot LDS ring by direct
// global->LDS copies: the 32 rows of o (one 1 KB row per copy instruction, whole 128-byte
// lines) and the 32 gate rows of head h (four 256-byte rows per copy), one tile ahead.  Per
// tile a wave runs 32 v_mfma_f32_32x32x16_bf16 (A = query rows of o from LDS at a 1040-byte
// row stride, bank-conflict-free), applies the gate to the fp32 sums (sigmoid in fp32) and
// stores bf16 (round to nearest even).  Block index = split x 96 + h, so all blocks of a head
// run on one XCD (96 is a multiple of 8) and share W_UV[h] in its L2.
#include "common.h"

namespace dsa {

constexpr int kValueDim = 128;          // value head width
constexpr int kVgRows = 32;             // queries per tile
constexpr int kVgStride = kLatent + 8;  // LDS row stride of o in bf16 elements (1040 bytes)
constexpr int kVgCopies = 8 + 2;        // copies per wave and tile: 8 rows of o, 2 x 4 gate rows
constexpr int kVgQuarter = kLatent / 4;  // latent dims of W_UV per LDS stage
constexpr int kVgWCopies = kValueDim * kVgQuarter * 2 / 1024 / 4;  // 1 KB copies per wave and quarter (8)

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

__global__ __launch_bounds__(256, 1) void value_gate_kernel(const uint16_t* __restrict__ o,
                                                            const uint16_t* __restrict__ w_uv,
                                                            const uint16_t* __restrict__ gate,
                                                            int32_t T, int32_t n_tiles,
                                                            int32_t n_split,
                                                            uint16_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint16_t a_lds[2][kVgRows * kVgStride];
    __shared__ __attribute__((aligned(16))) uint16_t g_lds[2][kVgRows * kValueDim];
    __shared__ __attribute__((aligned(16))) uint16_t w_lds[2][kValueDim * kVgQuarter];
    const int h = static_cast<int>(blockIdx.x) % kMlaHeads;
    const int split = static_cast<int>(blockIdx.x) / kMlaHeads;
    const int tt0 = static_cast<int>(static_cast<int64_t>(n_tiles) * split / n_split);
    const int tt1 = static_cast<int>(static_cast<int64_t>(n_tiles) * (split + 1) / n_split);
    const int lane = lane_id();
    const int cg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave = column group
    const int r = lane & 31;
    const int hh = lane >> 5;
    // The first two quarters of the latent dims of W_UV[h] (128 rows x 256 bytes each) reach
    // LDS by whole-line global->LDS copies: copy k of a quarter moves rows 4k .. 4k+3, lane l
    // the 16-byte piece (l % 16) ^ (row % 16) of row 4k + l / 16 into piece slot l % 16.  Each
    // wave then reads its B operands (row 32 cg + r, piece 2 s' + hh of the quarter) into
    // registers; eight lanes at a time read eight rows at distinct slots, so the reads are
    // free of bank conflicts.  Loaded straight into registers, every load instruction gathers
    // 32 bytes from each of 32 rows; all four quarters through a two-slot ring left only two
    // in flight at a time, which a cold call paid for twice.
    const uint16_t* wh = w_uv + static_cast<int64_t>(h) * kValueDim * kLatent;
    auto stage_w = [&](int q, int b) {
#pragma unroll
        for (int k = 0; k < kVgWCopies; ++k) {
            const int c = kVgWCopies * cg + k;  // copy index of the quarter, 0 .. 31
            const int row = 4 * c + (lane >> 4);
            const int piece = (lane & 15) ^ (row & 15);
            copy_to_lds(wh + static_cast<int64_t>(row) * kLatent + kVgQuarter * q + 8 * piece,
                        lds_offset(w_lds[b] + c * 4 * kVgQuarter));
        }
    };
    u32x4 bw[kLatent / 16];
    auto read_w = [&](int q, int b) {
        const int row = 32 * cg + r;
        const uint16_t* wr = w_lds[b] + row * kVgQuarter;
#pragma unroll
        for (int s = 0; s < kVgQuarter / 16; ++s)
            bw[(kVgQuarter / 16) * q + s] =
                *reinterpret_cast<const u32x4*>(wr + 8 * ((2 * s + hh) ^ (row & 15)));
    };
    // copies of tile tt into slot b: rows 8 cg .. 8 cg + 7 of o, gate rows 8 cg .. 8 cg + 7
    // (lane l of a gate copy moves bytes 16 (l % 16) .. of gate row 4 k + l / 16); rows past T
    // copy the last query.  Each row is read by this block only: the copies carry the
    // non-temporal hint (cold calls 14.4 -> 13.7 us at 64 queries, 35.4 -> 31.3 us at 300).
    auto stage = [&](int tt, int b) {
        const int t0 = tt * kVgRows;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int row = 8 * cg + k;
            const int tq = t0 + row < T ? t0 + row : T - 1;
            copy_to_lds<true>(o + (static_cast<int64_t>(tq) * kMlaHeads + h) * kLatent + 8 * lane,
                        lds_offset(a_lds[b] + row * kVgStride));
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int row = 8 * cg + 4 * k + (lane >> 4);
            const int tq = t0 + row < T ? t0 + row : T - 1;
            copy_to_lds<true>(gate + (static_cast<int64_t>(tq) * kMlaHeads + h) * kValueDim + 8 * (lane & 15),
                        lds_offset(g_lds[b] + (8 * cg + 4 * k) * kValueDim));
        }
    };
    // quarters 0 and 1 through LDS, quarters 2 and 3 straight into registers (each lane its 16
    // bytes of row 32 cg + r per K-step), then the first tile: every byte of W_UV[h] is in
    // flight at once
    stage_w(0, 0);
    stage_w(1, 1);
    {
        const uint16_t* wrow = wh + static_cast<int64_t>(32 * cg + r) * kLatent + 8 * hh;
#pragma unroll
        for (int s = kLatent / 32; s < kLatent / 16; ++s) bw[s] = *reinterpret_cast<const u32x4*>(wrow + 16 * s);
    }
    if (tt0 < tt1) stage(tt0, 0);
    // quarter 0 is in once at most the 8 copies of quarter 1, the 16 register loads and the
    // tile's copies are outstanding; quarter 1 once only the latter two are
    if (tt0 < tt1) wait_vmcnt<kVgWCopies + 16 + kVgCopies>(); else wait_vmcnt<kVgWCopies + 16>();
    lds_barrier();
    read_w(0, 0);
    if (tt0 < tt1) wait_vmcnt<16 + kVgCopies>(); else wait_vmcnt<16>();
    lds_barrier();
    read_w(1, 1);
    for (int tt = tt0; tt < tt1; ++tt) {
        const int b = (tt - tt0) & 1;
        // tile tt landed once only the copies issued after it may be outstanding
        if (tt + 1 < tt1) {
            stage(tt + 1, b ^ 1);
            wait_vmcnt<kVgCopies>();
        } else {
            wait_vmcnt<0>();
        }
        __syncthreads();  // every wave's copies of tile tt are in
        const uint16_t* ap = a_lds[b] + r * kVgStride + 8 * hh;
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < kLatent / 16; ++s)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                as_bf16x8(*reinterpret_cast<const u32x4*>(ap + 16 * s)), as_bf16x8(bw[s]), acc, 0, 0, 0);
        // epilogue: acc[e] is query row 8(e/4) + 4hh + e%4 of the tile, value column 32 cg + r
        const int t0 = tt * kVgRows;
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = 8 * (e >> 2) + 4 * hh + (e & 3);
            v[e] = acc[e] * sigmoidf_(bf16_to_f32(g_lds[b][row * kValueDim + 32 * cg + r]));
        }
        store_tile_bf16(out + (static_cast<int64_t>(t0) * kMlaHeads + h) * kValueDim,
                        kMlaHeads * kValueDim, 0, 32 * cg, v, lane, T - t0);
        __syncthreads();  // slot b is refilled by the next iteration's copies
    }
}

hipError_t launch_value_gate(const uint16_t* o, const uint16_t* w_uv, const uint16_t* gate,
                             int32_t T, uint16_t* out, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    const int n_tiles = (T + kVgRows - 1) / kVgRows;
    // splits per head: up to 8 (768 blocks: three rounds of one block per CU), at most one
    // per tile
    const int n_split = n_tiles < 8 ? n_tiles : 8;
    hipLaunchKernelGGL(value_gate_kernel, dim3(static_cast<unsigned>(kMlaHeads * n_split)), dim3(256),
                       0, stream, o, w_uv, gate, T, n_tiles, n_split, out);
    return hipGetLastError();
}

}  // namespace dsa
