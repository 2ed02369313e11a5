// Stage 2 for prefill chunks: indexer scores  s_tj = sum_h w_th * max(0, q_th . k_j)  of many
// queries of one request over their causal key ranges.
//
// Page "Kimi K3.1 Pro: Sparse-Zugriffe, keine kleinere Historie", section "Eine Query durch
// den Indexer verfolgen": 32 index-query heads of width 128 per query, one shared 128-wide
// key per stored position, 32 head weights; section "Warum Top-2048 keinen 2048-Token-Cache
// bedeutet": scoring still covers every admissible position.
//
// Every key tile is reused by 16 queries x 32 heads, so the work is a dense contraction on
// the matrix cores: v_mfma_f32_32x32x16_bf16 with the 32 heads of one query as M, 32 keys as
// N and the 128 dims as K (8 steps).  The ReLU, the head weights and the head sum are a VALU
// epilogue of 2 instructions per (head, key) -- half the VALU issue rate at full MFMA rate,
// so it must overlap the MFMAs rather than follow them.  Each wave therefore runs a
// two-stage pipeline over half tiles of 32 keys: while the MFMAs of one half tile execute,
// the epilogue of the previous half tile (other accumulator set) issues in between.
//
// Keys reach LDS by direct global->LDS copies (no register staging) into a four-slot ring of
// 64-key tiles, three tiles ahead of the MFMAs; one barrier per tile.
#include "common.h"

namespace dsa {

namespace {

constexpr int kPQ = 16;          // queries per block: 2 per wave, 8 waves
constexpr int kPTile = 64;       // keys per LDS tile (16 KB)
constexpr int kPRing = 4;        // ring slots: tiles i..i+3 (i+3 being copied)
constexpr int kPCopies = kPTile / 4 / 8;  // 1 KB copies (4 keys each) per wave per tile: 2

__device__ __forceinline__ int64_t admissible_n(const int64_t* kv_off, int b, int32_t pos,
                                                int64_t max_s) {
    const int64_t s_b = kv_off[b + 1] - kv_off[b];
    int64_t n = static_cast<int64_t>(pos) + 1;
    n = n < s_b ? n : s_b;
    n = n < max_s ? n : max_s;
    return n > 0 ? n : 0;
}

}  // namespace

// grid: one block per 16 consecutive queries; 512 threads (8 waves, 2 per SIMD), each wave
// owning two queries (query 2w + j of the block, j = 0, 1).
// LDS tile layout: key r of the tile occupies 256 bytes; its 16-byte piece p (dims 8p..8p+7)
// sits at position p ^ (r % 16).  Copy d (0..15) of a tile moves keys 4d..4d+3: lane 16g + c
// loads piece c ^ (r % 16) of key r = 4d + g to position c, so one copy fills 1 KB of LDS
// contiguously.  The B-operand read of step s (16 lanes, 16 keys with distinct r % 16, one
// piece each) then touches 16 distinct 16-byte bank groups.
// MFMA 32x32x16: lane l (hh = l / 32) supplies head / key l % 32 and dims [64 hh + 8 s, +8)
// at step s; the accumulator gives lane l the key l % 32 and the heads
// 8 (r / 4) + 4 hh + r % 4, r = 0..15.
__global__ __launch_bounds__(512) void indexer_prefill_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ keys, const int64_t* __restrict__ kv_off,
    const int32_t* __restrict__ q_req, const int32_t* __restrict__ q_pos, int32_t T,
    int64_t max_s, float* __restrict__ scores, int64_t ld) {
    __shared__ __attribute__((aligned(1024))) uint16_t ring[kPRing][kPTile * kIndexDim];
    __shared__ int64_t s_n[kPQ];
    __shared__ int32_t s_req[kPQ];

    const int t0 = blockIdx.x * kPQ;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5;
    const int col = lane & 31;
    const int g = lane >> 4;
    const int c = lane & 15;

    if (tid < kPQ) {
        const int t = t0 + tid;
        if (t < T) {
            s_req[tid] = q_req[t];
            s_n[tid] = admissible_n(kv_off, q_req[t], q_pos[t], max_s);
        } else {
            s_req[tid] = -1;
            s_n[tid] = 0;
        }
    }
    lds_barrier();

    // the wave's two queries: A operands (8 K-steps each) and head weights in accumulator order
    bf16x8 qa[2][8];
    float wr[2][16];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int t = t0 + 2 * wave + j;
        const int tt = t < T ? t : 0;
        const uint16_t* qt = q_idx + static_cast<int64_t>(tt) * kIndexHeads * kIndexDim;
#pragma unroll
        for (int s = 0; s < 8; ++s)
            qa[j][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qt + col * kIndexDim + 64 * hh + 8 * s));
#pragma unroll
        for (int r = 0; r < 16; ++r)
            wr[j][r] = bf16_to_f32(w[tt * kIndexHeads + 8 * (r >> 2) + 4 * hh + (r & 3)]);
    }
    // After the epilogue's half swap, lanes 0..31 hold query 2w and lanes 32..63 query 2w+1.
    const int my_q = 2 * wave + hh;
    float* my_row = scores + static_cast<int64_t>(t0 + my_q) * ld;

    // The queries of a block normally share one request.  If they do not, the block makes
    // one pass per distinct request, each pass scoring only that request's queries.
    int done_mask = 0;  // bit i: query i of the block handled (uniform across the block)
    for (int qi = 0; qi < kPQ; ++qi)
        if (s_req[qi] < 0 || s_n[qi] == 0) done_mask |= 1 << qi;
    while (done_mask != (1 << kPQ) - 1) {
        int req = -1;
        for (int qi = 0; qi < kPQ; ++qi)
            if (!(done_mask & (1 << qi))) { req = s_req[qi]; break; }
        int64_t n_max = 0;
        int pass_mask = 0;
        for (int qi = 0; qi < kPQ; ++qi)
            if (!(done_mask & (1 << qi)) && s_req[qi] == req) {
                pass_mask |= 1 << qi;
                n_max = s_n[qi] > n_max ? s_n[qi] : n_max;
            }
        // this lane's store limit: its query's count if the query is in this pass, else 0
        const int64_t my_n = (pass_mask >> my_q) & 1 ? s_n[my_q] : 0;
        const uint16_t* kb = keys + kv_off[req] * kIndexDim;
        const int n_tiles = static_cast<int>((n_max + kPTile - 1) / kPTile);

        // This wave's two copies of `tile` into its ring slot.  Keys past n_max (the tail of
        // the last tile, and the tiles past the end that keep the copy count uniform) copy an
        // in-bounds key of the request instead; their scores are never stored.
        auto issue = [&](int tile) {
            const uint16_t* slot = ring[tile & (kPRing - 1)];
#pragma unroll
            for (int d = 0; d < kPCopies; ++d) {
                const int cp = kPCopies * wave + d;
                const int r = 4 * cp + g;
                int64_t key = static_cast<int64_t>(tile) * kPTile + r;
                key = key < n_max ? key : n_max - 1;
                copy_to_lds(kb + key * kIndexDim + 8 * (c ^ (r & 15)),
                            lds_offset(slot + cp * 4 * kIndexDim));
            }
        };

        // MFMAs of half tile `half` (keys 32 half .. +31) of the tile in `kt`
        auto mfma_half = [&](const uint16_t* kt, int half, f32x16 (&acc)[2]) {
            const uint16_t* krow = kt + (32 * half + col) * kIndexDim;
            bf16x8 kf[8];
#pragma unroll
            for (int s = 0; s < 8; ++s)
                kf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(krow + 8 * ((8 * hh + s) ^ (col & 15))));
            acc[0] = f32x16{};
            acc[1] = f32x16{};
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], kf[s], acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], kf[s], acc[1], 0, 0, 0);
            }
        };

        // epilogue of a half tile whose first key is key0 (negative: nothing to store)
        auto epilogue = [&](const f32x16 (&acc)[2], int64_t key0) {
            float v0 = 0.f, v1 = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                v0 = __builtin_fmaf(wr[0][r], fmaxf(acc[0][r], 0.f), v0);
                v1 = __builtin_fmaf(wr[1][r], fmaxf(acc[1][r], 0.f), v1);
            }
            // v_permlane32_swap: the upper half of v0 trades places with the lower half of v1,
            // so lane l < 32 gets v0 of lane l + 32 and lane l + 32 gets v1 of lane l; the sum
            // is query 2w's score in lanes 0..31 and query 2w+1's in lanes 32..63.
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0),
                                                             __float_as_uint(v1), false, false);
            const float v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            const int64_t key = key0 + col;
            if (key >= 0 && key < my_n) my_row[key] = v;
        };

        issue(0);
        issue(1);
        issue(2);
        f32x16 acc_a[2], acc_b[2];
        acc_b[0] = f32x16{};
        acc_b[1] = f32x16{};
        for (int i = 0; i < n_tiles; ++i) {
            // this wave's copies of tile i are done once at most the 2 x kPCopies copies of
            // tiles i+1 and i+2 remain outstanding (loads complete in issue order; score
            // stores in between only make the wait stricter); the barrier then covers every
            // wave's copies, and every wave is done reading tile i-1, whose slot is refilled
            // below
            wait_vmcnt<2 * kPCopies>();
            lds_barrier();
            const uint16_t* kt = ring[i & (kPRing - 1)];
            const int64_t key0 = static_cast<int64_t>(i) * kPTile;
            mfma_half(kt, 0, acc_a);
            epilogue(acc_b, key0 - 32);   // second half of tile i-1 (none before tile 0)
            mfma_half(kt, 1, acc_b);
            epilogue(acc_a, key0);        // first half of tile i
            issue(i + kPRing - 1);
        }
        epilogue(acc_b, static_cast<int64_t>(n_tiles) * kPTile - 32);
        // no copy may still be writing this block's LDS when the ring is reused or the
        // block ends
        wait_vmcnt<0>();
        lds_barrier();
        done_mask |= pass_mask;
    }
}

hipError_t launch_indexer_prefill(const uint16_t* q_idx, const uint16_t* w, const uint16_t* keys,
                                  const int64_t* kv_off, const int32_t* q_req,
                                  const int32_t* q_pos, int32_t T, int64_t max_s, float* scores,
                                  int64_t ld, hipStream_t stream) {
    const int blocks = (T + kPQ - 1) / kPQ;
    hipLaunchKernelGGL(indexer_prefill_kernel, dim3(blocks), dim3(512), 0, stream, q_idx, w, keys,
                       kv_off, q_req, q_pos, T, max_s, scores, ld);
    return hipGetLastError();
}

}  // namespace dsa
