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
// two-stage pipeline over sub-tiles of 32 keys: while the MFMAs of one sub-tile execute,
// the epilogue of the previous sub-tile (other accumulator set) issues in between.
//
// Keys reach LDS by direct global->LDS copies (no register staging) into a four-slot ring of
// 128-key tiles, three tiles ahead of the MFMAs; one barrier per tile.  Within a tile the key
// operands roll: the register holding step s of one sub-tile is refilled with step s of the
// next sub-tile as soon as both MFMAs of step s have issued.
//
// Measured on the 4096-query chunk at 61440..65535 (2.13 TFLOP of causal scoring): the
// sustained clock under this load is about 1.7 GHz, at which the matrix cores are busy about
// 62% of cycles.  Without the epilogue the loop reached 1.68 ms, without the score stores
// 1.86 ms, against 2.01 ms for the whole kernel; 64-key tiles, an eight-slot ring and
// non-temporal score stores were all within 1% of this shape, and one wave per SIMD with four
// queries each (512 registers) was 20% slower; staging each tile's scores in LDS and storing
// them as 16-byte rows two tiles later (fewer stores between the key copies) was 4% slower.
#include "common.h"

namespace dsa {

namespace {

constexpr int kPQ = 16;          // queries per block
constexpr int kQPW = 2;          // queries per wave: 8 waves, 2 per SIMD
constexpr int kPTile = 128;      // keys per LDS tile (32 KB)
constexpr int kPRing = 4;        // ring slots: tiles i..i+3 (i+3 being copied)

}  // namespace

// grid: one block per 16 consecutive queries; 512 threads (8 waves), wave w owning queries
// 2w and 2w + 1 of the block.
// LDS tile layout: key r of the tile occupies 256 bytes; its 16-byte piece p (dims 8p..8p+7)
// sits at position p ^ (r % 16).  Copy d (0..15) of a tile moves keys 4d..4d+3: lane 16g + c
// loads piece c ^ (r % 16) of key r = 4d + g to position c, so one copy fills 1 KB of LDS
// contiguously.  The B-operand read of step s (16 lanes, 16 keys with distinct r % 16, one
// piece each) then touches 16 distinct 16-byte bank groups.
// MFMA 32x32x16: lane l (hh = l / 32) supplies head / key l % 32 and dims [64 hh + 8 s, +8)
// at step s; the accumulator gives lane l the key l % 32 and the heads
// 8 (r / 4) + 4 hh + r % 4, r = 0..15.
__global__ __launch_bounds__(64 * (kPQ / kQPW)) void indexer_prefill_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ keys, const int64_t* __restrict__ kv_off,
    const int32_t* __restrict__ q_req, const int32_t* __restrict__ q_pos, int32_t T, int32_t B,
    int64_t max_s, float* __restrict__ scores, int64_t ld) {
    constexpr int QPW = kQPW;
    constexpr int kWaves = kPQ / QPW;
    constexpr int kCopies = kPTile / 4 / kWaves;  // 1 KB copies (4 keys each) per wave per tile
    constexpr int kPairs = QPW / 2;
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
            const int b = query_request(q_req, t, B);
            s_req[tid] = b;  // -1 outside the batch: no admissible position
            s_n[tid] = admissible_count(kv_off, b, q_pos[t], max_s);
        } else {
            s_req[tid] = -1;
            s_n[tid] = 0;
        }
    }
    lds_barrier();

    // the wave's queries: A operands (8 K-steps each) and head weights in accumulator order
    bf16x8 qa[QPW][8];
    float wr[QPW][16];
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
        const int t = t0 + QPW * wave + j;
        const int tt = t < T ? t : 0;
        const uint16_t* qt = q_idx + static_cast<int64_t>(tt) * kIndexHeads * kIndexDim;
#pragma unroll
        for (int s = 0; s < 8; ++s)
            qa[j][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qt + col * kIndexDim + 64 * hh + 8 * s));
#pragma unroll
        for (int r = 0; r < 16; ++r)
            wr[j][r] = bf16_to_f32(w[tt * kIndexHeads + 8 * (r >> 2) + 4 * hh + (r & 3)]);
    }
    // After the epilogue's half swap of pair p, lanes 0..31 hold query QPW w + 2p and lanes
    // 32..63 query QPW w + 2p + 1.
    int my_q[kPairs];
    float* my_row[kPairs];
#pragma unroll
    for (int p = 0; p < kPairs; ++p) {
        my_q[p] = QPW * wave + 2 * p + hh;
        my_row[p] = scores + static_cast<int64_t>(t0 + my_q[p]) * ld;
    }

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
        // this lane's store limits: its queries' counts if they are in this pass, else 0
        int64_t my_n[kPairs];
#pragma unroll
        for (int p = 0; p < kPairs; ++p) my_n[p] = (pass_mask >> my_q[p]) & 1 ? s_n[my_q[p]] : 0;
        const uint16_t* kb = keys + kv_off[req] * kIndexDim;
        const int n_tiles = static_cast<int>((n_max + kPTile - 1) / kPTile);

        // This wave's copies of `tile` into its ring slot.  Keys past n_max (the tail of the
        // last tile, and the tiles past the end that keep the copy count uniform) copy an
        // in-bounds key of the request instead; their scores are never stored.
        auto issue = [&](int tile) {
            const uint16_t* slot = ring[tile % kPRing];
#pragma unroll
            for (int d = 0; d < kCopies; ++d) {
                const int cp = kCopies * wave + d;
                const int r = 4 * cp + g;
                int64_t key = static_cast<int64_t>(tile) * kPTile + r;
                key = key < n_max ? key : n_max - 1;
                copy_to_lds(kb + key * kIndexDim + 8 * (c ^ (r & 15)),
                            lds_offset(slot + cp * 4 * kIndexDim));
            }
        };

        // epilogue of a sub-tile whose first key is key0 (negative: nothing to store)
        auto epilogue = [&](const f32x16 (&acc)[QPW], int64_t key0) {
            const int64_t key = key0 + col;
#pragma unroll
            for (int p = 0; p < kPairs; ++p) {
                float v0 = 0.f, v1 = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    v0 = __builtin_fmaf(wr[2 * p][r], fmaxf(acc[2 * p][r], 0.f), v0);
                    v1 = __builtin_fmaf(wr[2 * p + 1][r], fmaxf(acc[2 * p + 1][r], 0.f), v1);
                }
                // v_permlane32_swap: the upper half of v0 trades places with the lower half
                // of v1, so lane l < 32 gets v0 of lane l + 32 and lane l + 32 gets v1 of lane
                // l; the sum is query 2p's score in lanes 0..31 and query 2p+1's in 32..63.
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0),
                                                                 __float_as_uint(v1), false, false);
                const float v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                if (key >= 0 && key < my_n[p]) my_row[p][key] = v;
            }
        };

#pragma unroll
        for (int j = 0; j < kPRing - 1; ++j) issue(j);
        f32x16 acc_a[QPW], acc_b[QPW];
#pragma unroll
        for (int j = 0; j < QPW; ++j) acc_b[j] = f32x16{};
        for (int i = 0; i < n_tiles; ++i) {
            // this wave's copies of tile i are done once at most the copies of the kPRing - 2
            // tiles after it remain outstanding (loads complete in issue order; score stores
            // in between only make the wait stricter); the barrier then covers every wave's
            // copies, and every wave is done reading tile i-1, whose slot is refilled below
            wait_vmcnt<(kPRing - 2) * kCopies>();
            lds_barrier();
            const uint16_t* kt = ring[i % kPRing];
            const int64_t key0 = static_cast<int64_t>(i) * kPTile;
            // B operands of sub-tile h (keys 32 h .. 32 h + 31 of the tile), step s
            auto operand = [&](int h, int s) {
                const uint16_t* krow = kt + (32 * h + col) * kIndexDim;
                return as_bf16x8(*reinterpret_cast<const u32x4*>(krow + 8 * ((8 * hh + s) ^ (col & 15))));
            };
            bf16x8 kf[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) kf[s] = operand(0, s);
#pragma unroll
            for (int h = 0; h < kPTile / 32; ++h) {
                // even sub-tiles accumulate into acc_a, odd ones into acc_b; the epilogue of
                // the previous sub-tile (the other set) issues between these MFMAs
                f32x16 (&acc)[QPW] = (h & 1) ? acc_b : acc_a;
                f32x16 (&prev)[QPW] = (h & 1) ? acc_a : acc_b;
#pragma unroll
                for (int j = 0; j < QPW; ++j) acc[j] = f32x16{};
                // raised wave priority while this wave issues its MFMAs, so the SIMD's other
                // wave (in its epilogue) yields the issue slot to them (1% measured)
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int s = 0; s < 8; ++s) {
#pragma unroll
                    for (int j = 0; j < QPW; ++j)
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[j][s], kf[s], acc[j], 0, 0, 0);
                    if (h + 1 < kPTile / 32) kf[s] = operand(h + 1, s);
                }
                __builtin_amdgcn_s_setprio(0);
                epilogue(prev, key0 + 32 * h - 32);   // none before key 0
            }
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
                                  const int32_t* q_pos, int32_t T, int32_t B, int64_t max_s,
                                  float* scores, int64_t ld, hipStream_t stream) {
    const int blocks = (T + kPQ - 1) / kPQ;
    hipLaunchKernelGGL(indexer_prefill_kernel, dim3(blocks), dim3(64 * (kPQ / kQPW)), 0, stream,
                       q_idx, w, keys, kv_off, q_req, q_pos, T, B, max_s, scores, ld);
    return hipGetLastError();
}

}  // namespace dsa
