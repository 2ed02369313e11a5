// Stage 2: indexer scores  s_tj = sum_h w_th * max(0, q_th . k_j)  over the admissible
// (causal) positions of each query.
//
// Page "Kimi K3.1 Pro: Sparse-Zugriffe, keine kleinere Historie", section "Eine Query durch
// den Indexer verfolgen" and the indexer paragraph before it: 32 query heads of width 128
// [T,32,128], one shared 128-wide key per stored position [S,128], 32 head weights per
// query on the BF16 head-gate path, scoring over every admissible position (section "Warum
// Top-2048 keinen 2048-Token-Cache bedeutet": scoring still covers the whole history).
//
// The per-(query, key) work is a 32 x 128 by 128 x 1 contraction, so the heads form the
// M dimension of BF16 MFMA tiles and keys the N dimension; the ReLU, the head weighting and
// the sum over heads are an epilogue on the accumulators.
//
// Two kernels:
//  * decode  -- one query per request.  Each query streams its S keys once from HBM
//    (256 B per key, 32 flop/B), so the kernel is HBM-bound.  Keys stream through per-wave
//    LDS rings by direct global->LDS copies of whole 1 KB spans (non-temporal), feed the B
//    operand of v_mfma_f32_16x16x32_bf16 from there, and the scores leave in one burst per
//    block.
//  * prefill -- many queries of one request.  A block owns 16 consecutive queries and walks
//    their causal key range in 32-key tiles staged through LDS (double-buffered); every key
//    tile feeds 16 queries x 32 heads of v_mfma_f32_32x32x16_bf16, so the kernel is bound by
//    MFMA throughput rather than HBM.
#include "common.h"

namespace dsa {

// Admissible count n_t = min(q_pos + 1, S_b), clamped to [0, max_s].
__device__ __forceinline__ int64_t admissible(const int64_t* kv_off, int b, int32_t pos,
                                              int64_t max_s) {
    const int64_t s_b = kv_off[b + 1] - kv_off[b];
    int64_t n = static_cast<int64_t>(pos) + 1;
    n = n < s_b ? n : s_b;
    n = n < max_s ? n : max_s;
    return n > 0 ? n : 0;
}

// ---------------------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------------------
constexpr int kDecodeTile = 16;          // keys per wave step: 4 KB, four 1 KB copies
constexpr int kDecodeRing = 3;           // ring slots per wave (two steps in flight)
constexpr int kDecodeCopies = kDecodeTile / 4;
constexpr int kDecodeMaxChunk = 4096;    // keys per block at most (their scores: 16 KB of LDS)
constexpr int kDecodeMinChunk = 1024;

// Keys per block: the whole job spread over about two blocks per CU (64 KB of LDS each, so
// two fit; all blocks then end at about the same time and the score writes leave as one
// burst), within [1024, 4096] keys and a multiple of one block step (64 keys).  With one
// block (four waves) per CU the MFMA and reduction latency of each tile is no longer hidden
// (8192-key blocks measured 60% slower).
static int64_t decode_chunk(int32_t T, int64_t max_s) {
    int64_t c = (static_cast<int64_t>(T) * max_s + 511) / 512;
    c = (c + 63) & ~static_cast<int64_t>(63);
    c = c < kDecodeMinChunk ? kDecodeMinChunk : c;
    return c > kDecodeMaxChunk ? kDecodeMaxChunk : c;
}

// grid: one block per (query, chunk of keys); 4 waves per block, each streaming its own
// 16-key tiles (tile i of the chunk belongs to wave i % 4) through a private three-slot LDS
// ring.  Each copy instruction moves 1 KB = 4 whole keys, so every instruction covers whole
// 128-byte lines (key-major loads of 64 bytes per key and instruction measured 15% slower).
// Lane l = 16 g + c of a copy loads key 4 d + g of the tile, 16-byte piece c ^ (key % 16)
// into LDS slot c of that key's 256-byte row: the MFMA operand reads below (16 lanes, 16
// different keys, one piece each) then fall in 16 distinct bank groups.
// MFMA 16x16x32: A = q (rows: 16 heads), B = keys (cols: 16 keys), K = 32 dims per step.
// Lane l = 16 g + c supplies head/key c and the dims [32 s + 8 g, +8) at step s; the 16x16
// accumulator gives lane l the key c and heads 4 g + r (r = 0..3).
// Scores collect in LDS and leave at the end of the block in full 16-byte stores: writes
// interleaved with the key stream measured about 10% slower than one burst at the end.
__global__ __launch_bounds__(256) void indexer_decode_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ keys, const int64_t* __restrict__ kv_off,
    const int32_t* __restrict__ q_req, const int32_t* __restrict__ q_pos, int32_t chunks_per_q,
    int32_t chunk, int64_t max_s, float* __restrict__ scores, int64_t ld, int vec_store) {
    __shared__ __attribute__((aligned(16))) uint16_t ring[4][kDecodeRing][kDecodeTile * kIndexDim];
    __shared__ __attribute__((aligned(16))) float sbuf[kDecodeMaxChunk];
    const int t = blockIdx.x / chunks_per_q;
    const int ci = blockIdx.x - t * chunks_per_q;
    const int b = q_req[t];
    const int64_t n = admissible(kv_off, b, q_pos[t], max_s);
    const int64_t k0 = static_cast<int64_t>(ci) * chunk;
    if (k0 >= n) return;  // block-uniform
    const int len = static_cast<int>((k0 + chunk < n ? k0 + chunk : n) - k0);

    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int c = lane & 15;
    const uint16_t* kb = keys + (kv_off[b] + k0) * kIndexDim;
    const int n_tiles = (len + kDecodeTile - 1) / kDecodeTile;
    const int my_tiles = n_tiles > wave ? (n_tiles - wave + 3) / 4 : 0;
    // copies of this wave's j-th tile into ring slot j % 3; keys past the end copy key 0
    auto issue = [&](int j) {
        const int kt = (wave + 4 * j) * kDecodeTile;
        const uint16_t* slot = ring[wave][j % kDecodeRing];
#pragma unroll
        for (int d = 0; d < kDecodeCopies; ++d) {
            const int r = 4 * d + g;
            const int key = kt + r < len ? kt + r : 0;
            copy_to_lds<true>(kb + static_cast<int64_t>(key) * kIndexDim + 8 * (c ^ r),
                              lds_offset(slot + d * 4 * kIndexDim));
        }
    };
#pragma unroll
    for (int j = 0; j < kDecodeRing - 1; ++j)
        if (j < my_tiles) issue(j);

    bf16x8 qa[2][4];
    const uint16_t* qt = q_idx + static_cast<int64_t>(t) * kIndexHeads * kIndexDim;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            qa[mt][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qt + (16 * mt + c) * kIndexDim + 32 * s + 8 * g));
    float wr[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) wr[mt][r] = bf16_to_f32(w[t * kIndexHeads + 16 * mt + 4 * g + r]);

    for (int j = 0; j < my_tiles; ++j) {
        // tile j landed once only the copies issued after it may be outstanding
        if (j + kDecodeRing - 1 < my_tiles) {
            issue(j + kDecodeRing - 1);
            wait_vmcnt<(kDecodeRing - 1) * kDecodeCopies>();
        } else {
            wait_vmcnt<0>();
        }
        const uint16_t* buf = ring[wave][j % kDecodeRing] + c * kIndexDim;
        u32x4 kf[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) kf[s] = *reinterpret_cast<const u32x4*>(buf + 8 * ((4 * s + g) ^ c));
        f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[0][s], as_bf16x8(kf[s]), a0, 0, 0, 0);
            a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[1][s], as_bf16x8(kf[s]), a1, 0, 0, 0);
        }
        float v = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) v += wr[0][r] * fmaxf(a0[r], 0.f) + wr[1][r] * fmaxf(a1[r], 0.f);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (g == 0) sbuf[(wave + 4 * j) * kDecodeTile + c] = v;
    }
    __syncthreads();
    float* srow = scores + static_cast<int64_t>(t) * ld + k0;
    for (int i = 4 * static_cast<int>(threadIdx.x); i < len; i += 4 * 256) {
        if (vec_store && i + 3 < len) {
            *reinterpret_cast<f32x4*>(srow + i) = *reinterpret_cast<const f32x4*>(sbuf + i);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (i + k < len) srow[i + k] = sbuf[i + k];
        }
    }
}

// ---------------------------------------------------------------------------------------
// prefill
// ---------------------------------------------------------------------------------------
constexpr int kPrefillQ = 16;        // queries per block (2 per wave, 8 waves)
constexpr int kPrefillTile = 32;     // keys per LDS tile
constexpr int kKeyStride = kIndexDim + 8;  // padded LDS row (bf16 elements): 272 bytes

// MFMA 32x32x16: A = q (rows: the 32 heads of one query), B = key tile (cols: 32 keys).
// Lane l (h = l/32) supplies head/key l%32 and dims [64h + 8s, 64h + 8s + 8) at step s.
// The accumulator gives lane l the key l%32 and the heads 8(r/4) + 4h + r%4, r = 0..15.
__global__ __launch_bounds__(512) void indexer_prefill_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ keys, const int64_t* __restrict__ kv_off,
    const int32_t* __restrict__ q_req, const int32_t* __restrict__ q_pos, int32_t T,
    int64_t max_s, float* __restrict__ scores, int64_t ld) {
    __shared__ __attribute__((aligned(16))) uint16_t ks[2][kPrefillTile * kKeyStride];
    __shared__ int64_t s_n[kPrefillQ];
    __shared__ int32_t s_req[kPrefillQ];

    const int t0 = blockIdx.x * kPrefillQ;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int col = lane & 31;

    if (tid < kPrefillQ) {
        const int t = t0 + tid;
        if (t < T) {
            s_req[tid] = q_req[t];
            s_n[tid] = admissible(kv_off, q_req[t], q_pos[t], max_s);
        } else {
            s_req[tid] = -1;
            s_n[tid] = 0;
        }
    }
    lds_barrier();

    // this wave's two queries
    const int qi0 = 2 * wave, qi1 = 2 * wave + 1;
    bf16x8 qa[2][8];
    float wr[2][16];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int t = t0 + 2 * wave + j;
        const int tt = t < T ? t : 0;
        const uint16_t* qt = q_idx + static_cast<int64_t>(tt) * kIndexHeads * kIndexDim;
#pragma unroll
        for (int s = 0; s < 8; ++s)
            qa[j][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qt + col * kIndexDim + 64 * h + 8 * s));
#pragma unroll
        for (int r = 0; r < 16; ++r)
            wr[j][r] = bf16_to_f32(w[tt * kIndexHeads + 8 * (r >> 2) + 4 * h + (r & 3)]);
    }

    // The queries of a block normally share one request.  If they do not, the block makes
    // one pass per distinct request, each pass scoring only that request's queries.
    int done_mask = 0;  // bit i: query i of the block handled (uniform across the block)
    for (int qi = 0; qi < kPrefillQ; ++qi)
        if (s_req[qi] < 0 || s_n[qi] == 0) done_mask |= 1 << qi;
    while (done_mask != (1 << kPrefillQ) - 1) {
        int req = -1;
        for (int qi = 0; qi < kPrefillQ; ++qi)
            if (!(done_mask & (1 << qi))) { req = s_req[qi]; break; }
        int64_t n_max = 0;
        int pass_mask = 0;
        for (int qi = 0; qi < kPrefillQ; ++qi)
            if (!(done_mask & (1 << qi)) && s_req[qi] == req) {
                pass_mask |= 1 << qi;
                n_max = s_n[qi] > n_max ? s_n[qi] : n_max;
            }
        const bool act0 = pass_mask & (1 << qi0), act1 = pass_mask & (1 << qi1);
        const int64_t n0 = act0 ? s_n[qi0] : 0, n1 = act1 ? s_n[qi1] : 0;
        const uint16_t* kb = keys + kv_off[req] * kIndexDim;
        const int n_tiles = static_cast<int>((n_max + kPrefillTile - 1) / kPrefillTile);

        // each thread moves one 16-byte chunk of a 32-key tile (32 keys x 16 chunks = 512)
        const int lrow = tid >> 4, lchunk = tid & 15;
        auto load_chunk = [&](int tile) -> u32x4 {
            int64_t key = static_cast<int64_t>(tile) * kPrefillTile + lrow;
            key = key < n_max ? key : n_max - 1;
            return *reinterpret_cast<const u32x4*>(kb + key * kIndexDim + 8 * lchunk);
        };
        u32x4 pre = load_chunk(0);
        *reinterpret_cast<u32x4*>(&ks[0][lrow * kKeyStride + 8 * lchunk]) = pre;
        if (n_tiles > 1) pre = load_chunk(1);
        lds_barrier();

        for (int tile = 0; tile < n_tiles; ++tile) {
            const uint16_t* kt = ks[tile & 1];
            const int64_t key0 = static_cast<int64_t>(tile) * kPrefillTile;
            f32x16 acc0 = {}, acc1 = {};
            if (key0 < n0 || key0 < n1) {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + col * kKeyStride + 64 * h + 8 * s));
                    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], kf, acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], kf, acc1, 0, 0, 0);
                }
            }
            // stage the next tile into the other buffer while the epilogue runs
            if (tile + 1 < n_tiles) {
                *reinterpret_cast<u32x4*>(&ks[(tile + 1) & 1][lrow * kKeyStride + 8 * lchunk]) = pre;
                if (tile + 2 < n_tiles) pre = load_chunk(tile + 2);
            }
            float v0 = 0.f, v1 = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                v0 += wr[0][r] * fmaxf(acc0[r], 0.f);
                v1 += wr[1][r] * fmaxf(acc1[r], 0.f);
            }
            v0 += __shfl_xor(v0, 32);
            v1 += __shfl_xor(v1, 32);
            const int64_t key = key0 + col;
            if (h == 0 && key < n0) scores[static_cast<int64_t>(t0 + qi0) * ld + key] = v0;
            if (h == 1 && key < n1) scores[static_cast<int64_t>(t0 + qi1) * ld + key] = v1;
            lds_barrier();
        }
        done_mask |= pass_mask;
    }
}

hipError_t launch_indexer_scores(const uint16_t* q_idx, const uint16_t* w, const uint16_t* keys,
                                 const int64_t* kv_off, const int32_t* q_req,
                                 const int32_t* q_pos, int32_t T, int32_t B, int64_t max_s,
                                 float* scores, int64_t ld, hipStream_t stream) {
    // Prefill kernel when queries come in runs of one request (on average >= 8 per
    // request); per-query streaming otherwise.  Both are exact for any layout.
    if (static_cast<int64_t>(T) >= 8 * static_cast<int64_t>(B)) {
        const int blocks = (T + kPrefillQ - 1) / kPrefillQ;
        hipLaunchKernelGGL(indexer_prefill_kernel, dim3(blocks), dim3(512), 0, stream, q_idx, w,
                           keys, kv_off, q_req, q_pos, T, max_s, scores, ld);
    } else {
        const int64_t chunk = decode_chunk(T, max_s);
        const int64_t cpq = (max_s + chunk - 1) / chunk;
        const int64_t blocks = cpq * T;
        if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        const bool vec = reinterpret_cast<uintptr_t>(scores) % 16 == 0 && ld % 4 == 0;
        hipLaunchKernelGGL(indexer_decode_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256),
                           0, stream, q_idx, w, keys, kv_off, q_req, q_pos,
                           static_cast<int32_t>(cpq), static_cast<int32_t>(chunk), max_s, scores,
                           ld, vec ? 1 : 0);
    }
    return hipGetLastError();
}

}  // namespace dsa
