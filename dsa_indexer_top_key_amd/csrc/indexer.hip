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
//  * prefill -- many queries of one request (indexer_prefill.hip): every key tile feeds
//    16 queries x 32 heads of v_mfma_f32_32x32x16_bf16, so that kernel is bound by MFMA
//    throughput rather than HBM.
#include "common.h"

namespace dsa {

// ---------------------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------------------
constexpr int kDecodeTile = 16;          // keys per wave step: 4 KB, four 1 KB copies
constexpr int kDecodeRing = 3;           // ring slots per wave (two steps in flight)
constexpr int kDecodeCopies = kDecodeTile / 4;
constexpr int kDecodeMaxChunk = 4096;    // keys per block at most (their scores: 16 KB of LDS)
constexpr int kDecodeMinChunk = 64;      // one block step

// Keys per block: the whole job spread over about two blocks per CU (64 KB of LDS each, so
// two fit; all blocks then end at about the same time and the score writes leave as one
// burst), within [64, 4096] keys and a multiple of one block step (64 keys).  With one
// block (four waves) per CU the MFMA and reduction latency of each tile is no longer hidden
// (8192-key blocks measured 60% slower).  Small jobs keep the spread too: 4 queries of 4096
// positions run 256 blocks of 64 keys (with at least 1024 keys per block they ran 16 blocks,
// and the indexer + top-k took 20.7 instead of 15.6 us).
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
// PAGED: the keys live in a page pool; logical position p of request b is pool row
// page_table[b * max_pages + (p >> lg_page)] * 2^lg_page + p % 2^lg_page (kv_off then only gives
// the request lengths).  Pages hold at least 64 positions, so a block's chunk (a multiple of 64,
// at most 4096 keys) spans at most 64 pages: lane i holds the physical page of the chunk's i-th
// page, and each 16-key tile, which lies in one page, reads it with a wave-uniform readlane.
template <bool PAGED>
__global__ __launch_bounds__(256) void indexer_decode_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ keys, const int64_t* __restrict__ kv_off,
    const int32_t* __restrict__ q_req, const int32_t* __restrict__ q_pos, int32_t B,
    int32_t chunks_per_q, int32_t chunk, int64_t max_s, float* __restrict__ scores, int64_t ld,
    int vec_store,
    const int32_t* __restrict__ page_table, int lg_page, int max_pages) {
    __shared__ __attribute__((aligned(16))) uint16_t ring[4][kDecodeRing][kDecodeTile * kIndexDim];
    __shared__ __attribute__((aligned(16))) float sbuf[kDecodeMaxChunk];
    const int t = blockIdx.x / chunks_per_q;
    const int ci = blockIdx.x - t * chunks_per_q;
    const int b = query_request(q_req, t, B);
    const int64_t n = admissible_count(kv_off, b, q_pos[t], max_s);
    const int64_t k0 = static_cast<int64_t>(ci) * chunk;
    if (k0 >= n) return;  // block-uniform
    const int len = static_cast<int>((k0 + chunk < n ? k0 + chunk : n) - k0);

    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int c = lane & 15;
    const uint16_t* kb = PAGED ? keys : keys + (kv_off[b] + k0) * kIndexDim;
    const int n_tiles = (len + kDecodeTile - 1) / kDecodeTile;
    const int my_tiles = n_tiles > wave ? (n_tiles - wave + 3) / 4 : 0;
    int pte = 0;  // PAGED: physical page of the chunk's page `lane`
    if constexpr (PAGED) {
        const int64_t lp = (k0 >> lg_page) + lane;
        const int64_t np = (k0 + len + (int64_t{1} << lg_page) - 1) >> lg_page;
        // entries past the table's row (S_b > max_pages * page_size breaks the contract) are
        // never read: such positions score page 0
        pte = lp < np && lp < max_pages ? page_table[static_cast<int64_t>(b) * max_pages + lp] : 0;
    }
    // copies of this wave's j-th tile into ring slot j % 3; keys past the end copy key 0 (the
    // tile's first key when paged, which keeps the whole tile in one page)
    auto issue = [&](int j) {
        const int kt = (wave + 4 * j) * kDecodeTile;
        const uint16_t* slot = ring[wave][j % kDecodeRing];
        const uint16_t* tb = kb;
        if constexpr (PAGED) {
            const int rel = static_cast<int>(((k0 + kt) >> lg_page) - (k0 >> lg_page));
            const int64_t page = __builtin_amdgcn_readlane(pte, rel);
            tb = keys + ((page << lg_page) + ((k0 + kt) & ((int64_t{1} << lg_page) - 1)) - kt) * kIndexDim;
        }
#pragma unroll
        for (int d = 0; d < kDecodeCopies; ++d) {
            const int r = 4 * d + g;
            const int key = kt + r < len ? kt + r : (PAGED ? kt : 0);
            copy_to_lds<true>(tb + static_cast<int64_t>(key) * kIndexDim + 8 * (c ^ r),
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

    // Head-weighted ReLU sum of a tile's 32 x 16 products, the four 16-lane rows reduced by
    // the cross-row swaps (v_permlane16_swap, then v_permlane32_swap: lane l adds lane l ^ 16,
    // then l ^ 32, on the VALU); row 0 holds key c's score.
    auto epilogue = [&](const f32x4& a0, const f32x4& a1, int jj) {
        float v = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) v += wr[0][r] * fmaxf(a0[r], 0.f) + wr[1][r] * fmaxf(a1[r], 0.f);
        const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                          false, false);
        v = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
        const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                          false, false);
        v = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
        if (g == 0) sbuf[(wave + 4 * jj) * kDecodeTile + c] = v;
    };
    // A tile's epilogue runs after the next tile's MFMAs are issued, so it overlaps them.
    f32x4 pa0 = {0.f, 0.f, 0.f, 0.f}, pa1 = {0.f, 0.f, 0.f, 0.f};
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
        if (j > 0) epilogue(pa0, pa1, j - 1);
        pa0 = a0;
        pa1 = a1;
    }
    if (my_tiles > 0) epilogue(pa0, pa1, my_tiles - 1);
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

hipError_t launch_indexer_prefill(const uint16_t* q_idx, const uint16_t* w, const uint16_t* keys,
                                  const int64_t* kv_off, const int32_t* q_req,
                                  const int32_t* q_pos, int32_t T, int32_t B, int64_t max_s,
                                  float* scores, int64_t ld, hipStream_t stream);

hipError_t launch_indexer_scores(const uint16_t* q_idx, const uint16_t* w, const uint16_t* keys,
                                 const int64_t* kv_off, const int32_t* q_req,
                                 const int32_t* q_pos, int32_t T, int32_t B, int64_t max_s,
                                 float* scores, int64_t ld, hipStream_t stream,
                                 const int32_t* page_table, int lg_page, int max_pages) {
    // Prefill kernel when queries come in runs of one request (on average >= 8 per
    // request); per-query streaming otherwise (always for a paged cache).  Both are exact for
    // any layout.
    if (!page_table && static_cast<int64_t>(T) >= 8 * static_cast<int64_t>(B)) {
        return launch_indexer_prefill(q_idx, w, keys, kv_off, q_req, q_pos, T, B, max_s, scores,
                                      ld, stream);
    } else {
        const int64_t chunk = decode_chunk(T, max_s);
        const int64_t cpq = (max_s + chunk - 1) / chunk;
        const int64_t blocks = cpq * T;
        if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        const bool vec = reinterpret_cast<uintptr_t>(scores) % 16 == 0 && ld % 4 == 0;
        if (page_table)
            hipLaunchKernelGGL(indexer_decode_kernel<true>, dim3(static_cast<unsigned>(blocks)),
                               dim3(256), 0, stream, q_idx, w, keys, kv_off, q_req, q_pos, B,
                               static_cast<int32_t>(cpq), static_cast<int32_t>(chunk), max_s,
                               scores, ld, vec ? 1 : 0, page_table, lg_page, max_pages);
        else
            hipLaunchKernelGGL(indexer_decode_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                               dim3(256), 0, stream, q_idx, w, keys, kv_off, q_req, q_pos, B,
                               static_cast<int32_t>(cpq), static_cast<int32_t>(chunk), max_s,
                               scores, ld, vec ? 1 : 0, nullptr, 0, 0);
    }
    return hipGetLastError();
}

}  // namespace dsa
