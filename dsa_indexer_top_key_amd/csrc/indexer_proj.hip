// Before stages 1 and 2: the indexer-side projections of T new tokens, fused with the key
// LayerNorm and the append of the keys to the index-key cache.
//
// Page "Kimi K3.1 Pro: Sparse-Zugriffe, keine kleinere Historie", section "Eine Query durch
// den Indexer verfolgen": the indexer projects the query latent to [T,32,128]; another
// projection maps residual states to [S,128] keys, followed by LayerNorm; a further one makes
// 32 head weights from the residual state of each query.  Section "Was ändert sich – und was
// nicht?": query latent rank 1536, residual width 7168.  The adapter paragraph: FP32 key
// normalisation, BF16 head-gate path.
//
//   q_idx[t] = W_qi c_q[t]            [4096] -> [32,128] bf16   (W_qi [4096,1536])
//   key[t]   = LN(W_k h[t]) -> bf16, written to cache row key_rows[t]   (W_k [128,7168])
//   w[t]     = W_w h[t]               [32] bf16                 (W_w [32,7168])
//
// Two products X W^T with bf16 operands and fp32 sums on the matrix cores
// (v_mfma_f32_32x32x16_bf16): the query product (K = 1536, N = 4096) and the residual
// product (K = 7168, N = 160: the key's 128 columns followed by the 32 head weights), both by
// proj_gemm_lds_kernel (128 x 128 block tiles staged through LDS by whole-line global->LDS
// copies).  The K range is split so that small T (decode: one token per request) still
// spreads the weight stream over hundreds of blocks; each split writes fp32 partial sums, and
// one epilogue block per token adds the splits in a fixed order (deterministic), rounds q_idx
// and w to bf16, and normalises the key in fp32 (mean, biased variance, rsqrt(var + eps),
// gamma, beta) before rounding it into the cache.  An unsplit query product (large T) rounds
// its sums to bf16 q_idx in the product kernel itself (no fp32 round trip).  256 x 256 tiles
// for the query product of 4096 tokens (one wave per SIMD, 16 accumulators each, a four-slot
// ring of 32-wide K chunks) took 83 us against about 90 us for its share of the combined
// launch, but the residual product then ran alone in 41 us: 130 us in all against 121.  A
// register-direct variant (each wave loading its operands in MFMA layout, 64 lanes over 64
// cache lines per load) measured 3.8x slower at 4096 tokens (480 vs 126 us per call) and 15%
// slower at 64 (35 vs 30 us).
//
// Roofline: decode (T = 64) streams 15 MB of weights once -- HBM-bound; a prefill chunk
// (T = 4096) is 61 GFLOP of contraction -- bound by the matrix cores.
#include "common.h"

namespace dsa {

constexpr int kQLatent = 1536;
constexpr int kResidual = 7168;
constexpr int kQOut = kIndexHeads * kIndexDim;   // 4096 query outputs
constexpr int kKWOut = kIndexDim + kIndexHeads;  // 160: key columns, then head-weight columns
constexpr int kLdsTile = 128;                    // block tile: rows of A and of the weight
constexpr int kLdsChunk = 64;                    // K per chunk: 4 MFMA steps
constexpr int kProjTargetBlocks = 256;           // split K until about this many blocks
constexpr int kProjMaxSplits = 32;               // ... with at most this many partial sums

struct ProjSplits {
    int q_splits, q_cps;    // query product: splits, chunks per split
    int kw_splits, kw_cps;  // residual product
    int ring;               // LDS ring slots of the product kernel (2 or 4)
};

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

static void split_k(int blocks_mn, int chunks, int* splits, int* cps) {
    int s = ceil_div(kProjTargetBlocks, blocks_mn);
    s = s < 1 ? 1 : (s > chunks ? chunks : s);
    s = s < kProjMaxSplits ? s : kProjMaxSplits;
    *cps = ceil_div(chunks, s);
    *splits = ceil_div(chunks, *cps);
}

// Up to 128 tokens (one row tile) the products run on a four-slot ring, one block per CU, with
// K split into runs of at most four chunks, so that all of a block's chunks are in flight at
// once: 6 + 28 splits, 192 + 56 = 248 blocks.  (Through the two-slot ring, one chunk ahead,
// each of a block's three or four chunks cost a round trip to memory.)
constexpr int kSmallRing = 4;
static ProjSplits proj_splits(int32_t T) {
    ProjSplits p;
    const int mt = ceil_div(T, kLdsTile);
    if (mt == 1) {
        p.ring = kSmallRing;
        p.q_cps = p.kw_cps = kSmallRing;
        p.q_splits = ceil_div(kQLatent / kLdsChunk, kSmallRing);
        p.kw_splits = ceil_div(kResidual / kLdsChunk, kSmallRing);
        return p;
    }
    p.ring = 2;
    split_k(mt * ceil_div(kQOut, kLdsTile), kQLatent / kLdsChunk, &p.q_splits, &p.q_cps);
    split_k(mt * ceil_div(kKWOut, kLdsTile), kResidual / kLdsChunk, &p.kw_splits, &p.kw_cps);
    return p;
}

// fp32 partial sums of the query product (none when it is unsplit: its blocks round their sums
// to bf16 q_idx themselves).
static size_t q_partial_bytes(const ProjSplits& p, int32_t T) {
    return p.q_splits > 1 ? static_cast<size_t>(p.q_splits) * T * kQOut * sizeof(float) : 0;
}

size_t proj_workspace_bytes(int32_t T) {
    if (T <= 0) return 0;
    const ProjSplits p = proj_splits(T);
    const size_t q = q_partial_bytes(p, T);
    const size_t kw = static_cast<size_t>(p.kw_splits) * T * kKWOut * sizeof(float);
    return ((q + 255) & ~static_cast<size_t>(255)) + kw;
}

// part[split][m][n] = sum over the split's K chunks of sum_k a[m][k] * b(n)[k], where rows
// n < n_b0 of the weight come from b0 and the others from b1 (row n - n_b0).  A 128 x 128
// block tile: its A rows and weight rows stream through LDS, shared by the block's four waves
// (2 x 2, each a 64 x 64 tile of four accumulators), so every operand byte is read from L2
// once per block.
// K moves in 64-wide chunks (four MFMA steps, 128 bytes per row) through a ring of RING slots
// filled by direct global->LDS copies RING - 1 chunks ahead; one barrier per chunk.  Beyond
// 128 tokens the ring has two slots (64 KB), so two blocks share a CU and each covers the
// other's copy latency and barriers (a three-slot ring, one block per CU, measured 5% slower
// at 4096 tokens and 18% at 64 with the older split of K).  Up to 128 tokens it has four
// (128 KB, one block per CU) and every split has at most four chunks (see proj_splits).  Row r of a
// slot occupies 128 bytes; its 16-byte piece p sits at position p ^ ((r / 2) % 8), so the 16
// rows an operand read touches (same p) fall in 16 distinct 16-byte bank groups.  Copy d of a
// chunk moves rows 8d..8d+7 (A rows for d < 16, weight rows for d >= 16): lane 8 rr + c loads
// piece c ^ ((row / 2) % 8) of row 8d + rr into position c.  At step s lane l supplies
// row l % 32 and the dims [32 (l / 32) + 8 s, +8) of the chunk, for both operands.
constexpr int kLdsSlot = 2 * kLdsTile * kLdsChunk;  // bf16 elements per slot (A then weight)
constexpr int kLdsCopies = 2 * kLdsTile / 8 / 4;  // 1 KB copies per wave per chunk: 8

struct ProjProduct {
    const uint16_t* a;   // [M, K]
    const uint16_t* b0;  // weight rows 0 .. n_b0-1, [n_b0, K]
    const uint16_t* b1;  // weight rows n_b0 .. N-1, [N - n_b0, K]
    int n_b0, N, K, cps;
    int col_tiles, row_tiles, blocks;  // blocks = col_tiles * row_tiles * splits
    float* part;         // [splits, M, N]
    uint16_t* out_bf16;  // unsplit product with N a multiple of 128: [M, N] bf16 written here
                         // (rounded to nearest even) instead of part
};

// Both products run in one launch: blocks [0, p0.blocks) take the first product, the rest the
// second (their latencies overlap; one launch instead of two).  Within a product,
// block index = (split * row_tiles + row tile) * col_tiles + column tile.
// This wave's copies of chunk i are done once only those of the chunks issued after it (at
// most RING - 2) remain outstanding.
template <int RING>
__device__ __forceinline__ void wait_chunk(int after) {
    if constexpr (RING >= 4)
        if (after >= 2) { wait_vmcnt<2 * kLdsCopies>(); return; }
    if constexpr (RING >= 3)
        if (after >= 1) { wait_vmcnt<kLdsCopies>(); return; }
    wait_vmcnt<0>();
}

template <int RING>
__global__ __launch_bounds__(256) void proj_gemm_lds_kernel(ProjProduct p0, ProjProduct p1,
                                                            int M) {
    __shared__ __attribute__((aligned(1024))) uint16_t ring[RING][kLdsSlot];
    const bool first = static_cast<int>(blockIdx.x) < p0.blocks;  // block-uniform
    const ProjProduct& pr = first ? p0 : p1;
    const int bid = first ? static_cast<int>(blockIdx.x) : static_cast<int>(blockIdx.x) - p0.blocks;
    const uint16_t* __restrict__ a = pr.a;
    const uint16_t* __restrict__ b0 = pr.b0;
    const uint16_t* __restrict__ b1 = pr.b1;
    const int n_b0 = pr.n_b0, N = pr.N, K = pr.K, cps = pr.cps;
    float* __restrict__ part = pr.part;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave >> 1, wc = wave & 1;
    const int ct = bid % pr.col_tiles;
    const int rt = (bid / pr.col_tiles) % pr.row_tiles;
    const int split = bid / (pr.col_tiles * pr.row_tiles);
    const int m0 = kLdsTile * rt;
    const int n0 = kLdsTile * ct;
    const int col = lane & 31, hh = lane >> 5;
    const int chunks = K / kLdsChunk;
    const int c_begin = split * cps;
    int c_end = c_begin + cps;
    c_end = c_end < chunks ? c_end : chunks;
    const int n_chunks = c_end - c_begin;

    // this wave's copies: rows 8d + rr of A (d < 16) or of the weight (d >= 16); rows past
    // M or N read the last row (in bounds), their results are never stored
    const int rr = lane >> 3, cpos = lane & 7;
    const uint16_t* src[kLdsCopies];
    uint32_t dst[kLdsCopies];
#pragma unroll
    for (int j = 0; j < kLdsCopies; ++j) {
        const int d = kLdsCopies * wave + j;
        const int r = 8 * (d & 15) + rr;
        const int piece = cpos ^ ((r >> 1) & 7);
        if (d < 16) {
            const int m = m0 + r < M ? m0 + r : M - 1;
            src[j] = a + static_cast<int64_t>(m) * K + 8 * piece;
        } else {
            const int n = n0 + r < N ? n0 + r : N - 1;
            src[j] = (n < n_b0 ? b0 + static_cast<int64_t>(n) * K
                               : b1 + static_cast<int64_t>(n - n_b0) * K) + 8 * piece;
        }
        dst[j] = static_cast<uint32_t>((d >= 16 ? kLdsTile * kLdsChunk : 0) + 8 * (d & 15) * kLdsChunk) * 2;
    }
    auto issue = [&](int i) {  // copies of the split's chunk i into slot i % RING
        const int c = c_begin + i;
        const uint32_t base = lds_offset(ring[i % RING]);
#pragma unroll
        for (int j = 0; j < kLdsCopies; ++j) {
            // one row tile (RING 4): every weight row is read by this block only, so its
            // copies carry the non-temporal hint (64 tokens, cold: 23.4 -> 21.5 us per call)
            if (RING == 4 && kLdsCopies * wave + j >= 16)
                copy_to_lds<true>(src[j] + static_cast<int64_t>(c) * kLdsChunk, base + dst[j]);
            else
                copy_to_lds(src[j] + static_cast<int64_t>(c) * kLdsChunk, base + dst[j]);
        }
    };

    f32x16 acc[2][2] = {};
    // RING - 1 chunks ahead (all of them when the split has no more); a chunk past the split's
    // end is never issued
    const int ahead = n_chunks < RING - 1 ? n_chunks : RING - 1;  // block-uniform
    for (int j = 0; j < ahead; ++j) issue(j);
    for (int i = 0; i < n_chunks; ++i) {
        // the barrier covers every wave's copies of chunk i and frees slot
        // (i + RING - 1) % RING, chunk i - 1's
        wait_chunk<RING>(n_chunks - 1 - i < RING - 2 ? n_chunks - 1 - i : RING - 2);
        lds_barrier();
        if (i + RING - 1 < n_chunks) issue(i + RING - 1);
        const uint16_t* sa = ring[i % RING];
        const uint16_t* sb = sa + kLdsTile * kLdsChunk;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int ra = 64 * wr + 32 * t + col;
                const int rb = 64 * wc + 32 * t + col;
                const int p = 4 * hh + s;
                fa[t] = as_bf16x8(*reinterpret_cast<const u32x4*>(sa + ra * kLdsChunk + 8 * (p ^ ((ra >> 1) & 7))));
                fb[t] = as_bf16x8(*reinterpret_cast<const u32x4*>(sb + rb * kLdsChunk + 8 * (p ^ ((rb >> 1) & 7))));
            }
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int y = 0; y < 2; ++y)
                    acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[x], fb[y], acc[x][y], 0, 0, 0);
        }
    }
    // no copy may still be writing LDS when the block ends
    wait_vmcnt<0>();

    if (pr.out_bf16) {  // block-uniform
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) {
                float v[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) v[r] = acc[x][y][r];
                store_tile_bf16(pr.out_bf16, N, m0 + 64 * wr + 32 * x, n0 + 64 * wc + 32 * y, v,
                                lane, M);
            }
        return;
    }
    float* out = part + static_cast<int64_t>(split) * M * N;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
            const int n = n0 + 64 * wc + 32 * y + col;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + 64 * wr + 32 * x + 8 * (r >> 2) + 4 * hh + (r & 3);
                if (m < M && n < N) out[static_cast<int64_t>(m) * N + n] = acc[x][y][r];
            }
        }
}

// `parts` blocks (256 threads) per token t: block part j adds the splits of query columns
// [j 4096 / parts, (j + 1) 4096 / parts) (two adjacent ones per thread and step) and rounds
// them; part 0's first wave also finishes the key (two columns per lane, LayerNorm over the
// wave) and the last part's the 32 head weights.  Splits are added in ascending order.  Small
// T spreads a token over 8 blocks (T = 64: 64 blocks would leave most CUs idle), large T
// takes one block per token.
static int epilogue_parts(int32_t T) { return T < 1024 ? 8 : 1; }

__global__ __launch_bounds__(256) void proj_epilogue_kernel(
    const float* __restrict__ pq, int q_splits, const float* __restrict__ pkw, int kw_splits,
    int32_t T, const float* __restrict__ gamma, const float* __restrict__ beta, float eps,
    uint16_t* __restrict__ q_idx, uint16_t* __restrict__ w, uint16_t* __restrict__ keys,
    const int64_t* __restrict__ key_rows, int parts) {
    const int t = static_cast<int>(blockIdx.x) / parts;
    const int j = static_cast<int>(blockIdx.x) - t * parts;
    const int tid = threadIdx.x;
    const int64_t q_stride = static_cast<int64_t>(T) * kQOut;
    const int c_end = q_splits > 0 ? (j + 1) * (kQOut / parts) : 0;  // 0 splits: q_idx is done
    for (int n = j * (kQOut / parts) + 2 * tid; n < c_end; n += 512) {
        const float* p = pq + static_cast<int64_t>(t) * kQOut + n;
        f32x2 v = *reinterpret_cast<const f32x2*>(p);
        // unrolled so that the loads of several splits are in flight at once; the sums still
        // go in ascending split order
#pragma unroll 8
        for (int s = 1; s < q_splits; ++s) {
            const f32x2 u = *reinterpret_cast<const f32x2*>(p + s * q_stride);
            v[0] += u[0];
            v[1] += u[1];
        }
        *reinterpret_cast<uint32_t*>(q_idx + static_cast<int64_t>(t) * kQOut + n) = pack_bf16x2(v[0], v[1]);
    }
    const int wave = tid >> 6, lane = lane_id();
    const int64_t kw_stride = static_cast<int64_t>(T) * kKWOut;
    const float* pk = pkw + static_cast<int64_t>(t) * kKWOut;
    if (j == 0 && wave == 0) {
        float x0 = pk[2 * lane], x1 = pk[2 * lane + 1];
#pragma unroll 8
        for (int s = 1; s < kw_splits; ++s) {
            x0 += pk[s * kw_stride + 2 * lane];
            x1 += pk[s * kw_stride + 2 * lane + 1];
        }
        constexpr float inv_d = 1.0f / kIndexDim;
        float sum = x0 + x1;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m);
        const float mean = sum * inv_d;
        const float d0 = x0 - mean, d1 = x1 - mean;
        float sq = d0 * d0 + d1 * d1;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) sq += __shfl_xor(sq, m);
        const float r = 1.0f / sqrtf(sq * inv_d + eps);
        const float y0 = d0 * r * gamma[2 * lane] + beta[2 * lane];
        const float y1 = d1 * r * gamma[2 * lane + 1] + beta[2 * lane + 1];
        *reinterpret_cast<uint32_t*>(keys + key_rows[t] * kIndexDim + 2 * lane) = pack_bf16x2(y0, y1);
    }
    if (j == parts - 1 && wave == 1 && lane < kIndexHeads) {
        float v = pk[kIndexDim + lane];
#pragma unroll 8
        for (int s = 1; s < kw_splits; ++s) v += pk[s * kw_stride + kIndexDim + lane];
        w[static_cast<int64_t>(t) * kIndexHeads + lane] = f32_to_bf16(v);
    }
}

hipError_t launch_indexer_proj(const uint16_t* c_q, const uint16_t* h, const uint16_t* w_qi,
                               const uint16_t* w_k, const uint16_t* w_w, const float* gamma,
                               const float* beta, float eps, int32_t T, uint16_t* q_idx,
                               uint16_t* w, uint16_t* keys, const int64_t* key_rows,
                               void* workspace, hipStream_t stream) {
    const ProjSplits p = proj_splits(T);
    const size_t q_bytes = q_partial_bytes(p, T);
    float* pq = static_cast<float*>(workspace);
    float* pkw = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          ((q_bytes + 255) & ~static_cast<size_t>(255)));
    const int mt = ceil_div(T, kLdsTile);
    ProjProduct q{c_q, w_qi, w_qi, kQOut, kQOut, kQLatent, p.q_cps, ceil_div(kQOut, kLdsTile), mt, 0, pq};
    q.blocks = q.col_tiles * mt * p.q_splits;
    if (p.q_splits == 1) q.out_bf16 = q_idx;  // (N = 4096: whole column tiles)
    ProjProduct kw{h, w_k, w_w, kIndexDim, kKWOut, kResidual, p.kw_cps, ceil_div(kKWOut, kLdsTile), mt, 0, pkw};
    kw.blocks = kw.col_tiles * mt * p.kw_splits;
    // the residual product's blocks (K = 7168) are the longest: dispatched first
    if (p.ring == kSmallRing)
        hipLaunchKernelGGL(proj_gemm_lds_kernel<kSmallRing>, dim3(q.blocks + kw.blocks), dim3(256), 0,
                           stream, kw, q, T);
    else
        hipLaunchKernelGGL(proj_gemm_lds_kernel<2>, dim3(q.blocks + kw.blocks), dim3(256), 0,
                           stream, kw, q, T);
    const int parts = epilogue_parts(T);
    hipLaunchKernelGGL(proj_epilogue_kernel, dim3(T * parts), dim3(256), 0, stream, pq,
                       p.q_splits > 1 ? p.q_splits : 0, pkw, p.kw_splits, T, gamma, beta, eps,
                       q_idx, w, keys, key_rows,
                       parts);
    return hipGetLastError();
}

}  // namespace dsa
