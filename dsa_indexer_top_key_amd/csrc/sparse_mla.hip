// Stage 4: absorbed-MLA read restricted to the selected positions I_t.
//
// Page "Kimi K3.1 Pro: Sparse-Zugriffe, keine kleinere Historie", section "Die Mathematik
// der Sparse Attention und ihrer fehlenden Masse": for each main-attention head the read is
// a softmax over the logits a_tj restricted to j in I_t; the notation abstracts absorbed
// MLA projections (per-head K/V are never materialised).  Section "Warum Top-2048 ..." (last
// paragraphs) and the Gated-MLA paragraph: all 96 heads share one 512-wide latent, with a
// 64-wide companion key component beside it and no rotation (skip_rope).
//
//   a_thj = scale * q_th . [c_j ; kpe_j]     (576 dims)
//   o_th  = sum_j softmax_j(a_thj) c_j        (512 dims, j in I_t)
//
// Work per query: 2048 gathered rows of 1152 B, 96 x 2048 x (576 + 512) MACs.
//
// Block = 4 waves for one (query, split of the ID row).  Waves 0..2 each own 32 heads:
// their 32 x 576 absorbed queries live in registers for the whole block, as the B operand
// of  S^T = C . Q^T  (v_mfma_f32_32x32x16_bf16, M = 32 gathered rows, N = 32 heads), which
// leaves each lane with one head and 16 rows -- exactly the A-operand layout the P . V
// product needs, so probabilities never leave registers.  The 32 x 352 output of a head
// group (11 of the 16 latent tiles) accumulates in its registers across the split.  The selected rows stream into a
// three-deep LDS ring: at the start of a step every wave loads its eight latent rows (1 KB
// each, wave-uniform address) of the tile two ahead into registers, and wave 3 also the four
// blocks of eight companion rows; they are written into the tile's slot at the end of the
// step, before the barrier that publishes it.  Wave 3 computes the last 160 latent columns of
// all 96 heads from P fragments the head groups publish in LDS.  The V operand of P . V (rows
// x latent dims) is read from the row-major LDS tile with the transposing load
// ds_read_b64_tr_b16.
//
// Softmax (fp32, log2 domain) uses a fixed per-head reference: the maximum logit of the
// first tile.  Later probabilities p = 2^(x - ref) may exceed 1; that is exact after the
// final division by the sum, and fp32/bf16 keep full relative precision while p <= 2^32.
// If any logit exceeds its reference by more than 32 (never for sane data), the split is
// recomputed once with the exact per-head maximum recorded during the first pass, so no
// accumulator is ever rescaled in the hot loop (which would not fit the register budget:
// the 32 x 352 accumulators of a head group already fill most of its registers).
// Splits write normalised partials (in the output's precision: bf16 or fp32) and a
// log2-sum-exp; a small kernel over all CUs merges them (merging inside the last split of
// each query measured slower: the agent-scope release/acquire and a merge on only one CU per
// query cost more than the extra launch).  A block maps to an XCD chosen by its query, so all
// splits of a query share one L2.
#include "common.h"

namespace dsa {

constexpr int kTile = 32;                    // gathered rows per step
constexpr int kNBuf = 3;                     // LDS ring depth
constexpr int kLatStride = kLatent + 24;     // latent row in LDS: 1024 B + 48 B pad
constexpr int kNTiles = kLatent / 32;        // 16 output tiles of 32 latent dims
constexpr int kHelpTiles = 5;                // computed by wave 3 for all heads
constexpr int kConsTiles = kNTiles - kHelpTiles;  // kept by the head-group waves (11)
constexpr int kKSteps = kQK / 16;            // 36 MFMA K-steps over the 576 dims
// K order of the 576-dim dot (any order works as long as q and the rows agree): at K-step
// s < 32 lane half hh holds latent dims 256 hh + 8s .. +8; at s >= 32 it holds companion
// dims 32 hh + 8 (s - 32) .. +8, so both halves reach the companion block together.
constexpr int kLatSteps = kLatent / 16;      // 32
constexpr int kQfInAcc = 12;                 // q fragments kept in accumulation registers
constexpr int kPrefA = 4;                    // LDS prefetch depth of S^T A fragments
constexpr int kPrefV = 4;                    // LDS prefetch depth of P.V B fragments
constexpr float kLn2 = 0.69314718055994531f;

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

typedef __attribute__((address_space(3))) const uint16_t lds_u16;

// The transposing read takes an LDS-address-space pointer: offsets added there fold into the
// instruction's immediate (a generic pointer cast per read costs a VALU add and a VGPR each).
__device__ __forceinline__ bf16x4 lds_read_tr16(lds_u16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// Output staging (bf16 output): row h of the [96][512] result at stage + h * kStageLd, so the
// four rows one paired store instruction writes (R, R + 1, R + 4, R + 5) fall at 64-byte bank
// offsets 0, 64, 0, 64 (two-way at most); the block then leaves it in full 1 KB rows.
constexpr int kStageLd = kLatent + 32;

// One ring slot: 32 latent rows (1072-byte stride: the rows read by one A-operand fetch, and
// the four rows behind each 16-lane group of a transposing V read, fall in distinct banks)
// and 32 companion rows of 128 B whose 16-byte chunks are XOR-swizzled by (row % 8) for the
// same reason.
struct MlaSmem {
    union {
        struct {  // the ring
            uint16_t lat[kNBuf][kTile * kLatStride];
            uint16_t kpe[kNBuf][kTile * kCompanion];
        };
        uint16_t stage[kMlaHeads * kStageLd];  // after the last step: the block's bf16 result
    };
    int32_t rows[kTopK];                     // the split's IDs, padding replaced by ID 0
    uint32_t tmask[kTopK / kTile];           // per tile: bit r set if row r holds a real ID
    u32x4 pfrag[2][3][64][2];                // P (bf16) in A-operand layout, per head group,
                                             // double-buffered by tile parity
    float inv_l[kMlaHeads];                  // per-head 1/l at the end
    uint32_t wend[4];                        // per wave: 1 + index of its last real ID
    uint32_t redo;                           // some logit exceeded its reference by > 2^32
};
static_assert(kMlaHeads * kStageLd <= kNBuf * kTile * (kLatStride + kCompanion),
              "the output stage fits in the ring");

// Paired bf16 store of one 32 x 32 accumulator tile into the LDS stage (the layout of
// store_tile_bf16, with LDS row stride kStageLd).  Lane 2j holds column c and lane 2j + 1
// column c + 1, each for rows R and R + 1 (v[r], v[r + 1]); one DPP swap gives the even lane
// row R of both columns and the odd lane row R + 1.  Everything is selects and one hardware
// conversion (v_cvt_pk_bf16_f32, round to nearest even): no branches.
__device__ __forceinline__ void stage_tile_bf16(uint16_t* stage, int row0, int col0,
                                                const float (&v)[16], int lane) {
    const bool odd = lane & 1;
    const int hh = (lane >> 5) & 1;
    uint16_t* base = stage + (row0 + 4 * hh + (odd ? 1 : 0)) * kStageLd + col0 + (lane & 30);
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
        const float send = odd ? v[r] : v[r + 1];
        const float recv = __uint_as_float(dpp_u32<kDppQuadXor1>(0u, __float_as_uint(send)));
        const float lo = odd ? recv : v[r];
        const float hi = odd ? v[r + 1] : recv;
        const bf16x2 pk = __builtin_convertvector((f32x2{lo, hi}), bf16x2);
        const int row = 8 * (r >> 2) + (r & 3);
        *reinterpret_cast<bf16x2*>(base + row * kStageLd) = pk;
    }
}

// The staged [96][512] bf16 result to global memory (dst: 96 contiguous rows of 512): every
// thread moves 16-byte pieces, a wave one whole 1 KB row per instruction.
__device__ __forceinline__ void stage_out(const uint16_t* stage, uint16_t* dst, int tid) {
#pragma unroll 4
    for (int c = tid; c < kMlaHeads * (kLatent / 8); c += 256) {
        const int row = c >> 6, piece = c & 63;
        *reinterpret_cast<u32x4*>(dst + row * kLatent + 8 * piece) =
            *reinterpret_cast<const u32x4*>(stage + row * kStageLd + 8 * piece);
    }
}

// Ring fill of one tile (32 rows; padding rows load row 0 of the request, so every slot holds
// finite data).  Every wave loads eight latent rows (rows 8 wave .. 8 wave + 7; lane l holds 16
// bytes at offset 16 l of each 1 KB row) into registers at the start of a step and writes them
// into the slot at its end; wave 3 also loads the four blocks of eight companion rows.  Loads
// into registers, not direct global->LDS copies: on these random 1 KB rows a gather-only probe
// moved 2.45 TB/s from HBM with plain register loads and 1.8 TB/s with the copies (5.2 and
// 3.1 TB/s from the Infinity Cache); with the non-temporal hint the register loads move
// 5.1 TB/s from HBM (missed rows are then not installed in the Infinity Cache).
constexpr int kConsRows = kTile / 4;  // latent rows per wave (8)

struct TileRegs {
    u32x4 lat[kConsRows];   // this wave's latent rows
    u32x4 kp[kTile / 8];    // wave 3: companion block kb, lane -> row 8 kb + lane / 8
};

// The per-step base of the transposing V reads, made opaque to the compiler.  Left visible,
// the compiler splits base + constant into a loop-invariant register per read and re-adds
// it with a VALU op before every read (44 per step per wave) instead of folding the constant
// into the instruction's 16-bit offset field; behind an empty asm the base is a fresh value
// each step and every constant folds.
__device__ __forceinline__ lds_u16* opaque_lds(lds_u16* p) {
    uint32_t v = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
    asm volatile("" : "+v"(v));
    return reinterpret_cast<lds_u16*>(static_cast<uintptr_t>(v));
}

// V operand of P . V for latent tile nt and K-chunk c (rows 16c .. 16c+15 of the tile).
// Lane l needs latent column 32 nt + (l % 32) at rows 16c + 4hh + {0..3} and
// 16c + 8 + 4hh + {0..3} (hh = l / 32), matching the P fragment's row order.  Within each
// 16-lane group, lane q points at row q/4, columns 4(q%4)..4(q%4)+3 of a 4 x 16 block; the
// transposing load returns column q of the block's four rows.
__device__ __forceinline__ bf16x8 v_fragment(lds_u16* vbase, int nt, int c) {
    lds_u16* vp = vbase + 16 * c * kLatStride + 32 * nt;
    const bf16x4 v0 = lds_read_tr16(vp);
    const bf16x4 v1 = lds_read_tr16(vp + 8 * kLatStride);
    return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void store_tile_f32(float* dst, int64_t ld, int row0, int col0,
                                               const float (&v)[16], int lane) {
    const int hh = (lane >> 5) & 1;
    const int col = col0 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r)
        dst[static_cast<int64_t>(row0 + 8 * (r >> 2) + 4 * hh + (r & 3)) * ld + col] = v[r];
}

// PAGED: the latent and companion rows live in a page pool; ID p of request b is pool row
// page_table[b * max_pages + (p >> lg_page)] * 2^lg_page + p % 2^lg_page, translated once in the
// ID phase (kv_off then only gives the request lengths).
// NT: the gathered rows are loaded with the non-temporal hint (see load_tile).
template <bool PAGED, bool NT>
__global__ __launch_bounds__(256, 1) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ latent, int64_t ld_lat,
    const uint16_t* __restrict__ kpe, int64_t ld_kpe, const int64_t* __restrict__ kv_off,
    const int32_t* __restrict__ q_req, const int32_t* __restrict__ ids, int32_t T, int32_t B,
    int32_t nsplit, float scale_log2, void* __restrict__ out, int out_f32,
    float* __restrict__ lse, void* __restrict__ part_o, float* __restrict__ part_lse,
    const int32_t* __restrict__ page_table, int lg_page, int max_pages) {
    __shared__ MlaSmem sm;
    const int g = blockIdx.x;
    const int j = g >> 3;
    const int lsplit = __builtin_ctz(static_cast<unsigned>(nsplit));  // nsplit: a power of two
    const int t = (g & 7) + 8 * (j >> lsplit);
    const int split = j & (nsplit - 1);
    if (t >= T) return;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in SGPRs
    const int hh = lane >> 5;  // lane half
    const int hl = lane & 31;  // head column (S^T) / A-operand row
    const int L = kTopK >> lsplit;
    // ---- the split's IDs into LDS: padding (ID < 0 or >= S_b) becomes row 0 of the request
    // (real data, so every ring slot stays finite) and is masked out of the softmax through a
    // per-tile bit mask.  Tiles after the last real ID are not processed.  The ID loads are
    // issued before the request lookups (q_req, then kv_off) they do not depend on.
    constexpr int kIdPerThread = kTopK / 256;
    const int32_t* idr = ids + static_cast<int64_t>(t) * kTopK + static_cast<int64_t>(split) * L;
    int32_t idv[kIdPerThread];
#pragma unroll
    for (int k = 0; k < kIdPerThread; ++k) {
        const int i = 256 * k + tid;
        idv[k] = i < L ? idr[i] : -1;
    }
    // a query outside the batch (q_req[t] not in [0, B)) has no valid ID: zero read, lse -inf
    const int b = query_request(q_req, t, B);
    const int64_t off = b >= 0 ? kv_off[b] : 0;
    int64_t s_b = b >= 0 ? kv_off[b + 1] - off : 0;
    // paged: IDs beyond the page table's row (S_b > max_pages * page_size breaks the
    // contract) count as padding, so no entry past the row is read
    if constexpr (PAGED) s_b = s_b < (static_cast<int64_t>(max_pages) << lg_page) ? s_b : (static_cast<int64_t>(max_pages) << lg_page);
    const int64_t base = PAGED ? 0 : off;  // paged: the rows below are pool rows
    if (tid == 0) sm.redo = 0;
    uint32_t end = 0;
#pragma unroll
    for (int k = 0; k < kIdPerThread; ++k) {
        const int i0 = 256 * k;
        if (i0 >= L) break;  // block-uniform
        const int i = i0 + tid;
        const int32_t id = idv[k];
        const bool ok = id >= 0 && static_cast<int64_t>(id) < s_b;
        const uint64_t m = __ballot(ok);  // lanes 0..31: one tile, lanes 32..63: the next
        if (i < L) {
            int32_t row = ok ? id : 0;
            if constexpr (PAGED)  // (b < 0 leaves no valid ID and no tile to copy)
                if (b >= 0)
                    row = (page_table[static_cast<int64_t>(b) * max_pages + (row >> lg_page)] << lg_page) |
                          (row & ((1 << lg_page) - 1));
            sm.rows[i] = row;
            if ((lane & 31) == 0) sm.tmask[i / kTile] = static_cast<uint32_t>(m >> (lane & 32));
        }
        if (ok) end = static_cast<uint32_t>(i + 1);
    }
    end = wave_max_u32(end);
    if (lane == 0) sm.wend[wave] = end;
    lds_barrier();
    end = max(max(sm.wend[0], sm.wend[1]), max(sm.wend[2], sm.wend[3]));
    // The head-group waves' 32 absorbed queries, loaded once the ID phase is over and issued
    // just before the first ring copies, so both travel together.  (Issued earlier, they held
    // up the ID phase: the compiler cannot count the loads of a branch that only some waves
    // take, so it waited for all of them before using the first ID.)
    u32x4 qf[kKSteps];
    if (wave < 3) {
        const uint16_t* qh = q + (static_cast<int64_t>(t) * kMlaHeads + 32 * wave + hl) * kQK;
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
            const int d = s < kLatSteps ? 256 * hh + 8 * s : kLatent + 32 * hh + 8 * (s - kLatSteps);
            qf[s] = *reinterpret_cast<const u32x4*>(qh + d);
        }
    }
    const int n_tiles = static_cast<int>((end + kTile - 1) / kTile);
    const int q16 = lane & 15;
    const int vrow = 4 * hh + (q16 >> 2);
    const int vcol = 16 * ((lane >> 4) & 1) + 4 * (q16 & 3);
    const int64_t ps = static_cast<int64_t>(t) * nsplit + split;

    // Ring fill: wave w < 3 loads latent rows 8w .. 8w + 7 of a tile, wave 3 rows 24 .. 31 and
    // the four companion blocks (whose 16-byte chunks it XOR-swizzles by row: lane l of block kb
    // holds chunk (l % 8) ^ (row % 8) of row 8 kb + l / 8); a tile goes to ring slot tile % 3.
    const int row0 = kConsRows * wave;
    // lanes 0..31 hold the tile's 32 row IDs (the loads read them with readlane)
    auto tile_ids = [&](int tile) -> int { return sm.rows[tile * kTile + (lane & 31)]; };
    // NT (at most one query per request, so no row is gathered twice in a call): the loads
    // carry the non-temporal hint, and the rows missed in the caches are not installed in the
    // Infinity Cache on the way (cold 64-query read 87 -> 66 us).  The queries of a prefill
    // chunk share one request's rows, and there the cached rows are reused (4096-query chunk:
    // 2.04 ms with cached loads, 2.39 ms with the hint).
    auto gather = [&](const uint16_t* p) -> u32x4 {
        if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        else return *reinterpret_cast<const u32x4*>(p);
    };
    auto load_tile = [&](int tile, TileRegs& tr) {
        const int rid = tile_ids(tile);
#pragma unroll
        for (int k = 0; k < kConsRows; ++k) {
            const int64_t row = base + __builtin_amdgcn_readlane(rid, row0 + k);
            tr.lat[k] = gather(latent + row * ld_lat + 8 * lane);
        }
        if (wave == 3) {
#pragma unroll
            for (int kb = 0; kb < kTile / 8; ++kb) {
                const int r = 8 * kb + (lane >> 3);
                const int64_t row = base + sm.rows[tile * kTile + r];
                tr.kp[kb] = gather(kpe + row * ld_kpe + 8 * ((lane & 7) ^ (r & 7)));
            }
        }
    };
    auto store_tile = [&](int tile, const TileRegs& tr) {
        uint16_t* lat_slot = sm.lat[tile % kNBuf];
#pragma unroll
        for (int k = 0; k < kConsRows; ++k)
            *reinterpret_cast<u32x4*>(lat_slot + (row0 + k) * kLatStride + 8 * lane) = tr.lat[k];
        if (wave == 3) {
#pragma unroll
            for (int kb = 0; kb < kTile / 8; ++kb)
                *reinterpret_cast<u32x4*>(sm.kpe[tile % kNBuf] + kb * 8 * kCompanion + 8 * lane) = tr.kp[kb];
        }
    };
    // Start of a pass: tiles 0 and 1 loaded, tile 0 written and published by the first barrier;
    // tile 1 is written before X_0.
    TileRegs tr1;
    auto prologue = [&]() {
        TileRegs tr0;
        if (n_tiles > 0) load_tile(0, tr0);
        if (n_tiles > 1) load_tile(1, tr1);
        if (n_tiles > 0) store_tile(0, tr0);
        lds_barrier();  // tile 0 published
    };
    auto prologue_end = [&]() {  // before X_0
        if (n_tiles > 1) store_tile(1, tr1);
    };

    // Software pipeline, one barrier per step.  X_i (i >= 0) publishes tile i+1 (ring slot
    // (i+1)%3) and P(i) (pfrag[i%2]).  During step i every wave copies its share of tile i+2
    // into slot (i+2)%3 (last read in step i-1); the head groups compute S of tile i+1 and,
    // interleaved with its softmax, P(i) . V(i); wave 3 computes its latent columns of
    // P(i) . V(i).  A second pass (rare) repeats everything.
    if (wave == 3) {
        // ================= wave 3: the last kHelpTiles latent tiles of every head
        f32x16 orest[3][kHelpTiles];
        for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
            for (int hg = 0; hg < 3; ++hg)
#pragma unroll
                for (int ht = 0; ht < kHelpTiles; ++ht) orest[hg][ht] = f32x16{};
            prologue();
            prologue_end();
            lds_barrier();  // X_0
            for (int i = 0; i < n_tiles; ++i) {
                TileRegs trn;
                const bool fill = i + 2 < n_tiles;
                if (fill) load_tile(i + 2, trn);
                // all operands first (one LDS latency), then the 30 MFMAs back to back
                lds_u16* vbase = opaque_lds((lds_u16*)sm.lat[i % kNBuf] + vrow * kLatStride + vcol);
                u32x4 pf[3][2];
                bf16x8 vf[2][kHelpTiles];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
#pragma unroll
                    for (int hg = 0; hg < 3; ++hg) pf[hg][c] = sm.pfrag[i & 1][hg][lane][c];
#pragma unroll
                    for (int ht = 0; ht < kHelpTiles; ++ht) vf[c][ht] = v_fragment(vbase, kConsTiles + ht, c);
                }
                __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of all the MFMAs
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int ht = 0; ht < kHelpTiles; ++ht)
#pragma unroll
                    for (int hg = 0; hg < 3; ++hg)
                        orest[hg][ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pf[hg][c]), vf[c][ht], orest[hg][ht], 0, 0, 0);
                if (fill) store_tile(i + 2, trn);
                lds_barrier();  // X_{i+1}
            }
            if (pass == 0) {
                lds_barrier();  // E: the head groups have published their overflow flags
                if (sm.redo == 0) break;
            }
        }
        lds_barrier();  // the head groups have published 1/l (the ring is idle from here on)
        // destination: the output (one split) or this split's partial, [96][512] either way
        const int64_t dbase = (nsplit > 1 ? ps : static_cast<int64_t>(t)) * kMlaHeads * kLatent;
        void* dst = nsplit > 1 ? part_o : out;
        uint16_t* stage = sm.stage;
#pragma unroll
        for (int hg = 0; hg < 3; ++hg)
#pragma unroll
            for (int ht = 0; ht < kHelpTiles; ++ht) {
                float v[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) v[r] = orest[hg][ht][r] * sm.inv_l[32 * hg + 8 * (r >> 2) + 4 * hh + (r & 3)];
                if (out_f32)
                    store_tile_f32(static_cast<float*>(dst) + dbase, kLatent, 32 * hg, 32 * (kConsTiles + ht), v, lane);
                else
                    stage_tile_bf16(stage, 32 * hg, 32 * (kConsTiles + ht), v, lane);
            }
        if (!out_f32) {  // (uniform)
            lds_barrier();  // the whole result is staged
            stage_out(stage, static_cast<uint16_t*>(dst) + dbase, tid);
        }
        return;
    }

    // ================= head-group waves: heads 32*wave .. 32*wave+31 (qf loaded above)
    f32x16 o[kConsTiles];
    float m_ref = -INFINITY;   // reference logit of this lane's head (log2 domain)
    float m_seen = -INFINITY;  // largest logit seen (exact maximum after a full pass)
    float l_run = 0.f;         // this lane's partial sum of the bf16-rounded 2^(x - m_ref)
    bool overflow = false;
    const int sw = hl & 7;     // companion-row swizzle of this lane's A row
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

    // S^T of tile `tile` (32 rows x 32 heads): A = gathered rows (LDS, prefetched), B = q
    // registers (one accumulation chain: a second one measured no faster and pushed output
    // accumulators out of the AGPRs).  When copy_tile >= 0 this wave's latent rows of that
    // tile are copied one every four K-steps.
    auto qk_tile = [&](int tile) -> f32x16 {
        const uint16_t* lat_row = sm.lat[tile % kNBuf] + hl * kLatStride + 256 * hh;
        const uint16_t* kpe_row = sm.kpe[tile % kNBuf] + hl * kCompanion;
        // A fragment of K-step s (same K order as qf); companion chunks are swizzled
        auto afrag = [&](int s) -> u32x4 {
            const uint16_t* p = s < kLatSteps ? lat_row + 8 * s
                                              : kpe_row + 8 * ((4 * hh + s - kLatSteps) ^ sw);
            return *reinterpret_cast<const u32x4*>(p);
        };
        f32x16 sacc = {};
        u32x4 abuf[kPrefA];
#pragma unroll
        for (int k = 0; k < kPrefA; ++k) abuf[k] = afrag(k);
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
            const u32x4 cur = abuf[s % kPrefA];
            if (s + kPrefA < kKSteps) abuf[s % kPrefA] = afrag(s + kPrefA);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur), as_bf16x8(qf[s]), sacc, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        const uint32_t tmask = __builtin_amdgcn_readfirstlane(sm.tmask[tile]);  // uniform
        if (tmask != 0xffffffffu) {  // uniform: the tile holds padding rows
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (!((tmask >> (8 * (r >> 2) + 4 * hh + (r & 3))) & 1u)) sacc[r] = -INFINITY;
        }
        return sacc;
    };
    // Probabilities of one S^T tile relative to the fixed per-head reference, packed to bf16
    // in A-operand layout (pa0: K-half 0, pa1: K-half 1); the normaliser sums the rounded P.
    auto softmax_tile = [&](f32x16 sacc, u32x4& pa0, u32x4& pa1) {
        float mx = sacc[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
        // the two lane halves hold the head's two K-halves: v_permlane32_swap pairs lane l
        // with lane l ^ 32 on the VALU (no LDS round trip)
        const auto mxs = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                          false, false);
        mx = fmaxf(__uint_as_float(mxs[0]), __uint_as_float(mxs[1])) * scale_log2;  // scale > 0 keeps the order
        m_seen = fmaxf(m_seen, mx);
        if (m_ref == -INFINITY) m_ref = mx;  // first tile of pass 0 (uniform per head)
        overflow |= mx > m_ref + 32.f;
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
        // p = 2^(x scale - m_ref) with one rounding before the raw v_exp_f32; results below
        // 2^-126 flush to zero (under bf16's normal range: below 2^-100 of the sum).  P enters
        // P . V in bf16 (v_cvt_pk_bf16_f32 rounds to nearest even) and the normaliser sums the
        // same rounded values (v_dot2 against 1.0), so the read is an exact convex combination
        // of the rounded weights (a dominant row's rounding cancels instead of showing up as a
        // 2^-9 relative error of the output).
#pragma unroll
        for (int r = 0; r < 16; ++r)
            sacc[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], scale_log2, -m_use));
        float psum0 = 0.f, psum1 = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const bf16x2 b0 = __builtin_convertvector((f32x2{sacc[2 * k], sacc[2 * k + 1]}), bf16x2);
            const bf16x2 b1 = __builtin_convertvector((f32x2{sacc[8 + 2 * k], sacc[9 + 2 * k]}), bf16x2);
            pa0[k] = __builtin_bit_cast(uint32_t, b0);
            pa1[k] = __builtin_bit_cast(uint32_t, b1);
            psum0 = __builtin_amdgcn_fdot2_f32_bf16(b0, ones, psum0, false);
            psum1 = __builtin_amdgcn_fdot2_f32_bf16(b1, ones, psum1, false);
        }
        l_run += psum0 + psum1;
    };
    // O += P . V over this wave's latent tiles (V fragments prefetched from LDS); step =
    // c * kConsTiles + nt, so both K-halves of an output tile are kConsTiles MFMAs apart.
    auto pv_tile = [&](int tile) {
        const u32x4 pa0 = sm.pfrag[tile & 1][wave][lane][0];
        const u32x4 pa1 = sm.pfrag[tile & 1][wave][lane][1];
        lds_u16* vbase = opaque_lds((lds_u16*)sm.lat[tile % kNBuf] + vrow * kLatStride + vcol);
        bf16x8 vbuf[kPrefV];
#pragma unroll
        for (int k = 0; k < kPrefV; ++k) vbuf[k] = v_fragment(vbase, k % kConsTiles, k / kConsTiles);
#pragma unroll
        for (int step = 0; step < 2 * kConsTiles; ++step) {
            const bf16x8 cur = vbuf[step % kPrefV];
            const int nx = step + kPrefV;
            if (nx < 2 * kConsTiles) vbuf[step % kPrefV] = v_fragment(vbase, nx % kConsTiles, nx / kConsTiles);
            const int nt = step % kConsTiles;
            o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(step < kConsTiles ? pa0 : pa1), cur, o[nt], 0, 0, 0);
            // keeps the rotating prefetch (left alone, the compiler re-reads each fragment
            // right before its MFMA and waits the full LDS latency every time)
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int nt = 0; nt < kConsTiles; ++nt) o[nt] = f32x16{};
        l_run = 0.f;
        overflow = false;
        prologue();
        // The last kQfInAcc query fragments move to accumulation registers (MFMA reads its B
        // operand from there directly), leaving VGPRs for deep LDS prefetch.  This is done only
        // here, after the prologue has waited for tile 0 (and so for the query loads issued
        // before it): an asm operand makes the compiler wait for the load, and placed right
        // after each load those waits serialised eleven round trips to memory.
        if (pass == 0) {
#pragma unroll
            for (int s = kKSteps - kQfInAcc; s < kKSteps; ++s) asm volatile("" : "+a"(qf[s]));
        }
        if (n_tiles > 0) {
            u32x4 p0, p1;
            softmax_tile(qk_tile(0), p0, p1);
            sm.pfrag[0][wave][lane][0] = p0;
            sm.pfrag[0][wave][lane][1] = p1;
        }
        prologue_end();
        lds_barrier();  // X_0
        for (int i = 0; i < n_tiles; ++i) {
            // one copy of each part in the loop body (two code paths doubled the register
            // footprint of the output accumulators)
            const bool next = i + 1 < n_tiles;
            u32x4 pn0 = {0u, 0u, 0u, 0u}, pn1 = {0u, 0u, 0u, 0u};
            // this wave's rows of tile i + 2 are loaded at the start of the step (they have the
            // whole step to arrive) and written into their slot at its end
            TileRegs trn;
            const bool fill = i + 2 < n_tiles;
            if (fill) load_tile(i + 2, trn);
            if (next) {
                const f32x16 s_next = qk_tile(i + 1);
                softmax_tile(s_next, pn0, pn1);
            }
            pv_tile(i);
            if (next) {
                sm.pfrag[(i + 1) & 1][wave][lane][0] = pn0;
                sm.pfrag[(i + 1) & 1][wave][lane][1] = pn1;
            }
            if (fill) store_tile(i + 2, trn);
            lds_barrier();  // X_{i+1}
        }
        if (pass == 0) {
            if (__ballot(overflow) && lane == 0) sm.redo = 1;
            lds_barrier();  // E
            if (sm.redo == 0) break;
            m_ref = m_seen;  // second pass: the exact maximum, so every p <= 1
        }
    }

    // ---- epilogue: rows of O are heads 8(r/4) + 4hh + r%4 of this group
    const auto ls = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run),
                                                     false, false);
    const float l_tot = __uint_as_float(ls[0]) + __uint_as_float(ls[1]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse2 = l_tot > 0.f ? m_ref + log2f(l_tot) : -INFINITY;
    const int head0 = 32 * wave;
    if (hh == 0) {
        sm.inv_l[head0 + hl] = inv;
        if (nsplit == 1) {
            if (lse) lse[static_cast<int64_t>(t) * kMlaHeads + head0 + hl] = lse2 * kLn2;
        } else {
            part_lse[ps * kMlaHeads + head0 + hl] = lse2;
        }
    }
    lds_barrier();  // publish 1/l to the gather wave
    float ir[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) ir[r] = __shfl(inv, 8 * (r >> 2) + 4 * hh + (r & 3));
    const int64_t dbase = (nsplit > 1 ? ps : static_cast<int64_t>(t)) * kMlaHeads * kLatent;
    void* dst = nsplit > 1 ? part_o : out;
    uint16_t* stage = sm.stage;
#pragma unroll
    for (int nt = 0; nt < kConsTiles; ++nt) {
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = o[nt][r] * ir[r];
        if (out_f32)
            store_tile_f32(static_cast<float*>(dst) + dbase, kLatent, head0, 32 * nt, v, lane);
        else
            stage_tile_bf16(stage, head0, 32 * nt, v, lane);
    }
    if (!out_f32) {  // (uniform)
        lds_barrier();  // the whole result is staged
        stage_out(stage, static_cast<uint16_t*>(dst) + dbase, tid);
    }
}

// Merge split partials: one wave per (query, head), 8 latent columns per lane.
//   O = sum_s 2^(l_s - m) O_s / sum_s 2^(l_s - m),  m = max_s l_s
// (partials in bf16 for a bf16 output, else fp32).  The split count is a template argument so
// every load of a wave is issued before the first one is needed (one memory round trip for
// the log-sum-exps, one for the partials).
template <bool F32, int NS>
__global__ __launch_bounds__(256) void mla_combine_kernel(const void* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          int32_t T, void* __restrict__ out,
                                                          float* __restrict__ lse) {
    const int64_t pair = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (pair >= static_cast<int64_t>(T) * kMlaHeads) return;
    const int t = static_cast<int>(pair / kMlaHeads), hd = static_cast<int>(pair % kMlaHeads);
    const int lane = lane_id();
    float ls[NS];
    u32x4 x[NS][F32 ? 2 : 1];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int64_t ps = static_cast<int64_t>(t) * NS + s;
        ls[s] = part_lse[ps * kMlaHeads + hd];
        const int64_t pi = (ps * kMlaHeads + hd) * kLatent + 8 * lane;
        if constexpr (F32) {
            const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const float*>(part_o) + pi);
            x[s][0] = src[0];
            x[s][1] = src[1];
        } else {
            x[s][0] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(part_o) + pi);
        }
    }
    float m = -INFINITY;
#pragma unroll
    for (int s = 0; s < NS; ++s) m = fmaxf(m, ls[s]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        // a split without valid IDs has l_s = -inf and weight 0 (its partial is all zeros)
        const float wgt = ls[s] == -INFINITY ? 0.f : exp2f(ls[s] - m);
        wsum += wgt;
        if constexpr (F32) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] += wgt * __uint_as_float(x[s][0][e]);
                acc[4 + e] += wgt * __uint_as_float(x[s][1][e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += wgt * __uint_as_float(x[s][0][e] << 16);
                acc[2 * e + 1] += wgt * __uint_as_float(x[s][0][e] & 0xffff0000u);
            }
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const int64_t oi = (static_cast<int64_t>(t) * kMlaHeads + hd) * kLatent + 8 * lane;
    if constexpr (F32) {
        f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(out) + oi);
        dst[0] = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
        dst[1] = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
    } else {
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + oi) = o;
    }
    if (lse && lane == 0)
        lse[static_cast<int64_t>(t) * kMlaHeads + hd] = wsum > 0.f ? (m + log2f(wsum)) * kLn2 : -INFINITY;
}

template <int NS>
static void launch_combine(bool out_f32, unsigned blocks, const void* part_o,
                           const float* part_lse, int32_t T, void* out, float* lse,
                           hipStream_t stream) {
    if (out_f32)
        hipLaunchKernelGGL((mla_combine_kernel<true, NS>), dim3(blocks), dim3(256), 0, stream,
                           part_o, part_lse, T, out, lse);
    else
        hipLaunchKernelGGL((mla_combine_kernel<false, NS>), dim3(blocks), dim3(256), 0, stream,
                           part_o, part_lse, T, out, lse);
}

int sparse_mla_nsplit(int32_t T) {
    int ns = 1;
    while (ns < 16 && static_cast<int64_t>(T) * ns < 256) ns *= 2;
    return ns;
}

// Split workspace: per-split partial outputs (sized for fp32), then per-split log2-sum-exp.
static size_t round256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t sparse_mla_workspace_bytes(int32_t T) {
    const int ns = sparse_mla_nsplit(T);
    if (ns == 1 || T <= 0) return 0;
    const size_t parts = static_cast<size_t>(T) * ns;
    return round256(parts * kMlaHeads * kLatent * sizeof(float)) + round256(parts * kMlaHeads * sizeof(float));
}

hipError_t launch_sparse_mla(const uint16_t* q, const uint16_t* latent, int64_t ld_lat,
                             const uint16_t* kpe, int64_t ld_kpe, const int64_t* kv_off,
                             const int32_t* q_req, const int32_t* ids, int32_t T, int32_t B,
                             float scale, void* out, bool out_f32, float* lse, void* workspace,
                             hipStream_t stream, const int32_t* page_table, int lg_page,
                             int max_pages) {
    const int ns = sparse_mla_nsplit(T);
    const int64_t groups = (static_cast<int64_t>(T) + 7) / 8;
    const int64_t blocks = groups * 8 * ns;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    void* part_o = nullptr;
    float* part_lse = nullptr;
    if (ns > 1) {
        part_o = workspace;
        part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                            round256(static_cast<size_t>(T) * ns * kMlaHeads * kLatent * sizeof(float)));
    }
    const float scale_log2 = scale * 1.4426950408889634f;
    const bool nt = T <= B;  // no more queries than requests: rows are not shared
    auto launch = [&](auto kernel, const int32_t* pt) {
        hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, q,
                           latent, ld_lat, kpe, ld_kpe, kv_off, q_req, ids, T, B, ns, scale_log2,
                           out, out_f32 ? 1 : 0, lse, part_o, part_lse, pt, pt ? lg_page : 0,
                           pt ? max_pages : 0);
    };
    if (page_table)
        nt ? launch(sparse_mla_kernel<true, true>, page_table) : launch(sparse_mla_kernel<true, false>, page_table);
    else
        nt ? launch(sparse_mla_kernel<false, true>, nullptr) : launch(sparse_mla_kernel<false, false>, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ns == 1) return e;
    const unsigned cblocks = static_cast<unsigned>((static_cast<int64_t>(T) * kMlaHeads + 3) / 4);
    switch (ns) {  // sparse_mla_nsplit gives a power of two up to 16
        case 2: launch_combine<2>(out_f32, cblocks, part_o, part_lse, T, out, lse, stream); break;
        case 4: launch_combine<4>(out_f32, cblocks, part_o, part_lse, T, out, lse, stream); break;
        case 8: launch_combine<8>(out_f32, cblocks, part_o, part_lse, T, out, lse, stream); break;
        default: launch_combine<16>(out_f32, cblocks, part_o, part_lse, T, out, lse, stream); break;
    }
    return hipGetLastError();
}

}  // namespace dsa
