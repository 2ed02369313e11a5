// Stage 3: per-row top-2048 selection -> request-local position IDs, ascending, -1 padded.
//
// Page "Kimi K3.1 Pro: Sparse-Zugriffe, keine kleinere Historie", section "Eine Query durch
// den Indexer verfolgen": up to 2048 causal candidates per query, a logical [T,2048]
// position-ID array, short prefixes and invalid entries handled by the backend; section
// "Die Mathematik der Sparse Attention ...": I_t holds the up-to-2048 highest-scoring
// positions.  Tie rule (the page is silent): equal scores go to the lower position, -0 ==
// +0, NaN ranks lowest -- so the selected set, and the ascending ID row, are unique.
//
// One 1024-thread block per row; rows of 32769..65536 elements (the prefill case) run one
// persistent block per CU instead, which copies half of its next row into LDS while it
// selects the current one and loads the other half into registers during the compaction.  Scores become order-preserving u32 keys (0 is reserved for "no
// element"), kept in registers (E per thread) when the row fits, re-streamed from global
// memory per pass otherwise.  Selection is a radix-style
// threshold search on an LDS histogram of 2048 bins:
//   level 0  bins linear in the score value between the row's finite min and max (a
//            monotone map, so whole bins are above / below the threshold; spreading the
//            bulk of the row over many bins keeps LDS atomic conflicts low),
//   level 1+ exact bins on the key bits inside the threshold bin's key range (11 bits per
//            level) until the threshold bin is taken whole or holds a single key value.
// The threshold bin of a level is found with a block-wide scan over the histogram.  The
// final compaction is an ordered scan (wave ballot + mbcnt within a wave, an LDS scan of the
// per-(element, wave) counts across the block) that writes the selected positions in
// ascending order; ties at the threshold key are ranked by position with the same scan.
#include <atomic>
#include <type_traits>

#include "common.h"

namespace dsa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBins = 2048;
constexpr int kBinBits = 11;
constexpr uint32_t kKeyNegInf = 0x007FFFFFu;  // key of -inf
constexpr uint32_t kKeyPosInf = 0xFF800000u;  // key of +inf

// The keys below need IEEE -0 and NaN semantics (x + 0 must not fold to x, isnan must not
// fold to false).
#if defined(__FAST_MATH__) || (defined(__FINITE_MATH_ONLY__) && __FINITE_MATH_ONLY__)
#error "topk.hip needs IEEE semantics for -0 and NaN: build it without fast-math"
#endif

// Order-preserving key: larger score -> larger key; -0 and +0 share a key; every NaN maps
// to 1 (below -inf); 0 is never produced (it marks an absent element).
// Five VALU instructions: x + 0 turns -0 into +0 and leaves every other non-NaN value as it is
// (fp32 denormals are kept: the kernels run with denormals preserved), an arithmetic shift and
// one three-input bit operation (v_bitop3_b32) flip the bits, and an ordered self-compare with
// a select sends NaN to 1.  (The same map as testing NaN and -0 on the bits, which took
// eight; equal on all 2^32 patterns.)
__device__ __forceinline__ uint32_t score_key(float x) {
    const uint32_t u = __float_as_uint(x + 0.0f);
    const uint32_t k = u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
    return __builtin_isnan(x) ? 1u : k;
}

// Score of a key: keys with the top bit set are non-negative scores (their sign bit was set),
// the others negative ones (all bits were flipped).  Key 1 (NaN) gives a NaN pattern.
__device__ __forceinline__ float key_to_score(uint32_t k) {
    const uint32_t m = static_cast<uint32_t>(static_cast<int32_t>(k) >> 31);  // ~0 if top bit set
    // k ^ (~m | 0x80000000) as one three-input bit operation: truth table f(s0, s1, s2) =
    // s0 ^ (~s1 | s2) is f(0xF0, 0xCC, 0xAA) = 0x4B.  (Written as C, the shift becomes a
    // compare and a select, and the xor a third instruction.)
    return __uint_as_float(__builtin_amdgcn_bitop3_b32(k, m, 0x80000000u, 0x4B));
}

// Value-linear bin of a key: trunc(clamp(x * scale + off, 0, 2047)) with x its score and
// off = -lo * scale.  fma, the clamps and truncation are each monotone non-decreasing, so the
// map is; NaN lands in bin 0 (the max with 0 drops it), -inf in bin 0, +inf in bin 2047.
__device__ __forceinline__ int value_bin(uint32_t k, float scale, float off) {
    const float f = fminf(fmaxf(__builtin_fmaf(key_to_score(k), scale, off), 0.f),
                          static_cast<float>(kBins - 1));
    return static_cast<int>(f);
}

__device__ __forceinline__ int shift_for(uint32_t span) {
    const int bits = span ? 32 - __clz(span) : 0;
    return bits > kBinBits ? bits - kBinBits : 0;
}

struct TopkSmem {
    uint32_t hist[kBins];             // histogram; at the end the output row being staged
    uint32_t bm[2][kBins];            // selection bitmaps (above, tie) of a register-resident row
    uint32_t wtot[kTopkWaves];
    uint32_t red[4][kTopkWaves];
    uint32_t cnt[2][2 * kTopkWaves];  // per-wave (above, tie) counts, double-buffered by chunk
    uint32_t prm[8];
    uint32_t cbuf[64];                // keys of a small threshold bin
};

constexpr uint32_t kFastCand = 64;  // threshold bins up to this size are resolved by one wave

// Exclusive prefix sum over the block (thread order); returns this thread's exclusive sum
// and writes the block total to *total (all threads).  Contains barriers.
template <class Smem>
__device__ __forceinline__ uint32_t block_exclusive_scan(Smem& sm, uint32_t v, uint32_t* total) {
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const uint32_t incl = wave_inclusive_scan(v);
    if (lane == 63) sm.wtot[wave] = incl;
    lds_barrier();
    uint32_t wbase = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kTopkWaves; ++i) {
        const uint32_t x = sm.wtot[i];
        wbase += (i < wave) ? x : 0u;
        tot += x;
    }
    lds_barrier();
    *total = tot;
    return wbase + incl - v;
}

// Find the bin b* holding the need-th largest candidate: count(bins > b*) < need <=
// count(bins >= b*).  Writes b* to prm[0] and count(bins > b*) to prm[1].
template <class Smem>
__device__ __forceinline__ void find_threshold_bin(Smem& sm, uint32_t need) {
    const int tid = threadIdx.x;
    const int hb = kBins - 1 - 2 * tid, lb = hb - 1;
    const uint32_t ch = sm.hist[hb], cl = sm.hist[lb];
    if (tid == 0) {
        sm.prm[0] = 0;
        sm.prm[1] = 0;
    }
    uint32_t total;
    const uint32_t before = block_exclusive_scan(sm, ch + cl, &total);
    if (before < need && before + ch >= need) {
        sm.prm[0] = hb;
        sm.prm[1] = before;
    } else if (before + ch < need && before + ch + cl >= need) {
        sm.prm[0] = lb;
        sm.prm[1] = before + ch;
    }
    lds_barrier();
}

// Block-wide min/max of up to four u32 values (results broadcast to all threads).
template <class Smem>
__device__ __forceinline__ void block_minmax(Smem& sm, uint32_t& a_min, uint32_t& a_max,
                                             uint32_t& b_min, uint32_t& b_max) {
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    a_min = wave_min_u32(a_min);
    a_max = wave_max_u32(a_max);
    b_min = wave_min_u32(b_min);
    b_max = wave_max_u32(b_max);
    if (lane == 0) {
        sm.red[0][wave] = a_min;
        sm.red[1][wave] = a_max;
        sm.red[2][wave] = b_min;
        sm.red[3][wave] = b_max;
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < kTopkWaves; ++i) {
        a_min = min(a_min, sm.red[0][i]);
        a_max = max(a_max, sm.red[1][i]);
        b_min = min(b_min, sm.red[2][i]);
        b_max = max(b_max, sm.red[3][i]);
    }
    lds_barrier();
}

// Exact key interval of value bin `bin` among keys in [a, b]: the smallest key whose bin is
// >= bin and the largest whose bin is <= bin (value_bin is monotone, so the keys of one bin
// form an interval; both ends exist because some key in [a, b] falls in the bin).  One wave:
// lanes 0..31 run a 32-ary search for the lower end, lanes 32..63 for the upper end; each
// step keeps one of 32 sub-intervals, so seven steps cover the 32-bit key space.
__device__ __forceinline__ void value_bin_key_range(uint32_t a, uint32_t b, int bin, float scale,
                                                    float bias, uint32_t* r_lo, uint32_t* r_hi) {
    const int lane = lane_id();
    const uint32_t j = static_cast<uint32_t>(lane & 31);
    const bool up = lane >= 32;
    uint32_t l = a, h = b;  // the end this half-wave looks for lies in [l, h]
    for (int step = 0; step < 10; ++step) {
        if (!__ballot(l != h)) break;
        const uint64_t w = static_cast<uint64_t>(h - l) + 1u;
        auto off = [&](uint32_t i) { return static_cast<uint32_t>((w * i) >> 5); };
        // lower end: probes ascend from l and pass once the bin reaches `bin`;
        // upper end: probes descend from h and pass once the bin drops to `bin`
        const uint32_t k = up ? h - off(j) : l + off(j);
        const int vb = value_bin(k, scale, bias);
        const uint64_t m = __ballot(up ? vb <= bin : vb >= bin);
        const uint32_t half = static_cast<uint32_t>(up ? (m >> 32) : (m & 0xffffffffu));
        const uint32_t j0 = half ? static_cast<uint32_t>(__builtin_ctz(half)) : 32u;
        if (l == h) continue;
        if (j0 == 0) {
            if (up) l = h; else h = l;
        } else if (up) {
            const uint32_t nh = h - off(j0 - 1) - 1u;
            l = j0 < 32 ? h - off(j0) : l;
            h = nh;
        } else {
            const uint32_t nl = l + off(j0 - 1) + 1u;
            h = j0 < 32 ? l + off(j0) : h;
            l = nl;
        }
    }
    *r_lo = __builtin_amdgcn_readlane(l, 0);
    *r_hi = __builtin_amdgcn_readlane(h, 32);
}

__device__ __forceinline__ uint32_t mbcnt64(uint64_t m, uint32_t acc) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), acc));
}

// Element e = 4g + c of a thread sits at offset 64E*wave + 256g + 4*lane + c of its chunk of
// 1024E positions: each wave owns a contiguous span, each load instruction reads 1 KB
// contiguous, and position order is (wave, g, lane, c) -- which the ordered compaction uses
// to rank elements with ballots and scalar running counts instead of block scans.
// What a launch of topk_kernel selects from:
//  kRow   -- row t of the score matrix (positions 0 .. n_t-1); writes the positions;
//  kParts -- part q of row t (block t*P + q): positions q*chunk .. q*chunk+chunk-1 of the
//            row; writes the part's top-2048 as part-local positions to cand, and their keys
//            (read back from the part's scores, which are in the L2) to cand_keys;
//  kMerge -- the P part lists of row t (P*2048 candidates in ascending position order, with
//            their keys); writes the selected positions.
// A row's top-2048 is always inside the union of its parts' top-2048 lists (an element
// beaten by 2048 others in its own part is beaten by them in the row), and the tie rule
// (equal scores: lower position first) is the same at both levels, so the merge is exact.
enum TopkMode { kRow = 0, kParts = 1, kMerge = 2 };

// Where each row's length comes from: explicit n_valid[t] when n_valid is given, else the
// causal prefix min(q_pos[t] + 1, S_b) of request q_req[t] (0 when q_req[t] lies outside
// [0, n_req)); at most max_n, at least 0.
struct RowLens {
    const int32_t* n_valid;
    const int64_t* kv_off;
    const int32_t* q_req;
    const int32_t* q_pos;
    int64_t max_n;
    int32_t n_req;
};

__device__ __forceinline__ int64_t topk_row_len(int t, const RowLens& rl) {
    int64_t n_row;
    if (rl.n_valid) {
        n_row = rl.n_valid[t];
        n_row = n_row < rl.max_n ? n_row : rl.max_n;
        return n_row > 0 ? n_row : 0;
    }
    return admissible_count(rl.kv_off, query_request(rl.q_req, t, rl.n_req), rl.q_pos[t], rl.max_n);
}

// Rows selected by a persistent block (one per CU, looping over rows) have the first
// kPreGroups load groups of every wave copied into LDS while the block still works on the
// previous row: the row load (256 KB for 65536 elements) otherwise leaves the CU idle for
// about half of a row's time.  The slices are wave-private (wave w copies exactly the 1 KB
// groups it reads itself), so only the wave's own vmcnt / lgkmcnt waits order them.
constexpr int kPreGroups = 8;  // 16 waves x 8 KB = 128 KB of LDS

// Wait until this wave's LDS operations have completed (lgkmcnt 0, the other counters at
// their maxima).
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Copy prefetch group g of this wave of a row of n elements into its LDS slice (only if the
// group lies wholly inside the row): group g of wave w holds positions 64E*w + 256g .. +255.
// The wave's reads of the slice (previous row) must be done (lgkmcnt 0).
template <int E>
__device__ __forceinline__ void topk_prefetch_group(f32x4* pre, const float* row, int64_t n, int g) {
    int lane = lane_id();
    __asm__ volatile("" : "+v"(lane));  // (recomputed per row, see topk_select)
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int64_t base = static_cast<int64_t>(wave) * 64 * E + 256 * g;
    if (base + 256 <= n)
        copy_to_lds<true>(row + base + 4 * lane, lds_offset(pre + (wave * kPreGroups + g) * 64));
}

// All of this wave's prefetch groups of a row.
template <int E>
__device__ __forceinline__ void topk_prefetch(f32x4* pre, const float* row, int64_t n) {
    wait_lgkmcnt0();  // the wave's reads of the slices (previous row) are done
#pragma unroll
    for (int g = 0; g < kPreGroups; ++g) topk_prefetch_group<E>(pre, row, n, g);
}

// Selection of one row (kRow, kMerge) or part (kParts) by the whole block; ob is the output
// row (the block's index without persistence).  PRE: when pre_rd, the LDS slices hold this
// row's first kPreGroups groups, and when nxt_rd, nxt holds its later groups (register
// loads issued during the previous row's compaction).  The next row's groups (next_row,
// n_next; null if none) are copied into the slices as soon as this row's elements are in
// registers, and loaded into nxt once they are in the selection bitmaps (*nxt_issued).
template <int E, bool STREAM, bool VEC, int MODE, bool PRE>
__device__ __forceinline__ void topk_select(
    TopkSmem& sm, const int t, const int part, const int64_t ob,
    const float* __restrict__ scores, int64_t ld, const RowLens& rl, int32_t* __restrict__ ids,
    int32_t parts, int64_t chunk, const int32_t* __restrict__ cands, uint32_t* __restrict__ cand_keys,
    f32x4* pre, bool pre_rd, const float* next_row, int64_t n_next, f32x4* nxt, bool nxt_rd,
    bool* nxt_issued) {
    static_assert(E % 4 == 0, "elements come in groups of four consecutive positions");
    static_assert(MODE != kMerge || !STREAM, "a merge holds its candidates in registers");
    static_assert(!PRE || (MODE == kRow && !STREAM && VEC && E >= 4 * kPreGroups),
                  "prefetch: register-resident rows with aligned 16-byte loads");
    constexpr int kGroups = E / 4;
    int tid = threadIdx.x;
    int lane = lane_id();
    // In the persistent row loop the per-lane address terms would be hoisted out of the loop
    // and stay live (spilled) through the whole selection: make them opaque per row.
    if constexpr (PRE) __asm__ volatile("" : "+v"(tid), "+v"(lane));
    const int wave = PRE ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;

    const int64_t n_row = topk_row_len(t, rl);
    int64_t n = n_row;  // elements this block selects from (element index p < n)
    if (MODE == kParts) {
        n = n_row - part * chunk;
        n = n < chunk ? n : chunk;
        n = n > 0 ? n : 0;
    } else if (MODE == kMerge) {
        n = static_cast<int64_t>(parts) * kTopK;
    }
    int32_t* out = ids + ob * kTopK;
    const int64_t n_short = MODE == kMerge ? n_row : n;
    if (n_short <= kTopK) {
        if constexpr (PRE) {
            topk_prefetch<E>(pre, next_row, n_next);
            *nxt_issued = false;
        }
        for (int i = tid; i < kTopK; i += kTopkThreads) out[i] = i < n_short ? i : -1;
        if constexpr (MODE == kParts) {
            const float* prow = scores + static_cast<int64_t>(t) * ld + part * chunk;
            for (int i = tid; i < kTopK; i += kTopkThreads)
                cand_keys[ob * kTopK + i] = i < n_short ? score_key(prow[i]) : 0u;
        }
        return;
    }
    const float* row = scores + static_cast<int64_t>(t) * ld + (MODE == kParts ? part * chunk : 0);
    constexpr int64_t kChunk = static_cast<int64_t>(kTopkThreads) * E;
    const int n_chunks = STREAM ? static_cast<int>((n + kChunk - 1) / kChunk) : 1;
    const int64_t tbase = static_cast<int64_t>(wave) * 64 * E + 4 * lane;
    uint32_t key[E];
    int32_t cpos[MODE == kMerge ? E : 1];  // merge: row position of each candidate (-1: none)
    auto load = [&](int ch) {
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            const int64_t p = ch * kChunk + tbase + 256 * g;
            if constexpr (MODE == kMerge) {
                // the candidates' positions and keys, both read contiguously
                const int q = static_cast<int>(p / kTopK);  // a group never straddles two lists
                const int64_t ci = (static_cast<int64_t>(t) * parts + q) * kTopK + (p - q * kTopK);
                const i32x4 local = *reinterpret_cast<const i32x4*>(cands + ci);
                const u32x4 kk = *reinterpret_cast<const u32x4*>(cand_keys + ci);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    cpos[4 * g + c] = local[c] >= 0 ? static_cast<int32_t>(q * chunk + local[c]) : -1;
                    key[4 * g + c] = local[c] >= 0 ? kk[c] : 0u;
                }
            } else if (PRE && g < kPreGroups && pre_rd &&
                       static_cast<int64_t>(wave) * 64 * E + 256 * g + 256 <= n) {  // wave-uniform
                const f32x4 v = pre[(wave * kPreGroups + g) * 64 + lane];
#pragma unroll
                for (int c = 0; c < 4; ++c) key[4 * g + c] = score_key(v[c]);
            } else if (PRE && g >= kPreGroups && nxt_rd &&
                       static_cast<int64_t>(wave) * 64 * E + 256 * g + 256 <= n) {  // wave-uniform
                const f32x4 v = nxt[PRE && g >= kPreGroups ? g - kPreGroups : 0];
#pragma unroll
                for (int c = 0; c < 4; ++c) key[4 * g + c] = score_key(v[c]);
            } else if (VEC && p + 3 < n) {
                const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + p));
#pragma unroll
                for (int c = 0; c < 4; ++c) key[4 * g + c] = score_key(v[c]);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) key[4 * g + c] = p + c < n ? score_key(row[p + c]) : 0u;
            }
        }
    };
    if (!STREAM) load(0);

    // ---- row statistics: range of all keys, and of the finite ones (a second pass only when
    // the row holds +-inf or NaN).  Absent elements (key 0) wrap to the top in k - 1.
    uint32_t amin = ~0u, amax = 0u;
    for (int ch = 0; ch < n_chunks; ++ch) {
        if (STREAM) load(ch);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            amin = min(amin, key[e] - 1u);
            amax = max(amax, key[e]);
        }
    }
    for (int i = tid; i < kBins; i += kTopkThreads) sm.hist[i] = 0;  // ordered by the barriers below
    if (tid == 0) sm.prm[4] = 0u;  // fill count of cbuf
    {
        uint32_t d0 = ~0u, d1 = 0u;
        block_minmax(sm, amin, amax, d0, d1);
    }
    amin += 1u;
    uint32_t fmin = amin, fmax = amax;
    if (amin <= kKeyNegInf || amax >= kKeyPosInf) {  // block-uniform
        fmin = ~0u;
        fmax = 0u;
        for (int ch = 0; ch < n_chunks; ++ch) {
            if (STREAM) load(ch);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const uint32_t k = key[e];
                if (k > kKeyNegInf && k < kKeyPosInf) {
                    fmin = min(fmin, k);
                    fmax = max(fmax, k);
                }
            }
        }
        uint32_t d0 = ~0u, d1 = 0u;
        block_minmax(sm, fmin, fmax, d0, d1);
    }

    bool value_mode = false;
    float scale = 0.f, off = 0.f;
    if (fmin < fmax) {
        const float lo = key_to_score(fmin);
        const float span = key_to_score(fmax) - lo;
        scale = static_cast<float>(kBins) / span;
        off = -lo * scale;
        value_mode = isfinite(scale) && scale > 0.f && isfinite(off);
    }

    uint32_t rlo = amin, rhi = amax;  // candidate key range (inclusive)
    uint32_t need = kTopK;            // candidates still to take
    uint32_t cand;                    // candidates in the current range

    // ---- level 0
    {
        // rows held in registers with up to 32 elements per thread keep each element's bin
        constexpr bool kSaveBins = E <= 32 && !STREAM;
        uint32_t kbin[kSaveBins ? E : 1];
        const int sh = value_mode ? 0 : shift_for(rhi - rlo);
        // one loop per binning (a per-element select on the block-uniform mode compiled into
        // a branch per element).  Absent elements (key 0, positions past n) are not counted:
        // a wave whose positions of the chunk all lie below n has none and counts without the
        // per-element guard (which costs a compare, an exec-mask save and restore and two
        // branches); only the wave that holds the row's end, and a merge (whose absent
        // candidates lie anywhere), keep it.  (Counting them into bin 0 and subtracting their
        // number instead made rows shorter than the chunk slower: their atomics all hit one
        // address.)
        auto count = [&](auto bin_of) {
            for (int ch = 0; ch < n_chunks; ++ch) {
                if (STREAM) load(ch);
                const bool full = MODE != kMerge &&
                                  static_cast<int64_t>(ch) * kChunk + static_cast<int64_t>(wave + 1) * 64 * E <= n;
                auto one = [&](int e, auto guarded) {
                    const uint32_t k = key[e];
                    const int bin = bin_of(k);
                    if constexpr (decltype(guarded)::value) {
                        if (k) atomicAdd(&sm.hist[bin], 1u);
                        if constexpr (kSaveBins) kbin[e] = k ? static_cast<uint32_t>(bin) : 0xFFFFu;
                    } else {
                        atomicAdd(&sm.hist[bin], 1u);
                        if constexpr (kSaveBins) kbin[e] = static_cast<uint32_t>(bin);
                    }
                    // Every wave's keys are in registers: the next row's copies now stream
                    // while this row is selected (issued earlier, they would compete with the
                    // slower waves' loads of this row).  One copy per eight elements counted:
                    // issued all at once they stalled the wave (2% slower overall).
                    if constexpr (PRE) {
                        if (e == 0) wait_lgkmcnt0();  // (this row's slice reads are done)
                        if (e % (E / kPreGroups) == E / kPreGroups - 1)
                            topk_prefetch_group<E>(pre, next_row, n_next, e / (E / kPreGroups));
                    }
                };
                if (full) {  // wave-uniform
#pragma unroll
                    for (int e = 0; e < E; ++e) one(e, std::false_type{});
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) one(e, std::true_type{});
                }
            }
        };
        if (value_mode)
            count([&](uint32_t k) { return value_bin(k, scale, off); });
        else
            count([&](uint32_t k) { return static_cast<int>((k - rlo) >> sh); });
        lds_barrier();
        find_threshold_bin(sm, need);
        const uint32_t bstar = sm.prm[0];
        need -= sm.prm[1];
        cand = sm.hist[bstar];
        // Small threshold bin (at most kFastCand keys, gathered in cbuf): one wave finds the
        // need-th largest key theta by counting (#keys > theta < need <= #keys >= theta); the
        // final range is then the single key theta.  Contains a barrier.
        auto resolve_small_bin = [&]() {
            if (wave == 0) {
                const uint32_t nc = __builtin_amdgcn_readfirstlane(cand);  // uniform loop bound
                const uint32_t mine = static_cast<uint32_t>(lane) < nc ? sm.cbuf[lane] : 0u;
                uint32_t gt = 0, ge = 0;
                for (uint32_t j = 0; j < nc; ++j) {
                    const uint32_t o = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mine), static_cast<int>(j)));
                    gt += o > mine ? 1u : 0u;
                    ge += o >= mine ? 1u : 0u;
                }
                const bool thr = static_cast<uint32_t>(lane) < nc && gt < need && need <= ge;
                const uint64_t m = __ballot(thr);
                if (m && lane == static_cast<int>(__builtin_ctzll(m))) {
                    sm.prm[2] = mine;
                    sm.prm[3] = gt;
                    sm.prm[5] = ge - gt;
                }
            }
            lds_barrier();
            rlo = rhi = sm.prm[2];
            need -= sm.prm[3];
            cand = sm.prm[5];
        };
        if (kSaveBins && value_mode && cand <= kFastCand) {  // block-uniform
            // the saved bins name the threshold bin's keys (saved bins imply one register-resident
            // chunk); one wave-uniform branch per group of four elements
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
                bool in[4];
                uint64_t any = 0;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    in[c] = kbin[kSaveBins ? 4 * g + c : 0] == bstar;
                    any |= __ballot(in[c]);
                }
                if (any) {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (in[c]) sm.cbuf[atomicAdd(&sm.prm[4], 1u)] = key[4 * g + c];
                }
            }
            lds_barrier();
            resolve_small_bin();
        } else if (value_mode) {
            if (wave == 0) {
                uint32_t klo, khi;
                value_bin_key_range(rlo, rhi, static_cast<int>(bstar), scale, off, &klo, &khi);
                if (lane == 0) {
                    sm.prm[2] = klo;
                    sm.prm[3] = khi;
                }
            }
            lds_barrier();
            rlo = sm.prm[2];
            rhi = sm.prm[3];
            if (!STREAM && cand <= kFastCand) {  // block-uniform
                // Register-resident row without saved bins: the threshold bin is exactly the
                // key range [rlo, rhi] (the bin map is monotone), so one compare per element
                // gathers its keys -- cheaper than recomputing every element's bin, and than a
                // refinement level over the range.  The gathered count must equal the bin's
                // count; if it does not (it always should), the refinement levels below run.
                // (k in [rlo, rhi]; absent keys (0) never are.)  One wave-uniform branch per
                // group of four elements: almost every group holds none of the bin's keys.
#pragma unroll
                for (int g = 0; g < kGroups; ++g) {
                    bool in[4];
                    uint64_t any = 0;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        in[c] = key[4 * g + c] - rlo <= rhi - rlo;
                        any |= __ballot(in[c]);
                    }
                    if (any) {
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            if (in[c]) {
                                const uint32_t i = atomicAdd(&sm.prm[4], 1u);
                                if (i < kFastCand) sm.cbuf[i] = key[4 * g + c];
                            }
                        }
                    }
                }
                lds_barrier();
                if (sm.prm[4] == cand) resolve_small_bin();  // block-uniform
            }
        } else {
            const uint64_t nlo = static_cast<uint64_t>(rlo) + (static_cast<uint64_t>(bstar) << sh);
            const uint64_t nhi = nlo + ((1ull << sh) - 1);
            rlo = static_cast<uint32_t>(nlo);
            rhi = nhi < rhi ? static_cast<uint32_t>(nhi) : rhi;
            lds_barrier();
        }
    }

    // ---- refinement levels on the key bits (each level narrows the range by 2^11, so three
    // levels always reach a single key; the bound only guards against a broken invariant)
    for (int level = 0; level < 4 && cand != need && rlo != rhi; ++level) {
        const int sh = shift_for(rhi - rlo);
        for (int i = tid; i < kBins; i += kTopkThreads) sm.hist[i] = 0;
        lds_barrier();
        for (int ch = 0; ch < n_chunks; ++ch) {
            if (STREAM) load(ch);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const uint32_t k = key[e];
                if (k - rlo <= rhi - rlo) atomicAdd(&sm.hist[(k - rlo) >> sh], 1u);  // k in [rlo, rhi]
            }
        }
        lds_barrier();
        find_threshold_bin(sm, need);
        const uint32_t bstar = sm.prm[0];
        need -= sm.prm[1];
        cand = sm.hist[bstar];
        const uint64_t nlo = static_cast<uint64_t>(rlo) + (static_cast<uint64_t>(bstar) << sh);
        const uint64_t nhi = nlo + ((1ull << sh) - 1);
        rlo = static_cast<uint32_t>(nlo);
        rhi = nhi < rhi ? static_cast<uint32_t>(nhi) : rhi;
        lds_barrier();
    }

    // ---- ordered compaction.  "Above" keys are taken outright: every key above the final
    // range, plus the whole range when it is taken whole (cand == need).  Otherwise the range
    // is the single key rlo and its "tie" keys are taken in position order until `need` of
    // them are in.  The output slot of a selected element is
    //   #above before it + min(#ties before it, need);
    // the row is staged in LDS (over the histogram) and copied out at the end.
    // (Keys never exceed the key of +inf, so rlo + 1 does not wrap.)
    const bool take_all = (cand == need);
    const uint32_t above_min = take_all ? rlo : rlo + 1u;  // keys >= this are "above"
    const uint32_t tie_key = take_all ? 0xFFFFFFFFu : rlo;  // never a key when take_all
    if constexpr (!STREAM) {
        // Register-resident row: selection bitmaps in LDS, one bit per position (word p / 32,
        // bit p % 32).  A lane's four consecutive positions of group g form a 4-bit mask; the
        // eight lanes of an octet cover one 32-bit word, which three DPP ORs assemble.  A
        // popcount scan over the words (in position order) then ranks every selected position:
        // first the tie bitmap keeps its first `need` bits, then the union is ranked.
        constexpr int kWords = 32 * E;                       // words of the row
        constexpr int kWpt = kWords >= kTopkThreads ? kWords / kTopkThreads : 1;  // words per thread
        const bool ties = !take_all;                          // block-uniform
        const uint32_t amin2 = above_min, tkey2 = tie_key;
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            uint32_t ma = 0u, mt = 0u;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                ma |= (key[4 * g + c] >= amin2 ? 1u : 0u) << c;
                mt |= (key[4 * g + c] == tkey2 ? 1u : 0u) << c;
            }
            const int sh = 4 * (lane & 7);
            uint32_t wa = ma << sh, wt = mt << sh;
            wa |= dpp_u32<kDppQuadXor1>(0u, wa);
            wa |= dpp_u32<kDppQuadXor2>(0u, wa);
            wa |= dpp_u32<kDppRowHalfMirror>(0u, wa);
            const int widx = 2 * E * wave + 8 * g + (lane >> 3);
            if ((lane & 7) == 0) sm.bm[0][widx] = wa;
            if (ties) {
                wt |= dpp_u32<kDppQuadXor1>(0u, wt);
                wt |= dpp_u32<kDppQuadXor2>(0u, wt);
                wt |= dpp_u32<kDppRowHalfMirror>(0u, wt);
                if ((lane & 7) == 0) sm.bm[1][widx] = wt;
            }
        }
        if constexpr (PRE) {
            // the keys are in the bitmaps and their registers free: load the next row's groups
            // that are not in LDS; they arrive during the ranking below
#pragma unroll
            for (int g = kPreGroups; g < kGroups; ++g) {
                const int64_t base = static_cast<int64_t>(wave) * 64 * E + 256 * g;
                // (assigned on every path, so no earlier value stays live through a row)
                nxt[g - kPreGroups] = next_row && base + 256 <= n_next  // wave-uniform
                    ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(next_row + base + 4 * lane))
                    : f32x4{0.f, 0.f, 0.f, 0.f};
            }
            *nxt_issued = true;
        }
        lds_barrier();
        // this thread's words, in position order
        const int w0 = tid * kWpt;
        const bool owns = w0 < kWords;
        uint32_t sel[kWpt];
#pragma unroll
        for (int k = 0; k < kWpt; ++k) sel[k] = owns ? sm.bm[0][w0 + k] : 0u;
        if (ties) {  // keep the first `need` tie bits in position order
            uint32_t tw[kWpt];
            uint32_t tc = 0;
#pragma unroll
            for (int k = 0; k < kWpt; ++k) {
                tw[k] = owns ? sm.bm[1][w0 + k] : 0u;
                tc += static_cast<uint32_t>(__popc(tw[k]));
            }
            uint32_t ttot;
            uint32_t before = block_exclusive_scan(sm, tc, &ttot);
#pragma unroll
            for (int k = 0; k < kWpt; ++k) {
                uint32_t x = tw[k];
                while (x) {  // drop bits from the lowest once `need` ties are in
                    const uint32_t bit = x & (0u - x);
                    if (before >= need) tw[k] &= ~bit;
                    ++before;
                    x &= x - 1u;
                }
                sel[k] |= tw[k];
            }
        }
        uint32_t cnt = 0;
#pragma unroll
        for (int k = 0; k < kWpt; ++k) cnt += static_cast<uint32_t>(__popc(sel[k]));
        uint32_t stot;
        uint32_t rank = block_exclusive_scan(sm, cnt, &stot);
#pragma unroll
        for (int k = 0; k < kWpt; ++k) {
            uint32_t x = sel[k];
            while (x) {
                const int p = 32 * (w0 + k) + __builtin_ctz(x);
                int32_t v = p;
                if constexpr (MODE == kMerge) {
                    const int q = p / kTopK;
                    const int32_t local = cands[(static_cast<int64_t>(t) * parts + q) * kTopK + (p - q * kTopK)];
                    v = static_cast<int32_t>(q * chunk + local);
                }
                if (rank < kTopK) sm.hist[rank] = static_cast<uint32_t>(v);
                ++rank;
                x &= x - 1u;
            }
        }
    } else {
        uint32_t above_done = 0, tie_done = 0;  // counts of earlier chunks (block-uniform)
        for (int ch = 0; ch < n_chunks; ++ch) {
            if (STREAM) load(ch);
            uint32_t na = 0, nt = 0;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                na += key[e] >= above_min ? 1u : 0u;
                nt += key[e] == tie_key ? 1u : 0u;
            }
            na = wave_sum_u32(na);
            nt = wave_sum_u32(nt);
            uint32_t* cnt = sm.cnt[ch & 1];
            if (lane == 0) {
                cnt[wave] = na;
                cnt[kTopkWaves + wave] = nt;
            }
            lds_barrier();
            uint32_t a_run = above_done, t_run = tie_done, a_tot = 0, t_tot = 0;
#pragma unroll
            for (int i = 0; i < kTopkWaves; ++i) {
                const uint32_t x = cnt[i], y = cnt[kTopkWaves + i];
                a_run += i < wave ? x : 0u;
                t_run += i < wave ? y : 0u;
                a_tot += x;
                t_tot += y;
            }
            // opaque copies keep the compiler from holding the counting loop's 2E lane masks
            // live (in scalar registers) until they are needed again below
            uint32_t amin2 = above_min, tkey2 = tie_key;
            asm volatile("" : "+v"(amin2), "+v"(tkey2));
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
                uint64_t ma[4], mt[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    ma[c] = __ballot(key[4 * g + c] >= amin2);
                    mt[c] = __ballot(key[4 * g + c] == tkey2);
                }
                // counts of this group's elements held by lower lanes, then by this lane's own
                // earlier elements (position order within a group is lane, then c)
                uint32_t ra = a_run, rt = t_run;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    ra = mbcnt64(ma[c], ra);
                    rt = mbcnt64(mt[c], rt);
                }
                const int64_t p0 = ch * kChunk + tbase + 256 * g;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t k = key[4 * g + c];
                    const bool ia = k >= amin2, it = k == tkey2;
                    const uint32_t rank = ra + (rt < need ? rt : need);
                    if ((ia || (it && rt < need)) && rank < kTopK) {
                        if constexpr (MODE == kMerge)
                            sm.hist[rank] = static_cast<uint32_t>(cpos[4 * g + c]);
                        else
                            sm.hist[rank] = static_cast<uint32_t>(p0 + c);
                    }
                    ra += ia ? 1u : 0u;
                    rt += it ? 1u : 0u;
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    a_run += static_cast<uint32_t>(__popcll(ma[c]));
                    t_run += static_cast<uint32_t>(__popcll(mt[c]));
                }
            }
            above_done += a_tot;
            tie_done += t_tot;
        }
    }
    // the ranks fill the staging row once each; it leaves in two coalesced stores per thread
    // (scattered 4-byte stores straight to global memory measured slightly slower)
    lds_barrier();
#pragma unroll
    for (int i = static_cast<int>(threadIdx.x); i < kTopK; i += kTopkThreads) {
        const int32_t v = static_cast<int32_t>(sm.hist[i]);
        out[i] = v;
        // a part hands the merge its candidates' keys too (two loads per thread from the part's
        // scores, just read, so in the L2), sparing the merge 2048 * parts scattered reads
        if constexpr (MODE == kParts) cand_keys[ob * kTopK + i] = score_key(row[v]);
    }
}

// One block per row (or part); PRE: a persistent grid of one block per CU, block b taking
// rows b, b + grid, ... of the n_rows rows.  No block waits for another, so results do not
// depend on how many blocks are resident at once.
template <int E, bool STREAM, bool VEC, int MODE, bool PRE>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const float* __restrict__ scores, int64_t ld, const RowLens rl, int32_t* __restrict__ ids,
    int32_t parts, int64_t chunk, const int32_t* __restrict__ cands, uint32_t* __restrict__ cand_keys,
    int32_t n_rows) {
    __shared__ TopkSmem sm;
    if constexpr (!PRE) {
        const int b = static_cast<int>(blockIdx.x);
        const int t = MODE == kParts ? b / parts : b;
        const int part = MODE == kParts ? b - t * parts : 0;
        topk_select<E, STREAM, VEC, MODE, false>(sm, t, part, b, scores, ld, rl, ids, parts,
                                                 chunk, cands, cand_keys,
                                                 nullptr, false, nullptr, 0, nullptr, false,
                                                 nullptr);
    } else {
        __shared__ f32x4 pre[kTopkWaves * kPreGroups * 64];
        f32x4 nxt[E / 4 - kPreGroups];  // the next row's later groups, loaded into registers
        bool nxt_rd = false;
        const int step = static_cast<int>(gridDim.x);
        for (int t = static_cast<int>(blockIdx.x); t < n_rows; t += step) {
            const bool has_pre = t != static_cast<int>(blockIdx.x);  // block-uniform
            if (has_pre) {
                wait_vmcnt<0>();                      // this wave's copies (and loads) of row t have landed
                __asm__ volatile("" ::: "memory");  // (no LDS read moves above the wait)
                lds_barrier();                        // the previous row's last LDS reads are done
            }
            const int tn = t + step;
            const float* next = tn < n_rows ? scores + static_cast<int64_t>(tn) * ld : nullptr;
            const int64_t n_next = next ? topk_row_len(tn, rl) : 0;
            bool issued = false;
            topk_select<E, STREAM, VEC, MODE, true>(sm, t, 0, t, scores, ld, rl, ids, parts,
                                                    chunk, cands, cand_keys, pre, has_pre, next, n_next, nxt,
                                                    has_pre && nxt_rd, &issued);
            nxt_rd = issued;
        }
    }
}

// ---- rows of 65537 .. 2^20 elements ------------------------------------------------------
// Streamed once per radix level (statistics, level 0, refinements, compaction), such a row
// is read five or more times.  Here it is read about 1.1 times:
//  pass 1   the max key of every segment of `seg` consecutive positions goes to LDS (seg = 8 ..
//           64, the smallest power of two that leaves at most 16384 segments: 8193 .. 16384);
//  theta    a value-linear histogram level over the segment maxima (then key-bit levels while
//           its threshold bin is wide) gives a key theta such that at least 2048 and at most
//           kSelSegs segments have a maximum >= theta.  Each such
//           segment holds an element >= theta, so at least 2048 elements are >= theta: the
//           row's top-2048 lies among them, and all of them lie in those segments;
//  pass 2   those segments (about 2048: an eighth of a 2^20 row at seg 64) are read again and
//           their elements >= theta gathered in LDS as (key, list position), where a list
//           position is the segment's index in the ascending segment list times seg plus the
//           offset inside the segment -- ascending list position is ascending row position;
//  select   radix levels over the gathered keys (in registers) find the exact threshold key;
//           selection bitmaps indexed by list position are ranked by a popcount scan, ties at
//           the threshold taken in position order, as in the register-resident path.
// Rows whose maxima are flat (more than kSelSegs segments at or above theta, e.g. many equal
// scores) or that gather more than kCandCap candidates fall back to the streamed selection,
// as do rows longer than 2^20; rows of at most 65536 elements take the register path.
constexpr int kSegSlots = 16384;  // segment maxima of one row
constexpr int kSelSegs = 4096;    // segments read in pass 2
constexpr int kCandCap = 8192;    // gathered candidates
constexpr int64_t kLongMaxN = static_cast<int64_t>(kSegSlots) * 64;
constexpr int kLongBatch = 8;     // 1 KB loads in flight per wave
// Launches for longer rows take this path.  Register-resident rows select faster: 64 rows of
// 32768 took 47 us here against 29 us, 4096 rows of up to 65536 took 727 us against 412 us.
constexpr int64_t kLongMinLaunch = 64 * kTopkThreads;

struct LongSmem {
    uint32_t hist[kBins];  // histogram; at the end the output row being staged
    uint32_t wtot[kTopkWaves];
    uint32_t red[4][kTopkWaves];
    uint32_t prm[8];
    union {
        uint32_t segmax[kSegSlots];          // pass 1: max key per segment
        uint32_t bm[2][kSelSegs * 64 / 32];  // (above, tie) bits by list position
    };
    uint32_t seglist[kSelSegs];  // segments with maximum >= theta, ascending
    uint32_t ckey[kCandCap];     // gathered keys ...
    uint32_t cpos[kCandCap];     // ... and their list positions
};
static_assert(sizeof(LongSmem) <= 160 * 1024, "fits the LDS of one CU");

// Max over aligned groups of 2^lg lanes (lg = 0 .. 4, block-uniform); every lane of a group
// receives the group's maximum.
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v, int lg) {
    if (lg >= 1) v = max(v, dpp_u32<kDppQuadXor1>(v, v));
    if (lg >= 2) v = max(v, dpp_u32<kDppQuadXor2>(v, v));
    if (lg >= 3) v = max(v, dpp_u32<kDppRowHalfMirror>(v, v));
    if (lg >= 4) v = max(v, dpp_u32<kDppRowMirror>(v, v));
    return v;
}

// Keys of positions p .. p+3 of a row of n elements (0 for positions >= n), element by element.
__device__ __forceinline__ u32x4 keys4_guarded(const float* row, int64_t p, int64_t n) {
    u32x4 k;
#pragma unroll
    for (int c = 0; c < 4; ++c) k[c] = p + c < n ? score_key(row[p + c]) : 0u;
    return k;
}

template <bool VEC, bool NT>
__device__ __forceinline__ u32x4 keys4(const float* row, int64_t p) {
    u32x4 k;
    if constexpr (VEC) {
        const f32x4* a = reinterpret_cast<const f32x4*>(row + p);
        const f32x4 v = NT ? __builtin_nontemporal_load(a) : *a;
#pragma unroll
        for (int c = 0; c < 4; ++c) k[c] = score_key(v[c]);
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) k[c] = score_key(row[p + c]);
    }
    return k;
}

// Selection of a row (kRow) or part (kParts) of n elements, 65536 < n <= 2^20; false (the
// block-uniform verdict) when the row must take the streamed selection instead.
template <int MODE, bool VEC>
__device__ __forceinline__ bool long_select(LongSmem& sm, const float* __restrict__ row, const int64_t n,
                            int32_t* __restrict__ out, uint32_t* __restrict__ out_keys) {
    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // log2 of lanes per segment: the smallest segments (4 << lg positions) that give at most
    // kSegSlots segments
    int lg = 0;
    while (n > (static_cast<int64_t>(kSegSlots) * 4 << lg)) ++lg;
    const int seg_sh = lg + 2;                                   // log2(seg)
    const int nseg = static_cast<int>((n + (1 << seg_sh) - 1) >> seg_sh);

    // ---- pass 1: one 1 KB load instruction covers positions 256u .. 256u + 255
    const int n_ins = static_cast<int>((n + 255) >> 8);
    const int n_full = static_cast<int>(n >> 8);  // instructions wholly inside the row
    auto emit = [&](int u, const u32x4 k) {
        const uint32_t m = group_max_u32(max(max(k[0], k[1]), max(k[2], k[3])), lg);
        if ((lane & ((1 << lg) - 1)) == 0) sm.segmax[(256 * u + 4 * lane) >> seg_sh] = m;
    };
    int u = wave;
    for (; u + (kLongBatch - 1) * kTopkWaves < n_full; u += kLongBatch * kTopkWaves) {
        u32x4 k[kLongBatch];
#pragma unroll
        for (int j = 0; j < kLongBatch; ++j)
            k[j] = keys4<VEC, true>(row, 256 * static_cast<int64_t>(u + j * kTopkWaves) + 4 * lane);
#pragma unroll
        for (int j = 0; j < kLongBatch; ++j) emit(u + j * kTopkWaves, k[j]);
    }
    for (; u < n_ins; u += kTopkWaves)  // the last instructions, the partial one included
        emit(u, keys4_guarded(row, 256 * static_cast<int64_t>(u) + 4 * lane, n));
    lds_barrier();

    // ---- theta: thread i holds the maxima of segments 16i .. 16i + 15
    uint32_t sk[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int s = 16 * tid + i;
        sk[i] = s < nseg ? sm.segmax[s] : 0u;  // every segment below nseg holds an element
    }
    uint32_t amin = ~0u, amax = 0u, fmin = ~0u, fmax = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t k = sk[i];
        amin = min(amin, k - 1u);  // absent (0) wraps to the top
        amax = max(amax, k);
        if (k > kKeyNegInf && k < kKeyPosInf) {
            fmin = min(fmin, k);
            fmax = max(fmax, k);
        }
    }
    for (int i = tid; i < kBins; i += kTopkThreads) sm.hist[i] = 0;  // ordered by the barriers below
    if (tid == 0) sm.prm[4] = 0u;                                     // gathered candidates
    block_minmax(sm, amin, amax, fmin, fmax);
    amin += 1u;
    bool value_mode = false;
    float scale = 0.f, off = 0.f;
    if (fmin < fmax) {
        const float lo = key_to_score(fmin);
        scale = static_cast<float>(kBins) / (key_to_score(fmax) - lo);
        off = -lo * scale;
        value_mode = isfinite(scale) && scale > 0.f && isfinite(off);
    }
    const int ksh = value_mode ? 0 : shift_for(amax - amin);
    auto bin_of = [&](uint32_t k) {
        return value_mode ? value_bin(k, scale, off) : static_cast<int>((k - amin) >> ksh);
    };
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (sk[i]) atomicAdd(&sm.hist[bin_of(sk[i])], 1u);
    lds_barrier();
    find_threshold_bin(sm, kTopK);  // more than 8192 maxima, so the bin exists
    const int bstar = static_cast<int>(sm.prm[0]);
    uint32_t above = sm.prm[1];     // maxima above the threshold bin
    uint32_t cand = sm.hist[bstar];  // maxima in it
    uint32_t rlo, rhi;               // key range of the threshold bin
    if (value_mode) {                // block-uniform: the keys present in the bin
        rlo = ~0u;
        rhi = 0u;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (sk[i] && bin_of(sk[i]) == bstar) {
                rlo = min(rlo, sk[i]);
                rhi = max(rhi, sk[i]);
            }
        uint32_t d0 = ~0u, d1 = 0u;
        block_minmax(sm, rlo, rhi, d0, d1);
    } else {
        const uint64_t lo = static_cast<uint64_t>(amin) + (static_cast<uint64_t>(bstar) << ksh);
        const uint64_t hi = lo + ((1ull << ksh) - 1);
        rlo = static_cast<uint32_t>(lo);
        rhi = hi < amax ? static_cast<uint32_t>(hi) : amax;
        lds_barrier();  // (hist read above)
    }
    // Keys >= rlo number above + cand.  A wide threshold bin (flat or heavy-tailed maxima) is
    // narrowed by key-bit levels until at most kSelSegs segments remain or it is one key.
    uint32_t need = kTopK - above;
    for (int level = 0; level < 4 && above + cand > static_cast<uint32_t>(kSelSegs) && rlo != rhi;
         ++level) {
        const int sh = shift_for(rhi - rlo);
        for (int i = tid; i < kBins; i += kTopkThreads) sm.hist[i] = 0;
        lds_barrier();
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (sk[i] - rlo <= rhi - rlo) atomicAdd(&sm.hist[(sk[i] - rlo) >> sh], 1u);
        lds_barrier();
        find_threshold_bin(sm, need);
        const uint32_t bs = sm.prm[0];
        above += sm.prm[1];
        need -= sm.prm[1];
        cand = sm.hist[bs];
        const uint64_t nlo = static_cast<uint64_t>(rlo) + (static_cast<uint64_t>(bs) << sh);
        const uint64_t nhi = nlo + ((1ull << sh) - 1);
        rlo = static_cast<uint32_t>(nlo);
        rhi = nhi < rhi ? static_cast<uint32_t>(nhi) : rhi;
        lds_barrier();
    }
    if (above + cand > static_cast<uint32_t>(kSelSegs)) return false;  // block-uniform
    const uint32_t theta = rlo;  // >= 1: the range holds present maxima only
    // (at least 2048 maxima are >= theta, each the key of an element of its segment)

    // ---- the segment list, in ascending segment order
    uint32_t flags = 0u, nf = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const bool f = sk[i] >= theta;  // theta >= 1: absent maxima never pass
        flags |= (f ? 1u : 0u) << i;
        nf += f ? 1u : 0u;
    }
    uint32_t nsel;  // == above + cand
    uint32_t slot = block_exclusive_scan(sm, nf, &nsel);  // (all segmax reads are done)
    if (nsel > static_cast<uint32_t>(kSelSegs)) return false;  // (never: a guard only)
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if ((flags >> i) & 1u) sm.seglist[slot++] = static_cast<uint32_t>(16 * tid + i);
    const int n_words = static_cast<int>(((nsel << seg_sh) + 31) >> 5);
    for (int i = tid; i < n_words; i += kTopkThreads) {
        sm.bm[0][i] = 0u;
        sm.bm[1][i] = 0u;
    }
    lds_barrier();

    // ---- pass 2: instruction w covers list entries spi*w .. spi*w + spi - 1 (spi segments of
    // 2^lg lanes each); lanes past the list, and a partial last segment, are handled apart
    const int spi = 64 >> lg;
    const int n_ins2 = static_cast<int>((nsel + spi - 1) / spi);
    const int my_off = 4 * (lane & ((1 << lg) - 1));
    for (int w = wave; w < n_ins2; w += kLongBatch * kTopkWaves) {
        u32x4 k[kLongBatch];
        int pos[kLongBatch];
        bool part[kLongBatch];
#pragma unroll
        for (int j = 0; j < kLongBatch; ++j) {
            const int e = spi * (w + j * kTopkWaves) + (lane >> lg);
            const bool in = e < static_cast<int>(nsel);
            pos[j] = in ? (static_cast<int>(sm.seglist[e]) << seg_sh) + my_off : -1;
            const bool whole = in && pos[j] + 3 < n;
            part[j] = in && !whole;
            // lanes without a whole group read the row's first group (in bounds) and discard it
            k[j] = keys4<VEC, false>(row, whole ? pos[j] : 0);
            if (!whole) k[j] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < kLongBatch; ++j) {
            if (part[j]) k[j] = keys4_guarded(row, pos[j], n);
            uint64_t m[4];
            uint32_t cnt = 0u;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                m[c] = __ballot(k[j][c] >= theta);  // (absent elements are 0 < theta)
                cnt += static_cast<uint32_t>(__popcll(m[c]));
            }
            if (cnt == 0u) continue;  // wave-uniform
            uint32_t base = 0u;
            if (lane == 0) base = atomicAdd(&sm.prm[4], cnt);
            base = __builtin_amdgcn_readfirstlane(base);
            const uint32_t lp0 = static_cast<uint32_t>(spi * (w + j * kTopkWaves) + (lane >> lg)) << seg_sh;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t at = mbcnt64(m[c], base);
                if (((m[c] >> lane) & 1u) && at < static_cast<uint32_t>(kCandCap)) {
                    sm.ckey[at] = k[j][c];
                    sm.cpos[at] = lp0 + static_cast<uint32_t>(my_off + c);
                }
                base += static_cast<uint32_t>(__popcll(m[c]));
            }
        }
    }
    lds_barrier();
    const uint32_t n_cand = sm.prm[4];  // >= nsel >= 2048: each listed segment gives its maximum
    if (n_cand > static_cast<uint32_t>(kCandCap)) return false;  // block-uniform

    // ---- the exact threshold among the candidates (thread i holds candidates i + 1024 j)
    constexpr int kCpt = kCandCap / kTopkThreads;
    uint32_t kc[kCpt];
    rlo = ~0u;
    rhi = 0u;
#pragma unroll
    for (int j = 0; j < kCpt; ++j) {
        const uint32_t i = static_cast<uint32_t>(tid + kTopkThreads * j);
        kc[j] = i < n_cand ? sm.ckey[i] : 0u;
        rlo = min(rlo, kc[j] - 1u);
        rhi = max(rhi, kc[j]);
    }
    {
        uint32_t d0 = ~0u, d1 = 0u;
        block_minmax(sm, rlo, rhi, d0, d1);
    }
    rlo += 1u;
    need = kTopK;
    cand = n_cand;
    for (int level = 0; level < 4 && cand != need && rlo != rhi; ++level) {
        const int sh = shift_for(rhi - rlo);
        for (int i = tid; i < kBins; i += kTopkThreads) sm.hist[i] = 0;
        lds_barrier();
#pragma unroll
        for (int j = 0; j < kCpt; ++j)
            if (kc[j] - rlo <= rhi - rlo) atomicAdd(&sm.hist[(kc[j] - rlo) >> sh], 1u);  // in [rlo, rhi]
        lds_barrier();
        find_threshold_bin(sm, need);
        const uint32_t bs = sm.prm[0];
        need -= sm.prm[1];
        cand = sm.hist[bs];
        const uint64_t nlo = static_cast<uint64_t>(rlo) + (static_cast<uint64_t>(bs) << sh);
        const uint64_t nhi = nlo + ((1ull << sh) - 1);
        rlo = static_cast<uint32_t>(nlo);
        rhi = nhi < rhi ? static_cast<uint32_t>(nhi) : rhi;
        lds_barrier();
    }
    // keys above the final range are taken, the range too when taken whole (cand == need);
    // else it is the single key rlo, of which the first `need` in position order are taken
    const bool take_all = cand == need;
    const uint32_t above_min = take_all ? rlo : rlo + 1u;
    const uint32_t tie_key = take_all ? 0xFFFFFFFFu : rlo;  // never a key when take_all
#pragma unroll
    for (int j = 0; j < kCpt; ++j) {
        const uint32_t i = static_cast<uint32_t>(tid + kTopkThreads * j);
        if (i < n_cand) {
            const uint32_t lp = sm.cpos[i];
            if (kc[j] >= above_min) atomicOr(&sm.bm[0][lp >> 5], 1u << (lp & 31));
            else if (kc[j] == tie_key) atomicOr(&sm.bm[1][lp >> 5], 1u << (lp & 31));
        }
    }
    lds_barrier();

    // ---- ranking: thread i owns bitmap words 8i .. 8i + 7 (list-position order)
    constexpr int kWpt = kSelSegs * 64 / 32 / kTopkThreads;
    const int w0 = kWpt * tid;
    uint32_t sel[kWpt];
#pragma unroll
    for (int q = 0; q < kWpt; ++q) sel[q] = w0 + q < n_words ? sm.bm[0][w0 + q] : 0u;
    if (!take_all) {  // block-uniform: keep the first `need` tie bits
        uint32_t tw[kWpt], tc = 0u, ttot;
#pragma unroll
        for (int q = 0; q < kWpt; ++q) {
            tw[q] = w0 + q < n_words ? sm.bm[1][w0 + q] : 0u;
            tc += static_cast<uint32_t>(__popc(tw[q]));
        }
        uint32_t before = block_exclusive_scan(sm, tc, &ttot);
#pragma unroll
        for (int q = 0; q < kWpt; ++q) {
            uint32_t x = tw[q];
            while (x) {
                const uint32_t low = x & (0u - x);
                if (before >= need) tw[q] &= ~low;
                ++before;
                x &= x - 1u;
            }
            sel[q] |= tw[q];
        }
    }
    uint32_t cnt = 0u, stot;
#pragma unroll
    for (int q = 0; q < kWpt; ++q) cnt += static_cast<uint32_t>(__popc(sel[q]));
    uint32_t rank = block_exclusive_scan(sm, cnt, &stot);  // stot == 2048
    const uint32_t seg_mask = (1u << seg_sh) - 1u;
#pragma unroll
    for (int q = 0; q < kWpt; ++q) {
        uint32_t x = sel[q];
        while (x) {
            const uint32_t lp = 32u * static_cast<uint32_t>(w0 + q) + static_cast<uint32_t>(__builtin_ctz(x));
            const uint32_t p = (sm.seglist[lp >> seg_sh] << seg_sh) + (lp & seg_mask);
            if (rank < kTopK) sm.hist[rank] = p;
            ++rank;
            x &= x - 1u;
        }
    }
    lds_barrier();
#pragma unroll
    for (int i = tid; i < kTopK; i += kTopkThreads) {
        const int32_t v = static_cast<int32_t>(sm.hist[i]);
        out[i] = v;
        if constexpr (MODE == kParts) out_keys[i] = v >= 0 && v < n ? score_key(row[v]) : 0u;
    }
    return true;
}

// One block per row (or part) of a launch whose rows hold up to 2^20 elements.
template <int MODE, bool VEC>
__global__ __launch_bounds__(kTopkThreads) void topk_long_kernel(
    const float* __restrict__ scores, int64_t ld, const RowLens rl, int32_t* __restrict__ ids,
    int32_t parts, int64_t chunk, uint32_t* __restrict__ cand_keys) {
    __shared__ union {
        TopkSmem ts;
        LongSmem ls;
    } sm;
    const int b = static_cast<int>(blockIdx.x);
    const int t = MODE == kParts ? b / parts : b;
    const int part = MODE == kParts ? b - t * parts : 0;
    int64_t n = topk_row_len(t, rl);
    if (MODE == kParts) {
        n -= part * chunk;
        n = n < chunk ? n : chunk;
        n = n > 0 ? n : 0;
    }
    if (n <= 64 * kTopkThreads) {  // (the register path is faster for such rows)
        topk_select<64, false, VEC, MODE, false>(sm.ts, t, part, b, scores, ld, rl, ids, parts, chunk,
                                                 nullptr, cand_keys, nullptr, false, nullptr, 0,
                                                 nullptr, false, nullptr);
        return;
    }
    const float* row = scores + static_cast<int64_t>(t) * ld + (MODE == kParts ? part * chunk : 0);
    if (n <= kLongMaxN &&
        long_select<MODE, VEC>(sm.ls, row, n, ids + static_cast<int64_t>(b) * kTopK,
                               cand_keys ? cand_keys + static_cast<int64_t>(b) * kTopK : nullptr))
        return;
    lds_barrier();  // the fast path's last LDS reads are done
    topk_select<16, true, VEC, MODE, false>(sm.ts, t, part, b, scores, ld, rl, ids, parts, chunk,
                                            nullptr, cand_keys, nullptr, false, nullptr, 0, nullptr,
                                            false, nullptr);
}

template <int E, bool STREAM, int MODE>
static void launch_topk_e(unsigned blocks, const float* scores, int64_t ld, const RowLens& rl,
                          int32_t* ids, int32_t parts, int64_t chunk, const int32_t* cands,
                          uint32_t* cand_keys, bool vec, hipStream_t stream) {
    if (vec)
        hipLaunchKernelGGL((topk_kernel<E, STREAM, true, MODE, false>), dim3(blocks),
                           dim3(kTopkThreads), 0, stream, scores, ld, rl, ids, parts, chunk,
                           cands, cand_keys, 0);
    else
        hipLaunchKernelGGL((topk_kernel<E, STREAM, false, MODE, false>), dim3(blocks),
                           dim3(kTopkThreads), 0, stream, scores, ld, rl, ids, parts, chunk,
                           cands, cand_keys, 0);
}

// Compute units of the current device (the persistent grid size, and the grid bound of the
// LayerNorm and FP8 cache fills), looked up once per device (threads that race on the first
// lookup store the same value).
int device_cus() {
    static std::atomic<int> cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// One selection pass over rows (or parts) of at most `len` elements each.
template <int MODE>
static void launch_pass(unsigned blocks, int64_t len, const float* scores, int64_t ld,
                        const RowLens& rl, int32_t* ids, int32_t parts, int64_t chunk,
                        uint32_t* cand_keys, bool vec, hipStream_t stream) {
    if (len <= 4 * kTopkThreads)
        launch_topk_e<4, false, MODE>(blocks, scores, ld, rl, ids, parts, chunk, nullptr, cand_keys, vec, stream);
    else if (len <= 8 * kTopkThreads)
        launch_topk_e<8, false, MODE>(blocks, scores, ld, rl, ids, parts, chunk, nullptr, cand_keys, vec, stream);
    else if (len <= 16 * kTopkThreads)
        launch_topk_e<16, false, MODE>(blocks, scores, ld, rl, ids, parts, chunk, nullptr, cand_keys, vec, stream);
    else if (len > kLongMinLaunch && len <= kLongMaxN && vec)
        hipLaunchKernelGGL((topk_long_kernel<MODE, true>), dim3(blocks), dim3(kTopkThreads), 0,
                           stream, scores, ld, rl, ids, parts, chunk, cand_keys);
    else if (len <= 32 * kTopkThreads)
        launch_topk_e<32, false, MODE>(blocks, scores, ld, rl, ids, parts, chunk, nullptr, cand_keys, vec, stream);
    else if (len <= 64 * kTopkThreads && MODE == kRow && vec) {
        // persistent blocks with the next row's LDS prefetch (one block per CU)
        const unsigned grid = std::min(blocks, static_cast<unsigned>(device_cus()));
        hipLaunchKernelGGL((topk_kernel<64, false, true, kRow, true>), dim3(grid),
                           dim3(kTopkThreads), 0, stream, scores, ld, rl, ids, parts, chunk,
                           nullptr, nullptr, static_cast<int32_t>(blocks));
    } else if (len <= 64 * kTopkThreads)
        launch_topk_e<64, false, MODE>(blocks, scores, ld, rl, ids, parts, chunk, nullptr, cand_keys, vec, stream);
    else if (len <= kLongMaxN && vec)
        hipLaunchKernelGGL((topk_long_kernel<MODE, true>), dim3(blocks), dim3(kTopkThreads), 0,
                           stream, scores, ld, rl, ids, parts, chunk, cand_keys);
    else if (len <= kLongMaxN)
        hipLaunchKernelGGL((topk_long_kernel<MODE, false>), dim3(blocks), dim3(kTopkThreads), 0,
                           stream, scores, ld, rl, ids, parts, chunk, cand_keys);
    else
        launch_topk_e<16, true, MODE>(blocks, scores, ld, rl, ids, parts, chunk, nullptr, cand_keys, vec, stream);
}

// Parts per row for the two-stage selection: rows are split while fewer than 256 blocks
// would run (one block per CU) and every part keeps at least 65536 elements; at most 16
// parts.  A selection pass has a large fixed cost (block-wide scans, barriers and dependent
// LDS round trips), so splitting shorter rows measured slower: 64 rows of 32768 in four parts
// of 8192 plus the merge took 12 us longer than one pass per row.
int topk_parts(int32_t T, int64_t max_n) {
    int p = 1;
    while (p < 16 && static_cast<int64_t>(T) * p < 256 && max_n >= static_cast<int64_t>(p) * 2 * 65536) p *= 2;
    return p;
}

// Candidate lists of a split selection: positions [T * parts, 2048] int32, then their keys
// [T * parts, 2048] u32.
size_t topk_workspace_bytes(int32_t T, int64_t max_n) {
    const int p = topk_parts(T, max_n);
    return p > 1 ? static_cast<size_t>(T) * p * kTopK * 2 * sizeof(int32_t) : 0;
}

// Either n_valid (explicit row lengths) or (kv_off, q_req, q_pos) of B requests gives each
// row's length.  With a candidate workspace (topk_workspace_bytes) rows may be split into parts.
hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* n_valid,
                       const int64_t* kv_off, const int32_t* q_req, const int32_t* q_pos,
                       int32_t B, int32_t T, int64_t max_n, int32_t* ids, hipStream_t stream,
                       int32_t* cand_ws) {
    const RowLens rl{n_valid, kv_off, q_req, q_pos, max_n, B};
    const bool vec = (reinterpret_cast<uintptr_t>(scores) % 16 == 0) && (ld % 4 == 0);
    const int parts = cand_ws ? topk_parts(T, max_n) : 1;
    if (parts == 1) {
        launch_pass<kRow>(static_cast<unsigned>(T), max_n, scores, ld, rl, ids, 1, 0, nullptr, vec,
                          stream);
        return hipGetLastError();
    }
    // parts start 16-byte aligned: chunk is a multiple of 4096 elements
    int64_t chunk = (max_n + parts - 1) / parts;
    chunk = (chunk + 4095) & ~static_cast<int64_t>(4095);
    uint32_t* cand_keys = reinterpret_cast<uint32_t*>(cand_ws + static_cast<int64_t>(T) * parts * kTopK);
    launch_pass<kParts>(static_cast<unsigned>(T * parts), chunk, scores, ld, rl, cand_ws, parts,
                        chunk, cand_keys, vec, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned blocks = static_cast<unsigned>(T);
    if (parts == 2)
        launch_topk_e<4, false, kMerge>(blocks, scores, ld, rl, ids, parts, chunk, cand_ws, cand_keys, false, stream);
    else if (parts == 4)
        launch_topk_e<8, false, kMerge>(blocks, scores, ld, rl, ids, parts, chunk, cand_ws, cand_keys, false, stream);
    else if (parts == 8)
        launch_topk_e<16, false, kMerge>(blocks, scores, ld, rl, ids, parts, chunk, cand_ws, cand_keys, false, stream);
    else
        launch_topk_e<32, false, kMerge>(blocks, scores, ld, rl, ids, parts, chunk, cand_ws, cand_keys, false, stream);
    return hipGetLastError();
}

}  // namespace dsa
