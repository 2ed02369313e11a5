// Reduced-precision index-key cache: FP8 (OCP E4M3) keys with one power-of-two scale per
// key row, and the indexer scores over that cache.
//
// Page "Kimi K3.1 Pro: Sparse-Zugriffe, keine kleinere Historie", section "Warum Top-2048
// keinen 2048-Token-Cache bedeutet": index quantisation and scale metadata change the
// physical cache; section "Was ein Deployment validieren muss": cache precision is an
// optional configuration, not a quality-preserving default (no quality is claimed here).
//
// Key row j is stored as 128 E4M3 codes c_jd and a scale 2^e_j, e_j the smallest exponent
// with max_d |k_jd| <= 448 * 2^e_j; c_jd = RNE(k_jd * 2^-e_j).  Scaling by a power of two is
// exact, and the rounding is done by integer operations on the fp32 bits, so the codes are
// reproducible bit for bit anywhere.  The scores use the decoded keys:
//   s_tj = sum_h w_th * max(0, q_th . (2^e_j c_j)) = 2^e_j * sum_h w_th * max(0, q_th . c_j),
// since ReLU commutes with a positive scale: the kernel contracts the exact bf16 images of the
// codes (an E4M3 value has 4 significant bits) and multiplies each score by 2^e_j once.
//
// The scoring stream moves 128 B per key instead of 256 B (plus 4 B of scale), which halves
// the dominant term of a decode step.
#include "common.h"

namespace dsa {

namespace {

// fp32 -> E4M3 code, round to nearest even, for |x| <= 448 (the scale guarantees it).  The sign
// bit is kept (-0 -> 0x80).  Below 2^-6 the code is a multiple of 2^-9 (subnormal codes;
// 8 * 2^-9 is code 0x08, the smallest normal).  Above, the fp32 mantissa is rounded to three
// bits by an integer add (a carry moves into the exponent).
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
    const uint32_t sign = (__float_as_uint(x) >> 31) << 7;
    const float a = fabsf(x);
    uint32_t mag;
    if (a < 0x1p-6f) {
        mag = static_cast<uint32_t>(rintf(a * 512.0f));
    } else {
        const uint32_t ua = __float_as_uint(a);
        const uint32_t r = ua + 0x7FFFFu + ((ua >> 20) & 1u);
        mag = ((((r >> 23) - 127u + 7u) << 3) | ((r >> 20) & 7u));
    }
    return sign | mag;
}

constexpr int kF8Key = kIndexDim;           // bytes per key row
constexpr int kF8Tile = 16;                 // keys per wave step: 2 KB, two 1 KB copies
constexpr int kF8Ring = 3;                  // ring slots per wave (two steps in flight)
constexpr int kF8Copies = kF8Tile / 8;
constexpr int kF8MaxChunk = 4096;           // keys per block at most (their scores: 16 KB)
constexpr int kF8MinChunk = 64;             // one block step (small jobs spread too)

int64_t f8_chunk(int32_t T, int64_t max_s) {
    int64_t c = (static_cast<int64_t>(T) * max_s + 511) / 512;
    c = (c + 63) & ~static_cast<int64_t>(63);
    c = c < kF8MinChunk ? kF8MinChunk : c;
    return c > kF8MaxChunk ? kF8MaxChunk : c;
}

}  // namespace

// A quarter of a wave (16 lanes) per key row: each lane holds eight consecutive bf16 values
// (one 16-byte load) and writes their eight codes (8 bytes); the row maximum is reduced with
// xor-shuffles.  A 256-thread block takes 64 consecutive rows per iteration, four per
// quarter-wave, all loaded before any is encoded; lane j of a quarter-wave keeps the scale of
// its j-th row, so the block's 64 scales leave as two whole 128-byte lines.  Grid-stride over
// rows, non-temporal loads and stores (each key is read once, each code written once).
// 2 M keys cold, codes and scales identical in every variant: half a wave per row (8-byte
// loads, 4-byte code stores, one scale store per row) 193-195 us; a quarter-wave per row 155
// us at two rows in flight per quarter and 16 blocks per CU, 146 us at four rows and 32 blocks
// per CU (kept).
constexpr int kF8FillR = 4;                   // rows per quarter-wave per iteration
constexpr int kF8FillRows = 16 * kF8FillR;    // consecutive rows per 256-thread block and iteration

__global__ __launch_bounds__(256) void quantize_keys_fp8_kernel(const uint16_t* __restrict__ keys,
                                                                int64_t n_rows,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales) {
    const int sub = threadIdx.x & 15;      // elements 8 sub .. 8 sub + 7 of a row
    const int quarter = threadIdx.x >> 4;  // quarter-wave of the block, 0 .. 15
    constexpr int R = kF8FillR;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kF8FillRows; base < n_rows;
         base += static_cast<int64_t>(gridDim.x) * kF8FillRows) {
        const int64_t row0 = base + R * quarter;  // this quarter-wave's rows row0 .. row0 + R - 1
        u32x4 raw[R];
        float my_scale = 0.f;  // lane j < R: the scale of row row0 + j
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int64_t row = row0 + j;
            raw[j] = row < n_rows ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(keys + row * kIndexDim + 8 * sub))
                                  : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int64_t row = row0 + j;
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = __uint_as_float(raw[j][i] << 16);
                x[2 * i + 1] = __uint_as_float(raw[j][i] & 0xFFFF0000u);
            }
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
            for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
            int e = 0;
            if (amax > 0.f) {
                int xe;
                const float f = frexpf(amax, &xe);  // amax = f * 2^xe, f in [0.5, 1)
                e = (xe - 1) - 8 + (f > 0.875f ? 1 : 0);
            }
            u32x2 packed = {0u, 0u};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                packed[0] |= e4m3_encode(ldexpf(x[i], -e)) << (8 * i);
                packed[1] |= e4m3_encode(ldexpf(x[4 + i], -e)) << (8 * i);
            }
            if (row < n_rows) __builtin_nontemporal_store(packed, reinterpret_cast<u32x2*>(codes + row * kF8Key + 8 * sub));
            if (sub == j) my_scale = ldexpf(1.0f, e);
        }
        // lanes 0 .. R-1 of every quarter-wave: the block's scales form one contiguous 128-byte line
        if (sub < R && row0 + sub < n_rows) scales[row0 + sub] = my_scale;
    }
}

// grid: one block per (query, chunk of keys); 4 waves per block, each streaming its own
// 16-key tiles (tile i of the chunk belongs to wave i % 4) through a private three-slot LDS
// ring, as the bf16 scoring kernel does, with 128-byte key rows: copy d of a tile moves keys
// 8d..8d+7 (whole 128-byte lines), lane 8k + p loading piece p ^ ((r / 2) % 8) of key
// r = 8d + k into position p of that key's LDS row.  MFMA 16x16x32 (bf16): A = q (16 heads),
// B = keys (16 keys); at step s lane 16g + c supplies key c and the dims [32 s + 8 g, +8) --
// eight codes read as 8 bytes (conflict-free: the 16 keys of a read sit in 16 distinct
// 16-byte slots, the two halves of a slot go to g and g ^ 1) and converted by
// v_cvt_scalef32_pk_bf16_fp8 (exact).  The block's unscaled scores collect in LDS and leave at
// the end multiplied by their keys' scales, four per store.
__global__ __launch_bounds__(256) void indexer_decode_fp8_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ codes, const float* __restrict__ kscale,
    const int64_t* __restrict__ kv_off, const int32_t* __restrict__ q_req,
    const int32_t* __restrict__ q_pos, int32_t B, int32_t chunks_per_q, int32_t chunk,
    int64_t max_s, float* __restrict__ scores, int64_t ld, int vec_store) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[4][kF8Ring][kF8Tile * kF8Key];
    __shared__ __attribute__((aligned(16))) float sbuf[kF8MaxChunk];
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
    const int64_t row0 = kv_off[b] + k0;
    const uint8_t* kb = codes + row0 * kF8Key;
    const int n_tiles = (len + kF8Tile - 1) / kF8Tile;
    const int my_tiles = n_tiles > wave ? (n_tiles - wave + 3) / 4 : 0;
    const int ck = lane >> 3, cp = lane & 7;  // copy roles: key within the copy, LDS position
    // copies of this wave's j-th tile into ring slot j % 3; keys past the end copy key 0
    auto issue = [&](int j) {
        const int kt = (wave + 4 * j) * kF8Tile;
        const uint8_t* slot = ring[wave][j % kF8Ring];
#pragma unroll
        for (int d = 0; d < kF8Copies; ++d) {
            const int r = 8 * d + ck;
            const int key = kt + r < len ? kt + r : 0;
            copy_to_lds<true>(kb + static_cast<int64_t>(key) * kF8Key + 16 * (cp ^ ((r >> 1) & 7)),
                              lds_offset(slot + d * 8 * kF8Key));
        }
    };
#pragma unroll
    for (int j = 0; j < kF8Ring - 1; ++j)
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
        if (g == 0) sbuf[(wave + 4 * jj) * kF8Tile + c] = v;
    };
    // A tile's epilogue runs after the next tile's MFMAs are issued, so it overlaps them.
    f32x4 pa0 = {0.f, 0.f, 0.f, 0.f}, pa1 = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < my_tiles; ++j) {
        // tile j landed once only the copies issued after it may be outstanding
        if (j + kF8Ring - 1 < my_tiles) {
            issue(j + kF8Ring - 1);
            wait_vmcnt<(kF8Ring - 1) * kF8Copies>();
        } else {
            wait_vmcnt<0>();
        }
        const uint8_t* buf = ring[wave][j % kF8Ring] + c * kF8Key;
        bf16x8 kf[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int p = 2 * s + (g >> 1);
            const u32x2 v = *reinterpret_cast<const u32x2*>(buf + 16 * (p ^ ((c >> 1) & 7)) + 8 * (g & 1));
            const bf16x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, false);
            const bf16x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, true);
            const bf16x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, false);
            const bf16x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, true);
            kf[s] = bf16x8{e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
        }
        f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[0][s], kf[s], a0, 0, 0, 0);
            a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[1][s], kf[s], a1, 0, 0, 0);
        }
        if (j > 0) epilogue(pa0, pa1, j - 1);
        pa0 = a0;
        pa1 = a1;
    }
    if (my_tiles > 0) epilogue(pa0, pa1, my_tiles - 1);
    __syncthreads();
    float* srow = scores + static_cast<int64_t>(t) * ld + k0;
    const float* sc = kscale + row0;
    for (int i = 4 * static_cast<int>(threadIdx.x); i < len; i += 4 * 256) {
        if (vec_store && i + 3 < len) {
            f32x4 o = *reinterpret_cast<const f32x4*>(sbuf + i);
            o[0] *= sc[i];
            o[1] *= sc[i + 1];
            o[2] *= sc[i + 2];
            o[3] *= sc[i + 3];
            *reinterpret_cast<f32x4*>(srow + i) = o;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (i + k < len) srow[i + k] = sbuf[i + k] * sc[i + k];
        }
    }
}

hipError_t launch_quantize_keys_fp8(const uint16_t* keys, int64_t n_rows, uint8_t* codes,
                                    float* scales, hipStream_t stream) {
    // 64 rows per 256-thread block per pass; at most 32 blocks per CU (grid-stride; 2 M keys
    // cold: 8 per CU 162 us, 16 per CU 153 us, 32 per CU 146 us)
    const int64_t want = (n_rows + kF8FillRows - 1) / kF8FillRows;
    const int64_t cap = 32 * static_cast<int64_t>(device_cus());
    const int blocks = static_cast<int>(want < cap ? (want < 1 ? 1 : want) : cap);
    hipLaunchKernelGGL(quantize_keys_fp8_kernel, dim3(blocks), dim3(256), 0, stream, keys, n_rows,
                       codes, scales);
    return hipGetLastError();
}

hipError_t launch_indexer_scores_fp8(const uint16_t* q_idx, const uint16_t* w, const uint8_t* codes,
                                     const float* kscale, const int64_t* kv_off,
                                     const int32_t* q_req, const int32_t* q_pos, int32_t T,
                                     int32_t B, int64_t max_s, float* scores, int64_t ld,
                                     hipStream_t stream) {
    const int64_t chunk = f8_chunk(T, max_s);
    const int64_t cpq = (max_s + chunk - 1) / chunk;
    const int64_t blocks = cpq * T;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool vec = reinterpret_cast<uintptr_t>(scores) % 16 == 0 && ld % 4 == 0;
    hipLaunchKernelGGL(indexer_decode_fp8_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       stream, q_idx, w, codes, kscale, kv_off, q_req, q_pos, B,
                       static_cast<int32_t>(cpq), static_cast<int32_t>(chunk), max_s, scores, ld,
                       vec ? 1 : 0);
    return hipGetLastError();
}

}  // namespace dsa
