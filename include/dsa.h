/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek-Sparse-Attention read path used by the
 * global Gated-MLA layers of Kimi K3.1.
 *
 * The operations are those of the page "Kimi K3.1 Pro: Sparse-Zugriffe, keine kleinere
 * Historie" (flozi.net guide on the K3.1 DSA indexer and cache):
 *   stage 1  index-key LayerNorm            section "Eine Query durch den Indexer verfolgen"
 *                                           (LayerNorm after the key projection; the adapter
 *                                           paragraph: FP32 normalisation, no Hadamard, no
 *                                           rotation of the index keys)
 *   stage 2  indexer scores                 same section (32 query heads of width 128, one
 *                                           shared 128-wide key per position, 32 BF16 head
 *                                           weights per query)
 *   stage 3  top-2048 causal selection      same section ([T,2048] position IDs; short
 *                                           prefixes and invalid entries are the backend's)
 *   stage 4  restricted-softmax MLA read    section "Die Mathematik der Sparse Attention und
 *                                           ihrer fehlenden Masse" (softmax restricted to I_t,
 *                                           absorbed projections, shared 512+64 latent)
 *   before 1 indexer-side projections      section "Eine Query durch den Indexer verfolgen"
 *                                           (query latent -> [T,32,128], residual -> key ->
 *                                           LayerNorm, residual -> 32 head weights)
 *   after 4  value up-projection + gate     section "Was ändert sich – und was nicht?" and
 *                                           the paragraph after the Gated-MLA one
 *
 * Conventions shared by every entry point
 *  - Every array argument is a DEVICE pointer (memory on the GPU the stream belongs to).
 *    The caller allocates and owns all buffers, inputs, outputs and workspaces.  The
 *    library allocates nothing and frees nothing; between calls it keeps only per-device
 *    lookups (compute-unit count, the address of dsa_indexer_topk_noalloc's scratch array),
 *    so calls on different streams are independent (except dsa_indexer_topk_noalloc calls
 *    on one GPU, which share its scratch array).
 *  - bf16 tensors are passed as uint16_t bit patterns; all layouts are row-major and
 *    densely packed unless a leading dimension (ld, in ELEMENTS) is given.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*, NULL = the null
 *    stream).  No call synchronises with the host or copies device data to the host.
 *  - Arguments are validated on the host BEFORE any HIP call.  A violation returns a
 *    status code and sets a thread-local message (dsa_last_error); nothing is launched.
 *    A failed launch returns DSA_ERR_HIP.  The library never aborts.
 *  - Zero-sized work (T == 0, n_rows == 0) returns DSA_OK without touching any pointer.
 *  - Device-resident metadata cannot be checked on the host without a synchronisation.  The
 *    kernels bound what indexes other arrays:
 *      q_req    a query whose q_req[t] lies outside [0, B) has no admissible position: its
 *               scores are not written, its ID row is all -1, its read is zero, lse -inf;
 *      q_pos    any value (n_t is clamped to [0, min(S_b, max_S)]);
 *      n_valid  clamped to [0, max_n];
 *      ids      any value outside [0, S_b) is padding;
 *      paged    no page-table entry past a request's max_pages is read: the indexer scores
 *               positions at or beyond max_pages * page_size against pool page 0 and the
 *               read treats them as padding.
 *    Two things are trusted, and breaking them is undefined behaviour (the library is never
 *    told the cache sizes):
 *      kv_off   0 <= kv_off[0] <= kv_off[1] <= ... <= kv_off[B] <= rows of every cache
 *               array the call reads;
 *      pages    every page-table entry a request uses names a page inside the pools.
 *
 * Request layout (stages 2-4).  B requests; request b owns the key/latent rows
 * [kv_off[b], kv_off[b+1]) of the packed caches, so its length is S_b = kv_off[b+1]-kv_off[b].
 * Query t belongs to request q_req[t] and sits at absolute position q_pos[t].  Its
 * admissible positions are j in [0, n_t) with n_t = min(q_pos[t] + 1, S_b): causal with the
 * diagonal.  Position IDs are request-local (0-based within the request).
 */
#ifndef DSA_AMD_DSA_H
#define DSA_AMD_DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSA_OK = 0,
    DSA_ERR_INVALID_ARG = 1,  /* null pointer, negative size, misaligned pointer, bad ld   */
    DSA_ERR_UNSUPPORTED = 2,  /* well-formed but outside what the kernels implement        */
    DSA_ERR_WORKSPACE = 3,    /* workspace missing, misaligned (256 B) or too small         */
    DSA_ERR_HIP = 4           /* the HIP runtime reported an error at launch                */
} dsa_status_t;

#define DSA_INDEX_HEADS 32
#define DSA_INDEX_DIM 128
#define DSA_TOPK 2048
#define DSA_MLA_HEADS 96
#define DSA_LATENT_DIM 512
#define DSA_VALUE_DIM 128
#define DSA_COMPANION_DIM 64
#define DSA_WORKSPACE_ALIGN 256

/* Element type of the sparse read's output. */
typedef enum { DSA_OUT_BF16 = 0, DSA_OUT_F32 = 1 } dsa_out_dtype_t;

/* Version of this ABI; bumped on any incompatible change. */
int dsa_abi_version(void);

/* Static description of a status code (never NULL). */
const char* dsa_status_string(int status);

/* Detail of the last error raised on the calling thread ("" if none). */
const char* dsa_last_error(void);

/*
 * Stage 1 -- index-key LayerNorm (cache write).
 * raw      [n_rows,128] float32, 16-byte aligned: projected keys before normalisation.
 * gamma    [128] float32, beta [128] float32: affine parameters.
 * eps      added to the biased variance (must be finite and >= 0).
 * keys     [n_rows,128] bf16 out, 16-byte aligned:
 *          keys = (x - mean(x)) / sqrt(var(x) + eps) * gamma + beta, computed in fp32 and
 *          rounded to bf16 with round-to-nearest-even.  No rotation, no Hadamard transform.
 * Errors: INVALID_ARG for null/misaligned pointers, n_rows < 0, eps < 0 or not finite.
 */
dsa_status_t dsa_index_keys_layernorm(const float* raw, const float* gamma, const float* beta,
                                      float eps, uint16_t* keys, int64_t n_rows,
                                      void* stream);

/*
 * Stage 2 alone -- indexer scores (diagnostic / parity hook; stage 2 inside
 * dsa_indexer_topk runs the same kernels into its workspace).
 * q_idx    [T,32,128] bf16 index queries, 16-byte aligned.
 * w        [T,32] bf16 head weights.
 * keys     [sum S_b,128] bf16 LayerNormed index keys, 16-byte aligned.
 * kv_off   [B+1] int64, q_req [T] int32, q_pos [T] int32: request layout (see above).
 * max_S    host-side upper bound of every S_b (n_t is clamped to it on the device).
 * n_heads  must be 32, head_dim must be 128 (else UNSUPPORTED).
 * scores   [T,ld_scores] float32 out, ld_scores >= max_S:
 *          scores[t][j] = sum_h w[t][h] * max(0, q_idx[t][h] . keys[kv_off[q_req[t]] + j])
 *          for j < n_t, fp32 arithmetic; entries j >= n_t are not written.
 */
dsa_status_t dsa_indexer_scores(const uint16_t* q_idx, const uint16_t* w, const uint16_t* keys,
                                const int64_t* kv_off, const int32_t* q_req,
                                const int32_t* q_pos, int32_t T, int32_t B, int64_t max_S,
                                int32_t n_heads, int32_t head_dim, float* scores,
                                int64_t ld_scores, void* stream);

/*
 * Stage 3 alone -- top-k of caller-given fp32 scores.
 * scores   [T,ld] float32; row t holds n_valid[t] scores at columns [0, n_valid[t]).
 * n_valid  [T] int32 (clamped to [0, max_n] on the device); max_n <= ld.
 * topk     must be 2048 (else UNSUPPORTED).
 * ids      [T,topk] int32 out.  If n <= topk the row is 0,1,...,n-1 followed by -1.
 *          Otherwise it holds the topk columns with the largest scores, listed in
 *          ascending column order.  Order: larger score first; -0 equals +0; NaN ranks
 *          below every number (-inf included); equal scores go to the lower column.
 *          The result is therefore unique and compared bit for bit.
 */
dsa_status_t dsa_topk(const float* scores, int64_t ld, const int32_t* n_valid, int32_t T,
                      int64_t max_n, int32_t topk, int32_t* ids, void* stream);

/*
 * Stages 2+3 -- indexer scores followed by the causal top-2048 selection.
 * Arguments as for dsa_indexer_scores; topk must be 2048.
 * ids       [T,2048] int32 out: request-local position IDs, selected set in ascending
 *           order, then -1 padding (short prefixes n_t <= 2048 select all of [0, n_t)).
 * workspace device buffer of at least dsa_indexer_topk_workspace_size(T, max_S) bytes,
 *           256-byte aligned (holds the fp32 scores of every admissible position, rows
 *           padded to a multiple of four floats, and -- when few long rows would leave
 *           most compute units idle -- per-part candidate lists of a two-stage selection).
 */
size_t dsa_indexer_topk_workspace_size(int32_t T, int64_t max_S);
dsa_status_t dsa_indexer_topk(const uint16_t* q_idx, const uint16_t* w, const uint16_t* keys,
                              const int64_t* kv_off, const int32_t* q_req,
                              const int32_t* q_pos, int32_t T, int32_t B, int64_t max_S,
                              int32_t n_heads, int32_t head_dim, int32_t topk, int32_t* ids,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Stages 2+3 without any allocation, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, kernels and results as dsa_indexer_topk, without the workspace: the scores and
 * candidate lists go to a device array of DSA_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends (its address is looked up on a device's first
 * call, with that device current).  The call itself allocates and frees nothing.
 * Limit: dsa_indexer_topk_workspace_size(T, max_S) <= DSA_NOALLOC_SCRATCH_BYTES (32 MiB: e.g.
 * 256 queries x 32,768 positions, or 64 x 65,536), else UNSUPPORTED before anything runs.
 * Calls that overlap on one GPU (different streams, or host threads) share that array and
 * race; serialise them.  Launch on a stream of the current device.
 */
#define DSA_NOALLOC_SCRATCH_BYTES (32u << 20)
dsa_status_t dsa_indexer_topk_noalloc(const uint16_t* q_idx, const uint16_t* w,
                                      const uint16_t* keys, const int64_t* kv_off,
                                      const int32_t* q_req, const int32_t* q_pos, int32_t T,
                                      int32_t B, int64_t max_S, int32_t n_heads,
                                      int32_t head_dim, int32_t topk, int32_t* ids,
                                      void* stream);

/*
 * Paged page-pool cache layout (a cache layout variant).  Page "Kimi K3.1 Pro: Sparse-
 * Zugriffe, keine kleinere Historie", section "Warum Top-2048 keinen 2048-Token-Cache
 * bedeutet": page allocation changes the physical cache while the logical [T,2048] position
 * IDs stay the same.
 * The index keys, latent rows and companion rows of every request live in pools of fixed-size
 * pages: logical position p of request b is pool row
 *     page_table[b * max_pages + p / page_size] * page_size + p % page_size
 * of key_pool [rows,128], latent_pool (row stride ld_latent) and kpe_pool (row stride ld_kpe).
 * page_size  a power of two in [64, 2^20] (else UNSUPPORTED); max_pages >= 1 is the row stride
 *            of page_table [B, max_pages] int32 (4-byte aligned).  Entries 0 .. ceil(S_b /
 *            page_size) - 1 of row b must name pages of the pools, and pool rows must stay below
 *            2^31 (device data is not checked).
 * kv_off     [B+1] int64 as elsewhere, but only its differences (the request lengths S_b) are
 *            used; the IDs, workspaces and outputs are those of dsa_indexer_topk and
 *            dsa_sparse_mla_attn, and for the same logical cache the results are identical.
 */
dsa_status_t dsa_indexer_topk_paged(const uint16_t* q_idx, const uint16_t* w,
                                    const uint16_t* key_pool, const int32_t* page_table,
                                    int32_t page_size, int32_t max_pages, const int64_t* kv_off,
                                    const int32_t* q_req, const int32_t* q_pos, int32_t T,
                                    int32_t B, int64_t max_S, int32_t n_heads, int32_t head_dim,
                                    int32_t topk, int32_t* ids, void* workspace,
                                    size_t workspace_bytes, void* stream);
dsa_status_t dsa_sparse_mla_attn_paged(const uint16_t* q, const uint16_t* latent_pool,
                                       int64_t ld_latent, const uint16_t* kpe_pool,
                                       int64_t ld_kpe, const int32_t* page_table,
                                       int32_t page_size, int32_t max_pages,
                                       const int64_t* kv_off, const int32_t* q_req,
                                       const int32_t* ids, int32_t T, int32_t B, int32_t n_heads,
                                       int32_t topk, float scale, void* out, int32_t out_dtype,
                                       float* lse, void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * FP8 index-key cache (a reduced-precision cache variant).  Page "Kimi K3.1 Pro: Sparse-
 * Zugriffe, keine kleinere Historie", section "Warum Top-2048 keinen 2048-Token-Cache
 * bedeutet" (index quantisation and scale metadata change the physical cache) and section
 * "Was ein Deployment validieren muss" (cache precision is an option, not a
 * quality-preserving default; no quality is claimed).
 * Row j is stored as 128 OCP FP8 E4M3 codes and a float scale 2^e_j, e_j the smallest
 * exponent with max_d |k_jd| <= 448 * 2^e_j (e_j = 0 for an all-zero row);
 * code = round-to-nearest-even(k_jd * 2^-e_j).  Decoded key = E4M3 value * scale.
 *
 * dsa_quantize_index_keys_fp8: keys [n_rows,128] bf16 (16-byte aligned) -> codes
 *   [n_rows,128] uint8 (16-byte aligned) and scales [n_rows] float32 (4-byte aligned).
 *   Bit-reproducible (exact power-of-two scaling, integer rounding).  Keys must be finite:
 *   a row holding +-inf or NaN gets unspecified codes and scale (no access leaves the row).
 * dsa_indexer_scores_fp8 / dsa_indexer_topk_fp8: as dsa_indexer_scores / dsa_indexer_topk with
 *   the keys replaced by (codes, scales): scores[t][j] = sum_h w[t][h] * max(0,
 *   q_idx[t][h] . decoded key j), fp32 sums; the workspace of dsa_indexer_topk_fp8 is sized by
 *   dsa_indexer_topk_workspace_size.
 * Errors: as the bf16 entry points; codes must be 16-byte and scales 4-byte aligned.
 */
dsa_status_t dsa_quantize_index_keys_fp8(const uint16_t* keys, int64_t n_rows, uint8_t* codes,
                                         float* scales, void* stream);
dsa_status_t dsa_indexer_scores_fp8(const uint16_t* q_idx, const uint16_t* w, const uint8_t* codes,
                                    const float* scales, const int64_t* kv_off,
                                    const int32_t* q_req, const int32_t* q_pos, int32_t T,
                                    int32_t B, int64_t max_S, int32_t n_heads, int32_t head_dim,
                                    float* scores, int64_t ld_scores, void* stream);
dsa_status_t dsa_indexer_topk_fp8(const uint16_t* q_idx, const uint16_t* w, const uint8_t* codes,
                                  const float* scales, const int64_t* kv_off,
                                  const int32_t* q_req, const int32_t* q_pos, int32_t T,
                                  int32_t B, int64_t max_S, int32_t n_heads, int32_t head_dim,
                                  int32_t topk, int32_t* ids, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Stage 4 -- absorbed-MLA read restricted to the selected positions.
 * q        [T,96,576] bf16 absorbed queries (512 latent + 64 companion dims), 16-B aligned.
 * latent   row r at latent + r*ld_latent holds the 512-wide latent (first 512 elements).
 * kpe      row r at kpe + r*ld_kpe holds the 64-wide companion key (first 64 elements).
 *          A packed [N,576] cache is passed as latent = base, kpe = base + 512,
 *          ld_latent = ld_kpe = 576.  Both pointers 16-B aligned, ld multiples of 8,
 *          ld_latent >= 512, ld_kpe >= 64.
 * kv_off, q_req: request layout; ids [T,topk] int32 request-local IDs; an ID < 0 or
 *          >= S_b is padding and is skipped.  Duplicate IDs are counted twice.
 * topk     must be 2048; n_heads must be 96.
 * scale    logit scale (1/sqrt(192) for K3.1), finite.
 * out      [T,96,512], element type out_dtype (DSA_OUT_BF16, rounded to nearest even, or
 *          DSA_OUT_F32), 16-byte aligned: o = sum_{j in I_t} p_j c_j[0:512],
 *          p_j = exp(a_j - m) / sum_{i in I_t} exp(a_i - m),  a_j = scale * q . [c_j ; kpe_j].
 *          fp32 softmax; P and the latent enter the P.V product as bf16, products are
 *          accumulated in fp32.  A row with no valid ID gives out = 0.
 * lse      [T,96] float32 out (may be NULL): log sum_{j in I_t} exp(a_j); -inf if empty.
 * workspace at least dsa_sparse_mla_workspace_size(T, 96, 2048) bytes, 256-byte aligned
 *          (may be NULL when that size is 0): split-KV partial results (small T splits each
 *          ID row over several blocks and merges their normalised partials afterwards).
 *          With bf16 output the partials are kept in bf16 (each split's normalised partial
 *          is rounded once more, by at most half a bf16 ulp), with fp32 output in fp32.
 */
size_t dsa_sparse_mla_workspace_size(int32_t T, int32_t n_heads, int32_t topk);
dsa_status_t dsa_sparse_mla_attn(const uint16_t* q, const uint16_t* latent, int64_t ld_latent,
                                 const uint16_t* kpe, int64_t ld_kpe, const int64_t* kv_off,
                                 const int32_t* q_req, const int32_t* ids, int32_t T,
                                 int32_t B, int32_t n_heads, int32_t topk, float scale,
                                 void* out, int32_t out_dtype, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * After stage 4 -- value up-projection and sigmoid output gate of the read.
 * Page "Kimi K3.1 Pro: Sparse-Zugriffe, keine kleinere Historie": 96 heads with 128-wide
 * value heads (section "Was ändert sich – und was nicht?"); a learned, coordinatewise,
 * input-dependent sigmoid output gate after the sparse attention and before the output
 * projection (the paragraph after the Gated-MLA one).
 * o        [T,96,512] bf16, 16-byte aligned: the read (dsa_sparse_mla_attn's bf16 output).
 * w_uv     [96,128,512] bf16, 16-byte aligned: per-head up-projection, row c of head h maps
 *          the latent to value coordinate c.
 * gate     [T,96,128] bf16 gate logits (2-byte aligned), produced upstream from the token.
 * n_heads  must be 96 (else UNSUPPORTED).
 * out      [T,96,128] bf16 out, 4-byte aligned:
 *          out[t][h][c] = (sum_k w_uv[h][c][k] * o[t][h][k]) * 1 / (1 + exp(-gate[t][h][c])),
 *          products and sums in fp32, the sigmoid in fp32, rounded to bf16 (nearest even).
 * Errors: INVALID_ARG for T < 0 or null/misaligned pointers when T > 0.
 */
dsa_status_t dsa_value_gate(const uint16_t* o, const uint16_t* w_uv, const uint16_t* gate,
                            int32_t T, int32_t n_heads, uint16_t* out, void* stream);

/*
 * Before stages 1 and 2 -- the indexer-side projections of T new tokens, with the key
 * LayerNorm and the append of the keys to the index-key cache.
 * Page "Kimi K3.1 Pro: Sparse-Zugriffe, keine kleinere Historie", section "Eine Query durch
 * den Indexer verfolgen": the query latent is projected to [T,32,128]; another projection maps
 * residual states to [S,128] keys, followed by LayerNorm; a further one makes 32 head weights
 * from each query's residual state.  Widths from section "Was ändert sich – und was nicht?"
 * (query latent 1536, residual 7168).  No bias, scale or activation (the page names none).
 * c_q       [T,1536] bf16 query latents, 16-byte aligned.
 * h         [T,7168] bf16 residual states, 16-byte aligned.
 * w_qi      [4096,1536] bf16, 16-byte aligned; row 128*head + dim makes q_idx[t][head][dim].
 * w_k       [128,7168] bf16 key projection, 16-byte aligned.
 * w_w       [32,7168] bf16 head-weight projection, 16-byte aligned.
 * gamma, beta [128] fp32 LayerNorm affine, 4-byte aligned; eps finite and >= 0.
 * q_idx     [T,32,128] bf16 out, 16-byte aligned: bf16(sum_i w_qi[j][i] * c_q[t][i]).
 * w         [T,32] bf16 out, 2-byte aligned: bf16(sum_i w_w[head][i] * h[t][i]).
 * keys      the index-key cache [rows,128] bf16, 16-byte aligned.  Row key_rows[t] receives
 *           bf16(LayerNorm(k)) with k = sum_i w_k[:][i] * h[t][i], LayerNorm as in
 *           dsa_index_keys_layernorm applied to the fp32 k; no other row is written.
 * key_rows  [T] int64 device array, 8-byte aligned: absolute destination rows of the packed
 *           cache (for request b at request-local position p: kv_off[b] + p).  The caller
 *           guarantees they are distinct and inside the cache (device data is not checked).
 * Sums are fp32 (bf16 products are exact), split over K in a fixed order (deterministic).
 * workspace >= dsa_indexer_project_workspace_size(T) bytes, 256-byte aligned (fp32 partial
 *           sums of the split contractions; the query product needs none from the T at which
 *           it is no longer split over K, about 900 tokens).
 * Errors: INVALID_ARG for T < 0, a bad eps or null/misaligned pointers when T > 0;
 * WORKSPACE for a missing, misaligned or short workspace.
 */
size_t dsa_indexer_project_workspace_size(int32_t T);
dsa_status_t dsa_indexer_project(const uint16_t* c_q, const uint16_t* h, const uint16_t* w_qi,
                                 const uint16_t* w_k, const uint16_t* w_w, const float* gamma,
                                 const float* beta, float eps, int32_t T, uint16_t* q_idx,
                                 uint16_t* w, uint16_t* keys, const int64_t* key_rows,
                                 void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_AMD_DSA_H */
