/*
 * taq.h - tiled causal attention over a grouped-quantized KV cache, for
 * AMD Instinct MI355X (gfx950).  Plain C ABI: every pointer is a plain host or
 * device address, every size a plain integer, no C++ or framework types.
 *
 * What the library computes
 * -------------------------
 * Scaled dot-product attention softmax(Q K^T / sqrt(d)) V (Space Bunny
 * inference-stack article, m.xxqk.cn, section 3.1), computed tile by tile with
 * the online-softmax merge of a running maximum and normaliser ("分块稀疏注意力
 * 与KV Cache量化：长文本推理显存优化实践", xdnf.cn, section 2.2), over a KV cache
 * whose values are stored as grouped asymmetric integer codes (same page,
 * section 2.4: adjacent channels form a group with its own scale and zero-point;
 * section 3.2: group size 32) and dequantised inside the tile load (section
 * 1.3: dequantise on read instead of a separate pass), with KV-tile skipping
 * driven by a block mask (section 2.3).  Query head h reads KV head
 * h / (num_q_heads / num_kv_heads) (grouped-query attention).  Below, "the
 * m.xxqk.cn page" and "the xdnf.cn page" name these two sources.
 *
 * Quantisation of one group x[0..31] (32 consecutive head_dim channels of one
 * token of one KV head), qmax = 2^bits - 1:
 *   lo = min(0, min x), hi = max(0, max x)
 *   s  = least fp16 value with s * qmax >= hi - lo   (s = +0 when hi == lo)
 *   z  = round-half-even(-lo / s)                     (exact quotient)
 *   c  = clamp(round-half-even(x / s) + z, 0, qmax)   (exact quotient)
 *   dequantised value: (c - z) * s  (exact in fp32)
 *
 * Memory layout (all buffers contiguous, owned by the caller)
 * -------------------------------------------------------------
 * A cache (K or V) has batch B, num_kv_heads Hkv, head_dim D (= 128 for the
 * attention calls; any multiple of 32 up to 1024 for quantise/dequantise),
 * capacity C (attention calls: C * D < 2^31)
 * (a multiple of 128) and per-head bit widths bits[h] in {4, 8}.
 * RB(h) = D * bits[h] / 8 code bytes per token.  The codes of (b, h) start at
 *     b * C * sum_h RB(h)  +  C * sum_{h' < h} RB(h').
 *   TAQ_LAYOUT_TOKEN (required for K): token t's RB(h) bytes at t * RB(h); in
 *     them channel c's code is byte c (int8) or nibble c % 2 (0 = low) of
 *     byte c / 2 (int4).  scales: fp16 [B][Hkv][C][D/32]; zeros: u8, same shape.
 *   TAQ_LAYOUT_CHANNEL (required for V): tokens in blocks of 32; block j holds
 *     D rows of 32 * bits / 8 bytes; row d holds channel d of the block's 32
 *     tokens: byte t % 32 (int8) or nibble (t % 32) % 2 of byte (t % 32) / 2
 *     (int4).  scales: fp16 [B][Hkv][D/32][C]; zeros: u8, same shape.
 *   The channel layout gives the PV matrix product its key-contiguous operand
 *   straight from memory, and one 32-token block is one contiguous run.
 * Q, O: fp16 bit patterns, decode [B][Hq][D], prefill [B][Hq][L][D].
 * Skip mask: u8, 1 = compute the 128x128 tile, 0 = skip it; element
 *   data[b*stride_b + g*stride_h + qt*n_k_tiles + kt] for KV head g (strides
 *   may be 0 to share one mask); causality still applies inside kept tiles and
 *   entries above the diagonal are ignored.
 *
 * Conventions
 * -----------
 * - Every call validates its host-visible arguments before launching anything
 *   and returns a status; on failure nothing is launched and taq_last_error()
 *   (thread-local) holds a message.  There is no fallback path: a device that
 *   is not gfx950 gets TAQ_ERR_UNSUPPORTED.
 * - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *   default stream).  Buffers must stay alive until the stream reaches it.
 * - The library allocates no device memory; scratch data goes to caller
 *   workspaces, each sized by its *_workspace_bytes call (decode partials,
 *   chunked-prefill key-range partials, mask-generator sums and scores,
 *   head-sensitivity caches).  The one exception is taq_attn_decode_noalloc,
 *   for callers that cannot allocate: its scratch is a fixed device array
 *   that comes with the library (TAQ_DECODE_SCRATCH_BYTES per GPU).
 * - Device pointers must be 16-byte aligned (TAQ_ERR_MISALIGNED otherwise).
 * - Device-resident lengths are clamped to [0, max_seq_len] by the kernels.
 * - softmax_scale = 0 means 1/sqrt(head_dim); negative scales are UNSUPPORTED.
 * - Rows with no permitted key (and prefill rows at or beyond the sequence's
 *   length) are written as zeros.
 */
#ifndef TAQ_H
#define TAQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TAQ_ABI_VERSION 1
#define TAQ_MAX_KV_HEADS 64
#define TAQ_TILE 128
#define TAQ_GROUP 32

typedef enum {
  TAQ_OK = 0,
  TAQ_ERR_INVALID_ARGUMENT = 1,
  TAQ_ERR_UNSUPPORTED = 2,
  TAQ_ERR_MISALIGNED = 3,
  TAQ_ERR_WORKSPACE_TOO_SMALL = 4,
  TAQ_ERR_HIP = 5
} taq_status;

typedef enum { TAQ_LAYOUT_TOKEN = 0, TAQ_LAYOUT_CHANNEL = 1 } taq_layout;

/* One quantised cache (K or V).  `bits` is a HOST array read only during the
 * call; codes/scales/zeros are device buffers of taq_kv_codes_bytes() bytes and
 * taq_kv_meta_count() elements each. */
typedef struct {
  int32_t batch;
  int32_t num_kv_heads;   /* 1 .. TAQ_MAX_KV_HEADS */
  int32_t head_dim;       /* multiple of 32, at most 1024 */
  int32_t group_size;     /* must be 32 */
  int32_t capacity;       /* tokens per (batch, head); multiple of 128 */
  int32_t layout;         /* taq_layout */
  const uint8_t* bits;    /* host [num_kv_heads], each 4 or 8 */
  uint8_t* codes;         /* device */
  uint16_t* scales;       /* device, fp16 bit patterns */
  uint8_t* zeros;         /* device */
} taq_kv_cache;

/* KV-tile skip mask over 128x128 tiles (device data). */
typedef struct {
  const uint8_t* data;
  int32_t tile;           /* must be 128 */
  int32_t n_q_tiles;      /* decode: 1 */
  int32_t n_k_tiles;      /* >= ceil(max_seq_len / 128) */
  int64_t stride_b;       /* elements between batch entries (0 = shared) */
  int64_t stride_h;       /* elements between KV heads (0 = shared) */
} taq_tile_mask;

/* Thread-local text of the last non-OK status of this thread. */
const char* taq_last_error(void);
int taq_abi_version(void);

/* TAQ_OK when `device` is a gfx950 GPU, TAQ_ERR_UNSUPPORTED otherwise. */
taq_status taq_device_check(int device);

/* Size of the codes buffer in bytes, and the number of scales (= zeros).
 * Return 0 for an invalid descriptor. */
size_t taq_kv_codes_bytes(const taq_kv_cache* cache);
size_t taq_kv_meta_count(const taq_kv_cache* cache);

/* Quantise fp16 x [B][Hkv][count][D] into tokens start .. start+count-1 of
 * every (batch, head) of `cache` (section 2.4 of the xdnf.cn page).
 * Codes, scales and zeros of other tokens are left unchanged.  Bit-exact with
 * the definition at the top of this file.  Errors: INVALID_ARGUMENT (null
 * pointer, start/count out of [0, capacity], bad shape), UNSUPPORTED (bits not
 * 4/8, group_size not 32, head_dim not a multiple of 32 in [32, 1024]),
 * MISALIGNED. */
taq_status taq_kv_quantize(const taq_kv_cache* cache, const void* x_f16,
                           int32_t start, int32_t count, void* stream);

/* The same quantisation for the K and the V cache of a layer in one launch:
 * xk into k_cache and xv into v_cache (each fp16 [B][Hkv][count][D] of its
 * own cache's shape), tokens start .. start+count-1 of both; the two caches
 * are quantised side by side instead of one after the other.  Results are
 * byte-identical to two taq_kv_quantize calls.  Both caches must have the same
 * head_dim (their layouts, bits and shapes may differ); the token range must
 * lie inside both capacities.  Errors: as taq_kv_quantize for either cache,
 * plus INVALID_ARGUMENT when the head_dims differ. */
taq_status taq_kv_quantize_pair(const taq_kv_cache* k_cache, const taq_kv_cache* v_cache,
                                const void* xk_f16, const void* xv_f16, int32_t start,
                                int32_t count, void* stream);

/* Quantise-on-append: the same quantisation, batch entry b's fp16 tokens
 * x[b][h][0 .. count-1] going to cache positions starts[b] .. starts[b] +
 * count - 1, so sequences of different lengths each append their next chunk
 * in one call (the quantisation happens as tokens enter the cache, section
 * 1.3 of the xdnf.cn page).  starts is a device int32 [B]; positions
 * outside [0, capacity) are skipped on the device (the host cannot check
 * device values), and an odd int4 start rewrites only the new token's nibble
 * of the shared V byte.  Errors: INVALID_ARGUMENT (null pointer, count
 * outside [0, capacity]), UNSUPPORTED, MISALIGNED (x, starts). */
taq_status taq_kv_append(const taq_kv_cache* cache, const void* x_f16,
                         const int32_t* starts, int32_t count, void* stream);

/* Dequantise tokens start .. start+count-1 into out [B][Hkv][count][D] as
 * fp32 (exact) and/or fp16 (round-to-nearest-even of the exact value); either
 * output may be NULL but not both.  The value of a code is (c - z) * s, the
 * inverse map of the grouped asymmetric quantisation (section 2.4 of the
 * xdnf.cn page).  A checking aid for the stored format: the attention calls
 * apply the same map inside their tile loads. */
taq_status taq_kv_dequantize(const taq_kv_cache* cache, int32_t start,
                             int32_t count, float* out_f32, void* out_f16,
                             void* stream);

/* Workspace bytes that taq_attn_decode needs for these shapes. */
size_t taq_attn_decode_workspace_bytes(const taq_kv_cache* k_cache,
                                       int32_t num_q_heads,
                                       int32_t max_seq_len);

/* Single-token decode: for each batch entry b and query head h, attention of
 * q[b][h] over keys 0 .. seq_lens[b]-1 of KV head h / (Hq/Hkv) (the new
 * token is already in the cache), skipping KV tiles the mask drops
 * (n_q_tiles must be 1, else INVALID_ARGUMENT).  What is computed:
 * softmax(q K^T * scale) V, the scaled dot-product attention of section 3.1
 * of the m.xxqk.cn page, with K and V the dequantised cache values (section
 * 2.4 of the xdnf.cn page), reduced tile by tile with the running
 * (maximum, normaliser) merge of section 2.2 of the xdnf.cn page and with the
 * tiles that the block mask of its section 2.3 drops left out.  Split over KV chunks; the partial (max, normaliser,
 * accumulator) triples are merged in a fixed order, so results are bitwise
 * repeatable.  k_cache must use TAQ_LAYOUT_TOKEN and v_cache
 * TAQ_LAYOUT_CHANNEL, with equal geometry; head_dim must be 128; num_q_heads /
 * num_kv_heads in {1, 2, 4, 8}.  seq_lens is a device int32 [B]; max_seq_len
 * (host) bounds it and must not exceed the capacity.  Errors: as above, plus
 * WORKSPACE_TOO_SMALL. */
taq_status taq_attn_decode(const taq_kv_cache* k_cache,
                           const taq_kv_cache* v_cache, const void* q_f16,
                           int32_t num_q_heads, const int32_t* seq_lens,
                           int32_t max_seq_len, const taq_tile_mask* mask,
                           float softmax_scale, void* o_f16, void* workspace,
                           size_t workspace_bytes, void* stream);

/* The same decode attention with the literal two-pass softmax: pass 1 reads
 * K only and finds each query head's exact maximum score, pass 2 accumulates
 * exp(s - max) v and exp(s - max) against that fixed maximum with no
 * rescaling, and the chunk partials are added.  This is the plain reading of
 * the "coarse maximum first, then correct the normaliser" wording of section
 * 2.2 of the xdnf.cn page, kept as an ablation and cross-check of the
 * online merge that taq_attn_decode uses (it reads K twice).  Arguments,
 * workspace size and errors as taq_attn_decode. */
taq_status taq_attn_decode_two_pass(const taq_kv_cache* k_cache,
                                    const taq_kv_cache* v_cache, const void* q_f16,
                                    int32_t num_q_heads, const int32_t* seq_lens,
                                    int32_t max_seq_len, const taq_tile_mask* mask,
                                    float softmax_scale, void* o_f16, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Bytes of the library's own decode scratch array on each GPU (used only by
 * taq_attn_decode_noalloc). */
#define TAQ_DECODE_SCRATCH_BYTES (16u * 1024u * 1024u)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * taq_attn_decode without a workspace argument.  The split partials go to a
 * file-scope device array of TAQ_DECODE_SCRATCH_BYTES bytes that the library
 * holds on every GPU it runs on until the process ends; the call itself
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * Limit: taq_attn_decode_workspace_bytes() of the call's shapes must not
 * exceed TAQ_DECODE_SCRATCH_BYTES, else WORKSPACE_TOO_SMALL and nothing is
 * launched (with Hq = 32 and Hkv = 8, B = 64 at 32K context needs 8.5 MB and
 * B = 8 at 128K needs 4.3 MB).  Every call on one GPU shares that GPU's array,
 * which keeps the last call's contents: calls that overlap on one GPU (other
 * streams, other threads) race and give undefined results, so serialise
 * them.  No part of the array needs to start at zero.  Results are bitwise
 * those of taq_attn_decode with the same arguments.  Arguments and other
 * errors as taq_attn_decode. */
taq_status taq_attn_decode_noalloc(const taq_kv_cache* k_cache,
                                   const taq_kv_cache* v_cache, const void* q_f16,
                                   int32_t num_q_heads, const int32_t* seq_lens,
                                   int32_t max_seq_len, const taq_tile_mask* mask,
                                   float softmax_scale, void* o_f16, void* stream);

/* Causal prefill with equal query and key lengths: q/o [B][Hq][L][D] where
 * L = max_seq_len; row i of batch b attends to keys j <= i, j < seq_lens[b],
 * in tiles the mask keeps (NULL = dense causal).  Row by row this is the
 * causal scaled dot-product attention of section 3.1 of the m.xxqk.cn page
 * over the dequantised cache (section 2.4 of the xdnf.cn page), computed per
 * 128x128 tile with the online softmax merge of section 2.2 of the xdnf.cn
 * page; tiles dropped by the block mask (its section 2.3) contribute nothing,
 * and query-row tiles whose whole KV range is skipped cost nothing.  The
 * dequantised K and V tiles enter the products as fp16 (the rounded exact
 * values), so the score error grows with softmax_scale * |q| * |k|
 * (unit-scale data at softmax_scale <= 1/sqrt(128) stays within 2e-3 of
 * exact fp64 attention).  Same cache requirements as decode;
 * mask n_q_tiles and n_k_tiles must both cover ceil(max_seq_len / 128). */
taq_status taq_attn_prefill(const taq_kv_cache* k_cache,
                            const taq_kv_cache* v_cache, const void* q_f16,
                            int32_t num_q_heads, const int32_t* seq_lens,
                            int32_t max_seq_len, const taq_tile_mask* mask,
                            float softmax_scale, void* o_f16, void* stream);

/* Workspace bytes that taq_attn_prefill_chunk can use for these shapes (0 when
 * it would not split the key range, or for invalid sizes). */
size_t taq_attn_prefill_chunk_workspace_bytes(const taq_kv_cache* k_cache,
                                              int32_t num_q_heads, int32_t q_len,
                                              int32_t max_seq_len);

/* Chunked prefill against an existing cache: q/o [B][Hq][q_len][D] are the
 * last q_len positions of each sequence, whose keys and values are already
 * in the cache (append them first with taq_kv_append), so row i of batch b
 * sits at position p = seq_lens[b] - q_len + i (bottom-right alignment) and
 * attends to keys j <= p in tiles the mask keeps, the mask being indexed by
 * positions; rows with p < 0 are written as zeros.  This is the step of the
 * multi-turn setting that section 4.2 of the xdnf.cn page discusses:
 * a new turn reads the quantised history through the same tiled kernel.
 * q_len must lie in [0, max_seq_len]; everything else as taq_attn_prefill,
 * which is the case q_len = max_seq_len with every seq_lens[b] =
 * max_seq_len.  A short chunk has few query blocks, so with a workspace
 * (device, 16-byte aligned, at least taq_attn_prefill_chunk_workspace_bytes())
 * the key range of each block is split over several workgroups whose partial
 * (max, normaliser, accumulator) triples are merged in a second kernel in
 * split order; workspace = NULL (bytes ignored) runs unsplit.  Errors: as
 * taq_attn_prefill, plus WORKSPACE_TOO_SMALL and MISALIGNED (workspace). */
taq_status taq_attn_prefill_chunk(const taq_kv_cache* k_cache,
                                  const taq_kv_cache* v_cache, const void* q_f16,
                                  int32_t num_q_heads, int32_t q_len,
                                  const int32_t* seq_lens, int32_t max_seq_len,
                                  const taq_tile_mask* mask, float softmax_scale,
                                  void* o_f16, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Workspace bytes that taq_tile_mask_generate needs (0 for an invalid
 * descriptor or max_seq_len). */
size_t taq_tile_mask_workspace_bytes(const taq_kv_cache* k_cache,
                                     int32_t max_seq_len);

/* Training-free KV-tile mask for block-sparse prefill, after the policy of
 * section 2.3 of the xdnf.cn page: a coarse pattern of skipped 128x128
 * blocks with dense local blocks and a capped skipped share.  That page
 * predicts the pattern with a learned head; this call scores tiles from the
 * data instead.  For batch entry b (n = seq_lens[b], nt_b = ceil(n / 128)),
 * KV head g and query tile i < nt_b it keeps KV tile 0 and tile i and, of
 * tiles 1 .. i-1, drops the floor((i-1) * skip_per_mille / 1000) with the
 * lowest importance (ties: lower j first), where importance(i, j) =
 * sum_d Qsum_i[d] * Kmean_j[d]: Qsum_i sums the query rows of tile i (rows
 * < n) over the Hq/Hkv query heads of g, Kmean_j is the mean dequantised key
 * of tile j.  The sums are exact, Kmean = double(Ksum) / count / 2^24 with
 * the sums in units of 2^-24, and the dot product runs over d in order as
 * double multiply then double add, so the result is reproducible bit for bit.
 * Tiles above the diagonal and rows i >= nt_b are 0.
 * q: fp16 [B][Hq][max_seq_len][128]; k_cache: TAQ_LAYOUT_TOKEN, head_dim 128;
 * seq_lens: device int32 [B] (clamped to [0, max_seq_len]); mask_out: device
 * uint8 [B][Hkv][nt][nt], nt = ceil(max_seq_len / 128), every byte written,
 * usable as a taq_tile_mask with n_q_tiles = n_k_tiles = nt, stride_h = nt^2,
 * stride_b = Hkv * nt^2; workspace: device, 16-byte aligned, of
 * taq_tile_mask_workspace_bytes() bytes = B * Hkv * nt * (2 * 128 + nt) * 8,
 * caller-owned (on return it holds the pooled sums and the scores).  max_seq_len is limited to 2048 tiles.  Errors:
 * INVALID_ARGUMENT (null pointer, Hq not a multiple of Hkv, max_seq_len or
 * skip_per_mille out of range), UNSUPPORTED (cache format, Hq / Hkv above
 * 64, max_seq_len beyond 2048 tiles), MISALIGNED, WORKSPACE_TOO_SMALL.
 * Non-finite queries or keys give an unspecified mask (tile 0 and the
 * diagonal still kept). */
taq_status taq_tile_mask_generate(const taq_kv_cache* k_cache, const void* q_f16,
                                  int32_t num_q_heads, const int32_t* seq_lens,
                                  int32_t max_seq_len, int32_t skip_per_mille,
                                  uint8_t* mask_out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* The same mask for one turn of a multi-turn prefill (section 4.2 of the
 * xdnf.cn page: a new turn reads the quantised history), to drive
 * taq_attn_prefill_chunk: q_f16 [B][Hq][q_len][128] holds the last q_len
 * positions of each sequence (row i of entry b at position
 * seq_lens[b] - q_len + i; rows at negative positions are padding and are not
 * read), whose keys are already in k_cache.  Every query tile that holds one
 * of the turn's positions gets the row taq_tile_mask_generate gives it, with
 * Qsum summing the turn's own rows of that tile (the rows of an earlier turn
 * that share the tile are not part of the call); every other row is written
 * as 0 (chunked prefill reads only the turn's rows).  The mask is indexed by
 * positions, in the layout and with the workspace of taq_tile_mask_generate
 * for the same max_seq_len; q_len must lie in [0, max_seq_len] (q_f16 may be
 * NULL when q_len is 0: every row is then 0); errors as
 * taq_tile_mask_generate. */
taq_status taq_tile_mask_generate_chunk(const taq_kv_cache* k_cache, const void* q_f16,
                                        int32_t num_q_heads, int32_t q_len,
                                        const int32_t* seq_lens, int32_t max_seq_len,
                                        int32_t skip_per_mille, uint8_t* mask_out,
                                        void* workspace, size_t workspace_bytes,
                                        void* stream);

/* Workspace bytes that taq_head_sensitivity needs (0 for invalid sizes). */
size_t taq_head_sensitivity_workspace_bytes(int32_t batch, int32_t num_kv_heads,
                                            int32_t num_q_heads, int32_t max_seq_len);

/* Per-KV-head precision assignment from measured sensitivity (section 2.4 of
 * the xdnf.cn page: sensitive heads are stored at higher precision, the
 * others with fewer bits; section 3.4: more high-precision heads, less memory
 * saved).  The page leaves the score open; here the score of KV head g is how
 * far its decode outputs move when its cache drops from int8 to int4:
 *   scores[g] = sum over b, the query heads h of g and channels d of
 *               (O4[b][h][d] - O8[b][h][d])^2,
 * O_bits being taq_attn_decode of the calibration queries q over tokens
 * 0 .. seq_lens[b]-1 with every head's K and V quantised at `bits` by
 * taq_kv_quantize.  bits[g] = 8 for the n_high largest scores (ties: the lower
 * g), 4 for the rest: a per-head bits array for taq_kv_cache.
 * k, v: device fp16 [B][Hkv][max_seq_len][128] (calibration context); q:
 * device fp16 [B][Hq][128]; seq_lens: device int32 [B] (clamped to
 * [0, max_seq_len]); scores: device double [Hkv] (8-byte aligned); bits:
 * device uint8 [Hkv]; workspace: device, 16-byte aligned, of
 * taq_head_sensitivity_workspace_bytes() bytes (holds int8 and int4 caches,
 * the two outputs and the decode partials).  Hq / Hkv in {1, 2, 4, 8}.
 * Errors: INVALID_ARGUMENT (null pointer, sizes, n_high outside [0, Hkv]),
 * UNSUPPORTED (head ratio, negative scale), MISALIGNED, WORKSPACE_TOO_SMALL. */
taq_status taq_head_sensitivity(const void* k_f16, const void* v_f16, const void* q_f16,
                                int32_t batch, int32_t num_kv_heads, int32_t num_q_heads,
                                const int32_t* seq_lens, int32_t max_seq_len,
                                float softmax_scale, int32_t n_high, double* scores,
                                uint8_t* bits, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Test hook: when `arch` is non-NULL, taq_device_check compares this string
 * instead of the device's architecture name (NULL restores the real check). */
void taq_debug_set_arch_override(const char* arch);

#ifdef __cplusplus
}
#endif
#endif /* TAQ_H */
