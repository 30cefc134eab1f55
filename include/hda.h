/*
 * hda.h -- C ABI of the hybrid decode-attention library (libhda.so).
 *
 * Single-token autoregressive decode attention over an explicit KV cache
 * for a hybrid sliding/full-attention, grouped-query model, as described by
 * the vllm-omni "edge/spark_export.py" page (Spark-X2.5 decode step: ring
 * cache for sliding layers, per-layer-type partial RoPE) and the vLLM
 * "hy_v4/nvidia/flashmla_sparse.py" page (per-head attention sink, sparse
 * top-k MLA decode).
 *
 * Conventions for every entry point
 *   - All tensor arguments are DEVICE pointers on the current HIP device,
 *     owned by the caller.  The library never allocates, frees or keeps
 *     them; it keeps no state between calls.
 *   - bf16 tensors are raw 16-bit bfloat16 values; fp32 tensors are IEEE
 *     float.  Every tensor is dense, row-major (last index fastest) and
 *     16-byte aligned.
 *   - `stream` is a hipStream_t (NULL: the null stream).  Calls only
 *     enqueue work: they never synchronise, so they may be captured into a
 *     HIP graph.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failed check returns a status and enqueues nothing.  Values that live
 *     in device memory (positions, lengths, indices) are not checked on the
 *     host: kernels skip rows outside the cache instead of touching them.
 *   - The library prints nothing.  hda_last_error_message() gives the
 *     reason for the calling thread's last failure.
 */
#ifndef HDA_H_
#define HDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hda_status {
    HDA_OK = 0,
    HDA_ERR_INVALID_ARGUMENT = 1, /* a shape, pointer or value breaks the contract */
    HDA_ERR_UNSUPPORTED = 2,      /* well-formed, but outside what the kernels handle */
    HDA_ERR_WORKSPACE = 3,        /* workspace missing or too small */
    HDA_ERR_HIP = 4               /* the HIP runtime reported an error */
} hda_status;

/* Layer types of the hybrid model (Spark export page, `layer_types`:
 * "sliding_attention" / "full_attention"; any other value is rejected, as
 * `SparkStepConfig.__post_init__` rejects unknown layer types). */
typedef enum hda_layer_type {
    HDA_SLIDING = 0,
    HDA_FULL = 1
} hda_layer_type;

/* Element type of a KV cache (hda_cache_desc.kv_dtype). */
typedef enum hda_kv_dtype {
    HDA_KV_BF16 = 0,
    HDA_KV_FP8_E4M3 = 1
} hda_kv_dtype;

/*
 * One layer's KV cache (Spark export page, `example_inputs`: caches are
 * laid out (batch, kv_heads, entries, head_dim)).
 *
 *   k, v        bf16 [batch, num_kv_heads, capacity, head_dim]
 *   capacity    full: the longest context the cache can hold.
 *               sliding: exactly `window` rows.  Rows 0 .. window-2 are the
 *               ring (the window counts the current token, so a ring holds
 *               window-1 previous entries: `SparkStepConfig.cache_len`);
 *               row window-1 holds the entry the last append evicted from
 *               its ring slot -- the oldest position of the current window.
 *               With it the step's keys are always the leading rows
 *               0 .. min(seq_len, window)-1 of the block, whatever the ring
 *               offset.
 *   rotary_dim  leading dims rotated by RoPE (`rotary_dim`: head_dim times
 *   rope_theta  the layer type's `partial_rotary_factor`), and its theta.
 *               Spark: sliding 256 dims / 1e4, full 64 dims / 5e6.
 *
 * Paged layout (full layers only; block_table NULL selects the contiguous
 * layout above).  The flashmla_sparse page's attention call takes a
 * block table and per-sequence cache lengths for serving many sequences of
 * different lengths from one pool of fixed-size pages:
 *   k, v         page pool bf16 [num_pages, num_kv_heads, page_size, head_dim]
 *   block_table  int32 [batch, max_pages] (device): row r of sequence b is
 *                row r % page_size of page block_table[b][r / page_size]
 *   page_size    rows per page, a positive multiple of 16
 *   capacity     max_pages * page_size
 * Entries must name pool pages for every page that holds one of the
 * sequence's rows; an entry outside [0, num_pages) is clamped into that
 * range (the result is then meaningless, but no access leaves the pool).
 * Pages may be shared between sequences for reading; an append writes row
 * pos of the page its sequence names.
 *
 * FP8 cache (kv_dtype HDA_KV_FP8_E4M3; HDA_KV_BF16, 0, is the bf16 cache
 * above).  The flashmla_sparse page's FP8 call hands the cache to the
 * kernel as raw bytes with an fp8 flag; the element format and scaling
 * used here: every element an e4m3 code (1 sign, 4 exponent bits with bias
 * 7, 3 mantissa bits; no infinities, S.1111.111 is NaN; largest finite
 * 448), every cached row -- one token of one KV head -- one fp32 scale:
 *   value = e4m3(code) * scale,   scale = amax(row) / 448.
 *   k, v        uint8 codes, same shapes as the bf16 cache (row = head_dim
 *               bytes); head_dim must be 256
 *   k_scale,    fp32 [batch, num_kv_heads, capacity] (paged: [num_pages,
 *   v_scale     num_kv_heads, page_size]), 4-byte aligned, device memory;
 *               a sliding layer's evicted-entry row has its scale at index
 *               window-1 like its codes
 * hda_rope_append quantizes the rotated new K row (rounded to bf16 first,
 * as the bf16 cache would store it) and the new V row: scale = amax / 448
 * in fp32, code = e4m3 of x / scale (fp32 division), round to nearest
 * even, saturating at +-448; an all-zero row gets scale 0 and zero codes.
 * The attention dequantizes exactly: K codes to bf16 for the matrix cores
 * with the K scale applied to each key's score, V codes to fp32 with the V
 * scale applied to each key's probability.
 */
typedef struct hda_cache_desc {
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t window;
    int32_t rotary_dim;
    int64_t capacity;
    double rope_theta;
    void *k;
    void *v;
    const int32_t *block_table;
    int32_t page_size;
    int32_t max_pages;
    int64_t num_pages;
    int32_t kv_dtype;
    float *k_scale;
    float *v_scale;
} hda_cache_desc;

/*
 * hda_rope_append -- fused partial RoPE of the step's q and new K, and the
 * KV append, for one layer.
 *
 * Spark export page: `_angles` (angle = position * theta^(-2i/rot), i <
 * rot/2, in fp32), `_rope` (neox halves: out = x*cos + cat(-x2, x1)*sin on
 * the leading rot dims, the rest pass through), `_Layer.forward` ring
 * branch (the new entry goes into the slot for its position, evicting the
 * oldest).
 *
 *   q       bf16 [batch, num_q_heads, head_dim], rotated IN PLACE.
 *   k_new   bf16 [batch, num_kv_heads, head_dim], read only; rotated copy
 *           is written to the cache.
 *   v_new   bf16 [batch, num_kv_heads, head_dim], read only; copied.
 *   pos     int32 [batch] (device): position of each sequence's new token.
 *   layer   HDA_FULL: entry pos of the cache takes the new K/V.
 *           HDA_SLIDING: slot s = pos mod (window-1).  When pos >= window-1
 *           that slot holds position pos-(window-1), still inside this
 *           step's window, so it is first copied to row window-1 (the
 *           evicted-entry row); then slot s takes the new K/V.
 *   Rows outside the cache (pos < 0, or pos >= capacity for a full layer)
 *   are skipped.  Math in fp32 (cos/sin of the fp32 angle evaluated in
 *   fp64), results rounded to nearest-even bf16.
 * Errors: INVALID_ARGUMENT for null pointers, misalignment, non-positive
 * head counts, num_q_heads % num_kv_heads != 0, odd or oversized
 * rotary_dim, sliding capacity != window, unknown layer; UNSUPPORTED for a
 * rotary_dim that is not a multiple of 16 or exceeds 512; HIP on a launch
 * failure.  batch == 0 is a no-op.  Paged cache: row pos is written into
 * the page the sequence's block table names for it; INVALID_ARGUMENT for
 * a page_size that is not a positive multiple of 16, max_pages or
 * num_pages < 1, capacity != max_pages * page_size or a misaligned table;
 * UNSUPPORTED for a paged sliding layer.
 */
hda_status hda_rope_append(void *q, const void *k_new, const void *v_new,
                           const int32_t *pos, hda_layer_type layer,
                           const hda_cache_desc *cache, void *stream);

/*
 * hda_decode_workspace_bytes -- device workspace hda_decode_attn needs for
 * this cache, layer, longest sequence and split size (chunk_keys = 0: the
 * library's default).  0 means no workspace is needed.  Returns 0 for an
 * invalid description as well; hda_decode_attn then reports why.
 */
size_t hda_decode_workspace_bytes(const hda_cache_desc *cache, hda_layer_type layer,
                                  int32_t max_seq_len, int32_t chunk_keys);

/*
 * hda_decode_attn -- decode attention of one layer, after hda_rope_append.
 *
 * For sequence b and query head h the KV head is h / (num_q_heads /
 * num_kv_heads) (Spark `_Layer.forward`: query heads folded per KV head,
 * K/V never expanded).  With n = seq_lens[b] (= pos + 1) the keys are
 *   full:    cache rows 0 .. n-1;
 *   sliding: rows 0 .. min(n, window)-1: the written ring slots plus, once
 *            the window is full, the evicted-entry row -- the last
 *            min(n, window) positions.  Slots never written are excluded,
 *            and ring order does not matter (Spark ring-branch comment).
 * scores = scale * q.k (Spark: scale 1/sqrt(head_dim)); softmax; out =
 * sum p v.  lse = ln sum exp(scores), before any sink.  With sinks, out is
 * multiplied by exp(lse)/(exp(lse)+exp(sink[h])) (flashmla_sparse page,
 * `HYV4FlashMLASparseImpl` docstring); a -inf sink leaves out bit-for-bit
 * unchanged (`_sinks_for_query`: -inf is a no-op sink).  With gate, out of
 * head h of sequence b is also multiplied by 1/(1+exp(-gate[b][h])) (Spark
 * export page, `_Layer.forward`: the sigmoid of g_proj, one value per query
 * head, multiplies that head's attention output); lse is not affected.
 *
 * The keys are split into pieces whose partial softmax results (out, lse)
 * land in the workspace; a merge kernel combines them, lse = ln sum_c
 * exp(lse_c), out = sum_c exp(lse_c - lse) out_c, then applies the sink
 * (Spark ring comment: an online softmax over key subsets gives the same
 * result).  chunk_keys = 0 (the default) splits all 16-key rounds of the
 * batch evenly over the GPU's resident waves, whatever the mix of lengths;
 * chunk_keys > 0 cuts every sequence into chunks of that many keys, one
 * workgroup each.
 *
 *   q          bf16 [batch, num_q_heads, head_dim] (already rotated)
 *   seq_lens   int32 [batch] (device); n <= 0 gives out 0, lse -inf
 *   sinks      fp32 [num_q_heads] (device) or NULL
 *   gate       fp32 [batch, num_q_heads] (device) output-gate logits, or NULL
 *   scale      softmax scale
 *   out        bf16 [batch, num_q_heads, head_dim]
 *   lse        fp32 [batch, num_q_heads] or NULL
 *   max_seq_len  host bound on seq_lens (sizes the split grid); full layers
 *              need max_seq_len <= capacity.  Sequences longer than this
 *              bound are cut to it.
 *   chunk_keys keys per split chunk, a multiple of 16 in [16, 512]; 0
 *              picks the default.
 *   workspace  device buffer of at least hda_decode_workspace_bytes(); calls
 *              that share a workspace must be ordered on one stream.
 * Errors: as hda_rope_append, plus UNSUPPORTED for head_dim != 256 or a
 * query group size outside {1, 2, 4, 8, 16}, WORKSPACE when the workspace
 * is NULL or smaller than required, INVALID_ARGUMENT for a bad chunk_keys
 * or max_seq_len.  The cache is only read.  A paged cache is read by the
 * balanced streaming kernel (the same rounds, summed in the same order as
 * for contiguous blocks): UNSUPPORTED for chunk_keys != 0 or batch above
 * 4096 with a paged cache.
 */
hda_status hda_decode_attn(const void *q, const hda_cache_desc *cache,
                           const int32_t *seq_lens, hda_layer_type layer,
                           const float *sinks, const float *gate, float scale, void *out,
                           float *lse, int32_t max_seq_len, int32_t chunk_keys,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * hda_decode_split_plan -- the chunking hda_decode_attn uses for these
 * arguments: keys per chunk and chunks per (sequence, KV head).  Callers of
 * the two-stage form below size their partial buffers from it.
 */
hda_status hda_decode_split_plan(const hda_cache_desc *cache, hda_layer_type layer,
                                 int32_t max_seq_len, int32_t chunk_keys,
                                 int32_t *chunk_out, int32_t *nsplit_out);

/*
 * hda_decode_attn_partials -- the split-K stage of hda_decode_attn alone
 * (flash-decoding): chunk c of sequence b covers keys [c*chunk, (c+1)*chunk)
 * of the key set hda_decode_attn defines, and yields for every query head
 *   part_o[b, h, c, :] = softmax-weighted mean of V over the chunk's keys,
 *   part_lse[b, h, c]  = ln sum over the chunk of exp(scores),
 * with part_lse = -inf (part_o left unwritten) for a chunk holding no keys.
 * Spark export page, ring-branch comment: a softmax split over key subsets
 * and merged online equals the single pass.  Same arguments as
 * hda_decode_attn; part_o fp32 [batch, num_q_heads, nsplit, head_dim],
 * part_lse fp32 [batch, num_q_heads, nsplit], nsplit from
 * hda_decode_split_plan.  No sink or gate is applied here.  UNSUPPORTED
 * for a paged cache.
 */
hda_status hda_decode_attn_partials(const void *q, const hda_cache_desc *cache,
                                    const int32_t *seq_lens, hda_layer_type layer,
                                    float scale, int32_t max_seq_len, int32_t chunk_keys,
                                    float *part_o, float *part_lse, void *stream);

/*
 * hda_lse_merge -- combine per-chunk partials into the attention output:
 *   lse = ln sum_c exp(part_lse_c),  out = sum_c exp(part_lse_c - lse) part_o_c,
 * chunks with part_lse = -inf weigh zero; then the sink factor
 * exp(lse)/(exp(lse)+exp(sink[h])) (flashmla_sparse page, class docstring)
 * and the output gate 1/(1+exp(-gate[b][h])) (Spark export page,
 * `_Layer.forward`).
 * No chunk holding keys: out 0, lse -inf.  Partials from several devices
 * (context parallelism) merge the same way once gathered.
 *   part_o   fp32 [batch, num_heads, nsplit, head_dim] (head_dim == 256)
 *   part_lse fp32 [batch, num_heads, nsplit]
 *   sinks    fp32 [num_heads] or NULL; gate fp32 [batch, num_heads] logits or
 *            NULL; out bf16 [batch, num_heads, head_dim];
 *   lse      fp32 [batch, num_heads] or NULL (pre-sink).
 */
hda_status hda_lse_merge(const float *part_o, const float *part_lse, int32_t batch,
                         int32_t num_heads, int32_t nsplit, int32_t head_dim,
                         const float *sinks, const float *gate, void *out, float *lse,
                         void *stream);

/*
 * hda_decode_step_workspace_bytes -- device workspace hda_decode_step needs
 * for this cache and layer type (0 for a description it refuses).
 */
size_t hda_decode_step_workspace_bytes(const hda_cache_desc *cache, hda_layer_type layer);

/*
 * hda_decode_step -- one layer's whole decode step in one call: the work of
 * hda_rope_append followed by hda_decode_attn with seq_lens[b] = pos[b] +
 * 1, with two differences: q is only read (its rotation stays in
 * registers), and keys are cut at the cache (full: min(pos+1, capacity),
 * sliding: min(pos+1, window)) rather than at a max_seq_len.  A sliding
 * layer is one launch; a full layer two (the streaming kernel over the rows
 * held before the token, then the merge, which scores the new token and
 * writes it to row pos; a paged full-layer cache is accepted).  After the
 * call the cache holds what hda_rope_append leaves (new K/V in the ring
 * slot or row pos; for a sliding layer at pos >= window-1 the slot's
 * previous entry in row window-1), and out / lse what hda_decode_attn
 * returns.  The sliding window counts the current token (Spark export
 * page, ring branch: window-1 cached entries plus the new one); sinks as in
 * hda_decode_attn (flashmla_sparse page, class docstring).
 *
 *   q, k_new, v_new, pos, layer, cache   as hda_rope_append
 *   sinks, gate, scale, out, lse         as hda_decode_attn
 *   workspace  device buffer of at least hda_decode_step_workspace_bytes()
 *              bytes.  Its first 4*batch*num_kv_heads bytes (rounded up to
 *              256) are arrival counters that must be zero before the first
 *              call; every call leaves them zero.  Zero-fill a new workspace
 *              once.  hda_decode_attn lays its data out after the same
 *              header, so one workspace serves both.  Calls sharing a
 *              workspace must be ordered on one stream.
 * Errors: as hda_decode_attn, plus UNSUPPORTED for rotary_dim other than
 * 64 or 256, batch above 4096, a paged sliding cache, or an fp8 sliding
 * cache whose window exceeds 1024 keys (use hda_rope_append +
 * hda_decode_attn there).  On an fp8 cache the new K and V rows are
 * quantized as hda_rope_append quantizes them, and the new key is scored
 * as stored.  batch == 0 is a no-op.
 */
hda_status hda_decode_step(const void *q, const void *k_new, const void *v_new,
                           const int32_t *pos, hda_layer_type layer,
                           const hda_cache_desc *cache, const float *sinks,
                           const float *gate, float scale, void *out, float *lse,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * hda_decode_step_noalloc -- hda_decode_step without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The workspace is
 * a static device array of the library: 16 MiB, one per GPU the library runs
 * on, held until the process ends.  Arguments, results and errors as
 * hda_decode_step, plus WORKSPACE when the step needs more than that array
 * holds (hda_decode_step_workspace_bytes() > 16 MiB: full layers past about
 * 1,500 sequences), and HIP when no device is current.  The first call on a
 * device also enqueues, on `stream`, one zero fill of the array.  Every call
 * on a GPU uses that GPU's one array, which keeps the last call's contents:
 * calls that overlap on one GPU (other streams, other host threads) race
 * and must be ordered by the caller.  Nothing here allocates or frees.
 */
hda_status hda_decode_step_noalloc(const void *q, const void *k_new, const void *v_new,
                                   const int32_t *pos, hda_layer_type layer,
                                   const hda_cache_desc *cache, const float *sinks,
                                   const float *gate, float scale, void *out, float *lse,
                                   void *stream);

/*
 * hda_decode_multi -- decode of a chunk of `tokens` new tokens per sequence
 * in one call, up to a prefill chunk of 512.  Spark export page,
 * `SparkStepConfig.cache_len` docstring: a ring holds a window's previous
 * entries and the new token is scored with them; for a chunk, token t
 * (position pos[b] + t) attends to the entries of its own window -- the
 * cached ones and new tokens 0..t -- exactly as `tokens` single-token steps
 * (hda_rope_append + hda_decode_attn with seq_len pos + t + 1) in order
 * would, and the cache ends as they leave it.
 *   q       bf16 [batch, tokens, num_q_heads, head_dim], rotated in place
 *           (as hda_rope_append rotates it)
 *   k_new   bf16 [batch, tokens, num_kv_heads, head_dim], read only (its
 *           rotation goes to the workspace and the cache)
 *   v_new   bf16 [batch, tokens, num_kv_heads, head_dim], read only
 *   pos     int32 [batch] (device): position of token 0; a negative value
 *           leaves the sequence's cache alone and its out 0, lse -inf
 *   out     bf16 [batch, tokens, num_q_heads, head_dim]
 *   lse     fp32 [batch, tokens, num_q_heads] or NULL (before the sink)
 *   sinks   fp32 [num_q_heads] or NULL; gate fp32 [batch, tokens,
 *           num_q_heads] logits or NULL (as in hda_decode_attn)
 *   max_seq_len host bound on pos + tokens (sizes how many workgroups share
 *           each sequence's keys for small chunks; results do not depend on it)
 *   workspace  device buffer of at least hda_decode_multi_workspace_bytes()
 *           (the rotated new K rows, and partials when the keys are split);
 *           calls sharing one must be ordered on one stream
 * The cache is read as it was before the chunk and written after the
 * attention (full: rows pos + t below capacity; sliding: the ring slots of
 * the last window-1 tokens, the evicted-entry row taking the entry of
 * position pos + tokens - window).  Chunks of more than 16 query rows per
 * KV head (tokens x num_q_heads / num_kv_heads) run the prefill kernel:
 * both attention products on the matrix cores.  Errors: as hda_decode_attn,
 * plus UNSUPPORTED for tokens outside 1..512, rotary_dim not a multiple of
 * 16, a cache of fewer than 16 rows (32 for the prefill kernel), a paged or
 * fp8 cache; INVALID_ARGUMENT for max_seq_len < 1; WORKSPACE for a missing
 * or short workspace.  batch == 0 is a no-op.
 */
hda_status hda_decode_multi(void *q, const void *k_new, const void *v_new, const int32_t *pos,
                            int32_t tokens, hda_layer_type layer, const hda_cache_desc *cache,
                            const float *sinks, const float *gate, float scale, void *out,
                            float *lse, int32_t max_seq_len, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * hda_decode_multi_workspace_bytes -- device workspace hda_decode_multi
 * needs for this cache, layer type, chunk size and max_seq_len (0 for an
 * invalid description).
 */
size_t hda_decode_multi_workspace_bytes(const hda_cache_desc *cache, hda_layer_type layer,
                                        int32_t tokens, int32_t max_seq_len);

/*
 * hda_sparse_workspace_bytes -- device workspace hda_sparse_decode_attn needs
 * for this many tokens, query heads and index-row length (0: none).
 * Returns 0 for an invalid shape as well; the call then reports why.
 */
size_t hda_sparse_workspace_bytes(int32_t tokens, int32_t num_q_heads, int32_t topk,
                                  int32_t dv);

/*
 * hda_sparse_decode_attn -- sparse top-k decode attention with a sink over
 * one latent KV head shared by every query head (flashmla_sparse page:
 * `_bf16_flash_mla_kernel` -- the cache viewed as (rows, 1, Dqk), per-token
 * top-k index rows, optional `topk_length`, the sink; `head_dim_v` = Dv).
 *
 * For token t the keys are the pool rows indices[t][i], i < len_t, where
 * len_t = topk_length[t] (clamped to [0, topk]) or topk when topk_length is
 * NULL; entries outside [0, pool_rows) (the -1 padding) name no row and are
 * skipped.  For query head h:
 *   s_i = scale * q[t][h] . kv[idx_i]          (all dqk dims)
 *   out[t][h] = sum_i softmax(s)_i kv[idx_i][0 .. dv-1]
 *   lse[t][h] = ln sum_i exp(s_i)              (before the sink)
 * then out *= exp(lse)/(exp(lse)+exp(sinks[h])) as in hda_decode_attn.  No
 * key at all: out 0, lse -inf.
 *
 *   q          bf16 [tokens, num_q_heads, dqk]
 *   kv         bf16 [pool_rows, dqk]: the latent part first, so the value
 *              of a row is its leading dv dims
 *   indices    int32 [tokens, topk] (device)
 *   topk_length int32 [tokens] (device) or NULL
 *   sinks      fp32 [num_q_heads] (device) or NULL
 *   out        bf16 [tokens, num_q_heads, dv]; lse fp32 [tokens, num_q_heads]
 *              or NULL
 *   workspace  device buffer of at least hda_sparse_workspace_bytes()
 *              (partials of the key splits); may be NULL when that is 0.
 * Errors: INVALID_ARGUMENT for null or misaligned pointers, negative
 * tokens/topk, pool_rows < 1, num_q_heads not a positive multiple of 16;
 * UNSUPPORTED for (dqk, dv) other than (576, 512); WORKSPACE when the
 * workspace is smaller than required; HIP on a launch failure.  tokens == 0
 * is a no-op.  The pool and indices are only read.
 */
hda_status hda_sparse_decode_attn(const void *q, const void *kv, int64_t pool_rows,
                                  const int32_t *indices, int32_t tokens, int32_t topk,
                                  const int32_t *topk_length, int32_t num_q_heads,
                                  int32_t dqk, int32_t dv, const float *sinks, float scale,
                                  void *out, float *lse, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * hda_sparse_decode_attn_fp8 -- hda_sparse_decode_attn over an fp8 latent
 * pool (flashmla_sparse page, `_fp8_flash_mla_kernel`: the cache handed to
 * the kernel as bytes, `head_dim_v` 512, top-k indices, the sink).  The page
 * names its fp8 layout without printing it; the reading taken is the one of
 * the fp8 decode cache above: e4m3 codes (bias 7, largest finite 448,
 * S.1111.111 NaN) with one fp32 scale per pool row, so the value of element
 * d of row r is decode(kv_codes[r][d]) * kv_scales[r] for its key dims and
 * its leading dv value dims alike.  Everything else -- indices, skipped
 * entries, the softmax, lse, the sink, the workspace -- as
 * hda_sparse_decode_attn (there is no topk_length: -1 padding ends a row).
 *
 *   kv_codes   uint8 [pool_rows, dqk], 16-byte aligned
 *   kv_scales  fp32 [pool_rows]
 * Errors: as hda_sparse_decode_attn.  The pool and indices are only read.
 */
hda_status hda_sparse_decode_attn_fp8(const void *q, const uint8_t *kv_codes, const float *kv_scales,
                                      int64_t pool_rows, const int32_t *indices, int32_t tokens,
                                      int32_t topk, int32_t num_q_heads, int32_t dqk, int32_t dv,
                                      const float *sinks, float scale, void *out, float *lse,
                                      void *workspace, size_t workspace_bytes, void *stream);

/* Human-readable name of a status code (static storage). */
const char *hda_status_string(hda_status status);

/* Reason for the calling thread's most recent failed call ("" if none). */
const char *hda_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* HDA_H_ */
