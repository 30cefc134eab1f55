// hda_api.cpp -- C ABI of libhda: host-side validation, split planning and
// kernel dispatch.  Declared in include/hda.h; every check here runs before
// anything is enqueued, and nothing here synchronises or allocates.
#include "hda.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "hda_kernels.h"

namespace {

thread_local char g_last_error[512] = "";

hda_status fail(hda_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

hda_status ok() {
    g_last_error[0] = '\0';
    return HDA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by both calls: the cache description and the layer type.
// Mirrors the Spark export page's config checks (`__post_init__`: query
// heads must be a multiple of KV heads; unknown layer types rejected).
hda_status check_cache(const hda_cache_desc *c, int layer) {
    if (!c) return fail(HDA_ERR_INVALID_ARGUMENT, "cache descriptor is NULL");
    if (layer != HDA_SLIDING && layer != HDA_FULL)
        return fail(HDA_ERR_INVALID_ARGUMENT, "unknown layer type %d", layer);
    if (c->batch < 0) return fail(HDA_ERR_INVALID_ARGUMENT, "batch %d < 0", c->batch);
    if (c->num_q_heads <= 0 || c->num_kv_heads <= 0)
        return fail(HDA_ERR_INVALID_ARGUMENT, "head counts must be positive (q %d, kv %d)",
                    c->num_q_heads, c->num_kv_heads);
    if (c->num_q_heads % c->num_kv_heads)
        return fail(HDA_ERR_INVALID_ARGUMENT,
                    "num_q_heads %d is not a multiple of num_kv_heads %d", c->num_q_heads,
                    c->num_kv_heads);
    if (c->head_dim <= 0 || c->head_dim % 8)
        return fail(HDA_ERR_INVALID_ARGUMENT, "head_dim %d must be a positive multiple of 8",
                    c->head_dim);
    if (c->rotary_dim < 0 || c->rotary_dim % 2 || c->rotary_dim > c->head_dim)
        return fail(HDA_ERR_INVALID_ARGUMENT, "rotary_dim %d must be even and in [0, head_dim]",
                    c->rotary_dim);
    if (!(c->rope_theta > 0.0) || !std::isfinite(c->rope_theta))
        return fail(HDA_ERR_INVALID_ARGUMENT, "rope_theta must be positive and finite");
    if (layer == HDA_SLIDING) {
        if (c->window < 2) return fail(HDA_ERR_INVALID_ARGUMENT, "window %d < 2", c->window);
        if (c->capacity != (int64_t)c->window)
            return fail(HDA_ERR_INVALID_ARGUMENT,
                        "sliding capacity %lld must equal window %d (window-1 ring slots plus "
                        "the evicted-entry row)",
                        (long long)c->capacity, c->window);
    } else {
        if (c->capacity < 1)
            return fail(HDA_ERR_INVALID_ARGUMENT, "full-layer capacity %lld < 1",
                        (long long)c->capacity);
    }
    if (!c->k || !c->v) return fail(HDA_ERR_INVALID_ARGUMENT, "cache k/v pointer is NULL");
    if (!aligned16(c->k) || !aligned16(c->v))
        return fail(HDA_ERR_INVALID_ARGUMENT, "cache k/v must be 16-byte aligned");
    if (c->kv_dtype != HDA_KV_BF16 && c->kv_dtype != HDA_KV_FP8_E4M3)
        return fail(HDA_ERR_INVALID_ARGUMENT, "unknown kv_dtype %d", c->kv_dtype);
    if (c->kv_dtype == HDA_KV_FP8_E4M3) {
        if (!c->k_scale || !c->v_scale)
            return fail(HDA_ERR_INVALID_ARGUMENT, "an fp8 cache needs k_scale and v_scale");
        if ((reinterpret_cast<uintptr_t>(c->k_scale) | reinterpret_cast<uintptr_t>(c->v_scale)) & 3u)
            return fail(HDA_ERR_INVALID_ARGUMENT, "k_scale and v_scale must be 4-byte aligned");
        if (c->head_dim != hda::kHeadDim)
            return fail(HDA_ERR_UNSUPPORTED, "the fp8 cache is built for head_dim %d, got %d",
                        hda::kHeadDim, c->head_dim);
    }
    if (c->block_table) {
        if (layer != HDA_FULL)
            return fail(HDA_ERR_UNSUPPORTED, "the paged layout is for full layers (a sliding "
                        "layer's window is a fixed block)");
        if (c->page_size < 16 || c->page_size % 16)
            return fail(HDA_ERR_INVALID_ARGUMENT, "page_size %d must be a positive multiple of 16",
                        c->page_size);
        if (c->max_pages < 1 || c->num_pages < 1)
            return fail(HDA_ERR_INVALID_ARGUMENT, "max_pages %d and num_pages %lld must be >= 1",
                        c->max_pages, (long long)c->num_pages);
        if (c->capacity != (int64_t)c->max_pages * c->page_size)
            return fail(HDA_ERR_INVALID_ARGUMENT, "paged capacity %lld must be max_pages * "
                        "page_size = %lld", (long long)c->capacity,
                        (long long)c->max_pages * c->page_size);
        if (reinterpret_cast<uintptr_t>(c->block_table) & 3u)
            return fail(HDA_ERR_INVALID_ARGUMENT, "block_table must be 4-byte aligned");
    }
    return HDA_OK;
}

// The page table of a cache (block_table NULL: contiguous blocks).
hda::PageTable page_table(const hda_cache_desc *c) {
    hda::PageTable t{};
    t.block_table = c->block_table;
    t.page_size = c->page_size;
    t.max_pages = c->max_pages;
    t.num_pages = c->num_pages;
    return t;
}

// Keys per sequence the grid must cover.
int64_t max_keys_of(const hda_cache_desc *c, int layer, int32_t max_seq_len) {
    if (layer == HDA_SLIDING) return max_seq_len < c->window ? max_seq_len : c->window;
    return max_seq_len;
}

// Split plan: chunk size and chunks per (sequence, KV head).  Chunks are
// sized so that the grid holds enough workgroups to cover the chip (256
// CUs), between 64 and 256 keys; a single chunk needs no merge.
struct Plan {
    int chunk;
    int nsplit;
};

Plan plan_split(const hda_cache_desc *c, int layer, int64_t max_keys, int32_t chunk_keys) {
    Plan pl;
    if (chunk_keys > 0) {
        pl.chunk = chunk_keys;
    } else {
        const int64_t pairs = (int64_t)c->batch * c->num_kv_heads;
        int64_t want = (max_keys * pairs) / 512;  // aim at ~512 workgroups or more
        want = (want + 15) / 16 * 16;
        if (want < 64) want = 64;
        if (want > 256) want = 256;
        pl.chunk = (int)want;
    }
    pl.nsplit = (int)((max_keys + pl.chunk - 1) / pl.chunk);
    if (pl.nsplit < 1) pl.nsplit = 1;
    return pl;
}

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

// RoPE frequencies theta^(-2i/rot), i < rot/2, each rounded once from fp64
// to fp32 (Spark export page, `_angles`: fp32 inverse frequencies).
void fill_inv_freq(float *dst, double theta, int rot) {
    for (int i = 0; i < rot / 2; ++i)
        dst[i] = (float)(1.0 / std::pow(theta, (double)(2 * i) / (double)rot));
}

// Every decode workspace starts with one int per (sequence, KV head): the
// fused step's arrival counters, which it keeps at zero between calls.  The
// other paths lay their data out after this header and never write it, so
// one workspace can serve all of them.
size_t counter_header(const hda_cache_desc *c) {
    return up256((size_t)c->batch * c->num_kv_heads * sizeof(int));
}

// Chunk path: [header | part_o | part_lse].
size_t workspace_for(const hda_cache_desc *c, const Plan &pl) {
    if (pl.nsplit <= 1) return 0;
    const size_t slots = (size_t)c->batch * c->num_q_heads * pl.nsplit;
    return counter_header(c) + up256(slots * hda::kHeadDim * sizeof(float)) + slots * sizeof(float);
}

// Balanced streaming path (chunk_keys == 0): a grid of resident
// single-wave workgroups shares all 16-key rounds; partial slots = waves +
// (sequence, KV head) pairs.
// Window path (chunk_keys == 0, every sequence at most kPairMaxKeys keys):
// one workgroup per (sequence, KV head, half query group), no workspace.
bool use_pairs(const hda_cache_desc *c, int layer, int32_t max_seq_len, int32_t chunk_keys) {
    return chunk_keys == 0 && !c->block_table && max_keys_of(c, layer, max_seq_len) <= hda::kPairMaxKeys;
}

bool use_stream(const hda_cache_desc *c, int32_t chunk_keys) {
    return chunk_keys == 0 && c->batch <= hda::kStreamMaxBatch;
}

// Half as many waves as fit on the device at once (measured on MI355X: the
// full-layer decode at batch 64 x 4k streams ~10% faster than with every
// slot filled -- fewer segments to merge, less in flight), but no more than
// ~4 rounds (64 keys) each would need.
int stream_waves(const hda_cache_desc *c, int64_t max_keys) {
    const int64_t rounds = (int64_t)c->batch * c->num_kv_heads * ((max_keys + 15) / 16);
    int slots = hda::stream_wave_slots(c->num_q_heads / c->num_kv_heads);
    if (slots <= 0 || slots > hda::kStreamMaxWaves) slots = hda::kStreamMaxWaves;
    // (an fp8 cache: every slot -- its rounds are half the bytes and bound by
    // their compute chain, and two waves per SIMD measured ~10% faster)
    if (c->kv_dtype == HDA_KV_BF16) slots = slots / 2 > 0 ? slots / 2 : 1;
    int64_t w = (rounds + 3) / 4;
    if (w > slots) w = slots;
    if (w < 1) w = 1;
    return (int)w;
}

// Workspace of the streaming path: [part_o | part_lse | round prefix],
// each part 256-byte aligned.
struct StreamLayout {
    size_t o_off, lse_off, pre_off, bytes;
};

StreamLayout stream_layout(const hda_cache_desc *c, int waves) {
    const size_t slots = (size_t)waves + (size_t)c->batch * c->num_kv_heads;
    const size_t g = (size_t)(c->num_q_heads / c->num_kv_heads);
    auto up = up256;
    StreamLayout L;
    L.o_off = counter_header(c);
    L.lse_off = up(slots * g * hda::kHeadDim * sizeof(float));
    L.pre_off = L.lse_off + up(slots * g * sizeof(float));
    L.bytes = L.pre_off + up(((size_t)c->batch + 1) * sizeof(int));
    return L;
}

hda_status check_decode_shape(const hda_cache_desc *c, int layer, int32_t max_seq_len,
                              int32_t chunk_keys) {
    hda_status st = check_cache(c, layer);
    if (st != HDA_OK) return st;
    if (c->head_dim != hda::kHeadDim)
        return fail(HDA_ERR_UNSUPPORTED, "decode kernels are built for head_dim %d, got %d",
                    hda::kHeadDim, c->head_dim);
    const int g = c->num_q_heads / c->num_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16)
        return fail(HDA_ERR_UNSUPPORTED, "query group size %d not in {1,2,4,8,16}", g);
    if (c->capacity < 16)
        return fail(HDA_ERR_UNSUPPORTED, "decode kernels need a cache of at least 16 rows, got %lld",
                    (long long)c->capacity);
    if (max_seq_len < 1) return fail(HDA_ERR_INVALID_ARGUMENT, "max_seq_len %d < 1", max_seq_len);
    if (layer == HDA_FULL && max_seq_len > c->capacity)
        return fail(HDA_ERR_INVALID_ARGUMENT, "max_seq_len %d exceeds cache capacity %lld",
                    max_seq_len, (long long)c->capacity);
    if (chunk_keys != 0 && (chunk_keys < 16 || chunk_keys > hda::kMaxChunk || chunk_keys % 16))
        return fail(HDA_ERR_INVALID_ARGUMENT,
                    "chunk_keys %d must be 0 or a multiple of 16 in [16, %d]", chunk_keys,
                    hda::kMaxChunk);
    return HDA_OK;
}

// ------------------------------------------------------------ fused step
// Waves of the fused step: as many as fit on the device at once, but no
// more than ~4 rounds each at the longest keys the cache can hold.
int step_waves(const hda_cache_desc *c, int layer) {
    const int64_t keys = layer == HDA_SLIDING ? (int64_t)c->window : c->capacity;
    const int64_t rounds = (int64_t)c->batch * c->num_kv_heads * ((keys + 15) / 16);
    int slots = hda::step_wave_slots(c->num_q_heads / c->num_kv_heads, c->rotary_dim);
    if (slots <= 0 || slots > hda::kStreamMaxWaves) slots = hda::kStreamMaxWaves;
    int64_t w = (rounds + 3) / 4;
    if (w > slots) w = slots;
    if (w < 1) w = 1;
    return (int)w;
}

// [counters | part_o | part_lse]; partial slots = waves + pairs.
struct StepLayout {
    size_t o_off, lse_off, bytes;
};

// Window form of the step: sliding layers whose window fits one workgroup.
bool use_window_step(const hda_cache_desc *c, int layer) {
    return layer == HDA_SLIDING && c->window <= hda::kPairMaxKeys;
}

// Window step workspace: the counters, then (a key split over S
// workgroups) each workgroup's partial o [pairs * S, G, D] and lse
// [pairs * S, G], fp32.
StepLayout window_layout(const hda_cache_desc *c) {
    const int g = c->num_q_heads / c->num_kv_heads;
    const int64_t pairs = (int64_t)c->batch * c->num_kv_heads;
    const hda::WindowPlan plan = hda::window_step_plan(g, pairs, c->window);
    StepLayout L;
    L.o_off = counter_header(c);
    if (!plan.key_split) {
        L.lse_off = L.bytes = L.o_off;
        return L;
    }
    const size_t slots = (size_t)pairs * plan.parts * g;
    L.lse_off = L.o_off + up256(slots * hda::kHeadDim * sizeof(float));
    L.bytes = L.lse_off + up256(slots * sizeof(float));
    return L;
}

StepLayout step_layout(const hda_cache_desc *c, int waves) {
    const size_t slots = (size_t)waves + (size_t)c->batch * c->num_kv_heads;
    const size_t g = (size_t)(c->num_q_heads / c->num_kv_heads);
    StepLayout L;
    L.o_off = counter_header(c);
    L.lse_off = L.o_off + up256(slots * g * hda::kHeadDim * sizeof(float));
    L.bytes = L.lse_off + up256(slots * g * sizeof(float));
    return L;
}

hda_status check_step_shape(const hda_cache_desc *c, int layer) {
    hda_status st = check_cache(c, layer);
    if (st != HDA_OK) return st;
    if (c->head_dim != hda::kHeadDim)
        return fail(HDA_ERR_UNSUPPORTED, "decode kernels are built for head_dim %d, got %d",
                    hda::kHeadDim, c->head_dim);
    const int g = c->num_q_heads / c->num_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16)
        return fail(HDA_ERR_UNSUPPORTED, "query group size %d not in {1,2,4,8,16}", g);
    if (c->capacity < 16)
        return fail(HDA_ERR_UNSUPPORTED, "decode kernels need a cache of at least 16 rows, got %lld",
                    (long long)c->capacity);
    if (c->rotary_dim != 64 && c->rotary_dim != 256)
        return fail(HDA_ERR_UNSUPPORTED, "the fused step is built for rotary_dim 64 or 256, got %d",
                    c->rotary_dim);
    if (c->batch > hda::kStreamMaxBatch)
        return fail(HDA_ERR_UNSUPPORTED, "the fused step handles at most %d sequences, got %d",
                    hda::kStreamMaxBatch, c->batch);
    if (c->block_table && layer != HDA_FULL)
        return fail(HDA_ERR_UNSUPPORTED, "the step on a paged cache is built for full layers");
    if (c->kv_dtype != HDA_KV_BF16 && layer == HDA_SLIDING && c->window > hda::kPairMaxKeys)
        return fail(HDA_ERR_UNSUPPORTED, "the step on an fp8 cache is built for full layers and "
                    "sliding windows of at most %d keys (bf16 otherwise)", hda::kPairMaxKeys);
    return HDA_OK;
}

// Full layers: the streaming decode in its step form -- two launches, the
// stream over the rows held before this token with q rotated in registers,
// then the merge, which scores the new token and appends it.  Measured on
// MI355X faster than the one-launch form (whose merge across waves and
// in-loop append need about 330 registers) and than hda_rope_append +
// hda_decode_attn (one launch fewer).  Its workspace is the streaming
// path's, sized for a full block of keys, then the new keys' scores
// [batch, num_q_heads].
// (An fp8 cache as well takes half the resident slots here: the step form
// of its streaming kernel needs more than 256 registers, one wave per SIMD.)
int stream_step_waves(const hda_cache_desc *c) {
    const int w = stream_waves(c, c->capacity);
    return c->kv_dtype == HDA_KV_BF16 || w < 2 ? w : w / 2;
}
size_t stream_step_bytes(const hda_cache_desc *c) {
    return stream_layout(c, stream_step_waves(c)).bytes +
           up256((size_t)c->batch * c->num_q_heads * sizeof(float));
}

// ---------------------------------------------------------------- sparse
// Key splits for the sparse decode.  Shared-tile kernel (bf16 pool, up to 64
// heads): one workgroup per (token, split), so a token's index row is split
// until there are 256 workgroups (never below 64 keys a split, never above
// kSparseMaxSplitKeys), in multiples of 32 keys.  Head-group kernel: one
// workgroup per (token, split, group of 16 heads), split only when the
// tokens and head groups alone leave fewer than 256 workgroups, in
// multiples of 16 keys.
struct SparsePlan {
    int nsplit, split_keys;
};

SparsePlan sparse_plan(int32_t tokens, int32_t heads, int32_t topk, bool fp8) {
    const bool tiles = hda::sparse_uses_tiles(heads, fp8);
    const int64_t wgs = tiles ? (int64_t)tokens : (int64_t)tokens * (heads / hda::kSparseHeadsPerWave);
    const int64_t mult = tiles ? 32 : 16;
    int64_t ns = 1;
    if (wgs > 0 && wgs < 256 && topk > 64) ns = std::min<int64_t>((256 + wgs - 1) / wgs, (topk + 63) / 64);
    if (tiles) ns = std::max<int64_t>(ns, ((int64_t)topk + hda::kSparseMaxSplitKeys - 1) / hda::kSparseMaxSplitKeys);
    int64_t ks = topk > 0 ? (topk + ns - 1) / ns : mult;
    ks = (ks + mult - 1) / mult * mult;
    ns = topk > 0 ? (topk + ks - 1) / ks : 1;
    return {(int)ns, (int)ks};
}

size_t sparse_part_o_bytes(int32_t tokens, int32_t heads, const SparsePlan &pl) {
    const size_t b = (size_t)tokens * heads * pl.nsplit * hda::kSparseDv * sizeof(float);
    return (b + 255) / 256 * 256;
}

size_t sparse_workspace(int32_t tokens, int32_t heads, const SparsePlan &pl) {
    if (pl.nsplit <= 1) return 0;
    return sparse_part_o_bytes(tokens, heads, pl) + (size_t)tokens * heads * pl.nsplit * sizeof(float);
}

hda_status check_sparse_shape(int32_t tokens, int32_t heads, int32_t topk, int32_t dqk, int32_t dv) {
    if (tokens < 0 || topk < 0)
        return fail(HDA_ERR_INVALID_ARGUMENT, "tokens %d and topk %d must be >= 0", tokens, topk);
    if (heads <= 0 || heads % hda::kSparseHeadsPerWave)
        return fail(HDA_ERR_INVALID_ARGUMENT, "num_q_heads %d must be a positive multiple of %d", heads,
                    hda::kSparseHeadsPerWave);
    if (dqk != hda::kSparseDqk || dv != hda::kSparseDv)
        return fail(HDA_ERR_UNSUPPORTED, "sparse kernels are built for dqk %d / dv %d, got %d / %d",
                    hda::kSparseDqk, hda::kSparseDv, dqk, dv);
    int64_t blocks = 0;
    for (const bool fp8 : {false, true}) {
        const SparsePlan pl = sparse_plan(tokens, heads, topk, fp8);
        const int64_t units = ((int64_t)tokens + 7) / 8 * 8 * pl.nsplit;
        blocks = std::max(blocks, hda::sparse_uses_tiles(heads, fp8) ? units
                                                                     : units * (heads / hda::kSparseHeadsPerWave));
    }
    if (blocks > INT32_MAX || (int64_t)tokens * heads > INT32_MAX)
        return fail(HDA_ERR_UNSUPPORTED, "%d tokens x %d heads exceed the launch grid", tokens, heads);
    return HDA_OK;
}

}  // namespace

namespace hda {
// Records msg as the calling thread's last error (for entry points defined
// in other sources of the library).
hda_status report_error(hda_status st, const char *msg) { return fail(st, "%s", msg); }
}  // namespace hda

extern "C" {

const char *hda_status_string(hda_status s) {
    switch (s) {
        case HDA_OK: return "HDA_OK";
        case HDA_ERR_INVALID_ARGUMENT: return "HDA_ERR_INVALID_ARGUMENT";
        case HDA_ERR_UNSUPPORTED: return "HDA_ERR_UNSUPPORTED";
        case HDA_ERR_WORKSPACE: return "HDA_ERR_WORKSPACE";
        case HDA_ERR_HIP: return "HDA_ERR_HIP";
    }
    return "HDA_ERR_UNKNOWN";
}

const char *hda_last_error_message(void) { return g_last_error; }

hda_status hda_rope_append(void *q, const void *k_new, const void *v_new, const int32_t *pos,
                           hda_layer_type layer, const hda_cache_desc *cache, void *stream) {
    hda_status st = check_cache(cache, layer);
    if (st != HDA_OK) return st;
    if (!q || !k_new || !v_new || !pos)
        return fail(HDA_ERR_INVALID_ARGUMENT, "q, k_new, v_new and pos must be non-NULL");
    if (cache->rotary_dim % 16 || cache->rotary_dim > 512)
        return fail(HDA_ERR_UNSUPPORTED,
                    "rope_append handles rotary_dim in multiples of 16 up to 512, got %d",
                    cache->rotary_dim);
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new))
        return fail(HDA_ERR_INVALID_ARGUMENT, "q, k_new and v_new must be 16-byte aligned");
    if (cache->batch == 0) return ok();
    hda::RopeAppendParams p{};
    p.q = static_cast<uint16_t *>(q);
    p.k_new = static_cast<const uint16_t *>(k_new);
    p.v_new = static_cast<const uint16_t *>(v_new);
    p.pos = pos;
    p.k = static_cast<uint16_t *>(cache->k);
    p.v = static_cast<uint16_t *>(cache->v);
    p.pages = page_table(cache);
    const bool fp8 = cache->kv_dtype == HDA_KV_FP8_E4M3;
    if (fp8) {
        p.kq = static_cast<uint8_t *>(cache->k);
        p.vq = static_cast<uint8_t *>(cache->v);
        p.ks = cache->k_scale;
        p.vs = cache->v_scale;
    }
    p.capacity = cache->capacity;
    p.theta = cache->rope_theta;
    p.batch = cache->batch;
    p.num_q_heads = cache->num_q_heads;
    p.num_kv_heads = cache->num_kv_heads;
    p.head_dim = cache->head_dim;
    p.rotary_dim = cache->rotary_dim;
    p.window = cache->window;
    p.sliding = layer == HDA_SLIDING;
    fill_inv_freq(p.inv_freq, cache->rope_theta, cache->rotary_dim);
    hipError_t e = fp8 ? hda::launch_rope_append_fp8(p, static_cast<hipStream_t>(stream))
                       : hda::launch_rope_append(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(HDA_ERR_HIP, "rope_append launch failed: %s", hipGetErrorString(e));
    return ok();
}

size_t hda_decode_workspace_bytes(const hda_cache_desc *cache, hda_layer_type layer,
                                  int32_t max_seq_len, int32_t chunk_keys) {
    if (check_decode_shape(cache, layer, max_seq_len, chunk_keys) != HDA_OK) return 0;
    const int64_t mk = max_keys_of(cache, layer, max_seq_len);
    if (use_pairs(cache, layer, max_seq_len, chunk_keys)) return 0;
    if (use_stream(cache, chunk_keys)) return stream_layout(cache, stream_waves(cache, mk)).bytes;
    return workspace_for(cache, plan_split(cache, layer, mk, chunk_keys));
}

namespace {

// Fills the decode parameter block shared by the one-call and two-stage forms.
hda::DecodeParams decode_params(const void *q, const hda_cache_desc *cache,
                                const int32_t *seq_lens, int layer, float scale,
                                int32_t max_seq_len, const Plan &pl) {
    hda::DecodeParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(cache->k);
    p.v = static_cast<const uint16_t *>(cache->v);
    p.pages = page_table(cache);
    if (cache->kv_dtype == HDA_KV_FP8_E4M3) {
        p.kq = static_cast<const uint8_t *>(cache->k);
        p.vq = static_cast<const uint8_t *>(cache->v);
        p.ks = cache->k_scale;
        p.vs = cache->v_scale;
    }
    p.seq_lens = seq_lens;
    p.capacity = cache->capacity;
    p.batch = cache->batch;
    p.num_q_heads = cache->num_q_heads;
    p.num_kv_heads = cache->num_kv_heads;
    p.window = cache->window;
    p.chunk = pl.chunk;
    p.nsplit = pl.nsplit;
    p.max_keys = max_seq_len;
    p.sliding = layer == HDA_SLIDING;
    p.scale_log2 = scale * 1.4426950408889634f;
    return p;
}

hda_status check_decode_io(const void *q, const int32_t *seq_lens, float scale) {
    if (!q || !seq_lens) return fail(HDA_ERR_INVALID_ARGUMENT, "q and seq_lens must be non-NULL");
    if (!aligned16(q)) return fail(HDA_ERR_INVALID_ARGUMENT, "q must be 16-byte aligned");
    if (!std::isfinite(scale)) return fail(HDA_ERR_INVALID_ARGUMENT, "scale must be finite");
    return HDA_OK;
}

// Optional fp32 arrays (sinks, gate logits, lse out): NULL or 4-byte aligned.
hda_status check_f32_ptrs(const float *sinks, const float *gate, const float *lse) {
    auto bad = [](const float *x) { return x && (reinterpret_cast<uintptr_t>(x) & 3u); };
    if (bad(sinks) || bad(gate) || bad(lse))
        return fail(HDA_ERR_INVALID_ARGUMENT, "sinks, gate and lse must be 4-byte aligned");
    return HDA_OK;
}

hda_status launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(HDA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

hda_status hda_decode_split_plan(const hda_cache_desc *cache, hda_layer_type layer,
                                 int32_t max_seq_len, int32_t chunk_keys, int32_t *chunk_out,
                                 int32_t *nsplit_out) {
    hda_status st = check_decode_shape(cache, layer, max_seq_len, chunk_keys);
    if (st != HDA_OK) return st;
    if (!chunk_out || !nsplit_out)
        return fail(HDA_ERR_INVALID_ARGUMENT, "chunk_out and nsplit_out must be non-NULL");
    const Plan pl = plan_split(cache, layer, max_keys_of(cache, layer, max_seq_len), chunk_keys);
    *chunk_out = pl.chunk;
    *nsplit_out = pl.nsplit;
    return ok();
}

hda_status hda_decode_attn(const void *q, const hda_cache_desc *cache, const int32_t *seq_lens,
                           hda_layer_type layer, const float *sinks, const float *gate, float scale,
                           void *out, float *lse, int32_t max_seq_len, int32_t chunk_keys,
                           void *workspace, size_t workspace_bytes, void *stream) {
    hda_status st = check_decode_shape(cache, layer, max_seq_len, chunk_keys);
    if (st != HDA_OK) return st;
    if ((st = check_decode_io(q, seq_lens, scale)) != HDA_OK) return st;
    if ((st = check_f32_ptrs(sinks, gate, lse)) != HDA_OK) return st;
    if (!out || !aligned16(out))
        return fail(HDA_ERR_INVALID_ARGUMENT, "out must be non-NULL and 16-byte aligned");
    if (cache->block_table && !use_stream(cache, chunk_keys))
        return fail(HDA_ERR_UNSUPPORTED, "a paged cache takes the streaming path: chunk_keys must "
                    "be 0 and batch at most %d", hda::kStreamMaxBatch);
    if (cache->kv_dtype == HDA_KV_FP8_E4M3 && !use_pairs(cache, layer, max_seq_len, chunk_keys) &&
        !use_stream(cache, chunk_keys))
        return fail(HDA_ERR_UNSUPPORTED, "an fp8 cache takes the window or streaming path: "
                    "chunk_keys must be 0 and batch at most %d", hda::kStreamMaxBatch);
    if (cache->batch == 0) return ok();
    const int g = cache->num_q_heads / cache->num_kv_heads;
    hipStream_t s = static_cast<hipStream_t>(stream);

    if (use_pairs(cache, layer, max_seq_len, chunk_keys)) {
        Plan one{hda::kMaxChunk, 1};
        hda::DecodeParams p = decode_params(q, cache, seq_lens, layer, scale, max_seq_len, one);
        p.sinks = sinks;
        p.gate = gate;
        p.out = static_cast<uint16_t *>(out);
        p.lse = lse;
        return launched(hda::launch_decode_pairs(p, g, s), "decode");
    }
    if (use_stream(cache, chunk_keys)) {
        const int64_t mk = max_keys_of(cache, layer, max_seq_len);
        const int waves = stream_waves(cache, mk);
        const StreamLayout L = stream_layout(cache, waves);
        if (!workspace || workspace_bytes < L.bytes)
            return fail(HDA_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu at %p", L.bytes,
                        workspace_bytes, workspace);
        if (!aligned16(workspace))
            return fail(HDA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
        Plan one{hda::kMaxChunk, 1};
        hda::DecodeParams p = decode_params(q, cache, seq_lens, layer, scale, max_seq_len, one);
        char *ws = static_cast<char *>(workspace);
        p.part_o = reinterpret_cast<float *>(ws + L.o_off);
        p.part_lse = reinterpret_cast<float *>(ws + L.lse_off);
        p.stream_pre = reinterpret_cast<int *>(ws + L.pre_off);
        p.sinks = sinks;
        p.gate = gate;
        p.out = static_cast<uint16_t *>(out);
        p.lse = lse;
        return launched(hda::launch_decode_stream(p, g, waves, s), "decode");
    }

    const Plan pl = plan_split(cache, layer, max_keys_of(cache, layer, max_seq_len), chunk_keys);
    const size_t need = workspace_for(cache, pl);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(HDA_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu at %p", need,
                    workspace_bytes, workspace);
    if (need > 0 && !aligned16(workspace))
        return fail(HDA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");

    hda::DecodeParams p = decode_params(q, cache, seq_lens, layer, scale, max_seq_len, pl);
    p.sinks = sinks;
    p.gate = gate;
    p.out = static_cast<uint16_t *>(out);
    p.lse = lse;
    if (pl.nsplit == 1)
        return launched(hda::launch_decode_chunks(p, g, true, s), "decode");

    const size_t slots = (size_t)cache->batch * cache->num_q_heads * pl.nsplit;
    char *ws = static_cast<char *>(workspace) + counter_header(cache);
    p.part_o = reinterpret_cast<float *>(ws);
    p.part_lse = reinterpret_cast<float *>(ws + up256(slots * hda::kHeadDim * sizeof(float)));
    hipError_t e = hda::launch_decode_chunks(p, g, false, s);
    if (e != hipSuccess) return launched(e, "decode partials");
    hda::MergeParams m{};
    m.part_o = p.part_o;
    m.part_lse = p.part_lse;
    m.sinks = sinks;
    m.gate = gate;
    m.out = p.out;
    m.lse = lse;
    m.batch = cache->batch;
    m.num_heads = cache->num_q_heads;
    m.nsplit = pl.nsplit;
    return launched(hda::launch_lse_merge(m, s), "lse merge");
}

hda_status hda_decode_attn_partials(const void *q, const hda_cache_desc *cache,
                                    const int32_t *seq_lens, hda_layer_type layer, float scale,
                                    int32_t max_seq_len, int32_t chunk_keys, float *part_o,
                                    float *part_lse, void *stream) {
    hda_status st = check_decode_shape(cache, layer, max_seq_len, chunk_keys);
    if (st != HDA_OK) return st;
    if ((st = check_decode_io(q, seq_lens, scale)) != HDA_OK) return st;
    if (!part_o || !part_lse || !aligned16(part_o))
        return fail(HDA_ERR_INVALID_ARGUMENT,
                    "part_o (16-byte aligned) and part_lse must be non-NULL");
    if (cache->block_table || cache->kv_dtype != HDA_KV_BF16)
        return fail(HDA_ERR_UNSUPPORTED, "partials are built for contiguous bf16 caches only");
    if (cache->batch == 0) return ok();
    const Plan pl = plan_split(cache, layer, max_keys_of(cache, layer, max_seq_len), chunk_keys);
    hda::DecodeParams p = decode_params(q, cache, seq_lens, layer, scale, max_seq_len, pl);
    p.part_o = part_o;
    p.part_lse = part_lse;
    const int g = cache->num_q_heads / cache->num_kv_heads;
    return launched(hda::launch_decode_chunks(p, g, false, static_cast<hipStream_t>(stream)),
                    "decode partials");
}

hda_status hda_lse_merge(const float *part_o, const float *part_lse, int32_t batch,
                         int32_t num_heads, int32_t nsplit, int32_t head_dim, const float *sinks,
                         const float *gate, void *out, float *lse, void *stream) {
    if (batch < 0 || num_heads <= 0 || nsplit < 1)
        return fail(HDA_ERR_INVALID_ARGUMENT, "need batch >= 0, num_heads > 0, nsplit >= 1");
    if (head_dim != hda::kHeadDim)
        return fail(HDA_ERR_UNSUPPORTED, "merge kernel is built for head_dim %d, got %d",
                    hda::kHeadDim, head_dim);
    if (!part_o || !part_lse || !out)
        return fail(HDA_ERR_INVALID_ARGUMENT, "part_o, part_lse and out must be non-NULL");
    hda_status st = check_f32_ptrs(sinks, gate, lse);
    if (st != HDA_OK) return st;
    if (batch == 0) return ok();
    hda::MergeParams m{};
    m.part_o = part_o;
    m.part_lse = part_lse;
    m.sinks = sinks;
    m.gate = gate;
    m.out = static_cast<uint16_t *>(out);
    m.lse = lse;
    m.batch = batch;
    m.num_heads = num_heads;
    m.nsplit = nsplit;
    return launched(hda::launch_lse_merge(m, static_cast<hipStream_t>(stream)), "lse merge");
}

size_t hda_decode_step_workspace_bytes(const hda_cache_desc *cache, hda_layer_type layer) {
    if (check_step_shape(cache, layer) != HDA_OK) return 0;
    if (use_window_step(cache, layer)) return window_layout(cache).bytes;
    if (layer == HDA_FULL) return stream_step_bytes(cache);
    return step_layout(cache, step_waves(cache, layer)).bytes;
}

hda_status hda_decode_step(const void *q, const void *k_new, const void *v_new, const int32_t *pos,
                           hda_layer_type layer, const hda_cache_desc *cache, const float *sinks,
                           const float *gate, float scale, void *out, float *lse, void *workspace,
                           size_t workspace_bytes, void *stream) {
    hda_status st = check_step_shape(cache, layer);
    if (st != HDA_OK) return st;
    if (!q || !k_new || !v_new || !pos || !out)
        return fail(HDA_ERR_INVALID_ARGUMENT, "q, k_new, v_new, pos and out must be non-NULL");
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
        return fail(HDA_ERR_INVALID_ARGUMENT, "q, k_new, v_new and out must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(pos) & 3u)
        return fail(HDA_ERR_INVALID_ARGUMENT, "pos must be 4-byte aligned");
    if ((st = check_f32_ptrs(sinks, gate, lse)) != HDA_OK) return st;
    if (!std::isfinite(scale)) return fail(HDA_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (layer == HDA_FULL) {
        const int waves = stream_step_waves(cache);
        const StreamLayout L = stream_layout(cache, waves);
        const size_t need = stream_step_bytes(cache);
        if (!workspace || workspace_bytes < need)
            return fail(HDA_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu at %p", need,
                        workspace_bytes, workspace);
        if (!aligned16(workspace))
            return fail(HDA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
        if (cache->batch == 0) return ok();
        Plan one{hda::kMaxChunk, 1};
        hda::DecodeParams p = decode_params(q, cache, nullptr, layer, scale, 0, one);
        char *ws = static_cast<char *>(workspace);
        p.part_o = reinterpret_cast<float *>(ws + L.o_off);
        p.part_lse = reinterpret_cast<float *>(ws + L.lse_off);
        p.stream_pre = reinterpret_cast<int *>(ws + L.pre_off);
        p.sinks = sinks;
        p.gate = gate;
        p.out = static_cast<uint16_t *>(out);
        p.lse = lse;
        hda::StreamStep ss{};
        ss.pos = pos;
        ss.k_new = static_cast<const uint16_t *>(k_new);
        ss.v_new = static_cast<const uint16_t *>(v_new);
        ss.k = static_cast<uint16_t *>(cache->k);
        ss.v = static_cast<uint16_t *>(cache->v);
        ss.s_new = reinterpret_cast<float *>(ws + L.bytes);
        if (cache->kv_dtype == HDA_KV_FP8_E4M3) {
            ss.k_scale = cache->k_scale;
            ss.v_scale = cache->v_scale;
        }
        ss.rotary_dim = cache->rotary_dim;
        fill_inv_freq(ss.inv_freq, cache->rope_theta, cache->rotary_dim);
        const int g = cache->num_q_heads / cache->num_kv_heads;
        return launched(hda::launch_decode_stream_step(p, ss, g, waves, static_cast<hipStream_t>(stream)),
                        "decode step");
    }
    const bool window = use_window_step(cache, layer);
    const int waves = window ? 0 : step_waves(cache, layer);
    const StepLayout L = window ? window_layout(cache) : step_layout(cache, waves);
    const size_t need = L.bytes;
    if (!workspace || workspace_bytes < need)
        return fail(HDA_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu at %p", need,
                    workspace_bytes, workspace);
    if (!aligned16(workspace)) return fail(HDA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    if (cache->batch == 0) return ok();
    hda::StepParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.k_new = static_cast<const uint16_t *>(k_new);
    p.v_new = static_cast<const uint16_t *>(v_new);
    p.pos = pos;
    p.k = static_cast<uint16_t *>(cache->k);
    p.v = static_cast<uint16_t *>(cache->v);
    if (cache->kv_dtype == HDA_KV_FP8_E4M3) {
        p.kq = static_cast<uint8_t *>(cache->k);
        p.vq = static_cast<uint8_t *>(cache->v);
        p.ks = cache->k_scale;
        p.vs = cache->v_scale;
    }
    p.sinks = sinks;
    p.gate = gate;
    p.out = static_cast<uint16_t *>(out);
    p.lse = lse;
    char *ws = static_cast<char *>(workspace);
    p.counters = reinterpret_cast<int *>(ws);
    p.part_o = reinterpret_cast<float *>(ws + L.o_off);
    p.part_lse = reinterpret_cast<float *>(ws + L.lse_off);
    p.capacity = cache->capacity;
    p.batch = cache->batch;
    p.num_q_heads = cache->num_q_heads;
    p.num_kv_heads = cache->num_kv_heads;
    p.window = cache->window;
    p.sliding = layer == HDA_SLIDING;
    p.scale_log2 = scale * 1.4426950408889634f;
    fill_inv_freq(p.inv_freq, cache->rope_theta, cache->rotary_dim);
    const int g = cache->num_q_heads / cache->num_kv_heads;
    if (window)
        return launched(hda::launch_decode_window_step(p, g, cache->rotary_dim, static_cast<hipStream_t>(stream)),
                        "decode step");
    return launched(hda::launch_decode_step(p, g, cache->rotary_dim, waves, static_cast<hipStream_t>(stream)),
                    "decode step");
}

namespace {

hda_status check_multi_shape(const hda_cache_desc *c, int layer, int32_t tokens,
                             int32_t max_seq_len) {
    hda_status st = check_cache(c, layer);
    if (st != HDA_OK) return st;
    if (c->head_dim != hda::kHeadDim)
        return fail(HDA_ERR_UNSUPPORTED, "decode kernels are built for head_dim %d, got %d",
                    hda::kHeadDim, c->head_dim);
    const int g = c->num_q_heads / c->num_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16)
        return fail(HDA_ERR_UNSUPPORTED, "query group size %d not in {1,2,4,8,16}", g);
    if (tokens < 1 || tokens > hda::kMultiMaxTokens)
        return fail(HDA_ERR_UNSUPPORTED, "a chunk holds 1..%d tokens, got %d", hda::kMultiMaxTokens, tokens);
    if (c->rotary_dim % 16)
        return fail(HDA_ERR_UNSUPPORTED, "rotary_dim %d is not a multiple of 16", c->rotary_dim);
    if (c->capacity < 16 || (g * tokens > 16 && c->capacity < 32))
        return fail(HDA_ERR_UNSUPPORTED, "chunk decode needs a cache of at least %d rows",
                    g * tokens > 16 ? 32 : 16);
    if (c->block_table || c->kv_dtype != HDA_KV_BF16)
        return fail(HDA_ERR_UNSUPPORTED, "chunk decode is built for contiguous bf16 caches");
    if (max_seq_len < 1)
        return fail(HDA_ERR_INVALID_ARGUMENT, "max_seq_len %d < 1", max_seq_len);
    return HDA_OK;
}

// Workgroups per (sequence, KV head) of the chunk decode.  Measured on
// MI355X (4-token chunks, bf16-dot P.V): at 128 pairs a 32-round sliding
// window and a 4k full layer are fastest split in 2; at 16 pairs splits of
// 4 and 8 -- more parts than that pay more in merge traffic than they
// gain.  So: about 256 workgroups (128 when there are few pairs), each with
// at least 16 rounds (8 with few pairs).  max_seq_len bounds pos + tokens; it only sizes the
// split (every workgroup takes its share of the rounds the sequence has).
int multi_split(const hda_cache_desc *c, int layer, int32_t tokens, int32_t max_seq_len) {
    int64_t n_old = (int64_t)max_seq_len - tokens;
    if (n_old < 0) n_old = 0;
    const int64_t lim = layer == HDA_SLIDING ? (int64_t)c->window - 1 : c->capacity;
    if (n_old > lim) n_old = lim;
    const int64_t pairs = (int64_t)c->batch * c->num_kv_heads;
    const int64_t g = c->num_q_heads / c->num_kv_heads;
    if (g * tokens > 16) {
        // the prefill kernel: cut the key tiles into ranges when its row
        // blocks leave the GPU short of 256 workgroups, keeping 8 tiles a range
        const int64_t blocks = pairs * ((g * tokens + hda::kPrefillRows - 1) / hda::kPrefillRows);
        const int64_t tiles = (n_old + tokens + hda::kPrefillTile - 1) / hda::kPrefillTile;
        int s = 1;
        while (s < hda::kPrefillMaxSplit && blocks * s < 256 && tiles / (2 * s) >= 8) s *= 2;
        return s;
    }
    const int64_t rounds = (n_old + 15) / 16;
    // sliding, 128 pairs or more, one token: one workgroup per pair, which
    // also does the append (measured at 128 pairs: 25.2 us against 25.4 for
    // split 2 + the merge launch, which then writes the append); two tokens
    // or more split as below (4 tokens: 30.7 against 31.5 us)
    if (layer == HDA_SLIDING && pairs >= 128 && tokens == 1) return 1;
    const bool many = pairs >= 64;
    const int64_t target = many ? 256 : 128, min_rounds = many ? 16 : 8;
    int64_t s = pairs > 0 ? (target + pairs - 1) / pairs : 1;
    const int64_t by_rounds = rounds / min_rounds;
    if (s > by_rounds) s = by_rounds;
    if (s > 64) s = 64;
    return s < 1 ? 1 : (int)s;
}

// Chunk-decode workspace: the rotated new K rows (bf16 [B, T, Hkv, D]),
// then, for a split, each part's partial o [rows, D] and lse [rows].
size_t multi_krot_bytes(const hda_cache_desc *c, int32_t tokens) {
    return up256((size_t)c->batch * tokens * c->num_kv_heads * hda::kHeadDim * sizeof(uint16_t));
}
size_t multi_workspace(const hda_cache_desc *c, int split, int32_t tokens) {
    size_t bytes = multi_krot_bytes(c, tokens);
    if (split <= 1) return bytes;
    const size_t rows = (size_t)c->batch * c->num_kv_heads * split * tokens *
                        (c->num_q_heads / c->num_kv_heads);
    return bytes + up256(rows * hda::kHeadDim * sizeof(float)) + rows * sizeof(float);
}

}  // namespace

size_t hda_decode_multi_workspace_bytes(const hda_cache_desc *cache, hda_layer_type layer,
                                        int32_t tokens, int32_t max_seq_len) {
    if (check_multi_shape(cache, layer, tokens, max_seq_len) != HDA_OK) return 0;
    return multi_workspace(cache, multi_split(cache, layer, tokens, max_seq_len), tokens);
}

hda_status hda_decode_multi(void *q, const void *k_new, const void *v_new, const int32_t *pos,
                            int32_t tokens, hda_layer_type layer, const hda_cache_desc *cache,
                            const float *sinks, const float *gate, float scale, void *out,
                            float *lse, int32_t max_seq_len, void *workspace,
                            size_t workspace_bytes, void *stream) {
    hda_status st = check_multi_shape(cache, layer, tokens, max_seq_len);
    if (st != HDA_OK) return st;
    if (!q || !k_new || !v_new || !pos || !out)
        return fail(HDA_ERR_INVALID_ARGUMENT, "q, k_new, v_new, pos and out must be non-NULL");
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
        return fail(HDA_ERR_INVALID_ARGUMENT, "q, k_new, v_new and out must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(pos) & 3u)
        return fail(HDA_ERR_INVALID_ARGUMENT, "pos must be 4-byte aligned");
    if ((st = check_f32_ptrs(sinks, gate, lse)) != HDA_OK) return st;
    if (!(scale > 0.f) || !std::isfinite(scale))
        return fail(HDA_ERR_INVALID_ARGUMENT, "scale must be positive and finite");
    const int g = cache->num_q_heads / cache->num_kv_heads;
    const int split = multi_split(cache, layer, tokens, max_seq_len);
    const size_t need = multi_workspace(cache, split, tokens);
    if (cache->batch == 0) return ok();
    if (!workspace || workspace_bytes < need)
        return fail(HDA_ERR_WORKSPACE, "chunk decode needs a %zu-byte workspace, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace))
        return fail(HDA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    hda::MultiParams p{};
    p.split = split;
    char *ws = static_cast<char *>(workspace);
    p.k_rot = reinterpret_cast<uint16_t *>(ws);
    if (split > 1) {
        const size_t rows = (size_t)cache->batch * cache->num_kv_heads * split * tokens * g;
        p.part_o = reinterpret_cast<float *>(ws + multi_krot_bytes(cache, tokens));
        p.part_lse = reinterpret_cast<float *>(ws + multi_krot_bytes(cache, tokens) +
                                               up256(rows * hda::kHeadDim * sizeof(float)));
    }
    p.q = static_cast<uint16_t *>(q);
    p.k_new = static_cast<const uint16_t *>(k_new);
    p.v_new = static_cast<const uint16_t *>(v_new);
    p.pos = pos;
    p.k = static_cast<uint16_t *>(cache->k);
    p.v = static_cast<uint16_t *>(cache->v);
    p.sinks = sinks;
    p.gate = gate;
    p.out = static_cast<uint16_t *>(out);
    p.lse = lse;
    p.capacity = cache->capacity;
    p.batch = cache->batch;
    p.tokens = tokens;
    p.num_q_heads = cache->num_q_heads;
    p.num_kv_heads = cache->num_kv_heads;
    p.rotary_dim = cache->rotary_dim;
    p.window = cache->window;
    p.sliding = layer == HDA_SLIDING;
    p.scale_log2 = scale * 1.4426950408889634f;
    fill_inv_freq(p.inv_freq, cache->rope_theta, cache->rotary_dim);
    return launched(hda::launch_decode_multi(p, g, static_cast<hipStream_t>(stream)), "chunk decode");
}

}  // extern "C"

namespace {

// Shared by the bf16 and fp8 sparse calls: kv is the bf16 pool, or kv8 /
// kv_scale the fp8 one.
hda_status sparse_call(const void *q, const void *kv, const uint8_t *kv8, const float *kv_scale,
                       int64_t pool_rows, const int32_t *indices, int32_t tokens, int32_t topk,
                       const int32_t *topk_length, int32_t num_q_heads, int32_t dqk, int32_t dv,
                       const float *sinks, float scale, void *out, float *lse, void *workspace,
                       size_t workspace_bytes, void *stream) {
    hda_status st = check_sparse_shape(tokens, num_q_heads, topk, dqk, dv);
    if (st != HDA_OK) return st;
    if (pool_rows < 1) return fail(HDA_ERR_INVALID_ARGUMENT, "pool_rows %lld < 1", (long long)pool_rows);
    if (!q || !(kv || kv8) || !indices || !out || (kv8 && !kv_scale))
        return fail(HDA_ERR_INVALID_ARGUMENT, "q, the pool (codes and scales for fp8), indices and out must be non-NULL");
    if (!aligned16(q) || !aligned16(kv ? kv : kv8) || !aligned16(out))
        return fail(HDA_ERR_INVALID_ARGUMENT, "q, the pool and out must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(indices) & 3u) || (topk_length && (reinterpret_cast<uintptr_t>(topk_length) & 3u)) ||
        (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) || (sinks && (reinterpret_cast<uintptr_t>(sinks) & 3u)) ||
        (kv_scale && (reinterpret_cast<uintptr_t>(kv_scale) & 3u)))
        return fail(HDA_ERR_INVALID_ARGUMENT, "indices, topk_length, sinks, scales and lse must be 4-byte aligned");
    if (!std::isfinite(scale)) return fail(HDA_ERR_INVALID_ARGUMENT, "scale must be finite");
    const SparsePlan pl = sparse_plan(tokens, num_q_heads, topk, kv8 != nullptr);
    const size_t need = sparse_workspace(tokens, num_q_heads, pl);
    if (need && (!workspace || workspace_bytes < need))
        return fail(HDA_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu%s", need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    if (need && !aligned16(workspace))
        return fail(HDA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    if (tokens == 0) return ok();
    hda::SparseParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.kv = static_cast<const uint16_t *>(kv);
    p.kv8 = kv8;
    p.kv_scale = kv_scale;
    p.indices = indices;
    p.topk_length = topk_length;
    p.sinks = sinks;
    p.out = static_cast<uint16_t *>(out);
    p.lse = lse;
    if (need) {
        p.part_o = static_cast<float *>(workspace);
        p.part_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) + sparse_part_o_bytes(tokens, num_q_heads, pl));
    }
    p.pool_rows = pool_rows;
    p.tokens = tokens;
    p.num_q_heads = num_q_heads;
    p.topk = topk;
    p.nsplit = pl.nsplit;
    p.split_keys = pl.split_keys;
    p.scale_log2 = scale * 1.4426950408889634f;
    return launched(hda::launch_sparse_decode(p, static_cast<hipStream_t>(stream)), "sparse decode");
}

}  // namespace

extern "C" {

hda_status hda_sparse_decode_attn(const void *q, const void *kv, int64_t pool_rows,
                                  const int32_t *indices, int32_t tokens, int32_t topk,
                                  const int32_t *topk_length, int32_t num_q_heads, int32_t dqk,
                                  int32_t dv, const float *sinks, float scale, void *out,
                                  float *lse, void *workspace, size_t workspace_bytes,
                                  void *stream) {
    if (!kv) return fail(HDA_ERR_INVALID_ARGUMENT, "kv must be non-NULL");
    return sparse_call(q, kv, nullptr, nullptr, pool_rows, indices, tokens, topk, topk_length,
                       num_q_heads, dqk, dv, sinks, scale, out, lse, workspace, workspace_bytes, stream);
}

hda_status hda_sparse_decode_attn_fp8(const void *q, const uint8_t *kv_codes, const float *kv_scales,
                                      int64_t pool_rows, const int32_t *indices, int32_t tokens,
                                      int32_t topk, int32_t num_q_heads, int32_t dqk, int32_t dv,
                                      const float *sinks, float scale, void *out, float *lse,
                                      void *workspace, size_t workspace_bytes, void *stream) {
    if (!kv_codes || !kv_scales)
        return fail(HDA_ERR_INVALID_ARGUMENT, "kv_codes and kv_scales must be non-NULL");
    return sparse_call(q, nullptr, kv_codes, kv_scales, pool_rows, indices, tokens, topk, nullptr,
                       num_q_heads, dqk, dv, sinks, scale, out, lse, workspace, workspace_bytes, stream);
}

size_t hda_sparse_workspace_bytes(int32_t tokens, int32_t num_q_heads, int32_t topk, int32_t dv) {
    if (check_sparse_shape(tokens, num_q_heads, topk, hda::kSparseDqk, dv) != HDA_OK) return 0;
    // enough for either pool type
    return std::max(sparse_workspace(tokens, num_q_heads, sparse_plan(tokens, num_q_heads, topk, false)),
                    sparse_workspace(tokens, num_q_heads, sparse_plan(tokens, num_q_heads, topk, true)));
}

}  // extern "C"
