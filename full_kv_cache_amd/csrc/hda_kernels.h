// hda_kernels.h -- kernel parameter blocks and launchers (library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace hda {

// Workgroups of `kernel` (blocks of `threads`, no dynamic LDS) resident on
// the current device at once: CUs x occupancy per CU, cached per device
// ordinal (several host threads may ask; 0 in a cache entry = not known
// yet).  Returns 0 when no device answers.
constexpr int kMaxDevices = 64;
inline int resident_slots(const void *kernel, int threads, std::atomic<int> (&cache)[kMaxDevices]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 0;
    }
    const int known = cache[dev].load(std::memory_order_relaxed);
    if (known > 0) return known;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    cache[dev].store(cus * per_cu, std::memory_order_relaxed);
    return cus * per_cu;
}

constexpr int kHeadDim = 256;     // head dim the decode kernels are built for
constexpr int kMaxChunk = 512;    // most keys one decode workgroup scores
constexpr int kDecodeThreads = 256;
constexpr int kStreamMaxBatch = 4096;  // sequences the balanced streaming path handles
constexpr int kStreamMaxWaves = 2048;  // its grid: 256 CUs x 8 resident waves
constexpr int kPairWaves = 8;          // waves per workgroup of the window decomposition
constexpr int kPairMaxKeys = 1024;     // windows up to this size use it by default

// Paged cache addressing (block_table null: contiguous [B, Hkv, cap, D]
// blocks): row r of sequence b is row r % page_size of pool page
// block_table[b * max_pages + r / page_size], clamped into [0, num_pages).
struct PageTable {
    const int32_t *block_table;  // [B, max_pages] or null
    int page_size, max_pages;
    int64_t num_pages;
};

// Pool page holding row `row` of sequence b, clamped into [0, num_pages).
__device__ __forceinline__ int64_t page_of(const PageTable &pt, int b, int64_t row) {
    const int64_t pg = pt.block_table[(int64_t)b * pt.max_pages + row / pt.page_size];
    return pg < 0 ? 0 : pg >= pt.num_pages ? pt.num_pages - 1 : pg;
}

struct RopeAppendParams {
    uint16_t *q;
    const uint16_t *k_new;
    const uint16_t *v_new;
    const int32_t *pos;
    uint16_t *k, *v;            // [B, Hkv, capacity, D]; sliding: row window-1 = evicted entry
    PageTable pages;            // full layers: paged pools instead of blocks
    uint8_t *kq, *vq;           // fp8 cache: e4m3 codes in place of k, v (else null)
    float *ks, *vs;             // fp8 cache: one scale per row [B, Hkv, capacity]
    int64_t capacity;
    double theta;
    int batch, num_q_heads, num_kv_heads, head_dim, rotary_dim, window;
    bool sliding;
    float inv_freq[256];        // fp32 theta^(-2i/rot), i < rot/2 (rot <= 512)
};

struct DecodeParams {
    const uint16_t *q;          // [B, Hq, D]
    const uint16_t *k, *v;      // [B, Hkv, cap, D], or page pools [pages, Hkv, page_size, D]
    PageTable pages;
    const uint8_t *kq, *vq;     // fp8 cache: e4m3 codes, same layout (else null)
    const float *ks, *vs;       // fp8 cache: one scale per row
    const int32_t *seq_lens;    // [B]
    const float *sinks;         // [Hq] or null
    const float *gate;          // [B, Hq] output-gate logits or null
    uint16_t *out;              // [B, Hq, D]
    float *lse;                 // [B, Hq] or null
    float *part_o;              // [B, Hq, S, D]
    float *part_lse;            // [B, Hq, S]
    int *stream_pre;            // [B + 1] rounds before each sequence (streaming path)
    int64_t capacity;
    int batch, num_q_heads, num_kv_heads, window;
    int chunk;                  // keys per chunk (multiple of 16, <= kMaxChunk)
    int nsplit;                 // chunks per (b, kv head) in the grid
    int max_keys;               // host bound on keys per sequence (max_seq_len)
    int sliding;                // keys = min(seq_len, window) instead of seq_len
    float scale_log2;           // softmax scale * log2(e)
};

// Fused decode step (RoPE + append + attention + merge in one launch).
struct StepParams {
    const uint16_t *q;          // [B, Hq, D], read only (rotated in registers)
    const uint16_t *k_new, *v_new;  // [B, Hkv, D]
    const int32_t *pos;         // [B]
    uint16_t *k, *v;            // [B, Hkv, cap, D]
    uint8_t *kq, *vq;           // fp8 cache (window form): e4m3 codes in place of k, v
    float *ks, *vs;             // fp8 cache: one scale per row [B, Hkv, cap]
    const float *sinks;         // [Hq] or null
    const float *gate;          // [B, Hq] output-gate logits or null
    uint16_t *out;              // [B, Hq, D]
    float *lse;                 // [B, Hq] or null
    float *part_o;              // [slots, G, D], slot = wave + pair
    float *part_lse;            // [slots, G]
    int *counters;              // [B * Hkv], zero before and after every launch
    int64_t capacity;
    int batch, num_q_heads, num_kv_heads, window;
    int sliding;
    float scale_log2;
    float inv_freq[kHeadDim / 2];  // fp32 theta^(-2i/rot), i < rot/2
};

// Step form of the streaming decode (hda_decode_step on a full layer): the
// keys of sequence b are the rows its block held before this token,
// min(pos, capacity) (none for pos < 0); the streaming kernel rotates q in
// registers, and the wave holding a pair's first round scores the new key
// (row pos when pos < capacity) and appends it; the merge folds that score
// in (and does both itself for a pair with no held rows).
struct StreamStep {
    const int32_t *pos;              // [B]
    const uint16_t *k_new, *v_new;   // [B, Hkv, D]
    uint16_t *k, *v;                 // the cache (or page pools), written at row pos
    float *k_scale, *v_scale;        // fp8 cache: per-row scales (else null); codes at k, v
    float *s_new;                    // [B, Hq] the new key's score (natural log units)
    int rotary_dim;                  // 64 or 256
    float inv_freq[kHeadDim / 2];    // fp32 theta^(-2i/rot), i < rot/2
};
struct NoStep {};

struct MergeParams {
    const float *part_o;        // [B, H, nsplit, D]
    const float *part_lse;      // [B, H, nsplit]
    const float *sinks;         // [H] or null
    const float *gate;          // [B, H] output-gate logits or null
    uint16_t *out;              // [B, H, D]
    float *lse;                 // [B, H] or null
    int batch, num_heads, nsplit;
};

// Sparse top-k decode over one latent KV head shared by all query heads.
constexpr int kSparseDqk = 576;    // key dims (latent + rotary part)
constexpr int kSparseDv = 512;     // value dims: the leading part of each row
constexpr int kSparseHeadsPerWave = 16;
constexpr int kSparseMaxSplitKeys = 2048;  // keys of one split of the shared-tile kernel
#ifndef HDA_SPARSE_WAVES
#define HDA_SPARSE_WAVES 4
#endif
constexpr int kSparseWaves = HDA_SPARSE_WAVES;  // waves per workgroup, each takes 16-key tiles in turn

struct SparseParams {
    const uint16_t *q;          // [T, Hq, Dqk]
    const uint16_t *kv;         // [pool_rows, Dqk] (bf16 pool)
    const uint8_t *kv8;         // [pool_rows, Dqk] e4m3 codes (fp8 pool; kv unused), else null
    const float *kv_scale;      // [pool_rows] fp8 pool: each row's scale
    const int32_t *indices;     // [T, topk]
    const int32_t *topk_length; // [T] or null
    const float *sinks;         // [Hq] or null
    uint16_t *out;              // [T, Hq, Dv]
    float *lse;                 // [T, Hq] or null
    float *part_o;              // [T, Hq, nsplit, Dv] (nsplit > 1)
    float *part_lse;            // [T, Hq, nsplit]
    int64_t pool_rows;
    int tokens, num_q_heads, topk;
    int nsplit, split_keys;     // key splits per token; keys per split (multiple of 16)
    float scale_log2;           // softmax scale * log2(e)
};

// Decode of a chunk of `tokens` new tokens per sequence (q [B, T, Hq, D],
// k_new / v_new [B, T, Hkv, D]; contiguous bf16 cache; tokens <= 512).
constexpr int kMultiMaxTokens = 512;  // a chunk's tokens: the window never drops a chunk key
constexpr int kPrefillRows = 128;     // query rows per workgroup of the prefill kernel
constexpr int kPrefillTile = 32;      // keys per tile of the prefill kernel
constexpr int kPrefillMaxSplit = 4;   // key splits of the prefill kernel

struct MultiParams {
    uint16_t *q;                // rotated in place
    const uint16_t *k_new;      // read only
    uint16_t *k_rot;            // [B, T, Hkv, D] workspace: the rotated new K
    const uint16_t *v_new;
    const int32_t *pos;         // [B] position of token 0
    uint16_t *k, *v;            // [B, Hkv, cap, D]
    const float *sinks;         // [Hq] or null
    const float *gate;          // [B, T, Hq] or null
    uint16_t *out;              // [B, T, Hq, D]
    float *lse;                 // [B, T, Hq] or null
    int64_t capacity;
    int batch, tokens, num_q_heads, num_kv_heads, rotary_dim, window;
    int sliding;
    int split;                  // workgroups per (sequence, KV head); > 1: partials + merge
    float *part_o;              // [B * Hkv * split, T * G, D] (split > 1)
    float *part_lse;            // [B * Hkv * split, T * G]
    float scale_log2;
    float inv_freq[kHeadDim / 2];
};
hipError_t launch_decode_multi(const MultiParams &p, int group, hipStream_t stream);

hipError_t launch_rope_append(const RopeAppendParams &p, hipStream_t stream);
// The same for an fp8 cache (kq/vq/ks/vs set; head_dim 256): the new K and
// V rows are quantized into e4m3 codes with one scale per row.
hipError_t launch_rope_append_fp8(const RopeAppendParams &p, hipStream_t stream);

// Grid of (token, key split, 16-head group) workgroups; nsplit == 1 writes
// out / lse with the sink, otherwise partials and then their merge.  An fp8
// pool (kv8 / kv_scale set) takes the kernel's fp8 form.
hipError_t launch_sparse_decode(const SparseParams &p, hipStream_t stream);
// Whether the sparse call runs the shared-tile kernel (one workgroup per
// (token, split) for all heads, bf16 or fp8 pool, up to kSparseTileHeads
// heads; its splits hold at most kSparseMaxSplitKeys keys, a multiple of 32)
// or the head-group kernel (splits a multiple of 16).
constexpr int kSparseTileHeads = 64;
inline bool sparse_uses_tiles(int num_q_heads, bool fp8) { return num_q_heads <= kSparseTileHeads; }

// Chunk kernel over grid (nsplit, Hkv, B).  final_out: nsplit must be 1 and
// the kernel writes out/lse with the sink; otherwise it writes partials.
// group must be one of 1, 2, 4, 8, 16.  Needs capacity >= 16.
hipError_t launch_decode_chunks(const DecodeParams &p, int group, bool final_out, hipStream_t stream);

// Balanced streaming path: `waves` resident single-wave workgroups share
// all 16-key rounds evenly; partials in slots (wave + pair) of part_o /
// part_lse, then the merge writes out / lse with the sink.  Needs
// capacity >= 16 and batch <= kStreamMaxBatch.
hipError_t launch_decode_stream(const DecodeParams &p, int group, int waves, hipStream_t stream);
// Streaming kernel in its step form, then the merge with the new token and
// the append (p.seq_lens unused).
hipError_t launch_decode_stream_step(const DecodeParams &p, const StreamStep &s, int group, int waves,
                                     hipStream_t stream);

// Single-wave workgroups of the streaming kernel that fit on the device at
// once (occupancy x CUs); 0 if no device is available.
int stream_wave_slots(int group);

// Window decomposition: one workgroup per (sequence, KV head, half of the
// query group); writes out / lse with the sink directly (no workspace).
// Needs capacity >= 16.
hipError_t launch_decode_pairs(const DecodeParams &p, int group, hipStream_t stream);

// Fused step over `waves` resident single-wave workgroups; group in
// {1, 2, 4, 8, 16}, rotary_dim in {64, 256}.  Needs capacity >= 16 and
// batch <= kStreamMaxBatch.
hipError_t launch_decode_step(const StepParams &p, int group, int rotary_dim, int waves,
                              hipStream_t stream);
int step_wave_slots(int group, int rotary_dim);

// The streaming merge alone (partials of `waves` streaming waves, prefix in
// p.stream_pre): out / lse with the sink.
hipError_t launch_stream_merge(const DecodeParams &p, int waves, hipStream_t stream);

// Split of the window step over the workgroups of one (sequence, KV head).
// Head split: each of `parts` workgroups serves heads_per_part query heads
// over every key (the pair's rows are read once per part, the second time
// mostly from the XCD's L2).  Key split: each of `parts` workgroups serves
// every query head over 1/parts of the keys, then the last to finish
// merges the partials (measured on MI355X: the merge's round trip through
// memory costs more than re-reading rows from L2, so it is taken only when
// head parts alone would leave CUs idle).  Query groups of 8 and 16 always
// split heads, 4 per workgroup.  Up to 4: two head parts (G = 4: 2 heads
// each; G = 2: 1; G = 1: one part) while that gives at least 256
// workgroups; otherwise a key split that doubles while the pairs give
// fewer than 256 workgroups, up to 8 parts of at least 4 rounds of 16 keys.
struct WindowPlan {
    bool key_split;
    int parts, heads_per_part;
};
inline WindowPlan window_step_plan(int group, int64_t pairs, int window) {
    if (group >= 8) return {false, group / 4, 4};
    const int hp = group >= 2 ? 2 : 1;  // head parts
    if (pairs * hp >= 256) return {false, hp, group / hp};
    const int rounds = (window + 15) / 16;
    int s = 1;
    while (s < 8 && pairs * s < 256 && rounds / (2 * s) >= 4) s *= 2;
    if (s == 1) return {false, hp, group / hp};
    return {true, s, group};
}

// Window form of the fused step (sliding layers with window <=
// kPairMaxKeys == capacity), split as window_step_plan says.  Needs the
// counters of StepParams and, for a key split over S parts, part_o
// [pairs * S, G, D] and part_lse [pairs * S, G].
hipError_t launch_decode_window_step(const StepParams &p, int group, int rotary_dim, hipStream_t stream);

hipError_t launch_lse_merge(const MergeParams &p, hipStream_t stream);

}  // namespace hda
