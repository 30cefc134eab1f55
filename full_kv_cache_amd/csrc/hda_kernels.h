// hda_kernels.h -- kernel parameter blocks and launchers (library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hda {

constexpr int kHeadDim = 256;     // head dim the decode kernels are built for
constexpr int kMaxChunk = 512;    // most keys one decode workgroup scores
constexpr int kDecodeThreads = 256;

struct RopeAppendParams {
    uint16_t *q;
    const uint16_t *k_new;
    const uint16_t *v_new;
    const int32_t *pos;
    uint16_t *k, *v;
    uint16_t *k_evict, *v_evict;
    int64_t capacity;
    double theta;
    int batch, num_q_heads, num_kv_heads, head_dim, rotary_dim, window;
    bool sliding;
};

struct DecodeParams {
    const uint16_t *q;          // [B, Hq, D]
    const uint16_t *k, *v;      // [B, Hkv, cap, D]
    const uint16_t *kev, *vev;  // [B, Hkv, D] side rows (sliding)
    const int32_t *seq_lens;    // [B]
    const float *sinks;         // [Hq] or null
    uint16_t *out;              // [B, Hq, D]
    float *lse;                 // [B, Hq] or null
    float *part_o;              // [B, Hq, S, D]
    float *part_lse;            // [B, Hq, S]
    int64_t capacity;
    int batch, num_q_heads, num_kv_heads, window;
    int chunk;                  // keys per chunk (multiple of 16, <= kMaxChunk)
    int nsplit;                 // chunks per (b, kv head) in the grid
    int max_keys;               // host bound on keys per sequence
    float scale_log2;           // softmax scale * log2(e)
};

struct MergeParams {
    const float *part_o;        // [B, H, nsplit, D]
    const float *part_lse;      // [B, H, nsplit]
    const float *sinks;         // [H] or null
    uint16_t *out;              // [B, H, D]
    float *lse;                 // [B, H] or null
    int batch, num_heads, nsplit;
};

hipError_t launch_rope_append(const RopeAppendParams &p, hipStream_t stream);

// Chunk kernel over grid (nsplit, Hkv, B).  final_out: nsplit must be 1 and
// the kernel writes out/lse with the sink; otherwise it writes partials.
// group must be one of 1, 2, 4, 8, 16.
hipError_t launch_decode_chunks(const DecodeParams &p, bool sliding, int group, bool final_out,
                               hipStream_t stream);

hipError_t launch_lse_merge(const MergeParams &p, hipStream_t stream);

}  // namespace hda
