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

hipError_t launch_rope_append(const RopeAppendParams &p, hipStream_t stream);

// Launches the chunk kernel (final output when nsplit == 1, partials and a
// merge otherwise).  group must be one of 1, 2, 4, 8, 16.
hipError_t launch_decode(const DecodeParams &p, bool sliding, int group, hipStream_t stream);

}  // namespace hda
