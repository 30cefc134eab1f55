// decode_attn.hip -- GQA decode attention over the explicit KV cache (gfx950).
//
// What is computed (Spark export page, `_Layer.forward`; flashmla_sparse
// page, `HYV4FlashMLASparseImpl` docstring for the sink):
//   for sequence b, query head h (KV head h / G), over the layer's keys
//   scores = scale * q.k; p = softmax(scores); out = sum p v;
//   lse = ln sum exp(scores); out *= exp(lse) / (exp(lse) + exp(sink_h)).
// The sink factor is evaluated as 1 / (1 + exp(sink - lse)), so a -inf
// sink multiplies by exactly 1.
//
// Work decomposition.  One workgroup (4 wave64s) takes one chunk of up to
// 512 keys of one (sequence, KV head) and serves all G query heads of the
// group from a single pass over the chunk's K and V rows:
//   1. QK^T on the matrix cores: v_mfma_f32_16x16x32_bf16 with the G query
//      heads as the 16-row A operand (rows >= G zero) and 16 keys as the
//      B operand.  Each lane feeds the B operand straight from HBM with
//      16-byte loads (8 dims of one key row), so K needs no conversion and
//      no LDS staging.  Scores (log2 domain) go to LDS.
//   2. Softmax statistics of the chunk, one wave per head: max and sum of
//      2^(s - max) with wave64 butterfly reductions; probabilities to LDS.
//   3. P.V on the vector ALUs: each half-wave streams whole V rows with
//      16-byte loads (lane = 8 dims), every row serving all G heads.
//   4. Halves, then waves, are summed through LDS; the chunk result is
//      either the final output (one chunk covers the keys) or a partial
//      (out_c normalised, lse_c) for the merge.
// Split-K merge (Spark ring-branch comment: a softmax split over key
// subsets and merged online is the same result): lse = ln sum_c
// exp(lse_c), out = sum_c exp(lse_c - lse) out_c, then the sink.
//
// The path is HBM-bound: every K and V byte is read once and serves G
// heads (4 flop per byte at G = 4), far below both the VALU and the MFMA
// ridge points.
#include "hda_device.h"
#include "hda_kernels.h"

namespace hda {

namespace {

constexpr float kLn2 = 0.693147180559945309f;

// Keys attended by one sequence.  Full: rows 0..n-1.  Sliding: ring slots
// 0..n_ring-1, then (index n_ring) the side row when a full window is
// present.
struct KeySpan {
    int n_keys;
    int n_ring;
};

template <bool SLIDING>
__device__ __forceinline__ KeySpan key_span(const DecodeParams &p, int b) {
    int seq = p.seq_lens[b];
    seq = seq < p.max_keys ? seq : p.max_keys;
    seq = seq > 0 ? seq : 0;
    KeySpan s;
    if (SLIDING) {
        s.n_ring = seq < p.window - 1 ? seq : p.window - 1;
        s.n_keys = seq < p.window ? seq : p.window;
    } else {
        s.n_ring = seq;
        s.n_keys = seq;
    }
    return s;
}

template <bool SLIDING>
__device__ __forceinline__ const uint16_t *row_ptr(const uint16_t *base, const uint16_t *side,
                                                   int idx, int n_ring) {
    if (SLIDING && idx >= n_ring) return side;
    return base + (int64_t)idx * kHeadDim;
}

template <int G, bool SLIDING, bool FINAL>
__global__ __launch_bounds__(kDecodeThreads) void decode_chunk_kernel(DecodeParams p) {
    constexpr int D = kHeadDim;
    constexpr int CH = kMaxChunk;
    constexpr int SC_FLOATS = 2 * G * CH;   // scores + probabilities
    constexpr int RED_FLOATS = 4 * G * D;   // per-wave partial outputs
    constexpr int SMEM_FLOATS = SC_FLOATS > RED_FLOATS ? SC_FLOATS : RED_FLOATS;
    __shared__ __align__(16) float smem[SMEM_FLOATS];
    __shared__ float s_m[G], s_l[G];
    float *s_sc = smem;            // [G][CH]  scores, log2 domain
    float *s_p = smem + G * CH;    // [CH][G]  probabilities, key-major

    const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Hq = p.num_q_heads;
    const KeySpan span = key_span<SLIDING>(p, b);
    const int c0 = c * p.chunk;
    const int n = min(p.chunk, span.n_keys - c0);
    const int64_t bh = (int64_t)b * p.num_kv_heads + kvh;

    if (n <= 0) {
        if (FINAL) {  // no keys at all: out 0, lse -inf
            for (int h = 0; h < G; ++h) {
                const int hq = kvh * G + h;
                p.out[((int64_t)b * Hq + hq) * D + tid] = 0;
                if (tid == 0 && p.lse) p.lse[(int64_t)b * Hq + hq] = -INFINITY;
            }
        } else if (tid < G) {  // partial: a chunk without keys weighs zero in the merge
            p.part_lse[((int64_t)b * Hq + kvh * G + tid) * p.nsplit + c] = -INFINITY;
        }
        return;
    }

    // ---- Q as the MFMA A operand: lane (m = lane%16, kg = lane/16) holds
    // q[head m][32j + 8kg .. +7] for k-step j; rows m >= G are zero.
    const int mrow = lane & 15, kg = lane >> 4;
    bf16x8 qa[8];
    {
        const int hrow = mrow < G ? mrow : 0;
        const uint16_t *qr = p.q + ((int64_t)b * Hq + kvh * G + hrow) * D + 8 * kg;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint4 u = ld16(qr + 32 * j);
            if (mrow >= G) u = make_uint4(0, 0, 0, 0);
            qa[j] = as_bf16x8(u);
        }
    }

    const uint16_t *kbase = p.k + bh * p.capacity * D;
    const uint16_t *vbase = p.v + bh * p.capacity * D;
    const uint16_t *kside = SLIDING ? p.kev + bh * D : nullptr;
    const uint16_t *vside = SLIDING ? p.vev + bh * D : nullptr;

    // ---- 1. scores of 16-key tiles; wave w takes tiles w, w+4, ...; two
    // tiles per iteration keep 16 loads per lane in flight.
    const int ntiles = (n + 15) >> 4;
    for (int t = wave; t < ntiles; t += 8) {
        uint4 ka[8], kb[8];
        const int keyA = t * 16 + mrow, keyB = keyA + 64;
        const bool vA = keyA < n, vB = keyB < n;
        const uint16_t *rA = row_ptr<SLIDING>(kbase, kside, c0 + (vA ? keyA : 0), span.n_ring) + 8 * kg;
        const uint16_t *rB = row_ptr<SLIDING>(kbase, kside, c0 + (vB ? keyB : 0), span.n_ring) + 8 * kg;
#pragma unroll
        for (int j = 0; j < 8; ++j) ka[j] = vA ? ld16_stream(rA + 32 * j) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 8; ++j) kb[j] = vB ? ld16_stream(rB + 32 * j) : make_uint4(0, 0, 0, 0);
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j)
            accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j], as_bf16x8(ka[j]), accA, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            accB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j], as_bf16x8(kb[j]), accB, 0, 0, 0);
        // lane holds heads 4*kg + i (i = 0..3) for key (tile*16 + mrow)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = 4 * kg + i;
            if (h < G) {
                s_sc[h * CH + keyA] = vA ? accA[i] * p.scale_log2 : -INFINITY;
                if (t + 4 < ntiles) s_sc[h * CH + keyB] = vB ? accB[i] * p.scale_log2 : -INFINITY;
            }
        }
    }
    __syncthreads();

    // ---- 2. chunk softmax statistics, one wave per head.
    for (int h = wave; h < G; h += 4) {
        float mx = -INFINITY;
        for (int k = lane; k < n; k += 64) mx = fmaxf(mx, s_sc[h * CH + k]);
        mx = wave_max(mx);
        float sum = 0.f;
        for (int k = lane; k < n; k += 64) {
            const float e = exp2f(s_sc[h * CH + k] - mx);
            s_p[k * G + h] = e;
            sum += e;
        }
        sum = wave_sum(sum);
        if (lane == 0) {
            s_m[h] = mx;
            s_l[h] = sum;
        }
    }
    __syncthreads();

    // ---- 3. P.V: 8 streams (4 waves x 2 half-waves) over the keys; a
    // half-wave reads one whole 512-byte V row per load, lane = 8 dims.
    const int hw = lane >> 5, dl = lane & 31;
    const int stream = wave * 2 + hw;
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

    constexpr int U = 8;
    for (int k0 = stream; k0 < n; k0 += 8 * U) {
        uint4 vv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + 8 * u;
            vv[u] = make_uint4(0, 0, 0, 0);
            if (k < n) vv[u] = ld16_stream(row_ptr<SLIDING>(vbase, vside, c0 + k, span.n_ring) + 8 * dl);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + 8 * u;
            if (k < n) {
                float pv[G];
#pragma unroll
                for (int h = 0; h < G; ++h) pv[h] = s_p[k * G + h];
                const uint32_t w[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
                float x[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[2 * i] = bf16_lo(w[i]);
                    x[2 * i + 1] = bf16_hi(w[i]);
                }
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pv[h], x[e], acc[h][e]);
            }
        }
    }

    // ---- 4. reduce the 8 streams: halves by shuffle, waves through LDS.
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], 32, 64);
    __syncthreads();  // s_p is dead from here: reuse smem
    float *red = smem;  // [4][G][D]
    if (hw == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[(wave * G + h) * D + 8 * dl + e] = acc[h][e];
    }
    __syncthreads();

    const int d = tid;  // blockDim == D
    for (int h = 0; h < G; ++h) {
        const float o = (red[(0 * G + h) * D + d] + red[(1 * G + h) * D + d]) +
                        (red[(2 * G + h) * D + d] + red[(3 * G + h) * D + d]);
        const float l = s_l[h];
        const float on = o / l;
        const float lse = (s_m[h] + log2f(l)) * kLn2;
        const int hq = kvh * G + h;
        if (FINAL) {
            float f = 1.f;
            if (p.sinks) f = 1.f / (1.f + expf(p.sinks[hq] - lse));
            p.out[((int64_t)b * Hq + hq) * D + d] = f32_to_bf16(on * f);
            if (d == 0 && p.lse) p.lse[(int64_t)b * Hq + hq] = lse;
        } else {
            const int64_t slot = ((int64_t)b * Hq + hq) * p.nsplit + c;
            p.part_o[slot * D + d] = on;
            if (d == 0) p.part_lse[slot] = lse;
        }
    }
}

// One workgroup per (query head, sequence); thread = output dim.  Chunks
// with lse = -inf hold no keys and are skipped (their out is never read).
__global__ __launch_bounds__(kDecodeThreads) void lse_merge_kernel(MergeParams p) {
    constexpr int D = kHeadDim;
    const int hq = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int64_t row = (int64_t)b * p.num_heads + hq;
    const float *pl = p.part_lse + row * p.nsplit;
    const float *po = p.part_o + row * p.nsplit * D + d;
    float M = -INFINITY;
    for (int c = 0; c < p.nsplit; ++c) M = fmaxf(M, pl[c]);
    uint16_t *outp = p.out + row * D + d;
    if (M == -INFINITY) {
        *outp = 0;
        if (d == 0 && p.lse) p.lse[row] = -INFINITY;
        return;
    }
    float L = 0.f, o = 0.f;
    for (int c = 0; c < p.nsplit; ++c) {
        const float lc = pl[c];
        if (lc == -INFINITY) continue;
        const float w = expf(lc - M);
        L += w;
        o = fmaf(w, po[(int64_t)c * D], o);
    }
    const float lse = M + logf(L);
    float f = 1.f;
    if (p.sinks) f = 1.f / (1.f + expf(p.sinks[hq] - lse));
    *outp = f32_to_bf16((o / L) * f);
    if (d == 0 && p.lse) p.lse[row] = lse;
}

template <int G, bool SLIDING, bool FINAL>
hipError_t launch_g(const DecodeParams &p, hipStream_t s) {
    const dim3 grid(p.nsplit, p.num_kv_heads, p.batch);
    hipLaunchKernelGGL((decode_chunk_kernel<G, SLIDING, FINAL>), grid, dim3(kDecodeThreads), 0, s, p);
    return hipGetLastError();
}

template <bool SLIDING, bool FINAL>
hipError_t launch_s(const DecodeParams &p, int group, hipStream_t s) {
    switch (group) {
        case 1: return launch_g<1, SLIDING, FINAL>(p, s);
        case 2: return launch_g<2, SLIDING, FINAL>(p, s);
        case 4: return launch_g<4, SLIDING, FINAL>(p, s);
        case 8: return launch_g<8, SLIDING, FINAL>(p, s);
        case 16: return launch_g<16, SLIDING, FINAL>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_chunks(const DecodeParams &p, bool sliding, int group, bool final_out,
                               hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    if (final_out)
        return sliding ? launch_s<true, true>(p, group, stream) : launch_s<false, true>(p, group, stream);
    return sliding ? launch_s<true, false>(p, group, stream) : launch_s<false, false>(p, group, stream);
}

hipError_t launch_lse_merge(const MergeParams &p, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    hipLaunchKernelGGL(lse_merge_kernel, dim3(p.num_heads, p.batch), dim3(kDecodeThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace hda
