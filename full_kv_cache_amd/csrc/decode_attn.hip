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

// Orders this wave's LDS writes before its later LDS reads (LDS executes a
// wave's instructions in order; this stops the compiler from moving them).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

template <int G, bool SLIDING, bool FINAL>
__global__ __launch_bounds__(kDecodeThreads) void decode_chunk_kernel(DecodeParams p) {
    constexpr int D = kHeadDim;
    constexpr int WAVES = kDecodeThreads / 64;
    constexpr int RK = 32;                       // keys per round per wave
    constexpr int HG = (G + 3) / 4;              // 16-lane groups holding real heads
    constexpr int RED_FLOATS = WAVES * G * D;    // per-wave partial outputs
    __shared__ __align__(16) float s_red[RED_FLOATS];
    __shared__ __align__(16) float s_p[WAVES][RK * G];  // this round's probabilities
    __shared__ float s_m[WAVES][G], s_l[WAVES][G];

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

    // Wave w owns chunk keys [kw0, kw0 + R*RK), processed in rounds of RK.
    const int R = (p.chunk + WAVES * RK - 1) / (WAVES * RK);
    const int kw0 = wave * R * RK;
    const int kw1 = min(kw0 + R * RK, n);
    const int rounds = kw1 > kw0 ? (kw1 - kw0 + RK - 1) / RK : 0;

    const uint16_t *kbase = p.k + bh * p.capacity * D;
    const uint16_t *vbase = p.v + bh * p.capacity * D;
    const uint16_t *kside = SLIDING ? p.kev + bh * D : nullptr;
    const uint16_t *vside = SLIDING ? p.vev + bh * D : nullptr;

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

    const int hw = lane >> 5, dl = lane & 31;  // V: half-wave = one row, lane = 8 dims
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    // Running max (log2 domain) and this lane's share of the running sum,
    // for heads 4*kg + i; uniform within each 16-lane group.
    float m_run[4], l_lane[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m_run[i] = -INFINITY;
        l_lane[i] = 0.f;
    }
    float *pw = s_p[wave];

    for (int r = 0; r < rounds; ++r) {
        const int kr = kw0 + r * RK;
        // Every load is unconditional (tail keys read the last valid row
        // and are masked below), so the compiler can count them exactly
        // and V stays in flight while the scores are computed.
        uint4 kt[2][8], vt[16];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int key = min(kr + t * 16 + mrow, n - 1);
            const uint16_t *rp = row_ptr<SLIDING>(kbase, kside, c0 + key, span.n_ring) + 8 * kg;
#pragma unroll
            for (int j = 0; j < 8; ++j) kt[t][j] = ld16_stream(rp + 32 * j);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int key = min(kr + 2 * u + hw, n - 1);
            vt[u] = ld16_stream(row_ptr<SLIDING>(vbase, vside, c0 + key, span.n_ring) + 8 * dl);
        }

        // QK^T: lane holds heads 4*kg + i for key kr + 16t + mrow.
        f32x4 sc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 8; ++j)
                sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j], as_bf16x8(kt[t][j]), sc[t], 0, 0, 0);
        }
        float alpha[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float s0 = kr + mrow < n ? sc[0][i] * p.scale_log2 : -INFINITY;
            float s1 = kr + 16 + mrow < n ? sc[1][i] * p.scale_log2 : -INFINITY;
            float mx = fmaxf(s0, s1);
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
            const float mn = fmaxf(m_run[i], mx);  // finite: key kr is valid
            alpha[i] = exp2f(m_run[i] - mn);
            s0 = exp2f(s0 - mn);
            s1 = exp2f(s1 - mn);
            l_lane[i] = fmaf(l_lane[i], alpha[i], s0 + s1);
            m_run[i] = mn;
            sc[0][i] = s0;
            sc[1][i] = s1;
        }
        if (kg < HG) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * kg + i < G) pw[(t * 16 + mrow) * G + 4 * kg + i] = sc[t][i];
        }
        // Rescale the running output by each head's alpha (uniform per head).
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float af =
                __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[h & 3]), 16 * (h >> 2)));
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= af;
        }
        wave_lds_fence();

        // P.V: key kr + 2u + hw, 8 dims per lane.
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            float pv[G];
#pragma unroll
            for (int h = 0; h < G; ++h) pv[h] = pw[(2 * u + hw) * G + h];
            const uint32_t w[4] = {vt[u].x, vt[u].y, vt[u].z, vt[u].w};
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
        wave_lds_fence();
    }

    // ---- merge the waves: halves by shuffle, waves through LDS with
    // their own maxima rescaled to the common one.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) l_lane[i] += __shfl_xor(l_lane[i], o, 64);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], 32, 64);
    if (hw == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) s_red[(wave * G + h) * D + 8 * dl + e] = acc[h][e];
    }
    if (mrow == 0 && kg < HG) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * kg + i < G) {
                s_m[wave][4 * kg + i] = m_run[i];
                s_l[wave][4 * kg + i] = l_lane[i];
            }
    }
    __syncthreads();

    const int d = tid;  // blockDim == D
    for (int h = 0; h < G; ++h) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) M = fmaxf(M, s_m[w][h]);
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float sc = exp2f(s_m[w][h] - M);  // wave without keys: 2^-inf = 0
            L = fmaf(sc, s_l[w][h], L);
            o = fmaf(sc, s_red[(w * G + h) * D + d], o);
        }
        const float on = o / L;
        const float lse = (M + log2f(L)) * kLn2;
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
