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
// Keys.  A (sequence, KV head) block holds `capacity` rows of K and of V;
// the step's keys are its leading n rows: n = seq_len for a full layer and
// min(seq_len, window) for a sliding one (ring slots plus the evicted-entry
// row), so both layer types stream contiguous rows.
//
// The building block is a 16-key round for one wave and one KV head:
//   * QK^T on the matrix cores, v_mfma_f32_16x16x32_bf16: the G query heads
//     are the 16-row A operand (rows >= G zero), the 16 keys the B
//     operand, fed straight from HBM with 16-byte loads (8 dims of a key row
//     per lane): no conversion and no LDS staging for K;
//   * an online softmax in the log2 domain: the round maximum over the 16
//     key lanes, rescale of the running sum and output;
//   * P.V on the vector ALUs: each half-wave streams whole 512-byte V rows
//     (lane = 8 dims), every row serving all G heads; the round's
//     probabilities reach those lanes through LDS.
// Every load is unconditional -- rows past the last key are replaced by
// in-bounds rows and masked -- so the compiler can count outstanding loads
// exactly and keep the next round in flight.
//
// Two decompositions:
//   * balanced streaming (default): all rounds of all pairs form one index
//     space split evenly over a grid of resident single-wave workgroups, two
//     rounds in flight per wave; one partial per (wave, pair) segment;
//   * chunks: every sequence cut into fixed chunks, one 4-wave workgroup
//     each (explicit chunk size; also the hda_decode_attn_partials layout).
// Partials merge as lse = ln sum_c exp(lse_c), out = sum_c exp(lse_c - lse)
// out_c, then the sink (Spark ring-branch comment: a softmax split over key
// subsets and merged online is the same result).
//
// The path is HBM-bound: every K and V byte is read once and serves G heads
// (4 flop per byte at G = 4), far below the VALU and MFMA ridge points.
#include "hda_device.h"
#include "hda_kernels.h"

namespace hda {

namespace {

constexpr float kLn2 = 0.693147180559945309f;

// Keys attended by sequence b (0 for seq_len <= 0).
__device__ __forceinline__ int num_keys(const DecodeParams &p, int b) {
    int n = p.seq_lens[b];
    n = n < p.max_keys ? n : p.max_keys;
    if (p.sliding) n = n < p.window ? n : p.window;
    return n > 0 ? n : 0;
}

// Orders this wave's LDS writes before its later LDS reads (LDS executes a
// wave's instructions in order; this stops the compiler from moving them).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ void bf16x8_to_f32(const uint4 &v, float *x) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(w[i]);
        x[2 * i + 1] = bf16_hi(w[i]);
    }
}

__device__ __forceinline__ float lane_value(float v, int src_lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src_lane));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// DPP lane moves inside each row of 16 lanes: swap neighbours, swap lane
// pairs, mirror each half-row, mirror the row.  Applied in that order they
// pair every lane with partners in the other quad, half-row and half, so
// max / sum over the row land in all its 16 lanes without touching LDS.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp<kQuadSwap1>(v));
    v = fmaxf(v, dpp<kQuadSwap2>(v));
    v = fmaxf(v, dpp<kHalfMirror>(v));
    return fmaxf(v, dpp<kRowMirror>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<kQuadSwap1>(v);
    v += dpp<kQuadSwap2>(v);
    v += dpp<kHalfMirror>(v);
    return v + dpp<kRowMirror>(v);
}

// 2^x on the transcendental unit; arguments here are <= 0 (and -inf), where
// a flushed denormal result is as good as exact for a softmax weight.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// MFMA A operand for KV head kvh of sequence b: lane (m = lane%16,
// kg = lane/16) holds q[head m][32j + 8kg .. +7] for k-step j; rows m >= G
// are zero.
template <int G>
__device__ __forceinline__ void load_q_operand(const DecodeParams &p, int b, int kvh, int lane,
                                               bf16x8 *qa) {
    const int mrow = lane & 15, kg = lane >> 4;
    const int hrow = mrow < G ? mrow : 0;
    const uint16_t *qr = p.q + ((int64_t)b * p.num_q_heads + kvh * G + hrow) * kHeadDim + 8 * kg;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint4 u = ld16(qr + 32 * j);
        if (mrow >= G) u = make_uint4(0, 0, 0, 0);
        qa[j] = as_bf16x8(u);
    }
}

// One wave's running softmax state over 16-key rounds.
//   acc[h][e]: unnormalised output, head h, dim 8*(lane%32) + e, summed
//              over this half-wave's keys (the two halves add up at the end);
//   m_run[i] / l_lane[i]: running max (log2 domain) and this lane's share of
//              the running sum, for head 4*(lane/16) + i.
template <int G>
struct WaveSoftmax {
    float acc[G][8];
    float m_run[4], l_lane[4];

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m_run[i] = -INFINITY;
            l_lane[i] = 0.f;
        }
    }

    // One 16-key round: kt = the 8 K operand loads (key = 16-lane index),
    // vt = the 8 V row loads (keys 2u + half), key x of the round valid iff
    // lo <= x < hi (at least one is).  pw: this wave's LDS scratch, 16*G floats.
    __device__ __forceinline__ void round(const bf16x8 *qa, const uint4 *kt, uint4 *vt, int lo,
                                          int hi, float scale_log2, float *pw, int lane) {
        const int mrow = lane & 15, kg = lane >> 4, hw = lane >> 5;
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j)
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j], as_bf16x8(kt[j]), sc, 0, 0, 0);
        // lane holds heads 4*kg + i of key mrow; a masked key's score is
        // replaced, never combined, so whatever its row holds cannot leak
        const bool valid = mrow >= lo && mrow < hi;
        float alpha[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float s = valid ? sc[i] * scale_log2 : -INFINITY;
            const float mn = fmaxf(m_run[i], row16_max(s));  // finite: the round holds a key
            alpha[i] = fast_exp2(m_run[i] - mn);
            s = fast_exp2(s - mn);
            l_lane[i] = fmaf(l_lane[i], alpha[i], s);
            m_run[i] = mn;
            sc[i] = s;
        }
        if (4 * kg < G) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * kg + i < G) pw[mrow * G + 4 * kg + i] = sc[i];
        }
        // Rescale the running output only when some head's maximum moved.
        float a_h[G];
        bool moved = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            a_h[h] = lane_value(alpha[h & 3], 16 * (h >> 2));
            moved |= a_h[h] != 1.f;
        }
        if (moved) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= a_h[h];
        }
        // Rows of masked keys may hold anything (even NaN, which a zero
        // weight would not cancel): a round that has some reads them as 0.
        if (lo > 0 || hi < 16) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int key = 2 * u + hw;
                if (key < lo || key >= hi) vt[u] = make_uint4(0, 0, 0, 0);
            }
        }
        wave_lds_fence();
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            float pv[G], x[8];
#pragma unroll
            for (int h = 0; h < G; ++h) pv[h] = pw[(2 * u + hw) * G + h];
            bf16x8_to_f32(vt[u], x);
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pv[h], x[e], acc[h][e]);
        }
        wave_lds_fence();
    }

    // Wave totals for head h (wave-uniform): running max and sum.
    __device__ __forceinline__ float max_of(int h) const { return lane_value(m_run[h & 3], 16 * (h >> 2)); }
    __device__ __forceinline__ void sums(float *l_h) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) l_h[i] = row16_sum(l_lane[i]);
    }
};

// Loads of one round: the 16 keys start at block row r0e (kept at most
// capacity - 16 so that every load stays inside the block); the caller
// masks keys outside [r0, n).  Passing lane 0 for every lane makes a
// placeholder round: the same number of load instructions, all of one
// 16-byte address, so the wait counts stay exact at no traffic.
__device__ __forceinline__ void issue_round(const uint16_t *kblk, const uint16_t *vblk, int r0e,
                                            int lane, uint4 *kt, uint4 *vt) {
    const int mrow = lane & 15, kg = lane >> 4, hw = lane >> 5, dl = lane & 31;
    const uint16_t *rk = kblk + (int64_t)(r0e + mrow) * kHeadDim + 8 * kg;
#pragma unroll
    for (int j = 0; j < 8; ++j) kt[j] = ld16_stream(rk + 32 * j);
    const uint16_t *rv = vblk + (int64_t)(r0e + hw) * kHeadDim + 8 * dl;
#pragma unroll
    for (int u = 0; u < 8; ++u) vt[u] = ld16_stream(rv + 2 * u * kHeadDim);
}

// Writes o / l for the G heads (first half-wave) and their lse.
template <int G>
__device__ __forceinline__ void store_partial(const WaveSoftmax<G> &st, float *po, float *plse,
                                              int lane) {
    const int hw = lane >> 5, dl = lane & 31;
    float l_h[4];
    st.sums(l_h);
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float l = lane_value(l_h[h & 3], 16 * (h >> 2));
        const float inv = 1.f / l;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (st.acc[h][e] + __shfl_xor(st.acc[h][e], 32, 64)) * inv;
        if (hw == 0) {
            float *dst = po + h * kHeadDim + 8 * dl;
            *reinterpret_cast<float4 *>(dst) = make_float4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<float4 *>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
        }
        if (lane == 0) plse[h] = (st.max_of(h) + log2f(l)) * kLn2;
    }
}

// ===================================================================
// Chunk decomposition: grid (nsplit, Hkv, B), 4 waves per workgroup; wave
// w takes the rounds of keys [w*R*16, (w+1)*R*16) of chunk c; the waves
// merge in LDS; the result is the final output (nsplit == 1) or a partial.
// ===================================================================
template <int G, bool FINAL>
__global__ __launch_bounds__(kDecodeThreads) void decode_chunk_kernel(DecodeParams p) {
    constexpr int D = kHeadDim;
    constexpr int WAVES = kDecodeThreads / 64;
    __shared__ __align__(16) float s_red[WAVES * G * D];
    __shared__ __align__(16) float s_pw[WAVES][16 * G];
    __shared__ float s_m[WAVES][G], s_l[WAVES][G];

    const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Hq = p.num_q_heads;
    const int n_all = num_keys(p, b);
    const int c0 = c * p.chunk;
    const int n = min(p.chunk, n_all - c0);  // keys of this chunk
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

    const int R = (p.chunk + WAVES * 16 - 1) / (WAVES * 16);  // rounds per wave
    const int kw0 = wave * R * 16;
    const int kw1 = min(kw0 + R * 16, n);
    const int64_t cap = p.capacity, cap16 = cap - 16;
    const uint16_t *kblk = p.k + bh * cap * D, *vblk = p.v + bh * cap * D;

    bf16x8 qa[8];
    load_q_operand<G>(p, b, kvh, lane, qa);
    WaveSoftmax<G> st;
    st.reset();
    for (int kr = kw0; kr < kw1; kr += 16) {
        const int r0 = c0 + kr;  // block row of the round's first key
        const int r0e = (int)(r0 < cap16 ? r0 : cap16);
        uint4 kt[8], vt[8];
        issue_round(kblk, vblk, r0e, lane, kt, vt);
        st.round(qa, kt, vt, r0 - r0e, c0 + kw1 - r0e, p.scale_log2, s_pw[wave], lane);
    }

    // merge the waves: each leaves its unnormalised o and its (m, l)
    float l_h[4];
    st.sums(l_h);
    const int hw = lane >> 5, dl = lane & 31;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float o = st.acc[h][e] + __shfl_xor(st.acc[h][e], 32, 64);
            if (hw == 0) s_red[(wave * G + h) * D + 8 * dl + e] = o;
        }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            s_m[wave][h] = kw1 > kw0 ? st.max_of(h) : -INFINITY;
            s_l[wave][h] = kw1 > kw0 ? lane_value(l_h[h & 3], 16 * (h >> 2)) : 0.f;
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

// ===================================================================
// Balanced streaming decomposition (the default path).
//
// Pair p = (b, kvh) holds R_b = ceil(n_b / 16) rounds of 16 keys; all
// rounds, pair after pair, form one index space of R_tot rounds.  Wave w of
// the W-wave grid (every wave resident at once) takes rounds
// [w*R_tot/W, (w+1)*R_tot/W): each wave streams the same number of keys
// (+-16) whatever the length mix.  A wave's range is cut at pair boundaries
// into segments; each leaves one partial in slot w + p -- unique, because
// the (wave, pair) overlaps are ordered the same way along both indices.
// Rounds are pipelined two deep: the next round's 16 loads are in flight
// while the current one is scored, softmaxed and accumulated.  (Claiming
// small tickets of work from atomic counters instead measured slower on
// MI355X: device-wide atomics serialise, and a partial per ticket adds
// traffic.)
// ===================================================================
struct RoundAddr {
    int b, kvh, rr;  // sequence, KV head, round within the pair
};

struct RoundGeo {
    const uint16_t *kblk, *vblk;
    int r0e, lo, hi;  // in-bounds first row; valid keys [lo, hi) of the round
};

template <int G>
__global__ __launch_bounds__(64) void decode_stream_kernel(DecodeParams p) {
    constexpr int D = kHeadDim;
    __shared__ int s_pre[kStreamMaxBatch + 1];     // rounds before sequence b, one KV head
    __shared__ __align__(16) float s_pw[16 * G];   // this round's probabilities [key][head]

    const int lane = threadIdx.x;
    const int w = blockIdx.x, W = gridDim.x;
    const int B = p.batch, Hkv = p.num_kv_heads;

    // prefix sum of rounds per sequence: wave scan, 64 sequences a pass
    {
        int carry = 0;
        for (int base = 0; base < B; base += 64) {
            const int b = base + lane;
            int x = b < B ? (num_keys(p, b) + 15) >> 4 : 0;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(x, o, 64);
                if (lane >= o) x += y;
            }
            if (b < B) s_pre[b + 1] = carry + x;
            carry += __shfl(x, 63, 64);
        }
        if (lane == 0) s_pre[0] = 0;
    }
    __syncthreads();
    if (w == 0)  // published for the merge kernel
        for (int b = lane; b <= B; b += 64) p.stream_pre[b] = s_pre[b];
    const int64_t r_tot = (int64_t)Hkv * s_pre[B];
    const int64_t g0 = (int64_t)w * r_tot / W, g1 = (int64_t)(w + 1) * r_tot / W;
    if (g0 >= g1) return;

    // locate round g0: the sequence by binary search, then KV head and round
    RoundAddr cur;
    {
        int lo = 0, hi = B;  // largest b with Hkv * pre[b] <= g0
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if ((int64_t)Hkv * s_pre[mid] <= g0) lo = mid; else hi = mid;
        }
        int b = lo;
        while ((int64_t)Hkv * s_pre[b + 1] <= g0) ++b;  // sequences without rounds
        const int rb = s_pre[b + 1] - s_pre[b];
        const int off = (int)(g0 - (int64_t)Hkv * s_pre[b]);
        cur.b = uniform(b);
        cur.kvh = uniform(off / rb);
        cur.rr = uniform(off % rb);
    }
    auto rounds_of = [&](int b) { return uniform(s_pre[b + 1] - s_pre[b]); };
    auto advance = [&](RoundAddr a) {
        if (++a.rr == rounds_of(a.b)) {
            a.rr = 0;
            if (++a.kvh == Hkv) {
                a.kvh = 0;
                do { ++a.b; } while (a.b < B && rounds_of(a.b) == 0);
            }
        }
        return a;
    };

    const int64_t cap = p.capacity, cap16 = cap - 16;
    auto geo = [&](const RoundAddr &a) {
        RoundGeo g;
        const int64_t bh = (int64_t)a.b * Hkv + a.kvh;
        g.kblk = p.k + bh * cap * D;
        g.vblk = p.v + bh * cap * D;
        const int r0 = a.rr * 16;
        g.r0e = (int)(r0 < cap16 ? r0 : cap16);
        g.lo = r0 - g.r0e;
        g.hi = uniform(num_keys(p, a.b)) - g.r0e;
        return g;
    };
    auto same_pair = [](const RoundAddr &x, const RoundAddr &y) { return x.b == y.b && x.kvh == y.kvh; };

    bf16x8 qa[8];
    WaveSoftmax<G> st;
    uint4 kA[8], vA[8], kB[8], vB[8];
    RoundGeo gc = geo(cur);
    issue_round(gc.kblk, gc.vblk, gc.r0e, lane, kA, vA);
    load_q_operand<G>(p, cur.b, cur.kvh, lane, qa);
    st.reset();

    auto end_segment = [&](const RoundAddr &a) {
        const int64_t slot = (int64_t)w + a.b * Hkv + a.kvh;
        store_partial<G>(st, p.part_o + slot * G * D, p.part_lse + slot * G, lane);
    };

    // Every half-iteration issues the next round's loads, then computes the
    // current round.  After the last round a placeholder round is issued
    // (never used) so that the loads stay unconditional and the compiler's
    // wait counts exact.
    int64_t g = g0;
    while (true) {
        bool more = g + 1 < g1;
        RoundAddr nxt = more ? advance(cur) : cur;
        RoundGeo gn = geo(nxt);
        issue_round(gn.kblk, gn.vblk, gn.r0e, more ? lane : 0, kB, vB);
        st.round(qa, kA, vA, gc.lo, gc.hi, p.scale_log2, s_pw, lane);
        if (!more || !same_pair(nxt, cur)) {
            end_segment(cur);
            if (!more) break;
            load_q_operand<G>(p, nxt.b, nxt.kvh, lane, qa);
            st.reset();
        }
        cur = nxt;
        gc = gn;
        ++g;

        more = g + 1 < g1;
        nxt = more ? advance(cur) : cur;
        gn = geo(nxt);
        issue_round(gn.kblk, gn.vblk, gn.r0e, more ? lane : 0, kA, vA);
        st.round(qa, kB, vB, gc.lo, gc.hi, p.scale_log2, s_pw, lane);
        if (!more || !same_pair(nxt, cur)) {
            end_segment(cur);
            if (!more) break;
            load_q_operand<G>(p, nxt.b, nxt.kvh, lane, qa);
            st.reset();
        }
        cur = nxt;
        gc = gn;
        ++g;
    }
}

// Merge of the streaming partials: one workgroup per (query head,
// sequence).  The pair's rounds [g_lo, g_hi] were covered by waves
// wave_of(g_lo) .. wave_of(g_hi), wave_of(g) = the largest w with
// w*R_tot/W <= g, whose partials sit in slots w + pair.
__global__ __launch_bounds__(kDecodeThreads) void stream_merge_kernel(DecodeParams p, int W) {
    constexpr int D = kHeadDim;
    const int hq = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int Hq = p.num_q_heads, Hkv = p.num_kv_heads, G = Hq / Hkv;
    const int kvh = hq / G, h = hq % G;
    const int rb = p.stream_pre[b + 1] - p.stream_pre[b];
    uint16_t *outp = p.out + ((int64_t)b * Hq + hq) * D + d;
    if (rb == 0) {
        *outp = 0;
        if (d == 0 && p.lse) p.lse[(int64_t)b * Hq + hq] = -INFINITY;
        return;
    }
    const int64_t r_tot = (int64_t)Hkv * p.stream_pre[p.batch];
    const int64_t g_lo = (int64_t)Hkv * p.stream_pre[b] + (int64_t)kvh * rb;
    const int64_t g_hi = g_lo + rb - 1;
    const int w_lo = (int)(((g_lo + 1) * W - 1) / r_tot);
    const int w_hi = (int)(((g_hi + 1) * W - 1) / r_tot);
    const int64_t pair = (int64_t)b * Hkv + kvh;
    float M = -INFINITY;
    for (int w = w_lo; w <= w_hi; ++w) M = fmaxf(M, p.part_lse[(w + pair) * G + h]);
    float L = 0.f, o = 0.f;
    for (int w = w_lo; w <= w_hi; ++w) {
        const int64_t slot = w + pair;
        const float e = expf(p.part_lse[slot * G + h] - M);
        L += e;
        o = fmaf(e, p.part_o[(slot * G + h) * D + d], o);
    }
    const float lse = M + logf(L);
    float f = 1.f;
    if (p.sinks) f = 1.f / (1.f + expf(p.sinks[hq] - lse));
    *outp = f32_to_bf16((o / L) * f);
    if (d == 0 && p.lse) p.lse[(int64_t)b * Hq + hq] = lse;
}

template <int G, bool FINAL>
hipError_t launch_chunks_g(const DecodeParams &p, hipStream_t s) {
    const dim3 grid(p.nsplit, p.num_kv_heads, p.batch);
    hipLaunchKernelGGL((decode_chunk_kernel<G, FINAL>), grid, dim3(kDecodeThreads), 0, s, p);
    return hipGetLastError();
}

template <bool FINAL>
hipError_t launch_chunks(const DecodeParams &p, int group, hipStream_t s) {
    switch (group) {
        case 1: return launch_chunks_g<1, FINAL>(p, s);
        case 2: return launch_chunks_g<2, FINAL>(p, s);
        case 4: return launch_chunks_g<4, FINAL>(p, s);
        case 8: return launch_chunks_g<8, FINAL>(p, s);
        case 16: return launch_chunks_g<16, FINAL>(p, s);
        default: return hipErrorInvalidValue;
    }
}

template <int G>
hipError_t launch_stream_g(const DecodeParams &p, int waves, hipStream_t s) {
    hipLaunchKernelGGL((decode_stream_kernel<G>), dim3(waves), dim3(64), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(stream_merge_kernel, dim3(p.num_q_heads, p.batch), dim3(kDecodeThreads), 0, s,
                       p, waves);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_chunks(const DecodeParams &p, int group, bool final_out, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    return final_out ? launch_chunks<true>(p, group, stream) : launch_chunks<false>(p, group, stream);
}

// Resident single-wave workgroups of the streaming kernel on this device:
// its occupancy per CU times the CU count (0 when no device answers).
template <int G>
int stream_slots_g() {
    static int cached = -1;
    if (cached < 0) {
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_stream_kernel<G>, 64, 0) !=
                hipSuccess) {
            (void)hipGetLastError();
            return 0;
        }
        cached = cus * per_cu;
    }
    return cached;
}

int stream_wave_slots(int group) {
    switch (group) {
        case 1: return stream_slots_g<1>();
        case 2: return stream_slots_g<2>();
        case 4: return stream_slots_g<4>();
        case 8: return stream_slots_g<8>();
        case 16: return stream_slots_g<16>();
        default: return 0;
    }
}

hipError_t launch_decode_stream(const DecodeParams &p, int group, int waves, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    switch (group) {
        case 1: return launch_stream_g<1>(p, waves, stream);
        case 2: return launch_stream_g<2>(p, waves, stream);
        case 4: return launch_stream_g<4>(p, waves, stream);
        case 8: return launch_stream_g<8>(p, waves, stream);
        case 16: return launch_stream_g<16>(p, waves, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_lse_merge(const MergeParams &p, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    hipLaunchKernelGGL(lse_merge_kernel, dim3(p.num_heads, p.batch), dim3(kDecodeThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace hda
