// decode_multi.hip -- decode of a chunk of T new tokens per sequence
// (gfx950): RoPE, attention, append.
//
// Spark export page, `SparkStepConfig.cache_len` docstring: a ring holds
// the window's previous entries and the new token is scored together with
// them.  For a chunk, token t (position pos + t) attends to the entries of
// its own window -- cached ones and new tokens 0..t -- which is what T
// single-token steps in order would compute.  Three launches:
//   1. rope_multi_kernel: q and the new K rotated in place at pos + t
//      (the single-token kernel's arithmetic, so the same bf16 values);
//   2. decode_multi_kernel: attention over the cache as it was before the
//      chunk plus the chunk's own rows.  `split` workgroups per (sequence,
//      KV head) share its cache rounds; the chunk's T x G query rows (row
//      t*G + h) fill the MFMA A operand, so every K/V row loaded serves all
//      T tokens.  Cache keys are masked per row: on a sliding layer token t
//      drops the t oldest entries (ring slots pos .. pos+t-1 mod window-1,
//      which tokens 0..t-1 replace); the new tokens are one more round, key
//      x visible to rows of token t >= x, taken by the last wave of the
//      last workgroup.  Each workgroup merges its waves in LDS and writes
//      out directly (split 1) or a partial (o, lse) per row that
//      multi_merge_kernel combines;
//   3. append_multi_kernel: the rotated new K and V rows into the cache
//      (full: rows pos + t; sliding: ring slots, and the block's
//      evicted-entry row receives what the last token's slot held, as a
//      single-token append leaves it).  It runs after the attention, which
//      reads the slots it overwrites.
#include <type_traits>

#include "decode_wave.h"

namespace hda {

using namespace wave;

namespace {

constexpr int kMultiRopeThreads = 256;

__device__ __forceinline__ uint4 ldm(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void stm(uint16_t *p, const uint4 &v) { *reinterpret_cast<uint4 *>(p) = v; }

// Block (b, token t): q [Hq] and new K [Hkv] rows rotated in place.
__global__ __launch_bounds__(kMultiRopeThreads) void rope_multi_kernel(MultiParams p) {
    __shared__ float s_cos[kHeadDim / 2], s_sin[kHeadDim / 2];
    constexpr int D = kHeadDim;
    const int bt = blockIdx.x, b = bt / p.tokens, t = bt % p.tokens;
    const int32_t p0 = p.pos[b];
    if (p0 < 0) return;  // no new tokens for this sequence
    const int rot = p.rotary_dim, half = rot / 2;
    for (int j = threadIdx.x; j < half; j += kMultiRopeThreads) {
        const float ang = (float)(p0 + t) * p.inv_freq[j];  // one fp32 multiply
        sincos_angle(ang, s_cos + j, s_sin + j);
    }
    __syncthreads();
    const int hc = half / 8;
    const int n_q = p.num_q_heads * hc, n_tasks = n_q + p.num_kv_heads * hc;
    for (int u = threadIdx.x; u < n_tasks; u += kMultiRopeThreads) {
        uint16_t *row;
        int j;
        if (u < n_q) {
            row = p.q + ((int64_t)bt * p.num_q_heads + u / hc) * D;
            j = (u % hc) * 8;
        } else {
            row = p.k_new + ((int64_t)bt * p.num_kv_heads + (u - n_q) / hc) * D;
            j = ((u - n_q) % hc) * 8;
        }
        uint4 ya, yb;
        rotate8(ldm(row + j), ldm(row + half + j), s_cos + j, s_sin + j, ya, yb);
        stm(row + j, ya);
        stm(row + half + j, yb);
    }
}

// Block (b, token t): the token's rotated K and its V into the cache.
__global__ __launch_bounds__(128) void append_multi_kernel(MultiParams p) {
    constexpr int D = kHeadDim;
    const int bt = blockIdx.x, b = bt / p.tokens, t = bt % p.tokens;
    const int32_t p0 = p.pos[b];
    if (p0 < 0) return;
    const int64_t P = (int64_t)p0 + t, cap = p.capacity;
    int64_t row;
    bool evict = false;
    if (p.sliding) {
        const int slots = p.window - 1;
        row = P % slots;
        evict = t == p.tokens - 1 && P >= slots;  // the last token's old entry
    } else {
        if (P >= cap) return;
        row = P;
    }
    const int Hkv = p.num_kv_heads;
    for (int u = threadIdx.x; u < 2 * Hkv * (D / 8); u += 128) {
        const bool is_v = u >= Hkv * (D / 8);
        const int w = is_v ? u - Hkv * (D / 8) : u, h = w / (D / 8), d = (w % (D / 8)) * 8;
        uint16_t *blk = (is_v ? p.v : p.k) + ((int64_t)b * Hkv + h) * cap * D;
        const uint16_t *src = (is_v ? p.v_new : p.k_new) + ((int64_t)bt * Hkv + h) * D;
        if (evict) stm(blk + (int64_t)(p.window - 1) * D + d, ldm(blk + row * D + d));
        stm(blk + row * D + d, ldm(src + d));
    }
}

template <int G, int T>
struct MultiShape {
    static constexpr int RG = G * T;                // query rows per (sequence, KV head)
    static constexpr int WAVES = RG >= 8 ? 4 : 8;   // merge area WAVES x RG rows; registers
};

template <int G, int T>
__global__ __launch_bounds__((G * T >= 8 ? 4 : 8) * 64) void decode_multi_kernel(MultiParams p) {
    constexpr int D = kHeadDim;
    constexpr int RG = MultiShape<G, T>::RG;
    constexpr int WAVES = MultiShape<G, T>::WAVES;
    __shared__ __align__(16) float s_red[WAVES * RG * D];
    __shared__ __align__(16) float s_pw[WAVES][16 * RG];
    __shared__ __align__(16) uint16_t s_kt[WAVES][kKTile];
    __shared__ float s_m[WAVES][RG], s_l[WAVES][RG];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int mrow = lane & 15, kg = lane >> 4;
    const int Hkv = p.num_kv_heads, Hq = p.num_q_heads;
    const int S = p.split, pair = blockIdx.x / S, part = blockIdx.x % S;
    const int b = pair / Hkv, kvh = pair % Hkv;
    const int32_t p0 = p.pos[b];
    const int64_t cap = p.capacity, cap16 = cap - 16;
    const int W1 = p.window - 1;
    int n_old = 0;  // cached keys before the chunk: rows / ring slots [0, n_old)
    if (p0 > 0) n_old = p.sliding ? min(p0, W1) : (int)min((int64_t)p0, cap);
    const int Rall = (n_old + 15) >> 4;
    const int R0 = part * Rall / S, R = (part + 1) * Rall / S - R0;  // this workgroup's rounds
    const int r_lo = R0 + wave * R / WAVES, r_hi = R0 + (wave + 1) * R / WAVES;
    const bool last = part == S - 1 && wave == WAVES - 1;  // also takes the chunk's own round
    const int64_t bh = (int64_t)b * Hkv + kvh;
    const uint16_t *kblk = p.k + bh * cap * D, *vblk = p.v + bh * cap * D;
    auto r0e_of = [&](int r) { return (int)((int64_t)(16 * r) < cap16 ? 16 * r : cap16); };

    // token of each of this lane's four score rows (4*kg + i); rows past RG
    // repeat row 0 and are never read
    int trow[4], ntrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * kg + i;
        trow[i] = m < RG ? m / G : 0;
        ntrow[i] = -trow[i];
    }

    WaveSoftmax<RG> st;
    st.reset();
    bf16x8 qa[8];
    if (p0 >= 0) {
        {   // A operand: row m = t*G + h is q[b, t, kvh*G + h]
            const int m = mrow < RG ? mrow : 0, t = m / G, h = m % G;
            const uint16_t *qr = p.q + (((int64_t)b * T + t) * Hq + kvh * G + h) * D + 8 * kg;
#pragma unroll
            for (int j = 0; j < 8; ++j) qa[j] = as_bf16x8(ld16(qr + 32 * j));
        }
        // this lane's key slot s of a cache round -> dkey: token t keeps it
        // iff dkey >= t (sliding: dkey = (s - pos) mod (window-1); full: all)
        auto dkey_of = [&](int r0e) {
            if (!p.sliding) return 0x7FFFFFFF;
            const int s = r0e + mrow;
            int d = (s - p0) % W1;
            return d < 0 ? d + W1 : d;
        };
        uint4 kA[8], vA[8], kB[8], vB[8];
        for (int r = r_lo; r < r_hi; r += 2) {
            const bool two = r + 1 < r_hi;
            issue_round(kblk, vblk, r0e_of(r), lane, kA, vA);
            issue_round(kblk, vblk, r0e_of(two ? r + 1 : r), two ? lane : 0, kB, vB);
            int e = r0e_of(r);
            st.template round<false, false, uint4, true, true>(qa, kA, vA, 16 * r - e, n_old - e,
                                                         p.scale_log2, s_pw[wave], s_kt[wave],
                                                         lane, -1, nullptr, nullptr, 1.f, 1.f,
                                                         dkey_of(e), trow);
            if (!two) break;
            e = r0e_of(r + 1);
            st.template round<false, false, uint4, true, true>(qa, kB, vB, 16 * (r + 1) - e, n_old - e,
                                                         p.scale_log2, s_pw[wave], s_kt[wave],
                                                         lane, -1, nullptr, nullptr, 1.f, 1.f,
                                                         dkey_of(e), trow);
        }
        if (last) {
            // the chunk's round: key x = token x (rows past T repeat token
            // 0, masked); token t sees x <= t, i.e. -x >= -t
            const int hw = lane >> 5, dl = lane & 31;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int x = 2 * j + hw, tok = x < T ? x : 0;
                const int64_t row = (((int64_t)b * T + tok) * Hkv + kvh) * D + 8 * dl;
                kA[j] = ld16(p.k_new + row);
                vA[j] = ld16(p.v_new + row);
            }
            st.template round<false, false, uint4, true, true>(qa, kA, vA, 0, T, p.scale_log2,
                                                         s_pw[wave], s_kt[wave], lane, -1,
                                                         nullptr, nullptr, 1.f, 1.f, -mrow, ntrow);
        }
    }

    // merge the waves (as the window kernel does), then out / lse per row
    float m_h[RG], l_h[RG];
    st.totals(m_h, l_h);
    const int hw = lane >> 5, dl = lane & 31;
    const bool has = p0 >= 0 && (r_lo < r_hi || last);
#pragma unroll
    for (int h = 0; h < RG; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float o = st.acc[h][e] + __shfl_xor(st.acc[h][e], 32, 64);
            if (hw == 0) s_red[(wave * RG + h) * D + 8 * dl + e] = o;
        }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < RG; ++h) {
            s_m[wave][h] = has ? m_h[h] : -INFINITY;
            s_l[wave][h] = has ? l_h[h] : 0.f;
        }
    }
    __syncthreads();
    for (int i = tid; i < RG * D; i += WAVES * 64) {
        const int m = i / D, d = i % D, t = m / G, hq = kvh * G + m % G;
        const int64_t orow = ((int64_t)b * T + t) * Hq + hq;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) M = fmaxf(M, s_m[w][m]);
        uint16_t *outp = p.out + orow * D + d;
        const int64_t prow = (int64_t)blockIdx.x * RG + m;  // partial row (split > 1)
        if (M == -INFINITY) {  // no keys here (a negative position, or none in this part)
            if (S > 1) {
                p.part_o[prow * D + d] = 0.f;
                if (d == 0) p.part_lse[prow] = -INFINITY;
                continue;
            }
            *outp = 0;
            if (d == 0 && p.lse) p.lse[orow] = -INFINITY;
            continue;
        }
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float sc = exp2f(s_m[w][m] - M);  // wave without keys: 2^-inf = 0
            L = fmaf(sc, s_l[w][m], L);
            o = fmaf(sc, s_red[(w * RG + m) * D + d], o);
        }
        const float lse = (M + log2f(L)) * kLn2;
        if (S > 1) {  // normalised partial and its lse
            p.part_o[prow * D + d] = o / L;
            if (d == 0) p.part_lse[prow] = lse;
            continue;
        }
        float f = 1.f / L;
        if (p.sinks) f *= 1.f / (1.f + expf(p.sinks[hq] - lse));
        if (p.gate) f *= gate_factor(p.gate[orow]);
        *outp = f32_to_bf16(o * f);
        if (d == 0 && p.lse) p.lse[orow] = lse;
    }
}

// The split partials of one (sequence, KV head, query row): out = sum_s
// e^(lse_s - lse) o_s with lse = ln sum_s e^(lse_s) (parts without keys
// weigh 0), then the sink and the gate.  One workgroup per (pair, row), a
// thread per dim (the row's S lse values are read by every thread: one
// cached broadcast).
__global__ __launch_bounds__(kHeadDim) void multi_merge_kernel(MultiParams p, int RG, int G) {
    constexpr int D = kHeadDim;
    const int S = p.split, Hkv = p.num_kv_heads, Hq = p.num_q_heads;
    const int pair = blockIdx.x / RG, m = blockIdx.x % RG, d = threadIdx.x;
    const int b = pair / Hkv, kvh = pair % Hkv;
    {
        const int t = m / G, hq = kvh * G + m % G;
        const int64_t orow = ((int64_t)b * p.tokens + t) * Hq + hq;
        float M = -INFINITY;
        for (int s = 0; s < S; ++s) M = fmaxf(M, p.part_lse[((int64_t)pair * S + s) * RG + m]);
        if (M == -INFINITY) {
            p.out[orow * D + d] = 0;
            if (d == 0 && p.lse) p.lse[orow] = -INFINITY;
            return;
        }
        float L = 0.f, o = 0.f;
        for (int s = 0; s < S; ++s) {
            const int64_t prow = ((int64_t)pair * S + s) * RG + m;
            const float e = expf(p.part_lse[prow] - M);  // -inf part: 0
            L += e;
            o = fmaf(e, p.part_o[prow * D + d], o);
        }
        const float lse = M + logf(L);
        float f = 1.f / L;
        if (p.sinks) f *= 1.f / (1.f + expf(p.sinks[hq] - lse));
        if (p.gate) f *= gate_factor(p.gate[orow]);
        p.out[orow * D + d] = f32_to_bf16(o * f);
        if (d == 0 && p.lse) p.lse[orow] = lse;
    }
}

template <int G, int T>
hipError_t launch_multi_gt(const MultiParams &p, hipStream_t s) {
    hipLaunchKernelGGL((decode_multi_kernel<G, T>), dim3(p.batch * p.num_kv_heads * p.split),
                       dim3(MultiShape<G, T>::WAVES * 64), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.split == 1) return e;
    hipLaunchKernelGGL(multi_merge_kernel, dim3(p.batch * p.num_kv_heads * G * T), dim3(kHeadDim),
                       0, s, p, G * T, G);
    return hipGetLastError();
}

template <int G>
hipError_t launch_multi_g(const MultiParams &p, hipStream_t s) {
    if constexpr (G * 4 <= 16) {
        switch (p.tokens) {
            case 1: return launch_multi_gt<G, 1>(p, s);
            case 2: return launch_multi_gt<G, 2>(p, s);
            case 3: return launch_multi_gt<G, 3>(p, s);
            case 4: return launch_multi_gt<G, 4>(p, s);
            default: return hipErrorInvalidValue;
        }
    } else if constexpr (G * 2 <= 16) {
        switch (p.tokens) {
            case 1: return launch_multi_gt<G, 1>(p, s);
            case 2: return launch_multi_gt<G, 2>(p, s);
            default: return hipErrorInvalidValue;
        }
    } else {
        return p.tokens == 1 ? launch_multi_gt<G, 1>(p, s) : hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_multi(const MultiParams &p, int group, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    const int bt = p.batch * p.tokens;
    hipLaunchKernelGGL(rope_multi_kernel, dim3(bt), dim3(kMultiRopeThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (group) {
        case 1: e = launch_multi_g<1>(p, stream); break;
        case 2: e = launch_multi_g<2>(p, stream); break;
        case 4: e = launch_multi_g<4>(p, stream); break;
        case 8: e = launch_multi_g<8>(p, stream); break;
        case 16: e = launch_multi_g<16>(p, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(append_multi_kernel, dim3(bt), dim3(128), 0, stream, p);
    return hipGetLastError();
}

}  // namespace hda
