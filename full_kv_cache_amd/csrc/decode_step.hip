// decode_step.hip -- one layer's decode step in one launch (gfx950): partial
// RoPE of q and k_new, the KV append, GQA attention over the layer's keys,
// the LSE merge of split pairs and the sink.
//
// What is computed is hda_rope_append followed by hda_decode_attn with
// seq_len = pos + 1 (Spark export page: `_angles`, `_rope`, `_Layer.forward`
// ring branch; flashmla_sparse page, `HYV4FlashMLASparseImpl` docstring, for
// the sink), except that the rotated q lives in registers only.
//
// hda_decode_step takes this kernel for sliding windows past one workgroup
// (more than 1024 keys); full layers take the streaming kernel's step form
// and sliding windows up to 1024 keys the window step below.  Its
// full-layer handling (sliding == 0) stays correct but is not routed to.
//
// Keys of sequence b at position P are rows 0..n-1 of its block, n =
// min(P+1, window) for a sliding layer, min(P+1, capacity) for a full one.
// Row vrow = min(P, window-1) (sliding) or P (full) stands for the new token:
// whatever memory holds there, the wave scoring that row replaces its K and V
// registers by the rotated k_new and v_new.  Every other key row is read
// before anything in this launch writes it:
//   * full, and sliding with P < window-1: the new token belongs in row vrow;
//     the wave that scores vrow's round stores it there.
//   * sliding with P >= window-1: it belongs in ring slot s = P mod
//     (window-1), whose entry (position P-window+1) is still a key of this
//     step.  The wave that scores s's round, once its loads of that round are
//     in, stores that entry to row window-1 (the evicted-entry row; only
//     vrow's round reads it, and replaces what it reads) and the new token
//     to slot s.
// The block thus ends as hda_rope_append leaves it, and no wave waits on
// another wave's store.
//
// The work is split like the balanced streaming decode: all 16-key rounds
// of all (sequence, KV head) pairs evenly over resident single-wave
// workgroups.  A pair inside one wave is finished there.  A pair spread over
// several waves leaves one partial per wave, written and read past the
// XCD-private caches; the last of them to finish (device-scope counter per
// pair, counted once the partial's stores are complete) merges them once its
// own rounds are done, writes out and lse with the sink, and resets the
// counter to zero for the next launch.
#include <type_traits>

#include "decode_wave.h"

namespace hda {

namespace {

using namespace wave;

// Keys of sequence b this step (0 for a negative position).
__device__ __forceinline__ int step_keys(const StepParams &p, int b) {
    const int P = p.pos[b];
    if (P < 0) return 0;
    const int64_t lim = p.sliding ? (int64_t)p.window : p.capacity;
    const int64_t n = (int64_t)P + 1;
    return (int)(n < lim ? n : lim);
}

struct RoundGeo {
    const uint16_t *kblk, *vblk;
    int r0e, lo, hi;  // in-bounds first row; valid keys [lo, hi) of the round
};

// Rows of the current pair that this launch treats specially.
struct PairRows {
    int vrow;  // row served by the new token (>= n: none)
    int srow;  // sliding past the window: slot taking the new token; else -1
    int erow;  // evicted-entry row, window-1
};

// Partials cross XCDs, whose L2 caches are not coherent with each other.
// Agent-scope relaxed atomic accesses are issued with the system-coherence
// bit, so they go past those caches; with them no L2 write-back or
// invalidation (what a device-wide fence costs) is needed around the count.
__device__ __forceinline__ void coherent_store(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// store_partial of decode_wave.h with coherent stores.
template <int G>
__device__ __forceinline__ void store_partial_coherent(const WaveSoftmax<G> &st, float *po, float *plse,
                                                       int lane) {
    const int hw = lane >> 5, dl = lane & 31;
    float m_h[G], l_h[G];
    st.totals(m_h, l_h);
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float l = l_h[h];
        const float inv = 1.f / l;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float o = xor32_sum(st.acc[h][e]) * inv;
            if (hw == 0) coherent_store(po + h * kHeadDim + 8 * dl + e, o);
        }
        if (lane == 0) coherent_store(plse + h, (m_h[h] + log2f(l)) * kLn2);
    }
}

// Writes out (bf16, with the sink) and lse of a pair finished in one wave.
template <int G>
__device__ __forceinline__ void store_final(const WaveSoftmax<G> &st, const StepParams &p, int b,
                                            int kvh, int lane) {
    const int hw = lane >> 5, dl = lane & 31;
    float m_h[G], l_h[G];
    st.totals(m_h, l_h);
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const int hq = kvh * G + h;
        const float l = l_h[h];
        const float lse = (m_h[h] + log2f(l)) * kLn2;
        float f = 1.f / l;
        if (p.sinks) f *= 1.f / (1.f + expf(p.sinks[hq] - lse));
        if (p.gate) f *= gate_factor(p.gate[(int64_t)b * p.num_q_heads + hq]);
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = xor32_sum(st.acc[h][2 * e]) * f;
            const float c = xor32_sum(st.acc[h][2 * e + 1]) * f;
            w[e] = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(c) << 16);
        }
        const int64_t row = (int64_t)b * p.num_q_heads + hq;
        if (hw == 0)
            *reinterpret_cast<uint4 *>(p.out + row * kHeadDim + 8 * dl) = make_uint4(w[0], w[1], w[2], w[3]);
        if (lane == 0 && p.lse) p.lse[row] = lse;
    }
}

// Merge of a pair's partials in slots [s0, s0 + nseg): lse = ln sum exp(lse_s),
// out = sum exp(lse_s - lse) o_s, then the sink.  Lane = dims 4*lane .. +3
// of every head; segments in batches, online rescaling between batches.
template <int G>
__device__ __forceinline__ void merge_pair(const StepParams &p, int64_t s0, int nseg, int b, int kvh,
                                           int lane) {
    constexpr int D = kHeadDim;
    constexpr int K = G >= 16 ? 2 : 32 / G;  // segments per batch
    float M[G], L[G];
    float4 o[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        M[h] = -INFINITY;
        L[h] = 0.f;
        o[h] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int base = 0; base < nseg; base += K) {
        float ls[K][G];
        float4 ov[K][G];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const bool in = base + k < nseg;
            const int64_t slot = s0 + (in ? base + k : nseg - 1);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float x = coherent_load(p.part_lse + slot * G + h);
                ls[k][h] = in ? x : -INFINITY;
                const float *src = p.part_o + (slot * G + h) * D + 4 * lane;
                ov[k][h] = make_float4(coherent_load(src), coherent_load(src + 1), coherent_load(src + 2),
                                       coherent_load(src + 3));
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float bm = M[h];
#pragma unroll
            for (int k = 0; k < K; ++k) bm = fmaxf(bm, ls[k][h]);  // finite: segment 0 holds keys
            const float sc = expf(M[h] - bm);                      // 0 on the first batch
            L[h] *= sc;
            o[h].x *= sc; o[h].y *= sc; o[h].z *= sc; o[h].w *= sc;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float wgt = expf(ls[k][h] - bm);  // padding: exp(-inf) = 0
                L[h] += wgt;
                o[h].x = fmaf(wgt, ov[k][h].x, o[h].x);
                o[h].y = fmaf(wgt, ov[k][h].y, o[h].y);
                o[h].z = fmaf(wgt, ov[k][h].z, o[h].z);
                o[h].w = fmaf(wgt, ov[k][h].w, o[h].w);
            }
            M[h] = bm;
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const int hq = kvh * G + h;
        const float lse = M[h] + logf(L[h]);
        float f = 1.f / L[h];
        if (p.sinks) f *= 1.f / (1.f + expf(p.sinks[hq] - lse));
        if (p.gate) f *= gate_factor(p.gate[(int64_t)b * p.num_q_heads + hq]);
        const int64_t row = (int64_t)b * p.num_q_heads + hq;
        const uint32_t lo = (uint32_t)f32_to_bf16(o[h].x * f) | ((uint32_t)f32_to_bf16(o[h].y * f) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(o[h].z * f) | ((uint32_t)f32_to_bf16(o[h].w * f) << 16);
        *reinterpret_cast<uint2 *>(p.out + row * D + 4 * lane) = make_uint2(lo, hi);
        if (lane == 0 && p.lse) p.lse[row] = lse;
    }
}

template <int G, int ROT>
__global__ __launch_bounds__(64) void decode_step_kernel(StepParams p) {
    constexpr int D = kHeadDim;
    static_assert(ROT % 16 == 0 && ROT <= D, "rotary dims in 16-byte chunk pairs");
    extern __shared__ int s_pre[];  // [B + 1]
    __shared__ __align__(16) float s_pw[16 * G];
    __shared__ __align__(16) uint16_t s_kt[kKTile];
    __shared__ __align__(16) float s_cos[ROT / 2], s_sin[ROT / 2];
    // rotated q of the pair's G heads, then its rotated new K, then new V
    __shared__ __align__(16) uint16_t s_rows[(G + 2) * D];
    __shared__ int s_merge[1 + 2 * 5];  // count, then (n, b, kvh, s0 lo, s0 hi) per merge owed
    uint16_t *const s_knew = s_rows + G * D, *const s_vnew = s_rows + (G + 1) * D;

    const int lane = threadIdx.x;
    const int mrow = lane & 15, kg = lane >> 4, hw = lane >> 5, dl = lane & 31;
    const int w = blockIdx.x, W = gridDim.x;
    const int B = p.batch, Hkv = p.num_kv_heads;

    round_prefix(s_pre, B, lane, [&](int b) { return step_keys(p, b); });
    __syncthreads();
    // sequences without keys (negative position): out 0, lse -inf
    for (int b = w; b < B; b += W) {
        if (s_pre[b + 1] != s_pre[b]) continue;
        const int64_t n_out = (int64_t)p.num_q_heads * D;
        uint16_t *ob = p.out + (int64_t)b * n_out;
        for (int64_t i = 8 * lane; i < n_out; i += 8 * 64)
            *reinterpret_cast<uint4 *>(ob + i) = make_uint4(0, 0, 0, 0);
        if (p.lse)
            for (int h = lane; h < p.num_q_heads; h += 64) p.lse[(int64_t)b * p.num_q_heads + h] = -INFINITY;
    }
    const int64_t r_tot = (int64_t)Hkv * s_pre[B];
    const int We = split_waves(W, r_tot);
    if (w >= We) return;
    const int64_t g0 = (int64_t)w * r_tot / We, g1 = (int64_t)(w + 1) * r_tot / We;

    RoundAddr cur = locate_round(s_pre, B, Hkv, g0);
    const int64_t cap = p.capacity, cap16 = cap - 16;
    auto geo = [&](const RoundAddr &a) HDA_INLINE {
        RoundGeo g;
        const int64_t bh = (int64_t)a.b * Hkv + a.kvh;
        g.kblk = p.k + bh * cap * D;
        g.vblk = p.v + bh * cap * D;
        const int r0 = a.rr * 16;
        g.r0e = (int)(r0 < cap16 ? r0 : cap16);
        g.lo = r0 - g.r0e;
        g.hi = uniform(step_keys(p, a.b)) - g.r0e;
        return g;
    };
    auto same_pair = [](const RoundAddr &x, const RoundAddr &y) { return x.b == y.b && x.kvh == y.kvh; };

    // Entering a pair: the angle table, then the pair's G query rows and its
    // new K row rotated (and the new V row copied) into LDS, 16-byte chunk
    // pairs spread over the lanes.
    auto enter_pair = [&](const RoundAddr &a) HDA_INLINE {
        PairRows pr;
        const int P = uniform(p.pos[a.b]);
        pr.erow = p.window - 1;
        pr.vrow = p.sliding ? min(P, p.window - 1) : P;
        pr.srow = (p.sliding && P >= p.window - 1) ? P % (p.window - 1) : -1;
        const int64_t bh = (int64_t)a.b * Hkv + a.kvh;
        // raw rows, one batch of 16-byte loads: rows r < G query heads,
        // r = G new K, r = G + 1 new V
        constexpr int kChunks = (G + 2) * D / 8, kPerLane = (kChunks + 63) / 64;
        const uint16_t *qrow = p.q + ((int64_t)a.b * p.num_q_heads + a.kvh * G) * D;
        uint4 raw[kPerLane];
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const int t = min(lane + 64 * i, kChunks - 1), r = t / (D / 8), d = 8 * (t % (D / 8));
            const uint16_t *src = r < G ? qrow + r * D : (r == G ? p.k_new : p.v_new) + bh * D;
            raw[i] = ld16(src + d);
        }
        wave_lds_fence();  // the previous pair's LDS reads are done
        for (int i = lane; i < ROT / 2; i += 64) {
            const float ang = (float)P * p.inv_freq[i];  // one fp32 multiply
            sincos_angle(ang, s_cos + i, s_sin + i);
        }
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const int t = lane + 64 * i;
            if (t < kChunks) *reinterpret_cast<uint4 *>(s_rows + 8 * t) = raw[i];
        }
        wave_lds_fence();
        // neox rotation in place: rows 0..G, 16-byte chunk pairs (i, i + ROT/2)
        constexpr int kRot = (G + 1) * (ROT / 16);
#pragma unroll
        for (int i = 0; i < (kRot + 63) / 64; ++i) {
            const int t = lane + 64 * i;
            if (t < kRot) {
                const int r = t / (ROT / 16), c = 8 * (t % (ROT / 16));
                uint16_t *row = s_rows + r * D;
                uint4 x1 = *reinterpret_cast<const uint4 *>(row + c);
                uint4 x2 = *reinterpret_cast<const uint4 *>(row + ROT / 2 + c);
                rotate8(x1, x2, s_cos + c, s_sin + c, x1, x2);
                *reinterpret_cast<uint4 *>(row + c) = x1;
                *reinterpret_cast<uint4 *>(row + ROT / 2 + c) = x2;
            }
        }
        wave_lds_fence();
        return pr;
    };
    // The q operand is read from LDS for every round instead of being held
    // in registers through the loop (rows >= G repeat row 0, as in
    // load_q_operand).
    const uint16_t *const q_lds = s_rows + (mrow < G ? mrow : 0) * D + 8 * kg;
    auto load_qa = [&](bf16x8 *qa) HDA_INLINE {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            qa[j] = as_bf16x8(*reinterpret_cast<const uint4 *>(q_lds + 32 * j));
        }
    };

    // Whether block row `row` is a valid key of this round (hi may exceed 16).
    auto in_round = [](const RoundGeo &g, int row) {
        const int x = row - g.r0e;
        return x >= g.lo && x < g.hi && x < 16;
    };
    // Key of the round served by the new token, or -1.
    auto sub_row = [&](const RoundGeo &g, const PairRows &pr) HDA_INLINE {
        return in_round(g, pr.vrow) ? pr.vrow - g.r0e : -1;
    };

    // After scoring a round: the append's stores (see the file comment).
    // The round's loads are consumed by then, so every old row it holds was
    // read before anything overwrites it.
    auto append_after = [&](const RoundAddr &a, const RoundGeo &g, const PairRows &pr, const uint4 *kt,
                            const uint4 *vt) HDA_INLINE {
        const int64_t bh = (int64_t)a.b * Hkv + a.kvh;
        const int sr = pr.srow - g.r0e;
        const bool has_s = pr.srow >= 0 && in_round(g, pr.srow);
        const bool has_v = pr.srow < 0 && in_round(g, pr.vrow);
        if (!has_s && !has_v) return;
        if (has_s) {  // the slot's old entry to the evicted-entry row
            uint16_t *ke = p.k + (bh * cap + pr.erow) * D, *ve = p.v + (bh * cap + pr.erow) * D;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (2 * u + hw == sr) {
                    *reinterpret_cast<uint4 *>(ke + 8 * dl) = kt[u];
                    *reinterpret_cast<uint4 *>(ve + 8 * dl) = vt[u];
                }
        }
        // the new token into its row: lanes 0..31 K, 32..63 V, 16 bytes each.
        // Slot s was loaded by this round; its store must not be issued before
        // those loads have returned, so its address is made to depend on a
        // register of each of the round's 16 loads (the compiler then waits
        // for all of them).
        const int64_t drow = has_s ? pr.srow : pr.vrow;
        int off = 8 * dl;
        asm volatile("" : "+v"(off)
                     : "v"(kt[0].w), "v"(kt[1].w), "v"(kt[2].w), "v"(kt[3].w), "v"(kt[4].w),
                       "v"(kt[5].w), "v"(kt[6].w), "v"(kt[7].w), "v"(vt[0].w), "v"(vt[1].w),
                       "v"(vt[2].w), "v"(vt[3].w), "v"(vt[4].w), "v"(vt[5].w), "v"(vt[6].w),
                       "v"(vt[7].w));
        uint16_t *dst = (lane < 32 ? p.k : p.v) + (bh * cap + drow) * D + off;
        *reinterpret_cast<uint4 *>(dst) =
            *reinterpret_cast<const uint4 *>((lane < 32 ? s_knew : s_vnew) + 8 * dl);
    };

    // Segment end: finish the pair here, or leave a partial and count in.
    // Returns the number of segments when this wave arrived last (the merge
    // is done after the wave's own rounds), else 0.
    WaveSoftmax<G> st;
    auto end_segment = [&](const RoundAddr &a, int64_t &s0) HDA_INLINE -> int {
        const int rb = s_pre[a.b + 1] - s_pre[a.b];
        const int64_t g_lo = (int64_t)Hkv * s_pre[a.b] + (int64_t)a.kvh * rb;
        const int w_lo = wave_of_round(g_lo, r_tot, We);
        const int w_hi = wave_of_round(g_lo + rb - 1, r_tot, We);
        if (w_lo == w_hi) {
            store_final<G>(st, p, a.b, a.kvh, lane);
            return 0;
        }
        const int64_t pair = (int64_t)a.b * Hkv + a.kvh;
        const int64_t slot = (int64_t)w + pair;
        store_partial_coherent<G>(st, p.part_o + slot * G * D, p.part_lse + slot * G, lane);
        // The partial's stores bypass the XCD-private L2 (see
        // store_partial_coherent); once they are complete the count may go up.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        int old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(p.counters + pair, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __shfl(old, 0, 64);
        asm volatile("" ::: "memory");
        if (old != w_hi - w_lo) return 0;
        if (lane == 0) __hip_atomic_store(p.counters + pair, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s0 = (int64_t)w_lo + pair;
        return w_hi - w_lo + 1;
    };

    // At most two of a wave's pairs are shared with other waves: its first
    // and its last.  The merges this wave owes are recorded in LDS (the
    // workgroup is this one wave) and done after its last round; carried in
    // registers through the loop they cost occupancy.
    if (lane == 0) s_merge[0] = 0;
    auto finish = [&](const RoundAddr &a) HDA_INLINE {
        int64_t s0 = 0;
        const int n = uniform(end_segment(a, s0));
        if (n && lane == 0) {
            const int k = s_merge[0];
            int *rec = s_merge + 1 + 5 * k;
            rec[0] = n;
            rec[1] = a.b;
            rec[2] = a.kvh;
            rec[3] = (int)(s0 & 0xffffffff);
            rec[4] = (int)(s0 >> 32);
            s_merge[0] = k + 1;
        }
    };

    uint4 kA[8], vA[8], kB[8], vB[8];
    RoundGeo gc = geo(cur);
    issue_round(gc.kblk, gc.vblk, gc.r0e, lane, kA, vA);
    PairRows pr = enter_pair(cur);
    st.reset();

    // Two rounds in flight, as in the streaming decode; the last round
    // issues a placeholder round of one address.
    int64_t g = g0;
    while (true) {
        bool more = g + 1 < g1;
        RoundAddr nxt = more ? next_round(s_pre, B, Hkv, cur) : cur;
        RoundGeo gn = geo(nxt);
        issue_round(gn.kblk, gn.vblk, gn.r0e, more ? lane : 0, kB, vB);
        {
            bf16x8 qa[8];
            load_qa(qa);
            st.template round<true>(qa, kA, vA, gc.lo, gc.hi, p.scale_log2, s_pw, s_kt, lane, sub_row(gc, pr),
                                    s_knew, s_vnew);
        }
        append_after(cur, gc, pr, kA, vA);
        if (!more || !same_pair(nxt, cur)) {
            finish(cur);
            if (!more) break;
            pr = enter_pair(nxt);
            st.reset();
        }
        cur = nxt;
        gc = gn;
        ++g;

        more = g + 1 < g1;
        nxt = more ? next_round(s_pre, B, Hkv, cur) : cur;
        gn = geo(nxt);
        issue_round(gn.kblk, gn.vblk, gn.r0e, more ? lane : 0, kA, vA);
        {
            bf16x8 qa[8];
            load_qa(qa);
            st.template round<true>(qa, kB, vB, gc.lo, gc.hi, p.scale_log2, s_pw, s_kt, lane, sub_row(gc, pr),
                                    s_knew, s_vnew);
        }
        append_after(cur, gc, pr, kB, vB);
        if (!more || !same_pair(nxt, cur)) {
            finish(cur);
            if (!more) break;
            pr = enter_pair(nxt);
            st.reset();
        }
        cur = nxt;
        gc = gn;
        ++g;
    }
    wave_lds_fence();
    const int n_merge = uniform(s_merge[0]);
    for (int k = 0; k < n_merge; ++k) {
        const int *rec = s_merge + 1 + 5 * k;
        const int64_t s0 = (int64_t)(uint32_t)uniform(rec[3]) | ((int64_t)uniform(rec[4]) << 32);
        merge_pair<G>(p, s0, uniform(rec[0]), uniform(rec[1]), uniform(rec[2]), lane);
    }
}

#ifndef HDA_WINDOW_WAVES
#define HDA_WINDOW_WAVES 8
#endif
constexpr int kWindowWaves = HDA_WINDOW_WAVES;

// ===================================================================
// Window form of the step (sliding layers, window <= kPairMaxKeys): S
// workgroups of kWindowWaves waves per (sequence, KV head), with the whole
// step inside:
//   * prologue: the angle table for the sequence's position, the
//     workgroup's query rows and the new K rotated into LDS, the new V
//     copied there;
//   * rounds: the new token's row (min(pos, window-1)) is served from LDS;
//     the round that reads ring slot s keeps its old entry (a key of this
//     step) in LDS as well;
//   * epilogue: the waves merge in LDS.
// Two ways to split a pair over its S workgroups:
//   * KS (key split; query groups up to 4): workgroup `part` scores rounds
//     [part R / S, (part+1) R / S) of the pair's R 16-key rounds for every
//     query head of the group, so each key row is read once.  With S > 1
//     each workgroup leaves a normalised partial (o, lse in log2 units),
//     written and read past the XCD-private caches; the last of the S to
//     count in (a counter per pair, taken once its partial's stores are
//     complete) merges them, writes out / lse with the sink and resets the
//     counter.  The append is written by the workgroup whose rounds hold
//     the row the new token takes (its ring slot, or row pos below a full
//     window), once its own loads are consumed: that row is read by no
//     other workgroup, and the evicted-entry row it also writes is only
//     read where the new token's row replaces what was loaded.
//   * head split (query groups of 8 and 16, whose accumulators would not
//     fit two rounds in flight, and any group once the pairs alone fill
//     the device): workgroup `part` serves query heads part GW .. +GW-1
//     over every key; it writes out / lse itself, and the last
//     of the S workgroups to count in writes the append.  A workgroup
//     counts in (the counter again) from the wave whose round holds the
//     row the new token takes, once that round's rows are in registers:
//     the append overwrites no other row any workgroup reads (the new
//     token's own row is served from LDS), so the count's return and the
//     append overlap the wave's later rounds instead of following the
//     merge.
// No data passes between the workgroups of a pair except the partials.
// F8 (fp8 cache: e4m3 codes + a scale per row): rounds load codes and the
// key scales (as the streaming kernel's fp8 form); the prologue quantizes
// the new K and V rows (scale = amax / 448) into LDS; the round holding the
// new token's row takes its codes and scales there; the kept old entry and
// the append move codes and scales together.
// ===================================================================
template <int GW, int ROT, bool F8, bool KS, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void decode_window_step_kernel(StepParams p, int S) {
    constexpr int D = kHeadDim;
    constexpr int NT = WAVES * 64;
    static_assert(ROT % 16 == 0 && ROT <= D, "rotary dims in 16-byte chunk pairs");
    static_assert(GW * D * sizeof(float) <= kKTile * sizeof(uint16_t), "a wave's o rows fit its K tile");
    __shared__ __align__(16) float s_pw[WAVES][16 * GW];
    // a wave's K tile; after its last round, its unnormalised o rows
    __shared__ __align__(16) uint16_t s_kt[WAVES][kKTile];
    __shared__ __align__(16) float s_cos[ROT / 2], s_sin[ROT / 2];
    // rows 0..GW-1 rotated q, GW rotated new K, GW+1 new V, GW+2/GW+3 the
    // old K/V entry of the ring slot the new token takes
    __shared__ __align__(16) uint16_t s_rows[(GW + 4) * D];
    __shared__ float s_m[WAVES][GW], s_l[WAVES][GW];
    __shared__ int s_last;
    // F8: codes of the new K, new V, old K, old V rows and their scales
    __shared__ __align__(16) uint8_t s_c8[F8 ? 4 * D : 16];
    __shared__ float s_c8s[4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hw = lane >> 5, dl = lane & 31, mrow = lane & 15, kg = lane >> 4;
    const int pairs = p.batch * p.num_kv_heads;
    const int x = blockIdx.x;
    const int part = (x >> 3) % S;
    const int pr = ((x >> 3) / S) * 8 + (x & 7);
    if (pr >= pairs) return;
    const int b = pr / p.num_kv_heads, kvh = pr % p.num_kv_heads;
    const int hsub = KS ? kvh : kvh * S + part;  // query heads hsub*GW .. +GW-1
    const int Hq = p.num_q_heads, W = p.window;
    const int P = p.pos[b];
    // the heads' sinks and output-gate logits, for the epilogue: uniform
    // addresses (scalar loads, which no wait for the K/V rows holds up)
    float sink[GW], glog[GW];
#pragma unroll
    for (int h = 0; h < GW; ++h) {
        sink[h] = p.sinks ? p.sinks[hsub * GW + h] : 0.f;
        glog[h] = p.gate ? p.gate[(int64_t)b * Hq + hsub * GW + h] : 0.f;
    }
    const int n = P < 0 ? 0 : min(P + 1, W);
    const int vrow = min(P, W - 1);                       // the new token's row
    const int srow = P >= W - 1 ? P % (W - 1) : -1;       // ring slot it takes
    const int64_t cap = p.capacity;
    const int64_t bh = (int64_t)b * p.num_kv_heads + kvh;
    uint16_t *kblk = p.k + bh * cap * D, *vblk = p.v + bh * cap * D;
    using KV = std::conditional_t<F8, uint2, uint4>;
    auto issue = [&](int r0e, int ln, KV *kt, KV *vt, float &ks, float &vs) HDA_INLINE {
        if constexpr (F8)
            issue_round8(p.kq + bh * cap * D, p.vq + bh * cap * D, p.ks + bh * cap, p.vs + bh * cap,
                         r0e, ln, kt, vt, ks, vs);
        else
            issue_round(kblk, vblk, r0e, ln, kt, vt);
    };
    uint16_t *const s_knew = s_rows + GW * D, *const s_vnew = s_rows + (GW + 1) * D;
    uint16_t *const s_oldk = s_rows + (GW + 2) * D, *const s_oldv = s_rows + (GW + 3) * D;

    // this workgroup's rounds [q_lo, q_hi), then this wave's share of them
    const int R = (n + 15) >> 4;
    const int q_lo = KS ? part * R / S : 0, q_hi = KS ? (part + 1) * R / S : R;
    const int r_lo = q_lo + wave * (q_hi - q_lo) / WAVES, r_hi = q_lo + (wave + 1) * (q_hi - q_lo) / WAVES;
    auto r0e_of = [&](int r) { return (int)((int64_t)(16 * r) < cap - 16 ? 16 * r : cap - 16); };

    // Prologue loads first, one 16-byte task per thread: the GW query rows
    // and the new K row as rotary chunk pairs (dims i..i+7 and i+ROT/2..)
    // or pass-through chunks, then the new V row; and this thread's
    // frequency.  Being older than every K/V load, they can be waited for
    // while the K/V loads stay in flight.  Branch-free: the row bases are
    // wave-uniform and the two loads of a thread are unconditional.
    constexpr int kRot = ROT / 16, kRow = kRot + (D - ROT) / 8;  // tasks per rotated row
    constexpr int kTasks = (GW + 1) * kRow + D / 8;
    static_assert(kTasks <= NT && ROT / 2 <= NT, "one prologue task per thread");
    const int tt = tid < kTasks ? tid : kTasks - 1;  // idle threads repeat the last task's loads
    const int tr = tt / kRow, tc = tt % kRow;
    const bool rotary = tr <= GW && tc < kRot;
    const uint16_t *qbase = uniform_ptr(p.q + ((int64_t)b * Hq + hsub * GW) * D);
    const uint16_t *kbase = uniform_ptr(p.k_new + bh * D), *vbase = uniform_ptr(p.v_new + bh * D);
    const uint16_t *src = tr < GW ? qbase + tr * D : tr == GW ? kbase : vbase;
    const int off = tr > GW ? 8 * (tt - (GW + 1) * kRow) : rotary ? 8 * tc : ROT + 8 * (tc - kRot);
    const uint4 x1_in = ld16_global(src + off), x2_in = ld16_global(src + off + (rotary ? ROT / 2 : 0));

    // The first round goes out before the rotation is computed (a wave
    // without one issues a placeholder round, so that every wave has the
    // same loads outstanding here), the second after it: measured on MI355X,
    // both rounds ahead of the prologue delay it more than they gain.
    KV kA[8], vA[8], kB[8], vB[8];
    float ksA = 1.f, vsA = 1.f, ksB = 1.f, vsB = 1.f;
    issue(r0e_of(r_lo), r_lo < r_hi ? lane : 0, kA, vA, ksA, vsA);
    // no load above may be moved below this point (next to its use)
    asm volatile("" ::: "memory");

    // Angle i = APW * wave + lane (lanes 0..APW-1): the wave reads its APW
    // frequencies with scalar loads, whose wait counter is not the vector
    // loads' (waiting for them does not wait for the K/V rows), and each
    // lane keeps its own.
    constexpr int APW = ROT / 2 <= 16 * WAVES ? 16 : 32;  // angles per wave
    static_assert(ROT / 2 <= APW * WAVES, "every angle has a lane");
    const int ai = APW * uniform(wave) + (lane & (APW - 1));
    float freq = 0.f;
    if (APW * uniform(wave) < ROT / 2) {
        const float4 *f4 = reinterpret_cast<const float4 *>(p.inv_freq + APW * uniform(wave));
        float f[APW];
#pragma unroll
        for (int k = 0; k < APW / 4; ++k) {
            const float4 v = f4[k];
            f[4 * k] = v.x;
            f[4 * k + 1] = v.y;
            f[4 * k + 2] = v.z;
            f[4 * k + 3] = v.w;
        }
#pragma unroll
        for (int k = 0; k < APW; ++k)
            if ((lane & (APW - 1)) == k) freq = f[k];
    }

    // Angles, then the rotated rows into LDS.  Done for an inactive
    // sequence too (nothing reads them then): a branch here would let the
    // compiler move the prologue loads behind the K/V loads.
    if (lane < APW && ai < ROT / 2) sincos_angle((float)P * freq, s_cos + ai, s_sin + ai);
    __syncthreads();
    if (tid < kTasks) {
        // the new V row (s_vnew) follows the new K row in s_rows
        uint16_t *dst = s_rows + tr * D;
        if (rotary) {
            uint4 y1, y2;
            rotate8(x1_in, x2_in, s_cos + off, s_sin + off, y1, y2);
            *reinterpret_cast<uint4 *>(dst + off) = y1;
            *reinterpret_cast<uint4 *>(dst + off + ROT / 2) = y2;
        } else {
            *reinterpret_cast<uint4 *>((tr > GW ? s_vnew : dst) + off) = x1_in;
        }
    }
    __syncthreads();
    {
        const bool has2 = r_lo + 1 < r_hi;
        issue(r0e_of(has2 ? r_lo + 1 : r_lo), has2 ? lane : 0, kB, vB, ksB, vsB);
    }
    if constexpr (F8) {  // the new rows' codes: wave 0 quantizes K, wave 1 V
        if (wave < 2) {
            const uint2 w = *reinterpret_cast<const uint2 *>((wave ? s_vnew : s_knew) + 4 * lane);
            const float xv[4] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
            float sc;
            const uint32_t c = quantize_row4(xv, sc);
            *reinterpret_cast<uint32_t *>(s_c8 + wave * D + 4 * lane) = c;
            if (lane == 0) s_c8s[wave] = sc;
        }
        __syncthreads();
    }

    // Head split: the wave whose round holds the row the new token takes
    // (its ring slot, or row pos below a full window) counts its workgroup
    // in on the pair's counter as soon as that round's rows are in
    // registers, and reads the count after its last round; the last of the
    // pair's workgroups to count in writes the append there.
    const int trow = srow >= 0 ? srow : vrow;
    int cnt = 0;           // lane 0 of the counting wave: the count before its own
    bool counted = false;  // wave-uniform
    auto count_in = [&](int r0e, int lo, int hi) HDA_INLINE {
        if constexpr (!KS) {
            const int tw = trow - r0e;
            if (tw >= lo && tw < hi && tw < 16) {
                // the round's loads (and every later one) complete first,
                // and no memory access moves across
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                if (lane == 0)
                    cnt = __hip_atomic_fetch_add(p.counters + pr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                counted = true;
            }
        }
    };

    WaveSoftmax<GW> st;
    st.reset();
    if (r_lo < r_hi) {
        // the q operand is read from LDS for every round (registers are short)
        const uint16_t *qs = s_rows + (mrow < GW ? mrow : 0) * D + 8 * kg;
        // a round's 16 rows start at r0e = min(16 r, capacity - 16): in bounds
        auto one = [&](int r, KV *kt, KV *vt, float ksc, float vsc) HDA_INLINE {
            bf16x8 qa[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                qa[j] = as_bf16x8(*reinterpret_cast<const uint4 *>(qs + 32 * j));  // rows >= GW repeat row 0
            }
            const int r0e = r0e_of(r), lo = 16 * r - r0e, hi = n - r0e;
            const int vr = vrow - r0e, sr = srow - r0e;
            if constexpr (F8) {
                if (vr >= lo && vr < hi && vr < 16) {  // the new token's row from LDS (wave-uniform)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (2 * j + hw == vr) {
                            kt[j] = *reinterpret_cast<const uint2 *>(s_c8 + 8 * dl);
                            vt[j] = *reinterpret_cast<const uint2 *>(s_c8 + D + 8 * dl);
                        }
                    if (mrow == vr) {
                        ksc = s_c8s[0];
                        vsc = s_c8s[1];
                    }
                }
                st.template round<false, true, KV, false, true>(qa, kt, vt, lo, hi, p.scale_log2,
                                                                s_pw[wave], s_kt[wave], lane, -1,
                                                                nullptr, nullptr, ksc, vsc);
                if (srow >= 0 && sr >= lo && sr < hi && sr < 16) {  // keep the slot's old entry
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        if (2 * u + hw == sr) {
                            *reinterpret_cast<uint2 *>(s_c8 + 2 * D + 8 * dl) = kt[u];
                            *reinterpret_cast<uint2 *>(s_c8 + 3 * D + 8 * dl) = vt[u];
                        }
                    if (lane == sr) {  // lane l holds key l's scales
                        s_c8s[2] = ksc;
                        s_c8s[3] = vsc;
                    }
                }
                count_in(r0e, lo, hi);
                return;
            } else {
            // the round holding the new token's row takes it from LDS
            // (the condition is wave-uniform); P.V on bf16 dot products
            if (vr >= lo && vr < hi && vr < 16) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (2 * j + hw == vr) {
                        kt[j] = *reinterpret_cast<const uint4 *>(s_knew + 8 * dl);
                        vt[j] = *reinterpret_cast<const uint4 *>(s_vnew + 8 * dl);
                    }
            }
            st.template round<false, false, uint4, false, true>(qa, kt, vt, lo, hi, p.scale_log2,
                                                                s_pw[wave], s_kt[wave], lane);
            if (srow >= 0 && sr >= lo && sr < hi && sr < 16) {  // keep the slot's old entry
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (2 * u + hw == sr) {
                        *reinterpret_cast<uint4 *>(s_oldk + 8 * dl) = kt[u];
                        *reinterpret_cast<uint4 *>(s_oldv + 8 * dl) = vt[u];
                    }
            }
            count_in(r0e, lo, hi);
            }
        };
        for (int r = r_lo; r < r_hi; r += 2) {
            const bool two = r + 1 < r_hi;
            if (r != r_lo) {
                issue(r0e_of(r), lane, kA, vA, ksA, vsA);
                issue(r0e_of(two ? r + 1 : r), two ? lane : 0, kB, vB, ksB, vsB);
            }
            one(r, kA, vA, ksA, vsA);
            if (!two) break;
            one(r + 1, kB, vB, ksB, vsB);
        }
    }
    if (!KS && counted && __builtin_amdgcn_readfirstlane(cnt) == S - 1) {
        // the last to count in: reset the counter, then the slot's old entry
        // (kept in LDS by this wave) to the evicted-entry row and the new
        // token to its slot -- lanes 0..31 the K row, 32..63 the V row
        if (lane == 0) __hip_atomic_store(p.counters + pr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int c = lane & 31, row = srow >= 0 ? srow : vrow;
        if constexpr (F8) {
            uint8_t *blk = (hw ? p.vq : p.kq) + bh * cap * D;
            float *sblk = (hw ? p.vs : p.ks) + bh * cap;
            const uint2 nw = *reinterpret_cast<const uint2 *>(s_c8 + hw * D + 8 * c);
            if (srow >= 0) {
                const uint2 od = *reinterpret_cast<const uint2 *>(s_c8 + (2 + hw) * D + 8 * c);
                *reinterpret_cast<uint2 *>(blk + (int64_t)(W - 1) * D + 8 * c) = od;
                if (c == 0) sblk[W - 1] = s_c8s[2 + hw];
            }
            *reinterpret_cast<uint2 *>(blk + (int64_t)row * D + 8 * c) = nw;
            if (c == 0) sblk[row] = s_c8s[hw];
        } else {
            uint16_t *blk = hw ? vblk : kblk;
            const uint4 nw = *reinterpret_cast<const uint4 *>((hw ? s_vnew : s_knew) + 8 * c);
            if (srow >= 0) {
                const uint4 od = *reinterpret_cast<const uint4 *>((hw ? s_oldv : s_oldk) + 8 * c);
                *reinterpret_cast<uint4 *>(blk + (int64_t)(W - 1) * D + 8 * c) = od;
            }
            *reinterpret_cast<uint4 *>(blk + (int64_t)row * D + 8 * c) = nw;
        }
    }

    // merge the waves: each leaves its unnormalised o rows in its own K
    // tile (its last round's reads of it come first in its LDS queue) and
    // its (m, l)
    float m_h[GW], l_h[GW];
    st.totals(m_h, l_h);
    float *red = reinterpret_cast<float *>(s_kt[wave]);
    wave_lds_fence();
#pragma unroll
    for (int h = 0; h < GW; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float o = xor32_sum(st.acc[h][e]);
            if (hw == 0) red[h * D + 8 * dl + e] = o;
        }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < GW; ++h) {
            s_m[wave][h] = r_lo < r_hi ? m_h[h] : -INFINITY;
            s_l[wave][h] = r_lo < r_hi ? l_h[h] : 0.f;
        }
    }
    // every wave's loads of the block are consumed past this barrier
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // out of head h (of this workgroup's GW), dim d, with the sink and gate
    auto write_out = [&](int h, int d, float o, float L, float lse) HDA_INLINE {
        const int hq = hsub * GW + h;
        uint16_t *outp = p.out + ((int64_t)b * Hq + hq) * D + d;
        if (L == 0.f) {  // no keys
            *outp = 0;
            if (d == 0 && p.lse) p.lse[(int64_t)b * Hq + hq] = -INFINITY;
            return;
        }
        float sk = 0.f, gl = 0.f;
#pragma unroll
        for (int j = 0; j < GW; ++j)
            if (j == h) {
                sk = sink[j];
                gl = glog[j];
            }
        float f = 1.f / L;
        if (p.sinks) f *= 1.f / (1.f + expf(sk - lse));
        if (p.gate) f *= gate_factor(gl);
        *outp = f32_to_bf16(o * f);
        if (d == 0 && p.lse) p.lse[(int64_t)b * Hq + hq] = lse;
    };
    // this workgroup's (o, l, max) of element i = h * D + d, merged over waves
    auto wave_merge = [&](int i, float &o, float &L, float &M) HDA_INLINE {
        const int h = i / D, d = i % D;
        M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) M = fmaxf(M, s_m[w][h]);
        L = 0.f;
        o = 0.f;
        if (M == -INFINITY) return;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float sc = exp2f(s_m[w][h] - M);
            L = fmaf(sc, s_l[w][h], L);
            o = fmaf(sc, reinterpret_cast<const float *>(s_kt[w])[h * D + d], o);
        }
    };

    if (!KS || S == 1) {
        for (int i = tid; i < GW * D; i += NT) {
            float o, L, M;
            wave_merge(i, o, L, M);
            write_out(i / D, i % D, o, L, L == 0.f ? -INFINITY : (M + log2f(L)) * kLn2);
        }
    } else if (P < 0) {  // no keys in any workgroup of the pair: the first writes
        if (part == 0)
            for (int i = tid; i < GW * D; i += NT) write_out(i / D, i % D, 0.f, 0.f, -INFINITY);
    } else {
        // this workgroup's normalised partial, lse in log2 units (-inf and
        // o = 0 without keys), past the XCD-private caches
        constexpr int EPT = (GW * D + NT - 1) / NT;  // elements per thread
        float own_o[EPT], own_l2[EPT];
        float *po = p.part_o + ((int64_t)pr * S + part) * GW * D;
        float *pl = p.part_lse + ((int64_t)pr * S + part) * GW;
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const int i = tid + k * NT;
            own_o[k] = 0.f;
            own_l2[k] = -INFINITY;
            if (i < GW * D) {
                float o, L, M;
                wave_merge(i, o, L, M);
                if (L > 0.f) {
                    own_o[k] = o / L;
                    own_l2[k] = M + log2f(L);
                }
                coherent_store(po + i, own_o[k]);
                if (i % D == 0) coherent_store(pl + i / D, own_l2[k]);
            }
        }
        // count in once this workgroup's partial stores are complete
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) {
            const int old = __hip_atomic_fetch_add(p.counters + pr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = old == S - 1;
            if (s_last) __hip_atomic_store(p.counters + pr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (s_last) {
            // every partial's loads go out before the first is used (S <= 8)
            const float *po0 = p.part_o + (int64_t)pr * S * GW * D;
            const float *pl0 = p.part_lse + (int64_t)pr * S * GW;
            float l2[EPT][8], ov[EPT][8];
#pragma unroll
            for (int k = 0; k < EPT; ++k) {
                const int i = min(tid + k * NT, GW * D - 1), h = i / D;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int sl = s < S && s != part ? s : (s == part ? part : S - 1);
                    l2[k][s] = coherent_load(pl0 + sl * GW + h);
                    ov[k][s] = coherent_load(po0 + (int64_t)sl * GW * D + i);
                }
            }
#pragma unroll
            for (int k = 0; k < EPT; ++k) {
                const int i = tid + k * NT;
                if (i >= GW * D) continue;
                float Mx = -INFINITY;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    if (s == part) {
                        l2[k][s] = own_l2[k];
                        ov[k][s] = own_o[k];
                    }
                    if (s >= S) l2[k][s] = -INFINITY;
                    Mx = fmaxf(Mx, l2[k][s]);
                }
                float L = 0.f, o = 0.f;  // Mx is finite: the last part holds a round
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const float w = s < S ? exp2f(l2[k][s] - Mx) : 0.f;
                    L += w;
                    o = fmaf(w, s < S ? ov[k][s] : 0.f, o);
                }
                write_out(i / D, i % D, o, L, (Mx + log2f(L)) * kLn2);
            }
        }
    }

    // The key split's append: the workgroup whose rounds hold the row the
    // new token takes (the head split's was written after the rounds).
    if constexpr (!KS) return;
    const bool app = P >= 0 && (trow >> 4) >= q_lo && (trow >> 4) < q_hi;
    if constexpr (F8) {
        if (app && tid < 128) {  // 8 code bytes per thread, K then V
            const int which = tid >> 6, c = tid & 31, half = (tid >> 5) & 1;
            uint8_t *blk = (which ? p.vq : p.kq) + bh * cap * D;
            float *sblk = (which ? p.vs : p.ks) + bh * cap;
            if (half == 0 && srow >= 0) {  // the slot's old entry to the evicted-entry row
                *reinterpret_cast<uint2 *>(blk + (int64_t)(W - 1) * D + 8 * c) =
                    *reinterpret_cast<const uint2 *>(s_c8 + (2 + which) * D + 8 * c);
                if (c == 0) sblk[W - 1] = s_c8s[2 + which];
            }
            if (half == 1) {  // the new token to its slot (row pos below a full window)
                const int row = srow >= 0 ? srow : vrow;
                *reinterpret_cast<uint2 *>(blk + (int64_t)row * D + 8 * c) =
                    *reinterpret_cast<const uint2 *>(s_c8 + which * D + 8 * c);
                if (c == 0) sblk[row] = s_c8s[which];
            }
        }
        return;
    }
    if (app && tid < 128) {  // 16 bytes per thread, K then V
        const int which = tid >> 6, c = tid & 31, half = (tid >> 5) & 1;
        uint16_t *blk = which ? vblk : kblk;
        if (half == 0 && srow >= 0)  // the slot's old entry to the evicted-entry row
            *reinterpret_cast<uint4 *>(blk + (int64_t)(W - 1) * D + 8 * c) =
                *reinterpret_cast<const uint4 *>((which ? s_oldv : s_oldk) + 8 * c);
        if (half == 1)  // the new token to its slot (row pos below a full window)
            *reinterpret_cast<uint4 *>(blk + (int64_t)(srow >= 0 ? srow : vrow) * D + 8 * c) =
                *reinterpret_cast<const uint4 *>((which ? s_vnew : s_knew) + 8 * c);
    }
}

template <int GW, int ROT, bool KS>
hipError_t launch_window_gr(const StepParams &p, int S, hipStream_t s) {
    constexpr int WAVES = kWindowWaves;
    const int64_t pairs = (int64_t)p.batch * p.num_kv_heads;
    const int64_t blocks = (pairs + 7) / 8 * 8 * S;
    if (p.kq)
        hipLaunchKernelGGL((decode_window_step_kernel<GW, ROT, true, KS, WAVES>), dim3((unsigned)blocks),
                           dim3(WAVES * 64), 0, s, p, S);
    else
        hipLaunchKernelGGL((decode_window_step_kernel<GW, ROT, false, KS, WAVES>), dim3((unsigned)blocks),
                           dim3(WAVES * 64), 0, s, p, S);
    return hipGetLastError();
}

template <int GW, bool KS>
hipError_t launch_window_g(const StepParams &p, int S, int rot, hipStream_t s) {
    if (rot == 64) return launch_window_gr<GW, 64, KS>(p, S, s);
    if (rot == 256) return launch_window_gr<GW, 256, KS>(p, S, s);
    return hipErrorInvalidValue;
}

template <int G, int ROT>
int step_slots_gr() {
    static std::atomic<int> cache[kMaxDevices];
    return resident_slots(reinterpret_cast<const void *>(decode_step_kernel<G, ROT>), 64, cache);
}

template <int G>
int step_slots_g(int rot) {
    return rot == 64 ? step_slots_gr<G, 64>() : rot == 256 ? step_slots_gr<G, 256>() : 0;
}

template <int G>
hipError_t launch_step_g(const StepParams &p, int rot, int waves, hipStream_t s) {
    if (rot == 64)
        hipLaunchKernelGGL((decode_step_kernel<G, 64>), dim3(waves), dim3(64), (p.batch + 1) * sizeof(int), s, p);
    else if (rot == 256)
        hipLaunchKernelGGL((decode_step_kernel<G, 256>), dim3(waves), dim3(64), (p.batch + 1) * sizeof(int), s, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

int step_wave_slots(int group, int rot) {
    switch (group) {
        case 1: return step_slots_g<1>(rot);
        case 2: return step_slots_g<2>(rot);
        case 4: return step_slots_g<4>(rot);
        case 8: return step_slots_g<8>(rot);
        case 16: return step_slots_g<16>(rot);
        default: return 0;
    }
}

hipError_t launch_decode_window_step(const StepParams &p, int group, int rot, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    const WindowPlan w = window_step_plan(group, (int64_t)p.batch * p.num_kv_heads, p.window);
    if (w.key_split) {
        switch (group) {
            case 1: return launch_window_g<1, true>(p, w.parts, rot, stream);
            case 2: return launch_window_g<2, true>(p, w.parts, rot, stream);
            case 4: return launch_window_g<4, true>(p, w.parts, rot, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (w.heads_per_part) {
        case 1: return launch_window_g<1, false>(p, w.parts, rot, stream);
        case 2: return launch_window_g<2, false>(p, w.parts, rot, stream);
        case 4: return launch_window_g<4, false>(p, w.parts, rot, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_step(const StepParams &p, int group, int rot, int waves, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    switch (group) {
        case 1: return launch_step_g<1>(p, rot, waves, stream);
        case 2: return launch_step_g<2>(p, rot, waves, stream);
        case 4: return launch_step_g<4>(p, rot, waves, stream);
        case 8: return launch_step_g<8>(p, rot, waves, stream);
        case 16: return launch_step_g<16>(p, rot, waves, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace hda
