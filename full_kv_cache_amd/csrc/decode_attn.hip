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
//     are the 16-row A operand (rows >= G repeat row 0, never read), the 16
//     keys the B operand, staged through a per-wave LDS tile from row-wise
//     16-byte loads;
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
#include <type_traits>

#include "decode_wave.h"

namespace hda {

namespace {

using namespace wave;

// Keys attended by sequence b (0 for seq_len <= 0).
__device__ __forceinline__ int num_keys(const DecodeParams &p, int b) {
    int n = p.seq_lens[b];
    n = n < p.max_keys ? n : p.max_keys;
    if (p.sliding) n = n < p.window ? n : p.window;
    return n > 0 ? n : 0;
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
    __shared__ __align__(16) uint16_t s_kt[WAVES][kKTile];
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
    load_q_operand<G>(p.q, p.num_q_heads, b, kvh, lane, qa);
    WaveSoftmax<G> st;
    st.reset();
    for (int kr = kw0; kr < kw1; kr += 16) {
        const int r0 = c0 + kr;  // block row of the round's first key
        const int r0e = (int)(r0 < cap16 ? r0 : cap16);
        uint4 kt[8], vt[8];
        issue_round(kblk, vblk, r0e, lane, kt, vt);
        st.round(qa, kt, vt, r0 - r0e, c0 + kw1 - r0e, p.scale_log2, s_pw[wave], s_kt[wave], lane);
    }

    // merge the waves: each leaves its unnormalised o and its (m, l)
    float m_h[G], l_h[G];
    st.totals(m_h, l_h);
    const int hw = lane >> 5, dl = lane & 31;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float o = xor32_sum(st.acc[h][e]);
            if (hw == 0) s_red[(wave * G + h) * D + 8 * dl + e] = o;
        }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            s_m[wave][h] = kw1 > kw0 ? m_h[h] : -INFINITY;
            s_l[wave][h] = kw1 > kw0 ? l_h[h] : 0.f;
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
            if (p.gate) f *= gate_factor(p.gate[(int64_t)b * Hq + hq]);
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
    if (p.gate) f *= gate_factor(p.gate[row]);
    *outp = f32_to_bf16((o / L) * f);
    if (d == 0 && p.lse) p.lse[row] = lse;
}

// ===================================================================
// Balanced streaming decomposition (the default path).
//
// Pair p = (b, kvh) holds R_b = ceil(n_b / 16) rounds of 16 keys; all
// rounds, pair after pair, form one index space of R_tot rounds.  Wave w of
// the W-wave grid (every wave resident at once; W is cut to R_tot when the
// lengths hold fewer rounds than the grid has waves) takes rounds
// [w*R_tot/W, (w+1)*R_tot/W): each wave streams the same number of keys
// (+-16) whatever the length mix, and no wave's range is empty.  A wave's range is cut at pair boundaries
// into segments; each leaves one partial in slot w + p -- unique, because
// the (wave, pair) overlaps are ordered the same way along both indices.
// Rounds are pipelined two deep: the next round's 16 loads are in flight
// while the current one is scored, softmaxed and accumulated.  (Claiming
// small tickets of work from atomic counters instead measured slower on
// MI355X: device-wide atomics serialise, and a partial per ticket adds
// traffic.)
// ===================================================================
struct RoundGeo {
    int64_t base;     // cache row index of the block (or page) row 0: codes at base * D
    int r0e, lo, hi;  // in-bounds first row; valid keys [lo, hi) of the round
};

template <bool STEP>
using StepArg = std::conditional_t<STEP, StreamStep, NoStep>;

// Keys of sequence b in the step form: the rows its block held before this
// token (the new one is scored apart and folded in by the merge).
__device__ __forceinline__ int held_keys(const StreamStep &ss, int64_t capacity, int b) {
    const int P = ss.pos[b];
    return P < 0 ? 0 : (int)((int64_t)P < capacity ? P : capacity);
}

// F8: the cache holds e4m3 codes and per-row scales (kq, vq, ks, vs).
// ROT > 0: the step form (rotary_dim ROT; bf16 or fp8): keys are the held
// rows, q is rotated at each pair's position, and the wave holding a pair's
// first round scores and appends the new token.  The fp8 step form runs
// the two-buffer loop below, not the plain fp8 loop.
template <int G, bool F8, int ROT = 0>
__global__ __launch_bounds__(64) void decode_stream_kernel(DecodeParams p, StepArg<(ROT > 0)> ss) {
    constexpr bool STEP = ROT > 0;
    constexpr int D = kHeadDim;
    extern __shared__ int s_pre[];                 // [B + 1] rounds before sequence b, one KV head
    __shared__ __align__(16) float s_pw[16 * G];   // this round's probabilities [key][head]
    __shared__ __align__(16) uint16_t s_kt[kKTile];
    __shared__ __align__(16) float2 s_cs[STEP ? D / 2 : 1];  // step form: (cos, sin) per angle
    __shared__ float s_freq[STEP ? D / 2 : 1];                // step form: frequencies
    __shared__ __align__(16) uint16_t s_q[STEP ? G * D : 1];  // step form: the pair's rotated q rows

    const int lane = threadIdx.x;
    const int w = blockIdx.x, W = gridDim.x;
    const int B = p.batch, Hkv = p.num_kv_heads;
    auto keys_of = [&](int b) HDA_INLINE {
        if constexpr (STEP)
            return held_keys(ss, p.capacity, b);
        else
            return num_keys(p, b);
    };
    // step form: the frequencies into LDS before any K/V row is loaded
    if constexpr (STEP) {
#pragma unroll
        for (int i = 0; i < (ROT / 2 + 63) / 64; ++i)
            if (lane + 64 * i < ROT / 2) s_freq[lane + 64 * i] = ss.inv_freq[lane + 64 * i];
    }

    round_prefix(s_pre, B, lane, [&](int b) { return keys_of(b); });
    __syncthreads();
    if (w == 0)  // published for the merge kernel
        for (int b = lane; b <= B; b += 64) p.stream_pre[b] = s_pre[b];
    const int64_t r_tot = (int64_t)Hkv * s_pre[B];
    const int We = split_waves(W, r_tot);
    if (w >= We) return;
    const int64_t g0 = (int64_t)w * r_tot / We, g1 = (int64_t)(w + 1) * r_tot / We;

    RoundAddr cur = locate_round(s_pre, B, Hkv, g0);
    auto advance = [&](RoundAddr a) { return next_round(s_pre, B, Hkv, a); };

    const int64_t cap = p.capacity, cap16 = cap - 16;
    auto geo = [&](const RoundAddr &a) {
        RoundGeo g;
        const int r0 = a.rr * 16;
        if (p.pages.block_table) {
            // paged: a round's 16 rows lie in one page (page_size is a
            // multiple of 16), rows r0 % page_size .. +15 of it
            const int ps = p.pages.page_size;
            const int64_t pg = uniform((int)page_of(p.pages, a.b, r0));
            g.base = (pg * Hkv + a.kvh) * ps;
            g.r0e = r0 % ps;
            g.lo = 0;
            g.hi = uniform(keys_of(a.b)) - r0;
            return g;
        }
        g.base = ((int64_t)a.b * Hkv + a.kvh) * cap;
        g.r0e = (int)(r0 < cap16 ? r0 : cap16);
        g.lo = r0 - g.r0e;
        g.hi = uniform(keys_of(a.b)) - g.r0e;
        return g;
    };
    auto same_pair = [](const RoundAddr &x, const RoundAddr &y) { return x.b == y.b && x.kvh == y.kvh; };

    using KV = std::conditional_t<F8, uint2, uint4>;
    auto issue = [&](const RoundGeo &g, int ln, KV *kt, KV *vt, float &ks, float &vs) {
        if constexpr (F8)
            issue_round8(p.kq + g.base * D, p.vq + g.base * D, p.ks + g.base, p.vs + g.base, g.r0e,
                         ln, kt, vt, ks, vs);
        else
            issue_round(p.k + g.base * D, p.v + g.base * D, g.r0e, ln, kt, vt);
    };

    bf16x8 qa[8];
    WaveSoftmax<G> st;
    auto end_segment = [&](const RoundAddr &a) {
        const int64_t slot = (int64_t)w + a.b * Hkv + a.kvh;
        store_partial<G>(st, p.part_o + slot * G * D, p.part_lse + slot * G, lane);
    };

    // Step form: the current pair's rotated q rows live in LDS, and every
    // round reads its operand from there (rows >= G repeat row 0), so no q
    // registers are carried through the loop: with them, the rotation code
    // at pair entry had changed the loop's register allocation (AGPR
    // copies) and slowed every round.
    const int mrow = lane & 15, kg = lane >> 4;
    // Entering a pair, the step form loads the new K and V rows with the q
    // rows (every lane, in the q operand's layout, whether or not it owns
    // the token: no value is then carried through the loop), rotates q and
    // K with the pair's angles and keeps the rotated q rows in LDS.  The
    // wave holding the pair's first round owns the new token: it scores it
    // against the G rotated rows (into the workspace, for the merge) and
    // writes the rotated K and the V row to row pos.  Other waves may read
    // row pos meanwhile only as a masked key.
    bf16x8 kn[8];
    uint4 vn8[8];
    auto load_pair = [&](const RoundAddr &a) HDA_INLINE {
        load_q_operand<G>(p.q, p.num_q_heads, a.b, a.kvh, lane, qa);
        if constexpr (STEP) {
            const int64_t nrow = ((int64_t)a.b * Hkv + a.kvh) * D + 8 * kg;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                kn[j] = as_bf16x8(ld16(ss.k_new + nrow + 32 * j));
                vn8[j] = ld16(ss.v_new + nrow + 32 * j);
            }
        }
    };
    auto finish_pair = [&](const RoundAddr &a) HDA_INLINE {
        if constexpr (STEP) {
            const int P = uniform(ss.pos[a.b]);
            rope_angles<ROT>(s_cs, s_freq, P, lane);
            rotate_q_operand<ROT>(qa, s_cs, lane);
            rotate_q_operand<ROT>(kn, s_cs, lane);
            if (mrow < G) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    *reinterpret_cast<uint4 *>(s_q + mrow * D + 32 * j + 8 * kg) =
                        __builtin_bit_cast(uint4, qa[j]);
            }
            // the pair has held rows, so P >= 1; P >= capacity: no new key
            if (a.rr == 0 && (int64_t)P < p.capacity) {
                const int64_t pr = (int64_t)a.b * Hkv + a.kvh;
                int64_t base;  // cache row index of row P
                if (p.pages.block_table) {
                    const int ps = p.pages.page_size;
                    base = (page_of(p.pages, a.b, P) * Hkv + a.kvh) * ps + P % ps;
                } else {
                    base = pr * p.capacity + P;
                }
                if constexpr (!F8) {
                    // score against the G rotated rows from registers (a
                    // lane's 64 dims of its row, then the 4 lane groups),
                    // the rows written as they are
                    float d = 0.f;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const uint4 qu = __builtin_bit_cast(uint4, qa[j]), ku = __builtin_bit_cast(uint4, kn[j]);
                        const uint32_t qw4[4] = {qu.x, qu.y, qu.z, qu.w}, kw4[4] = {ku.x, ku.y, ku.z, ku.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            d = fmaf(bf16_lo(qw4[e]), bf16_lo(kw4[e]), d);
                            d = fmaf(bf16_hi(qw4[e]), bf16_hi(kw4[e]), d);
                        }
                    }
                    d = xor32_sum(xor16_sum(d));
                    if (kg == 0 && mrow < G) ss.s_new[pr * G + mrow] = d * (p.scale_log2 * kLn2);
                    if (mrow == 0) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            *reinterpret_cast<uint4 *>(ss.k + base * D + 32 * j + 8 * kg) =
                                __builtin_bit_cast(uint4, kn[j]);
                            *reinterpret_cast<uint4 *>(ss.v + base * D + 32 * j + 8 * kg) = vn8[j];
                        }
                    }
                } else {
                    // The rotated K and the V row through LDS (the K tile is
                    // free between rounds), then 4 dims a lane as the append
                    // kernels lay a row out: fp8 rows are quantized as there
                    // (per-row amax / 448, codes e4m3(x / scale)), and the score
                    // reads the key as stored, times its scale, as a round does.
                    uint16_t *s_row = s_kt;  // [K row | V row]
                    if (mrow == 0) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            *reinterpret_cast<uint4 *>(s_row + 32 * j + 8 * kg) = __builtin_bit_cast(uint4, kn[j]);
                            *reinterpret_cast<uint4 *>(s_row + D + 32 * j + 8 * kg) = vn8[j];
                        }
                    }
                    wave_lds_fence();
                    const uint2 k4 = *reinterpret_cast<const uint2 *>(s_row + 4 * lane);
                    const uint2 v4 = *reinterpret_cast<const uint2 *>(s_row + D + 4 * lane);
                    float kx[4] = {bf16_lo(k4.x), bf16_hi(k4.x), bf16_lo(k4.y), bf16_hi(k4.y)};
                    float kscale;
                    {
                        const float vx[4] = {bf16_lo(v4.x), bf16_hi(v4.x), bf16_lo(v4.y), bf16_hi(v4.y)};
                        float vscale;
                        const uint32_t kc = quantize_row4(kx, kscale), vc = quantize_row4(vx, vscale);
                        *reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(ss.k) + base * D + 4 * lane) = kc;
                        *reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(ss.v) + base * D + 4 * lane) = vc;
                        if (lane == 0) {
                            ss.k_scale[base] = kscale;
                            ss.v_scale[base] = vscale;
                        }
                        const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)kc, false);
                        const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)kc, true);
                        kx[0] = lo.x;
                        kx[1] = lo.y;
                        kx[2] = hi.x;
                        kx[3] = hi.y;
                    }
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const uint2 q4 = *reinterpret_cast<const uint2 *>(s_q + h * D + 4 * lane);
                        float d = bf16_lo(q4.x) * kx[0];
                        d = fmaf(bf16_hi(q4.x), kx[1], d);
                        d = fmaf(bf16_lo(q4.y), kx[2], d);
                        d = fmaf(bf16_hi(q4.y), kx[3], d);
                        d = wave_sum(d);
                        if (lane == 0) ss.s_new[pr * G + h] = d * kscale * (p.scale_log2 * kLn2);
                    }
                }
            }
            wave_lds_fence();
        }
    };
    auto read_q = [&]() HDA_INLINE {
        if constexpr (STEP) {
            const uint16_t *qs = s_q + (mrow < G ? mrow : 0) * D + 8 * kg;
#pragma unroll
            for (int j = 0; j < 8; ++j) qa[j] = as_bf16x8(*reinterpret_cast<const uint4 *>(qs + 32 * j));
        }
    };
    if constexpr (F8 && !STEP) {
        // Rounds pipelined NB deep.  Buffer i % NB holds round g0 + i; the
        // loop body is unrolled NB times so that every buffer index is a
        // constant.  Rounds past g1 are placeholders (lane 0 addresses,
        // never computed).  Measured on MI355X: fp8 rounds are bound by
        // their compute chain, not by bytes in flight -- 4 deep at one wave
        // per SIMD ran slower than 2 deep with the grid at every resident
        // slot (two waves per SIMD hide each other's chains).
        constexpr int NB = 2;
        KV kb[NB][8], vb[NB][8];
        float ksb[NB], vsb[NB];
        RoundAddr ad[NB];
        RoundGeo ge[NB];
        ad[0] = cur;
#pragma unroll
        for (int i = 1; i < NB - 1; ++i) ad[i] = g0 + i < g1 ? advance(ad[i - 1]) : ad[i - 1];
        load_q_operand<G>(p.q, p.num_q_heads, cur.b, cur.kvh, lane, qa);
#pragma unroll
        for (int i = 0; i < NB - 1; ++i) {
            ge[i] = geo(ad[i]);
            issue(ge[i], g0 + i < g1 ? lane : 0, kb[i], vb[i], ksb[i], vsb[i]);
        }
        st.reset();
        int64_t g = g0;
        while (true) {
#pragma unroll
            for (int s = 0; s < NB; ++s) {
                const int t = (s + NB - 1) % NB, prv = (s + NB - 2) % NB;
                const bool live = g + NB - 1 < g1;
                ad[t] = live ? advance(ad[prv]) : ad[prv];
                ge[t] = geo(ad[t]);
                issue(ge[t], live ? lane : 0, kb[t], vb[t], ksb[t], vsb[t]);
                st.template round<false, F8, KV, false, true>(qa, kb[s], vb[s], ge[s].lo, ge[s].hi, p.scale_log2,
                                               s_pw, s_kt, lane, -1, nullptr, nullptr, ksb[s],
                                               vsb[s]);
                const bool more = g + 1 < g1;
                const RoundAddr &nx = ad[(s + 1) % NB];
                if (!more || !same_pair(nx, ad[s])) {
                    end_segment(ad[s]);
                    if (!more) return;
                    load_q_operand<G>(p.q, p.num_q_heads, nx.b, nx.kvh, lane, qa);
                    st.reset();
                }
                ++g;
            }
        }
    }

    KV kA[8], vA[8], kB[8], vB[8];
    float ksA = 1.f, vsA = 1.f, ksB = 1.f, vsB = 1.f;
    RoundGeo gc = geo(cur);
    if constexpr (STEP) {
        // the pair's rows before the first round's: rotating them waits for
        // them alone
        load_pair(cur);
        issue(gc, lane, kA, vA, ksA, vsA);
        finish_pair(cur);
    } else {
        issue(gc, lane, kA, vA, ksA, vsA);
        load_q_operand<G>(p.q, p.num_q_heads, cur.b, cur.kvh, lane, qa);
    }
    st.reset();
    // Entering a pair (step form: rotated at once; the wait for its rows
    // also waits for the next round's loads, once per pair per wave)
    auto enter_pair = [&](const RoundAddr &a) HDA_INLINE {
        load_pair(a);
        finish_pair(a);
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
        issue(gn, more ? lane : 0, kB, vB, ksB, vsB);
        read_q();
        st.template round<false, F8, KV, false, true>(qa, kA, vA, gc.lo, gc.hi, p.scale_log2, s_pw, s_kt, lane, -1,
                                      nullptr, nullptr, ksA, vsA);
        if (!more || !same_pair(nxt, cur)) {
            end_segment(cur);
            if (!more) break;
            enter_pair(nxt);
            st.reset();
        }
        cur = nxt;
        gc = gn;
        ++g;

        more = g + 1 < g1;
        nxt = more ? advance(cur) : cur;
        gn = geo(nxt);
        issue(gn, more ? lane : 0, kA, vA, ksA, vsA);
        read_q();
        st.template round<false, F8, KV, false, true>(qa, kB, vB, gc.lo, gc.hi, p.scale_log2, s_pw, s_kt, lane, -1,
                                      nullptr, nullptr, ksB, vsB);
        if (!more || !same_pair(nxt, cur)) {
            end_segment(cur);
            if (!more) break;
            enter_pair(nxt);
            st.reset();
        }
        cur = nxt;
        gc = gn;
        ++g;
    }
}

// Merge of the streaming partials: one wave per (sequence, query head),
// lane = 4 output dims.  The pair's rounds [g_lo, g_hi] were covered by
// waves wave_of(g_lo) .. wave_of(g_hi), whose partials sit in slots
// w + pair.  Lane s reads segment s's lse (64 segments a pass), the wave
// reduces max and sum, then the partials are read as float4 per lane in
// unrolled batches so that their loads are in flight together.
//
// STEP (hda_decode_step, full layer): the new token is one more key, row
// pos of its block when pos < capacity, taken as one more partial (its
// score, v_new).  The streaming kernel scored and appended it for every
// pair with held rows; for a pair without (pos 0) each wave rotates its
// head's q and the new K here (4 dims per lane; the partner dim i +- rot/2
// read from memory, the same fp32 fma and bf16 rounding as the append
// kernel) and scores them, and the wave of the group's first head appends
// the rotated K and V to row pos (nothing in this launch reads the cache).
template <bool STEP>
__global__ __launch_bounds__(64) void stream_merge_kernel(DecodeParams p, int W, StepArg<STEP> ss) {
    constexpr int D = kHeadDim;
    constexpr int kBatch = 16;
    const int hq = blockIdx.x % p.num_q_heads, b = blockIdx.x / p.num_q_heads;
    const int lane = threadIdx.x;
    const int Hq = p.num_q_heads, Hkv = p.num_kv_heads, G = Hq / Hkv;
    const int kvh = hq / G, h = hq % G;
    const int rb = p.stream_pre[b + 1] - p.stream_pre[b];
    const int64_t row = (int64_t)b * Hq + hq;
    uint16_t *outp = p.out + row * D + 4 * lane;
    bool fresh = false;  // step form: the new token is a key
    int P = 0;
    if constexpr (STEP) {
        P = ss.pos[b];
        fresh = P >= 0 && (int64_t)P < p.capacity;
    }
    if (rb == 0 && !fresh) {
        *reinterpret_cast<uint2 *>(outp) = make_uint2(0, 0);
        if (lane == 0 && p.lse) p.lse[row] = -INFINITY;
        return;
    }
    const int64_t r_tot = (int64_t)Hkv * p.stream_pre[p.batch];
    const int We = split_waves(W, r_tot);
    const int64_t g_lo = (int64_t)Hkv * p.stream_pre[b] + (int64_t)kvh * rb;
    const int w_lo = rb > 0 ? wave_of_round(g_lo, r_tot, We) : 0;
    const int nseg = rb > 0 ? wave_of_round(g_lo + rb - 1, r_tot, We) - w_lo + 1 : 0;
    const int64_t s0 = w_lo + (int64_t)b * Hkv + kvh;  // first slot
    // The new token's rows (step form), then the first batch of partials
    // and their lse go out first; the lse maximum (and for a pair with no
    // held rows the new token's rotation and score) run while they are in
    // flight.  A pair with held rows had its new key scored and appended by
    // the streaming wave that holds its first round.
    const bool self_score = fresh && rb == 0;
    uint2 qw = make_uint2(0, 0), kw = qw, vw = qw, qp = qw, kp = qw;
    float fr[4] = {0.f, 0.f, 0.f, 0.f};
    float s_ws = -INFINITY;
    const int d0 = 4 * lane;
    int rot = 0, half = 0, i0 = 0, pd = 0;
    bool first = false;
    const int64_t kvrow = ((int64_t)b * Hkv + kvh) * D;
    const bool f8 = p.kq != nullptr;  // fp8 cache: the new key and value as stored (codes x scale)
    int64_t nbase = 0;                // cache row index of row P
    uint32_t vcode = 0;
    float vsc = 1.f;
    if constexpr (STEP) {
        if (fresh && (self_score || f8)) {
            if (p.pages.block_table) {
                const int ps = p.pages.page_size;
                nbase = (page_of(p.pages, b, P) * Hkv + kvh) * ps + P % ps;
            } else {
                nbase = ((int64_t)b * Hkv + kvh) * p.capacity + P;
            }
        }
        if (fresh && (self_score || !f8)) vw = *reinterpret_cast<const uint2 *>(ss.v_new + kvrow + d0);
        if (fresh && !self_score) {
            s_ws = ss.s_new[row];
            if (f8) {  // written by the streaming kernel
                vcode = *reinterpret_cast<const uint32_t *>(p.vq + nbase * D + d0);
                vsc = p.vs[nbase];
            }
        }
        if (self_score) {
            rot = ss.rotary_dim;
            half = rot >> 1;
            first = d0 < half;  // x1 (first half) or x2
            pd = first ? d0 + half : d0 - half;
            i0 = first ? d0 : d0 - half;
            const uint16_t *qr = p.q + row * D, *kr = ss.k_new + kvrow;
            qw = *reinterpret_cast<const uint2 *>(qr + d0);
            kw = *reinterpret_cast<const uint2 *>(kr + d0);
            if (d0 < rot) {
                qp = *reinterpret_cast<const uint2 *>(qr + pd);
                kp = *reinterpret_cast<const uint2 *>(kr + pd);
#pragma unroll
                for (int e = 0; e < 4; ++e) fr[e] = ss.inv_freq[i0 + e];
            }
        }
    }
    float4 v[kBatch];
    float wgt[kBatch];
    auto load_batch = [&](int base) HDA_INLINE {
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int s = min(base + k, nseg - 1);
            v[k] = *reinterpret_cast<const float4 *>(p.part_o + ((s0 + s) * G + h) * D + 4 * lane);
            wgt[k] = base + k < nseg ? p.part_lse[(s0 + s) * G + h] : -INFINITY;
        }
    };
    if (nseg > 0) load_batch(0);
    float M = -INFINITY;
    for (int c = 0; c < nseg; c += 64)
        if (c + lane < nseg) M = fmaxf(M, p.part_lse[(s0 + c + lane) * G + h]);
    float s_new = s_ws;
    float vn[4] = {bf16_lo(vw.x), bf16_hi(vw.x), bf16_lo(vw.y), bf16_hi(vw.y)};
    // an fp8 row's 4 codes of this lane, decoded and scaled
    auto decode4 = [](uint32_t c, float sc, float *x) HDA_INLINE {
        const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);
        const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, true);
        x[0] = lo.x * sc;
        x[1] = lo.y * sc;
        x[2] = hi.x * sc;
        x[3] = hi.y * sc;
    };
    if constexpr (STEP) {
        if (fresh && !self_score && f8) decode4(vcode, vsc, vn);
        if (self_score) {
            float qx[4] = {bf16_lo(qw.x), bf16_hi(qw.x), bf16_lo(qw.y), bf16_hi(qw.y)};
            float kx[4] = {bf16_lo(kw.x), bf16_hi(kw.x), bf16_lo(kw.y), bf16_hi(kw.y)};
            uint2 krot = kw;
            if (d0 < rot) {
                const float qy[4] = {bf16_lo(qp.x), bf16_hi(qp.x), bf16_lo(qp.y), bf16_hi(qp.y)};
                const float ky[4] = {bf16_lo(kp.x), bf16_hi(kp.x), bf16_lo(kp.y), bf16_hi(kp.y)};
                uint16_t kb[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float c, sn;
                    sincos_angle((float)P * fr[e], &c, &sn);
                    // first half: x1 cos - x2 sin; second half: x2 cos + x1 sin
                    const uint16_t qb = f32_to_bf16(first ? fmaf(qx[e], c, -qy[e] * sn) : fmaf(qx[e], c, qy[e] * sn));
                    kb[e] = f32_to_bf16(first ? fmaf(kx[e], c, -ky[e] * sn) : fmaf(kx[e], c, ky[e] * sn));
                    qx[e] = bf16_to_f32(qb);
                    kx[e] = bf16_to_f32(kb[e]);
                }
                krot = make_uint2((uint32_t)kb[0] | ((uint32_t)kb[1] << 16),
                                  (uint32_t)kb[2] | ((uint32_t)kb[3] << 16));
            }
            float ksc = 1.f;
            uint32_t kc = 0, vc = 0;
            float vs_new = 0.f;
            if (f8) {  // quantized as the fp8 append kernel does; scores and P.V read the codes
                kc = quantize_row4(kx, ksc);
                vc = quantize_row4(vn, vs_new);
                decode4(kc, 1.f, kx);
                decode4(vc, vs_new, vn);
            }
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) dot = fmaf(qx[e], kx[e], dot);
            s_new = wave_sum(dot) * ksc * (p.scale_log2 * kLn2);  // natural-log units, as the partials
            if (h == 0) {
                if (f8) {
                    *reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(ss.k) + nbase * D + d0) = kc;
                    *reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(ss.v) + nbase * D + d0) = vc;
                    if (lane == 0) {
                        ss.k_scale[nbase] = ksc;
                        ss.v_scale[nbase] = vs_new;
                    }
                } else {
                    *reinterpret_cast<uint2 *>(ss.k + nbase * D + d0) = krot;
                    *reinterpret_cast<uint2 *>(ss.v + nbase * D + d0) = vw;
                }
            }
        }
    }
    M = fmaxf(wave_max(M), s_new);
    float L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (STEP && fresh) {
        const float e = expf(s_new - M);
        L = e;
        o = make_float4(e * vn[0], e * vn[1], e * vn[2], e * vn[3]);
    }
    for (int base = 0; base < nseg; base += kBatch) {
        if (base > 0) load_batch(base);
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const float e = expf(wgt[k] - M);  // padding: exp(-inf) = 0
            L += e;
            o.x = fmaf(e, v[k].x, o.x);
            o.y = fmaf(e, v[k].y, o.y);
            o.z = fmaf(e, v[k].z, o.z);
            o.w = fmaf(e, v[k].w, o.w);
        }
    }
    const float lse = M + logf(L);
    float f = 1.f / L;
    if (p.sinks) f *= 1.f / (1.f + expf(p.sinks[hq] - lse));
    if (p.gate) f *= gate_factor(p.gate[row]);
    const uint32_t lo = (uint32_t)f32_to_bf16(o.x * f) | ((uint32_t)f32_to_bf16(o.y * f) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(o.z * f) | ((uint32_t)f32_to_bf16(o.w * f) << 16);
    *reinterpret_cast<uint2 *>(outp) = make_uint2(lo, hi);
    if (lane == 0 && p.lse) p.lse[row] = lse;
}

// ===================================================================
// Window decomposition (sliding layers, every pair the same few hundred
// keys): one workgroup of kPairWaves waves per (sequence, KV head, 1/S of
// the query group).  The waves split the pair's rounds evenly, load them two
// at a time, merge in LDS and write out / lse with the sink: no partials, no
// merge kernel.  The S workgroups of a pair read the same K/V
// rows; their block ids are congruent mod 8 so that they run on the same XCD
// and the later reads hit its L2.
// ===================================================================
template <int GW, bool F8>
__global__ __launch_bounds__(kPairWaves * 64) void decode_pair_kernel(DecodeParams p, int S) {
    constexpr int D = kHeadDim;
    constexpr int WAVES = kPairWaves;
    __shared__ __align__(16) float s_red[WAVES * GW * D];
    __shared__ __align__(16) float s_pw[WAVES][16 * GW];
    __shared__ __align__(16) uint16_t s_kt[WAVES][kKTile];
    __shared__ float s_m[WAVES][GW], s_l[WAVES][GW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int pairs = p.batch * p.num_kv_heads;
    const int x = blockIdx.x;
    const int part = (x >> 3) % S;
    const int pr = ((x >> 3) / S) * 8 + (x & 7);
    if (pr >= pairs) return;
    const int b = pr / p.num_kv_heads, kvh = pr % p.num_kv_heads;
    const int hsub = kvh * S + part;  // heads hsub*GW .. +GW-1
    const int n = num_keys(p, b);
    const int R = (n + 15) >> 4;
    const int r_lo = wave * R / WAVES, r_hi = (wave + 1) * R / WAVES;
    const int64_t cap = p.capacity, cap16 = cap - 16;
    const int64_t bh = (int64_t)b * p.num_kv_heads + kvh;
    auto r0e_of = [&](int r) { return (int)((int64_t)(16 * r) < cap16 ? 16 * r : cap16); };
    using KV = std::conditional_t<F8, uint2, uint4>;
    auto issue = [&](int r0e, int ln, KV *kt, KV *vt, float &ks, float &vs) {
        if constexpr (F8)
            issue_round8(p.kq + bh * cap * D, p.vq + bh * cap * D, p.ks + bh * cap,
                         p.vs + bh * cap, r0e, ln, kt, vt, ks, vs);
        else
            issue_round(p.k + bh * cap * D, p.v + bh * cap * D, r0e, ln, kt, vt);
    };

    WaveSoftmax<GW> st;
    st.reset();
    if (r_lo < r_hi) {
        // Rounds in batches of two: both issued, then both scored (measured
        // on MI355X to stream faster here than keeping one round ahead).  An
        // odd last batch issues a placeholder second round.
        // The q operand goes out between the first batch's two rounds, so
        // that the first round waits for it and not for the second.
        bf16x8 qa[8];
        if constexpr (F8) {
            // Batches of NB rounds issued together (2 measured slightly
            // faster than 4 here).
            constexpr int NB = 2;
            KV kb[NB][8], vb[NB][8];
            float ksb[NB], vsb[NB];
            load_q_operand<GW>(p.q, p.num_q_heads, b, hsub, lane, qa);
            for (int r = r_lo; r < r_hi; r += NB) {
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    const bool live = r + i < r_hi;
                    issue(r0e_of(live ? r + i : r), live ? lane : 0, kb[i], vb[i], ksb[i], vsb[i]);
                }
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    if (r + i >= r_hi) break;
                    const int e = r0e_of(r + i);
                    st.template round<false, true, KV, false, true>(qa, kb[i], vb[i], 16 * (r + i) - e, n - e,
                                                   p.scale_log2, s_pw[wave], s_kt[wave], lane, -1,
                                                   nullptr, nullptr, ksb[i], vsb[i]);
                }
            }
        } else {
        KV kA[8], vA[8], kB[8], vB[8];
        float ksA = 1.f, vsA = 1.f, ksB = 1.f, vsB = 1.f;
        {
            const bool two = r_lo + 1 < r_hi;
            issue(r0e_of(r_lo), lane, kA, vA, ksA, vsA);
            load_q_operand<GW>(p.q, p.num_q_heads, b, hsub, lane, qa);
            issue(r0e_of(two ? r_lo + 1 : r_lo), two ? lane : 0, kB, vB, ksB, vsB);
        }
        for (int r = r_lo; r < r_hi; r += 2) {
            const bool two = r + 1 < r_hi;
            if (r != r_lo) {
                issue(r0e_of(r), lane, kA, vA, ksA, vsA);
                issue(r0e_of(two ? r + 1 : r), two ? lane : 0, kB, vB, ksB, vsB);
            }
            int e = r0e_of(r);
            st.template round<false, false, KV, false, true>(qa, kA, vA, 16 * r - e, n - e, p.scale_log2, s_pw[wave],
                                         s_kt[wave], lane, -1, nullptr, nullptr, ksA, vsA);
            if (!two) break;
            e = r0e_of(r + 1);
            st.template round<false, false, KV, false, true>(qa, kB, vB, 16 * (r + 1) - e, n - e, p.scale_log2,
                                         s_pw[wave], s_kt[wave], lane, -1, nullptr, nullptr, ksB,
                                         vsB);
        }
        }
    }

    // merge the waves: each leaves its unnormalised o and its (m, l)
    float m_h[GW], l_h[GW];
    st.totals(m_h, l_h);
    const int hw = lane >> 5, dl = lane & 31;
#pragma unroll
    for (int h = 0; h < GW; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float o = xor32_sum(st.acc[h][e]);
            if (hw == 0) s_red[(wave * GW + h) * D + 8 * dl + e] = o;
        }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < GW; ++h) {
            s_m[wave][h] = r_lo < r_hi ? m_h[h] : -INFINITY;
            s_l[wave][h] = r_lo < r_hi ? l_h[h] : 0.f;
        }
    }
    __syncthreads();
    const int Hq = p.num_q_heads;
    for (int i = tid; i < GW * D; i += WAVES * 64) {
        const int h = i / D, d = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) M = fmaxf(M, s_m[w][h]);
        const int hq = hsub * GW + h;
        uint16_t *outp = p.out + ((int64_t)b * Hq + hq) * D + d;
        if (M == -INFINITY) {  // no keys
            *outp = 0;
            if (d == 0 && p.lse) p.lse[(int64_t)b * Hq + hq] = -INFINITY;
            continue;
        }
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float sc = exp2f(s_m[w][h] - M);  // wave without keys: 2^-inf = 0
            L = fmaf(sc, s_l[w][h], L);
            o = fmaf(sc, s_red[(w * GW + h) * D + d], o);
        }
        const float lse = (M + log2f(L)) * kLn2;
        float f = 1.f / L;
        if (p.sinks) f *= 1.f / (1.f + expf(p.sinks[hq] - lse));
        if (p.gate) f *= gate_factor(p.gate[(int64_t)b * Hq + hq]);
        *outp = f32_to_bf16(o * f);
        if (d == 0 && p.lse) p.lse[(int64_t)b * Hq + hq] = lse;
    }
}

template <int GW>
hipError_t launch_pair_g(const DecodeParams &p, int S, hipStream_t s) {
    const int64_t pairs = (int64_t)p.batch * p.num_kv_heads;
    const int64_t blocks = (pairs + 7) / 8 * 8 * S;
    if (p.kq)
        hipLaunchKernelGGL((decode_pair_kernel<GW, true>), dim3((unsigned)blocks), dim3(kPairWaves * 64),
                           0, s, p, S);
    else
        hipLaunchKernelGGL((decode_pair_kernel<GW, false>), dim3((unsigned)blocks), dim3(kPairWaves * 64),
                           0, s, p, S);
    return hipGetLastError();
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
    if (p.kq)
        hipLaunchKernelGGL((decode_stream_kernel<G, true>), dim3(waves), dim3(64),
                           (p.batch + 1) * sizeof(int), s, p, NoStep{});
    else
        hipLaunchKernelGGL((decode_stream_kernel<G, false>), dim3(waves), dim3(64),
                           (p.batch + 1) * sizeof(int), s, p, NoStep{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_stream_merge(p, waves, s);
}

template <int G, bool F8>
void launch_stream_step_kernel(const DecodeParams &p, const StreamStep &ss, int waves, hipStream_t s) {
    if (ss.rotary_dim == 64)
        hipLaunchKernelGGL((decode_stream_kernel<G, F8, 64>), dim3(waves), dim3(64),
                           (p.batch + 1) * sizeof(int), s, p, ss);
    else
        hipLaunchKernelGGL((decode_stream_kernel<G, F8, 256>), dim3(waves), dim3(64),
                           (p.batch + 1) * sizeof(int), s, p, ss);
}

template <int G>
hipError_t launch_stream_step_g(const DecodeParams &p, const StreamStep &ss, int waves, hipStream_t s) {
    if (ss.rotary_dim != 64 && ss.rotary_dim != 256) return hipErrorInvalidValue;
    if (p.kq)
        launch_stream_step_kernel<G, true>(p, ss, waves, s);
    else
        launch_stream_step_kernel<G, false>(p, ss, waves, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(stream_merge_kernel<true>, dim3((unsigned)((int64_t)p.num_q_heads * p.batch)),
                       dim3(64), 0, s, p, waves, ss);
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
    static std::atomic<int> cache[kMaxDevices];
    return resident_slots(reinterpret_cast<const void *>(decode_stream_kernel<G, false>), 64, cache);
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

hipError_t launch_decode_stream_step(const DecodeParams &p, const StreamStep &ss, int group, int waves,
                                     hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    switch (group) {
        case 1: return launch_stream_step_g<1>(p, ss, waves, stream);
        case 2: return launch_stream_step_g<2>(p, ss, waves, stream);
        case 4: return launch_stream_step_g<4>(p, ss, waves, stream);
        case 8: return launch_stream_step_g<8>(p, ss, waves, stream);
        case 16: return launch_stream_step_g<16>(p, ss, waves, stream);
        default: return hipErrorInvalidValue;
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

// Query heads per workgroup: half the group when it has two or more heads.
hipError_t launch_decode_pairs(const DecodeParams &p, int group, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    switch (group) {
        case 1: return launch_pair_g<1>(p, 1, stream);
        case 2: return launch_pair_g<1>(p, 2, stream);
        case 4: return launch_pair_g<2>(p, 2, stream);
        case 8: return launch_pair_g<4>(p, 2, stream);
        case 16: return launch_pair_g<8>(p, 2, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_stream_merge(const DecodeParams &p, int waves, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    hipLaunchKernelGGL(stream_merge_kernel<false>, dim3((unsigned)((int64_t)p.num_q_heads * p.batch)),
                       dim3(64), 0, stream, p, waves, NoStep{});
    return hipGetLastError();
}

hipError_t launch_lse_merge(const MergeParams &p, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    hipLaunchKernelGGL(lse_merge_kernel, dim3(p.num_heads, p.batch), dim3(kDecodeThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace hda
