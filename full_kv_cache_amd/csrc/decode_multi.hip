// decode_multi.hip -- decode of a chunk of T new tokens per sequence
// (gfx950): RoPE, attention, append.
//
// Spark export page, `SparkStepConfig.cache_len` docstring: a ring holds
// the window's previous entries and the new token is scored together with
// them.  For a chunk, token t (position pos + t) attends to the entries of
// its own window -- cached ones and new tokens 0..t -- which is what T
// single-token steps in order would compute.  Three launches:
//   1. rope_multi_kernel: q rotated in place and the new K rotated into the
//      workspace at pos + t (the single-token kernel's arithmetic, so the
//      same bf16 values); k_new itself is only read;
//   2. attention over the cache as it was before the chunk plus the chunk's
//      own rows: prefill_chunk_kernel (below) when the chunk's tokens x G
//      query rows per KV head exceed one MFMA operand's 16, else
//      decode_multi_kernel: `split` workgroups per (sequence, KV head)
//      share its cache rounds; the chunk's T x G query rows (row t*G + h)
//      are the columns of both MFMA products, so every K/V row loaded
//      serves all T tokens.  Cache keys are masked per row: on a sliding layer token t
//      drops the t oldest entries (ring slots pos .. pos+t-1 mod window-1,
//      which tokens 0..t-1 replace); the new tokens are one more round, key
//      x visible to rows of token t >= x, taken by the last wave of the
//      last workgroup.  Each workgroup merges its waves in LDS and writes
//      out directly (split 1) or a partial (o, lse) per row that
//      multi_merge_kernel combines;
//   3. the append: the rotated new K and V rows into the cache (full:
//      rows pos + t; sliding: the ring slots of the last 511 tokens, and
//      the block's evicted-entry row receives the entry of position
//      pos + T - 512 -- a cached one or, for T = 512, token 0 -- as T
//      single-token appends leave it).  It runs after the attention, which
//      reads the slots it overwrites: in the merge launch when the keys
//      were split, in the attention kernel itself for an unsplit chunk
//      decode, else as append_multi_kernel.
#include <type_traits>

#include "decode_wave.h"

namespace hda {

using namespace wave;

namespace {

constexpr int kMultiRopeThreads = 256;

__device__ __forceinline__ uint4 ldm(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void stm(uint16_t *p, const uint4 &v) { *reinterpret_cast<uint4 *>(p) = v; }

// Block (b, token t): q [Hq] rows rotated in place, new K [Hkv] rows
// rotated into k_rot (the pass-through dims copied).
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
        const uint16_t *row;
        uint16_t *dst;
        int j;
        if (u < n_q) {
            dst = p.q + ((int64_t)bt * p.num_q_heads + u / hc) * D;
            row = dst;
            j = (u % hc) * 8;
        } else {
            const int64_t kr = ((int64_t)bt * p.num_kv_heads + (u - n_q) / hc) * D;
            row = p.k_new + kr;
            dst = p.k_rot + kr;
            j = ((u - n_q) % hc) * 8;
        }
        uint4 ya, yb;
        rotate8(ldm(row + j), ldm(row + half + j), s_cos + j, s_sin + j, ya, yb);
        stm(dst + j, ya);
        stm(dst + half + j, yb);
    }
    // the new K's pass-through dims
    const int npt = (D - rot) / 8;
    for (int u = threadIdx.x; u < p.num_kv_heads * npt; u += kMultiRopeThreads) {
        const int64_t kr = ((int64_t)bt * p.num_kv_heads + u / npt) * D + rot + 8 * (u % npt);
        stm(p.k_rot + kr, ldm(p.k_new + kr));
    }
}

// Where token t of a chunk at position p0 lands (the rules below).
struct AppendSlot {
    int64_t row;
    bool write, evict_old, evict_new;
};
__device__ __forceinline__ AppendSlot append_slot(const MultiParams &p, int32_t p0, int t) {
    const int64_t P = (int64_t)p0 + t;
    AppendSlot a{P, true, false, false};
    if (p.sliding) {
        const int slots = p.window - 1;
        const int64_t last = (int64_t)p0 + p.tokens - 1;  // the chunk's last position
        a.row = P % slots;
        a.write = t >= p.tokens - slots;
        if (last >= slots) {
            const int64_t e = last - slots;  // position the evicted-entry row ends holding
            a.evict_old = t == p.tokens - 1 && e < p0;
            a.evict_new = e >= p0 && P == e;
        }
    } else {
        a.write = P < p.capacity;
    }
    return a;
}

// Block (b, token t): the token's rotated K and its V into the cache.
// Sliding: only the last window-1 tokens land (an earlier token's slot is
// taken again by a later one); the evicted-entry row ends holding position
// pos + T - window (the entry a single-token step at pos + T - 1 moves
// there): written by the last token's block from its slot before that
// block overwrites it, or, when that position is in the chunk (T ==
// window), by that token's block from the chunk.
// Token bt = b * tokens + t of the chunk: its rows for every KV head, with
// nthreads threads (tid of them this one).
__device__ __forceinline__ void append_token(const MultiParams &p, int bt, int tid, int nthreads) {
    constexpr int D = kHeadDim;
    const int b = bt / p.tokens, t = bt % p.tokens;
    const int32_t p0 = p.pos[b];
    if (p0 < 0) return;
    const int64_t cap = p.capacity;
    const AppendSlot a = append_slot(p, p0, t);
    if (!a.write && !a.evict_old && !a.evict_new) return;
    const int64_t row = a.row;
    const bool evict_old = a.evict_old, evict_new = a.evict_new, write = a.write;
    const int Hkv = p.num_kv_heads;
    for (int u = tid; u < 2 * Hkv * (D / 8); u += nthreads) {
        const bool is_v = u >= Hkv * (D / 8);
        const int w = is_v ? u - Hkv * (D / 8) : u, h = w / (D / 8), d = (w % (D / 8)) * 8;
        uint16_t *blk = (is_v ? p.v : p.k) + ((int64_t)b * Hkv + h) * cap * D;
        const uint16_t *src = (is_v ? p.v_new : p.k_rot) + ((int64_t)bt * Hkv + h) * D;
        if (evict_old) stm(blk + (int64_t)(p.window - 1) * D + d, ldm(blk + row * D + d));
        if (evict_new) stm(blk + (int64_t)(p.window - 1) * D + d, ldm(src + d));
        if (write) stm(blk + row * D + d, ldm(src + d));
    }
}

__global__ __launch_bounds__(128) void append_multi_kernel(MultiParams p) {
    append_token(p, blockIdx.x, threadIdx.x, 128);
}

// Chunk decode, tokens x G <= 16 query rows per KV head: `split`
// workgroups of kMultiWaves waves per (sequence, KV head) share its cache
// rounds (16 keys; two in flight per wave, whole rows loaded into
// registers as the decode kernels load them).  The chunk's rows (row
// m = t G + h; rows past T G repeat row 0 and are never read) are the 16
// columns of both products, so every K/V row loaded serves all T tokens.
// Per round a wave writes the K and V rows into its LDS tiles in the
// prefill kernel's 1-KiB block layout, then:
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K the A operand, the
//     rotated query rows B, read from an LDS copy in the same layout);
//   * an online softmax per query row: lane (row m, kg) holds keys
//     4 kg .. 4 kg + 3 of the round;
//   * O^T += V^T P^T on v_mfma_f32_16x16x16_bf16: V^T one transposing read
//     per 16-dim tile, P^T the lane's own four probabilities (bf16).
// Cache keys are masked per row: on a sliding layer token t drops the t
// oldest entries (ring slots pos .. pos+t-1 mod window-1, which tokens
// 0..t-1 replace); the new tokens are one more round, key x visible to
// rows of token t >= x, taken by the last wave of the last workgroup.
// Each workgroup merges its waves in LDS and writes out directly (split 1)
// or a partial (o, lse) per row that multi_merge_kernel combines.
constexpr int kMultiWaves = 8;
constexpr int kMultiTile = 16 * kHeadDim * 2;  // bytes of 16 K (or V) rows
constexpr int kMultiPitch = kHeadDim + 4;      // floats per row of a wave's o rows
constexpr int kMultiAhead = 3;                 // K / q operand reads in flight
constexpr int kMultiTrAhead = 4;               // V^T reads in flight

template <int G, int T>
__global__ __launch_bounds__(kMultiWaves * 64, 1) void decode_multi_kernel(MultiParams p) {
    constexpr int D = kHeadDim;
    constexpr int RG = G * T;
    constexpr int WAVES = kMultiWaves;
    static_assert(RG <= 16, "the chunk's rows fill at most one operand");
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    // a wave's K and V tiles; after its rounds, its o rows [16][kMultiPitch]
    constexpr int kWaveLds = 16 * kMultiPitch * 4 > 2 * kMultiTile ? 16 * kMultiPitch * 4 : 2 * kMultiTile;
    __shared__ __align__(1024) unsigned char s_tile[WAVES][kWaveLds];
    __shared__ __align__(1024) unsigned char s_q[kMultiTile];  // the 16 query rows, block layout
    __shared__ float s_m[WAVES][16], s_l[WAVES][16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int mrow = lane & 15, kg = lane >> 4, hw = lane >> 5, dl = lane & 31;
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
    const int trow = mrow < RG ? mrow / G : 0;  // the token of this lane's row

    // Tile layout (1-KiB block j = dims 32j .. 32j+31): this lane's 16 bytes
    // of row r (dims 8 dl ..) go to slot r ^ 12 (c & 1) + 16 c of block dl / 4,
    // c = dl % 4; the K operand of row mrow, dims 32j + 8kg, is read from slot
    // drow + 16 kg; the transposing read of dim tile d from 512 d + tr_off
    // gives keys 4kg .. +3 of dim 16d + mrow.
    unsigned char *const ktl = s_tile[wave], *const vtl = s_tile[wave] + kMultiTile;
    const int wblk = 1024 * (dl >> 2) + 256 * (dl & 3), wsw = 12 * (dl & 1);
    const int drow = mrow ^ (12 * (kg & 1));
    const int tr_b = (mrow >> 1) & 1;
    const int tr_off = 256 * tr_b + 16 * ((4 * kg + (mrow >> 2)) ^ (12 * tr_b)) + 8 * (mrow & 1);

    f32x4 acc[D / 16];
#pragma unroll
    for (int d = 0; d < D / 16; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_lane = 0.f;  // row mrow; l over this lane's keys

    // One round: kt / vt the 16 rows (lane = 8 dims of row 2u + hw); key
    // 2u + hw's V row is taken only if vkeep (masked rows may hold anything,
    // even NaN, which a zero weight would not cancel); ok[i]: key 4kg + i
    // is seen by this lane's row.
    auto mround = [&](const uint4 *kt, const uint4 *vt, int lo, int hi, const bool *ok) HDA_INLINE {
        // (the store offsets are recomputed each round: kept across the
        // rounds they would take registers from the rounds in flight)
        int wb = wblk + 16 * hw, wx = 16 * wsw;
        asm volatile("" : "+v"(wb), "+v"(wx));
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int r = 2 * u + hw;
            const int off = wb + ((32 * u) ^ wx);
            *reinterpret_cast<uint4 *>(ktl + off) = kt[u];
            *reinterpret_cast<uint4 *>(vtl + off) = r >= lo && r < hi ? vt[u] : make_uint4(0, 0, 0, 0);
        }
        wave_lds_fence();
        // operand reads run kMultiAhead k-steps ahead of their products (all
        // eight at once would take the registers of the rounds in flight)
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
        uint4 ka[kMultiAhead], qa[kMultiAhead];
        auto op_read = [&](int j) HDA_INLINE {
            ka[j % kMultiAhead] = ld16(ktl + 1024 * j + 16 * (drow + 16 * kg));
            qa[j % kMultiAhead] = ld16(s_q + 1024 * j + 16 * (drow + 16 * kg));
        };
#pragma unroll
        for (int j = 0; j < kMultiAhead; ++j) op_read(j);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bf16x8 a = as_bf16x8(ka[j % kMultiAhead]), q = as_bf16x8(qa[j % kMultiAhead]);
            if (j + kMultiAhead < 8) op_read(j + kMultiAhead);
            __builtin_amdgcn_sched_barrier(0);
            if (j & 1) s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, q, s1, 0, 0, 0);
            else s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, q, s0, 0, 0, 0);
        }
        float s[4], tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[i] = ok[i] ? (s0[i] + s1[i]) * p.scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, s[i]);
        }
        tmax = xor32_max(xor16_max(tmax));
        const float m_new = fmaxf(m_run, tmax);
        const float mr = m_new == -INFINITY ? 0.f : m_new;  // no key for this row yet
        const float alpha = __builtin_amdgcn_exp2f(m_run - mr);  // -inf - x: 0
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int d = 0; d < D / 16; ++d) acc[d] *= alpha;
        }
        float pv[4], ps = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pv[i] = __builtin_amdgcn_exp2f(s[i] - mr);
            ps += pv[i];
        }
        l_lane = fmaf(l_lane, alpha, ps);
        m_run = m_new;
        const v4i16 pb = __builtin_bit_cast(v4i16, make_uint2(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])));
        v4i16 va[kMultiTrAhead];
#pragma unroll
        for (int d = 0; d < kMultiTrAhead; ++d)
            va[d] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vtl + 512 * d + tr_off));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < D / 16; ++d) {
            const v4i16 a = va[d % kMultiTrAhead];
            if (d + kMultiTrAhead < D / 16)
                va[d % kMultiTrAhead] =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vtl + 512 * (d + kMultiTrAhead) + tr_off));
            __builtin_amdgcn_sched_barrier(0);
            acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, acc[d], 0, 0, 0);
        }
        // the next round's stores follow these reads in this wave's LDS
        // queue, which runs in order; keep the compiler from moving them
        __builtin_amdgcn_wave_barrier();
    };

    // B operand rows: q[row mrow][32j + 8kg .. +7] at block j, slot drow + 16 kg
    // (wave 0 copies them; p0 is uniform over the workgroup)
    if (p0 >= 0 && wave == 0) {
        const int m = mrow < RG ? mrow : 0, t = m / G, h = m % G;
        const uint16_t *qr = p.q + (((int64_t)b * T + t) * Hq + kvh * G + h) * D + 8 * kg;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<uint4 *>(s_q + 1024 * j + 16 * (drow + 16 * kg)) = ld16(qr + 32 * j);
    }
    __syncthreads();
    if (p0 >= 0) {
        // cache round r: key x = slot r0e + x seen by token t iff lo <= x < hi
        // and, sliding, (slot - pos) mod (window-1) >= t
        auto cache_round = [&](int r, const uint4 *kt, const uint4 *vt) HDA_INLINE {
            const int e = r0e_of(r), lo = 16 * r - e, hi = n_old - e;
            bool ok[4];
            int dk = 0;
            if (p.sliding) {
                dk = (e + 4 * kg - p0) % W1;
                dk += dk < 0 ? W1 : 0;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int x = 4 * kg + i;
                bool v = x >= lo && x < hi;
                if (p.sliding) {
                    int d = dk + i;
                    d = W1 >= 4 ? (d >= W1 ? d - W1 : d) : d % W1;
                    v = v && d >= trow;
                }
                ok[i] = v;
            }
            mround(kt, vt, lo, hi, ok);
        };
        uint4 kA[8], vA[8], kB[8], vB[8];
        for (int r = r_lo; r < r_hi; r += 2) {
            const bool two = r + 1 < r_hi;
            issue_round(kblk, vblk, r0e_of(r), lane, kA, vA);
            issue_round(kblk, vblk, r0e_of(two ? r + 1 : r), two ? lane : 0, kB, vB);
            cache_round(r, kA, vA);
            if (!two) break;
            cache_round(r + 1, kB, vB);
        }
        if (last) {
            // the chunk's round: key x = token x (rows past T repeat token 0,
            // masked); token t sees x <= t
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int x = 2 * j + hw, tok = x < T ? x : 0;
                const int64_t row = (((int64_t)b * T + tok) * Hkv + kvh) * D + 8 * dl;
                kA[j] = ld16(p.k_rot + row);
                vA[j] = ld16(p.v_new + row);
            }
            bool ok[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) ok[i] = 4 * kg + i < T && 4 * kg + i <= trow;
            mround(kA, vA, 0, T, ok);
        }
    }

    // merge the waves: each leaves its o rows (unnormalised) in its own
    // tiles, then out / lse per row
    const float l_row = xor32_sum(xor16_sum(l_lane));
    const bool has = p0 >= 0 && (r_lo < r_hi || last);
    float *red = reinterpret_cast<float *>(s_tile[wave]);
    wave_lds_fence();
#pragma unroll
    for (int d = 0; d < D / 16; ++d)
        *reinterpret_cast<f32x4 *>(red + mrow * kMultiPitch + 16 * d + 4 * kg) = acc[d];
    if (kg == 0) {
        s_m[wave][mrow] = has ? m_run : -INFINITY;
        s_l[wave][mrow] = has ? l_row : 0.f;
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
            o = fmaf(sc, reinterpret_cast<const float *>(s_tile[w])[m * kMultiPitch + d], o);
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
    // Split 1: the append (append_multi_kernel's rules, for this KV head)
    // is done here -- no other workgroup reads this pair's rows, and every
    // wave's cache loads were consumed before the barrier above.  A thread
    // per 16-byte chunk of K or V takes the tokens in order, so the
    // evicted-entry copy reads its slot before the slot is rewritten.
    if (S == 1 && p0 >= 0) {
        const int W = p.window;
        for (int u = tid; u < 2 * (D / 8); u += WAVES * 64) {
            const bool is_v = u >= D / 8;
            const int d = (u % (D / 8)) * 8;
            uint16_t *blk = (is_v ? p.v : p.k) + bh * cap * D;
            for (int t = 0; t < T; ++t) {
                const AppendSlot a = append_slot(p, p0, t);
                const uint16_t *src = (is_v ? p.v_new : p.k_rot) + (((int64_t)b * T + t) * Hkv + kvh) * D + d;
                if (a.evict_old) stm(blk + (int64_t)(W - 1) * D + d, ldm(blk + a.row * D + d));
                if (a.evict_new) stm(blk + (int64_t)(W - 1) * D + d, ldm(src));
                if (a.write) stm(blk + a.row * D + d, ldm(src));
            }
        }
    }
}

// The split partials of one (sequence, KV head, query row): out = sum_s
// e^(lse_s - lse) o_s with lse = ln sum_s e^(lse_s) (parts without keys
// weigh 0), then the sink and the gate.  One wave per row, four dims a
// lane, four rows a workgroup.  A batch of kMergeParts parts has all its
// loads in flight at once (indices past the last part repeat it and weigh
// 0); more parts than one batch fold in batch by batch with the running
// maximum rescaled, as an online softmax does.  Workgroups from
// merge_blocks on write the append instead (one per chunk token, as
// append_multi_kernel does): nothing in this launch reads the cache, and
// the attention kernels that read it have completed before it starts.
constexpr int kMergeParts = 8;
constexpr int kMergeRows = 4;  // rows (waves) per workgroup
__global__ __launch_bounds__(64 * kMergeRows) void multi_merge_kernel(MultiParams p, int RG, int G, int merge_blocks) {
    constexpr int D = kHeadDim;
    static_assert(D == 4 * 64, "a lane's four dims cover the row");
    if ((int)blockIdx.x >= merge_blocks) {
        append_token(p, (int)blockIdx.x - merge_blocks, threadIdx.x, 64 * kMergeRows);
        return;
    }
    const int S = p.split, Hkv = p.num_kv_heads, Hq = p.num_q_heads;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kMergeRows + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nrows = (int64_t)p.batch * Hkv * RG;
    if (row >= nrows) return;
    const int64_t pair = row / RG;
    const int m = (int)(row % RG);
    const int b = (int)(pair / Hkv), kvh = (int)(pair % Hkv);
    const int t = m / G, hq = kvh * G + m % G;
    const int64_t orow = ((int64_t)b * p.tokens + t) * Hq + hq;
    float M = -INFINITY, L = 0.f;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += kMergeParts) {
        float lv[kMergeParts];
        float4 ov[kMergeParts];
#pragma unroll
        for (int k = 0; k < kMergeParts; ++k) {
            const int64_t prow = (pair * S + min(s0 + k, S - 1)) * RG + m;
            lv[k] = p.part_lse[prow];
            ov[k] = *reinterpret_cast<const float4 *>(p.part_o + prow * D + 4 * lane);
        }
        float mb = -INFINITY;
#pragma unroll
        for (int k = 0; k < kMergeParts; ++k)
            if (s0 + k < S) mb = fmaxf(mb, lv[k]);
        const float Mn = fmaxf(M, mb);
        if (Mn == -INFINITY) continue;  // no part with keys yet
        const float sc = M == -INFINITY ? 0.f : expf(M - Mn);
        L *= sc;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] *= sc;
#pragma unroll
        for (int k = 0; k < kMergeParts; ++k) {
            const float w = s0 + k < S ? expf(lv[k] - Mn) : 0.f;  // a part without keys: 0
            L += w;
            o[0] = fmaf(w, ov[k].x, o[0]);
            o[1] = fmaf(w, ov[k].y, o[1]);
            o[2] = fmaf(w, ov[k].z, o[2]);
            o[3] = fmaf(w, ov[k].w, o[3]);
        }
        M = Mn;
    }
    uint2 *dst = reinterpret_cast<uint2 *>(p.out + orow * D + 4 * lane);
    if (M == -INFINITY) {
        *dst = make_uint2(0u, 0u);
        if (lane == 0 && p.lse) p.lse[orow] = -INFINITY;
        return;
    }
    const float lse = M + logf(L);
    float f = 1.f / L;
    if (p.sinks) f *= 1.f / (1.f + expf(p.sinks[hq] - lse));
    if (p.gate) f *= gate_factor(p.gate[orow]);
    *dst = make_uint2(pack_bf16x2(o[0] * f, o[1] * f), pack_bf16x2(o[2] * f, o[3] * f));
    if (lane == 0 && p.lse) p.lse[orow] = lse;
}

// ---------------------------------------------------------------------
// Chunks of more query rows than one MFMA operand holds (tokens x G > 16):
// prefill_chunk_kernel.  One workgroup of kPfWaves waves per (sequence, KV
// head, block of kPfRows query rows); wave w owns rows 16w .. 16w+15 of its
// block (row m = t*G + h: token t, head h), so the waves never merge.  The
// keys -- the cache as it was before the chunk, then the chunk's own rows
// up to the block's last token -- pass through LDS in tiles of 32 that all
// waves of the workgroup score.  A tile is two 16-row halves of K then V,
// each in one-KiB blocks: block j of a half holds, at byte 16 l, lane
// l = r' + 16 c's 16 bytes (row r = r' ^ 12 (c & 1), dims 32j + 8c .. +7).  The rows go
// straight from memory into LDS (global_load_lds_dwordx4), each of the 8
// waves issuing 4 of a tile's 32 blocks; four tile buffers rotate, so three
// tiles are in flight while one is scored, and two waves share a SIMD.
// Per tile and wave:
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: block j of a K half is k-step
//     j's A operand as it lies, the wave's 16 rotated query rows are B (in
//     registers);
//   * an online softmax per query row (8 keys of one row per lane);
//   * O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 with 32 key slots (slot
//     8c + i: key 4c + i of the first half, 8c + 4 + i the same key of the
//     second), V^T's operand two transposing reads (ds_read_b64_tr_b16).
// Masks: a cached key is dropped for token t as in decode_multi_kernel
// (sliding: the ring slots tokens 0..t-1 replace); chunk key x is seen by
// token t iff x <= t (tokens <= 512, so the window never excludes one).
// Rows no query may read (past the cache's live rows or the chunk) are
// loaded from a zero row.  With p.split = S > 1 (small batches) the key
// tiles are cut into S ranges, one workgroup each, and each writes a
// normalised partial (o, lse) per row that multi_merge_kernel combines.
constexpr int kPfWaves = 8;
constexpr int kPfRows = 16 * kPfWaves;       // query rows per workgroup
constexpr int kPfTile = kPrefillTile;        // keys per LDS tile
static_assert(kPfRows == kPrefillRows, "the host plans with the same row blocks");
constexpr int kPfHalf = 16 * kHeadDim * 2;   // bytes of one 16-row half of K (or V)
constexpr int kPfKSteps = kHeadDim / 32;     // 8 blocks per half
constexpr int kPfBlocks = 4 * kPfKSteps;     // K a, K b, V a, V b
constexpr int kPfBlocksPerWave = kPfBlocks / kPfWaves;
constexpr int kPfBufs = 4;
constexpr int kPfAhead = 4;                  // K operand reads in flight
constexpr int kPfTrAhead = 6;                // V^T read pairs in flight
static_assert(kPfBlocksPerWave * kPfWaves == kPfBlocks && kPfBlocksPerWave < 16, "blocks split evenly");
static_assert(kHeadDim <= 576, "the zero row covers a row");

template <int G>
__global__ __launch_bounds__(kPfWaves * 64, 1) void prefill_chunk_kernel(MultiParams p, int nrb) {
    constexpr int D = kHeadDim;
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    __shared__ __align__(1024) unsigned char s_buf[kPfBufs][4 * kPfHalf];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int mrow = lane & 15, kg = lane >> 4;
    // the row whose 16 bytes land in this lane's slot of a block (odd
    // 16-byte columns swizzled, xor 12, for the transposing reads' banks)
    const int drow = mrow ^ (12 * (kg & 1));
    const int Hkv = p.num_kv_heads, Hq = p.num_q_heads, T = p.tokens;
    const int RG = T * G;
    // block ids: the row blocks of a pair are congruent mod 8 (one XCD, so
    // they meet the pair's keys in its L2)
    const int x = blockIdx.x, S = p.split;
    const int rb = (x >> 3) % nrb, rest = (x >> 3) / nrb;
    const int sp = rest % S, pair = (rest / S) * 8 + (x & 7);
    if (pair >= p.batch * Hkv) return;
    const int b = pair / Hkv, kvh = pair % Hkv;
    const int32_t p0 = p.pos[b];
    const int row0 = rb * kPfRows + 16 * wave;     // this wave's first query row
    const int my_row = row0 + mrow;                 // this lane's row (S^T column)
    const int t_row = min(my_row, RG - 1) / G;      // its token
    const int t_hi = min(RG - 1, rb * kPfRows + kPfRows - 1) / G;  // the block's last token

    // the wave's 16 rows: out and lse of row m at ((b, t), kvh * G + h)
    auto out_row = [&](int m) HDA_INLINE { return ((int64_t)b * T + m / G) * Hq + kvh * G + m % G; };
    auto part_row = [&](int m) HDA_INLINE { return ((int64_t)pair * S + sp) * RG + m; };
    if (p0 < 0) {  // no tokens: out 0, lse -inf (split: an empty partial)
        for (int i = lane; i < 16 * D / 8; i += 64) {
            const int m = row0 + i / (D / 8);
            if (m >= RG) continue;
            if (S == 1)
                *reinterpret_cast<uint4 *>(p.out + out_row(m) * D + 8 * (i % (D / 8))) = make_uint4(0, 0, 0, 0);
            else
                *reinterpret_cast<float4 *>(p.part_o + part_row(m) * D + 8 * (i % (D / 8))) =
                    *reinterpret_cast<float4 *>(p.part_o + part_row(m) * D + 8 * (i % (D / 8)) + 4) =
                        make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (lane < 16 && my_row < RG) {
            if (S > 1) p.part_lse[part_row(my_row)] = -INFINITY;
            else if (p.lse) p.lse[out_row(my_row)] = -INFINITY;
        }
        return;
    }
    const int64_t cap = p.capacity;
    const int W1 = p.window - 1;
    const int n_old = p0 == 0 ? 0 : p.sliding ? min(p0, W1) : (int)min((int64_t)p0, cap);
    const int n_ct = (n_old + kPfTile - 1) / kPfTile;         // cache tiles
    const int n_tiles = n_ct + t_hi / kPfTile + 1;            // + chunk tiles up to t_hi
    const int i0 = sp * n_tiles / S, i1 = (sp + 1) * n_tiles / S;  // this workgroup's tiles
    const int64_t bh = (int64_t)b * Hkv + kvh;
    const uint16_t *kblk = p.k + bh * cap * D, *vblk = p.v + bh * cap * D;

    // Row r of half h of tile i for this lane: K and V sources (the zero
    // row for a row no query reads).  Cache tiles keep their last rows
    // inside the block (r0 = min(32 i, cap - 32)).
    auto rows_of = [&](int i, int h, const uint16_t *&ks, const uint16_t *&vs) HDA_INLINE {
        ks = vs = g_zero_row;
        if (i < n_ct) {
            const int64_t r0 = min((int64_t)kPfTile * i, cap - kPfTile);
            const int64_t r = r0 + 16 * h + drow;
            if (r >= (int64_t)kPfTile * i && r < n_old) {
                ks = kblk + r * D;
                vs = vblk + r * D;
            }
        } else if (i < n_tiles) {  // chunk rows: rotated K from the workspace, V from v_new
            const int tok = kPfTile * (i - n_ct) + 16 * h + drow;
            if (tok < T) {
                const int64_t nr = (((int64_t)b * T + tok) * Hkv + kvh) * D;
                ks = p.k_rot + nr;
                vs = p.v_new + nr;
            }
        }
    };
    // This wave's blocks of tile i (blocks wave, wave + 4, ...: K of half
    // 0, K of half 1, V of half 0, V of half 1); past the last tile every
    // lane reads the zero row, so that each tile leaves the same number of
    // loads behind it.
    auto issue = [&](int i, unsigned char *buf) HDA_INLINE {
        const uint16_t *k0, *v0, *k1, *v1;
        if (i >= i1) i = n_tiles;  // past this workgroup's tiles: zero rows
        rows_of(i, 0, k0, v0);
        rows_of(i, 1, k1, v1);
#pragma unroll
        for (int m = 0; m < kPfBlocksPerWave; ++m) {
            const int blk = wave + kPfWaves * m;  // 0..31, wave-uniform
            const int sec = blk / kPfKSteps, j = blk % kPfKSteps;  // K a, K b, V a, V b
            const uint16_t *row = sec == 0 ? k0 : sec == 1 ? k1 : sec == 2 ? v0 : v1;
            load_to_lds(row + 32 * j + 8 * kg, buf + 1024 * blk);
        }
    };

    // B operand: lane (row mrow, kg) holds q[row][32j + 8kg .. +7] (rotated in place)
    uint4 qb[kPfKSteps];
    {
        const uint16_t *qr = p.q + out_row(min(my_row, RG - 1)) * D + 8 * kg;
#pragma unroll
        for (int j = 0; j < kPfKSteps; ++j) qb[j] = ld16(qr + 32 * j);
    }
    issue(i0, s_buf[0]);
    issue(i0 + 1, s_buf[1]);
    issue(i0 + 2, s_buf[2]);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): q and tiles 0..2 in
    __syncthreads();

    f32x4 acc[D / 16];
#pragma unroll
    for (int d = 0; d < D / 16; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_lane = 0.f;  // row mrow; l over this lane's keys
    // V^T transposing read of dim tile d in a half: row 4c + a, dims
    // 16d + 8b + 4e .. +3 for mrow = 4a + 2b + e, at 512 d + this offset
    // (the row's slot swizzled as the loads place it)
    const int tr_b = (mrow >> 1) & 1;
    const int tr_off = 256 * tr_b + 16 * ((4 * kg + (mrow >> 2)) ^ (12 * tr_b)) + 8 * (mrow & 1);

    auto compute = [&](int i, const unsigned char *buf) HDA_INLINE {
        // key 4kg + e of each half: its validity for this lane's row
        bool ok[8];
        const int64_t r0 = min((int64_t)kPfTile * i, cap - kPfTile);
        int dbase = 0;  // (r0 - p0) mod (window - 1): the tile's first slot's distance
        if (i < n_ct && p.sliding) {
            dbase = (int)((r0 - p0) % W1);
            dbase += dbase < 0 ? W1 : 0;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = 16 * h + 4 * kg + e;
                bool v;
                if (i < n_ct) {
                    const int slot = (int)(r0 + k);
                    v = slot >= kPfTile * i && slot < n_old;
                    if (p.sliding) {
                        int dk = dbase + k;
                        if (W1 >= kPfTile) dk -= dk >= W1 ? W1 : 0;  // one wrap at most
                        else dk %= W1;                              // a window under a tile
                        v = v && dk >= t_row;
                    }
                } else {
                    const int xk = kPfTile * (i - n_ct) + k;  // chunk token
                    v = xk <= t_row && xk < T;
                }
                ok[4 * h + e] = v;
            }
        // scores: lane (row mrow, kg) gets keys 4kg + e of each half
        f32x4 sa0 = {0.f, 0.f, 0.f, 0.f}, sa1 = sa0, sb0 = sa0, sb1 = sa0;
        uint4 ka[kPfAhead], kb[kPfAhead];
        auto k_read = [&](int j) HDA_INLINE {
            ka[j % kPfAhead] = ld16(buf + 1024 * j + 16 * (drow + 16 * kg));
            kb[j % kPfAhead] = ld16(buf + kPfHalf + 1024 * j + 16 * (drow + 16 * kg));
        };
#pragma unroll
        for (int j = 0; j < kPfAhead; ++j) k_read(j);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kPfKSteps; ++j) {
            const bf16x8 a = as_bf16x8(ka[j % kPfAhead]), bb = as_bf16x8(kb[j % kPfAhead]);
            if (j + kPfAhead < kPfKSteps) k_read(j + kPfAhead);
            __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead
            const bf16x8 qj = as_bf16x8(qb[j]);
            if (j & 1) {
                sa1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qj, sa1, 0, 0, 0);
                sb1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bb, qj, sb1, 0, 0, 0);
            } else {
                sa0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qj, sa0, 0, 0, 0);
                sb0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bb, qj, sb0, 0, 0, 0);
            }
        }
        float s[8], tmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s[e] = ok[e] ? (sa0[e] + sa1[e]) * p.scale_log2 : -INFINITY;
            s[4 + e] = ok[4 + e] ? (sb0[e] + sb1[e]) * p.scale_log2 : -INFINITY;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) tmax = fmaxf(tmax, s[e]);
        tmax = xor32_max(xor16_max(tmax));
        const float m_new = fmaxf(m_run, tmax);
        const float mr = m_new == -INFINITY ? 0.f : m_new;  // no key for this row yet
        const float alpha = __builtin_amdgcn_exp2f(m_run - mr);  // -inf - x: 0
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int d = 0; d < D / 16; ++d) acc[d] *= alpha;
        }
        float pw[8], ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pw[e] = __builtin_amdgcn_exp2f(s[e] - mr);
            ps += pw[e];
        }
        l_lane = fmaf(l_lane, alpha, ps);
        m_run = m_new;
        const bf16x8 pb = as_bf16x8(make_uint4(pack_bf16x2(pw[0], pw[1]), pack_bf16x2(pw[2], pw[3]),
                                               pack_bf16x2(pw[4], pw[5]), pack_bf16x2(pw[6], pw[7])));
        // V^T reads run kPfTrAhead dim tiles ahead of the products that use them
        const unsigned char *vt = buf + 2 * kPfHalf;
        v4i16 vlo[kPfTrAhead], vhi[kPfTrAhead];
        auto tr_read = [&](int d) HDA_INLINE {
            vlo[d % kPfTrAhead] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vt + tr_off + 512 * d));
            vhi[d % kPfTrAhead] =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vt + kPfHalf + tr_off + 512 * d));
        };
#pragma unroll
        for (int d = 0; d < kPfTrAhead; ++d) tr_read(d);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < D / 16; ++d) {
            const v4i16 lo = vlo[d % kPfTrAhead], hi = vhi[d % kPfTrAhead];
            if (d + kPfTrAhead < D / 16) tr_read(d + kPfTrAhead);
            __builtin_amdgcn_sched_barrier(0);
            uint4 vu;
            vu.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
            vu.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
            vu.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
            vu.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
            acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vu), pb, acc[d], 0, 0, 0);
        }
    };

    // One tile: wait for this wave's blocks of tile i (tiles i + 1 and i + 2
    // may still be in flight), meet the other waves (their blocks are in,
    // and all are done with tile i - 1's buffer), refill that buffer with
    // tile i + 3, score tile i.
    auto step = [&](int i, const unsigned char *cur, unsigned char *refill) HDA_INLINE {  // i from i0
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kPfBlocksPerWave));  // tiles i + 1, i + 2 may be out
        raw_barrier();
        issue(i + 3, refill);
        compute(i, cur);
    };
    static_assert(2 * kPfBlocksPerWave < 64, "vmcnt counts to 63");
    // (the tile loads are asm the compiler does not see, so a loop over
    // computed buffers keeps its waits exact)
    for (int k = 0; k < i1 - i0; ++k) step(i0 + k, s_buf[k % kPfBufs], s_buf[(k + kPfBufs - 1) % kPfBufs]);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the loads past the end have landed

    // out / lse of this lane's row: dims 16d + 4kg .. +3 of every tile d
    const float l = xor32_sum(xor16_sum(l_lane));
    if (my_row >= RG) return;
    if (S > 1) {  // this range's normalised partial and its lse (none: 0 and -inf)
        const int64_t prow = part_row(my_row);
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int d = 0; d < D / 16; ++d)
            *reinterpret_cast<float4 *>(p.part_o + prow * D + 16 * d + 4 * kg) =
                make_float4(acc[d][0] * inv, acc[d][1] * inv, acc[d][2] * inv, acc[d][3] * inv);
        if (kg == 0) p.part_lse[prow] = l > 0.f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
        return;
    }
    const int64_t orow = out_row(my_row);
    const int hq = kvh * G + my_row % G;
    const float lse = (m_run + log2f(l)) * kLn2;  // every row sees its own token's key
    float f = 1.f / l;
    if (p.sinks) f *= 1.f / (1.f + expf(p.sinks[hq] - lse));
    if (p.gate) f *= gate_factor(p.gate[orow]);
#pragma unroll
    for (int d = 0; d < D / 16; ++d)
        *reinterpret_cast<uint2 *>(p.out + orow * D + 16 * d + 4 * kg) =
            make_uint2(pack_bf16x2(acc[d][0] * f, acc[d][1] * f), pack_bf16x2(acc[d][2] * f, acc[d][3] * f));
    if (kg == 0 && p.lse) p.lse[orow] = lse;
}

template <int G>
hipError_t launch_prefill_g(const MultiParams &p, hipStream_t s) {
    const int nrb = (p.tokens * G + kPfRows - 1) / kPfRows;
    const int64_t pairs = (int64_t)p.batch * p.num_kv_heads;
    const int64_t blocks = (pairs + 7) / 8 * 8 * nrb * p.split;
    hipLaunchKernelGGL((prefill_chunk_kernel<G>), dim3((unsigned)blocks), dim3(kPfWaves * 64), 0, s, p, nrb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.split == 1) return e;
    const int mb = (int)((pairs * G * p.tokens + kMergeRows - 1) / kMergeRows);
    hipLaunchKernelGGL(multi_merge_kernel, dim3((unsigned)(mb + p.batch * p.tokens)), dim3(64 * kMergeRows), 0, s,
                       p, G * p.tokens, G, mb);
    return hipGetLastError();
}

template <int G, int T>
hipError_t launch_multi_gt(const MultiParams &p, hipStream_t s) {
    hipLaunchKernelGGL((decode_multi_kernel<G, T>), dim3(p.batch * p.num_kv_heads * p.split),
                       dim3(kMultiWaves * 64), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.split == 1) return e;
    const int mb = (p.batch * p.num_kv_heads * G * T + kMergeRows - 1) / kMergeRows;
    hipLaunchKernelGGL(multi_merge_kernel, dim3((unsigned)(mb + p.batch * T)), dim3(64 * kMergeRows), 0, s, p,
                       G * T, G, mb);
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
    if (p.tokens * group > 16) {
        switch (group) {
            case 1: e = launch_prefill_g<1>(p, stream); break;
            case 2: e = launch_prefill_g<2>(p, stream); break;
            case 4: e = launch_prefill_g<4>(p, stream); break;
            case 8: e = launch_prefill_g<8>(p, stream); break;
            case 16: e = launch_prefill_g<16>(p, stream); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (group) {
            case 1: e = launch_multi_g<1>(p, stream); break;
            case 2: e = launch_multi_g<2>(p, stream); break;
            case 4: e = launch_multi_g<4>(p, stream); break;
            case 8: e = launch_multi_g<8>(p, stream); break;
            case 16: e = launch_multi_g<16>(p, stream); break;
            default: return hipErrorInvalidValue;
        }
    }
    if (e != hipSuccess) return e;
    // the append: done by the merge launch (split > 1) or, for chunk decode
    // unsplit, by the attention kernel; the unsplit prefill needs its own
    if (p.split > 1 || p.tokens * group <= 16) return hipSuccess;
    hipLaunchKernelGGL(append_multi_kernel, dim3(bt), dim3(128), 0, stream, p);
    return hipGetLastError();
}

}  // namespace hda
