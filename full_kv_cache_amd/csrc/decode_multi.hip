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
//      decode_multi_kernel: attention over the cache as it was before the
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
//      (full: rows pos + t; sliding: the ring slots of the last 511 tokens,
//      and the block's evicted-entry row receives the entry of position
//      pos + T - 512 -- a cached one or, for T = 512, token 0 -- as T
//      single-token appends leave it).  It runs after the attention, which
//      reads the slots it overwrites.
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

// Block (b, token t): the token's rotated K and its V into the cache.
// Sliding: only the last window-1 tokens land (an earlier token's slot is
// taken again by a later one); the evicted-entry row ends holding position
// pos + T - window (the entry a single-token step at pos + T - 1 moves
// there): written by the last token's block from its slot before that
// block overwrites it, or, when that position is in the chunk (T ==
// window), by that token's block from the chunk.
__global__ __launch_bounds__(128) void append_multi_kernel(MultiParams p) {
    constexpr int D = kHeadDim;
    const int bt = blockIdx.x, b = bt / p.tokens, t = bt % p.tokens;
    const int32_t p0 = p.pos[b];
    if (p0 < 0) return;
    const int64_t P = (int64_t)p0 + t, cap = p.capacity;
    int64_t row;
    bool evict_old = false, evict_new = false, write = true;
    if (p.sliding) {
        const int slots = p.window - 1;
        const int64_t last = (int64_t)p0 + p.tokens - 1;  // the chunk's last position
        row = P % slots;
        write = t >= p.tokens - slots;
        if (last >= slots) {
            const int64_t e = last - slots;  // position the evicted-entry row ends holding
            evict_old = t == p.tokens - 1 && e < p0;
            evict_new = e >= p0 && P == e;
        }
    } else {
        if (P >= cap) return;
        row = P;
    }
    const int Hkv = p.num_kv_heads;
    for (int u = threadIdx.x; u < 2 * Hkv * (D / 8); u += 128) {
        const bool is_v = u >= Hkv * (D / 8);
        const int w = is_v ? u - Hkv * (D / 8) : u, h = w / (D / 8), d = (w % (D / 8)) * 8;
        uint16_t *blk = (is_v ? p.v : p.k) + ((int64_t)b * Hkv + h) * cap * D;
        const uint16_t *src = (is_v ? p.v_new : p.k_rot) + ((int64_t)bt * Hkv + h) * D;
        if (evict_old) stm(blk + (int64_t)(p.window - 1) * D + d, ldm(blk + row * D + d));
        if (evict_new) stm(blk + (int64_t)(p.window - 1) * D + d, ldm(src + d));
        if (write) stm(blk + row * D + d, ldm(src + d));
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
                kA[j] = ld16(p.k_rot + row);
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

// ---------------------------------------------------------------------
// Chunks of more query rows than one MFMA operand holds (tokens x G > 16):
// prefill_chunk_kernel.  One workgroup of kPfWaves waves per (sequence, KV
// head, block of kPfRows query rows); wave w owns rows 16w .. 16w+15 of its
// block (row m = t*G + h: token t, head h), so the waves never merge.  The
// keys -- the cache as it was before the chunk, then the chunk's own rows
// up to the block's last token -- pass through LDS in tiles of 32 that all
// waves of the workgroup score, the next tile's loads in flight while one
// is scored.  Per 16-key half of a tile, as the sparse kernel:
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (the keys' rows from LDS as
//     the A operand, the wave's 16 rotated query rows as B, in registers);
//   * an online softmax per query row (4 keys of one row per lane);
//   * O^T += V^T P^T on v_mfma_f32_16x16x16_bf16, the S^T accumulator
//     already P^T's operand layout, V^T through ds_read_b64_tr_b16.
// Masks: a cached key is dropped for token t as in decode_multi_kernel
// (sliding: the ring slots tokens 0..t-1 replace); chunk key x is seen by
// token t iff x <= t (tokens <= 512, so the window never excludes one).
constexpr int kPfWaves = 4;
constexpr int kPfRows = 16 * kPfWaves;        // query rows per workgroup
constexpr int kPfTile = 32;                   // keys per LDS tile
constexpr int kPfPitch = kHeadDim + 8;        // LDS row pitch (bf16)
constexpr int kPfStage = 2 * kPfTile * kPfPitch;  // K then V rows of one tile
constexpr int kPfLoads = 2 * kPfTile * (kHeadDim / 8) / (kPfWaves * 64);  // 16-byte loads a thread
static_assert(kPfLoads * kPfWaves * 64 == 2 * kPfTile * (kHeadDim / 8), "tile loads divide evenly");

template <int G>
__global__ __launch_bounds__(kPfWaves * 64, 2) void prefill_chunk_kernel(MultiParams p, int nrb) {
    constexpr int D = kHeadDim;
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    __shared__ __align__(16) uint16_t s_tile[2][kPfStage];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int mrow = lane & 15, kg = lane >> 4;
    const int Hkv = p.num_kv_heads, Hq = p.num_q_heads, T = p.tokens;
    const int RG = T * G;
    // block ids: the row blocks of a pair are congruent mod 8 (one XCD, so
    // they meet the pair's keys in its L2)
    const int x = blockIdx.x;
    const int rb = (x >> 3) % nrb, pair = ((x >> 3) / nrb) * 8 + (x & 7);
    if (pair >= p.batch * Hkv) return;
    const int b = pair / Hkv, kvh = pair % Hkv;
    const int32_t p0 = p.pos[b];
    const int row0 = rb * kPfRows + 16 * wave;     // this wave's first query row
    const int my_row = row0 + mrow;                 // this lane's row (S^T column)
    const int t_row = min(my_row, RG - 1) / G;      // its token
    const int t_hi = min(RG - 1, rb * kPfRows + kPfRows - 1) / G;  // the block's last token

    // the wave's 16 rows: out and lse of row m at ((b, t), kvh * G + h)
    auto out_row = [&](int m) HDA_INLINE { return ((int64_t)b * T + m / G) * Hq + kvh * G + m % G; };
    if (p0 < 0) {  // no tokens: out 0, lse -inf
        for (int i = lane; i < 16 * D / 8; i += 64) {
            const int m = row0 + i / (D / 8);
            if (m < RG) *reinterpret_cast<uint4 *>(p.out + out_row(m) * D + 8 * (i % (D / 8))) = make_uint4(0, 0, 0, 0);
        }
        if (lane < 16 && my_row < RG && p.lse) p.lse[out_row(my_row)] = -INFINITY;
        return;
    }
    const int64_t cap = p.capacity;
    const int W1 = p.window - 1;
    const int n_old = p0 == 0 ? 0 : p.sliding ? min(p0, W1) : (int)min((int64_t)p0, cap);
    const int n_ct = (n_old + kPfTile - 1) / kPfTile;         // cache tiles
    const int n_tiles = n_ct + t_hi / kPfTile + 1;            // + chunk tiles up to t_hi
    const int64_t bh = (int64_t)b * Hkv + kvh;
    const uint16_t *kblk = p.k + bh * cap * D, *vblk = p.v + bh * cap * D;

    // Tile i's 16-byte loads for this thread: chunk c = tid + 256 u covers
    // row (c / 32) % 32 of K (c < 1024) or V, dims 8 (c % 32) .. +7.
    auto load = [&](int i, uint4 *r) HDA_INLINE {
#pragma unroll
        for (int u = 0; u < kPfLoads; ++u) {
            const int c = tid + kPfWaves * 64 * u;
            const bool isv = c >= kPfTile * (D / 8);
            const int row = (c / (D / 8)) % kPfTile, d8 = 8 * (c % (D / 8));
            const uint16_t *src;
            bool keep = true;
            if (i < n_ct) {  // cache rows, the last tile kept inside the block
                const int64_t r0 = min((int64_t)kPfTile * i, cap - kPfTile);
                src = (isv ? vblk : kblk) + (r0 + row) * D + d8;
                // a row no query may read (unwritten, or the previous tile's)
                // goes in as 0: a zero weight would not cancel a NaN there
                keep = r0 + row >= (int64_t)kPfTile * i && r0 + row < n_old;
            } else {          // chunk rows: rotated K from the workspace, V from v_new
                const int tok = min(kPfTile * (i - n_ct) + row, T - 1);
                const int64_t nr = (((int64_t)b * T + tok) * Hkv + kvh) * D + d8;
                src = (isv ? p.v_new : p.k_rot) + nr;
            }
            const uint4 v = ld16(src);
            r[u] = keep ? v : make_uint4(0, 0, 0, 0);
        }
    };
    auto store = [&](int stage, const uint4 *r) HDA_INLINE {
#pragma unroll
        for (int u = 0; u < kPfLoads; ++u) {
            const int c = tid + kPfWaves * 64 * u;
            const int kv = c / (kPfTile * (D / 8)), row = (c / (D / 8)) % kPfTile, d8 = 8 * (c % (D / 8));
            *reinterpret_cast<uint4 *>(&s_tile[stage][(kv * kPfTile + row) * kPfPitch + d8]) = r[u];
        }
    };

    // B operand: lane (row mrow, kg) holds q[row][32j + 8kg .. +7] (rotated in place)
    bf16x8 qb[8];
    {
        const uint16_t *qr = p.q + out_row(min(my_row, RG - 1)) * D + 8 * kg;
#pragma unroll
        for (int j = 0; j < 8; ++j) qb[j] = as_bf16x8(ld16(qr + 32 * j));
    }
    f32x4 acc[D / 16];
#pragma unroll
    for (int d = 0; d < D / 16; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_lane = 0.f;  // row mrow; l over this lane's keys

    uint4 regs[kPfLoads];
    load(0, regs);
    store(0, regs);
    __syncthreads();
    for (int i = 0; i < n_tiles; ++i) {
        const int stage = i & 1;
        if (i + 1 < n_tiles) load(i + 1, regs);
        const uint16_t *kt = &s_tile[stage][0], *vt = &s_tile[stage][kPfTile * kPfPitch];
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
            // key k = 4kg + e of this half: its validity for this lane's row
            bool ok[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int kk = kPfTile * i + 16 * hlf + 4 * kg + e;  // key index over the sequence's key list
                if (i < n_ct) {
                    const int64_t r0 = min((int64_t)kPfTile * i, cap - kPfTile);
                    const int slot = (int)(r0 + 16 * hlf + 4 * kg + e);
                    bool v = slot >= kPfTile * i && slot < n_old;
                    if (p.sliding) {
                        int dk = (slot - p0) % W1;
                        dk = dk < 0 ? dk + W1 : dk;
                        v = v && dk >= t_row;
                    }
                    ok[e] = v;
                } else {
                    const int xk = kk - kPfTile * n_ct;  // chunk token
                    ok[e] = xk <= t_row && xk < T;
                }
            }
            f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint4 ka = *reinterpret_cast<const uint4 *>(kt + (16 * hlf + mrow) * kPfPitch + 32 * j + 8 * kg);
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka), qb[j], sc, 0, 0, 0);
            }
            float s[4], tmax = -INFINITY;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s[e] = ok[e] ? sc[e] * p.scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, s[e]);
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float m_new = fmaxf(m_run, tmax);
            const float mr = m_new == -INFINITY ? 0.f : m_new;  // no key for this row yet
            const float alpha = __builtin_amdgcn_exp2f(m_run - mr);  // -inf - x: 0
            if (__ballot(alpha != 1.f)) {
#pragma unroll
                for (int d = 0; d < D / 16; ++d) acc[d] *= alpha;
            }
            float pv[4], ps = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pv[e] = __builtin_amdgcn_exp2f(s[e] - mr);
                ps += pv[e];
            }
            l_lane = fmaf(l_lane, alpha, ps);
            m_run = m_new;
            const v4i16 pb = {(short)f32_to_bf16(pv[0]), (short)f32_to_bf16(pv[1]), (short)f32_to_bf16(pv[2]),
                              (short)f32_to_bf16(pv[3])};
            const uint16_t *trb = vt + (16 * hlf + 4 * kg + (mrow >> 2)) * kPfPitch + 4 * (mrow & 3);
#pragma unroll
            for (int d = 0; d < D / 16; ++d) {
                const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(trb + 16 * d));
                acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, acc[d], 0, 0, 0);
            }
        }
        if (i + 1 < n_tiles) {
            __syncthreads();  // every wave is done with the other stage
            store(stage ^ 1, regs);
            __syncthreads();
        }
    }

    // out / lse of this lane's row: dims 16d + 4kg .. +3 of every tile d
    float l = l_lane + __shfl_xor(l_lane, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (my_row >= RG) return;
    const int64_t orow = out_row(my_row);
    const int hq = kvh * G + my_row % G;
    const float lse = (m_run + log2f(l)) * kLn2;  // every row sees its own token's key
    float f = 1.f / l;
    if (p.sinks) f *= 1.f / (1.f + expf(p.sinks[hq] - lse));
    if (p.gate) f *= gate_factor(p.gate[orow]);
#pragma unroll
    for (int d = 0; d < D / 16; ++d) {
        const uint32_t lo = (uint32_t)f32_to_bf16(acc[d][0] * f) | ((uint32_t)f32_to_bf16(acc[d][1] * f) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(acc[d][2] * f) | ((uint32_t)f32_to_bf16(acc[d][3] * f) << 16);
        *reinterpret_cast<uint2 *>(p.out + orow * D + 16 * d + 4 * kg) = make_uint2(lo, hi);
    }
    if (kg == 0 && p.lse) p.lse[orow] = lse;
}

template <int G>
hipError_t launch_prefill_g(const MultiParams &p, hipStream_t s) {
    const int nrb = (p.tokens * G + kPfRows - 1) / kPfRows;
    const int64_t pairs = (int64_t)p.batch * p.num_kv_heads;
    const int64_t blocks = (pairs + 7) / 8 * 8 * nrb;
    hipLaunchKernelGGL((prefill_chunk_kernel<G>), dim3((unsigned)blocks), dim3(kPfWaves * 64), 0, s, p, nrb);
    return hipGetLastError();
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
    hipLaunchKernelGGL(append_multi_kernel, dim3(bt), dim3(128), 0, stream, p);
    return hipGetLastError();
}

}  // namespace hda
