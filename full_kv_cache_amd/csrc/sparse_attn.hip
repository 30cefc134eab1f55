// sparse_attn.hip -- sparse top-k decode over one shared latent KV head (gfx950).
//
// What is computed (flashmla_sparse page: the `_bf16_flash_mla_kernel` call
// shapes; the `HYV4FlashMLASparseImpl` docstring for the sink):
//   for token t and query head h, over the pool rows named by the first
//   len_t entries of indices[t] (len_t = topk_length[t], else topk; entries
//   outside [0, pool_rows) name no row and are skipped):
//     s_i = scale * q_h . kv[idx_i]                 all Dqk = 576 dims
//     out_h = sum_i softmax(s)_i kv[idx_i][0:Dv]     Dv = 512 leading dims
//     lse_h = ln sum_i exp(s_i);  out_h *= 1 / (1 + exp(sink_h - lse_h)).
// The fp8 form (the same page's `_fp8_flash_mla_kernel`: the cache handed
// over as bytes) reads e4m3 codes with one fp32 scale per pool row: a row's
// value is code x scale, for its key and its value dims alike.
//
// With 64 query heads per shared row the path does about 121 flop per
// gathered byte, so both products run on the matrix cores:
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: 16 gathered rows form the A
//     operand, loaded straight from memory with 16-byte loads (8 dims of a
//     row per lane; fp8: 8 codes, widened to bf16 exactly); the workgroup's
//     16 query heads form the B operand, read from LDS (registers hold the
//     accumulators and the tiles in flight);
//   * O^T += V^T P^T on v_mfma_f32_16x16x16_bf16: the S^T accumulator
//     already holds P^T in operand layout (4 keys of one head per lane), and
//     V^T comes out of LDS through the transposing read ds_read_b64_tr_b16
//     from the rows the wave has just stored there.
// A wave keeps two tiles of rows in flight behind the one it scores: the
// next tile's loads are issued as soon as the current tile's registers are
// stored, before its softmax and P.V.
// The softmax needs no running rescale: probabilities are taken against a
// fixed reference m_ref (log2 units), the maximum of each head's first
// scored tile, so weights 2^(s - m_ref) stay below 2^kSlack as long as no
// later score exceeds m_ref by more than kSlack (bf16 and fp32 hold such
// weights as well as ones below 1; the final normalisation divides by the
// sum taken against the same reference, so the result is the softmax).
// The 128 accumulator registers are then only ever touched by the matrix
// cores (a rescale of them in the loop pushed the compiler into spilling).
// Should a later score exceed the reference by more than that, the wave
// scores its keys again against the exact maximum, which it tracks.
// Work split: one workgroup of 4 waves per (token, key split, group of 16
// heads); the waves take the split's 16-key tiles in turn, each with its own
// online softmax, and merge in LDS at the end.  The head-group workgroups of
// one (token, split) get block ids congruent mod 8, so they run on the same
// XCD and meet the gathered rows in its L2.
#include <type_traits>

#include "hda_device.h"
#include "hda_kernels.h"

namespace hda {

namespace {

constexpr int kKSteps = kSparseDqk / 32;   // 16x16x32 steps over the key dims
constexpr int kVChunks = kSparseDv / 32;   // 16-byte chunks of the value part per lane
constexpr int kDimTiles = kSparseDv / 16;  // 16-dim output tiles
constexpr int kVPitch = kSparseDv + 16;    // LDS row pitch of a V tile (bf16)
constexpr int kOPitch = kSparseDv + 4;     // LDS row pitch of the merge buffer (fp32)
constexpr int kQPitch = kSparseDqk + 8;    // LDS row pitch of the q block (bf16): reads of 16 heads hit 16 bank groups
constexpr int kIdxBatch = 16;              // tiles whose row indices a lane holds at once
constexpr float kSlack = 32.f;             // largest weight 2^32 against the fixed reference
constexpr float kLn2 = 0.693147180559945309f;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ short bf16_bits(float f) { return (short)f32_to_bf16(f); }

// One tile's rows for this lane: row `row` (< 0: masked, row 0 is read and
// the key dropped), dims 32j + 8kg .. +7 for every k-step j; fp8 also the
// row's scale.
template <bool F8>
struct TileRegs {
    std::conditional_t<F8, uint2, uint4> k[kKSteps];
    float rs;
};

template <bool F8>
__device__ __forceinline__ void load_tile(const SparseParams &p, int row, int kg, TileRegs<F8> &t) {
    const int64_t r = row < 0 ? 0 : row;
    if constexpr (F8) {
        const uint8_t *src = p.kv8 + r * kSparseDqk + 8 * kg;
#pragma unroll
        for (int j = 0; j < kKSteps; ++j) t.k[j] = *reinterpret_cast<const uint2 *>(src + 32 * j);
        t.rs = p.kv_scale[r];
    } else {
        const uint16_t *src = p.kv + r * kSparseDqk + 8 * kg;
#pragma unroll
        for (int j = 0; j < kKSteps; ++j) t.k[j] = ld16(src + 32 * j);
        t.rs = 1.f;
    }
}

template <bool F8>
__device__ __forceinline__ bf16x8 operand(const TileRegs<F8> &t, int j) {
    if constexpr (F8)
        return as_bf16x8(e4m3x8_to_bf16x8(t.k[j]));
    else
        return as_bf16x8(t.k[j]);
}

// Pool row of key kk (< k1 names a list entry; k0 <= kk) for this lane, or
// -1 when the key is masked.  Branch-free: the entry is read at a clamped
// position whatever kk is, so that the loads of a batch issue back to back.
__device__ __forceinline__ int row_of(const SparseParams &p, const int32_t *idx, int kk, int k0, int k1) {
    const int r = idx[max(min(kk, k1 - 1), k0)];
    return (kk < k1 && r >= 0 && (int64_t)r < p.pool_rows) ? r : -1;
}


template <bool FINAL, bool F8>
__global__ __launch_bounds__(kSparseWaves * 64, 1) void sparse_decode_kernel(SparseParams p) {
    constexpr int W = kSparseWaves;
    constexpr int kTileBytes = 16 * kVPitch * 2;
    __shared__ __align__(16) unsigned char s_buf[W * kTileBytes];
    __shared__ float s_m[W][16], s_l[W][16];
    __shared__ __align__(16) uint16_t s_q[16 * kQPitch];
    static_assert(16 * kOPitch * 4 <= W * kTileBytes, "merge buffer fits the V tiles");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int mrow = lane & 15, kg = lane >> 4;
    const int Hq = p.num_q_heads, groups = Hq / kSparseHeadsPerWave;
    const int x = blockIdx.x;
    const int g = (x >> 3) % groups;
    const int u = ((x >> 3) / groups) * 8 + (x & 7);
    if (u >= p.tokens * p.nsplit) return;
    const int t = u / p.nsplit, sp = u % p.nsplit;
    int len = p.topk_length ? p.topk_length[t] : p.topk;
    len = len < 0 ? 0 : (len > p.topk ? p.topk : len);
    const int k0 = sp * p.split_keys;
    const int k1 = min(k0 + p.split_keys, len);
    const int ntile = k1 > k0 ? (k1 - k0 + 15) >> 4 : 0;
    const int h0 = g * kSparseHeadsPerWave;
    const int32_t *idx = p.indices + (int64_t)t * p.topk;

    // the workgroup's 16 query rows into LDS, 16 bytes per thread a pass
    {
        const uint16_t *qg = p.q + ((int64_t)t * Hq + h0) * kSparseDqk;
        constexpr int kChunks = 16 * kSparseDqk / 8;
        for (int c = tid; c < kChunks; c += W * 64) {
            const int hr = c / (kSparseDqk / 8), cc = c % (kSparseDqk / 8);
            *reinterpret_cast<uint4 *>(s_q + hr * kQPitch + 8 * cc) = ld16(qg + (int64_t)hr * kSparseDqk + 8 * cc);
        }
    }
    __syncthreads();
    // B operand: lane (head mrow, kg) reads q[t][h0 + mrow][32j + 8kg .. +7]
    const uint16_t *qs = s_q + mrow * kQPitch + 8 * kg;
    f32x4 acc[kDimTiles];
#pragma unroll
    for (int d = 0; d < kDimTiles; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    // head mrow: weights are 2^(s - m_ref); l over this lane's keys; m_max
    // the largest score seen, over in case a score passed m_ref + kSlack
    float m_ref = -INFINITY, l_lane = 0.f, m_max = -INFINITY;
    bool over = false;

    uint16_t *vt = reinterpret_cast<uint16_t *>(s_buf + wave * kTileBytes);
    const uint16_t *trb = vt + (4 * kg + (mrow >> 2)) * kVPitch + 4 * (mrow & 3);

    // One tile: scores, V rows to LDS, then (once `tr`'s registers are
    // free) the loads of the tile two ahead, the softmax and P.V.
    auto process = [&](TileRegs<F8> &tr, int row, int row_next2) HDA_INLINE {
        // scores of the tile: lane (head mrow, kg) gets keys 4kg + i
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kKSteps; ++j)
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(operand<F8>(tr, j),
                                                         *reinterpret_cast<const bf16x8 *>(qs + 32 * j), sc, 0, 0, 0);
        const uint32_t vmask = (uint32_t)__ballot(row >= 0) & 0xFFFFu;
        // value part of the rows into this wave's LDS tile; masked rows as 0
        // (a zero weight would not cancel a NaN they might hold)
        {
            uint16_t *dst = vt + mrow * kVPitch + 8 * kg;
            const bool keep = row >= 0;
#pragma unroll
            for (int j = 0; j < kVChunks; ++j) {
                uint4 v = __builtin_bit_cast(uint4, operand<F8>(tr, j));
                if (vmask != 0xFFFFu && !keep) v = make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4 *>(dst + 32 * j) = v;
            }
        }
        // key 4kg + i's row scale (fp8), from the lane that loaded that row;
        // 1 for a masked key (the row read in its place may hold anything)
        float rsk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rsk[i] = 1.f;
            if constexpr (F8) {
                const float r = __shfl(tr.rs, 4 * kg + i, 64);
                if ((vmask >> (4 * kg + i)) & 1u) rsk[i] = r;
            }
        }
        // the tile two ahead goes in flight in these registers (not before:
        // hoisted above the stores it would need a third tile's registers).
        // Unconditional -- past the last tile it reads row 0 for nothing --
        // so that every tile finds the same loads outstanding behind it and
        // its wait counts stay exact.
        asm volatile("" ::: "memory");
        load_tile<F8>(p, row_next2, kg, tr);

        // softmax against the fixed reference (log2 domain)
        float s[4], tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[i] = ((vmask >> (4 * kg + i)) & 1u) ? sc[i] * (p.scale_log2 * rsk[i]) : -INFINITY;
            tmax = fmaxf(tmax, s[i]);
        }
        tmax = xor32_max(xor16_max(tmax));
        m_max = fmaxf(m_max, tmax);
        if (m_ref == -INFINITY) m_ref = tmax;  // first keys: nothing accumulated yet
        over |= tmax > m_ref + kSlack;
        const float mr = m_ref == -INFINITY ? 0.f : m_ref;  // -inf: this head has no key yet
        float pv[4], ps = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pv[i] = __builtin_amdgcn_exp2f(s[i] - mr);
            ps += pv[i];
        }
        l_lane += ps;
        const v4i16 pb = {bf16_bits(pv[0] * rsk[0]), bf16_bits(pv[1] * rsk[1]), bf16_bits(pv[2] * rsk[2]),
                          bf16_bits(pv[3] * rsk[3])};
        wave_lds_fence();  // the tile's rows are in LDS
#pragma unroll
        for (int d = 0; d < kDimTiles; ++d) {
            const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(trb + 16 * d));
            acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, acc[d], 0, 0, 0);
        }
        // The next tile's stores follow these reads in this wave's LDS
        // queue, which runs in order; keep the compiler from moving them.
        __builtin_amdgcn_wave_barrier();
    };

    // this wave's tiles: wave, wave + W, ...; row indices a batch at a time
    TileRegs<F8> ta, tb;
    for (int pass = 0; pass < 2; ++pass) {
        for (int base = wave; base < ntile; base += W * kIdxBatch) {
            int rows[kIdxBatch];
#pragma unroll
            for (int i = 0; i < kIdxBatch; ++i) rows[i] = row_of(p, idx, k0 + 16 * (base + W * i) + mrow, k0, k1);
            const int nt = min(kIdxBatch, (ntile - base + W - 1) / W);  // this batch's tiles (>= 1)
            // Unrolled over the batch: loads stay in flight from one tile to
            // the next, and the compiler places exact waits only in straight
            // code (across a loop's back edge it waited for every load).
            load_tile<F8>(p, rows[0], kg, ta);
            load_tile<F8>(p, rows[1], kg, tb);
#pragma unroll
            for (int i = 0; i < kIdxBatch; i += 2) {
                if (i >= nt) break;  // an odd count ends on a tile of masked keys
                process(ta, rows[i], i + 2 < kIdxBatch ? rows[i + 2] : -1);
                process(tb, rows[i + 1], i + 3 < kIdxBatch ? rows[i + 3] : -1);
            }
        }
        if (!__ballot(over)) break;
        // a score passed the reference by more than kSlack: start over
        // against the exact maximum (weights <= 1)
#pragma unroll
        for (int d = 0; d < kDimTiles; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
        l_lane = 0.f;
        m_ref = m_max;
        over = false;
    }

    // merge the 4 waves: o = sum_w 2^(m_w - M) o_w, l likewise
    const float l_w = xor32_sum(xor16_sum(l_lane));
    if (kg == 0) {
        s_m[wave][mrow] = m_ref;
        s_l[wave][mrow] = l_w;
    }
    __syncthreads();  // also: every wave is done with its V tile
    float *ob = reinterpret_cast<float *>(s_buf);
    {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w][mrow]);
        const float c = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - M);
#pragma unroll
        for (int w = 0; w < W; ++w) {
            if (wave == w) {
#pragma unroll
                for (int d = 0; d < kDimTiles; ++d) {
                    float4 *o = reinterpret_cast<float4 *>(ob + mrow * kOPitch + 16 * d + 4 * kg);
                    float4 v = make_float4(c * acc[d][0], c * acc[d][1], c * acc[d][2], c * acc[d][3]);
                    if (w > 0) {
                        const float4 a = *o;
                        v.x += a.x; v.y += a.y; v.z += a.z; v.w += a.w;
                    }
                    *o = v;
                }
            }
            __syncthreads();
        }
    }

    // thread -> head n = tid / 16, dims 32 (tid % 16) .. +31
    const int n = tid >> 4, c32 = (tid & 15) * 32;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w][n]);
    float L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float mw = s_m[w][n];
            if (mw != -INFINITY) L += __builtin_amdgcn_exp2f(mw - M) * s_l[w][n];
        }
    }
    const int hq = h0 + n;
    const float lse = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const float *src = ob + n * kOPitch + c32;
    if (FINAL) {
        float f = inv;
        if (p.sinks) f *= 1.f / (1.f + expf(p.sinks[hq] - lse));
        uint16_t *dst = p.out + ((int64_t)t * Hq + hq) * kSparseDv + c32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t w4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = src[8 * q + 2 * e] * f, b = src[8 * q + 2 * e + 1] * f;
                w4[e] = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
            }
            *reinterpret_cast<uint4 *>(dst + 8 * q) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        }
        if ((tid & 15) == 0 && p.lse) p.lse[(int64_t)t * Hq + hq] = lse;
    } else {
        const int64_t slot = ((int64_t)t * Hq + hq) * p.nsplit + sp;
        float *dst = p.part_o + slot * kSparseDv + c32;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            *reinterpret_cast<float4 *>(dst + 4 * q) =
                make_float4(src[4 * q] * inv, src[4 * q + 1] * inv, src[4 * q + 2] * inv, src[4 * q + 3] * inv);
        if ((tid & 15) == 0) p.part_lse[slot] = lse;
    }
}

// ---------------------------------------------------------------------------
// Shared-tile form (bf16 pool, up to 64 query heads): one 4-wave workgroup
// per (token, key split) serves every head -- wave w owns heads 16w..16w+15
// -- so each gathered row crosses from L2 into the CU once, not once per
// head group.  A tile is 32 keys, two 16-row halves of 18 one-KiB blocks;
// block j of a half holds, at byte 16 l, lane l = r' + 16 c's 16 bytes: row
// r = r' ^ 12 (c & 1), dims 32j + 8c .. +7.  The rows go straight from memory into LDS
// (global_load_lds_dwordx4: lane l's 16 bytes land at base + 16 l), each
// wave issuing 9 of the tile's 36 blocks; three tile buffers rotate, so two
// tiles are in flight while one is scored.  Per wave and tile:
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: block j of a half is k-step
//     j's A operand as it lies (one ds_read_b128 at 16 l), q is the B
//     operand, held in registers for the call;
//   * O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 with 32 key slots: slot
//     8c + i is key 4c + i of the first half, slot 8c + 4 + i the same key
//     of the second half -- the S^T accumulators' lane layout -- and V^T's
//     operand is two transposing reads (ds_read_b64_tr_b16), one per half.
// Keys without a row (past the split's end, or an index outside the pool)
// read a zero row and are masked out of the softmax, so a NaN never meets a
// zero weight.  Softmax against a fixed reference as in the kernel above.
// F8 (e4m3 pool, a scale per row): a wave's blocks of a tile are loaded as
// codes into registers (8 per lane and block, with its two rows' scales),
// widened to bf16 (exact) and stored where the bf16 form's loads would put
// them; two tiles in flight in registers, two LDS buffers.  A key's scores
// take its row's scale, and so do the probabilities sent to P.V (the
// running sum keeps the unscaled ones), as the head-group kernel does.

constexpr int kTileKeys = 32;
constexpr int kHalfBytes = 16 * kSparseDqk * 2;  // one 16-row half: 18 blocks of 1 KiB
constexpr int kTileBlocks = 2 * kKSteps;         // 36 blocks per tile
constexpr int kTileWaves = 4;
constexpr int kTrAhead = 6;  // V^T read pairs in flight (lgkmcnt counts up to 15)
constexpr int kKAhead = 4;   // K operand read pairs in flight
constexpr int kBlocksPerWave = kTileBlocks / kTileWaves;
static_assert(kBlocksPerWave * kTileWaves == kTileBlocks, "blocks split evenly over the waves");
static_assert(kTileWaves * kSparseHeadsPerWave == kSparseTileHeads, "a wave per 16 heads");

template <bool FINAL, bool F8>
__global__ __launch_bounds__(kTileWaves * 64, 1) void sparse_tile_kernel(SparseParams p) {
    __shared__ __align__(1024) unsigned char s_b0[2 * kHalfBytes];
    __shared__ __align__(1024) unsigned char s_b1[2 * kHalfBytes];
    __shared__ __align__(1024) unsigned char s_b2[F8 ? 16 : 2 * kHalfBytes];
    __shared__ int s_idx[kSparseMaxSplitKeys];
    __shared__ int s_over[kTileWaves];
    __shared__ float s_tsc[2][F8 ? kTileKeys : 1];  // F8: the row scales of the tile in each buffer

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int mrow = lane & 15, kg = lane >> 4;
    // the row whose 16 bytes land in this lane's slot of a block: rows of the
    // odd 16-byte columns are swizzled (xor 12) so that the transposing reads
    // of a block's two column halves meet different banks
    const int drow = mrow ^ (12 * (kg & 1));
    const int x = blockIdx.x, j8 = x >> 3;
    const int t = (j8 / p.nsplit) * 8 + (x & 7), sp = j8 % p.nsplit;
    if (t >= p.tokens) return;  // the whole workgroup
    int len = p.topk_length ? p.topk_length[t] : p.topk;
    len = len < 0 ? 0 : (len > p.topk ? p.topk : len);
    const int k0 = sp * p.split_keys;
    const int nk = max(min(k0 + p.split_keys, len) - k0, 0);
    const int ntile = (nk + kTileKeys - 1) / kTileKeys;
    const int Hq = p.num_q_heads, h0 = wave * kSparseHeadsPerWave;
    const bool active = h0 < Hq;  // wave-uniform: a wave past the heads only loads

    const int32_t *idx = p.indices + (int64_t)t * p.topk + k0;
    auto row_at = [&](int i) HDA_INLINE {  // pool row of the split's key i, or -1
        int r = -1;
        if (i < nk) {
            r = idx[i];
            if (r < 0 || (int64_t)r >= p.pool_rows) r = -1;
        }
        return r;
    };
    // This wave's blocks of a tile whose halves' rows for this lane are ra
    // and rb (blocks wave, wave + 4, ...; -1 reads the zero row).
    auto issue_rows = [&](int ra, int rb, unsigned char *buf) HDA_INLINE {
        const uint16_t *pa = ra < 0 ? g_zero_row : p.kv + (int64_t)ra * kSparseDqk;
        const uint16_t *pb = rb < 0 ? g_zero_row : p.kv + (int64_t)rb * kSparseDqk;
#pragma unroll
        for (int m = 0; m < kBlocksPerWave; ++m) {
            const int blk = wave + kTileWaves * m;  // 0..35, wave-uniform
            const bool hb = blk >= kKSteps;
            const int j = hb ? blk - kKSteps : blk;
            const uint16_t *src = (hb ? pb : pa) + 32 * j + 8 * kg;
            load_to_lds(src, buf + 1024 * blk);
        }
    };
    // F8: this wave's blocks of a tile whose halves' rows for this lane are
    // ra and rb, as codes (the zero row for -1), and those rows' scales (1
    // for -1); then widened into a buffer where the bf16 form's loads would
    // put them, the scales of the tile's 32 rows beside it.
    struct Codes {
        uint2 c[F8 ? kBlocksPerWave : 1];
        float sa, sb;
    };
    auto load_codes = [&](int ra, int rb, Codes &x) HDA_INLINE {
        if constexpr (F8) {
            const uint8_t *pa = ra < 0 ? reinterpret_cast<const uint8_t *>(g_zero_row) : p.kv8 + (int64_t)ra * kSparseDqk;
            const uint8_t *pb = rb < 0 ? reinterpret_cast<const uint8_t *>(g_zero_row) : p.kv8 + (int64_t)rb * kSparseDqk;
#pragma unroll
            for (int m = 0; m < kBlocksPerWave; ++m) {
                const int blk = wave + kTileWaves * m;
                const bool hb = blk >= kKSteps;
                const int j = hb ? blk - kKSteps : blk;
                x.c[m] = *reinterpret_cast<const uint2 *>((hb ? pb : pa) + 32 * j + 8 * kg);
            }
            const float fa = p.kv_scale[ra < 0 ? 0 : ra], fb = p.kv_scale[rb < 0 ? 0 : rb];
            x.sa = ra < 0 ? 1.f : fa;
            x.sb = rb < 0 ? 1.f : fb;
        }
    };
    auto store_codes = [&](const Codes &x, unsigned char *buf, float *tsc) HDA_INLINE {
        if constexpr (F8) {
#pragma unroll
            for (int m = 0; m < kBlocksPerWave; ++m)
                *reinterpret_cast<uint4 *>(buf + 1024 * (wave + kTileWaves * m) + 16 * lane) = e4m3x8_to_bf16x8(x.c[m]);
            if (wave == 0 && kg == 0) {  // lane mrow holds rows mrow and 16 + mrow
                tsc[mrow] = x.sa;
                tsc[16 + mrow] = x.sb;
            }
        }
    };
    Codes cA, cB;
    // Tiles 0 and 1 go in flight first, their rows read straight from the
    // index row; then q and the rest of the split's rows (into s_idx).
    {
        int r0a = -1, r0b = -1, r1a = -1, r1b = -1;
        if (nk > 0) {  // the four entries' loads issued together (no index to read otherwise)
            const int e0 = idx[min(drow, nk - 1)], e1 = idx[min(16 + drow, nk - 1)];
            const int e2 = idx[min(kTileKeys + drow, nk - 1)], e3 = idx[min(kTileKeys + 16 + drow, nk - 1)];
            __builtin_amdgcn_sched_barrier(0);
            auto valid = [&](int k, int r) { return k < nk && r >= 0 && (int64_t)r < p.pool_rows ? r : -1; };
            r0a = valid(drow, e0);
            r0b = valid(16 + drow, e1);
            r1a = valid(kTileKeys + drow, e2);
            r1b = valid(kTileKeys + 16 + drow, e3);
        }
        if constexpr (F8) {
            load_codes(r0a, r0b, cA);
            load_codes(r1a, r1b, cB);
        } else {
            issue_rows(r0a, r0b, s_b0);
            issue_rows(r1a, r1b, s_b1);
        }
    }
    for (int i = tid; i < ntile * kTileKeys; i += kTileWaves * 64) s_idx[i] = row_at(i);
    // q: lane (head mrow, c) holds dims 32j + 8c .. +7 of its head, every j
    uint4 qb[kKSteps];
    if (active) {
        const uint16_t *qr = p.q + ((int64_t)t * Hq + h0 + mrow) * kSparseDqk + 8 * kg;
#pragma unroll
        for (int j = 0; j < kKSteps; ++j) qb[j] = ld16(qr + 32 * j);
    }
    if (tid < kTileWaves) s_over[tid] = 0;
    // q, the indices and tiles 0 and 1 in: the tile loop's waits count only
    // the loads it issues
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();

    // This wave's blocks of tile i into `buf`; past the last tile every lane
    // reads the zero row, so that each tile leaves the same number of loads
    // behind it.
    auto issue = [&](int i, unsigned char *buf) HDA_INLINE {
        int ra = -1, rb = -1;
        if (i < ntile) {
            ra = s_idx[kTileKeys * i + drow];
            rb = s_idx[kTileKeys * i + 16 + drow];
        }
        issue_rows(ra, rb, buf);
    };
    auto issue_codes = [&](int i, Codes &x) HDA_INLINE {
        int ra = -1, rb = -1;
        if (i < ntile) {
            ra = s_idx[kTileKeys * i + drow];
            rb = s_idx[kTileKeys * i + 16 + drow];
        }
        load_codes(ra, rb, x);
    };

    f32x4 acc[kDimTiles];
#pragma unroll
    for (int d = 0; d < kDimTiles; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY, l_lane = 0.f, m_max = -INFINITY;
    bool over = false;
    // V^T transposing read of dim tile d in a half: row 4c + a, dims
    // 16d + 8b + 4e .. +3 for mrow = 4a + 2b + e, at 512 d + this offset
    // (the row's slot swizzled as the loads place it)
    const int tr_b = (mrow >> 1) & 1;
    const int tr_off = 256 * tr_b + 16 * ((4 * kg + (mrow >> 2)) ^ (12 * tr_b)) + 8 * (mrow & 1);

    auto compute = [&](int i, const unsigned char *buf, const float *tsc) HDA_INLINE {
        const int ra = s_idx[kTileKeys * i + mrow], rb = s_idx[kTileKeys * i + 16 + mrow];
        const uint32_t va = (uint32_t)__ballot(ra >= 0) & 0xFFFFu;
        const uint32_t vb = (uint32_t)__ballot(rb >= 0) & 0xFFFFu;
        if (!active) return;
        // scores: lane (head mrow, c) gets keys 4c + i of each half
        // (the K operand reads run kKAhead k-steps ahead of their products)
        f32x4 sa0 = {0.f, 0.f, 0.f, 0.f}, sa1 = sa0, sb0 = sa0, sb1 = sa0;
        uint4 ka[kKAhead], kb[kKAhead];
        auto k_read = [&](int j) HDA_INLINE {
            ka[j % kKAhead] = ld16(buf + 1024 * j + 16 * (drow + 16 * kg));
            kb[j % kKAhead] = ld16(buf + kHalfBytes + 1024 * j + 16 * (drow + 16 * kg));
        };
#pragma unroll
        for (int j = 0; j < kKAhead; ++j) k_read(j);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kKSteps; ++j) {
            const bf16x8 a = as_bf16x8(ka[j % kKAhead]), b = as_bf16x8(kb[j % kKAhead]);
            if (j + kKAhead < kKSteps) k_read(j + kKAhead);
            __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead (the scheduler would sink them)
            const bf16x8 qj = as_bf16x8(qb[j]);
            if (j & 1) {
                sa1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qj, sa1, 0, 0, 0);
                sb1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, qj, sb1, 0, 0, 0);
            } else {
                sa0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qj, sa0, 0, 0, 0);
                sb0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, qj, sb0, 0, 0, 0);
            }
        }
        // V^T reads run kTrAhead dim tiles ahead of the products that use
        // them (each product would otherwise wait out a whole LDS round
        // trip); the first go out before the softmax, which runs meanwhile
        v4i16 vlo[kTrAhead], vhi[kTrAhead];
        auto tr_read = [&](int d) HDA_INLINE {
            vlo[d % kTrAhead] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(buf + tr_off + 512 * d));
            vhi[d % kTrAhead] =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(buf + kHalfBytes + tr_off + 512 * d));
        };
        // F8: key 4kg + e of each half's row scale (1 for a masked key)
        float rsk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) rsk[e] = F8 ? tsc[16 * (e >> 2) + 4 * kg + (e & 3)] : 1.f;
#pragma unroll
        for (int d = 0; d < kTrAhead; ++d) tr_read(d);
        __builtin_amdgcn_sched_barrier(0);
        float s[8], tmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s[e] = ((va >> (4 * kg + e)) & 1u) ? (sa0[e] + sa1[e]) * (p.scale_log2 * rsk[e]) : -INFINITY;
            s[4 + e] = ((vb >> (4 * kg + e)) & 1u) ? (sb0[e] + sb1[e]) * (p.scale_log2 * rsk[4 + e]) : -INFINITY;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) tmax = fmaxf(tmax, s[e]);
        tmax = xor32_max(xor16_max(tmax));
        m_max = fmaxf(m_max, tmax);
        if (m_ref == -INFINITY) m_ref = tmax;  // first keys: nothing accumulated yet
        over |= tmax > m_ref + kSlack;
        const float mr = m_ref == -INFINITY ? 0.f : m_ref;
        float pw[8], ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pw[e] = __builtin_amdgcn_exp2f(s[e] - mr);
            ps += pw[e];
        }
        l_lane += ps;
        if constexpr (F8) {
#pragma unroll
            for (int e = 0; e < 8; ++e) pw[e] *= rsk[e];  // P.V reads the codes: the rows' scales here
        }
        const uint4 pu = make_uint4(pack_bf16x2(pw[0], pw[1]), pack_bf16x2(pw[2], pw[3]),
                                    pack_bf16x2(pw[4], pw[5]), pack_bf16x2(pw[6], pw[7]));
        const bf16x8 pb = as_bf16x8(pu);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < kDimTiles; ++d) {
            const v4i16 lo = vlo[d % kTrAhead], hi = vhi[d % kTrAhead];
            if (d + kTrAhead < kDimTiles) tr_read(d + kTrAhead);
            __builtin_amdgcn_sched_barrier(0);
            uint4 vu;
            vu.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
            vu.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
            vu.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
            vu.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
            acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vu), pb, acc[d], 0, 0, 0);
        }
    };

    // One tile: wait for this wave's blocks of tile i (tile i + 1's 9 may
    // still be in flight), meet the other waves (their blocks are in, and
    // all are done with tile i - 1's buffer), refill that buffer with tile
    // i + 2, score tile i.
    auto step = [&](int i, const unsigned char *cur, unsigned char *refill) HDA_INLINE {
        __builtin_amdgcn_s_waitcnt(0x0F70 | kBlocksPerWave);  // vmcnt(9)
        raw_barrier();
        issue(i + 2, refill);
        compute(i, cur, nullptr);
    };
    static_assert(kBlocksPerWave < 16, "vmcnt immediate");
    // F8: wait for tile i's codes (tile i + 1's 11 loads may be out), widen
    // them into `buf`, meet the other waves (the tile's blocks are in, and
    // all are done with tile i - 2, this buffer's last), load tile i + 2's
    // codes into the registers just emptied, score tile i.
    auto step8 = [&](int i, Codes &x, unsigned char *buf, float *tsc) HDA_INLINE {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kBlocksPerWave + 2));
        store_codes(x, buf, tsc);
        wave_lds_fence();
        raw_barrier();
        issue_codes(i + 2, x);
        compute(i, buf, tsc);
    };

    for (int pass = 0; pass < 2; ++pass) {
        if constexpr (F8) {
            if (pass > 0) {  // tiles 0 and 1 again
                issue_codes(0, cA);
                issue_codes(1, cB);
            }
            for (int i = 0; i < ntile; i += 2) {
                step8(i, cA, s_b0, s_tsc[0]);
                if (i + 1 >= ntile) break;
                step8(i + 1, cB, s_b1, s_tsc[1]);
            }
        } else {
            if (pass > 0) {  // tiles 0 and 1 again
                issue(0, s_b0);
                issue(1, s_b1);
            }
            for (int i = 0; i < ntile; i += 3) {
                step(i, s_b0, s_b2);
                if (i + 1 >= ntile) break;
                step(i + 1, s_b1, s_b0);
                if (i + 2 >= ntile) break;
                step(i + 2, s_b2, s_b1);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the loads past the end have landed
        const bool any_over = __ballot(over) != 0;  // the whole wave votes
        if (lane == 0) s_over[wave] = (active && any_over) ? 1 : 0;
        __syncthreads();
        const bool again = s_over[0] | s_over[1] | s_over[2] | s_over[3];
        __syncthreads();
        if (!again) break;
        // a score passed its head's reference by more than kSlack: every
        // wave scores its keys again against the exact maximum
#pragma unroll
        for (int d = 0; d < kDimTiles; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
        l_lane = 0.f;
        m_ref = m_max;
        over = false;
    }
    if (!active) return;

    const float l = xor32_sum(xor16_sum(l_lane));
    const int hq = h0 + mrow;
    const float lse = l > 0.f ? (m_ref + log2f(l)) * kLn2 : -INFINITY;
    float f = l > 0.f ? 1.f / l : 0.f;
    if (FINAL) {
        if (p.sinks && l > 0.f) f *= 1.f / (1.f + expf(p.sinks[hq] - lse));
        uint16_t *dst = p.out + ((int64_t)t * Hq + hq) * kSparseDv + 4 * kg;
#pragma unroll
        for (int d = 0; d < kDimTiles; ++d)
            *reinterpret_cast<uint2 *>(dst + 16 * d) =
                make_uint2(pack_bf16x2(acc[d][0] * f, acc[d][1] * f), pack_bf16x2(acc[d][2] * f, acc[d][3] * f));
        if (kg == 0 && p.lse) p.lse[(int64_t)t * Hq + hq] = lse;
    } else {
        const int64_t slot = ((int64_t)t * Hq + hq) * p.nsplit + sp;
        float *dst = p.part_o + slot * kSparseDv + 4 * kg;
#pragma unroll
        for (int d = 0; d < kDimTiles; ++d)
            *reinterpret_cast<float4 *>(dst + 16 * d) =
                make_float4(acc[d][0] * f, acc[d][1] * f, acc[d][2] * f, acc[d][3] * f);
        if (kg == 0) p.part_lse[slot] = lse;
    }
}

// LSE merge of the key splits, then the sink: one workgroup per (token,
// head), 128 threads x 4 dims.  The splits are read kMergeBatch at a time,
// every load of a batch issued before the first is used (8: the splits of
// the shared-tile kernel's calls at 32 tokens fill one batch; 16, half of
// them repeats of the last split, measured ~0.8 us slower per call).
constexpr int kMergeBatch = 8;

__global__ __launch_bounds__(128) void sparse_merge_kernel(SparseParams p) {
    const int hq = blockIdx.x % p.num_q_heads, t = blockIdx.x / p.num_q_heads;
    const int d = 4 * threadIdx.x;
    const int S = p.nsplit;
    const int64_t base = ((int64_t)t * p.num_q_heads + hq) * S;
    float M = -INFINITY;
    for (int s0 = 0; s0 < S; s0 += kMergeBatch) {
        float lv[kMergeBatch];
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) lv[k] = p.part_lse[base + min(s0 + k, S - 1)];
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) M = fmaxf(M, lv[k]);
    }
    float L = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
        for (int s0 = 0; s0 < S; s0 += kMergeBatch) {
            float lv[kMergeBatch];
            float4 ov[kMergeBatch];
#pragma unroll
            for (int k = 0; k < kMergeBatch; ++k) {
                const int64_t sl = base + min(s0 + k, S - 1);
                lv[k] = p.part_lse[sl];
                ov[k] = *reinterpret_cast<const float4 *>(p.part_o + sl * kSparseDv + d);
            }
#pragma unroll
            for (int k = 0; k < kMergeBatch; ++k) {
                const float w = s0 + k < S ? expf(lv[k] - M) : 0.f;  // clamped repeats weigh nothing
                L += w;
                o[0] = fmaf(w, ov[k].x, o[0]);
                o[1] = fmaf(w, ov[k].y, o[1]);
                o[2] = fmaf(w, ov[k].z, o[2]);
                o[3] = fmaf(w, ov[k].w, o[3]);
            }
        }
    }
    const float lse = L > 0.f ? M + logf(L) : -INFINITY;
    float f = L > 0.f ? 1.f / L : 0.f;
    if (p.sinks && L > 0.f) f *= 1.f / (1.f + expf(p.sinks[hq] - lse));
    uint16_t *dst = p.out + ((int64_t)t * p.num_q_heads + hq) * kSparseDv + d;
    *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(o[0] * f, o[1] * f), pack_bf16x2(o[2] * f, o[3] * f));
    if (threadIdx.x == 0 && p.lse) p.lse[(int64_t)t * p.num_q_heads + hq] = lse;
}

template <bool F8>
hipError_t launch_sparse(const SparseParams &p, hipStream_t s) {
    const int groups = p.num_q_heads / kSparseHeadsPerWave;
    const int64_t units = (int64_t)p.tokens * p.nsplit;
    const int64_t blocks = (units + 7) / 8 * 8 * groups;
    if (p.nsplit == 1) {
        hipLaunchKernelGGL((sparse_decode_kernel<true, F8>), dim3((unsigned)blocks), dim3(kSparseWaves * 64),
                           0, s, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((sparse_decode_kernel<false, F8>), dim3((unsigned)blocks), dim3(kSparseWaves * 64), 0,
                       s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sparse_merge_kernel, dim3((unsigned)((int64_t)p.tokens * p.num_q_heads)),
                       dim3(kSparseDv / 4), 0, s, p);
    return hipGetLastError();
}

template <bool F8>
hipError_t launch_sparse_tile(const SparseParams &p, hipStream_t s) {
    const int64_t blocks = ((int64_t)p.tokens + 7) / 8 * 8 * p.nsplit;
    if (p.nsplit == 1) {
        hipLaunchKernelGGL((sparse_tile_kernel<true, F8>), dim3((unsigned)blocks), dim3(kTileWaves * 64), 0, s, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((sparse_tile_kernel<false, F8>), dim3((unsigned)blocks), dim3(kTileWaves * 64), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sparse_merge_kernel, dim3((unsigned)((int64_t)p.tokens * p.num_q_heads)),
                       dim3(kSparseDv / 4), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_decode(const SparseParams &p, hipStream_t s) {
    if (sparse_uses_tiles(p.num_q_heads, p.kv8 != nullptr))
        return p.kv8 ? launch_sparse_tile<true>(p, s) : launch_sparse_tile<false>(p, s);
    return p.kv8 ? launch_sparse<true>(p, s) : launch_sparse<false>(p, s);
}

}  // namespace hda
