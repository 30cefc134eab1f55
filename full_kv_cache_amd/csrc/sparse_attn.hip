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
//
// With 64 query heads per shared row the path does about 121 flop per
// gathered byte, so both products run on the matrix cores:
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: 16 gathered rows form the A
//     operand, loaded straight from memory with 16-byte loads (8 dims of a
//     row per lane); the wave's 16 query heads form the B operand, held in
//     registers for the whole call;
//   * O^T += V^T P^T on v_mfma_f32_16x16x16_bf16: the S^T accumulator
//     already holds P^T in operand layout (4 keys of one head per lane), and
//     V^T comes out of LDS through the transposing read ds_read_b64_tr_b16
//     from the rows the wave has just stored there.
// Work split: one workgroup of 4 waves per (token, key split, group of 16
// heads); the waves take the split's 16-key tiles in turn, each with its own
// online softmax, and merge in LDS at the end.  The head-group workgroups of
// one (token, split) get block ids congruent mod 8, so they run on the same
// XCD and meet the gathered rows in its L2.
#include "hda_device.h"
#include "hda_kernels.h"

namespace hda {

namespace {

constexpr int kKSteps = kSparseDqk / 32;   // 16x16x32 steps over the key dims
constexpr int kVChunks = kSparseDv / 32;   // 16-byte chunks of the value part per lane
constexpr int kDimTiles = kSparseDv / 16;  // 16-dim output tiles
constexpr int kVPitch = kSparseDv + 16;    // LDS row pitch of a V tile (bf16)
constexpr int kOPitch = kSparseDv + 4;     // LDS row pitch of the merge buffer (fp32)
constexpr float kLn2 = 0.693147180559945309f;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

// Pool row of key kk for this lane, or -1 when the key is masked.
__device__ __forceinline__ int row_of(const SparseParams &p, const int32_t *idx, int kk, int k1) {
    if (kk >= k1) return -1;
    const int r = idx[kk];
    return (r >= 0 && (int64_t)r < p.pool_rows) ? r : -1;
}

__device__ __forceinline__ void load_rows(const SparseParams &p, int row, int kg, uint4 *kr) {
    const uint16_t *src = p.kv + (int64_t)(row < 0 ? 0 : row) * kSparseDqk + 8 * kg;
#pragma unroll
    for (int j = 0; j < kKSteps; ++j) kr[j] = ld16(src + 32 * j);
}

__device__ __forceinline__ short bf16_bits(float f) { return (short)f32_to_bf16(f); }

template <bool FINAL>
__global__ __launch_bounds__(kSparseWaves * 64) void sparse_decode_kernel(SparseParams p) {
    constexpr int kTileBytes = 16 * kVPitch * 2;
    __shared__ __align__(16) unsigned char s_buf[kSparseWaves * kTileBytes];
    __shared__ float s_m[kSparseWaves][16], s_l[kSparseWaves][16];
    static_assert(16 * kOPitch * 4 <= kSparseWaves * kTileBytes, "merge buffer fits the V tiles");

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
    const int h0 = g * kSparseHeadsPerWave;
    const int32_t *idx = p.indices + (int64_t)t * p.topk;

    // B operand: lane (head mrow, kg) holds q[t][h0 + mrow][32j + 8kg .. +7]
    bf16x8 qb[kKSteps];
    {
        const uint16_t *qr = p.q + ((int64_t)t * Hq + h0 + mrow) * kSparseDqk + 8 * kg;
#pragma unroll
        for (int j = 0; j < kKSteps; ++j) qb[j] = as_bf16x8(ld16(qr + 32 * j));
    }
    f32x4 acc[kDimTiles];
#pragma unroll
    for (int d = 0; d < kDimTiles; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_lane = 0.f;  // head mrow; l over this lane's keys

    uint16_t *vt = reinterpret_cast<uint16_t *>(s_buf + wave * kTileBytes);
    const uint16_t *trb = vt + (4 * kg + (mrow >> 2)) * kVPitch + 4 * (mrow & 3);

    int kb = k0 + 16 * wave;
    int r_cur = row_of(p, idx, kb + mrow, k1);
    uint4 kr[kKSteps];
    if (kb < k1) load_rows(p, r_cur, kg, kr);
    int r_nxt = row_of(p, idx, kb + 16 * kSparseWaves + mrow, k1);

    while (kb < k1) {
        // scores of the tile: lane (head mrow, kg) gets keys 4kg + i
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kKSteps; ++j)
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[j]), qb[j], sc, 0, 0, 0);
        const uint32_t vmask = (uint32_t)__ballot(r_cur >= 0) & 0xFFFFu;
        // value part of the rows into this wave's LDS tile; masked rows as 0
        // (a zero weight would not cancel a NaN they might hold)
        {
            uint16_t *dst = vt + mrow * kVPitch + 8 * kg;
            const bool keep = r_cur >= 0;
#pragma unroll
            for (int j = 0; j < kVChunks; ++j) {
                uint4 v = kr[j];
                if (vmask != 0xFFFFu && !keep) v = make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4 *>(dst + 32 * j) = v;
            }
        }
        // next tile's rows go in flight while this one is finished
        const int kn = kb + 16 * kSparseWaves;
        r_cur = r_nxt;
        if (kn < k1) load_rows(p, r_cur, kg, kr);
        r_nxt = row_of(p, idx, kn + 16 * kSparseWaves + mrow, k1);

        // online softmax (log2 domain) for head mrow over keys 4kg + i
        float s[4], tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[i] = ((vmask >> (4 * kg + i)) & 1u) ? sc[i] * p.scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, s[i]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run, tmax);
        float alpha = 1.f;
        v4i16 pb;
        if (m_new == -INFINITY) {  // nothing valid yet
            pb = v4i16{0, 0, 0, 0};
        } else {
            alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            float ps = 0.f, pv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pv[i] = __builtin_amdgcn_exp2f(s[i] - m_new);
                ps += pv[i];
            }
            l_lane = fmaf(l_lane, alpha, ps);
            pb = v4i16{bf16_bits(pv[0]), bf16_bits(pv[1]), bf16_bits(pv[2]), bf16_bits(pv[3])};
        }
        m_run = m_new;
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int d = 0; d < kDimTiles; ++d) acc[d] *= alpha;
        }
        wave_lds_fence();  // the tile's rows are in LDS
#pragma unroll
        for (int d = 0; d < kDimTiles; ++d) {
            const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(trb + 16 * d));
            acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, acc[d], 0, 0, 0);
        }
        wave_lds_fence();  // reads done before the next tile is stored
        kb = kn;
    }

    // merge the 4 waves: o = sum_w 2^(m_w - M) o_w, l likewise
    float l_w = l_lane + __shfl_xor(l_lane, 16, 64);
    l_w += __shfl_xor(l_w, 32, 64);
    if (kg == 0) {
        s_m[wave][mrow] = m_run;
        s_l[wave][mrow] = l_w;
    }
    __syncthreads();  // also: every wave is done with its V tile
    float *ob = reinterpret_cast<float *>(s_buf);
    {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kSparseWaves; ++w) M = fmaxf(M, s_m[w][mrow]);
        const float c = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
#pragma unroll
        for (int w = 0; w < kSparseWaves; ++w) {
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
    for (int w = 0; w < kSparseWaves; ++w) M = fmaxf(M, s_m[w][n]);
    float L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kSparseWaves; ++w) {
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

// LSE merge of the key splits, then the sink: one workgroup per (token,
// head), 128 threads x 4 dims.
__global__ __launch_bounds__(128) void sparse_merge_kernel(SparseParams p) {
    const int hq = blockIdx.x % p.num_q_heads, t = blockIdx.x / p.num_q_heads;
    const int d = 4 * threadIdx.x;
    const int S = p.nsplit;
    const int64_t base = ((int64_t)t * p.num_q_heads + hq) * S;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, p.part_lse[base + s]);
    float L = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
        for (int s = 0; s < S; ++s) {
            const float w = expf(p.part_lse[base + s] - M);
            const float4 v = *reinterpret_cast<const float4 *>(p.part_o + (base + s) * kSparseDv + d);
            L += w;
            o[0] = fmaf(w, v.x, o[0]);
            o[1] = fmaf(w, v.y, o[1]);
            o[2] = fmaf(w, v.z, o[2]);
            o[3] = fmaf(w, v.w, o[3]);
        }
    }
    const float lse = L > 0.f ? M + logf(L) : -INFINITY;
    float f = L > 0.f ? 1.f / L : 0.f;
    if (p.sinks) f *= 1.f / (1.f + expf(p.sinks[hq] - lse));
    uint16_t *dst = p.out + ((int64_t)t * p.num_q_heads + hq) * kSparseDv + d;
    const uint32_t lo = (uint32_t)f32_to_bf16(o[0] * f) | ((uint32_t)f32_to_bf16(o[1] * f) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(o[2] * f) | ((uint32_t)f32_to_bf16(o[3] * f) << 16);
    *reinterpret_cast<uint2 *>(dst) = make_uint2(lo, hi);
    if (threadIdx.x == 0 && p.lse) p.lse[(int64_t)t * p.num_q_heads + hq] = lse;
}

}  // namespace

hipError_t launch_sparse_decode(const SparseParams &p, hipStream_t s) {
    const int groups = p.num_q_heads / kSparseHeadsPerWave;
    const int64_t units = (int64_t)p.tokens * p.nsplit;
    const int64_t blocks = (units + 7) / 8 * 8 * groups;
    if (p.nsplit == 1) {
        hipLaunchKernelGGL(sparse_decode_kernel<true>, dim3((unsigned)blocks), dim3(kSparseWaves * 64), 0,
                           s, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(sparse_decode_kernel<false>, dim3((unsigned)blocks), dim3(kSparseWaves * 64), 0, s,
                       p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sparse_merge_kernel, dim3((unsigned)((int64_t)p.tokens * p.num_q_heads)),
                       dim3(kSparseDv / 4), 0, s, p);
    return hipGetLastError();
}

}  // namespace hda
