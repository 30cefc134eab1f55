// decode_wave.h -- the wave-level building blocks of the GQA decode kernels
// (library-internal; included by decode_attn.hip and decode_step.hip).
//
// A 16-key round for one wave and one KV head:
//   * QK^T on the matrix cores, v_mfma_f32_16x16x32_bf16: the G query heads
//     are the 16-row A operand (rows >= G repeat row 0; their scores are
//     never read), the 16 keys the B operand.  K rows arrive like V rows -- each 16-byte load instruction
//     covers two whole 512-byte rows -- and pass through a per-wave LDS
//     tile into the operand layout (8 dims of one key per lane): loading the
//     operand layout straight from HBM (16 rows x 64 bytes per instruction)
//     streams about 30% slower;
//   * an online softmax in the log2 domain: round maximum over the 16 key
//     lanes (DPP), rescale of the running sum and output;
//   * P.V on the vector ALUs: each half-wave streams whole 512-byte V rows
//     (lane = 8 dims), every row serving all G heads; the probabilities
//     reach those lanes through LDS -- in the PVDOT form (the decode
//     kernels' default) as bf16, two keys per word, multiplied with
//     v_dot2c_f32_bf16 (fp32 accumulation; the running sum keeps the fp32
//     weights).
#pragma once

#include "hda_device.h"
#include "hda_kernels.h"

namespace hda {
namespace wave {

// Per-wave LDS tile of one round's 16 K rows; the row pitch is padded by 16
// bytes so the 16 rows of an operand read spread over the banks.
constexpr int kKPitch = kHeadDim + 8;
constexpr int kKTile = 16 * kKPitch;  // bf16 elements

constexpr float kLn2 = 0.693147180559945309f;


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

// A wave-uniform pointer as an opaque scalar value: selecting between such
// pointers compiles to a register select, never to a load of the selected
// pointer field from the kernel arguments.
template <typename T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return reinterpret_cast<T *>(((uint64_t)hi << 32) | lo);
}

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
// kg = lane/16) holds q[head m][32j + 8kg .. +7] for k-step j.  Rows m >= G
// repeat row 0: an output row of the product depends on its own A row
// only, and the softmax never reads those heads.  (Zeroing them instead is
// a select on the loaded values that the compiler hoists ahead of the K/V
// loads, so the stream would wait for q.)
template <int G>
__device__ __forceinline__ void load_q_operand(const uint16_t *q, int num_q_heads, int b, int kvh,
                                               int lane, bf16x8 *qa) {
    const int mrow = lane & 15, kg = lane >> 4;
    const int hrow = mrow < G ? mrow : 0;
    const uint16_t *qr = q + ((int64_t)b * num_q_heads + kvh * G + hrow) * kHeadDim + 8 * kg;
#pragma unroll
    for (int j = 0; j < 8; ++j) qa[j] = as_bf16x8(ld16(qr + 32 * j));
}

// Neox RoPE of the q operand in registers.  A lane holds dims 32j +
// 8(lane/16) .. +7 of chunk j; with rot = 64 NC, dim i < rot/2 pairs with
// i + rot/2, which sits in chunk j + NC of the same lane, so the rotation
// needs no lane exchange.  s_cs[i] holds (cos, sin) of angle i, shared
// through LDS (one fp64 evaluation per angle, written by rope_angles).
template <int NC>
__device__ __forceinline__ void rotate_q_chunks(bf16x8 *qa, const float2 *s_cs, int kg) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        float c[8], s[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float2 cs = s_cs[32 * j + 8 * kg + e];
            c[e] = cs.x;
            s[e] = cs.y;
        }
        uint4 ya, yb;
        rotate8(__builtin_bit_cast(uint4, qa[j]), __builtin_bit_cast(uint4, qa[j + NC]), c, s, ya, yb);
        qa[j] = as_bf16x8(ya);
        qa[j + NC] = as_bf16x8(yb);
    }
}
template <int ROT>
__device__ __forceinline__ void rotate_q_operand(bf16x8 *qa, const float2 *s_cs, int lane) {
    static_assert(ROT % 64 == 0 && ROT >= 64 && ROT <= 256, "rot = 64 NC, NC in 1..4");
    wave_lds_fence();  // rope_angles' stores are in
    rotate_q_chunks<ROT / 64>(qa, s_cs, lane >> 4);
}
// (cos, sin) of angles i < ROT/2 at position P into s_cs; s_freq holds
// the fp32 frequencies (kept in LDS: no register stays live for them
// through the rounds).  The angle is one fp32 product, as everywhere the
// rotation is applied.
template <int ROT>
__device__ __forceinline__ void rope_angles(float2 *s_cs, const float *s_freq, int P, int lane) {
    wave_lds_fence();  // earlier reads of s_cs are done
    float c, s;
#pragma unroll
    for (int i = 0; i < (ROT / 2 + 63) / 64; ++i) {
        const int a = lane + 64 * i;
        if (a < ROT / 2) {
            sincos_angle((float)P * s_freq[a], &c, &s);
            s_cs[a] = make_float2(c, s);
        }
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
    // kt / vt: the round's K and V rows as issue_round loads them (lane =
    // 8 dims of row 2u + half-wave).  ktile: this wave's LDS tile.
    // SUB: key vr of the round (if 0 <= vr < 16) takes its K row from knew
    // and its V row from vnew (LDS) instead of what was loaded.
    // FP8 (KV = uint2: 8 e4m3 codes of the same 8 dims): the K codes become
    // bf16 on their way into the tile (exact), the round's scores take the
    // key's K scale (ksc, lane = key mrow's scale), the probabilities sent to
    // the P.V lanes its V scale (vsc) -- the running sum keeps the unscaled
    // ones -- and the V codes become fp32 (exact).
    // ROWMASK (several query rows per head group, e.g. the tokens of a
    // chunk): row 4*kg + i also needs dkey >= trow[i] for this lane's key.
    // A row may then see no key in a round, so -inf maxima are guarded.
    // PVDOT (no SUB): the probabilities go to LDS as bf16, the
    // two keys a lane multiplies together (rows 2u + hw and 2u + 2 + hw)
    // side by side in one word, and P.V runs on v_dot2c_f32_bf16 -- half the
    // multiplies and no unpacking of V, for many query rows.  (pw holds
    // 16 * G floats; the bf16 layout uses half of it.)
    template <bool SUB = false, bool F8 = false, typename KV = uint4, bool ROWMASK = false,
              bool PVDOT = false>
    __device__ __forceinline__ void round(const bf16x8 *qa, const KV *kt, KV *vt, int lo,
                                          int hi, float scale_log2, float *pw, uint16_t *ktile, int lane,
                                          int vr = -1, const uint16_t *knew = nullptr,
                                          const uint16_t *vnew = nullptr, float ksc = 1.f,
                                          float vsc = 1.f, int dkey = 0,
                                          const int *trow = nullptr) {
        const int mrow = lane & 15, kg = lane >> 4, hw = lane >> 5, dl = lane & 31;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint4 kw;
            if constexpr (F8) kw = e4m3x8_to_bf16x8(kt[j]);
            else kw = kt[j];
            *reinterpret_cast<uint4 *>(ktile + (2 * j + hw) * kKPitch + 8 * dl) = kw;
        }
        if (SUB && vr >= 0 && hw == 0)
            *reinterpret_cast<uint4 *>(ktile + vr * kKPitch + 8 * dl) =
                *reinterpret_cast<const uint4 *>(knew + 8 * dl);
        wave_lds_fence();
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint4 kb = *reinterpret_cast<const uint4 *>(ktile + mrow * kKPitch + 32 * j + 8 * kg);
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j], as_bf16x8(kb), sc, 0, 0, 0);
        }
        // lane holds heads 4*kg + i of key mrow; a masked key's score is
        // replaced, never combined, so whatever its row holds cannot leak
        const bool valid = mrow >= lo && mrow < hi;
        const float kf = F8 ? scale_log2 * ksc : scale_log2;
        float alpha[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bool vi = valid;
            if constexpr (ROWMASK) vi = vi && dkey >= trow[i];
            float s = vi ? sc[i] * kf : -INFINITY;
            const float mn = fmaxf(m_run[i], row16_max(s));  // finite: the round holds a key
            if constexpr (ROWMASK) {
                const bool none = mn == -INFINITY;  // no key for this row yet
                alpha[i] = none ? 1.f : fast_exp2(m_run[i] - mn);
                s = none ? 0.f : fast_exp2(s - mn);
            } else {
                alpha[i] = fast_exp2(m_run[i] - mn);
                s = fast_exp2(s - mn);
            }
            l_lane[i] = fmaf(l_lane[i], alpha[i], s);
            m_run[i] = mn;
            sc[i] = s;
        }
        if constexpr (PVDOT) {
            // key k's slot in its row: 4 (k >> 2) + 2 (k & 1) + ((k >> 1) & 1)
            uint16_t *pw16 = reinterpret_cast<uint16_t *>(pw);
            const int slot = 4 * (mrow >> 2) + 2 * (mrow & 1) + ((mrow >> 1) & 1);
            if (4 * kg < G) {
                const float vf = F8 ? (valid ? vsc : 0.f) : 1.f;  // fp8: the key's V scale
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * kg + i < G)
                        pw16[(4 * kg + i) * 16 + slot] =
                            __builtin_bit_cast(uint16_t, (__bf16)(F8 ? sc[i] * vf : sc[i]));
            }
        } else if (4 * kg < G) {
            const float vf = valid ? vsc : 0.f;  // a masked key's scale may be anything
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * kg + i < G) pw[mrow * G + 4 * kg + i] = F8 ? sc[i] * vf : sc[i];
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
                if (key < lo || key >= hi) {
                    // (make_*, not KV{}: value-initialising the vector class
                    // kept the K/V arrays of some callers out of registers)
                    if constexpr (F8) vt[u] = make_uint2(0, 0);
                    else vt[u] = make_uint4(0, 0, 0, 0);
                }
            }
        }
        wave_lds_fence();
        if constexpr (PVDOT) {
            const uint32_t *pw32 = reinterpret_cast<const uint32_t *>(pw);
#pragma unroll
            for (int up = 0; up < 4; ++up) {
                // keys 4 up + hw and 4 up + 2 + hw: their dims paired per word
                // (fp8 codes become bf16 first: exact)
                uint4 va, vb;
                if constexpr (F8) {
                    va = e4m3x8_to_bf16x8(vt[2 * up]);
                    vb = e4m3x8_to_bf16x8(vt[2 * up + 1]);
                } else {
                    va = vt[2 * up];
                    vb = vt[2 * up + 1];
                }
                const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wb[4] = {vb.x, vb.y, vb.z, vb.w};
                uint32_t vp[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vp[2 * i] = __builtin_amdgcn_perm(wb[i], wa[i], 0x05040100u);
                    vp[2 * i + 1] = __builtin_amdgcn_perm(wb[i], wa[i], 0x07060302u);
                }
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const uint32_t pp = pw32[h * 8 + 2 * up + hw];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[h][e] = __builtin_amdgcn_fdot2_f32_bf16(
                            __builtin_bit_cast(bf16x2_t, vp[e]), __builtin_bit_cast(bf16x2_t, pp),
                            acc[h][e], false);
                }
            }
            // No wait here: the next round's tile and probability stores
            // come after these reads in this wave's LDS queue, which runs
            // in order; the barrier only keeps the compiler from moving them
            // (measured: 0.3 us off a sliding layer).
            __builtin_amdgcn_wave_barrier();
            return;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            float pv[G], x[8];
#pragma unroll
            for (int h = 0; h < G; ++h) pv[h] = pw[(2 * u + hw) * G + h];
            if constexpr (F8) {
                e4m3x8_to_f32(vt[u], x);
            } else {
                uint4 vv = vt[u];
                if (SUB && 2 * u + hw == vr) vv = *reinterpret_cast<const uint4 *>(vnew + 8 * dl);
                bf16x8_to_f32(vv, x);
            }
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pv[h], x[e], acc[h][e]);
        }
        wave_lds_fence();
    }

    // Wave totals of every head (wave-uniform): running max m_h and sum l_h.
    // Head h lives in lanes 16*(h/4) ..; the reads of those lanes must run
    // with the whole wave active, never inside a branch that some lane
    // skips: the compiler may sink the last step of the row sum into such a
    // branch, and the lanes it leaves out would then hold a partial sum.
    __device__ __forceinline__ void totals(float (&m_h)[G], float (&l_h)[G]) const {
        float l4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) l4[i] = row16_sum(l_lane[i]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            m_h[h] = lane_value(m_run[h & 3], 16 * (h >> 2));
            l_h[h] = lane_value(l4[h & 3], 16 * (h >> 2));
        }
    }
};

// Loads of one round: the 16 keys start at block row r0e (kept at most
// capacity - 16 so that every load stays inside the block); the caller
// masks keys outside [r0, n).  K and V alike: load u of the wave covers rows
// r0e + 2u and r0e + 2u + 1 whole (lane = 8 dims of row 2u + half-wave).
// Passing lane 0 for every lane makes a placeholder round: the same number
// of load instructions, all of one 16-byte address, so the wait counts stay
// exact at no traffic.
__device__ __forceinline__ void issue_round(const uint16_t *kblk, const uint16_t *vblk, int r0e,
                                            int lane, uint4 *kt, uint4 *vt) {
    const int hw = lane >> 5, dl = lane & 31;
    const uint16_t *rk = kblk + (int64_t)(r0e + hw) * kHeadDim + 8 * dl;
#pragma unroll
    for (int j = 0; j < 8; ++j) kt[j] = ld16_stream(rk + 2 * j * kHeadDim);
    const uint16_t *rv = vblk + (int64_t)(r0e + hw) * kHeadDim + 8 * dl;
#pragma unroll
    for (int u = 0; u < 8; ++u) vt[u] = ld16_stream(rv + 2 * u * kHeadDim);
}

// Loads of one fp8 round, the same rows and lanes as issue_round at half
// the bytes (lane = the 8 codes of row 2u + half-wave), plus each lane's
// key scales: lane l takes those of key l % 16, the key whose scores it
// holds after the QK^T product.  ksb / vsb: the scales of the block's rows.
__device__ __forceinline__ void issue_round8(const uint8_t *kblk, const uint8_t *vblk,
                                             const float *ksb, const float *vsb, int r0e,
                                             int lane, uint2 *kt, uint2 *vt, float &ksc,
                                             float &vsc) {
    const int hw = lane >> 5, dl = lane & 31;
    const uint8_t *rk = kblk + (int64_t)(r0e + hw) * kHeadDim + 8 * dl;
#pragma unroll
    for (int j = 0; j < 8; ++j) kt[j] = ld8_stream(rk + 2 * j * kHeadDim);
    const uint8_t *rv = vblk + (int64_t)(r0e + hw) * kHeadDim + 8 * dl;
#pragma unroll
    for (int u = 0; u < 8; ++u) vt[u] = ld8_stream(rv + 2 * u * kHeadDim);
    ksc = ksb[r0e + (lane & 15)];
    vsc = vsb[r0e + (lane & 15)];
}

// Writes o / l for the G heads (first half-wave) and their lse.
template <int G>
__device__ __forceinline__ void store_partial(const WaveSoftmax<G> &st, float *po, float *plse,
                                              int lane) {
    const int hw = lane >> 5, dl = lane & 31;
    float m_h[G], l_h[G];
    st.totals(m_h, l_h);
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float l = l_h[h];
        const float inv = 1.f / l;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = xor32_sum(st.acc[h][e]) * inv;
        if (hw == 0) {
            float *dst = po + h * kHeadDim + 8 * dl;
            *reinterpret_cast<float4 *>(dst) = make_float4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<float4 *>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
        }
        if (lane == 0) plse[h] = (m_h[h] + log2f(l)) * kLn2;
    }
}

// ---------------------------------------------------------------------
// Balanced streaming partition.  Pair (b, kvh) holds R_b = ceil(n_b / 16)
// rounds of 16 keys; all rounds, pair after pair, form one index space of
// R_tot = Hkv * sum_b R_b rounds, which a grid of W single-wave workgroups
// splits evenly: wave w takes [w*R_tot/W, (w+1)*R_tot/W).
struct RoundAddr {
    int b, kvh, rr;  // sequence, KV head, round within the pair
};

// s_pre[b] = rounds of sequences 0..b-1 (one KV head), keys(b) = n_b; one
// wave, 64 sequences a pass.  The caller synchronises before reading.
template <typename Keys>
__device__ __forceinline__ void round_prefix(int *s_pre, int B, int lane, Keys keys) {
    int carry = 0;
    for (int base = 0; base < B; base += 64) {
        const int b = base + lane;
        int x = b < B ? (keys(b) + 15) >> 4 : 0;
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

// Address of round g (< R_tot): the sequence by binary search, then the KV
// head and the round within the pair.
__device__ __forceinline__ RoundAddr locate_round(const int *s_pre, int B, int Hkv, int64_t g) {
    int lo = 0, hi = B;  // largest b with Hkv * pre[b] <= g
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)Hkv * s_pre[mid] <= g) lo = mid; else hi = mid;
    }
    int b = lo;
    while ((int64_t)Hkv * s_pre[b + 1] <= g) ++b;  // sequences without rounds
    const int rb = s_pre[b + 1] - s_pre[b];
    const int off = (int)(g - (int64_t)Hkv * s_pre[b]);
    RoundAddr a;
    a.b = uniform(b);
    a.kvh = uniform(off / rb);
    a.rr = uniform(off % rb);
    return a;
}

__device__ __forceinline__ RoundAddr next_round(const int *s_pre, int B, int Hkv, RoundAddr a) {
    auto rounds_of = [&](int b) { return uniform(s_pre[b + 1] - s_pre[b]); };
    if (++a.rr == rounds_of(a.b)) {
        a.rr = 0;
        if (++a.kvh == Hkv) {
            a.kvh = 0;
            do { ++a.b; } while (a.b < B && rounds_of(a.b) == 0);
        }
    }
    return a;
}

// Waves the rounds are split over: the grid's W, but never more than there
// are rounds (the grid is sized before the lengths are known), so that every
// wave holds at least one round and the waves from the first to the last
// of a pair's rounds each hold one of its segments.
__device__ __forceinline__ int split_waves(int W, int64_t r_tot) {
    return (int)(r_tot < W ? r_tot : W);
}

// Wave whose range holds round g: the largest w with w*R_tot/W <= g
// (W = split_waves(...), so that range is not empty).
__device__ __forceinline__ int wave_of_round(int64_t g, int64_t r_tot, int W) {
    return (int)(((g + 1) * W - 1) / r_tot);
}

}  // namespace wave
}  // namespace hda
