// rope_append.hip -- fused partial RoPE + KV append for one layer (gfx950).
//
// Spark export page: `_angles` builds angle_i = position * theta^(-2i/rot)
// in fp32; `_rope` rotates the neox halves (x1 = x[:rot/2], x2 =
// x[rot/2:rot]) by it and passes dims >= rot through; `_Layer.forward`
// (ring branch) drops the new entry into the slot for its position,
// evicting the oldest.  This kernel rotates q in place, rotates k_new into
// the cache row, copies v_new, and for a sliding layer first moves the
// evicted slot content (still inside this step's window) to the block's
// evicted-entry row, window-1.  A paged full layer writes row pos of the
// pool page its block table names for that row.
//
// One workgroup per sequence.  The work is cut into 16-byte tasks: a
// rotary task owns 8 consecutive pairs (dims j..j+7 and j+h..j+h+7, h =
// rot/2) of one head; a copy task owns 8 consecutive dims of a K
// pass-through range or of V.  Each element belongs to exactly one task,
// so the read of an old slot element and the write of its replacement
// happen in one thread.  All global loads are issued first; the angle
// table is built meanwhile (one pair index per thread: the fp32 frequency,
// rounded once from fp64 on the host, times the position in fp32, sin/cos
// evaluated in fp64 and rounded to fp32) and
// shared through LDS; then results are rotated and stored.  A few KB per
// sequence: latency, not bandwidth, bounds this kernel.
#include "hda_device.h"
#include "hda_kernels.h"

namespace hda {

namespace {

constexpr int kRopeThreads = 256;
constexpr int kMaxHalf = 256;  // rotary_dim <= 512

__device__ __forceinline__ uint4 ld(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void st(uint16_t *p, const uint4 &v) { *reinterpret_cast<uint4 *>(p) = v; }

}  // namespace

__global__ __launch_bounds__(kRopeThreads) void rope_append_kernel(RopeAppendParams p) {
    __shared__ float s_cos[kMaxHalf], s_sin[kMaxHalf];
    const int b = blockIdx.x;
    const int D = p.head_dim, rot = p.rotary_dim, half = rot / 2;
    const int32_t pos = p.pos[b];
    const int64_t cap = p.capacity;

    int64_t row = -1;
    bool evict = false;
    const int64_t erow = p.window - 1;  // evicted-entry row of a sliding block
    if (p.sliding) {
        const int32_t slots = p.window - 1;
        if (pos >= 0) {
            row = pos % slots;
            evict = pos >= slots;
        }
    } else if (pos >= 0 && (int64_t)pos < cap) {
        row = pos;
    }
    const bool write_cache = row >= 0;
    // element offset of cache row r of KV head h of this sequence: its
    // block's row, or (paged, full layers) the row in the page holding it
    auto row_off = [&](int h, int64_t r) -> int64_t {
        if (p.pages.block_table) {
            const int64_t pg = page_of(p.pages, b, r), ps = p.pages.page_size;
            return ((pg * p.num_kv_heads + h) * ps + r % ps) * D;
        }
        return (((int64_t)b * p.num_kv_heads + h) * cap + r) * D;
    };

    // Task space: [q rotary | k rotary | k pass-through | v], 16 bytes each.
    const int hc = half / 8, pc = (D - rot) / 8, vc = D / 8;
    const int n_q = p.num_q_heads * hc;
    const int n_k = p.num_kv_heads * hc;
    const int n_kp = p.num_kv_heads * pc;
    const int n_v = p.num_kv_heads * vc;
    const int n_tasks = n_q + n_k + n_kp + n_v;

    // Rounds of two tasks per thread; every round issues its loads first.
    for (int base = 0; base < n_tasks; base += 2 * kRopeThreads) {
        int task[2];
        uint4 xa[2], xb[2], oa[2], ob[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int t = base + threadIdx.x + r * kRopeThreads;
            task[r] = t < n_tasks ? t : -1;
            if (task[r] < 0) continue;
            if (t < n_q) {
                const int h = t / hc, j = (t % hc) * 8;
                const uint16_t *qr = p.q + ((int64_t)b * p.num_q_heads + h) * D;
                xa[r] = ld(qr + j);
                xb[r] = ld(qr + half + j);
            } else if (!write_cache) {
                task[r] = -1;
            } else if (t < n_q + n_k) {
                const int u = t - n_q, h = u / hc, j = (u % hc) * 8;
                const int64_t bh = (int64_t)b * p.num_kv_heads + h;
                xa[r] = ld(p.k_new + bh * D + j);
                xb[r] = ld(p.k_new + bh * D + half + j);
                if (evict) {
                    const uint16_t *kr = p.k + row_off(h, row);
                    oa[r] = ld(kr + j);
                    ob[r] = ld(kr + half + j);
                }
            } else if (t < n_q + n_k + n_kp) {
                const int u = t - n_q - n_k, h = u / pc, d = rot + (u % pc) * 8;
                const int64_t bh = (int64_t)b * p.num_kv_heads + h;
                xa[r] = ld(p.k_new + bh * D + d);
                if (evict) oa[r] = ld(p.k + row_off(h, row) + d);
            } else {
                const int u = t - n_q - n_k - n_kp, h = u / vc, d = (u % vc) * 8;
                const int64_t bh = (int64_t)b * p.num_kv_heads + h;
                xa[r] = ld(p.v_new + bh * D + d);
                if (evict) oa[r] = ld(p.v + row_off(h, row) + d);
            }
        }

        if (base == 0) {  // angle table while the first loads are in flight
            for (int j = threadIdx.x; j < half; j += kRopeThreads) {
                const float ang = (float)pos * p.inv_freq[j];  // one fp32 multiply
                sincos_angle(ang, s_cos + j, s_sin + j);
            }
            __syncthreads();
        }

#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int t = task[r];
            if (t < 0) continue;
            if (t < n_q) {
                const int h = t / hc, j = (t % hc) * 8;
                uint16_t *qr = p.q + ((int64_t)b * p.num_q_heads + h) * D;
                uint4 ya, yb;
                rotate8(xa[r], xb[r], s_cos + j, s_sin + j, ya, yb);
                st(qr + j, ya);
                st(qr + half + j, yb);
            } else if (t < n_q + n_k) {
                const int u = t - n_q, h = u / hc, j = (u % hc) * 8;
                if (evict) {
                    st(p.k + row_off(h, erow) + j, oa[r]);
                    st(p.k + row_off(h, erow) + half + j, ob[r]);
                }
                uint4 ya, yb;
                rotate8(xa[r], xb[r], s_cos + j, s_sin + j, ya, yb);
                uint16_t *kr = p.k + row_off(h, row);
                st(kr + j, ya);
                st(kr + half + j, yb);
            } else if (t < n_q + n_k + n_kp) {
                const int u = t - n_q - n_k, h = u / pc, d = rot + (u % pc) * 8;
                if (evict) st(p.k + row_off(h, erow) + d, oa[r]);
                st(p.k + row_off(h, row) + d, xa[r]);
            } else {
                const int u = t - n_q - n_k - n_kp, h = u / vc, d = (u % vc) * 8;
                if (evict) st(p.v + row_off(h, erow) + d, oa[r]);
                st(p.v + row_off(h, row) + d, xa[r]);
            }
        }
    }
}

// -------------------------------------------------------------------
// FP8 cache (e4m3 codes + one fp32 scale per row).  The same rotation as
// above -- identical arithmetic, so the rotated new K is the bf16 row the
// bf16 cache would hold -- then each new K and V row is quantized:
// scale = amax / 448, code = e4m3(x / scale), both fp32 divisions rounded
// to nearest.  One workgroup per sequence: the rotation tasks of the bf16
// kernel (q in place, K into LDS), then one wave per new row for the
// quantization (lane = 4 dims; amax by a wave reduction).
// -------------------------------------------------------------------
__global__ __launch_bounds__(kRopeThreads) void rope_append_fp8_kernel(RopeAppendParams p) {
    __shared__ float s_cos[kMaxHalf], s_sin[kMaxHalf];
    extern __shared__ __align__(16) uint16_t s_krow[];  // [Hkv, D] rotated new K, bf16
    constexpr int D = kHeadDim;
    const int b = blockIdx.x;
    const int rot = p.rotary_dim, half = rot / 2;
    const int32_t pos = p.pos[b];
    const int64_t cap = p.capacity;
    const int Hkv = p.num_kv_heads;

    int64_t row = -1;
    bool evict = false;
    const int64_t erow = p.window - 1;
    if (p.sliding) {
        const int32_t slots = p.window - 1;
        if (pos >= 0) {
            row = pos % slots;
            evict = pos >= slots;
        }
    } else if (pos >= 0 && (int64_t)pos < cap) {
        row = pos;
    }
    const bool write_cache = row >= 0;
    // cache row index (codes at index * D, scale at index) of row r of KV head h
    auto row_index = [&](int h, int64_t r) -> int64_t {
        if (p.pages.block_table) {
            const int64_t pg = page_of(p.pages, b, r), ps = p.pages.page_size;
            return (pg * Hkv + h) * ps + r % ps;
        }
        return ((int64_t)b * Hkv + h) * cap + r;
    };

    for (int j = threadIdx.x; j < half; j += kRopeThreads) {
        const float ang = (float)pos * p.inv_freq[j];  // one fp32 multiply
        sincos_angle(ang, s_cos + j, s_sin + j);
    }
    __syncthreads();

    // rotation tasks, 16 bytes each: [q rotary | k rotary | k pass-through]
    const int hc = half / 8, pc = (D - rot) / 8;
    const int n_q = p.num_q_heads * hc, n_k = Hkv * hc, n_kp = Hkv * pc;
    const int n_tasks = n_q + (write_cache ? n_k + n_kp : 0);
    for (int t = threadIdx.x; t < n_tasks; t += kRopeThreads) {
        if (t < n_q) {
            const int h = t / hc, j = (t % hc) * 8;
            uint16_t *qr = p.q + ((int64_t)b * p.num_q_heads + h) * D;
            uint4 ya, yb;
            rotate8(ld(qr + j), ld(qr + half + j), s_cos + j, s_sin + j, ya, yb);
            st(qr + j, ya);
            st(qr + half + j, yb);
        } else if (t < n_q + n_k) {
            const int u = t - n_q, h = u / hc, j = (u % hc) * 8;
            const uint16_t *kr = p.k_new + ((int64_t)b * Hkv + h) * D;
            uint4 ya, yb;
            rotate8(ld(kr + j), ld(kr + half + j), s_cos + j, s_sin + j, ya, yb);
            st(s_krow + h * D + j, ya);
            st(s_krow + h * D + half + j, yb);
        } else {
            const int u = t - n_q - n_k, h = u / pc, d = rot + (u % pc) * 8;
            st(s_krow + h * D + d, ld(p.k_new + ((int64_t)b * Hkv + h) * D + d));
        }
    }
    __syncthreads();
    if (!write_cache) return;

    // quantization: rows [K heads | V heads], one wave each, lane = 4 dims
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int r = wave; r < 2 * Hkv; r += kRopeThreads / 64) {
        const bool is_v = r >= Hkv;
        const int h = is_v ? r - Hkv : r;
        uint8_t *codes = is_v ? p.vq : p.kq;
        float *scales = is_v ? p.vs : p.ks;
        const int64_t slot = row_index(h, row);
        if (evict) {  // the slot's entry moves to the evicted-entry row first (same lane)
            const int64_t er = row_index(h, erow);
            const uint32_t old = *reinterpret_cast<const uint32_t *>(codes + slot * D + 4 * lane);
            const float old_s = scales[slot];
            *reinterpret_cast<uint32_t *>(codes + er * D + 4 * lane) = old;
            if (lane == 0) scales[er] = old_s;
        }
        const uint2 w = is_v ? *reinterpret_cast<const uint2 *>(p.v_new + ((int64_t)b * Hkv + h) * D + 4 * lane)
                             : *reinterpret_cast<const uint2 *>(s_krow + h * D + 4 * lane);
        const float x[4] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
        float sc;
        const uint32_t packed = quantize_row4(x, sc);
        *reinterpret_cast<uint32_t *>(codes + slot * D + 4 * lane) = packed;
        if (lane == 0) scales[slot] = sc;
    }
}

hipError_t launch_rope_append_fp8(const RopeAppendParams &p, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    const size_t lds = (size_t)p.num_kv_heads * kHeadDim * sizeof(uint16_t);
    hipLaunchKernelGGL(rope_append_fp8_kernel, dim3(p.batch), dim3(kRopeThreads), lds, stream, p);
    return hipGetLastError();
}

hipError_t launch_rope_append(const RopeAppendParams &p, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    hipLaunchKernelGGL(rope_append_kernel, dim3(p.batch), dim3(kRopeThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace hda
