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

hipError_t launch_rope_append(const RopeAppendParams &p, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    hipLaunchKernelGGL(rope_append_kernel, dim3(p.batch), dim3(kRopeThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace hda
