// rope_append.hip -- fused partial RoPE + KV append for one layer (gfx950).
//
// Spark export page: `_angles` builds angle_i = position * theta^(-2i/rot)
// in fp32; `_rope` rotates the neox halves (x1 = x[:rot/2], x2 =
// x[rot/2:rot]) by it and passes dims >= rot through; `_Layer.forward`
// (ring branch) drops the new entry into the slot for its position,
// evicting the oldest.  This kernel rotates q in place, rotates k_new into
// the cache row, copies v_new, and for a sliding layer first moves the
// evicted slot content (still inside this step's window) to the side row.
//
// One workgroup per sequence.  Work is split into "units": a rotary pair
// (dims j and j + rot/2) or one pass-through dim.  Each unit is owned by
// exactly one thread, for every head, so the read of an old slot element
// and the write of its replacement happen in the same thread and need no
// barrier.  The work is a few KB per sequence: latency, not bandwidth,
// bounds it.
#include "hda_device.h"
#include "hda_kernels.h"

namespace hda {

__global__ __launch_bounds__(256) void rope_append_kernel(RopeAppendParams p) {
    const int b = blockIdx.x;
    const int D = p.head_dim, rot = p.rotary_dim, half = rot / 2;
    const int32_t pos = p.pos[b];
    const int64_t cap = p.capacity;

    int64_t row;
    bool evict = false;
    if (p.sliding) {
        const int32_t slots = p.window - 1;
        if (pos < 0) return;
        row = pos % slots;
        evict = pos >= slots;
    } else {
        if (pos < 0 || (int64_t)pos >= cap) return;
        row = pos;
    }

    const int n_units = half + (D - rot);
    for (int u = threadIdx.x; u < n_units; u += blockDim.x) {
        if (u < half) {
            const int j = u;
            // Frequency rounded once to fp32 from an fp64 evaluation of
            // 1 / theta^(2j/rot); the angle is one fp32 multiply.
            const double expo = (double)(2 * j) / (double)rot;
            const float inv = (float)(1.0 / pow(p.theta, expo));
            const float ang = (float)pos * inv;
            double sd, cd;
            sincos((double)ang, &sd, &cd);
            const float c = (float)cd, s = (float)sd;

            for (int h = 0; h < p.num_q_heads; ++h) {
                uint16_t *qr = p.q + ((int64_t)b * p.num_q_heads + h) * D;
                const float x1 = bf16_to_f32(qr[j]), x2 = bf16_to_f32(qr[j + half]);
                qr[j] = f32_to_bf16(fmaf(x1, c, -x2 * s));
                qr[j + half] = f32_to_bf16(fmaf(x2, c, x1 * s));
            }
            for (int h = 0; h < p.num_kv_heads; ++h) {
                const int64_t bh = (int64_t)b * p.num_kv_heads + h;
                const uint16_t *kn = p.k_new + bh * D;
                const uint16_t *vn = p.v_new + bh * D;
                uint16_t *kr = p.k + (bh * cap + row) * D;
                uint16_t *vr = p.v + (bh * cap + row) * D;
                if (evict) {
                    p.k_evict[bh * D + j] = kr[j];
                    p.k_evict[bh * D + j + half] = kr[j + half];
                    p.v_evict[bh * D + j] = vr[j];
                    p.v_evict[bh * D + j + half] = vr[j + half];
                }
                const float x1 = bf16_to_f32(kn[j]), x2 = bf16_to_f32(kn[j + half]);
                kr[j] = f32_to_bf16(fmaf(x1, c, -x2 * s));
                kr[j + half] = f32_to_bf16(fmaf(x2, c, x1 * s));
                vr[j] = vn[j];
                vr[j + half] = vn[j + half];
            }
        } else {
            const int d = rot + (u - half);  // pass-through dim: q unchanged
            for (int h = 0; h < p.num_kv_heads; ++h) {
                const int64_t bh = (int64_t)b * p.num_kv_heads + h;
                uint16_t *kr = p.k + (bh * cap + row) * D;
                uint16_t *vr = p.v + (bh * cap + row) * D;
                if (evict) {
                    p.k_evict[bh * D + d] = kr[d];
                    p.v_evict[bh * D + d] = vr[d];
                }
                kr[d] = p.k_new[bh * D + d];
                vr[d] = p.v_new[bh * D + d];
            }
        }
    }
}

hipError_t launch_rope_append(const RopeAppendParams &p, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    hipLaunchKernelGGL(rope_append_kernel, dim3(p.batch), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace hda
