// Host-only stand-ins for the library's kernel launchers, so that the C-ABI
// entry points (hda_api.cpp) can be built for the CPU with AddressSanitizer
// and UndefinedBehaviorSanitizer and driven without a GPU.  Every launcher
// records that it was reached and checks that the pointers the entry point
// carved out of the caller's workspace lie inside it (the driver announces
// the workspace range before each call).  No kernel runs.
#include <cstdio>
#include <cstdlib>

#include "hda_kernels.h"

namespace stub {
const char *ws_lo = nullptr, *ws_hi = nullptr;  // the current call's workspace
bool caller_arrays = false;  // the call takes its partials from the caller: nothing to check
int launches = 0;
int failures = 0;

void in_ws(const void *p, size_t bytes, const char *what) {
    if (!p || caller_arrays) return;
    const char *c = static_cast<const char *>(p);
    if (!ws_lo || c < ws_lo || c + bytes > ws_hi) {
        std::printf("workspace overrun: %s [%p, +%zu) outside [%p, %p)\n", what, p, bytes, (const void *)ws_lo,
                    (const void *)ws_hi);
        ++failures;
    }
}
}  // namespace stub

extern "C" const char *hipGetErrorString(hipError_t) { return "stub"; }

namespace hda {
int stream_wave_slots(int) { return 2048; }
int step_wave_slots(int, int) { return 2048; }

hipError_t launch_rope_append(const RopeAppendParams &, hipStream_t) { ++stub::launches; return hipSuccess; }
hipError_t launch_rope_append_fp8(const RopeAppendParams &, hipStream_t) { ++stub::launches; return hipSuccess; }

hipError_t launch_decode_pairs(const DecodeParams &, int, hipStream_t) { ++stub::launches; return hipSuccess; }

hipError_t launch_decode_chunks(const DecodeParams &p, int group, bool, hipStream_t) {
    ++stub::launches;
    if (p.nsplit > 1) {
        const size_t rows = (size_t)p.batch * p.num_q_heads * p.nsplit;
        stub::in_ws(p.part_o, rows * kHeadDim * sizeof(float), "chunk part_o");
        stub::in_ws(p.part_lse, rows * sizeof(float), "chunk part_lse");
    }
    return hipSuccess;
}

hipError_t launch_decode_stream(const DecodeParams &p, int, int waves, hipStream_t) {
    ++stub::launches;
    stub::in_ws(p.part_o, 1, "stream part_o");
    stub::in_ws(p.part_lse, 1, "stream part_lse");
    stub::in_ws(p.stream_pre, ((size_t)p.batch + 1) * sizeof(int), "stream prefix");
    return hipSuccess;
}

hipError_t launch_decode_stream_step(const DecodeParams &p, const StreamStep &st, int, int, hipStream_t) {
    ++stub::launches;
    stub::in_ws(p.part_o, 1, "stream step part_o");
    stub::in_ws(p.stream_pre, ((size_t)p.batch + 1) * sizeof(int), "stream step prefix");
    stub::in_ws(st.s_new, (size_t)p.batch * p.num_q_heads * sizeof(float), "stream step new-key scores");
    return hipSuccess;
}

hipError_t launch_lse_merge(const MergeParams &, hipStream_t) { ++stub::launches; return hipSuccess; }

hipError_t launch_decode_step(const StepParams &p, int, int, int, hipStream_t) {
    ++stub::launches;
    stub::in_ws(p.counters, (size_t)p.batch * p.num_kv_heads * sizeof(int), "step counters");
    stub::in_ws(p.part_o, 1, "step part_o");
    return hipSuccess;
}

hipError_t launch_decode_window_step(const StepParams &p, int group, int, hipStream_t) {
    ++stub::launches;
    stub::in_ws(p.counters, (size_t)p.batch * p.num_kv_heads * sizeof(int), "window step counters");
    const WindowPlan w = window_step_plan(group, (int64_t)p.batch * p.num_kv_heads, p.window);
    if (w.key_split) {
        const size_t slots = (size_t)p.batch * p.num_kv_heads * w.parts;
        stub::in_ws(p.part_o, slots * group * kHeadDim * sizeof(float), "window step part_o");
        stub::in_ws(p.part_lse, slots * group * sizeof(float), "window step part_lse");
    }
    return hipSuccess;
}

hipError_t launch_decode_multi(const MultiParams &p, int, hipStream_t) {
    ++stub::launches;
    stub::in_ws(p.k_rot, (size_t)p.batch * p.tokens * p.num_kv_heads * kHeadDim * sizeof(uint16_t), "multi k_rot");
    if (p.split > 1) stub::in_ws(p.part_o, 1, "multi part_o");
    return hipSuccess;
}

hipError_t launch_sparse_decode(const SparseParams &p, hipStream_t) {
    ++stub::launches;
    if (p.nsplit > 1) {
        const size_t rows = (size_t)p.tokens * p.num_q_heads * p.nsplit;
        stub::in_ws(p.part_o, rows * kSparseDv * sizeof(float), "sparse part_o");
        stub::in_ws(p.part_lse, rows * sizeof(float), "sparse part_lse");
    }
    return hipSuccess;
}
}  // namespace hda
