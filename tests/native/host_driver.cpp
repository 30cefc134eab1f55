// Drives every C-ABI entry point built for the host (hda_api.cpp with the
// launcher stand-ins of host_stubs.cpp) over a sweep of valid and invalid
// shapes, under AddressSanitizer and UndefinedBehaviorSanitizer.  Device
// pointers are fake aligned addresses that the host never dereferences;
// workspaces are sized by the library's own *_workspace_bytes queries, and
// the stand-ins check that every workspace pointer an entry point hands to
// a launcher lies inside the workspace.  Exit status 1 on any overrun.
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "hda.h"

namespace stub {
extern const char *ws_lo, *ws_hi;
extern bool caller_arrays;
extern int launches, failures;
}

namespace {

void *fake(uint64_t slot) { return reinterpret_cast<void *>(0x7f0000000000ull + (slot << 32)); }

int calls = 0, accepted = 0;

void count(hda_status st) {
    ++calls;
    if (st == HDA_OK) ++accepted;
}

void workspace(void *ws, size_t bytes) {
    stub::ws_lo = static_cast<const char *>(ws);
    stub::ws_hi = stub::ws_lo + bytes;
}

hda_cache_desc desc(int batch, int hq, int hkv, int window, int rot, int64_t cap, int fp8, int page) {
    hda_cache_desc d{};
    d.batch = batch;
    d.num_q_heads = hq;
    d.num_kv_heads = hkv;
    d.head_dim = 256;
    d.window = window;
    d.rotary_dim = rot;
    d.capacity = cap;
    d.rope_theta = rot == 256 ? 1e4 : 5e6;
    d.k = fake(1);
    d.v = fake(2);
    if (fp8) {
        d.kv_dtype = HDA_KV_FP8_E4M3;
        d.k_scale = static_cast<float *>(fake(3));
        d.v_scale = static_cast<float *>(fake(4));
    }
    if (page) {
        d.block_table = static_cast<const int32_t *>(fake(5));
        d.page_size = page;
        d.max_pages = (int32_t)(cap / page);
        d.num_pages = (int64_t)batch * d.max_pages;
    }
    return d;
}

void decode_calls(const hda_cache_desc &d, hda_layer_type layer, int32_t msl) {
    void *ws = fake(10);
    void *q = fake(11), *kn = fake(12), *vn = fake(13), *out = fake(14);
    const int32_t *pos = static_cast<const int32_t *>(fake(15));
    const float *sinks = static_cast<const float *>(fake(16)), *gate = static_cast<const float *>(fake(17));
    float *lse = static_cast<float *>(fake(18));
    count(hda_rope_append(q, kn, vn, pos, layer, &d, nullptr));
    for (int32_t chunk : {0, 16, 256, 1024, 17, -16}) {
        const size_t need = hda_decode_workspace_bytes(&d, layer, msl, chunk);
        workspace(ws, need);
        count(hda_decode_attn(q, &d, pos, layer, sinks, gate, 0.0625f, out, lse, msl, chunk, need ? ws : nullptr,
                              need, nullptr));
        if (need) count(hda_decode_attn(q, &d, pos, layer, sinks, gate, 0.0625f, out, lse, msl, chunk, ws, need - 1,
                                        nullptr));
        int32_t c = 0, ns = 0;
        if (hda_decode_split_plan(&d, layer, msl, chunk, &c, &ns) == HDA_OK) {
            float *po = static_cast<float *>(fake(19)), *pl = static_cast<float *>(fake(20));
            stub::caller_arrays = true;  // partials in the caller's own arrays
            count(hda_decode_attn_partials(q, &d, pos, layer, 0.0625f, msl, chunk, po, pl, nullptr));
            count(hda_lse_merge(po, pl, d.batch, d.num_q_heads, ns, 256, sinks, gate, out, lse, nullptr));
            stub::caller_arrays = false;
        }
    }
    const size_t sneed = hda_decode_step_workspace_bytes(&d, layer);
    workspace(ws, sneed);
    count(hda_decode_step(q, kn, vn, pos, layer, &d, sinks, gate, 0.0625f, out, lse, sneed ? ws : nullptr, sneed,
                          nullptr));
    for (int32_t t : {1, 2, 4, 5, 16, 33, 100, 511, 512, 513, 0}) {
        const size_t mneed = hda_decode_multi_workspace_bytes(&d, layer, t, msl);
        workspace(ws, mneed);
        count(hda_decode_multi(q, kn, vn, pos, t, layer, &d, sinks, gate, 0.0625f, out, lse, msl,
                               mneed ? ws : nullptr, mneed, nullptr));
    }
}

void sparse_calls() {
    void *ws = fake(30), *q = fake(31), *kv = fake(32), *out = fake(33);
    const int32_t *idx = static_cast<const int32_t *>(fake(34)), *len = static_cast<const int32_t *>(fake(35));
    const float *sinks = static_cast<const float *>(fake(36)), *scales = static_cast<const float *>(fake(37));
    float *lse = static_cast<float *>(fake(38));
    for (int32_t tokens : {0, 1, 8, 32, 300, 4096})
        for (int32_t heads : {16, 24, 48, 64, 128})
            for (int32_t topk : {0, 1, 17, 64, 2048, 2080, 5000}) {
                const size_t need = hda_sparse_workspace_bytes(tokens, heads, topk, 512);
                workspace(ws, need);
                count(hda_sparse_decode_attn(q, kv, 32768, idx, tokens, topk, len, heads, 576, 512, sinks, 0.04f, out,
                                             lse, need ? ws : nullptr, need, nullptr));
                count(hda_sparse_decode_attn_fp8(q, static_cast<const uint8_t *>(kv), scales, 32768, idx, tokens, topk,
                                                 heads, 576, 512, sinks, 0.04f, out, lse, need ? ws : nullptr, need,
                                                 nullptr));
            }
}

}  // namespace

int main() {
    const int groups[][2] = {{8, 2}, {2, 2}, {4, 4}, {16, 2}, {32, 2}, {6, 2}, {8, 3}};
    for (const auto &g : groups)
        for (int batch : {0, 1, 3, 64, 1600})
            for (int fp8 : {0, 1}) {
                decode_calls(desc(batch, g[0], g[1], 512, 256, 512, fp8, 0), HDA_SLIDING, 4096);
                decode_calls(desc(batch, g[0], g[1], 2048, 256, 2048, fp8, 0), HDA_SLIDING, 2048);
                for (int64_t cap : {4096, 32768, 100})
                    for (int page : {0, 64, 16})
                        decode_calls(desc(batch, g[0], g[1], 512, 64, cap, fp8, page), HDA_FULL, (int32_t)cap);
                decode_calls(desc(batch, g[0], g[1], 512, 24, 4096, fp8, 0), HDA_FULL, 4096);
            }
    sparse_calls();
    std::printf("%d calls, %d accepted, %d launches reached, %d workspace overruns\n", calls, accepted,
                stub::launches, stub::failures);
    return stub::failures ? 1 : 0;
}
