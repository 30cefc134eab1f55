/*
 * oracle.c -- plain, slow CPU reference for hybrid decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no source with the HIP library.
 *
 * Arithmetic is IEEE fp64 except where the pages fix fp32 (the RoPE angle,
 * see or_rope_angles).  bf16 inputs are widened exactly; bf16 outputs are
 * rounded once, to nearest-even, straight from the fp64 value.
 *
 * Sources (all on the pages that define the method):
 *   [SPARK]  vllm-omni "edge/spark_export.py" page -- Spark-X2.5 decode step
 *            export: `_rope`, `_angles`, `SparkStepConfig.cache_len`,
 *            `_Layer.forward` (ring and roll branches), `kv_cache_bytes`.
 *   [SINK]   vLLM "hy_v4/nvidia/flashmla_sparse.py" page -- sink-capable
 *            FlashMLA sparse backend: the class docstring of
 *            `HYV4FlashMLASparseImpl` (sink formula), `_sinks_for_query`
 *            (-inf padding is a no-op sink), `_bf16_flash_mla_kernel`
 *            (sparse call: q, kv, indices, scale, sink, topk_length).
 *
 * Parity status of every function is listed in its header comment.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_SLIDING 0
#define OR_FULL 1

/* ------------------------------------------------------------------ bf16 */

/* Exact widening: a bf16 is the top half of an fp32. */
double or_bf16_to_f64(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round an fp64 value once, to nearest-even, to bf16 (8 significant bits,
 * fp32 exponent range, gradual underflow).  Not routed through fp32, which
 * would round twice. */
uint16_t or_f64_to_bf16(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int e;
    frexp(a, &e);                  /* a = m * 2^e, m in [0.5, 1) */
    int q = e - 8;                 /* quantum exponent for 8 significant bits */
    if (q < -133) q = -133;        /* bf16 subnormal quantum 2^-133 */
    double r = rint(ldexp(a, -q)); /* round half to even (default mode) */
    r = ldexp(r, q);
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80;
    float f = (float)r;            /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------ cache rules */

/* [SPARK] `SparkStepConfig.cache_len`: entries a layer holds at `context`
 * tokens.  Full layers hold the whole context.  A sliding window counts the
 * current token, so a ring holds window-1 previous entries; the roll layout
 * holds window.  Parity pinned by the page's 81/235 footprint figures. */
int64_t or_cache_len(int layer_type, int64_t context, int window, int ring) {
    if (layer_type != OR_SLIDING) return context;
    int64_t cap = ring ? (int64_t)(window - 1) : (int64_t)window;
    return context < cap ? context : cap;
}

/* [SPARK] `kv_cache_bytes`: per entry 2 (K and V) * kv_heads * head_dim *
 * bytes; hybrid = sum of cache_len over layers; uniform = layers * context.
 * out[0] = hybrid, out[1] = uniform. */
void or_kv_cache_bytes(const int *layer_types, int n_layers, int64_t context,
                       int window, int ring, int kv_heads, int head_dim,
                       int bytes_per_elem, int64_t *out) {
    int64_t per_entry = 2LL * kv_heads * head_dim * bytes_per_elem;
    int64_t hybrid = 0;
    for (int i = 0; i < n_layers; ++i)
        hybrid += or_cache_len(layer_types[i], context, window, ring);
    out[0] = hybrid * per_entry;
    out[1] = (int64_t)n_layers * context * per_entry;
}

/* Ring slot of the entry for position `pos`.  [SPARK] `_Layer.forward`,
 * ring branch: the runtime drops the new entry into the slot for its
 * position, evicting the oldest; with window-1 slots that slot is
 * pos mod (window-1), and the evicted entry is position pos-(window-1). */
int64_t or_ring_slot(int64_t pos, int window) { return pos % (int64_t)(window - 1); }

/* ------------------------------------------------------------------ RoPE */

/* [SPARK] `_angles`: inv[i] = 1 / theta^(2i/rot) for i < rot/2, built in
 * fp32 on the page; angle = position * inv in fp32.  Here inv is the exact
 * value rounded once to fp32 (fp64 evaluation, page order: power, then
 * reciprocal), and the angle is the page's single fp32 multiply.  cos and
 * sin of that fp32 angle are evaluated in fp64 and rounded to fp32, which
 * is the page's fp32 cos/sin to within one rounding.
 * Parity pinned: pos 0 identity, pos 1 frequency values, complex-rotation
 * form, relative-position property (tests/test_oracle_rope.py). */
void or_rope_angles(double theta, int rot, int64_t pos, float *cos_out, float *sin_out) {
    int half = rot / 2;
    for (int i = 0; i < half; ++i) {
        double expo = (double)(2 * i) / (double)rot;
        float inv = (float)(1.0 / pow(theta, expo));
        float ang = (float)pos * inv;   /* one fp32 multiply */
        cos_out[i] = (float)cos((double)ang);
        sin_out[i] = (float)sin((double)ang);
    }
}

/* [SPARK] `_rope`: neox-style rotation of the leading `rot` dims of each
 * head vector; with halves x1 = x[:rot/2], x2 = x[rot/2:rot],
 *   out = x_rot * cos + cat(-x2, x1) * sin,
 * cos/sin duplicated over both halves; dims rot..D-1 pass through.
 * x, y: bf16 [n_vec, D]; y may alias x.  Rotation in fp64, one rounding. */
void or_rope_apply(const uint16_t *x, uint16_t *y, int64_t n_vec, int D, int rot,
                   double theta, int64_t pos) {
    int half = rot / 2;
    float *c = (float *)malloc(sizeof(float) * (half > 0 ? half : 1));
    float *s = (float *)malloc(sizeof(float) * (half > 0 ? half : 1));
    or_rope_angles(theta, rot, pos, c, s);
    for (int64_t v = 0; v < n_vec; ++v) {
        const uint16_t *xv = x + v * D;
        uint16_t *yv = y + v * D;
        double *tmp = (double *)malloc(sizeof(double) * D);
        for (int d = 0; d < D; ++d) tmp[d] = or_bf16_to_f64(xv[d]);
        for (int j = 0; j < half; ++j) {
            double x1 = tmp[j], x2 = tmp[j + half];
            double r1 = x1 * (double)c[j] + (-x2) * (double)s[j];
            double r2 = x2 * (double)c[j] + x1 * (double)s[j];
            yv[j] = or_f64_to_bf16(r1);
            yv[j + half] = or_f64_to_bf16(r2);
        }
        for (int d = rot; d < D; ++d) yv[d] = xv[d];
        free(tmp);
    }
    free(c);
    free(s);
}

/* ------------------------------------------------------- rope + append */

/* One decode step's cache update for one layer, per sequence b:
 *   q[b]  (bf16 [Hq, D])  rotated in place at position pos[b];
 *   the new K (rotated) and V are written to the cache.
 * Full layer: K/V[b, h, pos[b], :] <- new.
 * Sliding layer ([SPARK] `_Layer.forward`, ring branch): slot
 *   s = pos mod (window-1).  The old slot content is position
 *   pos-(window-1), the oldest entry of the current window (a window counts
 *   the current token, [SPARK] `cache_len` docstring), so it is first kept
 *   in the side row kev/vev[b, h, :], then the slot takes the new entry.
 *   The side row is meaningful only when pos >= window-1; below that the
 *   slot was never written and the side row is left untouched.
 * A position outside the cache (negative, or at or past capacity on a full
 *   layer) writes no row; q is still rotated at it.
 * Layouts: k, v bf16 [B, Hkv, capacity, D]; kev, vev bf16 [B, Hkv, D];
 *   k_new, v_new bf16 [B, Hkv, D]; pos int32 [B].
 * Parity pinned bit-exact: slot arithmetic, untouched slots, side row =
 * prior slot content, ring vs roll streaming (tests/test_oracle_cache.py). */
void or_rope_append(uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                    const int32_t *pos, int layer_type, int B, int Hq, int Hkv,
                    int D, int rot, double theta, int window, int64_t capacity,
                    uint16_t *k, uint16_t *v, uint16_t *kev, uint16_t *vev) {
    uint16_t *krot = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)Hkv * D);
    for (int b = 0; b < B; ++b) {
        int64_t p = pos[b];
        or_rope_apply(q + (int64_t)b * Hq * D, q + (int64_t)b * Hq * D, Hq, D, rot, theta, p);
        or_rope_apply(k_new + (int64_t)b * Hkv * D, krot, Hkv, D, rot, theta, p);
        for (int h = 0; h < Hkv; ++h) {
            int64_t row;
            uint16_t *kb = k + ((int64_t)b * Hkv + h) * capacity * D;
            uint16_t *vb = v + ((int64_t)b * Hkv + h) * capacity * D;
            if (layer_type == OR_SLIDING) {
                if (p < 0) continue;
                row = or_ring_slot(p, window);
                if (p >= window - 1) {
                    memcpy(kev + ((int64_t)b * Hkv + h) * D, kb + row * D, sizeof(uint16_t) * D);
                    memcpy(vev + ((int64_t)b * Hkv + h) * D, vb + row * D, sizeof(uint16_t) * D);
                }
            } else {
                if (p < 0 || p >= capacity) continue;
                row = p;
            }
            memcpy(kb + row * D, krot + (int64_t)h * D, sizeof(uint16_t) * D);
            memcpy(vb + row * D, v_new + ((int64_t)b * Hkv + h) * D, sizeof(uint16_t) * D);
        }
    }
    free(krot);
}

/* ------------------------------------------------------ decode attention */

/* Attention of one query vector over an explicit list of key/value rows.
 * [SPARK] `_Layer.forward`: scores = q . k * scale, softmax over the keys,
 * weighted sum of values; scale = 1/sqrt(head_dim) there (passed in here).
 * Returns lse = ln(sum exp(scores)) (natural log, before any sink) and
 * writes the normalised output.  Empty key set: out 0, lse -inf. */
static void attend_rows(const double *qv, const uint16_t *const *krows,
                        const uint16_t *const *vrows, int64_t n, int Dqk, int Dv,
                        double scale, double *out, double *lse) {
    for (int d = 0; d < Dv; ++d) out[d] = 0.0;
    if (n == 0) {
        *lse = -INFINITY;
        return;
    }
    double *sc = (double *)malloc(sizeof(double) * n);
    double m = -INFINITY;
    for (int64_t i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int d = 0; d < Dqk; ++d) acc += qv[d] * or_bf16_to_f64(krows[i][d]);
        sc[i] = acc * scale;
        if (sc[i] > m) m = sc[i];
    }
    double l = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double p = exp(sc[i] - m);
        l += p;
        for (int d = 0; d < Dv; ++d) out[d] += p * or_bf16_to_f64(vrows[i][d]);
    }
    for (int d = 0; d < Dv; ++d) out[d] /= l;
    *lse = m + log(l);
    free(sc);
}

/* [SINK] `HYV4FlashMLASparseImpl` docstring: the sink folds into the
 * softmax denominator, out *= exp(lse) / (exp(lse) + exp(sink)), written
 * here exactly in that form.  A -inf sink gives factor 1 (the padding
 * no-op of `_sinks_for_query`). */
static double sink_factor(double lse, double sink) {
    double el = exp(lse);
    return el / (el + exp(sink));
}

/* Decode attention for one layer after the append.
 * For sequence b and query head h, the kv head is h / (Hq/Hkv)
 * ([SPARK] `_Layer.forward`: q folded to (kv, group, d), GQA without
 * expanded K/V).  Key set, with n = seq_lens[b] (= pos+1):
 *   full:    rows 0..n-1 of K/V[b, g];
 *   sliding: ring slots 0..min(n, window-1)-1, plus the side row when
 *            n >= window -- i.e. the last min(n, window) positions.
 *            Unwritten slots are excluded ([SPARK] ring comment: only
 *            slots not yet written need masking; ring order is arbitrary).
 * sinks: fp32 [Hq] or NULL.  out: fp64 [B, Hq, D]; lse: fp64 [B, Hq]
 * (pre-sink).  Parity pinned: fp64 brute force vs torch SDPA, one-key and
 * equal-key closed forms, sink as an extra zero-value key, -inf sink
 * bitwise no-op, slot permutation, ring vs roll
 * (tests/test_oracle_attention.py). */
void or_decode_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const uint16_t *kev, const uint16_t *vev, const int32_t *seq_lens,
                    int layer_type, int B, int Hq, int Hkv, int D, int window,
                    int64_t capacity, const float *sinks, double scale,
                    double *out, double *lse) {
    int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hq; ++h) {
            int g = h / G;
            int64_t n = seq_lens[b];
            const uint16_t *kb = k + ((int64_t)b * Hkv + g) * capacity * D;
            const uint16_t *vb = v + ((int64_t)b * Hkv + g) * capacity * D;
            int64_t nrows;
            const uint16_t **kr, **vr;
            if (layer_type == OR_SLIDING) {
                int64_t nring = n < window - 1 ? n : window - 1;
                int side = n >= window;
                nrows = nring + side;
                kr = (const uint16_t **)malloc(sizeof(void *) * (nrows + 1));
                vr = (const uint16_t **)malloc(sizeof(void *) * (nrows + 1));
                for (int64_t i = 0; i < nring; ++i) {
                    kr[i] = kb + i * D;
                    vr[i] = vb + i * D;
                }
                if (side) {
                    kr[nring] = kev + ((int64_t)b * Hkv + g) * D;
                    vr[nring] = vev + ((int64_t)b * Hkv + g) * D;
                }
            } else {
                nrows = n;
                kr = (const uint16_t **)malloc(sizeof(void *) * (nrows + 1));
                vr = (const uint16_t **)malloc(sizeof(void *) * (nrows + 1));
                for (int64_t i = 0; i < n; ++i) {
                    kr[i] = kb + i * D;
                    vr[i] = vb + i * D;
                }
            }
            double *qv = (double *)malloc(sizeof(double) * D);
            const uint16_t *qh = q + ((int64_t)b * Hq + h) * D;
            for (int d = 0; d < D; ++d) qv[d] = or_bf16_to_f64(qh[d]);
            double *o = out + ((int64_t)b * Hq + h) * D;
            double *ls = lse + (int64_t)b * Hq + h;
            attend_rows(qv, kr, vr, nrows, D, D, scale, o, ls);
            if (sinks) {
                double f = sink_factor(*ls, (double)sinks[h]);
                for (int d = 0; d < D; ++d) o[d] *= f;
            }
            free(qv);
            free(kr);
            free(vr);
        }
    }
}

/* ------------------------------------------------- split-K and LSE merge */

/* Attention of one query over rows [r0, r1) of a contiguous K/V block
 * ([SPARK] ring comment: softmax split over two key sets, merged online,
 * is the same result).  out: normalised over the chunk; lse_out: chunk
 * lse (-inf for an empty chunk). */
void or_attn_chunk(const uint16_t *qh, const uint16_t *kblk, const uint16_t *vblk,
                   int64_t r0, int64_t r1, int D, double scale, double *out,
                   double *lse_out) {
    int64_t n = r1 > r0 ? r1 - r0 : 0;
    const uint16_t **kr = (const uint16_t **)malloc(sizeof(void *) * (n + 1));
    const uint16_t **vr = (const uint16_t **)malloc(sizeof(void *) * (n + 1));
    for (int64_t i = 0; i < n; ++i) {
        kr[i] = kblk + (r0 + i) * D;
        vr[i] = vblk + (r0 + i) * D;
    }
    double *qv = (double *)malloc(sizeof(double) * D);
    for (int d = 0; d < D; ++d) qv[d] = or_bf16_to_f64(qh[d]);
    attend_rows(qv, kr, vr, n, D, D, scale, out, lse_out);
    free(qv);
    free(kr);
    free(vr);
}

/* Merge of per-chunk results into one softmax ([SPARK] ring comment on
 * the two-key-set online softmax): with lse_c the chunk lse and o_c the
 * chunk output,
 *   lse = ln sum_c exp(lse_c),  o = sum_c exp(lse_c - lse) o_c.
 * Empty chunks (lse_c = -inf) weigh zero.  Then the sink ([SINK] class
 * docstring) scales o, if given.  o_parts: [S, D]; lse_parts: [S]. */
void or_lse_merge(const double *o_parts, const double *lse_parts, int S, int D,
                  const float *sink, double *out, double *lse_out) {
    double m = -INFINITY;
    for (int c = 0; c < S; ++c)
        if (lse_parts[c] > m) m = lse_parts[c];
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    if (m == -INFINITY) {
        *lse_out = -INFINITY;
        return;
    }
    double tot = 0.0;
    for (int c = 0; c < S; ++c) tot += exp(lse_parts[c] - m);
    double lse = m + log(tot);
    for (int c = 0; c < S; ++c) {
        double w = exp(lse_parts[c] - lse);
        for (int d = 0; d < D; ++d) out[d] += w * o_parts[(int64_t)c * D + d];
    }
    *lse_out = lse;
    if (sink) {
        double f = sink_factor(lse, (double)*sink);
        for (int d = 0; d < D; ++d) out[d] *= f;
    }
}

/* Per-head output gate, [SPARK] `_Layer.forward`: every query head's
 * attention output is multiplied by that head's gate, the logistic sigmoid
 * of its g_proj value (one value per head, broadcast over head_dim):
 *   out[b][h][:] *= 1 / (1 + exp(-gate[b][h])).
 * The gate does not enter lse.  out: fp64 [B, Hq, D] in place; gate: fp32
 * logits [B, Hq].  Parity pinned: gate 0 halves out exactly, +inf leaves it
 * bit-for-bit unchanged, -inf zeroes it, ln 3 gives 3/4 (the sign of the
 * exponent), sigmoid(g) + sigmoid(-g) = 1, per-(b, h) indexing with B != Hq,
 * composition with the sink. */
void or_output_gate(double *out, int B, int Hq, int D, const float *gate) {
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            const double f = 1.0 / (1.0 + exp(-(double)gate[(int64_t)b * Hq + h]));
            double *o = out + ((int64_t)b * Hq + h) * D;
            for (int d = 0; d < D; ++d) o[d] *= f;
        }
}

/* ------------------------------------------------------------ FP8 KV */

/* FP8 KV cache, [SINK] `_fp8_flash_mla_kernel`: the cache is handed to the
 * kernel as raw bytes with an fp8 flag; the page prints no element format
 * and no scaling rule.  Reading (the plainest one the call supports):
 * elements are e4m3 -- 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
 * no infinities, S.1111.111 is NaN, largest finite 448 -- and every cached
 * row (one token, one KV head, head_dim elements) carries one fp32 scale:
 * value = decode(code) * scale. */

/* Value of an e4m3 code, from the format's definition. */
double or_e4m3_to_f64(uint8_t c) {
    const int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double a;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        a = ldexp((double)m, -9);            /* subnormal: m/8 * 2^-6 */
    else
        a = ldexp(8.0 + m, e - 7 - 3);       /* (1 + m/8) * 2^(e-7) */
    return sgn ? -a : a;
}

/* fp32 -> e4m3, round to nearest, ties to even, saturating to +-448 (a
 * scaled row never exceeds 448 by more than its own rounding; saturation
 * keeps such a value finite).  NaN -> 0x7F.  Parity pinned against torch's
 * float8_e4m3fn cast on |x| <= 448 (incl. exact ties and subnormals). */
uint8_t or_f32_to_e4m3(float x) {
    if (isnan(x)) return 0x7F;
    const uint8_t sgn = signbit(x) ? 0x80 : 0;
    double a = fabs((double)x);
    if (a == 0.0) return sgn;
    if (isinf(a)) return sgn | 0x7E;
    int e;
    frexp(a, &e);                  /* a in [2^(e-1), 2^e) */
    int ex = e - 1;                /* unbiased exponent of a */
    if (ex < -6) ex = -6;          /* subnormal range shares 2^-6's quantum */
    const double step = ldexp(1.0, ex - 3);
    double qn = rint(a / step);    /* exact quotient, half to even */
    /* qn in [0, 16]: 16 carries into the next binade (8 of its steps) */
    int code;
    if (ex == -6 && qn < 8)
        code = (int)qn;            /* subnormal (or zero) */
    else {
        if (qn >= 16) {
            qn = 8;
            ++ex;
        }
        code = ((ex + 7) << 3) | ((int)qn - 8);
    }
    if (code > 0x7E) code = 0x7E;  /* saturate at 448 */
    return sgn | (uint8_t)code;
}

/* Quantize rows of bf16 values: scale = amax / 448 (fp32 division; amax =
 * largest |x| of the row), code = e4m3(x / scale) with x / scale an fp32
 * division.  An all-zero row has scale 0 and zero codes.
 * x: bf16 [rows, D]; codes: [rows, D]; scales: fp32 [rows].
 * Parity pinned: the amax element maps to +-448, sign symmetry, zero row,
 * relative error <= 2^-4 (normal codes), agreement with dividing and
 * casting through torch. */
void or_quant_rows(const uint16_t *x, int64_t rows, int D, uint8_t *codes, float *scales) {
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * D;
        float amax = 0.f;
        for (int d = 0; d < D; ++d) {
            const float a = fabsf((float)or_bf16_to_f64(xr[d]));
            if (a > amax) amax = a;
        }
        const float sc = amax / 448.0f;
        scales[r] = sc;
        for (int d = 0; d < D; ++d)
            codes[r * D + d] = sc == 0.f ? 0 : or_f32_to_e4m3((float)or_bf16_to_f64(xr[d]) / sc);
    }
}

/* value = decode(code) * scale, in fp64 (exact: 4 + 24 significant bits).
 * codes: [rows, D], scales fp32 [rows] -> out fp64 [rows, D]. */
void or_dequant_rows(const uint8_t *codes, const float *scales, int64_t rows, int D, double *out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int d = 0; d < D; ++d)
            out[r * D + d] = or_e4m3_to_f64(codes[r * D + d]) * (double)scales[r];
}

/* The decode step's cache update on an fp8 cache: q rotated in place and
 * the new K rotated and rounded to bf16 exactly as or_rope_append does;
 * then the new K and V rows are quantized (or_quant_rows) into the slot.
 * Sliding: the old slot's codes and scale move to the side row first (when
 * pos >= window-1), as in or_rope_append.  Full: row pos (skipped outside
 * [0, capacity)).  Layouts: kc, vc [B, Hkv, capacity, D] codes; ks, vs fp32
 * [B, Hkv, capacity]; side rows kevc, vevc [B, Hkv, D] and kevs, vevs fp32
 * [B, Hkv].  Parity pinned: equals the bf16 append followed by quantizing
 * the written rows; side row = prior slot content. */
void or_rope_append_fp8(uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                        const int32_t *pos, int layer_type, int B, int Hq, int Hkv, int D,
                        int rot, double theta, int window, int64_t capacity, uint8_t *kc,
                        uint8_t *vc, float *ks, float *vs, uint8_t *kevc, uint8_t *vevc,
                        float *kevs, float *vevs) {
    uint16_t *krot = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)Hkv * D);
    for (int b = 0; b < B; ++b) {
        const int64_t p = pos[b];
        or_rope_apply(q + (int64_t)b * Hq * D, q + (int64_t)b * Hq * D, Hq, D, rot, theta, p);
        or_rope_apply(k_new + (int64_t)b * Hkv * D, krot, Hkv, D, rot, theta, p);
        for (int h = 0; h < Hkv; ++h) {
            const int64_t bh = (int64_t)b * Hkv + h;
            int64_t row;
            if (layer_type == OR_SLIDING) {
                if (p < 0) continue;
                row = or_ring_slot(p, window);
                if (p >= window - 1) {
                    memcpy(kevc + bh * D, kc + (bh * capacity + row) * D, (size_t)D);
                    memcpy(vevc + bh * D, vc + (bh * capacity + row) * D, (size_t)D);
                    kevs[bh] = ks[bh * capacity + row];
                    vevs[bh] = vs[bh * capacity + row];
                }
            } else {
                if (p < 0 || p >= capacity) continue;
                row = p;
            }
            or_quant_rows(krot + (int64_t)h * D, 1, D, kc + (bh * capacity + row) * D,
                          ks + bh * capacity + row);
            or_quant_rows(v_new + bh * D, 1, D, vc + (bh * capacity + row) * D,
                          vs + bh * capacity + row);
        }
    }
    free(krot);
}

/* Attention of one query over rows given as fp64 vectors (the dequantized
 * fp8 cache); otherwise attend_rows. */
static void attend_rows_f64(const double *qv, const double *const *krows,
                            const double *const *vrows, int64_t n, int D, double scale,
                            double *out, double *lse) {
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    if (n == 0) {
        *lse = -INFINITY;
        return;
    }
    double *sc = (double *)malloc(sizeof(double) * n);
    double m = -INFINITY;
    for (int64_t i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += qv[d] * krows[i][d];
        sc[i] = acc * scale;
        if (sc[i] > m) m = sc[i];
    }
    double l = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double p = exp(sc[i] - m);
        l += p;
        for (int d = 0; d < D; ++d) out[d] += p * vrows[i][d];
    }
    for (int d = 0; d < D; ++d) out[d] /= l;
    *lse = m + log(l);
    free(sc);
}

/* or_decode_attn over a cache held as fp64 values (an fp8 cache after
 * or_dequant_rows): the same key set, GQA map, softmax, lse and sink.
 * k, v fp64 [B, Hkv, capacity, D]; kev, vev fp64 [B, Hkv, D] (sliding).
 * Parity pinned: bit-identical to or_decode_attn when the values are
 * bf16-representable (power-of-two scales). */
void or_decode_attn_f64(const uint16_t *q, const double *k, const double *v, const double *kev,
                        const double *vev, const int32_t *seq_lens, int layer_type, int B,
                        int Hq, int Hkv, int D, int window, int64_t capacity,
                        const float *sinks, double scale, double *out, double *lse) {
    int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hq; ++h) {
            const int g = h / G;
            const int64_t n = seq_lens[b];
            const double *kb = k + ((int64_t)b * Hkv + g) * capacity * D;
            const double *vb = v + ((int64_t)b * Hkv + g) * capacity * D;
            int64_t nrows = n, nblk = n;
            int side = 0;
            if (layer_type == OR_SLIDING) {
                nblk = n < window - 1 ? n : window - 1;
                side = n >= window;
                nrows = nblk + side;
            }
            const double **kr = (const double **)malloc(sizeof(void *) * (nrows + 1));
            const double **vr = (const double **)malloc(sizeof(void *) * (nrows + 1));
            for (int64_t i = 0; i < nblk; ++i) {
                kr[i] = kb + i * D;
                vr[i] = vb + i * D;
            }
            if (side) {
                kr[nblk] = kev + ((int64_t)b * Hkv + g) * D;
                vr[nblk] = vev + ((int64_t)b * Hkv + g) * D;
            }
            double *qv = (double *)malloc(sizeof(double) * D);
            const uint16_t *qh = q + ((int64_t)b * Hq + h) * D;
            for (int d = 0; d < D; ++d) qv[d] = or_bf16_to_f64(qh[d]);
            double *o = out + ((int64_t)b * Hq + h) * D;
            double *ls = lse + (int64_t)b * Hq + h;
            attend_rows_f64(qv, kr, vr, nrows, D, scale, o, ls);
            if (sinks) {
                const double f = sink_factor(*ls, (double)sinks[h]);
                for (int d = 0; d < D; ++d) o[d] *= f;
            }
            free(qv);
            free(kr);
            free(vr);
        }
    }
}

/* Attention over fp64 rows whose keys are all Dqk dims and whose values
 * are the leading Dv dims (the sparse path's latent rows); the arithmetic
 * of attend_rows. */
static void attend_rows_kv_f64(const double *qv, const double *const *rows, int64_t n, int Dqk,
                               int Dv, double scale, double *out, double *lse) {
    for (int d = 0; d < Dv; ++d) out[d] = 0.0;
    if (n == 0) {
        *lse = -INFINITY;
        return;
    }
    double *sc = (double *)malloc(sizeof(double) * n);
    double m = -INFINITY;
    for (int64_t i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int d = 0; d < Dqk; ++d) acc += qv[d] * rows[i][d];
        sc[i] = acc * scale;
        if (sc[i] > m) m = sc[i];
    }
    double l = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double p = exp(sc[i] - m);
        l += p;
        for (int d = 0; d < Dv; ++d) out[d] += p * rows[i][d];
    }
    for (int d = 0; d < Dv; ++d) out[d] /= l;
    *lse = m + log(l);
    free(sc);
}

/* ---------------------------------------------------------- paged KV */

/* Paged cache addressing, [SINK] `_fp8_flash_mla_kernel`: the attention
 * call takes a block table and per-sequence cache lengths, i.e. each
 * sequence's rows live in fixed-size pages of a shared pool.  Reading (the
 * page's own layout is not printed; this is the plain one): row r of
 * sequence b is row r % page_size of pool page block_table[b][r / page_size].
 * Copies every sequence's rows 0 .. max_pages*page_size-1 out of the pool
 * into contiguous blocks, so that every other oracle function runs
 * unchanged on a paged cache.
 *   pool  bf16 [num_pages, Hkv, page_size, D]
 *   bt    int32 [B, max_pages]; an entry outside [0, num_pages) leaves its
 *         rows zero (no caller reads them)
 *   out   bf16 [B, Hkv, max_pages*page_size, D]
 * Parity pinned: a one-page-per-sequence table with the pool holding the
 * blocks in order is the identity; element-by-element brute force on a tiny
 * case; relabelling pool pages (permuting pool and table together) leaves
 * the result unchanged; each row lands at its page/offset position. */
void or_page_gather(const uint16_t *pool, const int32_t *bt, int B, int Hkv, int D,
                    int page_size, int max_pages, int64_t num_pages, uint16_t *out) {
    const int64_t cap = (int64_t)max_pages * page_size;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hkv; ++h)
            for (int64_t r = 0; r < cap; ++r) {
                uint16_t *dst = out + (((int64_t)b * Hkv + h) * cap + r) * D;
                const int32_t pg = bt[(int64_t)b * max_pages + r / page_size];
                if (pg < 0 || pg >= num_pages) {
                    memset(dst, 0, (size_t)D * sizeof(uint16_t));
                    continue;
                }
                const uint16_t *src = pool + (((int64_t)pg * Hkv + h) * page_size + r % page_size) * D;
                memcpy(dst, src, (size_t)D * sizeof(uint16_t));
            }
}

/* ------------------------------------------------------ sparse top-k */

/* Sparse top-k decode with a sink, [SINK] `_bf16_flash_mla_kernel`: one
 * latent KV head shared by all query heads; query t attends to pool rows
 * indices[t, i] for i < topk_length[t] (all topk when topk_length is NULL);
 * keys are the full Dqk-dim rows, values their leading Dv dims (the
 * `kv_c_and_k_pe` cache holds the latent part first; `head_dim_v` = Dv).
 * Negative indices are skipped.  q: bf16 [T, Hq, Dqk]; kv: bf16 [N, Dqk];
 * indices: int32 [T, topk]; out fp64 [T, Hq, Dv]; lse fp64 [T, Hq]
 * (pre-sink).  Parity pinned: dense reduction (topk = N, identity
 * indices) and gathered brute force vs torch SDPA; -inf sink no-op
 * (tests/test_oracle_sparse.py). */
void or_sparse_decode_attn(const uint16_t *q, const uint16_t *kv, int64_t N,
                           const int32_t *indices, int topk, const int32_t *topk_length,
                           int T, int Hq, int Dqk, int Dv, const float *sinks,
                           double scale, double *out, double *lse) {
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < Hq; ++h) {
            int len = topk_length ? topk_length[t] : topk;
            if (len > topk) len = topk;
            if (len < 0) len = 0;
            const uint16_t **rows = (const uint16_t **)malloc(sizeof(void *) * (len + 1));
            int64_t n = 0;
            for (int i = 0; i < len; ++i) {
                int32_t idx = indices[(int64_t)t * topk + i];
                if (idx < 0 || idx >= N) continue;
                rows[n++] = kv + (int64_t)idx * Dqk;
            }
            double *qv = (double *)malloc(sizeof(double) * Dqk);
            const uint16_t *qh = q + ((int64_t)t * Hq + h) * Dqk;
            for (int d = 0; d < Dqk; ++d) qv[d] = or_bf16_to_f64(qh[d]);
            double *o = out + ((int64_t)t * Hq + h) * Dv;
            double *ls = lse + (int64_t)t * Hq + h;
            attend_rows(qv, rows, rows, n, Dqk, Dv, scale, o, ls);
            if (sinks) {
                double f = sink_factor(*ls, (double)sinks[h]);
                for (int d = 0; d < Dv; ++d) o[d] *= f;
            }
            free(qv);
            free(rows);
        }
    }
}

/* Sparse top-k decode with a sink over an fp8 latent pool, [SINK]
 * `_fp8_flash_mla_kernel`: the same attention as or_sparse_decode_attn (no
 * topk_length in that call: every index entry counts, negative ones are
 * skipped), the cache handed over as bytes.  Reading (the call's layout is
 * named, not printed): e4m3 codes, one fp32 scale per pool row, the value
 * of element d of row r is or_e4m3_to_f64(codes[r][d]) * scales[r] -- for
 * the key dims and the leading Dv value dims alike (the same row).
 * Dequantization is exact in fp64; the attention is the fp64 one of
 * or_decode_attn_f64 (attend_rows_f64 with separate key and value dims).
 * q: bf16 [T, Hq, Dqk]; codes: uint8 [N, Dqk]; scales: fp32 [N]; indices:
 * int32 [T, topk]; out fp64 [T, Hq, Dv]; lse fp64 [T, Hq] (pre-sink).
 * Parity pinned: with power-of-two scales it equals or_sparse_decode_attn
 * over the bf16 pool holding the same values, bit for bit; brute force in
 * numpy fp64 on tiny inputs; -inf sink no-op (tests/test_oracle_sparse.py). */
void or_sparse_decode_attn_fp8(const uint16_t *q, const uint8_t *codes, const float *scales, int64_t N,
                               const int32_t *indices, int topk, int T, int Hq, int Dqk, int Dv,
                               const float *sinks, double scale, double *out, double *lse) {
    for (int t = 0; t < T; ++t) {
        /* the token's rows, dequantized once */
        double *rowv = (double *)malloc(sizeof(double) * ((size_t)topk * Dqk + 1));
        const double **rows = (const double **)malloc(sizeof(void *) * (topk + 1));
        int64_t n = 0;
        for (int i = 0; i < topk; ++i) {
            const int32_t idx = indices[(int64_t)t * topk + i];
            if (idx < 0 || idx >= N) continue;
            double *dst = rowv + n * Dqk;
            for (int d = 0; d < Dqk; ++d)
                dst[d] = or_e4m3_to_f64(codes[(int64_t)idx * Dqk + d]) * (double)scales[idx];
            rows[n++] = dst;
        }
#pragma omp parallel for schedule(dynamic)
        for (int h = 0; h < Hq; ++h) {
            double *qv = (double *)malloc(sizeof(double) * Dqk);
            const uint16_t *qh = q + ((int64_t)t * Hq + h) * Dqk;
            for (int d = 0; d < Dqk; ++d) qv[d] = or_bf16_to_f64(qh[d]);
            double *o = out + ((int64_t)t * Hq + h) * Dv;
            double *ls = lse + (int64_t)t * Hq + h;
            attend_rows_kv_f64(qv, rows, n, Dqk, Dv, scale, o, ls);
            if (sinks) {
                const double f = sink_factor(*ls, (double)sinks[h]);
                for (int d = 0; d < Dv; ++d) o[d] *= f;
            }
            free(qv);
        }
        free(rows);
        free(rowv);
    }
}

/* Threads the OpenMP runtime will use for the parallel loops above. */
int or_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
