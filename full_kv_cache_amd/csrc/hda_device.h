// hda_device.h -- small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Lambdas that capture kernel arguments by reference must be inlined: an
// out-of-line call makes the compiler copy the whole argument block to
// scratch memory.
#define HDA_INLINE __attribute__((always_inline))

namespace hda {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

// bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Two floats rounded to bf16 (nearest even) in one word, a low; the
// hardware conversion (v_cvt_pk_bf16_f32), branch-free.
typedef __bf16 hda_bf16x2 __attribute__((ext_vector_type(2)));
typedef float hda_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((hda_f32x2){a, b}, hda_bf16x2));
}

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// Streaming 16-byte load of data read exactly once (KV rows): non-temporal
// hint so it does not push reusable lines out of the caches.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ld8_stream(const void *p) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    return make_uint2(v.x, v.y);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// e4m3 codes -> values, exact (every e4m3 value is a bf16 and an fp32 value):
// the gfx950 conversions, two codes per instruction (word_sel picks bytes
// 0-1 or 2-3 of the source register; the lower byte becomes the lower
// element).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi) {
    const bf16x2_t r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true)
                          : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 w) {
    return make_uint4(e4m3x2_to_bf16x2(w.x, false), e4m3x2_to_bf16x2(w.x, true),
                      e4m3x2_to_bf16x2(w.y, false), e4m3x2_to_bf16x2(w.y, true));
}
// fp32 -> e4m3 (bias 7, 3 mantissa bits, largest finite 448, S.1111.111
// NaN), round to nearest even, saturating at +-448.
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sgn = (u >> 24) & 0x80u, a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return 0x7Fu;                  // NaN
    if (a >= 0x43E00000u) return sgn | 0x7Eu;           // >= 448 (and inf): saturate
    if (a < 0x3C800000u) {                              // below 2^-6: steps of 2^-9
        const float q = rintf(__uint_as_float(a) * 512.f);  // exact scaling, half to even
        return sgn | (uint32_t)q;                       // 8 is 2^-6's own code
    }
    const uint32_t keep = (a >> 20) & 7u, rem = a & 0xFFFFFu;
    const uint32_t up = rem > 0x80000u || (rem == 0x80000u && (keep & 1u));
    uint32_t v = (((a >> 23) - 127u + 7u) << 3) + keep + up;  // a carry moves into the exponent
    if (v > 0x7Eu) v = 0x7Eu;
    return sgn | v;
}

// Lane l with lane l ^ 16 (or l ^ 32) on the vector ALU: each permlane swap
// hands a lane both values of its pair (in some order), and a max or a sum
// does not depend on it -- the same result as a shuffle, without its LDS
// round trip (which queues behind the other waves' LDS reads).
__device__ __forceinline__ float xor16_max(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum over the wave: within each row of 16 lanes by DPP moves (the
// quad swaps, then the half-row and row mirrors), then across the rows by
// the permlane swaps -- no LDS round trip; a maximum does not depend on
// the order in which it is taken.
__device__ __forceinline__ float wave_max64(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));   // quad [1,0,3,2]
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));   // quad [2,3,0,1]
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));  // half-row mirror
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));  // row mirror
    return xor32_max(xor16_max(v));
}

// One row of 4 * 64 values quantized by a wave (lane = 4 consecutive
// values): scale = amax / 448 and code = e4m3(x / scale), both fp32
// divisions rounded to nearest; an all-zero row gets scale 0, codes 0.
// Returns this lane's 4 codes packed (lowest value in the low byte).
__device__ __forceinline__ uint32_t quantize_row4(const float (&x)[4], float &scale) {
    float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
    amax = wave_max64(amax);
    scale = __fdiv_rn(amax, 448.f);
    uint32_t packed = 0;
    if (scale != 0.f) {
#pragma unroll
        for (int e = 0; e < 4; ++e) packed |= e4m3_rne(__fdiv_rn(x[e], scale)) << (8 * e);
    }
    return packed;
}

__device__ __forceinline__ void e4m3x8_to_f32(uint2 w, float *x) {
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
    const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
    const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
    const f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
    x[0] = a.x; x[1] = a.y; x[2] = b.x; x[3] = b.y;
    x[4] = c.x; x[5] = c.y; x[6] = d.x; x[7] = d.y;
}

// A 16-byte load from a pointer known to address device (global) memory,
// for pointers whose address space the compiler cannot see.
__device__ __forceinline__ uint4 ld16_global(const void *p) {
    const u32x4 v = *(const __attribute__((address_space(1))) u32x4 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// neox RoPE of 8 consecutive dim pairs: a holds x[i .. i+7], b holds
// x[i+h .. i+h+7] (h = rot/2), c / s the fp32 cos / sin of angles i .. i+7.
// First half x1*cos - x2*sin, second half x2*cos + x1*sin, one fp32 fma
// each, rounded once to bf16.
__device__ __forceinline__ void rotate8(const uint4 &a, const uint4 &b, const float *c,
                                        const float *s, uint4 &ya, uint4 &yb) {
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
    uint32_t ra[4], rb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float x1l = bf16_lo(wa[i]), x1h = bf16_hi(wa[i]);
        const float x2l = bf16_lo(wb[i]), x2h = bf16_hi(wb[i]);
        const float cl = c[2 * i], sl = s[2 * i], ch = c[2 * i + 1], sh = s[2 * i + 1];
        // first half: x1*cos - x2*sin; second half: x2*cos + x1*sin
        const uint16_t y1l = f32_to_bf16(fmaf(x1l, cl, -x2l * sl));
        const uint16_t y1h = f32_to_bf16(fmaf(x1h, ch, -x2h * sh));
        const uint16_t y2l = f32_to_bf16(fmaf(x2l, cl, x1l * sl));
        const uint16_t y2h = f32_to_bf16(fmaf(x2h, ch, x1h * sh));
        ra[i] = (uint32_t)y1l | ((uint32_t)y1h << 16);
        rb[i] = (uint32_t)y2l | ((uint32_t)y2h << 16);
    }
    ya = make_uint4(ra[0], ra[1], ra[2], ra[3]);
    yb = make_uint4(rb[0], rb[1], rb[2], rb[3]);
}

// cos and sin of an fp32 angle, evaluated in fp64 and rounded once to fp32.
// Cody-Waite reduction x = k*pi/2 + r with pi/2 split in two doubles (hi
// = pi/2 rounded to double, lo = the remainder), each product subtracted
// by one fma: for |k| < 2^31 the dropped third term stays below 2^-70, far
// under half an fp32 ulp.  On |r| <= pi/4 the Taylor series of sin and cos
// to degree 17 / 18 leave errors below 2^-60; the quadrant k mod 4 picks
// signs and swaps the two.  The Horner factors 1/((n-1) n) are constants
// rounded once to double at compile time (a multiply, not a divide, per
// term: the whole evaluation is a short chain of fp64 fmas).
struct SinCosReduced {
    double r, r2;
    long q;
};
__host__ __device__ __forceinline__ SinCosReduced sincos_reduce(float angle) {
    constexpr double kPio2Hi = 1.5707963267948966;       // pi/2 rounded to double
    constexpr double kPio2Lo = 6.123233995736766e-17;    // pi/2 - kPio2Hi
    constexpr double k2OverPi = 0.63661977236758134;
    const double x = (double)angle;
    const double k = rint(x * k2OverPi);
    SinCosReduced red;
    red.r = fma(-k, kPio2Lo, fma(-k, kPio2Hi, x));
    red.r2 = red.r * red.r;
    red.q = (long)k & 3;
    return red;
}
__host__ __device__ __forceinline__ void sincos_finish(const SinCosReduced &red, double ps, double pc, float *c,
                                              float *s) {
    const double sv = red.r * ps, cv = pc;
    const long q = red.q;
    const double so = q == 0 ? sv : q == 1 ? cv : q == 2 ? -sv : -cv;
    const double co = q == 0 ? cv : q == 1 ? -sv : q == 2 ? -cv : sv;
    *c = (float)co;
    *s = (float)so;
}
__host__ __device__ __forceinline__ void sincos_angle(float angle, float *c, float *s) {
    const SinCosReduced red = sincos_reduce(angle);
    // sin r = r (1 - r^2/3! (1 - r^2/(4*5) (1 - ...))), cos likewise, Horner
    double ps = 1.0, pc = 1.0;
#pragma unroll
    for (int n = 17; n >= 3; n -= 2) ps = fma(-red.r2 * (1.0 / (double)((n - 1) * n)), ps, 1.0);
#pragma unroll
    for (int n = 18; n >= 2; n -= 2) pc = fma(-red.r2 * (1.0 / (double)((n - 1) * n)), pc, 1.0);
    sincos_finish(red, ps, pc, c, s);
}
// Factor of the per-head output gate: the logistic sigmoid of its logit
// (Spark export page, `_Layer.forward`: sigmoid of g_proj, one value per
// query head, multiplying that head's attention output).
__device__ __forceinline__ float gate_factor(float logit) { return 1.f / (1.f + expf(-logit)); }

// Wave64 reductions via butterfly shuffles.
__device__ __forceinline__ float wave_max(float v) { return wave_max64(v); }
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}


// ---------------------------------------------------------------- LDS tiles
// Stands in for the row of a key without one (a zero weight would not
// cancel a NaN that the row it replaces might hold); 576 bf16, the longest
// row any kernel reads.
static __device__ __align__(16) const uint16_t g_zero_row[576] = {};

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes a lane from src to LDS at dst + 16 lane (dst wave-uniform), with
// global_load_lds_dwordx4.  Written in asm so that the compiler, which
// cannot tell tile buffers apart behind a computed address, does not wait
// for every such load before each LDS read; the waits on these loads are
// the callers' explicit vmcnt waits, so a caller issues no other vector
// memory loads between them.  No register receives data.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; the clobber still orders it
__device__ __forceinline__ void load_to_lds(const void *src, unsigned char *dst) {
    // the LDS aperture is 4 GiB aligned: a shared pointer's low word is its LDS address
    const uint32_t m0 = (uint32_t)(uintptr_t)dst;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(src) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt immediate for vmcnt(n) alone (expcnt and lgkmcnt at their
// maxima): vmcnt's low four bits at [3:0], its high two at [15:14].
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// A workgroup barrier without the memory fences __syncthreads() brings
// (those wait for every outstanding load); the compiler may not move memory
// accesses across it.
__device__ __forceinline__ void raw_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace hda
