// Host-side check of the kernels' cos/sin evaluation (sincos_angle in the
// library's device header, compiled here for the CPU): for every angle the
// kernels form -- fp32 position times fp32 frequency for both RoPE
// configurations of the Spark export page (rotary dim 256 with theta 1e4,
// rotary dim 64 with theta 5e6), positions 0 .. 40000 -- and for random fp32
// angles up to 2^31, the fp32 results must equal libm's fp64 cos / sin of
// the same fp32 angle rounded once to fp32.  Prints one line per set and
// exits 1 on any mismatch.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>

#include "hda_device.h"

static long check_config(double theta, int rot, int max_pos) {
    long bad = 0, n = 0;
    for (int i = 0; i < rot / 2; ++i) {
        const float freq = (float)(1.0 / std::pow(theta, (double)(2 * i) / (double)rot));
        for (int pos = 0; pos <= max_pos; ++pos) {
            const float a = (float)pos * freq;
            float c, s;
            hda::sincos_angle(a, &c, &s);
            const float cr = (float)std::cos((double)a), sr = (float)std::sin((double)a);
            if (c != cr || s != sr) {
                if (bad < 5) std::printf("  mismatch angle %.9g: %.9g %.9g vs %.9g %.9g\n", a, c, s, cr, sr);
                ++bad;
            }
            ++n;
        }
    }
    std::printf("rot %d theta %g positions 0..%d: %ld angles, %ld mismatches\n", rot, theta, max_pos, n, bad);
    return bad;
}

static long check_random(long count) {
    std::mt19937_64 g(12345);
    std::uniform_real_distribution<double> u(-2147483648.0, 2147483648.0);
    long bad = 0;
    for (long k = 0; k < count; ++k) {
        const float a = (float)u(g);
        float c, s;
        hda::sincos_angle(a, &c, &s);
        if (c != (float)std::cos((double)a) || s != (float)std::sin((double)a)) ++bad;
    }
    std::printf("random |angle| < 2^31: %ld angles, %ld mismatches\n", count, bad);
    return bad;
}

int main() {
    long bad = check_config(1e4, 256, 40000) + check_config(5e6, 64, 40000) + check_random(1000000);
    return bad ? 1 : 0;
}
