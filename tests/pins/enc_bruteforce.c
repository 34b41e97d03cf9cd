/*
 * Exhaustive pin of the oracle's scalar encoders (test-only program).
 *
 * For every finite fp32 bit pattern it compares the oracle's encoder with a
 * brute-force reference written here from the format definitions alone: the
 * list of representable values, a nearest-value search, ties to the code with
 * an even mantissa (lowest code bit 0), and saturation at the largest finite
 * value.  It shares nothing with the oracle beyond calling it.
 *
 *   OCP FP4 E2M1: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}
 *   OCP FP8 E4M3: bias 7, 3 mantissa bits, max 448, S.1111.111 = NaN
 *   E8M0 MX scale: 2^(e+2) <= amax < 2^(e+3) unless clamped to [-127, 127]
 *   INT8: nearest integer (ties to even) of the fp32 product x*inv, in +-127
 *
 * Usage: enc_bruteforce <which> <stride>; prints "<which> <checked> <mismatches>".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint8_t orc_e4m3_encode(double x);
uint8_t orc_e2m1_encode(double x);
int orc_e8m0_exponent(float amax);
int8_t orc_i8_encode(float x, float inv);

static float as_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* value tables: index = magnitude code (sign bit excluded) */
static double e2m1_tab[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
static double e4m3_tab[127];  /* codes 0..126 (127 = NaN) */

static void build_e4m3(void) {
    for (int c = 0; c < 127; ++c) {
        int e = c >> 3, m = c & 7;
        e4m3_tab[c] = e == 0 ? (m / 8.0) * pow(2.0, -6) : (1.0 + m / 8.0) * pow(2.0, e - 7);
    }
}

/* nearest magnitude code in an ascending table; ties to the even code */
static int nearest(const double* tab, int n, double a) {
    if (a >= tab[n - 1]) return n - 1;      /* saturation */
    int lo = 0, hi = n - 1;                 /* invariant: tab[lo] <= a < tab[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (tab[mid] <= a) lo = mid; else hi = mid;
    }
    double dl = a - tab[lo], dh = tab[hi] - a;
    if (dl < dh) return lo;
    if (dh < dl) return hi;
    return (lo & 1) == 0 ? lo : hi;
}

int main(int argc, char** argv) {
    const char* which = argv[1];
    uint64_t stride = argc > 2 ? strtoull(argv[2], 0, 10) : 1;
    build_e4m3();
    uint64_t checked = 0, bad = 0;
#pragma omp parallel for reduction(+ : checked, bad) schedule(static, 65536)
    for (int64_t k = 0; k < (int64_t)(1ull << 32); k += (int64_t)stride) {
        uint32_t u = (uint32_t)k;
        float x = as_float(u);
        if (!isfinite(x)) continue;
        int neg = (u >> 31) & 1;
        double a = fabs((double)x);
        checked++;
        if (!strcmp(which, "e2m1")) {
            int want = nearest(e2m1_tab, 8, a) | (neg << 3);
            if (orc_e2m1_encode((double)x) != want) bad++;
        } else if (!strcmp(which, "e4m3")) {
            int want = nearest(e4m3_tab, 127, a) | (neg << 7);
            if (orc_e4m3_encode((double)x) != want) bad++;
        } else if (!strcmp(which, "e8m0")) {
            if (x <= 0.0f) { checked--; continue; }
            int e = orc_e8m0_exponent(x);
            int ok;
            if (e == -127) ok = a < ldexp(1.0, -127 + 3);
            else if (e == 127) ok = a >= ldexp(1.0, 127 + 2);
            else ok = ldexp(1.0, e + 2) <= a && a < ldexp(1.0, e + 3);
            if (!ok) bad++;
        } else if (!strcmp(which, "i8")) {
            /* a few inverse scales per input; the product is exact in fp64 */
            static const float invs[4] = {1.0f, 127.0f / 3.7f, 0.0312f, 5.5e-3f};
            for (int t = 0; t < 4; ++t) {
                float p = (float)((double)x * (double)invs[t]);    /* correctly rounded fp32 product */
                double fl = floor((double)p), want;
                double fr = (double)p - fl;
                if (fr > 0.5) want = fl + 1; else if (fr < 0.5) want = fl;
                else want = fmod(fl, 2.0) == 0.0 ? fl : fl + 1;   /* tie: even integer */
                if (want > 127) want = 127;
                if (want < -127) want = -127;
                if (isinf(p)) want = p > 0 ? 127 : -127;
                if (orc_i8_encode(x, invs[t]) != (int8_t)want) bad++;
            }
        }
    }
    printf("%s %llu %llu\n", which, (unsigned long long)checked, (unsigned long long)bad);
    return 0;
}
