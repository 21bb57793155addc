// trig.h -- sine and cosine of an f32 RoPE angle ("Chapter 14 - QK-norm and
// RoPE" 14.5: the angle is f32(p) * theta_i in f32, and its sin and cos are
// taken accurately), from plain double arithmetic with no table in memory.
//
// The angle, exact in double, is reduced by pi/2 with a three-part constant
// and fused multiply-adds (the additive reduction of Cody and Waite, "Software
// Manual for the Elementary Functions", 1980).  sin and cos of the remainder r
// (|r| <= pi/4 plus rounding) come from their Taylor series to degree 17 and
// 16, whose first omitted terms are below 1e-17, and each result is rounded
// once to f32.  The quotient's quadrant selects and signs the two.  Valid for
// |angle| < 2^30.  Compiled for the GPU and, for its own test, by a host
// compiler.
#pragma once

#if defined(__HIPCC__)
#define MUSE_TRIG_FN __host__ __device__ __forceinline__
#else
#define MUSE_TRIG_FN inline
#endif

namespace muse {

MUSE_TRIG_FN void sincos_rope(float angle, float* sin_out, float* cos_out) {
    constexpr double kTwoOverPi = 0.6366197723675814;
    constexpr double kPio2Hi = 0x1.921fb54442d18p+0;     // pi/2 = hi + mid + lo to about 160 bits
    constexpr double kPio2Mid = 0x1.1a62633145c07p-54;
    constexpr double kPio2Lo = -0x1.f1976b7ed8fbcp-110;
    const double x = angle;
    const double k = __builtin_rint(x * kTwoOverPi);
    double r = __builtin_fma(-k, kPio2Hi, x);
    r = __builtin_fma(-k, kPio2Mid, r);
    r = __builtin_fma(-k, kPio2Lo, r);
    const double r2 = r * r;
    // sin r = r (1 - r2/3! + r2^2/5! - ... + r2^8/17!), Horner in r2
    double sp = 1.0 / 355687428096000.0;                 // 17!
    sp = __builtin_fma(sp, r2, -1.0 / 1307674368000.0);  // 15!
    sp = __builtin_fma(sp, r2, 1.0 / 6227020800.0);      // 13!
    sp = __builtin_fma(sp, r2, -1.0 / 39916800.0);       // 11!
    sp = __builtin_fma(sp, r2, 1.0 / 362880.0);          // 9!
    sp = __builtin_fma(sp, r2, -1.0 / 5040.0);           // 7!
    sp = __builtin_fma(sp, r2, 1.0 / 120.0);             // 5!
    sp = __builtin_fma(sp, r2, -1.0 / 6.0);              // 3!
    sp = __builtin_fma(sp, r2, 1.0);
    const double s_r = r * sp;
    // cos r = 1 - r2/2! + r2^2/4! - ... + r2^8/16!
    double cp = 1.0 / 20922789888000.0;                  // 16!
    cp = __builtin_fma(cp, r2, -1.0 / 87178291200.0);    // 14!
    cp = __builtin_fma(cp, r2, 1.0 / 479001600.0);       // 12!
    cp = __builtin_fma(cp, r2, -1.0 / 3628800.0);        // 10!
    cp = __builtin_fma(cp, r2, 1.0 / 40320.0);           // 8!
    cp = __builtin_fma(cp, r2, -1.0 / 720.0);            // 6!
    cp = __builtin_fma(cp, r2, 1.0 / 24.0);              // 4!
    cp = __builtin_fma(cp, r2, -0.5);                    // 2!
    const double c_r = __builtin_fma(cp, r2, 1.0);
    // angle = k pi/2 + r: rotate (sin r, cos r) by the quadrant k mod 4
    const int q = (int)((long long)k & 3);
    const double s = (q & 1) ? c_r : s_r;
    const double c = (q & 1) ? s_r : c_r;
    *sin_out = (float)((q & 2) ? -s : s);
    *cos_out = (float)(((q + 1) & 2) ? -c : c);
}

}  // namespace muse
