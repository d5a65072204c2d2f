// Correctly rounded float32 logistic sigmoid, for the STS calibration
// c = sigmoid(z / T) of "DSpark 自适应 Verify 怎样分配候选预算" (akiyangdev),
// §二 (runtime STS formula).
//
// The result is the float32 nearest to the real 1 / (1 + e^-x) (ties to
// even). It depends only on x, so every device and the CPU reference produce
// the same bits. That matters because the survival values built from it
// decide the integer verify lengths.
//
// Method (Ziv's two-step strategy):
//   1. Fast path in fp64. Cody-Waite reduction t = n ln2 + r, |r| <= ln2/2,
//      with ln2 split as L1 (32 significant bits, so n*L1 and t - n*L1 are
//      exact) + L2. Then e^r by its Taylor series to degree 13 in Horner form
//      with fused multiply-adds (truncation < 2^-57), scaled by 2^n. Then
//      y = 1 / (1 + e^t) with t = -x. The relative error of y is below 2^-50.
//      If y(1 - 2^-45) and y(1 + 2^-45) round to the same float32, that
//      float32 is the correctly rounded result.
//   2. Otherwise (probability about 2^-20 per input): the same steps in
//      double-double arithmetic (Dekker's exact products via fma, Knuth's
//      two-sum), with ln2 split into three parts and the Taylor series to
//      degree 24. That is about 100 correct bits. The double-double value is
//      rounded to float32 with explicit midpoint handling.
//
// Constants, derived from the mathematics at 80 decimal digits:
//   L1 = ln2 truncated to 32 significant bits, L2 = RN64(ln2 - L1),
//   L3 = RN64(ln2 - L1 - L2); C_k = RN64(1/k!).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

#define DSPARK_HD __host__ __device__ inline

struct DD {
  double hi, lo;
};

DSPARK_HD DD two_sum(double a, double b) {
#pragma clang fp contract(off)
  double s = a + b;
  double bb = s - a;
  double err = (a - (s - bb)) + (b - bb);
  return {s, err};
}

DSPARK_HD DD fast_two_sum(double a, double b) {  // requires |a| >= |b|
#pragma clang fp contract(off)
  double s = a + b;
  return {s, b - (s - a)};
}

DSPARK_HD DD two_prod(double a, double b) {
#pragma clang fp contract(off)
  double p = a * b;
  return {p, __builtin_fma(a, b, -p)};
}

DSPARK_HD DD dd_add(DD x, DD y) {
#pragma clang fp contract(off)
  DD s = two_sum(x.hi, y.hi);
  DD t = two_sum(x.lo, y.lo);
  s.lo += t.hi;
  s = fast_two_sum(s.hi, s.lo);
  s.lo += t.lo;
  return fast_two_sum(s.hi, s.lo);
}

DSPARK_HD DD dd_mul(DD x, DD y) {
#pragma clang fp contract(off)
  DD p = two_prod(x.hi, y.hi);
  p.lo += x.hi * y.lo + x.lo * y.hi;
  return fast_two_sum(p.hi, p.lo);
}

DSPARK_HD DD dd_div_d(DD x, double d) {  // x / d, d a small exact integer here
#pragma clang fp contract(off)
  double q1 = x.hi / d;
  DD p = two_prod(q1, d);
  DD r = dd_add(x, DD{-p.hi, -p.lo});
  double q2 = r.hi / d;
  return fast_two_sum(q1, q2);
}

constexpr double kLn2_1 = 0x1.62e42fee00000p-1;
constexpr double kLn2_2 = 0x1.a39ef35793c76p-33;
constexpr double kLn2_3 = 0x1.cc01f97b57a08p-87;
constexpr double kLog2e = 0x1.71547652b82fep+0;
constexpr double kBand = 0x1p-45;

// A coefficient passed through a scalar register pair on the device: the
// three-operand v_fma_f64 takes no 64-bit literal, and a literal addend costs
// two v_mov_b32 ahead of a v_fmac_f64 per Horner step; from a scalar pair the
// step is one v_fma_f64. The value is unchanged.
__host__ inline double scalar_const(double c) { return c; }
__device__ inline double scalar_const(double c) {
  asm volatile("" : "+s"(c));
  return c;
}

// On the device, a point the instruction scheduler does not move code across:
// it keeps the steps of several interleaved dependency chains together (the
// scheduler would otherwise run the chains one after the other).
__host__ inline void sched_fence() {}
__device__ inline void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// e^t for |t| < 120 in fp64, relative error < 2^-50, for N independent
// arguments: each step is taken for all N before the next, so that their
// dependency chains interleave. Every argument gets the same operations.
template <int N>
DSPARK_HD void exp_fast_n(const double (&t)[N], double (&out)[N]) {
#pragma clang fp contract(off)
  double n[N], r[N], p[N];
  for (int i = 0; i < N; ++i) n[i] = __builtin_rint(t[i] * kLog2e);
  for (int i = 0; i < N; ++i) r[i] = t[i] - n[i] * kLn2_1;                // exact
  for (int i = 0; i < N; ++i) r[i] = __builtin_fma(-n[i], kLn2_2, r[i]);  // one rounding
  for (int i = 0; i < N; ++i) p[i] = 0x1.6124613a86d09p-33;                // 1/13!
  const double c[11] = {
      scalar_const(0x1.1eed8eff8d898p-29),  // 1/12!
      scalar_const(0x1.ae64567f544e4p-26),  // 1/11!
      scalar_const(0x1.27e4fb7789f5cp-22),  // 1/10!
      scalar_const(0x1.71de3a556c734p-19),  // 1/9!
      scalar_const(0x1.a01a01a01a01ap-16),  // 1/8!
      scalar_const(0x1.a01a01a01a01ap-13),  // 1/7!
      scalar_const(0x1.6c16c16c16c17p-10),  // 1/6!
      scalar_const(0x1.1111111111111p-7),   // 1/5!
      scalar_const(0x1.5555555555555p-5),   // 1/4!
      scalar_const(0x1.5555555555555p-3),   // 1/3!
      0x1p-1,                               // 1/2!
  };
  for (int k = 0; k < 11; ++k) {
    for (int i = 0; i < N; ++i) p[i] = __builtin_fma(p[i], r[i], c[k]);
    if (N > 1) sched_fence();
  }
  for (int i = 0; i < N; ++i) p[i] = __builtin_fma(p[i], r[i], 1.0);
  if (N > 1) sched_fence();
  for (int i = 0; i < N; ++i) p[i] = __builtin_fma(p[i], r[i], 1.0);
  for (int i = 0; i < N; ++i) out[i] = __builtin_ldexp(p[i], (int)n[i]);
}

DSPARK_HD double exp_fast(double t) {
  const double a[1] = {t};
  double e[1];
  exp_fast_n<1>(a, e);
  return e[0];
}

// e^t for |t| < 120 in double-double, about 100 correct bits.
DSPARK_HD DD exp_dd(double t) {
#pragma clang fp contract(off)
  double n = __builtin_rint(t * kLog2e);
  double r1 = t - n * kLn2_1;  // exact
  DD np2 = two_prod(n, kLn2_2);
  DD r = dd_add(DD{r1, 0.0}, DD{-np2.hi, -np2.lo});
  r = dd_add(r, DD{-n * kLn2_3, 0.0});
  DD p{1.0, 0.0};
  for (int k = 24; k >= 1; --k) {
    p = dd_add(DD{1.0, 0.0}, dd_div_d(dd_mul(r, p), (double)k));
  }
  int e = (int)n;
  return DD{__builtin_ldexp(p.hi, e), __builtin_ldexp(p.lo, e)};
}

DSPARK_HD float f32_next_up(float f) {  // f >= 0
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  return __builtin_bit_cast(float, b + 1u);
}

DSPARK_HD float f32_next_down(float f) {  // f > 0
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  return __builtin_bit_cast(float, b - 1u);
}

// Nearest float32 to the positive real y.hi + y.lo (ties to even).
DSPARK_HD float dd_to_f32(DD y) {
#pragma clang fp contract(off)
  float f = (float)y.hi;
  double fd = (double)f;
  if (fd == y.hi) return f;  // |y.lo| <= ulp64/2 cannot move it off f
  float a = fd < y.hi ? f : f32_next_down(f);
  float b = fd < y.hi ? f32_next_up(f) : f;
  double mid = 0.5 * ((double)a + (double)b);  // exact: 25 significant bits
  if (y.hi != mid) return f;  // no float32 midpoint between y.hi and y.hi + y.lo
  if (y.lo > 0.0) return b;
  if (y.lo < 0.0) return a;
  return (__builtin_bit_cast(uint32_t, a) & 1u) ? b : a;
}

DSPARK_HD float sigmoid_slow(float x) {
#pragma clang fp contract(off)
  DD e = exp_dd(-(double)x);
  DD d = dd_add(DD{1.0, 0.0}, e);
  double y0 = 1.0 / d.hi;
  DD dy = two_prod(d.hi, y0);
  // residual 1 - d * y0 in double-double, then one Newton step
  DD res = dd_add(DD{1.0, 0.0}, DD{-dy.hi, -dy.lo});
  res = dd_add(res, DD{-d.lo * y0, 0.0});
  DD corr = two_prod(y0, res.hi);
  corr.lo += y0 * res.lo;
  DD y = dd_add(DD{y0, 0.0}, corr);
  return dd_to_f32(y);
}

// The fast path alone, branch-free, for N independent inputs: y[i], and
// through ok[i] whether it is the correctly rounded sigmoid (false: take
// sigmoid_slow). Inputs at or past the saturation points and NaN are settled
// by selects; the N exponentials interleave (exp_fast_n).
template <int N>
DSPARK_HD void sigmoid_fast_n(const float (&x)[N], float (&y)[N], bool (&ok)[N]) {
#pragma clang fp contract(off)
  double t[N], e[N];
  for (int i = 0; i < N; ++i) {
    // clamped into the fast path's range (NaN becomes -104); the selects
    // below settle every input that was clamped
    t[i] = -(double)__builtin_fminf(__builtin_fmaxf(x[i], -104.0f), 17.5f);
  }
  exp_fast_n<N>(t, e);
  for (int i = 0; i < N; ++i) {
    const double yd = 1.0 / (1.0 + e[i]);
    const float lo = (float)(yd * (1.0 - kBand));
    const float hi = (float)(yd * (1.0 + kBand));
    float r = lo;
    bool k = lo == hi;
    if (x[i] >= 17.5f) {  // 1 - sigmoid < e^-x < 2^-25: rounds to 1
      r = 1.0f;
      k = true;
    }
    if (x[i] <= -104.0f) {  // sigmoid < e^x < 2^-150: rounds to +0
      r = 0.0f;
      k = true;
    }
    if (x[i] != x[i]) {
      r = x[i];
      k = true;
    }
    y[i] = r;
    ok[i] = k;
  }
}

// Returns the correctly rounded sigmoid and, through *slow, whether the
// double-double path ran.
DSPARK_HD float sigmoid_cr(float x, bool* slow = nullptr) {
  const float xs[1] = {x};
  float r[1];
  bool ok[1];
  sigmoid_fast_n<1>(xs, r, ok);
  if (slow) *slow = !ok[0];
  return ok[0] ? r[0] : sigmoid_slow(x);
}

}  // namespace dspark
