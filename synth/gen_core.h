/* Counter-based synthetic input generator, shared by the host filler (gen_cpu.c, g++/gcc)
 * and the device filler (gen_gpu.hip, hipcc for gfx950).
 *
 * Test and benchmark infrastructure only. It draws numbers and holds none of the
 * attention method's arithmetic.
 *
 * Every value is a pure function of (seed, tensor id, element index), so any sub-range of
 * any tensor can be regenerated on its own, on the host or on the device, with identical bits:
 *  - the hash is SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *    generators", OOPSLA 2014; constants as in Vigna's public splitmix64.c), integer only;
 *  - normals use the Box-Muller transform (Box and Muller, 1958) evaluated with IEEE-754 double
 *    add, subtract, multiply and divide only, in a fixed order. Both targets round those
 *    operations to nearest-even, and both builds pass -ffp-contract=off so nothing is fused;
 *  - log, square root, sine and cosine are computed below from their series or from Newton's
 *    iteration, never taken from a math library whose last bit could differ between targets.
 */
#ifndef SYNTH_GEN_CORE_H
#define SYNTH_GEN_CORE_H

#include <stdint.h>

#if defined(__HIPCC__)
#define SYN_FN __host__ __device__ static inline
#else
#define SYN_FN static inline
#endif

#define SYN_GAMMA 0x9E3779B97F4A7C15ULL

SYN_FN uint64_t syn_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* State of the SplitMix64 stream for one tensor: the (tensor+1)-th output of a SplitMix64
 * generator whose state starts from the first output of one seeded with `seed`. */
SYN_FN uint64_t syn_stream(uint64_t seed, uint64_t tensor) {
  uint64_t s1 = syn_mix64(seed + SYN_GAMMA);
  return syn_mix64(s1 + (tensor + 1) * SYN_GAMMA);
}

/* The i-th 64-bit output of SplitMix64 seeded with `stream`. */
SYN_FN uint64_t syn_bits(uint64_t stream, uint64_t i) {
  return syn_mix64(stream + (i + 1) * SYN_GAMMA);
}

SYN_FN double syn_u64_as_f64(uint64_t b) { double d; __builtin_memcpy(&d, &b, 8); return d; }
SYN_FN uint64_t syn_f64_as_u64(double d) { uint64_t b; __builtin_memcpy(&b, &d, 8); return b; }
SYN_FN uint32_t syn_f32_as_u32(float f) { uint32_t b; __builtin_memcpy(&b, &f, 4); return b; }
SYN_FN float syn_u32_as_f32(uint32_t b) { float f; __builtin_memcpy(&f, &b, 4); return f; }

/* Natural log of a normal double x in (0, 1]. x = 2^e * m with m in [sqrt(1/2), sqrt(2));
 * log(m) = 2*atanh(s), s = (m-1)/(m+1), |s| < 0.172, series to s^21 (error < 1e-17). */
SYN_FN double syn_log(double x) {
  uint64_t b = syn_f64_as_u64(x);
  int e = (int)((b >> 52) & 0x7FF) - 1023;
  double m = syn_u64_as_f64((b & 0x000FFFFFFFFFFFFFULL) | 0x3FF0000000000000ULL);
  if (m > 1.4142135623730951) { m = m * 0.5; e = e + 1; }
  double f = m - 1.0;
  double s = f / (f + 2.0);
  double s2 = s * s;
  double p = 0.047619047619047616;            /* 1/21 */
  p = p * s2 + 0.05263157894736842;           /* 1/19 */
  p = p * s2 + 0.058823529411764705;          /* 1/17 */
  p = p * s2 + 0.06666666666666667;           /* 1/15 */
  p = p * s2 + 0.07692307692307693;           /* 1/13 */
  p = p * s2 + 0.09090909090909091;           /* 1/11 */
  p = p * s2 + 0.1111111111111111;            /* 1/9 */
  p = p * s2 + 0.14285714285714285;           /* 1/7 */
  p = p * s2 + 0.2;                           /* 1/5 */
  p = p * s2 + 0.3333333333333333;            /* 1/3 */
  p = p * s2 + 1.0;
  double ls = s * p;
  ls = ls * 2.0;
  double le = (double)e * 0.6931471805599453;
  return le + ls;
}

/* Square root of x >= 0 by Newton's iteration on 1/sqrt(x) (multiply and subtract only). */
SYN_FN double syn_sqrt(double x) {
  if (x == 0.0) return 0.0;
  double y = syn_u64_as_f64(0x5FE6EB50C7B537A9ULL - (syn_f64_as_u64(x) >> 1));
  double h = 0.5 * x;
  for (int it = 0; it < 5; ++it) {
    double t = h * y;
    t = t * y;
    t = 1.5 - t;
    y = y * t;
  }
  return x * y;
}

/* cos and sin of theta in [0, pi/2) by their Taylor series to the theta^23 term. */
SYN_FN void syn_cos_sin(double th, double* c, double* s) {
  double t2 = th * th;
  double pc = -8.896791392450574e-22;
  pc = pc * t2 + 4.110317623312165e-19;
  pc = pc * t2 + -1.5619206968586225e-16;
  pc = pc * t2 + 4.779477332387385e-14;
  pc = pc * t2 + -1.1470745597729725e-11;
  pc = pc * t2 + 2.08767569878681e-09;
  pc = pc * t2 + -2.755731922398589e-07;
  pc = pc * t2 + 2.48015873015873e-05;
  pc = pc * t2 + -0.001388888888888889;
  pc = pc * t2 + 0.041666666666666664;
  pc = pc * t2 + -0.5;
  pc = pc * t2 + 1.0;
  double ps = -3.868170170630684e-23;
  ps = ps * t2 + 1.9572941063391263e-20;
  ps = ps * t2 + -8.22063524662433e-18;
  ps = ps * t2 + 2.8114572543455206e-15;
  ps = ps * t2 + -7.647163731819816e-13;
  ps = ps * t2 + 1.6059043836821613e-10;
  ps = ps * t2 + -2.505210838544172e-08;
  ps = ps * t2 + 2.7557319223985893e-06;
  ps = ps * t2 + -0.0001984126984126984;
  ps = ps * t2 + 0.008333333333333333;
  ps = ps * t2 + -0.16666666666666666;
  ps = ps * t2 + 1.0;
  *c = pc;
  *s = ps * th;
}

/* Standard normal number i of a stream: Box-Muller on the pair of uniforms (2p, 2p+1),
 * p = i/2; even i takes the cosine branch, odd i the sine branch. */
SYN_FN double syn_normal(uint64_t stream, uint64_t i) {
  uint64_t p = i >> 1;
  uint64_t a = syn_bits(stream, 2 * p) >> 11;      /* 53 bits */
  uint64_t b = syn_bits(stream, 2 * p + 1) >> 11;  /* 53 bits */
  double x = (double)((1ULL << 53) - a) * 1.1102230246251565e-16;  /* (0, 1], times 2^-53 */
  double l = syn_log(x);
  double r = syn_sqrt(-2.0 * l);
  uint64_t quadrant = b >> 51;
  double frac = (double)(b & ((1ULL << 51) - 1)) * 4.440892098500626e-16;  /* times 2^-51 */
  double th = frac * 1.5707963267948966;
  double c, s;
  syn_cos_sin(th, &c, &s);
  double cx, sx;
  if (quadrant == 0)      { cx = c;  sx = s;  }
  else if (quadrant == 1) { cx = -s; sx = c;  }
  else if (quadrant == 2) { cx = -c; sx = -s; }
  else                    { cx = s;  sx = -c; }
  return (i & 1) ? r * sx : r * cx;
}

/* Round an fp32 value to the nearest bfloat16, ties to even; returns the bf16 bits. */
SYN_FN uint16_t syn_f32_to_bf16(float f) {
  uint32_t u = syn_f32_as_u32(f);
  u = u + 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
SYN_FN float syn_bf16_to_f32(uint16_t h) { return syn_u32_as_f32(((uint32_t)h) << 16); }

/* One element of N(mean, std^2), rounded to fp32. */
SYN_FN float syn_normal_f32(uint64_t stream, uint64_t i, double mean, double stdv) {
  double z = syn_normal(stream, i);
  double v = z * stdv;
  v = v + mean;
  return (float)v;
}

/* One element of U[lo, hi), 24 random bits, rounded to fp32. */
SYN_FN float syn_uniform_f32(uint64_t stream, uint64_t i, double lo, double hi) {
  uint64_t u = syn_bits(stream, i) >> 40;
  double f = (double)u * 5.9604644775390625e-08;   /* times 2^-24 */
  double w = hi - lo;
  double v = w * f;
  v = v + lo;
  return (float)v;
}

/* Row `row` of the index-key tensor: noise N(0,1) plus alpha * sum_s A[row,s] * U[s,:], where
 * A[row,s] ~ N(0,1) comes from its own stream and U holds `nspike` basis rows of length dim. */
SYN_FN float syn_index_key(uint64_t s_noise, uint64_t s_load, uint64_t row, uint32_t t,
                           uint32_t dim, uint32_t nspike, const double* U, double alpha) {
  double acc = 0.0;
  for (uint32_t s = 0; s < nspike; ++s) {
    double a = syn_normal(s_load, row * nspike + s);
    double au = a * U[(uint64_t)s * dim + t];
    acc = acc + au;
  }
  double z = syn_normal(s_noise, row * dim + t);
  double sp = alpha * acc;
  double v = z + sp;
  return (float)v;
}

#endif /* SYNTH_GEN_CORE_H */
