/*
 * Exhaustive checks of two fp32 identities the packer's kernel relies on to reproduce the
 * quantiser of radiance_drafthead.py (_quantize_head_now: sc = (hi - lo) / 3, codes from w / sc)
 * with IEEE round-to-nearest-even results:
 *
 *  1. d / 3 for d >= 0 equals fma(fma(-q, 3, d), t, q) with t = RN(1/3), q = RN(d * t), for every
 *     non-negative finite fp32 d (subnormals included).
 *  2. a / b equals fma(fma(-b, q0, a), y, q0) with y = RN(1/b), q0 = RN(a * y), for every fp32
 *     significand of b and every bf16 significand of a. Signs and powers of two change none of
 *     the roundings while no intermediate overflows or underflows, so b in [1, 2) and a in [1, 2)
 *     cover every normal case.
 *
 *  3. The e4m3 decode of the FP8 weight source (radiance_drafthead.py, _rerank_exact: sign bit
 *     7, exponent field e = bits 3-6, mantissa m = bits 0-2, value m * 2^-9 for e = 0 else
 *     (1 + m/8) * 2^(e - 7)) equals the fp32 whose bits are (b & 0x7F) << 20 | (b & 0x80) << 24
 *     times 2^120, for all 256 codes.
 *
 * The references are IEEE division in fp32 (1) and fp64 division rounded to fp32 (2); the
 * latter is exact here because a / b (an 8-bit by 24-bit quotient) never lies within 2^-49 of
 * an fp32 rounding midpoint. Build: cc -O2 -ffp-contract=off [-fopenmp] pack_arith_check.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

int main(void) {
  const float third = 1.0f / 3.0f;
  unsigned long long bad_div3 = 0, n_div3 = 0;
#pragma omp parallel for reduction(+ : bad_div3, n_div3) schedule(static, 65536)
  for (long long b = 0; b <= 0x7F7FFFFFll; ++b) {
    const float d = from_bits((uint32_t)b);
    volatile float ref = d / 3.0f;
    const float q = d * third;
    const float got = fmaf(fmaf(-q, 3.0f, d), third, q);
    bad_div3 += got != ref;
    ++n_div3;
  }
  unsigned long long bad_quot = 0, n_quot = 0;
#pragma omp parallel for reduction(+ : bad_quot, n_quot) schedule(static, 4096)
  for (long long m = 0; m < (1ll << 23); ++m) {
    const float b = from_bits(0x3F800000u | (uint32_t)m);
    const float y = 1.0f / b;
    for (uint32_t am = 0; am < 128; ++am) {
      const float a = from_bits(0x3F800000u | (am << 16));
      const float q0 = a * y;
      const float got = fmaf(fmaf(-b, q0, a), y, q0);
      const float ref = (float)((double)a / (double)b);
      bad_quot += got != ref;
      ++n_quot;
    }
  }
  unsigned bad_fp8 = 0;
  for (uint32_t b = 0; b < 256; ++b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    const double mag = e == 0 ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, (int)e - 7);
    const double ref = (b & 0x80u) ? -mag : mag;
    const float got = from_bits(((b & 0x7fu) << 20) | ((b & 0x80u) << 24)) * 0x1p120f;
    bad_fp8 += (double)got != ref;
  }
  printf("fp8 checked 256 mismatches %u\n", bad_fp8);
  printf("div3 checked %llu mismatches %llu\n", n_div3, bad_div3);
  printf("quot checked %llu mismatches %llu\n", n_quot, bad_quot);
  return (bad_fp8 || bad_div3 || bad_quot || n_div3 != 0x7F800000ull || n_quot != (128ull << 23)) ? 1 : 0;
}
