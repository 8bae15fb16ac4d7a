// Host check of the NVFP4-style quotient sequence (csrc/nv_div.h) against
// IEEE division, bit for bit (sign of zero included). Built with g++
// -ffp-contract=off by tests/test_nv_div_cpu.py; the HIP function qualifiers
// are defined away, so the header's code is compiled as it stands.
//
// Cases, for every d = fl(dec(S) sg) with S each positive finite E4M3 code
// and sg from a set of tensor scales (random over 2^-60 .. 2^40, plus
// fl(A / 2688) for random amaxes A), keeping d where the sequence applies:
//   * x = +-0, and signed subnormals;
//   * x within a few ulps of q d for q each E2M1 decision point and grid
//     value (the quotients that decide a code);
//   * x uniform in (-6.5 d, 6.5 d) and log-uniform down to 2^-30 d.
// Where |x / d| >= 2^-3 the quotient must equal IEEE division bit for bit;
// everywhere its E2M1 code (sign included) must equal that of the IEEE
// quotient. Below 2^-3 a subnormal x can make the remainder x - d q
// underflow, and the last bits may then differ (counted, not an error: the
// code is a signed zero either way). Prints "cases N mismatches M
// code_mismatches C below_2^-3_differing L" and the first mismatches.
#define __host__
#define __device__
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>

#include "nv_div.h"

#ifdef PLANT_NO_CORRECTION  // a broken variant (the plain product x y): must be caught
static float quot(float x, float d, float y) { return __builtin_copysignf(x * y, x); }
#else
static float quot(float x, float d, float y) { return fp4r::nv_div(x, d, y); }
#endif

static uint32_t bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
static float from_bits(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }

// Signed E2M1 code (nearest, ties to the even code, saturating): the
// decision the quotient feeds.
static int code(float q) {
  const float a = std::fabs(q);
  const int m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return (std::signbit(q) ? 8 : 0) | m;
}

static float e4m3(int S) {
  const int e = S >> 3, m = S & 7;
  return e == 0 ? (float)m * 0x1p-9f : std::ldexp((float)(8 + m), e - 10);
}

int main(int argc, char** argv) {
  const int n_sg = argc > 1 ? std::atoi(argv[1]) : 400;
  std::mt19937_64 rng(12345);
  std::uniform_real_distribution<double> uni(0.0, 1.0);
  long long cases = 0, bad = 0, bad_code = 0, low_diff = 0;
  auto check = [&](float x, float d, float y) {
    const float want = x / d, got = quot(x, d, y);
    ++cases;
    if (code(want) != code(got)) {
      if (bad_code < 5) std::printf("code mismatch x=%a d=%a want=%a got=%a\n", x, d, want, got);
      ++bad_code;
    }
    if (bits(want) != bits(got)) {
      if (std::fabs(want) < 0.125f) {
        ++low_diff;  // below 2^-3: the code is a signed zero whatever the last bits
      } else {
        if (bad < 5) std::printf("mismatch x=%a d=%a want=%a got=%a\n", x, d, want, got);
        ++bad;
      }
    }
  };
  const float qs[] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  for (int i = 0; i < n_sg; ++i) {
    float sg;
    if (i % 2 == 0) sg = (float)std::ldexp(1.0 + uni(rng), (int)(uni(rng) * 100) - 60);
    else sg = (float)std::ldexp(1.0 + uni(rng), (int)(uni(rng) * 80) - 40) / 2688.0f;
    for (int S = 1; S <= 0x7E; ++S) {
      const float d = e4m3(S) * sg;
      const float y = 1.0f / d;
      if (!fp4r::nv_div_applies(d, 6.5f * d, y)) continue;
      check(0.0f, d, y);
      check(-0.0f, d, y);
      for (int j = 0; j < 8; ++j) {
        const float s = from_bits((uint32_t)(rng() % 0x007FFFFF) + 1u);
        check(s, d, y);
        check(-s, d, y);
      }
      for (float q : qs) {
        const float c = q * d;
        for (int u = -4; u <= 4; ++u) {
          const float x = from_bits(bits(c) + (uint32_t)u);
          check(x, d, y);
          check(-x, d, y);
        }
      }
      for (int j = 0; j < 64; ++j) {
        check((float)((2.0 * uni(rng) - 1.0) * 6.5) * d, d, y);
        check((float)std::ldexp(1.0 + uni(rng), -(int)(uni(rng) * 30)) * d, d, y);
      }
    }
  }
  std::printf("cases %lld mismatches %lld code_mismatches %lld below_2^-3_differing %lld\n", cases, bad, bad_code,
              low_diff);
  return 0;
}
