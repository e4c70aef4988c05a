// Host-side check of the library's quotient routines (fp8q_common.hpp:
// div_rn_f64 with the reciprocals recip_or_one and recip_refine, and
// scale_div) against IEEE fp32 division, bit for bit.  The device runs the
// same arithmetic (fp64 multiply of the widened fp32 value, RNE narrowing to
// fp32, fp64 Newton steps), so agreement here shows the method, not just this
// compiler, is right.  The device seeds recip_refine with the hardware fp32
// reciprocal (within 1 ulp); here every seed from 4 ulp below to 4 ulp above
// RN32(1/s) is tried.
//
// Quotients y / s: for each scale s in a list (random, structured, range
// ends, subnormal), every fp32 y of several binades (all 2^23 significands),
// plus random y of any magnitude up to 449 s and beyond.  Scales amax / d for
// d = 448 and 127: every fp32 amax of several binades, random amax over the
// whole fp32 range, subnormals included.  Prints the number of mismatches.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "fp8q_common.hpp"

static float from_bits(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
static uint32_t bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }

static uint64_t checked = 0, bad = 0;

// Quotients below 2^-126 are only promised their sign and a magnitude below
// 2^-125 (all of them encode to signed zeros); every other one exactly.
static void check_quotient(float y, float s, double r) {
  const float want = y / s;
  const float got = fp8q::div_rn_f64(y, r);
  ++checked;
  bool ok;
  if (std::fabs(want) < 0x1p-126f)
    ok = std::signbit(want) == std::signbit(got) && std::fabs(got) < 0x1p-125f;
  else
    ok = bits(want) == bits(got);
  if (!ok) {
    if (bad < 10) std::printf("quotient mismatch y=%a s=%a want=%a got=%a\n", y, s, want, got);
    ++bad;
  }
}

static void check_scale(float amax) {
  const float pairs_d[2] = {448.0f, 127.0f};
  const double pairs_r[2] = {fp8q::kRecip448, fp8q::kRecip127};
  for (int k = 0; k < 2; ++k) {
    const float want = amax / pairs_d[k];
    const float got = fp8q::scale_div(amax, pairs_r[k], pairs_d[k]);
    ++checked;
    if (bits(want) != bits(got)) {
      if (bad < 10) std::printf("scale mismatch amax=%a d=%g want=%a got=%a\n", amax, pairs_d[k], want, got);
      ++bad;
    }
  }
}

int main(int argc, char** argv) {
  const int n_random_scales = argc > 1 ? std::atoi(argv[1]) : 24;
  std::mt19937_64 rng(12345);
  // the constants are the correctly rounded reciprocals
  if (fp8q::kRecip448 != 1.0 / 448.0 || fp8q::kRecip127 != 1.0 / 127.0) {
    std::printf("reciprocal constants wrong\n");
    return 1;
  }
  std::vector<float> scales = {1.0f, 13.0f / 448.0f, 0x1p-76f, 0x1.fffffep-76f, 0x1p-20f,
                               0x1.fffffep0f, 0x1.000002p0f, 3.0f, 0x1p100f, 0x1.8p119f,
                               1.0f / 448.0f, 7.0f, 0x1p-127f, 0x1.5p-140f, 0x1p-149f,
                               0x1.fffffep127f, 0x1.800002p-100f};
  std::uniform_real_distribution<double> ue(-149.0, 127.0);
  for (int i = 0; i < n_random_scales; ++i) {
    float s = std::exp2(static_cast<float>(ue(rng)));
    if (s >= 0x1p-126f) s = from_bits((bits(s) & 0xFF800000u) | (rng() & 0x7FFFFFu));
    scales.push_back(s);
  }
  for (float s : scales) {
    // the reciprocals the library may use for this s: the correctly rounded
    // one, and where the scale path refines a seed, every seed within 4 ulp
    std::vector<double> rs = {fp8q::recip_or_one(s)};
    const bool refined = s >= 0x1p-110f && s <= 0x1p120f;
    if (refined) {
      const uint32_t c = bits(1.0f / s);
      for (int k = -4; k <= 4; ++k) rs.push_back(fp8q::recip_refine(s, from_bits(c + k)));
    }
    const int es = std::ilogb(s);
    // exhaustive significands for y in three binades near the top of the
    // range, with the correctly rounded reciprocal and the extreme seeds
    for (int de = 6; de <= 8; ++de) {
      const int ey = es + de;
      if (ey > 127 || ey < -126) continue;
      for (uint32_t m = 0; m < (1u << 23); ++m) {
        const float y = std::ldexp(from_bits(0x3F800000u | m), ey);
        for (size_t j : {0, 1, 5, 9}) {  // correctly rounded; seeds -4, 0 and +4 ulp
          if (j >= rs.size()) break;
          check_quotient(y, s, rs[j]);
          check_quotient(-y, s, rs[j]);
        }
      }
    }
    // random y of any magnitude up to 2^20 * 449 s (static scales allow
    // quotients beyond 448), tiny and subnormal y included
    const double top = std::fmin(127.0, std::log2(449.0) + es + 20);
    std::uniform_real_distribution<double> uy(-149.0, top);
    for (int i = 0; i < 2000000; ++i) {
      float y = std::exp2(static_cast<float>(uy(rng))) * (rng() & 1 ? -1.0f : 1.0f);
      if (std::fabs(y) >= 0x1p-126f) y = from_bits((bits(y) & 0xFF800000u) | (rng() & 0x7FFFFFu));
      if (std::isinf(y / s)) continue;  // fp32 overflow: both sides saturate in the encoder
      check_quotient(y, s, rs[rng() % rs.size()]);
    }
    for (double r : rs)
      for (float y : {0.0f, -0.0f}) check_quotient(y, s, r);
  }
  // scales: every amax of a few binades, the fallback boundary, random over
  // the whole range, subnormals included
  for (int e : {-100, -99, -1, 0, 8, 9, 100}) {
    for (uint32_t m = 0; m < (1u << 23); ++m) check_scale(std::ldexp(from_bits(0x3F800000u | m), e));
  }
  std::uniform_real_distribution<double> ua(-149.0, 128.0);
  for (int i = 0; i < 4000000; ++i) {
    float a = std::exp2(static_cast<float>(ua(rng)));
    if (a >= 0x1p-126f && !std::isinf(a)) a = from_bits((bits(a) & 0xFF800000u) | (rng() & 0x7FFFFFu));
    if (std::isinf(a)) continue;
    check_scale(a);
  }
  for (uint32_t u = 1; u < (1u << 23); u += 7) check_scale(from_bits(u));  // subnormal amax
  check_scale(0.0f);
  std::printf("checked %llu mismatches %llu\n", (unsigned long long)checked,
              (unsigned long long)bad);
  return bad == 0 ? 0 : 1;
}
