// Host-side check of the library's corrected quotient (fp8q_common.hpp,
// div_rn_corrected) against IEEE fp32 division, bit for bit.  The device runs
// the same arithmetic (fp32 multiply, fp32 fma), so agreement here shows the
// algorithm, not just this compiler, is right.
//
// Cases: for each scale s in a list (random, structured, range ends), every
// fp32 y of several binades (all 2^23 significands), plus random y over the
// whole contract range |y| <= 449 s.  Prints the number of mismatches.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "fp8q_common.hpp"

static float from_bits(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
static uint32_t bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }

int main(int argc, char** argv) {
  const int n_random_scales = argc > 1 ? std::atoi(argv[1]) : 24;
  std::mt19937_64 rng(12345);
  std::vector<float> scales = {1.0f, 13.0f / 448.0f, 0x1p-76f, 0x1.fffffep-76f, 0x1p-20f,
                               0x1.fffffep0f, 0x1.000002p0f, 3.0f, 0x1p100f, 0x1.8p119f,
                               1.0f / 448.0f, 7.0f};
  std::uniform_real_distribution<double> ue(-76.0, 119.0);
  for (int i = 0; i < n_random_scales; ++i) {
    float s = std::exp2(static_cast<float>(ue(rng)));
    scales.push_back(from_bits((bits(s) & 0xFF800000u) | (rng() & 0x7FFFFFu)));
  }
  uint64_t checked = 0, bad = 0;
  for (float s : scales) {
    const float r = 1.0f / s;
    const int es = std::ilogb(s);
    // exhaustive significands for y in three binades near the top of the range
    for (int de = 6; de <= 8; ++de) {
      const int ey = es + de;
      for (uint32_t m = 0; m < (1u << 23); ++m) {
        for (int sg = 0; sg < 2; ++sg) {
          float y = std::ldexp(from_bits(0x3F800000u | m), ey);
          if (sg) y = -y;
          if (std::fabs(y) > 449.0f * s) continue;
          const float want = y / s;
          const float got = fp8q::div_rn_corrected(y, s, r);
          ++checked;
          if (std::fabs(want) < 0x1p-125f) {  // subnormal quotient: weaker promise
            if (std::signbit(want) != std::signbit(got) || std::fabs(got) >= 0x1p-22f) ++bad;
            continue;
          }
          if (bits(want) != bits(got)) {
            if (bad < 10) std::printf("mismatch y=%a s=%a want=%a got=%a\n", y, s, want, got);
            ++bad;
          }
        }
      }
    }
    // random y over the contract range, including tiny magnitudes
    std::uniform_real_distribution<double> uy(-140.0, std::log2(449.0) + es + 1);
    for (int i = 0; i < 2000000; ++i) {
      float y = std::exp2(static_cast<float>(uy(rng))) * (rng() & 1 ? -1.0f : 1.0f);
      y = from_bits((bits(y) & 0xFF800000u) | (rng() & 0x7FFFFFu));
      if (std::fabs(y) > 449.0f * s) continue;
      const float want = y / s;
      const float got = fp8q::div_rn_corrected(y, s, r);
      ++checked;
      // for |y| < 2^-100 or a subnormal quotient only the sign and a
      // magnitude below 2^-22 are promised (such quotients encode to +-0)
      const bool tiny = std::fabs(y) < 0x1p-100f || std::fabs(want) < 0x1p-125f;
      const bool ok = tiny ? (std::signbit(want) == std::signbit(got) && std::fabs(got) < 0x1p-22f)
                           : bits(want) == bits(got);
      if (!ok) {
        if (bad < 10) std::printf("mismatch y=%a s=%a want=%a got=%a\n", y, s, want, got);
        ++bad;
      }
    }
    // signed zeros
    for (float y : {0.0f, -0.0f}) {
      ++checked;
      if (bits(fp8q::div_rn_corrected(y, s, r)) != bits(y / s)) ++bad;
    }
  }
  std::printf("checked %llu mismatches %llu\n", (unsigned long long)checked,
              (unsigned long long)bad);
  return bad == 0 ? 0 : 1;
}
