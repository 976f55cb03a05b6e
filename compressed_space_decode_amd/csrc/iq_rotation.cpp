// iq_make_rotation: seeded rotation parameters (host only).
//
// "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
// Compressed-Space Attention" (arXiv 2608.08081), Abstract: 256 stored
// parameters per head.  The pages do not say how they are drawn; each block's
// left and right quaternions are drawn uniformly on the 3-sphere with
// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) and Marsaglia's method
// (Ann. Math. Statist. 43, 1972).  Only IEEE +, -, *, / and sqrt are used, with
// contraction off, so the fp64 steps are reproducible bit for bit.
#include <cmath>
#include <cstdint>

#include "iq.h"
#include "iq_internal.h"

#pragma clang fp contract(off)

namespace {

struct SplitMix64 {
  uint64_t seed;
  uint64_t i = 0;
  uint64_t next() {
    uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
    ++i;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  // Uniform on [-1, 1): (z >> 11) * 2^-52 - 1, exact in fp64.
  double uniform_pm1() { return (double)(next() >> 11) * 0x1p-52 - 1.0; }
};

void point_on_s3(SplitMix64& g, float out[4]) {
  double x1, x2, s1;
  do {
    x1 = g.uniform_pm1();
    x2 = g.uniform_pm1();
    s1 = x1 * x1 + x2 * x2;
  } while (!(s1 < 1.0));
  double x3, x4, s2;
  do {
    x3 = g.uniform_pm1();
    x4 = g.uniform_pm1();
    s2 = x3 * x3 + x4 * x4;
  } while (!(s2 > 0.0 && s2 < 1.0));
  const double f = std::sqrt((1.0 - s1) / s2);
  out[0] = (float)x1;
  out[1] = (float)x2;
  out[2] = (float)(x3 * f);
  out[3] = (float)(x4 * f);
}

}  // namespace

extern "C" int iq_make_rotation(uint64_t seed, int32_t n_heads, float* params_host) {
  iq::clear_error();
  if (n_heads < 1) {
    iq::set_error("iq_make_rotation: n_heads must be >= 1 (got %d)", n_heads);
    return IQ_EINVAL;
  }
  if (params_host == nullptr) {
    iq::set_error("iq_make_rotation: params_host is NULL");
    return IQ_EINVAL;
  }
  SplitMix64 g{seed};
  for (int32_t h = 0; h < n_heads; ++h)
    for (int b = 0; b < 32; ++b) {
      float* p = params_host + ((int64_t)h * 32 + b) * 8;
      point_on_s3(g, p);
      point_on_s3(g, p + 4);
    }
  return IQ_OK;
}
