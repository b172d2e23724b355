// The two ways of rounding a float64 value to bf16 (nearest, ties to even) that the RMSNorm kernels
// have used, run on the host: the bit-field form (keep 7 stored mantissa bits, carry into the
// exponent, subnormals by scaling to an integer) and the branch-free form (add and subtract
// 1.5 * 2^(p+52), p the bf16 spacing exponent, copy the sign, convert to float32 exactly).  They must
// agree on every edge value, on every bf16 value, midpoint and its neighbours, and on random doubles
// across the range.  Exit status 0 when they agree everywhere.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <stdlib.h>

static uint64_t d2u(double v) { uint64_t u; memcpy(&u, &v, 8); return u; }
static uint32_t f2u(float v) { uint32_t u; memcpy(&u, &v, 4); return u; }

static uint32_t old_rne(double v) {
  const uint64_t u = d2u(v);
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
  const int e = (int)(a >> 52) - 1023;
  if (e < -126) {
    const double q = rint(fabs(v) * 0x1p133);
    return sign | (uint32_t)q;
  }
  const uint64_t r = (a + 0x00000FFFFFFFFFFFull + ((a >> 45) & 1u)) & ~0x00001FFFFFFFFFFFull;
  const int er = (int)(r >> 52) - 1023;
  if (er > 127) return sign | 0x7F80u;
  return sign | ((uint32_t)(er + 127) << 7) | (uint32_t)((r >> 45) & 0x7Fu);
}

static uint32_t new_rne(double v) {
  int ex;
  frexp(v, &ex);                                   // v_frexp_exp_i32_f64 (0 for v = 0)
  int e = ex - 1;
  e = e < -126 ? -126 : (e > 128 ? 128 : e);
  const double c = ldexp(1.5, e - 7 + 52);
  volatile double s = v + c;                       // no reassociation on the host either
  const double r = copysign(s - c, v);
  return f2u((float)r) >> 16;
}

static uint64_t rng = 88172645463325252ull;
static uint64_t xs(void) { rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17; return rng; }

int main(void) {
  long bad = 0, n = 0;
  #define CHK(v) do { double _v = (v); uint32_t a = old_rne(_v), b = new_rne(_v); ++n; \
    if (a != b) { if (bad < 10) printf("mismatch %a: old %04x new %04x\n", _v, a, b); ++bad; } } while (0)
  // edge values
  double edges[] = {0.0, -0.0, 1.0, -1.0, 0x1p-126, -0x1p-126, 0x1p-133, 0x1p-134, 0x1.8p-134, 0x1p-135,
                    0x1.fcp127, 0x1.fdp127, 0x1.fep127, 0x1.ffp127, 0x1p128, 0x1p129, 0x1p200, -0x1p300,
                    0x1.02p0, 0x1.03p0, 0x1.01p0, 0x1.01000001p0, 0x1.fffp-127, 0x1.ffp-127, 0x1.fep-127,
                    0x1.7fp-133, 0x1.8p-133, 0x1.80001p-133, 3.4e38, -3.4e38, 1e-40, -1e-40, 1e-45, -1e-45};
  for (size_t i = 0; i < sizeof edges / sizeof *edges; ++i) CHK(edges[i]);
  // every bf16 value, its midpoints to the next, and points just around them, both signs
  for (uint32_t b = 0; b < 0x7F80u; ++b) {
    float f, g; uint32_t fb = b << 16, gb = (b + 1) << 16; memcpy(&f, &fb, 4); memcpy(&g, &gb, 4);
    double lo = f, hi = g, mid = 0.5 * (lo + hi);
    double pts[] = {lo, mid, nextafter(mid, 0.0), nextafter(mid, 1e300), nextafter(lo, 1e300), nextafter(hi, 0.0)};
    for (int k = 0; k < 6; ++k) { CHK(pts[k]); CHK(-pts[k]); }
  }
  // random doubles: random sign, exponent in [-160, 140], random 52-bit mantissa
  for (long i = 0; i < 50000000; ++i) {
    uint64_t m = xs() & 0x000FFFFFFFFFFFFFull;
    int e = (int)(xs() % 301) - 160;
    uint64_t u = ((uint64_t)(e + 1023) << 52) | m | ((xs() & 1) << 63);
    double v; memcpy(&v, &u, 8);
    CHK(v);
  }
  // products of the norm's form: bf16 x * r * gamma with r, gamma in realistic and extreme ranges
  for (long i = 0; i < 20000000; ++i) {
    uint32_t xb = (uint32_t)(xs() & 0xFFFF); if (((xb >> 7) & 0xFF) == 0xFF) continue;
    float xf; uint32_t xfb = xb << 16; memcpy(&xf, &xfb, 4);
    double r = ldexp(1.0 + (double)(xs() % 1000000) / 1e6, (int)(xs() % 40) - 20);
    float g = (float)ldexp(1.0 + (double)(xs() % 1000) / 1e3, (int)(xs() % 20) - 10);
    CHK(((double)xf * r) * (double)g);
  }
  printf("%ld values, %ld mismatches\n", n, bad);
  return bad != 0;
}
