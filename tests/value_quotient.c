/* Host check of the value quantiser's quotient.  The store kernels compute
   q = rint((v - z) / s) (Hub page, technical principle: per-group min/max
   value quantisation) without a division per element: t0 = d * rs with
   rs = 1 / s correctly rounded, then t = t0 + (d - t0 s) rs with the
   residual by fused multiply-add (Markstein's correction).  This program
   checks, in IEEE fp32 with fused multiply-add, that t equals the IEEE
   quotient d / s and rounds the same way for every positive finite fp16
   scale s, for the fp32 values d nearest every half-integer multiple
   (k + 1/2) s, k = -2 .. 17, and for random d in [-2 s, 17 s].
   Exit status 0 when every case agrees. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

static float f16_value(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  return e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), e - 25);
}

static int check(float d, float s, float rs, long* quotient_diff) {
  volatile float t0 = d * rs;
  const float t = fmaf(fmaf(-t0, s, d), rs, t0);
  volatile float ex = d / s;
  if (t != ex) ++*quotient_diff;
  return rintf(t) != rintf(ex);
}

int main(int argc, char** argv) {
  const int ulps = argc > 1 ? atoi(argv[1]) : 40;
  long n = 0, bad = 0, qdiff = 0;
  uint64_t rng = 0x9E3779B97F4A7C15ull;
  for (uint32_t hb = 1; hb < 0x7C00; ++hb) {
    const float s = f16_value((uint16_t)hb);
    volatile float one = 1.0f;
    const float rs = one / s;
    for (int k = -2; k <= 17; ++k) {
      float d = (float)(((double)k + 0.5) * (double)s);
      for (int i = 0; i < ulps; ++i) d = nextafterf(d, -INFINITY);
      for (int i = 0; i <= 2 * ulps; ++i, d = nextafterf(d, INFINITY), ++n) bad += check(d, s, rs, &qdiff);
    }
    for (int i = 0; i < 64; ++i, ++n) {
      rng ^= rng << 13;
      rng ^= rng >> 7;
      rng ^= rng << 17;
      const float d = (float)(((double)(rng >> 11) / 9007199254740992.0 * 19.0 - 2.0) * (double)s);
      bad += check(d, s, rs, &qdiff);
    }
  }
  printf("cases %ld rounding mismatches %ld quotient mismatches %ld\n", n, bad, qdiff);
  return bad != 0 || qdiff != 0;
}
