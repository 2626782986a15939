/* Checks the quantizer's division-free group scale: for qmax in {3, 15, 255}
 * and c = fl(1/qmax), q = fl(q0 + r c) with q0 = fl(D c) and r = D - q0 qmax
 * (exact by fma) must equal the correctly rounded quotient fl(D / qmax).
 * Every fp32 D of the binades given on the command line is tried (argument:
 * first and last binade exponent); all three steps scale exactly with D's
 * exponent while no result leaves the normal range, so whole binades stand
 * for every D of the same significand.  Prints "mismatches N". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

int main(int argc, char** argv) {
  const int e_lo = argc > 1 ? atoi(argv[1]) : 0, e_hi = argc > 2 ? atoi(argv[2]) : 0;
  const float qmaxes[3] = {3.0f, 15.0f, 255.0f};
  long bad = 0, n = 0;
  for (int i = 0; i < 3; ++i) {
    const float b = qmaxes[i];
    const float c = 1.0f / b;
    for (int e = e_lo; e <= e_hi; ++e) {
      const uint32_t first = (uint32_t)(e + 127) << 23;
      for (uint32_t m = 0; m < (1u << 23); ++m) {
        const float D = from_bits(first | m);
        const float q0 = D * c;
        const float r = fmaf(-q0, b, D);
        const float q = fmaf(r, c, q0);
        const float want = D / b;                 /* IEEE division, correctly rounded */
        if (q != want) {
          if (bad < 5) printf("qmax %g D %a: %a != %a\n", b, D, q, want);
          ++bad;
        }
        ++n;
      }
    }
  }
  printf("checked %ld mismatches %ld\n", n, bad);
  return bad != 0;
}
