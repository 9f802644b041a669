/* Exhaustive check that an FMA division sequence yields the same quantization
 * codes as IEEE binary32 division, for every input the per-row quantizers can
 * meet with 16-bit activations.
 *
 * For a scale S and its correctly rounded reciprocal r = RN(1/S):
 *     y0 = RN(x * r);  e = RN(x - S*y0) (one fma);  y1 = RN(y0 + e*r) (one fma)
 * and the code is taken from y1 (sign of x restored, so -0 stays -0) instead of
 * from RN(x / S).  Domain: x any finite bf16 (or fp16) value with |x| <= alpha,
 * S = max(RN(alpha / qmax), 1e-8) for every positive finite bf16 (fp16) alpha.
 *   mode i8:   code = clamp(rne(q), -127, 127)          (qmax 127)
 *   mode e4m3: code = e4m3fn_rne(clamp(q, -448, 448))   (qmax 448)
 * Prints the number of pairs checked and the number whose codes differ.
 * Build: gcc -O2 -ffp-contract=off -fopenmp (x86-64 SSE arithmetic). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static float bf16_val(uint32_t h) { return from_bits(h << 16); }
static float f16_val(uint32_t h) {            /* IEEE binary16 -> binary32, exact */
  uint32_t s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  float v;
  if (e == 0) v = ldexpf((float)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexpf((float)(m | 1024), (int)e - 25);
  return s ? -v : v;
}
/* OCP e4m3fn, round to nearest even, |v| <= 448 (spacing 2^(e-3) in binade e,
 * 2^-9 below the smallest normal 2^-6); the sign of zero is kept. */
static int e4m3(float v) {
  int s = signbit(v) ? 0x80 : 0;
  double a = fabs((double)v);
  int ex;
  frexp(a, &ex);
  int e = ex - 1;
  if (a == 0 || e < -6) e = -6;
  double n = nearbyint(a / ldexp(1.0, e - 3));
  if (n == 16) { e++; n = 8; }
  int fe = n >= 8 ? e + 7 : 0, fm = n >= 8 ? (int)n - 8 : (int)n;
  return s | (fe << 3) | fm;
}
static int code(float q, int fp8) {
  if (fp8) return e4m3(fminf(fmaxf(q, -448.0f), 448.0f));
  return (int)fminf(fmaxf(rintf(q), -127.0f), 127.0f);
}

int main(int argc, char** argv) {
  const int use_f16 = argc > 1 && strcmp(argv[1], "f16") == 0;
  const int fp8 = argc > 2 && strcmp(argv[2], "e4m3") == 0;
  const float qmax = fp8 ? 448.0f : 127.0f;
  float* vals = malloc(sizeof(float) * 65536);
  int nv = 0;
  for (uint32_t h = 0; h < 65536; ++h) {
    float v = use_f16 ? f16_val(h) : bf16_val(h);
    if (isfinite(v)) vals[nv++] = v;
  }
  long long checked = 0, bad = 0;
#pragma omp parallel for reduction(+ : checked, bad) schedule(dynamic, 64)
  for (int ia = 0; ia < nv; ++ia) {
    const float alpha = vals[ia];
    if (!(alpha > 0.0f)) continue;
    float S = alpha / qmax;
    if (S < 1e-8f) S = 1e-8f;
    const float r = 1.0f / S;
    for (int ix = 0; ix < nv; ++ix) {
      const float x = vals[ix];
      if (fabsf(x) > alpha) continue;
      const float y0 = x * r;
      const float e = fmaf(-S, y0, x);
      const float y1 = copysignf(fmaf(e, r, y0), x);
      ++checked;
      if (code(x / S, fp8) != code(y1, fp8)) {
#pragma omp critical
        if (bad < 5) printf("mismatch x=%.9g S=%.9g ref=%.9g seq=%.9g\n", x, S, x / S, y1);
        ++bad;
      }
    }
  }
  printf("%s %s checked=%lld mismatches=%lld\n", use_f16 ? "f16" : "bf16", fp8 ? "e4m3" : "i8", checked, bad);
  free(vals);
  return bad != 0;
}
