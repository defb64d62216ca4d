/*
 * Check of the division the one-launch linear layer uses when it quantizes activations inside
 * the GEMM (test infrastructure, host code only).
 *
 * The per-token-group quantizer computes, for a 1x128 group with amax a, the scale
 * s = fl(max(a, 1e-10) / 448) and each element's quotient fl(x / s) (correctly rounded), then
 * clamps it to +-448 and rounds it to e4m3. The fused kernel replaces the division by
 *     r = fl(1 / s),  q0 = fl(x * r),  e = fma(-q0, s, x),  y = copysign(fma(e, r, q0), x).
 * This program compares clamp(y) with clamp(fl(x / s)) bit for bit, for every finite input x
 * of the format (bf16 or fp16) with |x| <= a and every finite positive a of that format that
 * step divides (step 1: all of them), and reports the pairs whose quotients differ and, among
 * those, the ones that could round to different e4m3 codes: a magnitude of at least 2^-10
 * (below it both round to a zero), or different signs.
 *
 * Usage: fused_division_check bf16|fp16 [step]; prints one line
 *     "<format> pairs=<n> differ=<n> code_mismatch=<n>"
 * and exits 0 when code_mismatch is 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}
static uint32_t to_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}
static float bf16_value(uint16_t h) { return from_bits((uint32_t)h << 16); }
static float fp16_value(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  float v;
  if (e == 0) v = ldexpf((float)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexpf((float)(m | 1024), e - 25);
  return (h & 0x8000) ? -v : v;
}
static float clamp448(float y) { return fminf(fmaxf(y, -448.0f), 448.0f); }

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  const int fp16 = strcmp(argv[1], "fp16") == 0;
  const int step = argc > 2 ? atoi(argv[2]) : 1;
  if (step < 1) return 2;
  long long pairs = 0, differ = 0, bad = 0;
#pragma omp parallel for reduction(+ : pairs, differ, bad) schedule(dynamic, 16)
  for (int ha = 1; ha < 0x7fff; ha += step) {
    const float a = fp16 ? fp16_value((uint16_t)ha) : bf16_value((uint16_t)ha);
    if (!isfinite(a) || a <= 0.0f) continue;
    volatile float floor_v = 1e-10f;
    const float s = fmaxf(a, floor_v) / 448.0f;
    const float r = 1.0f / s;
    for (int hx = 0; hx < 0x10000; ++hx) {
      const float x = fp16 ? fp16_value((uint16_t)hx) : bf16_value((uint16_t)hx);
      if (!isfinite(x) || fabsf(x) > a) continue;
      ++pairs;
      const float want = clamp448(x / s);
      const float q0 = x * r;
      const float e = fmaf(-q0, s, x);
      const float got = clamp448(copysignf(fmaf(e, r, q0), x));
      if (to_bits(want) != to_bits(got)) {
        ++differ;
        if (fabsf(want) >= 0x1p-10f || fabsf(got) >= 0x1p-10f || signbit(want) != signbit(got)) ++bad;
      }
    }
  }
  printf("%s pairs=%lld differ=%lld code_mismatch=%lld\n", fp16 ? "fp16" : "bf16", pairs, differ, bad);
  return bad == 0 ? 0 : 1;
}
