/*
 * Host emulation of the GPU quantizer's fp32 arithmetic (bit_ptq_looped_amd/
 * csrc/quant_core.h and quant_act.hip), checked against the plain
 * definitions of Eq.(4) ("paper_specification.yaml", lq1_quantization):
 *
 *   step: base = fl32(absmax / qmax).  The kernels form it as
 *         q0 = fl32(absmax * rq), rq = fl32(1 / qmax), then one FMA
 *         correction fma(fma(-q0, qmax, absmax), rq, q0).  Checked over every
 *         finite non-negative fp32 absmax against the correctly rounded IEEE
 *         quotient, for qmax 7 and 127.
 *   code: clamp(rint(fl32(x / s)), -qmax, qmax).  The kernels take
 *         p = fl32(x * r) with r the hardware reciprocal of s (within 1 ulp
 *         of 1/s), accept rint(p) unless the element sits within 2^-14 of a
 *         rounding boundary (run form: |fma(x, r, -rint(p))|; group form:
 *         |p - rint(p)|), and redo flagged elements with the true division.
 *         Checked on random and near-tie (x, s) for every r within 1 ulp of
 *         1/s: an unflagged element must give the true code.
 *
 * Built with -ffp-contract=off (no implicit FMA); x86-64 evaluates float
 * expressions in single precision (SSE), so every operation below is one
 * IEEE fp32 rounding, as on the GPU.
 *
 * Usage: quant_arith_check [step|step_nocorr|codes|codes_loose]; prints counts
 * and exits 0 when there are no mismatches ("step_nocorr" drops the FMA
 * correction and "codes_loose" the near-tie margin; both are expected to
 * report mismatches: they show the checks can fail).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static float step_base(float amax, float qmaxf, float rq, int corr) {
  const float q0 = amax * rq;
  if (!corr) return q0;
  return fmaf(fmaf(-q0, qmaxf, amax), rq, q0);
}

static long long check_step(int qmax, int corr) {
  const float qmaxf = (float)qmax;
  const float rq = 1.0f / qmaxf;
  long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(dynamic, 8)
  for (long long hi = 0; hi < 0x7F80; ++hi) {  /* exponent/high bits of every finite non-negative float */
    for (uint32_t lo = 0; lo < 0x10000u; ++lo) {
      const float amax = f_of(((uint32_t)hi << 16) | lo);
      const float want = amax / qmaxf; /* correctly rounded */
      const float got = step_base(amax, qmaxf, rq, corr);
      if (memcmp(&want, &got, 4) != 0) ++bad;
    }
  }
  return bad;
}

/* splitmix64 */
static uint64_t mix(uint64_t* s) {
  uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static double unit(uint64_t* s) { return (double)(mix(s) >> 11) * (1.0 / 9007199254740992.0); }

static float clampf(float v, float q) { return v < -q ? -q : (v > q ? q : v); }

/* the kernels' margin below 0.5; "codes_loose" sets it to 0, which accepts
 * every rint(p) and must then show wrong codes at near-ties */
static float g_margin = 6.103515625e-05f;

/* the kernel's decision for one element; returns 1 if the fast path accepts
 * it (then *code is its code) */
static int fast_code(float x, float r, float qmaxf, int group_form, float* code) {
  if (!(r > 1.0e-37f && r < 1.0e37f)) return 0;
  const float p = x * r;
  const float rp = rintf(p);
  const float d = group_form ? fabsf(p - rp) : fabsf(fmaf(x, r, -rp));
  if (d > 0.5f - g_margin) return 0;
  *code = clampf(rp, qmaxf);
  return 1;
}

static long long check_codes(long long n, long long* accepted) {
  long long bad = 0, acc = 0;
  const int qmaxes[2] = {7, 127};
#pragma omp parallel for reduction(+ : bad, acc) schedule(static)
  for (long long i = 0; i < n; ++i) {
    uint64_t st = 0x5EEDull * 1000003ull + (uint64_t)i;
    const float qmaxf = (float)qmaxes[i & 1];
    /* a step over a wide range of exponents */
    const float s = (float)ldexp(1.0 + unit(&st), (int)(mix(&st) % 160) - 80);
    double q;
    switch (mix(&st) % 4) {
      case 0: /* anywhere in and past the code range */
        q = (unit(&st) * 2.0 - 1.0) * (qmaxf + 8.0);
        break;
      case 1: /* on a half-integer */
        q = (double)((int64_t)(mix(&st) % (uint64_t)(2 * qmaxf + 8)) - (qmaxf + 4)) + 0.5;
        break;
      default: { /* within 2^-9 .. 2^-26 of a half-integer */
        const double h = (double)((int64_t)(mix(&st) % (uint64_t)(2 * qmaxf + 8)) - (qmaxf + 4)) + 0.5;
        const double e = ldexp(unit(&st) * 2.0 - 1.0, -9 - (int)(mix(&st) % 18));
        q = h + e;
      }
    }
    const float x = (float)(q * (double)s);
    const float want = clampf(rintf(x / s), qmaxf);
    const float rn = 1.0f / s;
    const float rs[3] = {nextafterf(rn, 0.0f), rn, nextafterf(rn, INFINITY)};
    for (int k = 0; k < 3; ++k) {
      for (int form = 0; form < 2; ++form) {
        float got;
        if (fast_code(x, rs[k], qmaxf, form, &got)) {
          ++acc;
          if (got != want) ++bad;
        }
      }
    }
  }
  *accepted = acc;
  return bad;
}

int main(int argc, char** argv) {
  const char* mode = argc > 1 ? argv[1] : "step";
  if (!strcmp(mode, "step") || !strcmp(mode, "step_nocorr")) {
    const int corr = !strcmp(mode, "step");
    long long b7 = check_step(7, corr), b127 = check_step(127, corr);
    printf("step%s mismatches qmax7 %lld qmax127 %lld over %lld values each\n", corr ? "" : "_nocorr", b7, b127,
           (long long)0x7F80 * 0x10000);
    return (b7 || b127) ? 1 : 0;
  }
  if (!strcmp(mode, "codes") || !strcmp(mode, "codes_loose")) {
    if (!strcmp(mode, "codes_loose")) g_margin = 0.0f;
    long long accepted = 0;
    const long long n = 20000000;
    long long bad = check_codes(n, &accepted);
    printf("codes mismatches %lld of %lld fast-path decisions (%lld cases)\n", bad, accepted, n);
    return bad ? 1 : 0;
  }
  fprintf(stderr, "unknown mode %s\n", mode);
  return 2;
}
