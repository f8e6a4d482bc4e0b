/*
 * Host driver for the sanitizer build of the CPU oracle (AddressSanitizer
 * and UndefinedBehaviorSanitizer; test infrastructure).  Runs the oracle on
 * small random shapes in both modes -- every output, and a list of points --
 * and requires the two to agree bit for bit; then the rejected arguments.
 * Exit status 0 when every check held; a sanitizer report aborts the run.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int cc3d_oracle_out_shape(int64_t tx, int64_t tc, int64_t h, int64_t wd, int64_t kt, int64_t kh, int64_t kw,
                          int64_t st, int64_t sh, int64_t sw, int64_t dt, int64_t dh, int64_t dw, int64_t ph,
                          int64_t pw, int64_t pbase, int64_t* to, int64_t* ho, int64_t* wo);
int cc3d_oracle_conv3d(const void* x, const void* cache, int in_dtype, const void* w, const void* bias, int64_t n,
                       int64_t tx, int64_t tc, int64_t h, int64_t wd, int64_t cin, int64_t cout, int64_t kt,
                       int64_t kh, int64_t kw, int64_t st, int64_t sh, int64_t sw, int64_t dt, int64_t dh,
                       int64_t dw, int64_t ph, int64_t pw, int64_t pbase, const int64_t* points, int64_t npoints,
                       double* out, int nthreads);

static uint64_t rng_state = 88172645463325252ull;
static uint64_t next_u64(void) { /* xorshift64 */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return rng_state;
}
static int64_t rnd(int64_t lo, int64_t hi) { return lo + (int64_t)(next_u64() % (uint64_t)(hi - lo + 1)); }

int main(void) {
  int failures = 0, runs = 0;
  for (int iter = 0; iter < 300; ++iter) {
    const int64_t n = rnd(1, 2), tx = rnd(1, 4), tc = rnd(0, 3), h = rnd(1, 7), w = rnd(1, 9);
    const int64_t cin = rnd(1, 6), cout = rnd(1, 5), kt = rnd(1, 3), kh = rnd(1, 3), kw = rnd(1, 3);
    const int64_t st = rnd(1, 2), sh = rnd(1, 2), sw = rnd(1, 2), dt = rnd(1, 2), dh = rnd(1, 2), dw = rnd(1, 2);
    const int64_t ph = rnd(0, 2), pw = rnd(0, 2), pbase = rnd(0, 4);
    const int dtype = (int)rnd(0, 1), has_bias = (int)rnd(0, 1);
    int64_t to, ho, wo;
    if (cc3d_oracle_out_shape(tx, tc, h, w, kt, kh, kw, st, sh, sw, dt, dh, dw, ph, pw, pbase, &to, &ho, &wo))
      continue;
    const size_t es = dtype ? 2 : 4;
    const int64_t nx = n * tx * h * w * cin, nc = n * tc * h * w * cin, nw = cout * kt * kh * kw * cin;
    unsigned char* x = malloc((size_t)nx * es);
    unsigned char* c = tc ? malloc((size_t)nc * es) : NULL;
    unsigned char* wt = malloc((size_t)nw * es);
    unsigned char* b = malloc((size_t)cout * es);
    for (int64_t i = 0; i < nx * (int64_t)es; ++i) x[i] = (unsigned char)(next_u64() & 0x3F);
    for (int64_t i = 0; i < nc * (int64_t)es; ++i) c[i] = (unsigned char)(next_u64() & 0x3F);
    for (int64_t i = 0; i < nw * (int64_t)es; ++i) wt[i] = (unsigned char)(next_u64() & 0x3F);
    for (int64_t i = 0; i < cout * (int64_t)es; ++i) b[i] = (unsigned char)(next_u64() & 0x3F);
    const int64_t total = n * to * ho * wo;
    double* full = malloc(sizeof(double) * (size_t)(total * cout));
    double* part = malloc(sizeof(double) * (size_t)(total * cout));
    int64_t* pts = malloc(sizeof(int64_t) * 4 * (size_t)total);
    int64_t q = 0;
    for (int64_t nn = 0; nn < n; ++nn)
      for (int64_t o = 0; o < to; ++o)
        for (int64_t i = 0; i < ho; ++i)
          for (int64_t j = 0; j < wo; ++j) {
            pts[4 * q] = nn; pts[4 * q + 1] = o; pts[4 * q + 2] = i; pts[4 * q + 3] = j; ++q;
          }
    const void* bias = has_bias ? b : NULL;
    int r1 = cc3d_oracle_conv3d(x, c, dtype, wt, bias, n, tx, tc, h, w, cin, cout, kt, kh, kw, st, sh, sw, dt, dh, dw,
                                ph, pw, pbase, NULL, 0, full, 1);
    int r2 = cc3d_oracle_conv3d(x, c, dtype, wt, bias, n, tx, tc, h, w, cin, cout, kt, kh, kw, st, sh, sw, dt, dh, dw,
                                ph, pw, pbase, pts, total, part, 1);
    if (r1 != 0 || r2 != 0 || memcmp(full, part, sizeof(double) * (size_t)(total * cout)) != 0) {
      fprintf(stderr, "mismatch at iteration %d (rc %d %d)\n", iter, r1, r2);
      ++failures;
    }
    /* an out-of-range point is rejected */
    pts[2] = ho;
    if (cc3d_oracle_conv3d(x, c, dtype, wt, bias, n, tx, tc, h, w, cin, cout, kt, kh, kw, st, sh, sw, dt, dh, dw, ph,
                           pw, pbase, pts, 1, part, 1) != 2) {
      fprintf(stderr, "out-of-range point accepted at iteration %d\n", iter);
      ++failures;
    }
    ++runs;
    free(x); free(c); free(wt); free(b); free(full); free(part); free(pts);
  }
  /* invalid sizes and a missing cache */
  double out[4];
  if (cc3d_oracle_conv3d(out, NULL, 0, out, NULL, 1, 0, 0, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 0, 0, 0, NULL, 0,
                         out, 1) != 1) ++failures;
  if (cc3d_oracle_conv3d(out, NULL, 0, out, NULL, 1, 1, 2, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 0, 0, 0, NULL, 0,
                         out, 1) != 1) ++failures;
  printf("%d oracle runs, %d failed checks\n", runs, failures);
  return failures == 0 && runs > 100 ? 0 : 1;
}
