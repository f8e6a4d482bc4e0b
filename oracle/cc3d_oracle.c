/*
 * TEST INFRASTRUCTURE ONLY -- the CPU oracle for the cached causal Conv3D.
 *
 * A plain, slow, obviously correct fp64 implementation of what the GPU path
 * computes.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load it; the product library never links or calls it, and it
 * shares no code, header or table with the product library.
 *
 * What it computes follows "Cache-Aware Conv3D Lowering Across Embedded
 * World-Model Decoders", the lowering section (the paper's Sec. 4, whose
 * display equations are lost in the page text and are restated here from the
 * surrounding prose):
 *   - the source is Z = [C; X] joined along time, |Z| = |C| + |X|;
 *   - the effective causal left pad is p_l = p_base - |C| (zero frames in
 *     front of Z, none behind);
 *   - output frame o, temporal tap k reads source time t = o*s_t + k*d_t - p_l,
 *     and a time outside [0, |Z|) contributes nothing;
 *   - the spatial part of each tap is an ordinary PyTorch Conv2D
 *     (cross-correlation, no kernel flip) with the original stride, zero
 *     padding and dilation, so the full result is the bias added once plus
 *     the sum over taps of the bias-free spatial responses.
 * Together these are exactly a plain Conv3D over Z padded with p_l zero
 * frames in front, which is what this file evaluates, output by output:
 *
 *   y[n,o,i,j,co] = b[co] + sum over (k, a, c, ci), in that lexicographic
 *                   order, of Z[n, t, u, v, ci] * W[co, k, a, c, ci]
 *   t = o*s_t + k*d_t - p_l,  u = i*s_h - p_h + a*d_h,  v = j*s_w - p_w + c*d_w,
 *   terms whose (t, u, v) falls outside Z are skipped.
 *
 * Layouts (dense, row-major in the order written):
 *   x      [N][Tx][H][W][Cin]        cache [N][Tc][H][W][Cin]
 *   w      [Cout][Kt][Kh][Kw][Cin]   b     [Cout]
 *   out    [N][To][Ho][Wo][Cout] (all outputs) or [npoints][Cout] (sampled)
 * Inputs are float32 (in_dtype 0) or bfloat16 bit patterns (in_dtype 1);
 * both convert to double exactly.  Accumulation is in double without fused
 * multiply-add (the build uses -ffp-contract=off), and the per-output
 * summation order is fixed, so results do not depend on thread count.
 *
 * Output time length (standard convolution length of Z padded by p_l in
 * front and nothing behind):  To = floor((|Z| + p_l - d_t*(Kt-1) - 1)/s_t) + 1.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double to_double(const void* p, int64_t idx, int dtype) {
  if (dtype == 0) return (double)((const float*)p)[idx];
  uint32_t u = (uint32_t)((const uint16_t*)p)[idx] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* floor((num)/den) for den > 0, any sign of num */
static int64_t floordiv(int64_t num, int64_t den) {
  int64_t q = num / den;
  if ((num % den != 0) && (num < 0)) q -= 1;
  return q;
}

/* Output sizes of the cached causal Conv3D; returns 0 when all are >= 1. */
int cc3d_oracle_out_shape(int64_t tx, int64_t tc, int64_t h, int64_t wd,
                          int64_t kt, int64_t kh, int64_t kw,
                          int64_t st, int64_t sh, int64_t sw,
                          int64_t dt, int64_t dh, int64_t dw,
                          int64_t ph, int64_t pw, int64_t pbase,
                          int64_t* to, int64_t* ho, int64_t* wo) {
  int64_t zt = tc + tx;
  int64_t pl = pbase - tc;
  *to = floordiv(zt + pl - dt * (kt - 1) - 1, st) + 1;
  *ho = floordiv(h + 2 * ph - dh * (kh - 1) - 1, sh) + 1;
  *wo = floordiv(wd + 2 * pw - dw * (kw - 1) - 1, sw) + 1;
  return (*to >= 1 && *ho >= 1 && *wo >= 1) ? 0 : 1;
}

/*
 * Direct cached causal Conv3D.  points == NULL: every output, written to
 * out[N][To][Ho][Wo][Cout].  Otherwise npoints tuples (n, o, i, j) and
 * out[npoints][Cout].  bias may be NULL (no bias term).  Returns 0 on
 * success, 1 on an invalid size, 2 on an out-of-range point, 3 on no memory.
 */
int cc3d_oracle_conv3d(const void* x, const void* cache, int in_dtype,
                       const void* w, const void* bias,
                       int64_t n, int64_t tx, int64_t tc, int64_t h, int64_t wd,
                       int64_t cin, int64_t cout,
                       int64_t kt, int64_t kh, int64_t kw,
                       int64_t st, int64_t sh, int64_t sw,
                       int64_t dt, int64_t dh, int64_t dw,
                       int64_t ph, int64_t pw, int64_t pbase,
                       const int64_t* points, int64_t npoints,
                       double* out, int nthreads) {
  if (n < 1 || tx < 1 || tc < 0 || h < 1 || wd < 1 || cin < 1 || cout < 1 ||
      kt < 1 || kh < 1 || kw < 1 || st < 1 || sh < 1 || sw < 1 ||
      dt < 1 || dh < 1 || dw < 1 || ph < 0 || pw < 0 || pbase < 0)
    return 1;
  if (tc > 0 && cache == NULL) return 1;
  int64_t to, ho, wo;
  if (cc3d_oracle_out_shape(tx, tc, h, wd, kt, kh, kw, st, sh, sw, dt, dh, dw,
                            ph, pw, pbase, &to, &ho, &wo))
    return 1;
  const int64_t zt = tc + tx;
  const int64_t pl = pbase - tc;
  const int64_t total = points ? npoints : n * to * ho * wo;
  if (points) {
    for (int64_t p = 0; p < npoints; ++p) {
      const int64_t* q = points + 4 * p;
      if (q[0] < 0 || q[0] >= n || q[1] < 0 || q[1] >= to || q[2] < 0 ||
          q[2] >= ho || q[3] < 0 || q[3] >= wo)
        return 2;
    }
  }
  /* W as doubles, regrouped [k][a][c][ci][co] so the innermost loop over co
     is contiguous; each output's own summation order is unchanged. */
  const int64_t taps = kt * kh * kw;
  double* wr = (double*)malloc(sizeof(double) * (size_t)(taps * cin * cout));
  if (!wr) return 3;
  for (int64_t co = 0; co < cout; ++co)
    for (int64_t s = 0; s < taps; ++s)
      for (int64_t ci = 0; ci < cin; ++ci)
        wr[(s * cin + ci) * cout + co] = to_double(w, (co * taps + s) * cin + ci, in_dtype);
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double* acc = (double*)malloc(sizeof(double) * (size_t)cout);
    double* zv = (double*)malloc(sizeof(double) * (size_t)cin);
    if (!acc || !zv) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
    }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
    for (int64_t e = 0; e < total; ++e) {
      if (!acc || !zv) continue;
      int64_t nn, o, i, j;
      if (points) {
        nn = points[4 * e]; o = points[4 * e + 1]; i = points[4 * e + 2]; j = points[4 * e + 3];
      } else {
        int64_t r = e;
        j = r % wo; r /= wo;
        i = r % ho; r /= ho;
        o = r % to; nn = r / to;
      }
      for (int64_t co = 0; co < cout; ++co)
        acc[co] = bias ? to_double(bias, co, in_dtype) : 0.0;
      for (int64_t k = 0; k < kt; ++k) {
        const int64_t t = o * st + k * dt - pl;
        if (t < 0 || t >= zt) continue;
        for (int64_t a = 0; a < kh; ++a) {
          const int64_t u = i * sh - ph + a * dh;
          if (u < 0 || u >= h) continue;
          for (int64_t c = 0; c < kw; ++c) {
            const int64_t v = j * sw - pw + c * dw;
            if (v < 0 || v >= wd) continue;
            const void* src;
            int64_t base;
            if (t < tc) { src = cache; base = (((nn * tc + t) * h + u) * wd + v) * cin; }
            else        { src = x;     base = (((nn * tx + (t - tc)) * h + u) * wd + v) * cin; }
            for (int64_t ci = 0; ci < cin; ++ci) zv[ci] = to_double(src, base + ci, in_dtype);
            const double* wk = wr + ((k * kh + a) * kw + c) * cin * cout;
            for (int64_t ci = 0; ci < cin; ++ci) {
              const double z = zv[ci];
              const double* wrow = wk + ci * cout;
              for (int64_t co = 0; co < cout; ++co) acc[co] += z * wrow[co];
            }
          }
        }
      }
      memcpy(out + e * cout, acc, sizeof(double) * (size_t)cout);
    }
    free(acc);
    free(zv);
  }
  free(wr);
  return failed ? 3 : 0;
}
