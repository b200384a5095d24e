/*
 * CPU oracle for the fused small-channel convolution + epilogue operators.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  The GPU library
 * never includes, links or calls it, and it never includes anything of the
 * GPU library: the two share no code.
 *
 * Everything here is the plain definition of the operation, written out as
 * loop nests and accumulated in double precision.  There is no tiling, no
 * fusion and no reordering beyond what the definitions state, so each
 * function can be checked against the pages by eye.  Inputs are the fp32
 * values the GPU sees; outputs are double.
 *
 * Sources (the three POPCORNBENCH Kimi-K2.6 level-2 transcripts):
 *   "l2_p57": Conv2d 3x3 (8->64) -> ReLU -> HardSwish.
 *   "l2_p10": ConvTranspose2d 3x3 s1 p1 (64->64) -> MaxPool2d(2,2) ->
 *             Hardtanh -> mean over H,W (keepdim) -> tanh.
 *   "l2_p90": Conv3d 3x3x3 (8->64) -> LeakyReLU(0.2) -> + per-channel
 *             sum_tensor -> clamp[-1,1] -> exact GELU.
 *
 * Parity pins for every function live in tests/test_oracle_pins.py; none
 * of the functions below is "parity unpinned".
 *
 * Layouts: contiguous NCHW / NCDHW activations; conv weights
 * [C_out][C_in][k][k](k); transposed-conv weights [C_in][C_out][k][k]
 * (the layout l2_p10 states for ConvTranspose2d weights).
 * A NULL bias means zero bias (l2_p57's first kernel reads the bias as
 * "bias ? bias[c_out] : 0").
 *
 * Return values: 0 on success, -1 on a bad argument (NULL pointer where a
 * buffer is required, non-positive size, output size below 1).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EBADARG (-1)

static double bias_of(const float *b, int o) { return b ? (double)b[o] : 0.0; }

/* Number of OpenMP threads the oracle runs on (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* Elementwise epilogues                                                      */
/* ------------------------------------------------------------------------ */

/* ReLU: max(v, 0).  l2_p57 problem statement, step 2. */
double oracle_relu(double v) { return v > 0.0 ? v : 0.0; }

/* HardSwish: v * clamp((v + 3) / 6, 0, 1), the formula l2_p57 states for
 * step 3 (it evaluates it at 0, 3 and 6 in its worked check). */
double oracle_hardswish(double v) {
  double g = (v + 3.0) / 6.0;
  if (g < 0.0) g = 0.0;
  if (g > 1.0) g = 1.0;
  return v * g;
}

/* LeakyReLU: v for v >= 0, slope * v otherwise (l2_p90 step 2, slope 0.2). */
double oracle_leaky_relu(double v, double slope) { return v >= 0.0 ? v : slope * v; }

/* clamp(v, lo, hi) = min(max(v, lo), hi).  Used for l2_p90's clamp step and
 * for l2_p10's Hardtanh (clip to [-1, 1]). */
double oracle_clamp(double v, double lo, double hi) {
  if (v < lo) v = lo;
  if (v > hi) v = hi;
  return v;
}

/* Exact GELU: 0.5 * t * (1 + erf(t / sqrt(2))), l2_p90's "approximate=False"
 * formulation, with libm's erf. */
double oracle_gelu(double t) { return 0.5 * t * (1.0 + erf(t / sqrt(2.0))); }

/* Full l2_p90 epilogue on one conv output v of channel with offset s:
 * LeakyReLU -> + s -> clamp -> GELU, in the order of its problem statement. */
double oracle_lrelu_add_clamp_gelu(double v, double s, double slope, double lo, double hi) {
  double t = oracle_leaky_relu(v, slope);
  t = t + s;
  t = oracle_clamp(t, lo, hi);
  return oracle_gelu(t);
}

/* ------------------------------------------------------------------------ */
/* Conv2d (stride 1, padding 0, dilation 1, groups 1) -- l2_p57               */
/* ------------------------------------------------------------------------ */

/* One output of the direct convolution (a gather over C_in x k x k):
 *   z[n,o,h,w] = b[o] + sum_{i,kh,kw} x[n,i,h+kh,w+kw] * W[o,i,kh,kw]
 * l2_p57 states padding 0 / stride 1 (output 126 from 128 with k = 3) and
 * writes the per-output loop over (c_in, kh, kw) with this indexing. */
static double conv2d_at(const float *x, const float *w, const float *b, int C_in, int H, int W,
                        int k, int n, int o, int h, int ww) {
  double acc = bias_of(b, o);
  for (int i = 0; i < C_in; ++i)
    for (int kh = 0; kh < k; ++kh)
      for (int kw = 0; kw < k; ++kw) {
        double xv = x[(((size_t)n * C_in + i) * H + (h + kh)) * W + (ww + kw)];
        double wv = w[(((size_t)o * C_in + i) * k + kh) * k + kw];
        acc += xv * wv;
      }
  return acc;
}

/* Pre-activation Conv2d output z[N][C_out][H-k+1][W-k+1]. */
int oracle_conv2d(const float *x, const float *w, const float *b, double *z, int N, int C_in, int H,
                  int W, int C_out, int k) {
  if (!x || !w || !z || N < 1 || C_in < 1 || C_out < 1 || k < 1) return ORACLE_EBADARG;
  int Ho = H - k + 1, Wo = W - k + 1;
  if (Ho < 1 || Wo < 1) return ORACLE_EBADARG;
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < N; ++n)
    for (int o = 0; o < C_out; ++o)
      for (int h = 0; h < Ho; ++h)
        for (int ww = 0; ww < Wo; ++ww)
          z[(((size_t)n * C_out + o) * Ho + h) * Wo + ww] =
              conv2d_at(x, w, b, C_in, H, W, k, n, o, h, ww);
  return ORACLE_OK;
}

/* y = HardSwish(ReLU(Conv2d(x))): the whole l2_p57 model. */
int oracle_conv2d_relu_hswish(const float *x, const float *w, const float *b, double *y, int N,
                              int C_in, int H, int W, int C_out, int k) {
  if (!x || !w || !y || N < 1 || C_in < 1 || C_out < 1 || k < 1) return ORACLE_EBADARG;
  int Ho = H - k + 1, Wo = W - k + 1;
  if (Ho < 1 || Wo < 1) return ORACLE_EBADARG;
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < N; ++n)
    for (int o = 0; o < C_out; ++o)
      for (int h = 0; h < Ho; ++h)
        for (int ww = 0; ww < Wo; ++ww) {
          double v = conv2d_at(x, w, b, C_in, H, W, k, n, o, h, ww);
          y[(((size_t)n * C_out + o) * Ho + h) * Wo + ww] = oracle_hardswish(oracle_relu(v));
        }
  return ORACLE_OK;
}

/* Same model evaluated only at the given flat output indices (into the
 * [N][C_out][Ho][Wo] output), for spot checks of full-size runs. */
int oracle_conv2d_relu_hswish_at(const float *x, const float *w, const float *b, int N, int C_in,
                                 int H, int W, int C_out, int k, const int64_t *idx, int64_t count,
                                 double *out) {
  if (!x || !w || !idx || !out || count < 0) return ORACLE_EBADARG;
  int Ho = H - k + 1, Wo = W - k + 1;
  if (Ho < 1 || Wo < 1) return ORACLE_EBADARG;
  int64_t total = (int64_t)N * C_out * Ho * Wo;
  for (int64_t j = 0; j < count; ++j)
    if (idx[j] < 0 || idx[j] >= total) return ORACLE_EBADARG;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j) {
    int64_t q = idx[j];
    int ww = (int)(q % Wo); q /= Wo;
    int h = (int)(q % Ho); q /= Ho;
    int o = (int)(q % C_out); q /= C_out;
    int n = (int)q;
    double v = conv2d_at(x, w, b, C_in, H, W, k, n, o, h, ww);
    out[j] = oracle_hardswish(oracle_relu(v));
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Conv3d (stride 1, padding 0) -- l2_p90                                     */
/* ------------------------------------------------------------------------ */

/* z[n,o,d,h,w] = b[o] + sum_{i,kd,kh,kw} x[n,i,d+kd,h+kh,w+kw] * W[o,i,kd,kh,kw]
 * l2_p90: weight [C_out, C_in, K_d, K_h, K_w], default stride 1, padding 0
 * (D_out = D - K_d + 1 etc.). */
static double conv3d_at(const float *x, const float *w, const float *b, int C_in, int D, int H,
                        int W, int k, int n, int o, int d, int h, int ww) {
  double acc = bias_of(b, o);
  for (int i = 0; i < C_in; ++i)
    for (int kd = 0; kd < k; ++kd)
      for (int kh = 0; kh < k; ++kh)
        for (int kw = 0; kw < k; ++kw) {
          double xv = x[((((size_t)n * C_in + i) * D + (d + kd)) * H + (h + kh)) * W + (ww + kw)];
          double wv = w[((((size_t)o * C_in + i) * k + kd) * k + kh) * k + kw];
          acc += xv * wv;
        }
  return acc;
}

/* Pre-activation Conv3d output z[N][C_out][D-k+1][H-k+1][W-k+1]. */
int oracle_conv3d(const float *x, const float *w, const float *b, double *z, int N, int C_in, int D,
                  int H, int W, int C_out, int k) {
  if (!x || !w || !z || N < 1 || C_in < 1 || C_out < 1 || k < 1) return ORACLE_EBADARG;
  int Do = D - k + 1, Ho = H - k + 1, Wo = W - k + 1;
  if (Do < 1 || Ho < 1 || Wo < 1) return ORACLE_EBADARG;
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < N; ++n)
    for (int o = 0; o < C_out; ++o)
      for (int d = 0; d < Do; ++d)
        for (int h = 0; h < Ho; ++h)
          for (int ww = 0; ww < Wo; ++ww)
            z[((((size_t)n * C_out + o) * Do + d) * Ho + h) * Wo + ww] =
                conv3d_at(x, w, b, C_in, D, H, W, k, n, o, d, h, ww);
  return ORACLE_OK;
}

/* y = GELU(clamp(LeakyReLU(Conv3d(x)) + s[o], lo, hi)): the l2_p90 model.
 * s is the [C_out,1,1,1] sum_tensor, broadcast per output channel. */
int oracle_conv3d_lrelu_add_clamp_gelu(const float *x, const float *w, const float *b,
                                       const float *s, double *y, int N, int C_in, int D, int H,
                                       int W, int C_out, int k, double slope, double lo,
                                       double hi) {
  if (!x || !w || !s || !y || N < 1 || C_in < 1 || C_out < 1 || k < 1) return ORACLE_EBADARG;
  int Do = D - k + 1, Ho = H - k + 1, Wo = W - k + 1;
  if (Do < 1 || Ho < 1 || Wo < 1) return ORACLE_EBADARG;
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < N; ++n)
    for (int o = 0; o < C_out; ++o)
      for (int d = 0; d < Do; ++d)
        for (int h = 0; h < Ho; ++h)
          for (int ww = 0; ww < Wo; ++ww) {
            double v = conv3d_at(x, w, b, C_in, D, H, W, k, n, o, d, h, ww);
            y[((((size_t)n * C_out + o) * Do + d) * Ho + h) * Wo + ww] =
                oracle_lrelu_add_clamp_gelu(v, (double)s[o], slope, lo, hi);
          }
  return ORACLE_OK;
}

/* Same model at the given flat indices into the [N][C_out][Do][Ho][Wo] output. */
int oracle_conv3d_lrelu_add_clamp_gelu_at(const float *x, const float *w, const float *b,
                                          const float *s, int N, int C_in, int D, int H, int W,
                                          int C_out, int k, double slope, double lo, double hi,
                                          const int64_t *idx, int64_t count, double *out) {
  if (!x || !w || !s || !idx || !out || count < 0) return ORACLE_EBADARG;
  int Do = D - k + 1, Ho = H - k + 1, Wo = W - k + 1;
  if (Do < 1 || Ho < 1 || Wo < 1) return ORACLE_EBADARG;
  int64_t total = (int64_t)N * C_out * Do * Ho * Wo;
  for (int64_t j = 0; j < count; ++j)
    if (idx[j] < 0 || idx[j] >= total) return ORACLE_EBADARG;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j) {
    int64_t q = idx[j];
    int ww = (int)(q % Wo); q /= Wo;
    int h = (int)(q % Ho); q /= Ho;
    int d = (int)(q % Do); q /= Do;
    int o = (int)(q % C_out); q /= C_out;
    int n = (int)q;
    double v = conv3d_at(x, w, b, C_in, D, H, W, k, n, o, d, h, ww);
    out[j] = oracle_lrelu_add_clamp_gelu(v, (double)s[o], slope, lo, hi);
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* ConvTranspose2d -- l2_p10                                                  */
/* ------------------------------------------------------------------------ */

/* Output size of a transposed convolution, l2_p10's formula
 *   H_out = (H_in - 1) * stride - 2 * padding + kernel_size + output_padding
 * with output_padding = 0. */
int oracle_convT_out_size(int in, int k, int stride, int pad) { return (in - 1) * stride - 2 * pad + k; }

/* Scatter form, straight from what a transposed convolution does: every input
 * value x[n,i,ih,iw] is multiplied by the kernel W[i,o,:,:] and added into the
 * output at (ih*stride - pad + kh, iw*stride - pad + kw); positions that fall
 * outside the output are dropped.  The bias is added to every output.
 * z is [N][C_out][Ho][Wo]. */
int oracle_convT2d_scatter(const float *x, const float *w, const float *b, double *z, int N,
                           int C_in, int H, int W, int C_out, int k, int stride, int pad) {
  if (!x || !w || !z || N < 1 || C_in < 1 || C_out < 1 || k < 1 || stride < 1 || pad < 0)
    return ORACLE_EBADARG;
  int Ho = oracle_convT_out_size(H, k, stride, pad), Wo = oracle_convT_out_size(W, k, stride, pad);
  if (Ho < 1 || Wo < 1) return ORACLE_EBADARG;
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < N; ++n)
    for (int o = 0; o < C_out; ++o) {
      double *zp = z + ((size_t)n * C_out + o) * Ho * Wo;
      for (size_t p = 0; p < (size_t)Ho * Wo; ++p) zp[p] = bias_of(b, o);
      for (int i = 0; i < C_in; ++i)
        for (int ih = 0; ih < H; ++ih)
          for (int iw = 0; iw < W; ++iw) {
            double xv = x[(((size_t)n * C_in + i) * H + ih) * W + iw];
            for (int kh = 0; kh < k; ++kh)
              for (int kw = 0; kw < k; ++kw) {
                int oh = ih * stride - pad + kh, ow = iw * stride - pad + kw;
                if (oh < 0 || oh >= Ho || ow < 0 || ow >= Wo) continue;
                zp[(size_t)oh * Wo + ow] += xv * (double)w[(((size_t)i * C_out + o) * k + kh) * k + kw];
              }
          }
    }
  return ORACLE_OK;
}

/* Gather form of the same operator: output (h, w) collects every input
 * (ih, iw) and tap (kh, kw) with ih*stride - pad + kh = h, i.e.
 *   z[n,o,h,w] = b[o] + sum_{i,kh,kw} x[n,i,(h+pad-kh)/stride,(w+pad-kw)/stride] * W[i,o,kh,kw]
 * over taps where the division is exact and the input index is in range.  At
 * stride 1, pad 1 this is a correlation with the kernel flipped in both
 * spatial axes and with in/out channels swapped, the equivalence l2_p10
 * states as W' = W.permute(1,0,2,3).flip(2,3) with padding k-1-p. */
static double convT2d_gather_at(const float *x, const float *w, const float *b, int C_in, int H,
                                int W, int C_out, int k, int stride, int pad, int n, int o, int h,
                                int ww) {
  double acc = bias_of(b, o);
  for (int i = 0; i < C_in; ++i)
    for (int kh = 0; kh < k; ++kh) {
      int th = h + pad - kh;
      if (th < 0 || th % stride) continue;
      int ih = th / stride;
      if (ih >= H) continue;
      for (int kw = 0; kw < k; ++kw) {
        int tw = ww + pad - kw;
        if (tw < 0 || tw % stride) continue;
        int iw = tw / stride;
        if (iw >= W) continue;
        acc += (double)x[(((size_t)n * C_in + i) * H + ih) * W + iw] *
               (double)w[(((size_t)i * C_out + o) * k + kh) * k + kw];
      }
    }
  return acc;
}

int oracle_convT2d_gather(const float *x, const float *w, const float *b, double *z, int N,
                          int C_in, int H, int W, int C_out, int k, int stride, int pad) {
  if (!x || !w || !z || N < 1 || C_in < 1 || C_out < 1 || k < 1 || stride < 1 || pad < 0)
    return ORACLE_EBADARG;
  int Ho = oracle_convT_out_size(H, k, stride, pad), Wo = oracle_convT_out_size(W, k, stride, pad);
  if (Ho < 1 || Wo < 1) return ORACLE_EBADARG;
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < N; ++n)
    for (int o = 0; o < C_out; ++o)
      for (int h = 0; h < Ho; ++h)
        for (int ww = 0; ww < Wo; ++ww)
          z[(((size_t)n * C_out + o) * Ho + h) * Wo + ww] =
              convT2d_gather_at(x, w, b, C_in, H, W, C_out, k, stride, pad, n, o, h, ww);
  return ORACLE_OK;
}

/* MaxPool2d output size with padding 0 and dilation 1, from l2_p10's
 * floor((H + 2*padding - dilation*(kernel_size-1) - 1) / stride + 1). */
int oracle_pool_out_size(int in, int pk, int ps) {
  if (in < pk) return 0;
  return (in - pk) / ps + 1;
}

/* Epilogue of l2_p10 on one (n, o) plane z[Ho][Wo] of the transposed conv:
 * MaxPool2d(pk, ps) -> Hardtanh[lo, hi] -> mean over the pooled plane -> tanh.
 * The mean divides by the pooled element count (l2_p10: 1/16384 for 128x128). */
double oracle_pool_htanh_mean_tanh_plane(const double *z, int Ho, int Wo, int pk, int ps, double lo,
                                         double hi) {
  int PH = oracle_pool_out_size(Ho, pk, ps), PW = oracle_pool_out_size(Wo, pk, ps);
  double sum = 0.0;
  for (int ph = 0; ph < PH; ++ph)
    for (int pw = 0; pw < PW; ++pw) {
      double m = z[(size_t)(ph * ps) * Wo + (pw * ps)];
      for (int dh = 0; dh < pk; ++dh)
        for (int dw = 0; dw < pk; ++dw) {
          double v = z[(size_t)(ph * ps + dh) * Wo + (pw * ps + dw)];
          if (v > m) m = v;
        }
      sum += oracle_clamp(m, lo, hi);
    }
  return tanh(sum / ((double)PH * (double)PW));
}

/* One (n, o) plane of the transposed conv, z[Ho][Wo], in the scatter form
 * with the kernel taps outermost: start from the bias, then for each input
 * channel i and tap (kh, kw) in turn, add the input plane x[n,i] times
 * W[i,o,kh,kw] into the output at (ih*stride - pad + kh, iw*stride - pad + kw),
 * dropping positions outside the output.  Each output receives its terms in
 * ascending (i, kh, kw) order -- the order of the gather form above -- so the
 * two evaluations give the same doubles (the tests pin that bit for bit); this
 * order reads each input plane row by row. */
static void convT2d_plane(const float *x, const float *w, const float *b, int C_in, int H, int W,
                          int C_out, int k, int stride, int pad, int n, int o, double *z) {
  int Ho = oracle_convT_out_size(H, k, stride, pad), Wo = oracle_convT_out_size(W, k, stride, pad);
  for (size_t p = 0; p < (size_t)Ho * Wo; ++p) z[p] = bias_of(b, o);
  for (int i = 0; i < C_in; ++i) {
    const float *xp = x + ((size_t)n * C_in + i) * H * W;
    for (int kh = 0; kh < k; ++kh)
      for (int kw = 0; kw < k; ++kw) {
        double wv = (double)w[(((size_t)i * C_out + o) * k + kh) * k + kw];
        for (int ih = 0; ih < H; ++ih) {
          int oh = ih * stride - pad + kh;
          if (oh < 0 || oh >= Ho) continue;
          for (int iw = 0; iw < W; ++iw) {
            int ow = iw * stride - pad + kw;
            if (ow < 0 || ow >= Wo) continue;
            z[(size_t)oh * Wo + ow] += (double)xp[(size_t)ih * W + iw] * wv;
          }
        }
      }
  }
}

/* y[N][C_out] (= [N,C_out,1,1]) = tanh(mean(hardtanh(maxpool(convT2d(x))))),
 * the whole l2_p10 model, one (n, o) plane at a time. */
static int convT_model_plane(const float *x, const float *w, const float *b, int C_in, int H,
                             int W, int C_out, int k, int stride, int pad, int pk, int ps,
                             double lo, double hi, int n, int o, double *plane, double *out) {
  int Ho = oracle_convT_out_size(H, k, stride, pad), Wo = oracle_convT_out_size(W, k, stride, pad);
  convT2d_plane(x, w, b, C_in, H, W, C_out, k, stride, pad, n, o, plane);
  *out = oracle_pool_htanh_mean_tanh_plane(plane, Ho, Wo, pk, ps, lo, hi);
  return ORACLE_OK;
}

/* The transposed conv's output planes as the model path computes them
 * (convT2d_plane), z[N][C_out][Ho][Wo]: lets the tests compare that path with
 * the gather and scatter forms directly. */
int oracle_convT2d_planes(const float *x, const float *w, const float *b, double *z, int N,
                          int C_in, int H, int W, int C_out, int k, int stride, int pad) {
  if (!x || !w || !z || N < 1 || C_in < 1 || C_out < 1 || k < 1 || stride < 1 || pad < 0)
    return ORACLE_EBADARG;
  int Ho = oracle_convT_out_size(H, k, stride, pad), Wo = oracle_convT_out_size(W, k, stride, pad);
  if (Ho < 1 || Wo < 1) return ORACLE_EBADARG;
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < N; ++n)
    for (int o = 0; o < C_out; ++o)
      convT2d_plane(x, w, b, C_in, H, W, C_out, k, stride, pad, n, o,
                    z + ((size_t)n * C_out + o) * Ho * Wo);
  return ORACLE_OK;
}

/* The caller provides `scratch`, room for (number of threads) * Ho * Wo
 * doubles, so the oracle itself never allocates. */
int oracle_convT2d_pool_htanh_mean_tanh_at(const float *x, const float *w, const float *b, int N,
                                           int C_in, int H, int W, int C_out, int k, int stride,
                                           int pad, int pk, int ps, double lo, double hi,
                                           const int64_t *nc_idx, int64_t count, double *scratch,
                                           int64_t scratch_doubles, double *out) {
  if (!x || !w || !nc_idx || !out || !scratch || count < 0 || pk < 1 || ps < 1) return ORACLE_EBADARG;
  int Ho = oracle_convT_out_size(H, k, stride, pad), Wo = oracle_convT_out_size(W, k, stride, pad);
  if (Ho < 1 || Wo < 1) return ORACLE_EBADARG;
  if (oracle_pool_out_size(Ho, pk, ps) < 1 || oracle_pool_out_size(Wo, pk, ps) < 1) return ORACLE_EBADARG;
  int nt = oracle_num_threads();
  if (scratch_doubles < (int64_t)nt * Ho * Wo) return ORACLE_EBADARG;
  for (int64_t j = 0; j < count; ++j)
    if (nc_idx[j] < 0 || nc_idx[j] >= (int64_t)N * C_out) return ORACLE_EBADARG;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t j = 0; j < count; ++j) {
    int t = 0;
#ifdef _OPENMP
    t = omp_get_thread_num();
#endif
    double *plane = scratch + (size_t)t * Ho * Wo;
    int n = (int)(nc_idx[j] / C_out), o = (int)(nc_idx[j] % C_out);
    convT_model_plane(x, w, b, C_in, H, W, C_out, k, stride, pad, pk, ps, lo, hi, n, o, plane, &out[j]);
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Epilogue-only operators over a precomputed convolution output            */
/* ------------------------------------------------------------------------ */

/* l2_p10's fused tail, the path that page implemented after a library
 * transposed conv: y[n,c] = tanh(mean(Hardtanh(MaxPool2d(z[n,c])))) for every
 * (n, c) plane of z[N][C][H][W].  Each plane goes through the same plane
 * function as the fused model above. */
int oracle_pool_htanh_mean_tanh(const double *z, double *y, int N, int C, int H, int W, int pk,
                                int ps, double lo, double hi) {
  if (!z || !y || N < 1 || C < 1 || pk < 1 || ps < 1) return ORACLE_EBADARG;
  if (oracle_pool_out_size(H, pk, ps) < 1 || oracle_pool_out_size(W, pk, ps) < 1) return ORACLE_EBADARG;
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < N; ++n)
    for (int c = 0; c < C; ++c)
      y[(size_t)n * C + c] =
          oracle_pool_htanh_mean_tanh_plane(z + ((size_t)n * C + c) * H * W, H, W, pk, ps, lo, hi);
  return ORACLE_OK;
}

/* Same tail reading fp32 input (what the GPU operator consumes): each plane
 * is widened to double in the caller's scratch (room for (number of threads)
 * * H * W doubles) and goes through the plane function above. */
int oracle_pool_htanh_mean_tanh_f32(const float *z, double *y, int N, int C, int H, int W, int pk,
                                    int ps, double lo, double hi, double *scratch,
                                    int64_t scratch_doubles) {
  if (!z || !y || !scratch || N < 1 || C < 1 || H < 1 || W < 1 || pk < 1 || ps < 1)
    return ORACLE_EBADARG;
  if (oracle_pool_out_size(H, pk, ps) < 1 || oracle_pool_out_size(W, pk, ps) < 1) return ORACLE_EBADARG;
  if (scratch_doubles < (int64_t)oracle_num_threads() * H * W) return ORACLE_EBADARG;
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < N; ++n)
    for (int c = 0; c < C; ++c) {
      int t = 0;
#ifdef _OPENMP
      t = omp_get_thread_num();
#endif
      double *plane = scratch + (size_t)t * H * W;
      const float *zp = z + ((size_t)n * C + c) * H * W;
      for (size_t p = 0; p < (size_t)H * W; ++p) plane[p] = (double)zp[p];
      y[(size_t)n * C + c] = oracle_pool_htanh_mean_tanh_plane(plane, H, W, pk, ps, lo, hi);
    }
  return ORACLE_OK;
}

/* l2_p90's elementwise fallback after a library Conv3d: for z[N][C][S] (S =
 * spatial elements per channel), y = GELU(clamp(LeakyReLU(z) + s[c], lo, hi)),
 * each element through the same scalar epilogue as the fused model. */
int oracle_lrelu_add_clamp_gelu_f32(const float *z, const float *s, double *y, int N, int C,
                                    int64_t S, double slope, double lo, double hi) {
  if (!z || !s || !y || N < 1 || C < 1 || S < 1) return ORACLE_EBADARG;
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < N; ++n)
    for (int c = 0; c < C; ++c) {
      const size_t base = ((size_t)n * C + c) * (size_t)S;
      for (int64_t e = 0; e < S; ++e)
        y[base + e] = oracle_lrelu_add_clamp_gelu((double)z[base + e], (double)s[c], slope, lo, hi);
    }
  return ORACLE_OK;
}
