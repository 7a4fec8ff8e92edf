/*
 * oracle.c -- plain, slow, direct-loop CPU implementation of the convolutional
 * block backward pass, in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link or call this file; it exists so the
 * tests, the smoke check and the CPU-baseline leg of the benchmark can compare
 * the GPU results against an independent reading of the pages.  It shares no
 * source, header, table or helper with the HIP code.
 *
 * Every loop below is the textbook definition of the quantity, written out in
 * the order the pages state it; there is no blocking, tiling or reordering.
 * Parallel loops (OpenMP) split only over independent output elements, so the
 * summation order of every output value is fixed and the result does not depend
 * on the thread count.
 *
 * Pages cited (title, address), tagged [P1]..[P5] below:
 *  [P1] "YOLOv3 backpropagation: full-flow source analysis"
 *       (suzhouguqin.com/content/1291550.html)
 *  [P2] "Caffe source study ch.4 (5): the LeNet backward pass"
 *       (csdndocs.com/article/9344743)
 *  [P3] "AlexeyAB DarkNet analysis (4): network forward/backward and the layer struct"
 *       (m.dandelioncloud.cn/article/details/1675816420510003202)
 *  [P4] "caffe source study -- one article is enough"
 *       (geek-share.com/detail/2722348220.html)
 *  [P5] "Understanding BatchNorm" (javaforall.cn/143067.html)
 *
 * Layouts: activations NCHW contiguous (the delta/output layout of the layer
 * struct in [P3], Blob::offset in [P4]); conv weights OIHW ([P3] layer struct,
 * "weights"); inner-product weights out x in ([P2] layer 8).
 */
#include <math.h>
#include <stddef.h>
#include <string.h>

#define ORC_ACT_LINEAR 0
#define ORC_ACT_LEAKY 1
#define ORC_ACT_LOGISTIC 2
#define ORC_ACT_RELU 3
#define ORC_ACT_TANH 4
#define ORC_ACT_ELU 5
#define ORC_ACT_SELU 6
#define ORC_ACT_PLSE 7
#define ORC_ACT_LHTAN 8
#define ORC_ACT_HARDTAN 9
#define ORC_ACT_STAIR 10
#define ORC_ACT_RAMP 11
#define ORC_ACT_RELIE 12
#define ORC_ACT_LOGGY 13

int orc_version(void) { return 1; }

#ifdef _OPENMP
#include <omp.h>
int orc_num_threads(void) { return omp_get_max_threads(); }
/* threads of the following parallel loops (timing the oracle on one core) */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int orc_num_threads(void) { return 1; }
void orc_set_threads(int n) { (void)n; }
#endif

/* ------------------------------------------------------------------ */
/* activations                                                         */
/* ------------------------------------------------------------------ */

/* Forward activations used to build saved tensors, as the *_activate functions
 * of [P1] section 7 define them: linear x, logistic 1/(1+e^-x), relu x*(x>0),
 * leaky (x>0)?x:0.1x (the slope is a parameter here, 0.1 in all pages' uses);
 * tanh (e^2x-1)/(e^2x+1) (written as tanh(), the same function without the
 * overflow of e^2x); elu x for x>=0, e^x-1 below; selu 1.0507 x for x>=0,
 * 1.0507*1.6732 (e^x-1) below; plse .01(x+4) below -4, .01(x-4)+1 above 4,
 * .125x+.5 between; lhtan .001x below 0, .001(x-1)+1 above 1, x between;
 * hardtan x clamped to [-1, 1]; stair with n = floor(x): floor(x/2) for even n,
 * (x-n)+floor(x/2) for odd n; ramp x*(x>0)+.1x; relie x for x>0, .01x otherwise;
 * loggy 2/(1+e^-x)-1. */
static double act_fwd(int act, double slope, double u) {
  switch (act) {
    case ORC_ACT_LINEAR: return u;
    case ORC_ACT_LEAKY: return (u > 0) ? u : slope * u;
    case ORC_ACT_LOGISTIC: return 1.0 / (1.0 + exp(-u));
    case ORC_ACT_RELU: return (u > 0) ? u : 0.0;
    case ORC_ACT_TANH: return tanh(u);
    case ORC_ACT_ELU: return (u >= 0) ? u : exp(u) - 1.0;
    case ORC_ACT_SELU: return (u >= 0) ? 1.0507 * u : 1.0507 * 1.6732 * (exp(u) - 1.0);
    case ORC_ACT_PLSE:
      if (u < -4) return .01 * (u + 4);
      if (u > 4) return .01 * (u - 4) + 1;
      return .125 * u + .5;
    case ORC_ACT_LHTAN:
      if (u < 0) return .001 * u;
      if (u > 1) return .001 * (u - 1) + 1;
      return u;
    case ORC_ACT_HARDTAN: return (u < -1) ? -1.0 : ((u > 1) ? 1.0 : u);
    case ORC_ACT_STAIR: {
      const double n = floor(u);
      if (fmod(n, 2.0) == 0) return floor(u / 2.);
      return (u - n) + floor(u / 2.);
    }
    case ORC_ACT_RAMP: return u * (u > 0) + .1 * u;
    case ORC_ACT_RELIE: return (u > 0) ? u : .01 * u;
    case ORC_ACT_LOGGY: return 2. / (1. + exp(-u)) - 1;
  }
  return NAN;
}

/* Activation derivative evaluated on the OUTPUT y, as Darknet's *_gradient
 * functions do ([P1] section 7): linear 1; leaky (y>0)?1:slope; logistic
 * (1-y)y; relu (y>0); tanh 1-y^2; elu (y>=0) + (y<0)(y+1); selu (y>=0)1.0507 +
 * (y<0)(y + 1.0507*1.6732); plse (y<0 || y>1) ? .01 : .125; lhtan (0<y<1) ? 1 :
 * .001; hardtan (-1<y<1) ? 1 : 0; stair floor(y)==y ? 0 : 1; ramp (y>0) + .1;
 * relie (y>0) ? 1 : .01; loggy 2(1-s)s with s = (y+1)/2. */
static double act_grad(int act, double slope, double y) {
  switch (act) {
    case ORC_ACT_LINEAR: return 1.0;
    case ORC_ACT_LEAKY: return (y > 0) ? 1.0 : slope;
    case ORC_ACT_LOGISTIC: return (1.0 - y) * y;
    case ORC_ACT_RELU: return (y > 0) ? 1.0 : 0.0;
    case ORC_ACT_TANH: return 1.0 - y * y;
    case ORC_ACT_ELU: return (y >= 0) + (y < 0) * (y + 1.0);
    case ORC_ACT_SELU: return (y >= 0) * 1.0507 + (y < 0) * (y + 1.0507 * 1.6732);
    case ORC_ACT_PLSE: return (y < 0 || y > 1) ? .01 : .125;
    case ORC_ACT_LHTAN: return (y > 0 && y < 1) ? 1.0 : .001;
    case ORC_ACT_HARDTAN: return (y > -1 && y < 1) ? 1.0 : 0.0;
    case ORC_ACT_STAIR: return (floor(y) == y) ? 0.0 : 1.0;
    case ORC_ACT_RAMP: return (y > 0) + .1;
    case ORC_ACT_RELIE: return (y > 0) ? 1.0 : .01;
    case ORC_ACT_LOGGY: {
      const double s = (y + 1.) / 2.;
      return 2 * (1 - s) * s;
    }
  }
  return NAN;
}

void orc_act_forward(int act, double slope, const double* u, double* y, long count) {
#pragma omp parallel for schedule(static)
  for (long i = 0; i < count; ++i) y[i] = act_fwd(act, slope, u[i]);
}

/* gradient_array ([P1] section 3.1 and section 7): g = delta * act'(y). */
void orc_act_backward(int act, double slope, const double* y, const double* delta, double* g,
                      long count) {
#pragma omp parallel for schedule(static)
  for (long i = 0; i < count; ++i) g[i] = delta[i] * act_grad(act, slope, y[i]);
}

/* ------------------------------------------------------------------ */
/* batch normalisation                                                 */
/* ------------------------------------------------------------------ */

/* Training-mode forward, per channel over (batch, spatial): mean, BIASED
 * variance E[(z-mean)^2] (the one Caffe normalises with, [P5] Forward_cpu),
 * xhat = (z-mean)/sqrt(var+eps) with eps inside the root, u = gamma*xhat+beta
 * (scale_bias / add_bias of [P1] section 4). */
void orc_bn_forward(int n, int c, long hw, double eps, const double* z, const double* gamma,
                    const double* beta, double* mean, double* var, double* xhat, double* u) {
  const double m = (double)n * (double)hw;
#pragma omp parallel for schedule(dynamic, 1)
  for (int ch = 0; ch < c; ++ch) {
    double s = 0.0;
    for (int b = 0; b < n; ++b)
      for (long i = 0; i < hw; ++i) s += z[((long)b * c + ch) * hw + i];
    const double mu = s / m;
    double v = 0.0;
    for (int b = 0; b < n; ++b)
      for (long i = 0; i < hw; ++i) {
        const double d = z[((long)b * c + ch) * hw + i] - mu;
        v += d * d;
      }
    v /= m;
    mean[ch] = mu;
    var[ch] = v;
    const double inv = 1.0 / sqrt(v + eps);
    for (int b = 0; b < n; ++b)
      for (long i = 0; i < hw; ++i) {
        const long idx = ((long)b * c + ch) * hw + i;
        xhat[idx] = (z[idx] - mu) * inv;
        u[idx] = gamma[ch] * xhat[idx] + beta[ch];
      }
  }
}

/* Training-mode BN backward from g = dL/du.
 * Steps in the order of backward_batchnorm_layer ([P1] section 4):
 *   backward_bias:       dbeta_c  += sum g
 *   backward_scale_cpu:  dgamma_c += sum g * xhat
 *   scale_bias:          g' = gamma_c * g
 * then the input gradient in the closed form of Caffe's BatchNormLayer
 * Backward_cpu ([P5]), which takes exactly xhat and sqrt(var+eps):
 *   dz = (g' - mean(g') - mean(g' * xhat) * xhat) / sqrt(var + eps)
 * means over (batch, spatial).  [P5] states this equals the three-step
 * mean_delta / variance_delta / normalize_delta route of [P1] section 4; the
 * tests check that equality independently. */
void orc_bn_backward(int n, int c, long hw, double eps, const double* g, const double* xhat,
                     const double* var, const double* gamma, double* dz, double* dgamma,
                     double* dbeta) {
  const double m = (double)n * (double)hw;
#pragma omp parallel for schedule(dynamic, 1)
  for (int ch = 0; ch < c; ++ch) {
    double sg = 0.0, sgx = 0.0;
    for (int b = 0; b < n; ++b)
      for (long i = 0; i < hw; ++i) {
        const long idx = ((long)b * c + ch) * hw + i;
        sg += g[idx];
        sgx += g[idx] * xhat[idx];
      }
    dbeta[ch] += sg;
    dgamma[ch] += sgx;
    const double gm = gamma[ch];
    const double mean_g = gm * sg / m;      /* mean(g')        */
    const double mean_gx = gm * sgx / m;    /* mean(g' * xhat) */
    const double sd = sqrt(var[ch] + eps);
    for (int b = 0; b < n; ++b)
      for (long i = 0; i < hw; ++i) {
        const long idx = ((long)b * c + ch) * hw + i;
        dz[idx] = (gm * g[idx] - mean_g - mean_gx * xhat[idx]) / sd;
      }
  }
}

/* Forward with fixed (stored) statistics: xhat = (z - mean)/sqrt(var + eps)
 * with the given mean and variance, u = gamma*xhat + beta (normalize_cpu with
 * the rolling mean and variance when not training, [P1] section 4; Caffe's
 * use_global_stats, [P5] Forward_cpu). */
void orc_bn_forward_fixed(int n, int c, long hw, double eps, const double* z, const double* mean,
                          const double* var, const double* gamma, const double* beta,
                          double* xhat, double* u) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int ch = 0; ch < c; ++ch) {
    const double inv = 1.0 / sqrt(var[ch] + eps);
    for (int b = 0; b < n; ++b)
      for (long i = 0; i < hw; ++i) {
        const long idx = ((long)b * c + ch) * hw + i;
        xhat[idx] = (z[idx] - mean[ch]) * inv;
        u[idx] = gamma[ch] * xhat[idx] + beta[ch];
      }
  }
}

/* Backward with fixed statistics from g = dL/du.  The mean and variance do not
 * depend on z, so u is affine in z per channel.  backward_bias and
 * backward_scale_cpu as in training ([P1] section 4), scale_bias by gamma, then
 * Caffe's use_global_stats branch of Backward_cpu ([P5]), which divides the top
 * gradient by sqrt(var + eps):
 *   dbeta += sum g;  dgamma += sum g*xhat;  dz = gamma*g / sqrt(var + eps). */
void orc_bn_backward_fixed(int n, int c, long hw, double eps, const double* g, const double* xhat,
                           const double* var, const double* gamma, double* dz, double* dgamma,
                           double* dbeta) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int ch = 0; ch < c; ++ch) {
    double sg = 0.0, sgx = 0.0;
    const double sd = sqrt(var[ch] + eps);
    for (int b = 0; b < n; ++b)
      for (long i = 0; i < hw; ++i) {
        const long idx = ((long)b * c + ch) * hw + i;
        sg += g[idx];
        sgx += g[idx] * xhat[idx];
        dz[idx] = gamma[ch] * g[idx] / sd;
      }
    dbeta[ch] += sg;
    dgamma[ch] += sgx;
  }
}

/* ------------------------------------------------------------------ */
/* convolution                                                         */
/* ------------------------------------------------------------------ */

/* Output size of a padded strided window, im2col_cpu of [P1] section 3.2:
 * (size + 2*pad - ksize)/stride + 1. */
int orc_conv_out_dim(int size, int k, int s, int p) { return (size + 2 * p - k) / s + 1; }

/* Input value at (row, col) of plane `plane`, zero outside the image (the
 * padding reading of im2col_get_pixel, whose body the pages do not show). */
static double pix(const double* plane, int h, int w, int row, int col) {
  if (row < 0 || col < 0 || row >= h || col >= w) return 0.0;
  return plane[(long)row * w + col];
}

/* Forward convolution (cross-correlation, as im2col + gemm computes it):
 * z[n,o,ho,wo] = sum_{i,kh,kw} W[o,i,kh,kw] * x[n,i,ho*s+kh-p,wo*s+kw-p] (+b[o]). */
void orc_conv_forward(int n, int c, int h, int w, int oc, int k, int s, int p, const double* x,
                      const double* wt, const double* bias, double* z) {
  const int oh = orc_conv_out_dim(h, k, s, p), ow = orc_conv_out_dim(w, k, s, p);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < n; ++b)
    for (int o = 0; o < oc; ++o)
      for (int y = 0; y < oh; ++y)
        for (int xo = 0; xo < ow; ++xo) {
          double acc = bias ? bias[o] : 0.0;
          for (int i = 0; i < c; ++i) {
            const double* plane = x + ((long)b * c + i) * h * w;
            for (int kh = 0; kh < k; ++kh)
              for (int kw = 0; kw < k; ++kw)
                acc += wt[(((long)o * c + i) * k + kh) * k + kw] *
                       pix(plane, h, w, y * s + kh - p, xo * s + kw - p);
          }
          z[(((long)b * oc + o) * oh + y) * ow + xo] = acc;
        }
}

/* Weight gradient, the gemm(0,1,...,beta=1) of backward_convolutional_layer
 * ([P1] section 3.1) summed over images (section 1.2: per-image gradients are
 * accumulated, not averaged):
 *   dW[o,i,kh,kw] += sum_{n,ho,wo} dz[n,o,ho,wo] * x[n,i,ho*s+kh-p,wo*s+kw-p]. */
void orc_conv_backward_weights(int n, int c, int h, int w, int oc, int k, int s, int p,
                               const double* x, const double* dz, double* dw) {
  const int oh = orc_conv_out_dim(h, k, s, p), ow = orc_conv_out_dim(w, k, s, p);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int o = 0; o < oc; ++o)
    for (int i = 0; i < c; ++i)
      for (int kh = 0; kh < k; ++kh)
        for (int kw = 0; kw < k; ++kw) {
          double acc = 0.0;
          for (int b = 0; b < n; ++b) {
            const double* plane = x + ((long)b * c + i) * h * w;
            const double* d = dz + ((long)b * oc + o) * oh * ow;
            for (int y = 0; y < oh; ++y)
              for (int xo = 0; xo < ow; ++xo)
                acc += d[(long)y * ow + xo] * pix(plane, h, w, y * s + kh - p, xo * s + kw - p);
          }
          dw[(((long)o * c + i) * k + kh) * k + kw] += acc;
        }
}

/* One weight-gradient element (same sum as above, not accumulated). */
double orc_conv_dw_at(int n, int c, int h, int w, int oc, int k, int s, int p, const double* x,
                      const double* dz, int o, int i, int kh, int kw) {
  const int oh = orc_conv_out_dim(h, k, s, p), ow = orc_conv_out_dim(w, k, s, p);
  double acc = 0.0;
  for (int b = 0; b < n; ++b) {
    const double* plane = x + ((long)b * c + i) * h * w;
    const double* d = dz + ((long)b * oc + o) * oh * ow;
    for (int y = 0; y < oh; ++y)
      for (int xo = 0; xo < ow; ++xo)
        acc += d[(long)y * ow + xo] * pix(plane, h, w, y * s + kh - p, xo * s + kw - p);
  }
  return acc;
}

/* Bias gradient, backward_bias ([P1] section 3.1 / section 4; Caffe
 * backward_cpu_bias in [P2] layer 4): db[o] += sum_{n,ho,wo} dz[n,o,ho,wo]. */
void orc_conv_backward_bias(int n, int oc, long ohw, const double* dz, double* db) {
#pragma omp parallel for schedule(static)
  for (int o = 0; o < oc; ++o) {
    double acc = 0.0;
    for (int b = 0; b < n; ++b)
      for (long i = 0; i < ohw; ++i) acc += dz[((long)b * oc + o) * ohw + i];
    db[o] += acc;
  }
}

/* Input gradient: the gemm(1,0,...) W^T x delta of backward_convolutional_layer
 * followed by col2im_cpu, which ADDS every column value back at the pixel
 * im2col read it from ([P1] section 3.2).  Written as that scatter, without the
 * column buffer: for every (o, ho, wo, kh, kw),
 *   dx[n,i,ho*s+kh-p,wo*s+kw-p] += W[o,i,kh,kw] * dz[n,o,ho,wo]  (in-image taps only).
 * Each (n,i) plane is owned by one thread; within it the contributions are
 * added in (o, ho, wo, kh, kw) order. */
void orc_conv_backward_data(int n, int c, int h, int w, int oc, int k, int s, int p,
                            const double* wt, const double* dz, double* dx) {
  const int oh = orc_conv_out_dim(h, k, s, p), ow = orc_conv_out_dim(w, k, s, p);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < n; ++b)
    for (int i = 0; i < c; ++i) {
      double* plane = dx + ((long)b * c + i) * h * w;
      for (int o = 0; o < oc; ++o) {
        const double* d = dz + ((long)b * oc + o) * oh * ow;
        for (int y = 0; y < oh; ++y)
          for (int xo = 0; xo < ow; ++xo) {
            const double dv = d[(long)y * ow + xo];
            for (int kh = 0; kh < k; ++kh)
              for (int kw = 0; kw < k; ++kw) {
                const int row = y * s + kh - p, col = xo * s + kw - p;
                if (row < 0 || col < 0 || row >= h || col >= w) continue;
                plane[(long)row * w + col] += wt[(((long)o * c + i) * k + kh) * k + kw] * dv;
              }
          }
      }
    }
}

/* One input-gradient element: the same sum, collected at a single pixel
 * (all (o, ho, wo, kh, kw) whose tap lands on (row, col)), not accumulated. */
double orc_conv_dx_at(int n, int c, int h, int w, int oc, int k, int s, int p, const double* wt,
                      const double* dz, int b, int i, int row, int col) {
  const int oh = orc_conv_out_dim(h, k, s, p), ow = orc_conv_out_dim(w, k, s, p);
  (void)n;
  double acc = 0.0;
  for (int o = 0; o < oc; ++o) {
    const double* d = dz + ((long)b * oc + o) * oh * ow;
    for (int kh = 0; kh < k; ++kh)
      for (int kw = 0; kw < k; ++kw) {
        const int ty = row + p - kh, tx = col + p - kw;
        if (ty < 0 || tx < 0 || ty % s || tx % s) continue;
        const int y = ty / s, xo = tx / s;
        if (y >= oh || xo >= ow) continue;
        acc += wt[(((long)o * c + i) * k + kh) * k + kw] * d[(long)y * ow + xo];
      }
  }
  return acc;
}

/* ------------------------------------------------------------------ */
/* max pooling                                                         */
/* ------------------------------------------------------------------ */

/* Forward max pool (square window k, stride s, no padding); idx holds the
 * per-plane flat index h*W+w of the winner, the mask Caffe's backward reads
 * ([P2] layer 5).  Ties: first maximum in row-major window order. */
void orc_maxpool_forward(int n, int c, int h, int w, int k, int s, const double* x, double* y,
                         int* idx) {
  const int oh = (h - k) / s + 1, ow = (w - k) / s + 1;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < n; ++b)
    for (int ch = 0; ch < c; ++ch) {
      const double* plane = x + ((long)b * c + ch) * h * w;
      for (int py = 0; py < oh; ++py)
        for (int px = 0; px < ow; ++px) {
          int best = -1;
          double bv = 0.0;
          for (int ky = 0; ky < k; ++ky)
            for (int kx = 0; kx < k; ++kx) {
              const int r = py * s + ky, q = px * s + kx;
              const double v = plane[(long)r * w + q];
              if (best < 0 || v > bv) { best = r * w + q; bv = v; }
            }
          const long o = (((long)b * c + ch) * oh + py) * ow + px;
          y[o] = bv;
          idx[o] = best;
        }
    }
}

/* Max-pool backward ([P2] layer 5): clear bottom_diff, then for every pooled
 * output add its top_diff at the bottom position its mask names. */
void orc_maxpool_backward(int n, int c, int ih, int iw, int oh, int ow, const int* idx,
                          const double* delta, double* dx) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < n; ++b)
    for (int ch = 0; ch < c; ++ch) {
      double* plane = dx + ((long)b * c + ch) * ih * iw;
      const long base = ((long)b * c + ch) * oh * ow;
      for (long i = 0; i < (long)ih * iw; ++i) plane[i] = 0.0;
      for (long j = 0; j < (long)oh * ow; ++j) plane[idx[base + j]] += delta[base + j];
    }
}

/* ------------------------------------------------------------------ */
/* grouped and dilated convolution                                     */
/* ------------------------------------------------------------------ */

/* Output size with dilation d: the window spans d*(k-1)+1 input pixels. */
int orc_conv_out_dim_d(int size, int k, int s, int p, int d) {
  return (size + 2 * p - d * (k - 1) - 1) / s + 1;
}

/* Grouped, dilated convolution.  Group j ([P1] section 3.1,
 * backward_convolutional_layer with l.groups) owns output channels
 * [j*oc/g, (j+1)*oc/g), input channels [j*c/g, (j+1)*c/g) and weight block j
 * ([oc][c/g][k][k]); tap (kh, kw) of output (ho, wo) reads input row
 * ho*s + kh*d - p and column wo*s + kw*d - p (the layer's dilation field, [P3];
 * zero outside the image).
 *   z[n,o,ho,wo] = sum_{i in group, kh, kw} W[o,i-c0,kh,kw] * x[n,i,ho*s+kh*d-p,wo*s+kw*d-p] */
void orc_conv_forward_gd(int n, int c, int h, int w, int oc, int k, int s, int p, int d, int groups,
                         const double* x, const double* wt, const double* bias, double* z) {
  const int oh = orc_conv_out_dim_d(h, k, s, p, d), ow = orc_conv_out_dim_d(w, k, s, p, d);
  const int cg = c / groups, og = oc / groups;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < n; ++b)
    for (int o = 0; o < oc; ++o) {
      const int c0 = (o / og) * cg;
      for (int y = 0; y < oh; ++y)
        for (int xo = 0; xo < ow; ++xo) {
          double acc = bias ? bias[o] : 0.0;
          for (int i = 0; i < cg; ++i)
            for (int kh = 0; kh < k; ++kh)
              for (int kw = 0; kw < k; ++kw) {
                const int row = y * s + kh * d - p, col = xo * s + kw * d - p;
                if (row < 0 || col < 0 || row >= h || col >= w) continue;
                acc += wt[(((long)o * cg + i) * k + kh) * k + kw] *
                       x[(((long)b * c + c0 + i) * h + row) * w + col];
              }
          z[(((long)b * oc + o) * oh + y) * ow + xo] = acc;
        }
    }
}

/* dW[o,i,kh,kw] += sum_{n,ho,wo} dz[n,o,ho,wo] * x[n, c0+i, ho*s+kh*d-p, wo*s+kw*d-p]
 * (the gemm(0,1,...) of group j with beta = 1, accumulated over the images). */
void orc_conv_backward_weights_gd(int n, int c, int h, int w, int oc, int k, int s, int p, int d,
                                  int groups, const double* x, const double* dz, double* dw) {
  const int oh = orc_conv_out_dim_d(h, k, s, p, d), ow = orc_conv_out_dim_d(w, k, s, p, d);
  const int cg = c / groups, og = oc / groups;
#pragma omp parallel for schedule(dynamic, 1)
  for (int o = 0; o < oc; ++o) {
    const int c0 = (o / og) * cg;
    for (int i = 0; i < cg; ++i)
      for (int kh = 0; kh < k; ++kh)
        for (int kw = 0; kw < k; ++kw) {
          double acc = 0.0;
          for (int b = 0; b < n; ++b)
            for (int y = 0; y < oh; ++y)
              for (int xo = 0; xo < ow; ++xo) {
                const int row = y * s + kh * d - p, col = xo * s + kw * d - p;
                if (row < 0 || col < 0 || row >= h || col >= w) continue;
                acc += dz[(((long)b * oc + o) * oh + y) * ow + xo] *
                       x[(((long)b * c + c0 + i) * h + row) * w + col];
              }
          dw[(((long)o * cg + i) * k + kh) * k + kw] += acc;
        }
  }
}

/* dX of input channel i (group j = i / (c/g)): the col2im scatter of W^T x dz
 * over the group's output channels, dilated taps as in the forward. */
void orc_conv_backward_data_gd(int n, int c, int h, int w, int oc, int k, int s, int p, int d,
                               int groups, const double* wt, const double* dz, double* dx) {
  const int oh = orc_conv_out_dim_d(h, k, s, p, d), ow = orc_conv_out_dim_d(w, k, s, p, d);
  const int cg = c / groups, og = oc / groups;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < n; ++b)
    for (int i = 0; i < c; ++i) {
      const int j = i / cg, il = i - j * cg;
      double* plane = dx + ((long)b * c + i) * h * w;
      for (int o = j * og; o < (j + 1) * og; ++o) {
        const double* dzp = dz + ((long)b * oc + o) * oh * ow;
        for (int y = 0; y < oh; ++y)
          for (int xo = 0; xo < ow; ++xo) {
            const double dv = dzp[(long)y * ow + xo];
            for (int kh = 0; kh < k; ++kh)
              for (int kw = 0; kw < k; ++kw) {
                const int row = y * s + kh * d - p, col = xo * s + kw * d - p;
                if (row < 0 || col < 0 || row >= h || col >= w) continue;
                plane[(long)row * w + col] += wt[(((long)o * cg + il) * k + kh) * k + kw] * dv;
              }
          }
      }
    }
}

/* ------------------------------------------------------------------ */
/* inner product and softmax loss                                      */
/* ------------------------------------------------------------------ */

/* y[b,o] = sum_i x[b,i] * W[o,i] + bias[o]  (InnerProduct, [P2] layer 8). */
void orc_fc_forward(int batch, int in, int out, const double* x, const double* wt,
                    const double* bias, double* y) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < batch; ++b)
    for (int o = 0; o < out; ++o) {
      double acc = bias ? bias[o] : 0.0;
      for (int i = 0; i < in; ++i) acc += x[(long)b * in + i] * wt[(long)o * in + i];
      y[(long)b * out + o] = acc;
    }
}

/* InnerProduct Backward ([P2] layer 8):
 *   dW (out x in)  += delta^T (out x batch) * X (batch x in)     (gemm T,N, beta 1)
 *   db (out)       += delta^T * ones                              (gemv, beta 1)
 *   dX (batch x in) = delta (batch x out) * W (out x in)          (gemm N,N, beta 0)
 * dx may be NULL (bottom not propagated); dx_accumulate adds instead of
 * overwriting. */
void orc_fc_backward(int batch, int in, int out, const double* x, const double* wt,
                     const double* delta, double* dw, double* db, double* dx, int dx_accumulate) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int o = 0; o < out; ++o)
    for (int i = 0; i < in; ++i) {
      double acc = 0.0;
      for (int b = 0; b < batch; ++b) acc += delta[(long)b * out + o] * x[(long)b * in + i];
      dw[(long)o * in + i] += acc;
    }
  if (db)
    for (int o = 0; o < out; ++o) {
      double acc = 0.0;
      for (int b = 0; b < batch; ++b) acc += delta[(long)b * out + o];
      db[o] += acc;
    }
  if (dx) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < batch; ++b)
      for (int i = 0; i < in; ++i) {
        double acc = 0.0;
        for (int o = 0; o < out; ++o) acc += delta[(long)b * out + o] * wt[(long)o * in + i];
        dx[(long)b * in + i] = (dx_accumulate ? dx[(long)b * in + i] : 0.0) + acc;
      }
  }
}

/* Softmax over the class axis (Caffe SoftmaxLayer Forward, [P4]: subtract the
 * row max, exponentiate, divide by the row sum). */
void orc_softmax_forward(int batch, int classes, const double* logits, double* prob) {
  for (int b = 0; b < batch; ++b) {
    const double* r = logits + (long)b * classes;
    double mx = r[0];
    for (int j = 1; j < classes; ++j) mx = r[j] > mx ? r[j] : mx;
    double sum = 0.0;
    for (int j = 0; j < classes; ++j) sum += exp(r[j] - mx);
    for (int j = 0; j < classes; ++j) prob[(long)b * classes + j] = exp(r[j] - mx) / sum;
  }
}

/* Softmax backward along the channel axis (Caffe's SoftmaxLayer Backward_cpu,
 * [P4]): for each outer index i and inner position k, with the channel stride
 * `inner`: copy top_diff, take the strided dot of top_diff and top_data over the
 * channels, subtract it from every channel, then multiply by top_data:
 *   dx[i,c,k] = (dy[i,c,k] - sum_c' dy[i,c',k] y[i,c',k]) * y[i,c,k]. */
void orc_softmax_backward(int outer, int channels, long inner, const double* y, const double* dy,
                          double* dx) {
  const long dim = (long)channels * inner;
#pragma omp parallel for schedule(static)
  for (int i = 0; i < outer; ++i)
    for (long k = 0; k < inner; ++k) {
      double dot = 0.0;
      for (int c = 0; c < channels; ++c) dot += dy[i * dim + c * inner + k] * y[i * dim + c * inner + k];
      for (int c = 0; c < channels; ++c) {
        const long e = i * dim + c * inner + k;
        dx[e] = (dy[e] - dot) * y[e];
      }
    }
}

/* Mean cross-entropy of the softmax, the loss SoftmaxWithLoss reports. */
double orc_softmax_loss(int batch, int classes, const double* prob, const int* labels) {
  double l = 0.0;
  for (int b = 0; b < batch; ++b) l -= log(prob[(long)b * classes + labels[b]]);
  return l / batch;
}

/* SoftmaxWithLoss Backward ([P2] layer 9): copy prob into the bottom diff,
 * subtract 1 at each sample's label, scale by loss_weight / count (count =
 * number of labelled samples = batch here, one label per sample). */
void orc_softmax_loss_backward(int batch, int classes, const double* prob, const int* labels,
                               double loss_weight, double* dlogits) {
  for (long i = 0; i < (long)batch * classes; ++i) dlogits[i] = prob[i];
  for (int b = 0; b < batch; ++b) dlogits[(long)b * classes + labels[b]] -= 1.0;
  const double scale = loss_weight / batch;
  for (long i = 0; i < (long)batch * classes; ++i) dlogits[i] *= scale;
}

/* ------------------------------------------------------------------ */
/* shortcut, route, upsample                                           */
/* ------------------------------------------------------------------ */

/* backward_shortcut_layer for equal shapes ([P1] section 5): the delta goes
 * to the previous layer with weight alpha (axpy) and to the shortcut source
 * with weight beta (shortcut_cpu with s1 = 1, s2 = beta). */
void orc_shortcut_backward(long count, double alpha, double beta, const double* delta,
                           double* d_main, double* d_from) {
#pragma omp parallel for schedule(static)
  for (long i = 0; i < count; ++i) {
    d_main[i] += alpha * delta[i];
    d_from[i] = 1.0 * d_from[i] + beta * delta[i];
  }
}

/* backward_shortcut_layer when the two shapes differ ([P1] section 5): the delta
 * (batch x c1 x h1 x w1, the shortcut's output) goes to the previous layer with
 * weight alpha, and shortcut_cpu adds it into the source's delta (batch x c2 x
 * h2 x w2) over the smaller of the two shapes: with stride = w1/w2 and sample =
 * w2/w1 (each at least 1),
 *   d_from[b, k, j*sample, i*sample] = 1 * d_from[...] + beta * delta[b, k, j*stride, i*stride]
 * for k < min(c1, c2), j < min(h1, h2), i < min(w1, w2).  The page asserts
 * stride == h1/h2 and sample == h2/h1 (same aspect); the caller checks it. */
void orc_shortcut_backward_resize(int batch, int w1, int h1, int c1, int w2, int h2, int c2,
                                  double alpha, double beta, const double* delta, double* d_main,
                                  double* d_from) {
  const long n1 = (long)batch * c1 * h1 * w1;
  if (d_main)
    for (long e = 0; e < n1; ++e) d_main[e] += alpha * delta[e];
  int stride = w1 / w2, sample = w2 / w1;
  if (stride < 1) stride = 1;
  if (sample < 1) sample = 1;
  const int minw = w1 < w2 ? w1 : w2, minh = h1 < h2 ? h1 : h2, minc = c1 < c2 ? c1 : c2;
  for (int b = 0; b < batch; ++b)
    for (int k = 0; k < minc; ++k)
      for (int j = 0; j < minh; ++j)
        for (int i = 0; i < minw; ++i) {
          const long out = i * sample + (long)w2 * (j * sample + (long)h2 * (k + (long)c2 * b));
          const long add = i * stride + (long)w1 * (j * stride + (long)h1 * (k + (long)c1 * b));
          d_from[out] = 1.0 * d_from[out] + beta * delta[add];
        }
}

/* backward_route_layer ([P1] section 6): for input t and image j, add the
 * slice [offset_t + j*outputs, +in_sizes[t]) of the route delta into that
 * input's delta at j*in_sizes[t]; offsets advance by in_sizes[t]. */
void orc_route_backward(int batch, int n_in, const long* in_sizes, const double* delta,
                        double** d_in) {
  long outputs = 0;
  for (int t = 0; t < n_in; ++t) outputs += in_sizes[t];
  long offset = 0;
  for (int t = 0; t < n_in; ++t) {
    for (int j = 0; j < batch; ++j)
      for (long e = 0; e < in_sizes[t]; ++e)
        d_in[t][(long)j * in_sizes[t] + e] += delta[offset + (long)j * outputs + e];
    offset += in_sizes[t];
  }
}

/* Nearest-neighbour upsample by `scale` (the pages do not show it; its
 * plain definition): y[n,c,h,w] = x[n,c,h/scale,w/scale]. */
void orc_upsample_forward(int n, int c, int h, int w, int scale, const double* x, double* y) {
  const int H = h * scale, W = w * scale;
  for (long pl = 0; pl < (long)n * c; ++pl)
    for (int r = 0; r < H; ++r)
      for (int q = 0; q < W; ++q)
        y[(pl * H + r) * W + q] = x[(pl * h + r / scale) * w + q / scale];
}

/* Its adjoint: each small pixel collects the scale x scale block of the big
 * delta, dx[n,c,h,w] += sum_{a,b<scale} delta[n,c,h*scale+a,w*scale+b]. */
void orc_upsample_backward(int n, int c, int h, int w, int scale, const double* delta,
                           double* dx) {
  const int H = h * scale, W = w * scale;
#pragma omp parallel for schedule(static)
  for (long pl = 0; pl < (long)n * c; ++pl)
    for (int r = 0; r < h; ++r)
      for (int q = 0; q < w; ++q) {
        double acc = 0.0;
        for (int a = 0; a < scale; ++a)
          for (int b = 0; b < scale; ++b)
            acc += delta[(pl * H + r * scale + a) * W + q * scale + b];
        dx[(pl * h + r) * w + q] += acc;
      }
}

/* ------------------------------------------------------------------ */
/* Parameter update after a full batch ([P1] section 1: update_network ->
 * l.update once (seen / batch) % subdivisions == 0; [P3] layer struct: update
 * takes (layer, batch, learning_rate, momentum, decay), and weight_updates holds
 * the gradient term that the step size scales).  The pages give
 * no formula; the reading used here is gradient descent with momentum and L2
 * weight decay in which the accumulated-gradient buffer doubles as the momentum
 * buffer (the next backward adds onto it):
 *   u = dw + decay * batch * w      (dw holds the gradient summed over the batch)
 *   w = w - (learning_rate / batch) * u
 *   dw = momentum * u
 * Biases and BN scales take decay = 0. */
void orc_sgd_update(long n, int batch, double lr, double momentum, double decay, double* w,
                    double* dw) {
  for (long i = 0; i < n; ++i) {
    const double u = dw[i] + decay * batch * w[i];
    w[i] -= lr / batch * u;
    dw[i] = momentum * u;
  }
}
