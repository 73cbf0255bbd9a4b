// Per-head window calibration.
//
// Source: ijyty.com/news/870645 section 1.1 -- each head's sliding window is
// chosen greedily as the smallest one whose relative squared error against
// full attention stays within a bound on a set of analysis samples.
// Reading: e_b(r) = ||O_window(r) - O_dense||_F^2 / ||O_dense||_F^2 over the
// head's rows for sample b; a radius meets the bound tau when max_b e_b(r)
// <= tau; the dense window (r = N - 1, error 0) when no candidate does.
//
// The attention outputs come from the sparse-attention kernel (the dense
// one is the window kernel with r = N - 1, every tile full); these kernels
// only reduce and choose.  Sums are fp64 in a fixed order.
#include "common.h"
#include "kernels.h"

namespace salad {

// Partial sums of (o_w - o_d)^2 and o_d^2 over a row chunk of one (b, h):
// grid (splits, B*H), 256 threads, thread t adds elements t, t + 256, ...
__global__ void __launch_bounds__(256) calib_err_kernel(Geom g, const float *__restrict__ od,
                                                        const float *__restrict__ ow, int splits,
                                                        double *__restrict__ part) {
  const int s = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const long long per = (long long)g.N * g.D;
  const long long chunk = (per + splits - 1) / splits;
  const long long e0 = s * chunk, e1 = min(per, e0 + chunk);
  const float *a = od + (long long)bh * per, *w = ow + (long long)bh * per;
  double num = 0.0, den = 0.0;
  for (long long e = e0 + t; e < e1; e += 256) {
    const double d0 = a[e], d1 = double(w[e]) - d0;
    num = fma(d1, d1, num);
    den = fma(d0, d0, den);
  }
  __shared__ double rn[256], rd[256];
  rn[t] = num;
  rd[t] = den;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (t < st) {
      rn[t] += rn[t + st];
      rd[t] += rd[t + st];
    }
    __syncthreads();
  }
  if (t == 0) {
    part[((long long)bh * splits + s) * 2] = rn[0];
    part[((long long)bh * splits + s) * 2 + 1] = rd[0];
  }
}

// err[i][b][h] = sum of the numerator partials / sum of the denominator
// partials, one thread per (b, h), splits in order.
__global__ void __launch_bounds__(256) calib_ratio_kernel(int BH, int splits, const double *__restrict__ part,
                                                          double *__restrict__ err) {
  const int bh = blockIdx.x * 256 + threadIdx.x;
  if (bh >= BH) return;
  double num = 0.0, den = 0.0;
  for (int s = 0; s < splits; ++s) {
    num += part[((long long)bh * splits + s) * 2];
    den += part[((long long)bh * splits + s) * 2 + 1];
  }
  err[bh] = num / den;
}

// choice[h] = the first radius whose error is <= tau on every sample, else N - 1.
__global__ void __launch_bounds__(256) calib_choose_kernel(Geom g, CalibRadii radii, float tau,
                                                           const double *__restrict__ err,
                                                           int32_t *__restrict__ choice) {
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h >= g.H) return;
  int pick = g.N - 1;
  for (int i = 0; i < radii.n; ++i) {
    double worst = 0.0;
    for (int b = 0; b < g.B; ++b) worst = fmax(worst, err[((long long)i * g.B + b) * g.H + h]);
    if (worst <= double(tau)) {
      pick = radii.r[i];
      break;
    }
  }
  choice[h] = pick;
}

int calib_splits(const Geom &g) {
  const long long per = (long long)g.N * g.D;
  const long long want = (per + 65535) / 65536;
  return int(want < 1 ? 1 : (want > 256 ? 256 : want));
}

hipError_t launch_calib_err(const Geom &g, const float *od, const float *ow, double *part, double *err,
                            hipStream_t st) {
  const int splits = calib_splits(g), BH = g.B * g.H;
  calib_err_kernel<<<dim3(splits, BH), 256, 0, st>>>(g, od, ow, splits, part);
  calib_ratio_kernel<<<(BH + 255) / 256, 256, 0, st>>>(BH, splits, part, err);
  return hipGetLastError();
}

hipError_t launch_calib_choose(const Geom &g, const CalibRadii &radii, float tau, const double *err,
                               int32_t *choice, hipStream_t st) {
  calib_choose_kernel<<<(g.H + 255) / 256, 256, 0, st>>>(g, radii, tau, err, choice);
  return hipGetLastError();
}

}  // namespace salad
