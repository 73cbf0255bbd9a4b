// Backward of the gate.
//
// Sources: SALAD structured summary (paper.rainbus.top/paper/2601.16515)
// method step 5, ijyty.com/news/870645 section 2.3 and news.axiwang.com
// section 六.
//   * s_b = sigmoid(w . mean_n X_b[n] + b): with ds_b = dL/ds_b and
//     dt_b = ds_b s_b (1 - s_b): dL/dw = sum_b dt_b mean_n X_b[n],
//     dL/db = sum_b dt_b, dL/dX_b[n] = dt_b w / N for every token.
#include "common.h"
#include "kernels.h"

namespace salad {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_g;

// ---- gate -------------------------------------------------------------------

int gate_bwd_splits(const Geom &g) { return g.N < 128 ? g.N : 128; }

// Column sums of X over one row chunk: grid (splits, B); thread t owns
// 8-column groups t, t + 256, ...; fp32 sums in row order.
__global__ void __launch_bounds__(256) gate_colsum_kernel(Geom g, const bf16_t *__restrict__ x,
                                                          float *__restrict__ partial, int splits) {
  const int s = blockIdx.x, b = blockIdx.y, C = g.H * g.D;
  const int rows = (g.N + splits - 1) / splits;
  const int n0 = s * rows, n1 = min(g.N, n0 + rows);
  for (int cg = threadIdx.x; cg * 8 < C; cg += 256) {
    float cs[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 4
    for (int n = n0; n < n1; ++n) {
      const u32x4_g v = *(const u32x4_g *)(x + ((long long)b * g.N + n) * C + cg * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) cs[e] += bf16_to_f32(bf16_t((v[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
    }
    float *dst = partial + ((long long)b * splits + s) * C + cg * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = cs[e];
  }
}

hipError_t launch_gate_colsum(const Geom &g, const bf16_t *x, float *partial, hipStream_t st) {
  const int splits = gate_bwd_splits(g);
  gate_colsum_kernel<<<dim3(splits, g.B), 256, 0, st>>>(g, x, partial, splits);
  return hipGetLastError();
}

// One wave.  Lane 0 forms ds_b (the heads' 16 partials each, in order) and
// dt_b per sample, and dgate_b.  dgate_w / dgate_b may be NULL (not wanted).
__global__ void __launch_bounds__(64) gate_bwd_kernel(Geom g, const float *__restrict__ ds_part,
                                                      const float *__restrict__ s, int has_gate,
                                                      float *__restrict__ dt, float *__restrict__ ds_out,
                                                      float *__restrict__ dgate_b) {
  if (threadIdx.x != 0) return;
  double db = 0.0;
  for (int b = 0; b < g.B; ++b) {
    double ds = 0.0;
    for (int i = 0; i < g.H * 16; ++i) ds += double(ds_part[(long long)b * g.H * 16 + i]);
    if (s[b] < g.drop_tau) ds = 0.0;  // dropped: the gate does not reach the output
    const double sb = double(s[b]);
    const double t = has_gate ? ds * sb * (1.0 - sb) : 0.0;
    dt[b] = float(t);
    if (ds_out) ds_out[b] = float(ds);
    db += t;
  }
  if (has_gate && dgate_b) *dgate_b = float(db);
}

// dgate_w[c] = sum_b dt_b mean_n X_b[n][c].  A workgroup owns 32 columns;
// thread t adds splits t/32, t/32 + 8, ... of column t%32 (coalesced across
// the columns), then the 8 partial sums of a column are added in order.
__global__ void __launch_bounds__(256) gate_dw_kernel(Geom g, const float *__restrict__ dt,
                                                      const float *__restrict__ colsum, int splits,
                                                      float *__restrict__ dgate_w) {
  const int C = g.H * g.D, t = threadIdx.x;
  const int c = blockIdx.x * 32 + (t & 31), sg = t >> 5;
  __shared__ double part[8][32];
  double acc = 0.0;
  if (c < C)
    for (int b = 0; b < g.B; ++b) {
      double xs = 0.0;
      for (int sp = sg; sp < splits; sp += 8) xs += double(colsum[((long long)b * splits + sp) * C + c]);
      acc += double(dt[b]) * xs;
    }
  part[sg][t & 31] = acc;
  __syncthreads();
  if (sg == 0 && c < C) {
    double sum = 0.0;
    for (int i = 0; i < 8; ++i) sum += part[i][t];
    dgate_w[c] = float(sum / double(g.N));
  }
}

hipError_t launch_gate_bwd(const Geom &g, const float *ds_part, const float *s, int has_gate,
                           const float *colsum, float *dt, float *ds_out, float *dgate_w,
                           float *dgate_b, hipStream_t st) {
  gate_bwd_kernel<<<1, 64, 0, st>>>(g, ds_part, s, has_gate, dt, ds_out, dgate_b);
  if (has_gate && dgate_w) {
    const int C = g.H * g.D;
    gate_dw_kernel<<<(C + 31) / 32, 256, 0, st>>>(g, dt, colsum, gate_bwd_splits(g), dgate_w);
  }
  return hipGetLastError();
}

// dX[b, n, c] = dt_b w[c] / N: grid (ceil(N*C / 2048), B), 8 elements a thread.
__global__ void __launch_bounds__(256) gate_dx_kernel(Geom g, const float *__restrict__ dt,
                                                      const bf16_t *__restrict__ w, bf16_t *__restrict__ dx) {
  const int b = blockIdx.y, C = g.H * g.D;
  const long long e = ((long long)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e >= (long long)g.N * C) return;
  const int c = int(e % C);
  const float k = dt[b] / float(g.N);
  bf16_t wv[8], o[8];
  *(u32x4_g *)wv = *(const u32x4_g *)(w + c);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32_to_bf16(k * bf16_to_f32(wv[i]));
  *(u32x4_g *)(dx + (long long)b * g.N * C + e) = *(const u32x4_g *)o;
}

hipError_t launch_gate_dx(const Geom &g, const float *dt, const bf16_t *w, bf16_t *dx, hipStream_t st) {
  const long long n = (long long)g.N * g.H * g.D;
  gate_dx_kernel<<<dim3(unsigned((n + 2047) / 2048), g.B), 256, 0, st>>>(g, dt, w, dx);
  return hipGetLastError();
}

}  // namespace salad
