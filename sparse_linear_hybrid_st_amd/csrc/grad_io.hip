// Backward pieces around the attention kernels: the gradient rows' way back
// to the token order (with the transposed RoPE rotation), and the gate's
// backward.
//
// Sources: RoPE -- SALAD structured summary (paper.rainbus.top/paper/
// 2601.16515) method step 3 and news.axiwang.com section 六; head-wise token
// order -- ijyty.com/news/870645 section 1.1; gate -- the summary's method
// step 5, ijyty.com section 2.3 and news.axiwang.com section 六.
//   * RoPE turns each pair (x0, x1) of an axis segment by an angle a; the
//     rotation is orthogonal, so a gradient goes back through it turned by
//     -a: (g0, g1) -> (g0 cos a + g1 sin a, -g0 sin a + g1 cos a).
//   * s_b = sigmoid(w . mean_n X_b[n] + b): with ds_b = dL/ds_b and
//     dt_b = ds_b s_b (1 - s_b): dL/dw = sum_b dt_b mean_n X_b[n],
//     dL/db = sum_b dt_b, dL/dX_b[n] = dt_b w / N for every token.
#include "common.h"
#include "kernels.h"

namespace salad {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_g;

// Grid B * ceil(N / 8); a workgroup owns 8 tokens of one sample and moves
// them for every head; thread t handles floats 4(t%32) .. +3 of token
// n0 + t/32.  Working row of token n: n, or site * F + frame for temporal
// heads.  The rotation is done in float64 and rounded once to bf16.
template <bool ROPE>
__global__ void __launch_bounds__(256) grad_scatter_kernel(Geom g, const float *__restrict__ src,
                                                           bf16_t *__restrict__ dst,
                                                           const double2 *__restrict__ table) {
  constexpr int D = 128, TOK = 8;
  const int chunks = (g.N + TOK - 1) / TOK;
  const int b = int(blockIdx.x) / chunks;
  const int tok = (int(blockIdx.x) - b * chunks) * TOK + int(threadIdx.x) / 32;
  const int c = (int(threadIdx.x) % 32) * 4;
  if (tok >= g.N) return;
  const int S = g.Hg * g.Wg;
  const int f = int(fdiv(g.fdS, uint32_t(tok)));
  const int site = tok - f * S;
  const int p_temporal = site * g.F + f;
  double cs[2] = {1.0, 1.0}, sn[2] = {0.0, 0.0};
  if (ROPE) {
    const int y = int(fdiv(g.fdW, uint32_t(site)));
    const int x = site - y * g.Wg;
    const int d0 = g.rope_dims[0], d1 = g.rope_dims[1];
    const int t0 = f * (d0 >> 1);
    const int t1 = g.F * (d0 >> 1) + y * (d1 >> 1);
    const int t2 = g.F * (d0 >> 1) + g.Hg * (d1 >> 1) + x * (g.rope_dims[2] >> 1);
#pragma unroll
    for (int t = 0; t < 4; t += 2) {
      const int e = c + t;
      const bool ax0 = e < d0, ax1 = !ax0 && e < d0 + d1;
      const int off = ax0 ? 0 : (ax1 ? d0 : d0 + d1);
      const double2 v = table[(ax0 ? t0 : (ax1 ? t1 : t2)) + ((e - off) >> 1)];
      cs[t >> 1] = v.x;
      sn[t >> 1] = v.y;
    }
  }
  const long long brow = ((long long)b * g.N + tok) * g.H * D + c;
#pragma unroll 4
  for (int h = 0; h < g.H; ++h) {
    const int p = bit(g.temporal, h) ? p_temporal : tok;
    const f32x4 v = *(const f32x4 *)(src + ((long long)(b * g.H + h) * g.N + p) * D + c);
    bf16_t o[4];
    if (ROPE) {
#pragma unroll
      for (int t = 0; t < 4; t += 2) {
        const double g0 = double(v[t]), g1 = double(v[t + 1]);
        o[t] = f64_to_bf16(g0 * cs[t >> 1] + g1 * sn[t >> 1]);
        o[t + 1] = f64_to_bf16(-g0 * sn[t >> 1] + g1 * cs[t >> 1]);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] = f32_to_bf16(v[t]);
    }
    *(uint2 *)(dst + brow + (long long)h * D) = *(const uint2 *)o;
  }
}

hipError_t launch_grad_scatter(const Geom &g, const float *src, bf16_t *dst, const double2 *table,
                               hipStream_t st) {
  if (g.D != 128) return hipErrorInvalidValue;
  const dim3 grid(unsigned((g.N + 7) / 8) * g.B);
  if (table)
    grad_scatter_kernel<true><<<grid, 256, 0, st>>>(g, src, dst, table);
  else
    grad_scatter_kernel<false><<<grid, 256, 0, st>>>(g, src, dst, nullptr);
  return hipGetLastError();
}

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

// One workgroup.  Thread 0 forms ds_b (the heads' 16 partials each, in
// order) and dt_b per sample; then every thread takes columns of dgate_w.
// dgate_w / dgate_b may be NULL (not wanted).
__global__ void __launch_bounds__(256) gate_bwd_kernel(Geom g, const float *__restrict__ ds_part,
                                                       const float *__restrict__ s, int has_gate,
                                                       const float *__restrict__ colsum, int splits,
                                                       float *__restrict__ dt, float *__restrict__ ds_out,
                                                       float *__restrict__ dgate_w, float *__restrict__ dgate_b) {
  const int C = g.H * g.D;
  if (threadIdx.x == 0) {
    double db = 0.0;
    for (int b = 0; b < g.B; ++b) {
      double ds = 0.0;
      for (int i = 0; i < g.H * 16; ++i) ds += double(ds_part[(long long)b * g.H * 16 + i]);
      const bool kept = !(s[b] < g.drop_tau);
      if (!kept) ds = 0.0;
      const double sb = double(s[b]);
      const double t = has_gate ? ds * sb * (1.0 - sb) : 0.0;
      dt[b] = float(t);
      if (ds_out) ds_out[b] = float(ds);
      db += t;
    }
    if (has_gate && dgate_b) *dgate_b = float(db);
  }
  __syncthreads();
  if (!has_gate || !dgate_w) return;
  __threadfence_block();
  for (int c = threadIdx.x; c < C; c += 256) {
    double acc = 0.0;
    for (int b = 0; b < g.B; ++b) {
      double xs = 0.0;
      for (int sp = 0; sp < splits; ++sp) xs += double(colsum[((long long)b * splits + sp) * C + c]);
      acc += double(dt[b]) * xs / double(g.N);
    }
    dgate_w[c] = float(acc);
  }
}

hipError_t launch_gate_bwd(const Geom &g, const float *ds_part, const float *s, int has_gate,
                           const float *colsum, float *dt, float *ds_out, float *dgate_w,
                           float *dgate_b, hipStream_t st) {
  gate_bwd_kernel<<<1, 256, 0, st>>>(g, ds_part, s, has_gate, colsum, gate_bwd_splits(g), dt, ds_out,
                                     dgate_w, dgate_b);
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
  bf16_t o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32_to_bf16(k * bf16_to_f32(w[c + i]));
  *(u32x4_g *)(dx + (long long)b * g.N * C + e) = *(const u32x4_g *)o;
}

hipError_t launch_gate_dx(const Geom &g, const float *dt, const bf16_t *w, bf16_t *dx, hipStream_t st) {
  const long long n = (long long)g.N * g.H * g.D;
  gate_dx_kernel<<<dim3(unsigned((n + 2047) / 2048), g.B), 256, 0, st>>>(g, dt, w, dx);
  return hipGetLastError();
}

}  // namespace salad
