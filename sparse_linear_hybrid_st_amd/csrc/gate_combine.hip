// Gate s = sigmoid(w . mean_n X[n,:] + b) and the combine
// out = O_s + s * (O_l W_p) scattered back to token order.
//
// Sources: SALAD structured summary (paper.rainbus.top/paper/2601.16515),
// method steps 4 (zero-initialised projection of the linear output),
// 5 (scalar gate in (0,1)) and 6 (residual sum); ijyty.com/news/870645
// section 2.3 and news.axiwang.com section 六 (token average, then a linear
// layer and a sigmoid).
//
// Both are HBM-bound.  The gate reads X once: per sample, tiles of (row
// chunk, column band) reduce to partial dot products w . sum X[n] (fp32
// inside a lane, fp64 across lanes and tiles) and one workgroup per sample
// finishes the mean and the sigmoid -- a fixed summation order throughout.
#include "common.h"
#include "kernels.h"
#include "mfma_util.h"

namespace salad {

// The gate is linear before the sigmoid: w . mean_n X[n] = (1/N) sum_n w . X[n],
// so each workgroup reduces its share of X straight to one number.
// Grid (column bands, row chunks, B), 256 threads.  A column band is 64
// groups of 8 columns (one per lane); a chunk is kGateRows = 64 rows, and
// wave w of the workgroup takes rows n0 + w, n0 + w + 4, ..., so each wave
// reads 64 consecutive 8-column groups of a row (1 KB of bf16) per load.
// A lane issues all 16 of its row loads before it adds any (one memory
// latency per workgroup), accumulates w[c] * X[n][c] in fp32, and the
// workgroup adds the 256 lane sums in fp64 in a fixed order (within each
// wave, then the four waves).
template <typename T>
__global__ void __launch_bounds__(256) gate_partial_kernel(Geom g, const T *__restrict__ x,
                                                           const T *__restrict__ w,
                                                           double *__restrict__ partial) {
  const int band = blockIdx.x, ch = blockIdx.y, b = blockIdx.z;
  const int C = g.H * g.D, groups = C / 8;
  const int n0 = ch * kGateRows, n1 = min(g.N, n0 + kGateRows);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int cg = band * 64 + lane;
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  float acc = 0.f;
  if (cg < groups) {
    float wv8[8], cs[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e) wv8[e] = io<T>::ld(w + cg * 8 + e);
    const T *src = x + ((long long)b * g.N + n0 + wv) * C + cg * 8;
    constexpr int R = kGateRows / 4;  // rows per lane
    T v[R][8];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (n0 + wv + 4 * i < n1) {
        *(u32x4 *)v[i] = *(const u32x4 *)(src + 4ll * i * C);
        if (sizeof(T) == 4) *(u32x4 *)(v[i] + 4) = *(const u32x4 *)(src + 4ll * i * C + 4);
      } else {
        *(u32x4 *)v[i] = u32x4{0, 0, 0, 0};
        if (sizeof(T) == 4) *(u32x4 *)(v[i] + 4) = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) cs[e] += io<T>::ld(v[i] + e);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(wv8[e], cs[e], acc);
  }
  // fixed-order fp64 sums: a butterfly within the wave, then the four waves
  double d = double(acc);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) d += __shfl_xor(d, o);
  __shared__ double red[4];
  if (lane == 0) red[wv] = d;
  __syncthreads();
  if (threadIdx.x == 0)
    partial[((long long)b * gridDim.y + ch) * gridDim.x + band] = ((red[0] + red[1]) + red[2]) + red[3];
}

// s_b = sigmoid(sum_i partial[b][i] / N + bias) over the n partial sums of
// sample b: one workgroup per sample, thread t adds partials t, t+256, ...
// in order, then a fixed-order tree.
__global__ void __launch_bounds__(256) gate_final_kernel(int N, int n, const double *__restrict__ partial,
                                                         float bias, float *__restrict__ s_out) {
  const int b = blockIdx.x;
  __shared__ double red[256];
  double acc = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) acc += partial[(long long)b * n + i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double t = red[0] / double(N) + double(bias);
    s_out[b] = float(1.0 / (1.0 + exp(-t)));
  }
}

hipError_t launch_gate(const Geom &g, int bf16, const void *x, const void *w, float bias,
                       void *ws, float *s, hipStream_t st) {
  const int bands = gate_bands(g), chunks = gate_chunks(g);
  double *partial = (double *)ws;
  dim3 grid(bands, chunks, g.B);
  if (bf16)
    gate_partial_kernel<bf16_t><<<grid, 256, 0, st>>>(g, (const bf16_t *)x, (const bf16_t *)w, partial);
  else
    gate_partial_kernel<float><<<grid, 256, 0, st>>>(g, (const float *)x, (const float *)w, partial);
  gate_final_kernel<<<g.B, 256, 0, st>>>(g.N, bands * chunks, partial, bias, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine.  Grid (ceil(N/64), B*H); 64 working rows per workgroup; thread t
// computes rows 4*(t/16)..+3 and columns (t%16) + 16*m of O_l W_p (fp32),
// then out[b, pi(p), h, :] = o_s + s * that, in the storage type.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) combine_kernel(Geom g, const float *__restrict__ o_s,
                                                      const float *__restrict__ o_l,
                                                      const T *__restrict__ w_p,
                                                      const float *__restrict__ s,
                                                      T *__restrict__ out) {
  extern __shared__ float smem[];
  float *Wp = smem;            // [D][D]
  float *Ol = smem + D * D;    // [64][D + 1]
  constexpr int NC = D / 16, LD = D + 1;
  const int bh = blockIdx.y, h = bh % g.H, b = bh / g.H;
  const int p0 = blockIdx.x * 64, t = threadIdx.x;
  for (int e = t; e < D * D; e += 256) Wp[e] = io<T>::ld(w_p + e);
  for (int e = t; e < 64 * D; e += 256) {
    const int r = e / D, c = e % D, p = p0 + r;
    Ol[r * LD + c] = p < g.N ? o_l[((long long)bh * g.N + p) * D + c] : 0.f;
  }
  __syncthreads();
  const int rg = t >> 4, cg = t & 15;
  float acc[4][NC];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int m = 0; m < NC; ++m) acc[a][m] = 0.f;
  for (int i = 0; i < D; ++i) {
    float ol[4], wv[NC];
#pragma unroll
    for (int a = 0; a < 4; ++a) ol[a] = Ol[(4 * rg + a) * LD + i];
#pragma unroll
    for (int m = 0; m < NC; ++m) wv[m] = Wp[i * D + cg + 16 * m];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int m = 0; m < NC; ++m) acc[a][m] = fmaf(ol[a], wv[m], acc[a][m]);
  }
  const float sb = s[b];
  const bool dropped = sb < g.drop_tau;  // branch dropping ([G] 2 C): out = O_s
  const bool temporal = bit(g.temporal, h);
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int p = p0 + 4 * rg + a;
    if (p >= g.N) continue;
    const int tok = temporal ? st_token(g, p) : p;
    const float *os = o_s + ((long long)bh * g.N + p) * D;
    T *dst = out + (((long long)b * g.N + tok) * g.H + h) * D;
#pragma unroll
    for (int m = 0; m < NC; ++m) {
      const int c = cg + 16 * m;
      io<T>::st(dst + c, dropped ? os[c] : os[c] + sb * acc[a][m]);
    }
  }
}

// Combine, bf16, d = 128, on MFMA.  Grid (ceil(N/128), B*H), 4 waves of 32
// working rows.  (O_l W_p)^T = W_p^T O_l^T with W_p^T staged in LDS (bf16,
// the K-tile swizzle) as A operands and each row's O_l as B operands, split
// into bf16 hi + lo parts (O_l = hi + lo to about 2^-17 relative; the
// products are exact and accumulate in fp32), so 2 MFMAs per step.  A lane
// then holds its row's features 32db + 8r4 + 4hl + e and writes them as
// bf16x4 next to the matching O_s.
__global__ void __launch_bounds__(256) combine_bf16_kernel(Geom g, const float *__restrict__ o_s,
                                                           const float *__restrict__ o_l,
                                                           const bf16_t *__restrict__ w_p,
                                                           const float *__restrict__ s,
                                                           bf16_t *__restrict__ out) {
  __shared__ __attribute__((aligned(16))) bf16_t Wt[kD * kD];  // Wt[j][k] = W_p[k][j]
  const int bh = blockIdx.y, h = bh % g.H, b = bh / g.H;
  const int t = threadIdx.x, lane = t & 63, hl = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  // W_p^T into LDS: thread t reads 8 consecutive columns j of row k
  for (int u = t; u < kD * kD / 8; u += 256) {
    const int k = u >> 4, j0 = (u & 15) * 8;
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_l;
    const u32x4_l v = *(const u32x4_l *)(w_p + k * kD + j0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = j0 + e;
      Wt[j * kD + (((k >> 3) ^ kv_swz(j)) << 3) + (k & 7)] = bf16_t((v[e >> 1] >> ((e & 1) * 16)) & 0xffffu);
    }
  }
  const int p = blockIdx.x * 128 + 32 * w + l32, pc = min(p, g.N - 1);
  const float *orow = o_l + ((long long)bh * g.N + pc) * kD;
  bf16x8 hi[8], lo[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const f32x4 a = *(const f32x4 *)(orow + 16 * ks + 8 * hl);
    const f32x4 c = *(const f32x4 *)(orow + 16 * ks + 8 * hl + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = e < 4 ? a[e] : c[e - 4];
      const __bf16 xh = (__bf16)x;
      hi[ks][e] = xh;
      lo[ks][e] = (__bf16)(x - float(xh));
    }
  }
  __syncthreads();
  const int kswz = kv_swz(l32);
  const int k_lane = l32 * kD + 8 * (hl ^ (kswz & 1)), k_x = kswz >> 1;
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const bf16x8 a = *(const bf16x8 *)(Wt + db * 32 * kD + k_lane + 16 * (ks ^ k_x));
      acc[db] = mfma_32x32x16(a, hi[ks], acc[db]);
      acc[db] = mfma_32x32x16(a, lo[ks], acc[db]);
    }
  if (p >= g.N) return;
  const float sb = s[b];
  const float sl = sb < g.drop_tau ? 0.f : sb;  // branch dropping ([G] 2 C): out = O_s
  const int tok = bit(g.temporal, h) ? st_token(g, p) : p;
  const float *os = o_s + ((long long)bh * g.N + p) * kD;
  bf16_t *dst = out + (((long long)b * g.N + tok) * g.H + h) * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int f = 32 * db + 8 * r4 + 4 * hl;
      const f32x4 o = *(const f32x4 *)(os + f);
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[e] + sl * acc[db][4 * r4 + e]);
      *(bf16x4 *)(dst + f) = v;
    }
}

hipError_t launch_combine(const Geom &g, int bf16, const float *o_s, const float *o_l,
                          const void *w_p, const float *s, void *out, hipStream_t st) {
  if (bf16 && g.D == 128) {
    combine_bf16_kernel<<<dim3((g.N + 127) / 128, g.B * g.H), 256, 0, st>>>(
        g, o_s, o_l, (const bf16_t *)w_p, s, (bf16_t *)out);
    return hipGetLastError();
  }
  dim3 grid((g.N + 63) / 64, g.B * g.H);
  const size_t lds = (size_t(g.D) * g.D + 64 * (g.D + 1)) * sizeof(float);
#define SALAD_COMBINE(T, DD)                                                                 \
  do {                                                                                       \
    hipFuncSetAttribute((const void *)combine_kernel<T, DD>,                                 \
                        hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));               \
    combine_kernel<T, DD><<<grid, 256, lds, st>>>(g, o_s, o_l, (const T *)w_p, s, (T *)out); \
  } while (0)
  if (bf16) {
    if (g.D == 128) SALAD_COMBINE(bf16_t, 128); else SALAD_COMBINE(bf16_t, 64);
  } else {
    if (g.D == 128) SALAD_COMBINE(float, 128); else SALAD_COMBINE(float, 64);
  }
#undef SALAD_COMBINE
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Staged full-width projection, first half: O_s and s_b * O_l back to token
// rows (the GEMM over whole token rows follows).  Grid (ceil(N*D/1024), B*H),
// thread t moves elements 4t..4t+3 of its workgroup's 1024-element slice of
// the head's N x D working rows.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) split_full_kernel(Geom g, const float *__restrict__ o_s,
                                                         const float *__restrict__ o_l,
                                                         const float *__restrict__ s,
                                                         T *__restrict__ out, T *__restrict__ olt) {
  const int bh = blockIdx.y, h = bh % g.H, b = bh / g.H;
  const long long e = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= (long long)g.N * g.D) return;
  const int p = int(e / g.D), c = int(e % g.D);
  const float sb = s[b];
  const float sl = sb < g.drop_tau ? 0.f : sb;  // branch dropping ([G] 2 C)
  const int tok = bit(g.temporal, h) ? st_token(g, p) : p;
  const long long src = (long long)bh * g.N * g.D + e;
  const long long dst = ((long long)b * g.N + tok) * g.H * g.D + (long long)h * g.D + c;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    io<T>::st(out + dst + i, o_s[src + i]);
    io<T>::st(olt + dst + i, sl * o_l[src + i]);
  }
}

hipError_t launch_split_full(const Geom &g, int bf16, const float *o_s, const float *o_l,
                             const float *s, void *out, void *olt, hipStream_t st) {
  dim3 grid(unsigned(((long long)g.N * g.D + 1023) / 1024), g.B * g.H);
  if (bf16)
    split_full_kernel<bf16_t><<<grid, 256, 0, st>>>(g, o_s, o_l, s, (bf16_t *)out, (bf16_t *)olt);
  else
    split_full_kernel<float><<<grid, 256, 0, st>>>(g, o_s, o_l, s, (float *)out, (float *)olt);
  return hipGetLastError();
}

}  // namespace salad
