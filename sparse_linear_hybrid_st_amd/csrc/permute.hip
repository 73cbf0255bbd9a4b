// Head-wise token permutation between the boundary layout [B,N,H,d] and the
// working layout [B,H,N,d], with optional 3D rotary position encoding.
//
// Source: ijyty.com/news/870645, section 1.1 -- the latent is flattened
// frame-major; heads with temporal locality regroup the tokens by spatial
// site so that one site's frames are contiguous.  RoPE: SALAD structured
// summary (paper.rainbus.top), method step 3, and news.axiwang.com section 六.
//
// HBM-bound copy: each thread moves 16 bytes of one row; a row of d=128 bf16
// is 256 contiguous bytes on both sides, so both the gather and the store
// are full 256-byte segments.
#include "common.h"
#include "kernels.h"

namespace salad {

// Entry (axis, pos, i) of the RoPE table: (cos, sin) of pos * base^(-2i/D_axis),
// computed by rope_cs, stored at rope_index(axis, pos, i).
__device__ __forceinline__ int rope_index(const Geom &g, int axis, int pos, int i) {
  const int off1 = g.F * (g.rope_dims[0] >> 1);
  const int off2 = off1 + g.Hg * (g.rope_dims[1] >> 1);
  const int base = axis == 0 ? 0 : (axis == 1 ? off1 : off2);
  return base + pos * (g.rope_dims[axis] >> 1) + i;
}

__global__ void __launch_bounds__(256) rope_table_kernel(Geom g, double2 *__restrict__ table) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int n0 = g.F * (g.rope_dims[0] >> 1), n1 = g.Hg * (g.rope_dims[1] >> 1);
  const int n2 = g.Wg * (g.rope_dims[2] >> 1);
  int axis, r;
  if (e < n0) { axis = 0; r = e; }
  else if (e < n0 + n1) { axis = 1; r = e - n0; }
  else if (e < n0 + n1 + n2) { axis = 2; r = e - n0 - n1; }
  else return;
  const int half = g.rope_dims[axis] >> 1;
  double c, sn;
  rope_cs(r / half, r % half, g.rope_dims[axis], double(g.rope_base), &c, &sn);
  table[e] = make_double2(c, sn);
}

// Grid (ceil(N / rows_per_wg), B*H): a workgroup moves rows_per_wg
// consecutive working rows of one (b, h); thread t handles 16-byte chunk
// t % per_row of row t / per_row.  (b, h) come from the block index and the
// token decomposition uses multiply-high division, so no per-element
// integer division remains.
template <typename T, bool ROPE>
__global__ void __launch_bounds__(256) permute_kernel(Geom g, const T *__restrict__ src,
                                                      T *__restrict__ dst, int inverse,
                                                      const double2 *__restrict__ table) {
  constexpr int VEC = 16 / sizeof(T);
  const int per_row = g.D / VEC;
  const int rows_per_wg = 256 / per_row;
  const int bh = blockIdx.y, h = bh % g.H, b = bh / g.H;
  const int p = blockIdx.x * rows_per_wg + int(threadIdx.x) / per_row;
  const int c = (int(threadIdx.x) % per_row) * VEC;
  if (p >= g.N) return;
  const int tok = bit(g.temporal, h) ? st_token(g, p) : p;
  const long long woff = ((long long)bh * g.N + p) * g.D + c;
  const long long boff = (((long long)b * g.N + tok) * g.H + h) * g.D + c;

  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  if (!ROPE) {
    const long long from = inverse ? woff : boff;
    const long long to = inverse ? boff : woff;
    *reinterpret_cast<u32x4 *>(dst + to) = *reinterpret_cast<const u32x4 *>(src + from);
    return;
  }
  // RoPE (forward only): rotate the VEC/2 pairs held by this thread.
  T in[VEC];
  *reinterpret_cast<u32x4 *>(in) = *reinterpret_cast<const u32x4 *>(src + boff);
  const int f = int(fdiv(g.fdS, uint32_t(tok)));
  const int rem = tok - f * g.Hg * g.Wg;
  const int y = int(fdiv(g.fdW, uint32_t(rem)));
  const int pos3[3] = {f, y, rem - y * g.Wg};
  T out[VEC];
#pragma unroll
  for (int t = 0; t < VEC; t += 2) {
    int e = c + t, axis = 0, off = 0;
    while (axis < 2 && e >= off + g.rope_dims[axis]) { off += g.rope_dims[axis]; ++axis; }
    double cs, sn;
    if (table) {
      const double2 v = table[rope_index(g, axis, pos3[axis], (e - off) >> 1)];
      cs = v.x;
      sn = v.y;
    } else {
      rope_cs(pos3[axis], (e - off) >> 1, g.rope_dims[axis], double(g.rope_base), &cs, &sn);
    }
    double a = double(io<T>::ld(&in[t])), bb = double(io<T>::ld(&in[t + 1]));
    out[t] = io<T>::from_f64(a * cs - bb * sn);
    out[t + 1] = io<T>::from_f64(a * sn + bb * cs);
  }
  *reinterpret_cast<u32x4 *>(dst + woff) = *reinterpret_cast<const u32x4 *>(out);
}

int rope_table_entries(const Geom &g) {
  return g.F * (g.rope_dims[0] / 2) + g.Hg * (g.rope_dims[1] / 2) + g.Wg * (g.rope_dims[2] / 2);
}

hipError_t launch_rope_table(const Geom &g, double2 *table, hipStream_t st) {
  const int n = rope_table_entries(g);
  rope_table_kernel<<<(n + 255) / 256, 256, 0, st>>>(g, table);
  return hipGetLastError();
}

hipError_t launch_permute(const Geom &g, int dtype_bf16, int rope, int inverse, const void *src,
                          void *dst, hipStream_t st, const double2 *table) {
  const int vec = dtype_bf16 ? 8 : 4;
  const int rows_per_wg = 256 / (g.D / vec);
  const dim3 grid((g.N + rows_per_wg - 1) / rows_per_wg, g.B * g.H);
  if (dtype_bf16) {
    if (rope)
      permute_kernel<bf16_t, true><<<grid, 256, 0, st>>>(g, (const bf16_t *)src, (bf16_t *)dst, 0, table);
    else
      permute_kernel<bf16_t, false><<<grid, 256, 0, st>>>(g, (const bf16_t *)src, (bf16_t *)dst, inverse, nullptr);
  } else {
    if (rope)
      permute_kernel<float, true><<<grid, 256, 0, st>>>(g, (const float *)src, (float *)dst, 0, table);
    else
      permute_kernel<float, false><<<grid, 256, 0, st>>>(g, (const float *)src, (float *)dst, inverse, nullptr);
  }
  return hipGetLastError();
}

}  // namespace salad
