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

template <typename T, bool ROPE>
__global__ void __launch_bounds__(256) permute_kernel(Geom g, const T *__restrict__ src,
                                                      T *__restrict__ dst, int inverse) {
  constexpr int VEC = 16 / sizeof(T);
  const int per_row = g.D / VEC;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long rows = (long long)g.B * g.H * g.N;
  const long long row = gid / per_row;  // working row (b*H + h)*N + p
  const int c = int(gid - row * per_row) * VEC;
  if (row >= rows) return;
  const int p = int(row % g.N);
  const long long bh = row / g.N;
  const int h = int(bh % g.H);
  const int b = int(bh / g.H);
  const int tok = bit(g.temporal, h) ? st_token(g, p) : p;
  const long long woff = row * g.D + c;
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
  const int S = g.Hg * g.Wg;
  const int pos3[3] = {tok / S, (tok / g.Wg) % g.Hg, tok % g.Wg};
  T out[VEC];
#pragma unroll
  for (int t = 0; t < VEC; t += 2) {
    int e = c + t, axis = 0, off = 0;
    while (axis < 2 && e >= off + g.rope_dims[axis]) { off += g.rope_dims[axis]; ++axis; }
    double cs, sn;
    rope_cs(pos3[axis], (e - off) >> 1, g.rope_dims[axis], double(g.rope_base), &cs, &sn);
    double a = double(io<T>::ld(&in[t])), bb = double(io<T>::ld(&in[t + 1]));
    out[t] = io<T>::from_f64(a * cs - bb * sn);
    out[t + 1] = io<T>::from_f64(a * sn + bb * cs);
  }
  *reinterpret_cast<u32x4 *>(dst + woff) = *reinterpret_cast<const u32x4 *>(out);
}

hipError_t launch_permute(const Geom &g, int dtype_bf16, int rope, int inverse, const void *src,
                          void *dst, hipStream_t st) {
  const int vec = dtype_bf16 ? 8 : 4;
  const long long threads = (long long)g.B * g.H * g.N * (g.D / vec);
  const unsigned grid = unsigned((threads + 255) / 256);
  if (dtype_bf16) {
    if (rope)
      permute_kernel<bf16_t, true><<<grid, 256, 0, st>>>(g, (const bf16_t *)src, (bf16_t *)dst, 0);
    else
      permute_kernel<bf16_t, false><<<grid, 256, 0, st>>>(g, (const bf16_t *)src, (bf16_t *)dst, inverse);
  } else {
    if (rope)
      permute_kernel<float, true><<<grid, 256, 0, st>>>(g, (const float *)src, (float *)dst, 0);
    else
      permute_kernel<float, false><<<grid, 256, 0, st>>>(g, (const float *)src, (float *)dst, inverse);
  }
  return hipGetLastError();
}

}  // namespace salad
