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

// RoPE table: (cos, sin) of pos * base^(-2i/D_axis) from rope_cs, one run
// per axis in axis order (frame, row, column), each run [pos][i] with
// i < D_axis / 2.
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

// Grid B * ceil(N / TOK) workgroups; a workgroup owns TOK consecutive
// tokens of one sample and moves them for every head, so on the boundary
// side ([B,N,H,d], one token's heads are one contiguous H*d record) it
// touches whole records, and a token's RoPE angles are looked up once and
// reused for all heads.  Thread t handles 16-byte chunk t % PER_ROW of
// token n0 + t / PER_ROW.  A token's working row is the token itself in
// spatial and Top-K heads and site * F + frame in temporal heads (the
// inverse of st_token), found with multiply-high division.  B*H*N < 2^31
// rows (checked at the boundary) keeps row indices in 32 bits.  MODE 0
// copies (forward or inverse), MODE 1 rotates with the (cos, sin) table,
// MODE 2 rotates computing (cos, sin) in place (no table).  keep_layout = 1
// (rotation only) writes each row back to its own place in a [B,N,H,d]
// destination.  Heads outside `heads` are skipped.
template <typename T, int MODE, int D>
__global__ void __launch_bounds__(256) permute_kernel(Geom g, const T *__restrict__ src,
                                                      T *__restrict__ dst, int inverse,
                                                      const double2 *__restrict__ table,
                                                      int keep_layout, HeadSet heads) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int PER_ROW = D / VEC;
  constexpr int TOK = 256 / PER_ROW;
  const int chunks = (g.N + TOK - 1) / TOK;
  const int b = int(blockIdx.x) / chunks;
  const int tok = (int(blockIdx.x) - b * chunks) * TOK + int(threadIdx.x) / PER_ROW;
  const int c = (int(threadIdx.x) % PER_ROW) * VEC;
  if (tok >= g.N) return;
  const int S = g.Hg * g.Wg;
  const int f = int(fdiv(g.fdS, uint32_t(tok)));
  const int site = tok - f * S;
  const int p_temporal = site * g.F + f;
  const T *bsrc = src;
  T *bdst = dst;
  const uint64_t brow = uint64_t(uint32_t(b) * uint32_t(g.N) + uint32_t(tok)) * uint32_t(g.H * D) + c;
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

  // (cos, sin) of the VEC/2 pairs of this thread's columns at this token
  double cs[VEC / 2], sn[VEC / 2];
  if (MODE != 0) {
    const int y = int(fdiv(g.fdW, uint32_t(site)));
    const int x = site - y * g.Wg;
    const int d0 = g.rope_dims[0], d1 = g.rope_dims[1], d2 = g.rope_dims[2];
    // first table entry of this token's run on each axis
    const int t0 = f * (d0 >> 1);
    const int t1 = g.F * (d0 >> 1) + y * (d1 >> 1);
    const int t2 = g.F * (d0 >> 1) + g.Hg * (d1 >> 1) + x * (d2 >> 1);
#pragma unroll
    for (int t = 0; t < VEC; t += 2) {
      // axis of column e: the three axes own consecutive column ranges
      const int e = c + t;
      const bool ax0 = e < d0, ax1 = !ax0 && e < d0 + d1;
      const int off = ax0 ? 0 : (ax1 ? d0 : d0 + d1);
      if (MODE == 1) {
        const double2 v = table[(ax0 ? t0 : (ax1 ? t1 : t2)) + ((e - off) >> 1)];
        cs[t >> 1] = v.x;
        sn[t >> 1] = v.y;
      } else {
        rope_cs(ax0 ? f : (ax1 ? y : x), (e - off) >> 1, ax0 ? d0 : (ax1 ? d1 : d2),
                double(g.rope_base), &cs[t >> 1], &sn[t >> 1]);
      }
    }
  }

#pragma unroll 4
  for (int h = 0; h < g.H; ++h) {
    if (!bit(heads.w, h)) continue;
    const int p = bit(g.temporal, h) ? p_temporal : tok;
    const uint64_t boff = brow + uint32_t(h * D);
    const uint64_t woff =
        keep_layout ? boff : uint64_t(uint32_t(b * g.H + h) * uint32_t(g.N) + uint32_t(p)) * D + c;
    if (MODE == 0) {
      const uint64_t from = inverse ? woff : boff;
      const uint64_t to = inverse ? boff : woff;
      *reinterpret_cast<u32x4 *>(bdst + to) = *reinterpret_cast<const u32x4 *>(bsrc + from);
      continue;
    }
    // RoPE (forward only): rotate the VEC/2 pairs, in float64, one rounding
    T in[VEC], out[VEC];
    *reinterpret_cast<u32x4 *>(in) = *reinterpret_cast<const u32x4 *>(bsrc + boff);
#pragma unroll
    for (int t = 0; t < VEC; t += 2) {
      const double a = double(io<T>::ld(&in[t])), bb = double(io<T>::ld(&in[t + 1]));
      out[t] = io<T>::from_f64(a * cs[t >> 1] - bb * sn[t >> 1]);
      out[t + 1] = io<T>::from_f64(a * sn[t >> 1] + bb * cs[t >> 1]);
    }
    *reinterpret_cast<u32x4 *>(bdst + woff) = *reinterpret_cast<const u32x4 *>(out);
  }
}

template <typename T, int D>
static void permute_launch(const Geom &g, int mode, int inverse, const void *src, void *dst,
                           hipStream_t st, const double2 *table, int keep_layout = 0,
                           const uint64_t *heads = nullptr) {
  constexpr int TOK = 256 / (D / (16 / sizeof(T)));
  const dim3 grid(((g.N + TOK - 1) / TOK) * g.B);
  const T *s = (const T *)src;
  T *d = (T *)dst;
  HeadSet hs;
  for (int i = 0; i < 4; ++i) hs.w[i] = heads ? heads[i] : ~0ull;
  if (mode == 1) permute_kernel<T, 1, D><<<grid, 256, 0, st>>>(g, s, d, 0, table, keep_layout, hs);
  else if (mode == 2) permute_kernel<T, 2, D><<<grid, 256, 0, st>>>(g, s, d, 0, nullptr, keep_layout, hs);
  else permute_kernel<T, 0, D><<<grid, 256, 0, st>>>(g, s, d, inverse, nullptr, 0, hs);
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
                          void *dst, hipStream_t st, const double2 *table, const uint64_t *heads) {
  const int mode = rope ? (table ? 1 : 2) : 0;
  if (dtype_bf16) {
    if (g.D != 128) return hipErrorInvalidValue;
    permute_launch<bf16_t, 128>(g, mode, inverse, src, dst, st, table, 0, heads);
  } else if (g.D == 128) {
    permute_launch<float, 128>(g, mode, inverse, src, dst, st, table, 0, heads);
  } else if (g.D == 64) {
    permute_launch<float, 64>(g, mode, inverse, src, dst, st, table, 0, heads);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rope_rows(const Geom &g, int dtype_bf16, const void *src, void *dst,
                            const double2 *table, hipStream_t st) {
  if (!table) return hipErrorInvalidValue;
  if (dtype_bf16) {
    if (g.D != 128) return hipErrorInvalidValue;
    permute_launch<bf16_t, 128>(g, 1, 0, src, dst, st, table, 1);
  } else if (g.D == 128) {
    permute_launch<float, 128>(g, 1, 0, src, dst, st, table, 1);
  } else if (g.D == 64) {
    permute_launch<float, 64>(g, 1, 0, src, dst, st, table, 1);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace salad
