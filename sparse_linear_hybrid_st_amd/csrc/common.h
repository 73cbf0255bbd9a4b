// Device-side helpers shared by the gfx950 kernels of the hybrid attention
// library: storage-type conversion, tensor views with the head-wise token
// order, and the launch geometry of one layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace salad {

typedef uint16_t bf16_t;  // bfloat16 bits
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kMaxHeads = 256;

// ---- storage-type conversion --------------------------------------------

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(uint32_t(h) << 16);
}

// float32 -> bfloat16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return bf16_t((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16_t(u >> 16);
}

// float64 -> bfloat16 with a single rounding (nearest even), branch-free.
// Rounding to float32 first and then to bf16 would round twice; rounding
// the first step to odd instead (truncate, then set the last bit when any
// discarded bit was set) keeps the second rounding correct, because float32
// carries more than two bits beyond bf16's eight (Boldo and Melquiond,
// "Emulation of FMA and correctly rounded sums: proved algorithms using
// rounding to odd", IEEE TC 2008).  The hardware conversion rounds to
// nearest; when that went away from zero the pattern is stepped back one
// unit, which is the truncation.  NaN stays NaN, and overflow lands on the
// largest float32, which bf16 rounding then takes to infinity as it must.
__device__ __forceinline__ bf16_t f64_to_bf16(double x) {
  const float f = float(x);
  const double back = double(f);
  uint32_t u = __float_as_uint(f);
  const bool inexact = back != x;
  const bool away = fabs(back) > fabs(x);
  u = (u - (away ? 1u : 0u)) | (inexact ? 1u : 0u);
  return f32_to_bf16(__uint_as_float(u));
}

template <typename T> struct io;
template <> struct io<float> {
  static __device__ __forceinline__ float ld(const float *p) { return *p; }
  static __device__ __forceinline__ void st(float *p, float v) { *p = v; }
  static __device__ __forceinline__ float from_f64(double v) { return float(v); }
};
template <> struct io<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t *p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void st(bf16_t *p, float v) { *p = f32_to_bf16(v); }
  static __device__ __forceinline__ bf16_t from_f64(double v) { return f64_to_bf16(v); }
};

// ---- geometry ------------------------------------------------------------

// Division by a runtime constant d >= 1: m = ceil(2^32 / d) (0 when d == 1).
// q = floor(n * m / 2^32) is floor(n / d) or one more, because m exceeds
// 2^32 / d by less than 1 and n < 2^32; one multiply-compare fixes the
// overshoot.  Exact for 0 <= n < 2^31 (then q * d cannot wrap).
struct FastDiv {
  uint32_t d, m;
};

__host__ __device__ inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  f.m = d <= 1 ? 0u : uint32_t(((1ull << 32) + d - 1) / d);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(const FastDiv &f, uint32_t n) {
  if (f.m == 0) return n;
  uint32_t q = __umulhi(n, f.m);
  return q * f.d > n ? q - 1 : q;
}

// Per-layer geometry passed by value to every kernel.
struct Geom {
  int B, H, D, N;
  int F, Hg, Wg;
  uint64_t temporal[4];  // bit h: head h is temporal (spatial-major order)
  uint64_t topk[4];      // bit h: head h is Top-K
  int r;                 // window radius
  int block, k, nb;      // Top-K block size, kept blocks, number of blocks
  float scale;           // softmax scale
  float eps;             // linear denominator guard
  float drop_tau;        // branch dropping: samples with s_b < drop_tau keep only O_s
  int rope_dims[3];
  float rope_base;
  FastDiv fdF, fdS, fdW;  // division by F, Hg*Wg and Wg
};

__device__ __forceinline__ bool bit(const uint64_t *m, int h) {
  return (m[h >> 6] >> (h & 63)) & 1ull;
}

// A set of heads passed by value to a kernel (bit h: head h).
struct HeadSet {
  uint64_t w[4];
};

// Working position p of a temporal head holds this token.
__device__ __forceinline__ int st_token(const Geom &g, int p) {
  const int q = int(fdiv(g.fdF, uint32_t(p)));
  return (p - q * g.F) * (g.Hg * g.Wg) + q;
}

// Row addressing of a [B, *, *, d] tensor.  Element offset of (b, h, row)
// is b*sB + h*sH + row*sN; when `perm` is set, working row p of a temporal
// head is read from token st_token(p) (boundary layout gathered on load).
struct View {
  const void *base;
  long long sB, sH, sN;
  int perm;
};

__device__ __forceinline__ long long row_offset(const Geom &g, const View &v, int b, int h, int p) {
  int tok = (v.perm && bit(g.temporal, h)) ? st_token(g, p) : p;
  return (long long)b * v.sB + (long long)h * v.sH + (long long)tok * v.sN;
}

// RoPE angle for pair i of an axis segment of D dims at integer position
// pos: pos * base^(-2i/D), in float64.
__device__ __forceinline__ void rope_cs(int pos, int i, int D, double base, double *c, double *s) {
  double theta = pow(base, -2.0 * double(i) / double(D));
  sincos(double(pos) * theta, s, c);
}

}  // namespace salad
