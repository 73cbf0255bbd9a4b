// Top-K block selection: block-mean pooling of Q and K, block scores and
// the k best key blocks per query block (fp64 scores, radix select).
//
// Source: ijyty.com/news/870645, section 1.2 -- cut the tokens into blocks,
// take each block's mean, compare queries with the key-block means and keep
// the K most similar blocks.  Scoring a query block by its mean query gives
// the mean of its queries' scores (linearity).
//
// Precision: sums of bf16 or f32 inputs are accumulated in float64 (exact
// for these inputs), divided once by the row count, and the 128-term dot
// products run in float64 too, so only genuine near-ties can depend on the
// order of additions.
#include "common.h"
#include "kernels.h"

namespace salad {

// One workgroup per (b, h, block) of one tensor (blockIdx.z: 0 = Q, 1 = K),
// with (b, h) varying fastest so that workgroups in flight together read
// every head of the same tokens (whole [B,N,H,d] records).  256 threads:
// 16 row groups x 16 column chunks of 8 elements; a thread issues all of
// its rows' loads before it adds.
template <typename T>
__global__ void __launch_bounds__(256) block_mean_kernel(Geom g, View qv, View kv,
                                                         double *__restrict__ qbar,
                                                         double *__restrict__ kbar) {
  const int bh = blockIdx.x;
  const int blk = blockIdx.y;
  const int h = bh % g.H, b = bh / g.H;
  if (!bit(g.topk, h)) return;
  const View v = blockIdx.z ? kv : qv;
  double *out = (blockIdx.z ? kbar : qbar) + ((long long)bh * g.nb + blk) * g.D;
  const T *base = (const T *)v.base;
  const int t = threadIdx.x, rg = t >> 4, ch = t & 15;
  const int row0 = blk * g.block;
  const int rows = min(g.block, g.N - row0);
  __shared__ double part[16][128];
  const int cols = g.D / 8;  // column chunks in use (8 or 16)
  typedef T chunk8 __attribute__((ext_vector_type(8)));  // 16 B (bf16) or 32 B (f32)
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (ch < cols) {
    for (int r0 = rg; r0 < rows; r0 += 64) {
      // up to four rows in flight: rows r0, r0+16, r0+32, r0+48
      chunk8 raw[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = r0 + 16 * u;
        if (r < rows) raw[u] = *(const chunk8 *)(base + row_offset(g, v, b, h, row0 + r) + ch * 8);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (r0 + 16 * u >= rows) break;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const T x = raw[u][e];
          acc[e] += double(io<T>::ld(&x));
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[rg][ch * 8 + e] = acc[e];
  }
  __syncthreads();
  if (t < g.D) {
    double s = 0.0;
    for (int i = 0; i < 16; ++i) s += part[i][t];
    out[t] = s / double(rows);
  }
}

// Block scores S[qb][kb] = qbar[qb] . kbar[kb] for every Top-K (b, h), on
// the fp64 matrix cores (v_mfma_f64_16x16x4_f64; a dot product of 128
// terms has no room for a third operand per FMA in the vector units'
// register banks).  Workgroup (tile_q, tile_k, bh) computes a 128 x 128
// tile from 16-feature slices of both operands staged in LDS
// (feature-major); wave w owns the 64 x 64 quadrant (64*(w/2), 64*(w%2)) as
// 4 x 4 blocks of 16 x 16.  MFMA layout: lane l supplies A[i = l%16][k =
// l/16] and B[k = l/16][j = l%16]; its four results are D[i = 4r + l/16][j
// = l%16], r = 0..3.  Each product is an fp64 sum over the d features (the
// matrix unit's own order inside each step of 4).
constexpr int kScoreTile = 128;
typedef __attribute__((ext_vector_type(4))) double f64x4;

__global__ void __launch_bounds__(256) block_score_kernel(Geom g, const double *__restrict__ qbar,
                                                          const double *__restrict__ kbar,
                                                          double *__restrict__ scores) {
  constexpr int TS = kScoreTile, LD = TS + 2;  // +2: the feature-major stores spread over banks
  const int bh = blockIdx.z, h = bh % g.H;
  if (!bit(g.topk, h)) return;
  const int nb = g.nb, D = g.D, t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int q0 = blockIdx.x * TS, k0 = blockIdx.y * TS;
  __shared__ __attribute__((aligned(16))) double qs[16 * LD];
  __shared__ __attribute__((aligned(16))) double ks[16 * LD];
  const double *qb = qbar + (long long)bh * nb * D;
  const double *kb = kbar + (long long)bh * nb * D;
  const int wq = 64 * (w >> 1), wk = 64 * (w & 1);
  const int li = lane & 15, lk = lane >> 4;
  // staging: thread t loads features f8..f8+7 of row r (64 contiguous bytes)
  const int lr = t >> 1, f8 = 8 * (t & 1);
  f64x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  // the next slice is fetched into registers while the current one computes
  double qv[8], kv[8];
  auto fetch = [&](int f0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qv[e] = (q0 + lr < nb) ? qb[(long long)(q0 + lr) * D + f0 + f8 + e] : 0.0;
      kv[e] = (k0 + lr < nb) ? kb[(long long)(k0 + lr) * D + f0 + f8 + e] : 0.0;
    }
  };
  fetch(0);
  for (int f0 = 0; f0 < D; f0 += 16) {
    __syncthreads();  // previous slice's reads are done
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qs[(f8 + e) * LD + lr] = qv[e];
      ks[(f8 + e) * LD + lr] = kv[e];
    }
    __syncthreads();
    if (f0 + 16 < D) fetch(f0 + 16);
#pragma unroll
    for (int s4 = 0; s4 < 16; s4 += 4) {
      double a[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = qs[(s4 + lk) * LD + wq + 16 * i + li];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = ks[(s4 + lk) * LD + wk + 16 * j + li];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], bv[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = q0 + wq + 16 * i + 4 * r + lk;
      if (row >= nb) continue;
      double *dst = scores + ((long long)bh * nb + row) * nb;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = k0 + wk + 16 * j + li;
        if (col < nb) dst[col] = acc[i][j][r];
      }
    }
}

// Selection, one single-wave workgroup per query block: the k best key
// blocks under the order "higher score first, equal scores lower block
// first", written ascending.
//
// Radix select on an order-preserving 64-bit key of the score (sign bit
// flipped for non-negative values, all bits flipped for negative ones; -0
// is first turned into +0 so that it ties with +0): eight passes over 8-bit
// digits from the top, each counting in an LDS histogram the digits of the
// keys that still match the prefix found so far and picking the digit where
// the running count from the top reaches the number still to be chosen.
// The passes stop as soon as every key matching the prefix is to be kept
// (usually after two or three digits); otherwise after the last pass the
// prefix is T, the k-th largest key.  Then `rem` of the keys whose top bits
// equal the prefix are to be kept: a last sweep in index order keeps the
// keys above the prefix and the first `rem` keys equal to it, and compacts
// them with ballot prefix counts.  Exact, and independent of the schedule.
__device__ __forceinline__ unsigned long long score_key(double s) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(s + 0.0);
  return (u >> 63) ? ~u : (u | (1ull << 63));
}

__global__ void __launch_bounds__(64) topk_select_kernel(Geom g, const double *__restrict__ scores,
                                                         int32_t *__restrict__ idx) {
  extern __shared__ unsigned long long key[];  // [nb]
  __shared__ unsigned hist[256];
  const int bh = blockIdx.y, h = bh % g.H;
  if (!bit(g.topk, h)) return;
  const int nb = g.nb, k = g.k, lane = threadIdx.x;
  const int qb = blockIdx.x;
  const double *row = scores + ((long long)bh * nb + qb) * nb;
  for (int j = lane; j < nb; j += 64) key[j] = score_key(row[j]);

  unsigned long long prefix = 0, mask = 0;
  int rem = k;
  for (int shift = 56; shift >= 0; shift -= 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[lane + 64 * i] = 0;
    __syncthreads();
    for (int j = lane; j < nb; j += 64) {
      const unsigned long long kk = key[j];
      if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> shift) & 255], 1u);
    }
    __syncthreads();
    // lane L owns bins 4L..4L+3; suf = number of matching keys with digit >= 4L
    const unsigned c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                   c3 = hist[4 * lane + 3];
    const unsigned c = c0 + c1 + c2 + c3;
    unsigned suf = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned v = __shfl_down(suf, o);
      if (lane + o < 64) suf += v;
    }
    const unsigned need = unsigned(rem);
    const bool mine = suf >= need && suf - c < need;  // exactly one lane
    int d;
    unsigned greater, in_bin;
    if (suf - c0 - c1 - c2 >= need) { d = 4 * lane + 3; greater = suf - c; in_bin = c3; }
    else if (suf - c0 - c1 >= need) { d = 4 * lane + 2; greater = suf - c0 - c1 - c2; in_bin = c2; }
    else if (suf - c0 >= need) { d = 4 * lane + 1; greater = suf - c0 - c1; in_bin = c1; }
    else { d = 4 * lane; greater = suf - c0; in_bin = c0; }
    const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
    d = __shfl(d, src);
    greater = __shfl(greater, src);
    in_bin = __shfl(in_bin, src);
    prefix |= (unsigned long long)d << shift;
    mask |= 255ull << shift;
    rem -= int(greater);
    __syncthreads();  // histogram reads done before the next clear
    if (in_bin == unsigned(rem)) break;  // every key with this prefix is kept
  }

  int32_t *dst = idx + ((long long)bh * nb + qb) * k;
  int taken = 0, eq_seen = 0;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int j0 = 0; j0 < nb; j0 += 64) {
    const int j = j0 + lane;
    const unsigned long long kk = j < nb ? key[j] & mask : 0ull;
    const bool gt = j < nb && kk > prefix;
    const bool eq = j < nb && kk == prefix;
    const unsigned long long beq = __ballot(eq);
    const bool keep = gt || (eq && eq_seen + __popcll(beq & below) < rem);
    const unsigned long long bk = __ballot(keep);
    if (keep) dst[taken + __popcll(bk & below)] = j;
    taken += __popcll(bk);
    eq_seen += __popcll(beq);
  }
}

hipError_t launch_block_select(const Geom &g, int dtype_bf16, View qv, View kv, double *qbar,
                               double *kbar, double *scores, int32_t *idx, hipStream_t st) {
  dim3 grid1(g.B * g.H, g.nb, 2);
  if (dtype_bf16)
    block_mean_kernel<bf16_t><<<grid1, 256, 0, st>>>(g, qv, kv, qbar, kbar);
  else
    block_mean_kernel<float><<<grid1, 256, 0, st>>>(g, qv, kv, qbar, kbar);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid2((g.nb + kScoreTile - 1) / kScoreTile, (g.nb + kScoreTile - 1) / kScoreTile, g.B * g.H);
  block_score_kernel<<<grid2, 256, 0, st>>>(g, qbar, kbar, scores);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = size_t(g.nb) * sizeof(unsigned long long);
  if (lds > 48 * 1024)
    hipFuncSetAttribute((const void *)topk_select_kernel,
                        hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  dim3 grid3(g.nb, g.B * g.H);
  topk_select_kernel<<<grid3, 64, lds, st>>>(g, scores, idx);
  return hipGetLastError();
}

}  // namespace salad
