// Top-K block selection: block-mean pooling of Q and K, block scores and
// the k best key blocks per query block (fp64 scores, bitonic sort).
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

// One workgroup per (b, h, block) of one tensor (blockIdx.y: 0 = Q, 1 = K).
// 256 threads: 16 row groups x 16 column chunks of 8 elements.
template <typename T>
__global__ void __launch_bounds__(256) block_mean_kernel(Geom g, View qv, View kv,
                                                         double *__restrict__ qbar,
                                                         double *__restrict__ kbar) {
  const int blk = blockIdx.x;
  const int bh = blockIdx.z;
  const int h = bh % g.H, b = bh / g.H;
  if (!bit(g.topk, h)) return;
  const View v = blockIdx.y ? kv : qv;
  double *out = (blockIdx.y ? kbar : qbar) + ((long long)bh * g.nb + blk) * g.D;
  const T *base = (const T *)v.base;
  const int t = threadIdx.x, rg = t >> 4, ch = t & 15;
  const int row0 = blk * g.block;
  const int rows = min(g.block, g.N - row0);
  __shared__ double part[16][128];
  const int cols = g.D / 8;  // column chunks in use (8 or 16)
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (ch < cols) {
    for (int r = rg; r < rows; r += 16) {
      const T *src = base + row_offset(g, v, b, h, row0 + r) + ch * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += double(io<T>::ld(src + e));
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

// Block scores S[qb][kb] = qbar[qb] . kbar[kb] for every Top-K (b, h), as a
// tiled fp64 product: workgroup (tile_q, tile_k, bh) computes a 32 x 32 tile,
// staging 32-column slices of both operands in LDS; thread t owns rows
// 4*(t/32)..+3 at column t%32.  Each product is a plain left-to-right fp64
// sum over the d features.
__global__ void __launch_bounds__(256) block_score_kernel(Geom g, const double *__restrict__ qbar,
                                                          const double *__restrict__ kbar,
                                                          double *__restrict__ scores) {
  const int bh = blockIdx.z, h = bh % g.H;
  if (!bit(g.topk, h)) return;
  const int nb = g.nb, D = g.D, t = threadIdx.x;
  const int q0 = blockIdx.x * 32, k0 = blockIdx.y * 32;
  __shared__ double qs[32][33];
  __shared__ double ks[32][33];
  const double *qb = qbar + (long long)bh * nb * D;
  const double *kb = kbar + (long long)bh * nb * D;
  const int r0 = 4 * (t >> 5), c = t & 31;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int f0 = 0; f0 < D; f0 += 32) {
    __syncthreads();
    for (int e = t; e < 32 * 32; e += 256) {
      const int r = e >> 5, f = e & 31;
      qs[r][f] = (q0 + r < nb) ? qb[(long long)(q0 + r) * D + f0 + f] : 0.0;
      ks[r][f] = (k0 + r < nb) ? kb[(long long)(k0 + r) * D + f0 + f] : 0.0;
    }
    __syncthreads();
    for (int f = 0; f < 32; ++f) {
      const double kv = ks[c][f];
#pragma unroll
      for (int a = 0; a < 4; ++a) acc[a] = fma(qs[r0 + a][f], kv, acc[a]);
    }
  }
  if (k0 + c < nb) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
      if (q0 + r0 + a < nb) scores[((long long)bh * nb + q0 + r0 + a) * nb + k0 + c] = acc[a];
  }
}

// Selection for one query block per workgroup: bitonic sort of the P =
// next_pow2(nb) (score, block) pairs in LDS into the order "higher score
// first, equal scores lower block first" (padding sorts last), flag the
// first k blocks, then write the flagged block indices ascending with a
// ballot prefix count.  The order is total, so the result does not depend on
// the sort's internal schedule.
__device__ __forceinline__ bool sel_before(double sa, int ia, double sb, int ib) {
  return sa > sb || (sa == sb && ia < ib);
}

__global__ void __launch_bounds__(256) topk_sort_kernel(Geom g, const double *__restrict__ scores,
                                                        int32_t *__restrict__ idx, int P) {
  extern __shared__ double sel_smem[];
  const int bh = blockIdx.y, h = bh % g.H;
  if (!bit(g.topk, h)) return;
  const int nb = g.nb, qb = blockIdx.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  double *key = sel_smem;                       // [P]
  int *id = (int *)(sel_smem + P);              // [P]
  unsigned char *flag = (unsigned char *)(id + P);  // [P]
  __shared__ int wave_count[4];
  const double *row = scores + ((long long)bh * nb + qb) * nb;
  for (int j = t; j < P; j += 256) {
    key[j] = j < nb ? row[j] : -INFINITY;
    id[j] = j < nb ? j : 0x7fffffff;
    flag[j] = 0;
  }
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int p = t; p < (P >> 1); p += 256) {
        const int i = 2 * p - (p & (stride - 1));
        const int j = i + stride;
        const double ki = key[i], kj = key[j];
        const int ii = id[i], ij = id[j];
        // ascending runs (i & size == 0) put the "before" element first
        const bool first_i = ((i & size) == 0);
        const bool swap = first_i ? sel_before(kj, ij, ki, ii) : sel_before(ki, ii, kj, ij);
        if (swap) {
          key[i] = kj;
          key[j] = ki;
          id[i] = ij;
          id[j] = ii;
        }
      }
      __syncthreads();
    }
  }
  for (int r = t; r < g.k; r += 256) flag[id[r]] = 1;
  __syncthreads();
  int32_t *dst = idx + ((long long)bh * nb + qb) * g.k;
  int base_count = 0;
  for (int j0 = 0; j0 < nb; j0 += 256) {
    const int j = j0 + t;
    const bool keep = j < nb && flag[j];
    const uint64_t m = __ballot(keep);
    if (lane == 0) wave_count[wv] = __popcll(m);
    __syncthreads();
    int before = base_count;
    for (int w2 = 0; w2 < wv; ++w2) before += wave_count[w2];
    before += __popcll(m & ((1ull << lane) - 1ull));
    if (keep && before < g.k) dst[before] = j;
    base_count += wave_count[0] + wave_count[1] + wave_count[2] + wave_count[3];
    __syncthreads();
  }
}

int select_pow2(int nb) {
  int P = 2;
  while (P < nb) P <<= 1;
  return P;
}

hipError_t launch_block_select(const Geom &g, int dtype_bf16, View qv, View kv, double *qbar,
                               double *kbar, double *scores, int32_t *idx, hipStream_t st) {
  dim3 grid1(g.nb, 2, g.B * g.H);
  if (dtype_bf16)
    block_mean_kernel<bf16_t><<<grid1, 256, 0, st>>>(g, qv, kv, qbar, kbar);
  else
    block_mean_kernel<float><<<grid1, 256, 0, st>>>(g, qv, kv, qbar, kbar);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid2((g.nb + 31) / 32, (g.nb + 31) / 32, g.B * g.H);
  block_score_kernel<<<grid2, 256, 0, st>>>(g, qbar, kbar, scores);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int P = select_pow2(g.nb);
  const size_t lds = size_t(P) * (sizeof(double) + sizeof(int) + 1);
  if (lds > 64 * 1024)
    hipFuncSetAttribute((const void *)topk_sort_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                        int(lds));
  dim3 grid3(g.nb, g.B * g.H);
  topk_sort_kernel<<<grid3, 256, lds, st>>>(g, scores, idx, P);
  return hipGetLastError();
}

}  // namespace salad
