// Top-K block selection: block-mean pooling of Q and K, block scores and
// the k best key blocks per query block.
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

// Scores and selection.  One workgroup handles `qpb` query blocks of one
// (b, h): scores[q][kb] = qbar[q] . kbar[kb] (float64, LDS), then for each
// query block a candidate kb is kept iff fewer than k candidates beat it
// (higher score, or equal score and lower index); kept indices are written
// ascending via a prefix count.
__global__ void __launch_bounds__(256) topk_select_kernel(Geom g, const double *__restrict__ qbar,
                                                          const double *__restrict__ kbar,
                                                          int32_t *__restrict__ idx, int qpb) {
  extern __shared__ double smem[];
  const int bh = blockIdx.y;
  const int h = bh % g.H;
  if (!bit(g.topk, h)) return;
  const int nb = g.nb, D = g.D, t = threadIdx.x;
  const int qb0 = blockIdx.x * qpb;
  const int nq = min(qpb, nb - qb0);
  double *qs = smem;              // [qpb][D]
  double *sc = smem + qpb * D;    // [qpb][nb]
  __shared__ int wave_count[4];
  for (int i = t; i < nq * D; i += 256) qs[i] = qbar[((long long)bh * nb + qb0) * D + i];
  __syncthreads();
  const double *kb_base = kbar + (long long)bh * nb * D;
  for (int kb = t; kb < nb; kb += 256) {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const double *kr = kb_base + (long long)kb * D;
    for (int c = 0; c < D; ++c) {
      double kvv = kr[c];
      for (int q = 0; q < nq; ++q) acc[q] = fma(qs[q * D + c], kvv, acc[q]);
    }
    for (int q = 0; q < nq; ++q) sc[q * nb + kb] = acc[q];
  }
  __syncthreads();
  const int lane = t & 63, wv = t >> 6;
  for (int q = 0; q < nq; ++q) {
    const double *s = sc + q * nb;
    int32_t *dst = idx + ((long long)bh * nb + qb0 + q) * g.k;
    int base_count = 0;  // kept candidates with a lower index than this pass
    for (int j0 = 0; j0 < nb; j0 += 256) {
      const int j = j0 + t;
      bool keep = false;
      if (j < nb) {
        const double sj = s[j];
        int beat = 0;
        for (int i = 0; i < nb; ++i) {
          const double si = s[i];
          beat += (si > sj) || (si == sj && i < j);
        }
        keep = beat < g.k;
      }
      const uint64_t m = __ballot(keep);
      if (lane == 0) wave_count[wv] = __popcll(m);
      __syncthreads();
      int before = base_count;
      for (int w = 0; w < wv; ++w) before += wave_count[w];
      before += __popcll(m & ((1ull << lane) - 1ull));
      if (keep && before < g.k) dst[before] = j;  // NaN scores cannot overrun the row
      base_count += wave_count[0] + wave_count[1] + wave_count[2] + wave_count[3];
      __syncthreads();
    }
  }
}

hipError_t launch_block_select(const Geom &g, int dtype_bf16, View qv, View kv, double *qbar,
                               double *kbar, int32_t *idx, hipStream_t st) {
  dim3 grid1(g.nb, 2, g.B * g.H);
  if (dtype_bf16)
    block_mean_kernel<bf16_t><<<grid1, 256, 0, st>>>(g, qv, kv, qbar, kbar);
  else
    block_mean_kernel<float><<<grid1, 256, 0, st>>>(g, qv, kv, qbar, kbar);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int qpb = topk_queries_per_group(g.nb, g.D);
  dim3 grid2((g.nb + qpb - 1) / qpb, g.B * g.H);
  size_t lds = size_t(qpb) * (g.D + g.nb) * sizeof(double);
  topk_select_kernel<<<grid2, 256, lds, st>>>(g, qbar, kbar, idx, qpb);
  return hipGetLastError();
}

}  // namespace salad
