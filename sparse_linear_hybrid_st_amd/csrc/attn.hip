// Sparse branch: softmax attention of each working query over its kept keys.
//
// Sources: SALAD structured summary (paper.rainbus.top/paper/2601.16515),
// Prerequisites > Sparse Attention (a {-inf, 0} mask restricts the softmax
// to the kept query-key pairs; sliding window = static, Top-K = dynamic);
// ijyty.com/news/870645 sections 1.1 (1-D sliding window on the per-head
// re-ordered sequence) and 1.2 (attention restricted to the selected key
// blocks).  Window reading: keep key j for query p iff |p - j| <= r.
//
// bf16 path (d = 128): flash-style on v_mfma_f32_32x32x16_bf16.
//   * A workgroup owns a query tile (128 queries for window heads, one
//     64-query block for Top-K heads); each wave owns 32 queries and keeps
//     them in registers as MFMA B operands.
//   * Key tiles of 64 rows are staged in LDS: K row-major (XOR-swizzled
//     16-byte units), V transposed to [d][key] (swizzled 8-byte granules) so
//     that both MFMA operand reads are contiguous.  The next tile's global
//     loads are issued before the current tile's MFMAs.
//   * S^T = K Q^T puts one query per lane column, so the online softmax
//     (max, exp2, running sum) is lane-local except for one exchange between
//     the two half-waves; P^T then feeds O^T += V^T P^T directly from
//     registers (the key order inside an MFMA k-step is free, so P needs no
//     shuffle).
//   * Window heads skip key tiles outside the window, and tiles that lie
//     wholly inside every query's window skip the mask.  Top-K heads walk
//     the selected block list.
// f32 path (d = 64 or 128): one thread per query walks its key set.
#include "common.h"
#include "kernels.h"

namespace salad {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// f32 reference-grade kernel: thread = (b, h, p).
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(64) attn_f32_kernel(Geom g, View qv, View kv, View vv,
                                                      const int32_t *__restrict__ idx,
                                                      float *__restrict__ o_s) {
  const int bh = blockIdx.y, h = bh % g.H, b = bh / g.H;
  const int p = blockIdx.x * 64 + threadIdx.x;
  if (p >= g.N) return;
  const float *qb = (const float *)qv.base + row_offset(g, qv, b, h, p);
  float q[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = qb[c] * g.scale;
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const bool topk = bit(g.topk, h);
  const int nseg = topk ? g.k : 1;
  for (int sgi = 0; sgi < nseg; ++sgi) {
    int j0, j1;
    if (topk) {
      const int kb = idx[((long long)bh * g.nb + p / g.block) * g.k + sgi];
      if (kb < 0 || kb >= g.nb) continue;  // not a block index: no keys
      j0 = kb * g.block;
      j1 = min(g.N, j0 + g.block);
    } else {
      j0 = max(0, p - g.r);
      j1 = min(g.N, p + g.r + 1);
    }
    for (int j = j0; j < j1; ++j) {
      const float *kr = (const float *)kv.base + row_offset(g, kv, b, h, j);
      const float *vr = (const float *)vv.base + row_offset(g, vv, b, h, j);
      float sc = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) sc = fmaf(q[c], kr[c], sc);
      const float mn = fmaxf(m, sc);
      const float alpha = expf(m - mn), pj = expf(sc - mn);
      l = l * alpha + pj;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = fmaf(pj, vr[c], o[c] * alpha);
      m = mn;
    }
  }
  float *dst = o_s + ((long long)bh * g.N + p) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int c = 0; c < D; ++c) dst[c] = o[c] * inv;
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel, d = 128.
// ---------------------------------------------------------------------------
constexpr int kD = 128;   // head dim
constexpr int kBN = 64;   // keys per tile

// K tile: row = key (256 B), 16-byte unit u of row j stored at u ^ (j & 15).
__device__ __forceinline__ int k_unit(int j, int u) { return u ^ (j & 15); }
// V^T tile: row = feature (128 B = 16 granules of 4 keys); granule G of row
// rho stored at G ^ (((rho >> 1) ^ (rho >> 3)) & 15).
__device__ __forceinline__ int v_gran(int rho, int G) { return G ^ (((rho >> 1) ^ (rho >> 3)) & 15); }

struct AttnArgs {
  Geom g;
  View q, k, v;
  const int32_t *idx;
  float *o_s;            // working layout fp32 output
  int topk_mode;         // 0: window heads, 1: Top-K heads
  int n_heads_sel;       // heads handled by this launch
  uint8_t heads[kMaxHeads];
  int tiles_per_head;    // query tiles per (b, head)
};

template <int NW>
__global__ void __launch_bounds__(NW * 64) attn_bf16_kernel(AttnArgs a) {
  constexpr int BM = NW * 32;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[kBN * kD];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[kD * kBN];
  const Geom &g = a.g;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, hl = lane >> 5, l32 = lane & 31;

  // tile -> (b, head, query tile)
  const int tile = blockIdx.x;
  const int qt = tile % a.tiles_per_head;
  const int bhs = tile / a.tiles_per_head;
  const int h = a.heads[bhs % a.n_heads_sel];
  const int b = bhs / a.n_heads_sel;
  const int q0 = qt * BM;
  const int bh = b * g.H + h;

  const bf16_t *qbase = (const bf16_t *)a.q.base;
  const bf16_t *kbase = (const bf16_t *)a.k.base;
  const bf16_t *vbase = (const bf16_t *)a.v.base;

  // this wave's queries as B operands: lane -> query q0 + 32w + l32, features 16ks + 8hl + e
  const int pq = q0 + 32 * w + l32;
  bf16x8 qf[8];
  {
    const long long off = row_offset(g, a.q, b, h, min(pq, g.N - 1));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8 *)(qbase + off + (2 * ks + hl) * 8);
  }

  // key tile range
  int n_tiles, kt_first = 0;
  const int32_t *sel = nullptr;
  if (a.topk_mode) {
    n_tiles = g.k;
    sel = a.idx + ((long long)bh * g.nb + q0 / g.block) * g.k;
  } else {
    const int lo = max(0, q0 - g.r);
    const int hi = min(g.N - 1, q0 + BM - 1 + g.r);
    kt_first = lo / kBN;
    n_tiles = hi / kBN - kt_first + 1;
  }
  // wave's own query range (for skipping and mask-free tiles)
  const int wq_lo = q0 + 32 * w, wq_hi = min(q0 + 32 * w + 31, g.N - 1);

  const float sl2 = g.scale * 1.4426950408889634f;  // scale * log2(e)
  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // loader mapping (per thread): K: units (row, u) over 64 x 16; V: 4-key
  // groups kq x feature chunk c over 16 x 16.
  constexpr int KLOADS = (kBN * 16) / (NW * 64);
  constexpr int VLOADS = (16 * 16) / (NW * 64);
  u32x4 kreg[KLOADS];
  u32x4 vreg[VLOADS][4];

  // first key row of tile `it`; an out-of-range block index (only possible
  // if idx was not produced by the selection) maps past the end, where
  // every row is zero-filled and masked
  auto tile_start = [&](int it) -> int {
    if (!a.topk_mode) return (kt_first + it) * kBN;
    const int kb = sel[it];
    return (kb >= 0 && kb < g.nb) ? kb * g.block : g.N;
  };
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int e = t + i * NW * 64;
      const int row = e >> 4, u = e & 15;
      const int j = k0 + row;
      kreg[i] = j < g.N ? *(const u32x4 *)(kbase + row_offset(g, a.k, b, h, j) + u * 8)
                        : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int e = t + i * NW * 64;
      const int c = e & 15, kq = e >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = k0 + kq * 4 + r;
        vreg[i][r] = j < g.N ? *(const u32x4 *)(vbase + row_offset(g, a.v, b, h, j) + c * 8)
                             : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int e = t + i * NW * 64;
      const int row = e >> 4, u = e & 15;
      *(u32x4 *)(Ks + row * kD + k_unit(row, u) * 8) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int e = t + i * NW * 64;
      const int c = e & 15, kq = e >> 4;
      // feature c*8 + f for keys 4kq .. 4kq+3 -> one 8-byte granule
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int word = f >> 1, sh = (f & 1) * 16;
        const uint32_t k0v = (vreg[i][0][word] >> sh) & 0xffffu;
        const uint32_t k1v = (vreg[i][1][word] >> sh) & 0xffffu;
        const uint32_t k2v = (vreg[i][2][word] >> sh) & 0xffffu;
        const uint32_t k3v = (vreg[i][3][word] >> sh) & 0xffffu;
        const int rho = c * 8 + f;
        u32x2 gv = {k0v | (k1v << 16), k2v | (k3v << 16)};
        *(u32x2 *)(Vt + rho * kBN + v_gran(rho, kq) * 4) = gv;
      }
    }
  };

  if (n_tiles > 0) load_tile(tile_start(0));
  for (int it = 0; it < n_tiles; ++it) {
    const int k0 = tile_start(it);
    __syncthreads();
    store_tile();
    __syncthreads();
    if (it + 1 < n_tiles) load_tile(tile_start(it + 1));

    // does this wave have any kept pair in this tile?
    const int k1 = min(k0 + kBN, g.N) - 1;
    bool any, full;
    if (a.topk_mode) {
      any = true;
      full = (k0 + kBN) <= g.N;
    } else {
      any = (k0 <= wq_hi + g.r) && (k1 >= wq_lo - g.r) && (wq_lo <= wq_hi);
      full = (k0 + kBN <= g.N) && (k0 >= wq_hi - g.r) && (k0 + kBN - 1 <= wq_lo + g.r);
    }
    if (!any) continue;

    // S^T[key][query] for 2 blocks of 32 keys
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const int row = kb * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 ka = *(const bf16x8 *)(Ks + row * kD + k_unit(row, 2 * ks + hl) * 8);
        s[kb] = mfma_32x32x16(ka, qf[ks], s[kb]);
      }
    }
    // scale to log2 units, mask
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = s[kb][r] * sl2;
        if (!full) {
          const int j = k0 + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          const bool keep = j < g.N && (a.topk_mode || abs(pq - j) <= g.r);
          v = keep ? v : -INFINITY;
        }
        s[kb][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint16_t tmp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = exp2f(s[kb][8 * half + e] - m_use);
          psum += pv;
          tmp[e] = f32_to_bf16(pv);
        }
        pb[2 * kb + half] = *(const bf16x8 *)tmp;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    // O^T[d][q] += V^T[d][keys] P^T[keys][q]; k-step kk covers, for half hl,
    // keys 32*(kk/2) + 8*(2*(kk%2) + e/4) + 4*hl + e%4 (e = 0..7)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int kb = kk >> 1, k2 = kk & 1;
      const int G0 = (kb * 32 + 8 * (2 * k2) + 4 * hl) >> 2;
      const int G1 = (kb * 32 + 8 * (2 * k2 + 1) + 4 * hl) >> 2;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int rho = 32 * db + l32;
        const u32x2 lo = *(const u32x2 *)(Vt + rho * kBN + v_gran(rho, G0) * 4);
        const u32x2 hi = *(const u32x2 *)(Vt + rho * kBN + v_gran(rho, G1) * 4);
        u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
        o[db] = mfma_32x32x16(*(const bf16x8 *)&va, pb[kk], o[db]);
      }
    }
  }

  // finish: l over both half-waves, divide, store fp32 working rows
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (pq >= g.N) return;
  const float inv = 1.f / l_tot;
  float *dst = a.o_s + ((long long)bh * g.N + pq) * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 v = {o[db][4 * r4] * inv, o[db][4 * r4 + 1] * inv, o[db][4 * r4 + 2] * inv,
                 o[db][4 * r4 + 3] * inv};
      *(f32x4 *)(dst + 32 * db + 8 * r4 + 4 * hl) = v;
    }
}

hipError_t launch_sparse_attn(const Geom &g, int bf16, View qv, View kv, View vv,
                              const int32_t *idx, float *o_s, hipStream_t st) {
  if (!bf16) {
    dim3 grid((g.N + 63) / 64, g.B * g.H);
    if (g.D == 128)
      attn_f32_kernel<128><<<grid, 64, 0, st>>>(g, qv, kv, vv, idx, o_s);
    else
      attn_f32_kernel<64><<<grid, 64, 0, st>>>(g, qv, kv, vv, idx, o_s);
    return hipGetLastError();
  }
  for (int mode = 0; mode < 2; ++mode) {
    AttnArgs a;
    a.g = g;
    a.q = qv;
    a.k = kv;
    a.v = vv;
    a.idx = idx;
    a.o_s = o_s;
    a.topk_mode = mode;
    a.n_heads_sel = 0;
    for (int h = 0; h < g.H; ++h) {
      const bool is_topk = (g.topk[h >> 6] >> (h & 63)) & 1ull;
      if (is_topk == bool(mode)) a.heads[a.n_heads_sel++] = uint8_t(h);
    }
    if (a.n_heads_sel == 0) continue;
    const int BM = mode ? 64 : 128;
    a.tiles_per_head = (g.N + BM - 1) / BM;
    const unsigned grid = unsigned(a.tiles_per_head) * a.n_heads_sel * g.B;
    if (mode)
      attn_bf16_kernel<2><<<grid, 128, 0, st>>>(a);
    else
      attn_bf16_kernel<4><<<grid, 256, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace salad
