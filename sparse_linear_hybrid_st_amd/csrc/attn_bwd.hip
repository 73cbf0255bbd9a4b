// Backward of the sparse branch: dQ, dK and dV of softmax attention
// restricted to the kept query-key pairs, bf16, d = 128.  Rows are read in
// each head's working order: temporal heads from working copies, the other
// heads in place from the boundary layout.
//
// The forward is the sparse branch of the SALAD structured summary
// (paper.rainbus.top/paper/2601.16515), Prerequisites > Sparse Attention,
// with the window and Top-K key sets of ijyty.com/news/870645 sections 1.1
// and 1.2.  Its derivative, per query i over its kept keys j, with
// P_ij = exp(scale q_i.k_j) / sum_j' exp(scale q_i.k_j'):
//   dV_j += P_ij dO_i,   dP_ij = dO_i . v_j,   D_i = dO_i . O_i,
//   dS_ij = P_ij (dP_ij - D_i),
//   dQ_i = scale sum_j dS_ij k_j,   dK_j += scale dS_ij q_i.
// P is recomputed from the per-row normaliser that the preparation pass
// stored (lse2, in log2 units: P = exp2(scale log2(e) s - lse2)), so no N x N
// matrix is kept.  The Top-K selection is held fixed.
//
// The epilogues finish the layer's gradient rows: they add the linear
// branch's per-row terms (see linear_bwd.hip: dq from g M^T, den and dden;
// dk, dv from dH and dZ, all computed on MFMA with M, dH, dH^T staged in
// LDS), turn dQ and dK back through the transposed RoPE rotation, and store
// bf16 rows in the token-order boundary layout.
//
// Two kernels, each accumulating in registers and writing every output row
// once (no atomics, so results do not depend on scheduling):
//   * attn_bwd_dq_kernel walks the kept key tiles of a query tile, like the
//     forward: S^T = K Q^T and dP^T = V dO^T put one query per lane column,
//     then dQ^T += K^T dS^T with K^T from transposing LDS reads;
//   * attn_bwd_dkv_kernel walks the query tiles that keep a key tile:
//     S = Q K^T and dP = dO V^T put one key per lane column, then
//     dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T from transposing
//     LDS reads.  Top-K heads find their query blocks in an inverse list
//     (key block -> the query blocks that selected it) built per head.
#include "common.h"
#include "kernels.h"
#include "mfma_util.h"

namespace salad {

struct BwdArgs {
  Geom g;
  const bf16_t *q, *k, *v, *go;      // working layout [B*H][N][128] (Q, K rotated): heads in `work`
  const bf16_t *qd, *kd, *vd, *god;  // boundary layout [B][N][H][128] (Q, K rotated): other heads
  uint64_t work[4];                  // heads read from the working copies
  const float *lse2, *dsum;      // [B*H][Np]: normaliser (log2 units) and D per row
  int Np;                        // row stride of lse2 / dsum: N rounded up to 64
  const int32_t *idx;            // Top-K selection [B*H][nb][k]
  const int32_t *inv_off;        // Top-K: [B*H][nb + 1] offsets into inv_list of each key block
  const int32_t *inv_list;       // Top-K: [B*H][nb * k] selecting query blocks, ascending per key block
  BwdOut out;                    // linear-branch inputs and the bf16 outputs
  int n_heads_sel;
  uint8_t heads[kMaxHeads];
  int tiles_per_head;
  int n_blocks;
};

// ---------------------------------------------------------------------------
// Top-K inverse lists.  For key block kb of head (b, h): the query blocks
// whose selection contains kb, in ascending order.  One workgroup per head
// transposes the head's selection through a bitmap in LDS (row kb, bit qb),
// a chunk of key-block rows at a time: every selection entry sets its bit
// (LDS atomic OR, so the result does not depend on the order), each row's
// population count gives the counts, a workgroup scan the offsets (carried
// across chunks), and the set bits read in ascending order give the list.
// ---------------------------------------------------------------------------
constexpr int kInvThreads = 256;
constexpr int kInvLdsWords = 16384;  // 64 KB of bitmap per chunk

__host__ __device__ inline int inv_words(const Geom &g) { return (g.nb + 31) / 32; }
__host__ __device__ inline int inv_chunk_rows(const Geom &g) {
  const int r = kInvLdsWords / inv_words(g);
  return r < g.nb ? r : g.nb;
}

__global__ void __launch_bounds__(kInvThreads) topk_inverse_kernel(Geom g, const int32_t *__restrict__ idx,
                                                                   int32_t *__restrict__ off,
                                                                   int32_t *__restrict__ list) {
  extern __shared__ uint32_t bm[];  // [rows of the chunk][W]
  __shared__ int part[kInvThreads];
  const int bh = blockIdx.x, h = bh % g.H, t = threadIdx.x;
  if (!bit(g.topk, h)) return;
  const int W = inv_words(g), KC = inv_chunk_rows(g), nk = g.nb * g.k;
  const int32_t *sel = idx + (long long)bh * nk;
  int32_t *o = off + (long long)bh * (g.nb + 1);
  int32_t *lst = list + (long long)bh * nk;
  int carry = 0;  // entries in the chunks before this one
  for (int kc0 = 0; kc0 < g.nb; kc0 += KC) {
    const int rows = min(KC, g.nb - kc0);
    for (int i = t; i < rows * W; i += kInvThreads) bm[i] = 0u;
    __syncthreads();
    for (int e = t; e < nk; e += kInvThreads) {
      const int kb = sel[e] - kc0, qb = e / g.k;
      if (kb >= 0 && kb < rows) atomicOr(&bm[kb * W + (qb >> 5)], 1u << (qb & 31));
    }
    __syncthreads();
    // thread t owns rows [r0, r1) of the chunk, in order
    const int per = (rows + kInvThreads - 1) / kInvThreads;
    const int r0 = min(rows, t * per), r1 = min(rows, r0 + per);
    int mine = 0;
    for (int r = r0; r < r1; ++r)
      for (int i = 0; i < W; ++i) mine += __popc(bm[r * W + i]);
    part[t] = mine;
    __syncthreads();
    if (t == 0) {
      int run = carry;
      for (int i = 0; i < kInvThreads; ++i) {
        const int c = part[i];
        part[i] = run;
        run += c;
      }
    }
    __syncthreads();
    int n = part[t];
    for (int r = r0; r < r1; ++r) {
      o[kc0 + r] = n;
      for (int i = 0; i < W; ++i) {
        uint32_t word = bm[r * W + i];
        while (word) {
          lst[n++] = i * 32 + (__ffs(word) - 1);
          word &= word - 1u;
        }
      }
    }
    __syncthreads();  // every thread has read `part` and the bitmap
    if (t == kInvThreads - 1) part[0] = n;
    __syncthreads();
    carry = part[0];
    __syncthreads();
  }
  if (t == 0) o[g.nb] = carry;
}

// Rows of one (b, h): the working copy (rows 128 apart) for heads in
// `work`, else the boundary layout in place (rows H*128 apart), which holds
// those heads' rows in their working order, the token order.
struct HeadRows {
  const bf16_t *q, *k, *v, *go;
  int stride;
};
__device__ __forceinline__ HeadRows head_rows(const BwdArgs &a, int b, int h) {
  const Geom &g = a.g;
  HeadRows r;
  if (bit(a.work, h)) {
    const long long o = ((long long)b * g.H + h) * g.N * kD;
    r.q = a.q + o;
    r.k = a.k + o;
    r.v = a.v + o;
    r.go = a.go + o;
    r.stride = kD;
  } else {
    const long long o = ((long long)b * g.N * g.H + h) * kD;
    r.q = a.qd + o;
    r.k = a.kd + o;
    r.v = a.vd + o;
    r.go = a.god + o;
    r.stride = g.H * kD;
  }
  return r;
}

// ---------------------------------------------------------------------------
// Shared tile machinery.  A 64 x 128 bf16 tile of working rows (K, V, Q or
// dO) is staged in LDS row-major with the kv_swz unit swizzle; DMA op i of
// wave w fills rows 4*(i*NW + w) .. +3 (lane l: row + l/16, physical unit
// l%16, which holds logical unit (l%16) ^ kv_swz(row)); source rows are
// `stride` elements apart.  Rows past N re-read row N-1: finite values whose
// pairs are masked.
// ---------------------------------------------------------------------------
template <int NW>
struct TileDma {
  static constexpr int PER_WAVE = 16 / NW;  // 1-KB DMA ops per tile per wave
  int row[PER_WAVE], unit[PER_WAVE];
  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      row[i] = 4 * (i * NW + w) + (lane >> 4);
      unit[i] = (lane & 15) ^ kv_swz(row[i]);
    }
  }
  __device__ __forceinline__ void issue(const bf16_t *head, int r0, int N, bf16_t *dst, int w,
                                        int stride = kD) const {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int r = min(r0 + row[i], N - 1);
      __builtin_amdgcn_global_load_lds((const void *)(head + (long long)r * stride + unit[i] * 8),
                                       (lds_void *)(dst + (4 * (i * NW + w)) * kD), 16, 0, 0);
    }
  }
};

// LDS element offsets used by both kernels.  Row operand (row l32 of a
// 32-row block, logical unit 2ks + hl): k_lane + 16 * (ks ^ k_x).
// Transposing operand (rows of a k-step as the MFMA k index, features of
// d-block db as the lane index): t_off[r][db] plus 16*kk rows.
struct OperandOffsets {
  int k_lane, k_x;
  int t_off[2][4];
  __device__ __forceinline__ void init(int lane) {
    const int hl = lane >> 5, l32 = lane & 31;
    const int kswz = kv_swz(l32);
    k_lane = l32 * kD + 8 * (hl ^ (kswz & 1));
    k_x = kswz >> 1;
    const int gq = lane >> 4, jl = lane & 15;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int row = 8 * r + 4 * hl + (jl >> 2);
        const int d = 32 * db + 16 * (gq & 1) + 4 * (jl & 3);
        t_off[r][db] = row * kD + (((d >> 3) ^ kv_swz(row)) << 3) + (d & 4);
      }
  }
};

typedef __attribute__((ext_vector_type(8))) short s16x8;

// (cos, sin) of the RoPE pair starting at even feature f for the token at
// latent position (fr, y, x): the table holds one run per axis.
__device__ __forceinline__ double2 rope_entry(const Geom &g, const double2 *tab, int fr, int y, int x, int f) {
  const int h0 = g.rope_dims[0] >> 1, h1 = g.rope_dims[1] >> 1, h2 = g.rope_dims[2] >> 1;
  const int d0 = g.rope_dims[0], d1 = g.rope_dims[1];
  if (f < d0) return tab[fr * h0 + (f >> 1)];
  if (f < d0 + d1) return tab[g.F * h0 + y * h1 + ((f - d0) >> 1)];
  return tab[g.F * h0 + g.Hg * h1 + x * h2 + ((f - d0 - d1) >> 1)];
}

// Store gradient row values v[db][4 r4 + e] (feature 32db + 8r4 + 4hl + e)
// of working row p of head h as bf16 at the row's token in the boundary
// layout, rotated back by the transposed RoPE rotation when tab is set.
__device__ __forceinline__ void store_grad_row(const Geom &g, const double2 *tab, bf16_t *dst, int b, int h,
                                               int p, int hl, const f32x16 (&v)[4]) {
  const int tok = bit(g.temporal, h) ? st_token(g, p) : p;
  bf16_t *row = dst + (((long long)b * g.N + tok) * g.H + h) * kD;
  int fr = 0, y = 0, x = 0;
  if (tab) {
    const int S = g.Hg * g.Wg;
    fr = int(fdiv(g.fdS, uint32_t(tok)));
    const int site = tok - fr * S;
    y = int(fdiv(g.fdW, uint32_t(site)));
    x = site - y * g.Wg;
  }
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int f = 32 * db + 8 * r4 + 4 * hl;
      bf16_t o[4];
      if (tab) {
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const double2 cs = rope_entry(g, tab, fr, y, x, f + e);
          const double g0 = double(v[db][4 * r4 + e]), g1 = double(v[db][4 * r4 + e + 1]);
          o[e] = f64_to_bf16(g0 * cs.x + g1 * cs.y);
          o[e + 1] = f64_to_bf16(-g0 * cs.y + g1 * cs.x);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16(v[db][4 * r4 + e]);
      }
      *(uint2 *)(row + f) = *(const uint2 *)o;
    }
}

// A operand of k-step kk from a transposing read of tile Ts (rows 16kk..):
// lane -> feature 32db + l32, k index -> rows 16kk + 8r + 4hl + e.
__device__ __forceinline__ bf16x8 tr_operand(const bf16_t *Ts, const OperandOffsets &oo, int kk, int db) {
  const s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(Ts + 16 * kk * kD + oo.t_off[0][db]));
  const s16x4 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(Ts + 16 * kk * kD + oo.t_off[1][db]));
  const s16x8 v = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
  return *(const bf16x8 *)&v;
}

// ---------------------------------------------------------------------------
// dQ.  A workgroup owns a query tile (128 queries, 4 waves, window heads;
// one 64-query block, 2 waves, Top-K heads); wave w keeps queries
// q0 + 32w + l32 and their dO rows as MFMA B operands.  Key tiles of 64 are
// double-buffered in LDS.
// ---------------------------------------------------------------------------
template <int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_bwd_dq_kernel(BwdArgs a) {
  constexpr int BM = NW * 32;
  constexpr bool TOPK = NW == 2;
  // Top-K workgroups (2 waves) keep one K and one V buffer: 32 KB lets four
  // of them share a CU, whose other workgroups cover each one's DMA wait;
  // window workgroups (4 waves) double-buffer.
  constexpr bool SINGLE = TOPK;
  constexpr int TILE = kBN * kD;
  __shared__ __attribute__((aligned(1024))) bf16_t K0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16_t K1[SINGLE ? 8 : TILE];
  __shared__ __attribute__((aligned(1024))) bf16_t V0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16_t V1[SINGLE ? 8 : TILE];
  extern __shared__ int32_t sel_lds[];  // Top-K: first key row of each selected block
  const Geom &g = a.g;
  const int t = threadIdx.x, lane = t & 63, hl = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int tile = xcd_order(blockIdx.x, a.n_blocks);
  const int qt = tile % a.tiles_per_head, bhs = tile / a.tiles_per_head;
  const int h = a.heads[bhs % a.n_heads_sel], b = bhs / a.n_heads_sel;
  const int q0 = qt * BM, bh = b * g.H + h;
  const HeadRows hr = head_rows(a, b, h);
  const bf16_t *hk = hr.k, *hv = hr.v;
  const int rs = hr.stride;
  const int pq = q0 + 32 * w + l32, pqc = min(pq, g.N - 1);

  bf16x8 qf[8], gf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    qf[ks] = *(const bf16x8 *)(hr.q + (long long)pqc * rs + (2 * ks + hl) * 8);
    gf[ks] = *(const bf16x8 *)(hr.go + (long long)pqc * rs + (2 * ks + hl) * 8);
  }
  const float lse = a.lse2[(long long)bh * a.Np + pqc];
  const float dsv = a.dsum[(long long)bh * a.Np + pqc];
  const float c2 = g.scale * 1.4426950408889634f;

  int n_tiles, kt_first = 0;
  if (TOPK) {
    n_tiles = g.k;
    const int32_t *sel = a.idx + ((long long)bh * g.nb + q0 / g.block) * g.k;
    for (int j = t; j < n_tiles; j += NW * 64) {
      const int kb = sel[j];
      sel_lds[j] = (kb >= 0 && kb < g.nb) ? kb * g.block : g.N;
    }
    __syncthreads();
  } else {
    const int lo = max(0, q0 - g.r), hi = min(g.N - 1, q0 + BM - 1 + g.r);
    kt_first = lo / kBN;
    n_tiles = hi / kBN - kt_first + 1;
  }
  auto tile_start = [&](int it) -> int { return TOPK ? sel_lds[it] : (kt_first + it) * kBN; };
  const int wq_lo = q0 + 32 * w, wq_hi = min(q0 + 32 * w + 31, g.N - 1);

  TileDma<NW> dma;
  dma.init(w, lane);
  OperandOffsets oo;
  oo.init(lane);

  f32x16 dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dq[i] = f32x16{};

  auto compute = [&](int k0, const bf16_t *__restrict__ Ks, const bf16_t *__restrict__ Vs) {
    bool any, full;
    if (TOPK) {
      any = k0 < g.N;
      full = k0 + kBN <= g.N;
    } else {
      const int k1 = min(k0 + kBN, g.N) - 1;
      any = (k0 <= wq_hi + g.r) && (k1 >= wq_lo - g.r) && (wq_lo <= wq_hi);
      full = (k0 + kBN <= g.N) && (k0 >= wq_hi - g.r) && (k0 + kBN - 1 <= wq_lo + g.r);
    }
    if (!any) return;
    // S^T = K Q^T and dP^T = V dO^T, two blocks of 32 keys each
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int o = kb * 32 * kD + oo.k_lane + 16 * (ks ^ oo.k_x);
        s[kb] = mfma_32x32x16(*(const bf16x8 *)(Ks + o), qf[ks], s[kb]);
        dp[kb] = mfma_32x32x16(*(const bf16x8 *)(Vs + o), gf[ks], dp[kb]);
      }
    // dS^T = P^T (dP^T - D); key of register r of block kb:
    // k0 + 32kb + 8(r/4) + 4hl + r%4.  Edge tiles first set the scores of
    // dropped pairs to -inf, so their P (and dS, as dP is finite) is 0.
    if (!full) {
      const int jl = k0 + 4 * hl;
      const unsigned wb = unsigned(pq - jl + g.r);
      const int lim = g.N - jl;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + 8 * (r >> 2) + (r & 3);
          const bool keep = (c < lim) & (TOPK | (wb - unsigned(c) <= unsigned(2 * g.r)));
          s[kb][r] = keep ? s[kb][r] : -INFINITY;
        }
    }
    bf16x8 dsb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * half + e;
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c2, -lse));
          v[e] = (__bf16)(p * (dp[kb][r] - dsv));
        }
        dsb[2 * kb + half] = v;
      }
    // dQ^T[d][q] += K^T[d][keys] dS^T[keys][q]
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 ka[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) ka[db] = tr_operand(Ks, oo, kk, db);
#pragma unroll
      for (int db = 0; db < 4; ++db) dq[db] = mfma_32x32x16(ka[db], dsb[kk], dq[db]);
    }
  };

  int k_cur = n_tiles > 0 ? tile_start(0) : 0;
  if (n_tiles > 0) {
    dma.issue(hk, k_cur, g.N, K0, w, rs);
    dma.issue(hv, k_cur, g.N, V0, w, rs);
  }
  if constexpr (SINGLE) {
    // one buffer: wait for tile it, compute, then (every wave done) refill
    for (int it = 0; it < n_tiles; ++it) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      compute(k_cur, K0, V0);
      if (it + 1 < n_tiles) {
        k_cur = tile_start(it + 1);
        __syncthreads();
        dma.issue(hk, k_cur, g.N, K0, w, rs);
        dma.issue(hv, k_cur, g.N, V0, w, rs);
      }
    }
  } else {
    for (int it = 0; it < n_tiles; it += 2) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      const int k_nxt = it + 1 < n_tiles ? tile_start(it + 1) : 0;
      if (it + 1 < n_tiles) {
        dma.issue(hk, k_nxt, g.N, K1, w, rs);
        dma.issue(hv, k_nxt, g.N, V1, w, rs);
      }
      compute(k_cur, K0, V0);
      if (it + 1 >= n_tiles) break;
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      const int k_nn = it + 2 < n_tiles ? tile_start(it + 2) : 0;
      if (it + 2 < n_tiles) {
        dma.issue(hk, k_nn, g.N, K0, w, rs);
        dma.issue(hv, k_nn, g.N, V0, w, rs);
      }
      compute(k_nxt, K1, V1);
      k_cur = k_nn;
    }
  }

  // ---- epilogue: dq = scale * (sparse) + linear-branch term, rotated back
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] *= g.scale;
  const float sb = a.out.s_gate[b];
  if (!(sb < g.drop_tau)) {
    // gm^T = M g^T with M rows 0..63 in K0 and 64..127 in K1 (V0 when
    // single-buffered)
    __syncthreads();  // every wave is done with the key tiles
    bf16_t *const M1 = SINGLE ? V0 : K1;
    const bf16_t *mh = a.out.mb + (long long)bh * kD * kD;
    dma.issue(mh, 0, kD, K0, w);
    dma.issue(mh, 64, kD, M1, w);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    // one d-block of gm^T at a time (16 registers): a first pass forms
    // den = relu(q) . Z + eps and t = relu(q) . gm over this lane's 64
    // features and the other half-wave's (same query), a second pass
    // recomputes the block and adds the term
    const float *zr = a.out.zv + (long long)bh * kD;
    const bf16_t *qrow = hr.q + (long long)pqc * rs;
    auto gm_block = [&](int db) __attribute__((always_inline)) {
      const bf16_t *ms = (db < 2 ? K0 : M1) + (db & 1) * 32 * kD;
      f32x16 r = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) r = mfma_32x32x16(*(const bf16x8 *)(ms + oo.k_lane + 16 * (ks ^ oo.k_x)), gf[ks], r);
      return r;
    };
    float tp = 0.f, dp = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const f32x16 gm = gm_block(db);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int f = 32 * db + 8 * r4 + 4 * hl;
        const bf16x4 q4 = *(const bf16x4 *)(qrow + f);
        const f32x4 z4 = *(const f32x4 *)(zr + f);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float av = fmaxf(float(q4[e]), 0.f);
          tp = fmaf(av, gm[4 * r4 + e], tp);
          dp = fmaf(av, z4[e], dp);
        }
      }
    }
    tp += __shfl_xor(tp, 32);
    dp += __shfl_xor(dp, 32);
    const float den = dp + g.eps;
    const float dden = -sb * tp / (den * den), cq = sb / den;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const f32x16 gm = gm_block(db);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int f = 32 * db + 8 * r4 + 4 * hl;
        const bf16x4 q4 = *(const bf16x4 *)(qrow + f);
        const f32x4 z4 = *(const f32x4 *)(zr + f);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (float(q4[e]) > 0.f) dq[db][4 * r4 + e] += fmaf(cq, gm[4 * r4 + e], dden * z4[e]);
      }
    }
  }
  if (pq >= g.N) return;
  store_grad_row(g, a.out.rope_tab, a.out.dq, b, h, pq, hl, dq);
}

// ---------------------------------------------------------------------------
// dK, dV.  A workgroup owns a key tile (128 keys, 4 waves, window heads; one
// 64-key block, 2 waves, Top-K heads); wave w keeps keys k0 + 32w + l32 and
// their V rows as MFMA B operands.  Query tiles of 64 rows (Q, dO, lse2, D)
// are double-buffered in LDS and consumed as two 32-query halves.
// WHICH = 0 computes dK and dV together (one wave per SIMD: two 32 x 128
// accumulators and the K, V rows exceed the 256 registers that two waves
// per SIMD allow); WHICH = 1 computes dV only (S, P, dV) and WHICH = 2 dK
// only (S, dP, dS, dK), each within two waves per SIMD, at the price of S
// computed in both passes.
// ---------------------------------------------------------------------------
template <int NW, int WHICH>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WHICH == 0 ? 1 : 2, WHICH == 0 ? 1 : 2)))
attn_bwd_dkv_kernel(BwdArgs a) {
  constexpr int BK = NW * 32;
  constexpr bool TOPK = NW == 2;
  constexpr bool DO_V = WHICH != 2, DO_K = WHICH != 1;
  // Top-K workgroups of a single pass could keep one Q and one dO buffer
  // (four workgroups per CU, as in the dQ kernel); the others double-buffer.
  // Top-K heads run the joint pass: measured at 480p Top-K, the two
  // single-buffered passes took 7.3 ms against 6.2 ms joint.
  constexpr bool SINGLE = TOPK && WHICH != 0;
  constexpr int TILE = kBN * kD;
  __shared__ __attribute__((aligned(1024))) bf16_t Q0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16_t Q1[SINGLE ? 8 : TILE];
  __shared__ __attribute__((aligned(1024))) bf16_t G0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16_t G1[SINGLE ? 8 : TILE];
  __shared__ __attribute__((aligned(16))) float L0[kBN], L1[SINGLE ? 4 : kBN], D0[kBN], D1[SINGLE ? 4 : kBN];
  extern __shared__ int32_t qsel_lds[];  // Top-K: first query row of each selecting block
  const Geom &g = a.g;
  const int t = threadIdx.x, lane = t & 63, hl = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int tile = xcd_order(blockIdx.x, a.n_blocks);
  const int kt = tile % a.tiles_per_head, bhs = tile / a.tiles_per_head;
  const int h = a.heads[bhs % a.n_heads_sel], b = bhs / a.n_heads_sel;
  const int k0 = kt * BK, bh = b * g.H + h;
  const HeadRows hr = head_rows(a, b, h);
  const bf16_t *hq = hr.q, *hg = hr.go;
  const int rs = hr.stride;
  const float *hl2 = a.lse2 + (long long)bh * a.Np, *hds = a.dsum + (long long)bh * a.Np;
  const int pk = k0 + 32 * w + l32, pkc = min(pk, g.N - 1);

  bf16x8 kf[8], vf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    kf[ks] = *(const bf16x8 *)(hr.k + (long long)pkc * rs + (2 * ks + hl) * 8);
    if (DO_K) vf[ks] = *(const bf16x8 *)(hr.v + (long long)pkc * rs + (2 * ks + hl) * 8);
  }
  const float c2 = g.scale * 1.4426950408889634f;

  int n_tiles, qt_first = 0;
  if (TOPK) {
    const int kb = k0 / g.block;
    const int32_t *o = a.inv_off + (long long)bh * (g.nb + 1);
    const int beg = o[kb];
    n_tiles = o[kb + 1] - beg;
    const int32_t *lst = a.inv_list + (long long)bh * g.nb * g.k + beg;
    for (int j = t; j < n_tiles; j += NW * 64) qsel_lds[j] = lst[j] * g.block;
    __syncthreads();
  } else {
    const int lo = max(0, k0 - g.r), hi = min(g.N - 1, k0 + BK - 1 + g.r);
    qt_first = lo / kBN;
    n_tiles = hi / kBN - qt_first + 1;
  }
  auto tile_start = [&](int it) -> int { return TOPK ? qsel_lds[it] : (qt_first + it) * kBN; };
  const int wk_lo = k0 + 32 * w, wk_hi = k0 + 32 * w + 31;

  TileDma<NW> dma;
  dma.init(w, lane);
  OperandOffsets oo;
  oo.init(lane);
  // lse2 and D of a query tile: 16 lanes of wave 0 move 64 floats each
  // (the arrays are padded to a multiple of 64 rows per head)
  auto issue_tile = [&](int q0, bf16_t *Qd, bf16_t *Gd, float *Ld, float *Dd) {
    dma.issue(hq, q0, g.N, Qd, w, rs);
    dma.issue(hg, q0, g.N, Gd, w, rs);
    if (w == 0 && lane < 16) {
      __builtin_amdgcn_global_load_lds((const void *)(hl2 + q0 + 4 * lane), (lds_void *)Ld, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void *)(hds + q0 + 4 * lane), (lds_void *)Dd, 16, 0, 0);
    }
  };

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  auto compute = [&](int q0, const bf16_t *__restrict__ Qs, const bf16_t *__restrict__ Gs,
                     const float *__restrict__ Ls, const float *__restrict__ Ds) {
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const int i0 = q0 + 32 * qs;
      bool any, full;
      if (TOPK) {
        any = i0 < g.N;
        full = i0 + 31 < g.N;
      } else {
        any = (i0 < g.N) && (i0 <= wk_hi + g.r) && (i0 + 31 >= wk_lo - g.r);
        full = (i0 + 31 < g.N) && (i0 + 31 - wk_lo <= g.r) && (wk_hi - i0 <= g.r);
      }
      if (!any) continue;
      // S = Q K^T and dP = dO V^T for 32 queries (rows) x this wave's keys
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int o = qs * 32 * kD + oo.k_lane + 16 * (ks ^ oo.k_x);
        s = mfma_32x32x16(*(const bf16x8 *)(Qs + o), kf[ks], s);
        if (DO_K) dp = mfma_32x32x16(*(const bf16x8 *)(Gs + o), vf[ks], dp);
      }
      // query of register r: i0 + 8(r/4) + 4hl + r%4.  Edge blocks first
      // set the scores of dropped pairs to -inf (P = 0); rows past N also
      // get D = 0, as their lse2 / D slots hold no values
      bf16x8 pb[2], dsb[2];
      const unsigned wb = unsigned(i0 + 4 * hl - pk + g.r);  // i - pk + r = wb + c
      const int lim = g.N - i0 - 4 * hl;                    // i < N  <=>  c < lim
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f32x4 lv = *(const f32x4 *)(Ls + 32 * qs + 8 * m + 4 * hl);
        f32x4 dv4 = DO_K ? *(const f32x4 *)(Ds + 32 * qs + 8 * m + 4 * hl) : f32x4{};
        if (!full) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * m + e, c = 8 * m + e;
            const bool valid = c < lim;
            const bool keep = valid & (TOPK | (wb + unsigned(c) <= unsigned(2 * g.r)));
            s[r] = keep ? s[r] : -INFINITY;
            lv[e] = valid ? lv[e] : 0.f;
            dv4[e] = valid ? dv4[e] : 0.f;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * m + e;
          const float p = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -lv[e]));
          if (DO_V) pb[r >> 3][r & 7] = (__bf16)p;
          if (DO_K) dsb[r >> 3][r & 7] = (__bf16)(p * (dp[r] - dv4[e]));
        }
      }
      // dV^T[d][keys] += dO^T[d][q] P[q][keys];  dK^T += Q^T dS
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 ga[4], qa[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          if (DO_V) ga[db] = tr_operand(Gs + qs * 32 * kD, oo, kk, db);
          if (DO_K) qa[db] = tr_operand(Qs + qs * 32 * kD, oo, kk, db);
        }
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          if (DO_V) dv[db] = mfma_32x32x16(ga[db], pb[kk], dv[db]);
          if (DO_K) dk[db] = mfma_32x32x16(qa[db], dsb[kk], dk[db]);
        }
      }
    }
  };

  int q_cur = n_tiles > 0 ? tile_start(0) : 0;
  if (n_tiles > 0) issue_tile(q_cur, Q0, G0, L0, D0);
  if constexpr (SINGLE) {
    for (int it = 0; it < n_tiles; ++it) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      compute(q_cur, Q0, G0, L0, D0);
      if (it + 1 < n_tiles) {
        q_cur = tile_start(it + 1);
        __syncthreads();
        issue_tile(q_cur, Q0, G0, L0, D0);
      }
    }
  } else {
    for (int it = 0; it < n_tiles; it += 2) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      const int q_nxt = it + 1 < n_tiles ? tile_start(it + 1) : 0;
      if (it + 1 < n_tiles) issue_tile(q_nxt, Q1, G1, L1, D1);
      compute(q_cur, Q0, G0, L0, D0);
      if (it + 1 >= n_tiles) break;
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      const int q_nn = it + 2 < n_tiles ? tile_start(it + 2) : 0;
      if (it + 2 < n_tiles) issue_tile(q_nn, Q0, G0, L0, D0);
      compute(q_nxt, Q1, G1, L1, D1);
      q_cur = q_nn;
    }
  }

  // ---- epilogue: dk = scale * (sparse) + (dH v + dZ) [k > 0],
  //      dv = (sparse) + dH^T relu(k); dk rotated back
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[db][r] *= g.scale;
  if (!(a.out.s_gate[b] < g.drop_tau)) {
    // dH rows 0..63 in Q0, 64..127 in Q1; dH^T rows likewise in G0, G1.
    // Single-buffered (one of the two per pass): rows 64..127 in G0 / Q0.
    __syncthreads();  // every wave is done with the query tiles
    bf16_t *const H0 = Q0, *const H1 = SINGLE ? G0 : Q1;
    bf16_t *const T0 = SINGLE ? Q0 : G0, *const T1 = SINGLE ? G0 : G1;
    const long long hm_off = (long long)bh * kD * kD;
    if (DO_K) {
      dma.issue(a.out.dhb + hm_off, 0, kD, H0, w);
      dma.issue(a.out.dhb + hm_off, 64, kD, H1, w);
    }
    if (DO_V) {
      dma.issue(a.out.dhtb + hm_off, 0, kD, T0, w);
      dma.issue(a.out.dhtb + hm_off, 64, kD, T1, w);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    // dv^T[j][key] += sum_i dH^T[j][i] relu(k)[i]
#pragma unroll
    for (int ks = 0; ks < 8 && DO_V; ++ks) {
      bf16x8 kr;
#pragma unroll
      for (int e = 0; e < 8; ++e) kr[e] = float(kf[ks][e]) > 0.f ? kf[ks][e] : (__bf16)0.f;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16_t *ht = (db < 2 ? T0 : T1) + (db & 1) * 32 * kD;
        dv[db] = mfma_32x32x16(*(const bf16x8 *)(ht + oo.k_lane + 16 * (ks ^ oo.k_x)), kr, dv[db]);
      }
    }
    // dk^T[i][key] += ([k_i > 0] (sum_j dH[i][j] v[j] + dZ[i])), one d-block at a time
    const float *dz = a.out.dz + (long long)bh * kD;
#pragma unroll
    for (int db = 0; db < 4 && DO_K; ++db) {
      f32x16 lk = f32x16{};
      const bf16_t *hs = (db < 2 ? H0 : H1) + (db & 1) * 32 * kD;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) lk = mfma_32x32x16(*(const bf16x8 *)(hs + oo.k_lane + 16 * (ks ^ oo.k_x)), vf[ks], lk);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int f = 32 * db + 8 * r4 + 4 * hl;
        const bf16x4 k4 = *(const bf16x4 *)(hr.k + (long long)pkc * rs + f);
        const f32x4 z4 = *(const f32x4 *)(dz + f);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (float(k4[e]) > 0.f) dk[db][4 * r4 + e] += lk[4 * r4 + e] + z4[e];
      }
    }
  }
  if (pk >= g.N) return;
  if (DO_K) store_grad_row(g, a.out.rope_tab, a.out.dk, b, h, pk, hl, dk);
  if (DO_V) store_grad_row(g, nullptr, a.out.dv, b, h, pk, hl, dv);
}

// ---------------------------------------------------------------------------
// Launchers: one launch per head kind and kernel (window heads with 4
// waves, Top-K heads with 2).
// ---------------------------------------------------------------------------
hipError_t launch_topk_inverse(const Geom &g, const int32_t *idx, int32_t *off, int32_t *list,
                               hipStream_t st) {
  const size_t lds = size_t(inv_chunk_rows(g)) * inv_words(g) * sizeof(uint32_t);
  if (lds > 48 * 1024)
    hipFuncSetAttribute((const void *)topk_inverse_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  topk_inverse_kernel<<<g.B * g.H, kInvThreads, lds, st>>>(g, idx, off, list);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const Geom &g, const bf16_t *q, const bf16_t *k, const bf16_t *v,
                           const bf16_t *go, const bf16_t *qd, const bf16_t *kd, const bf16_t *vd,
                           const bf16_t *god, const uint64_t work[4], const float *lse2, const float *dsum,
                           int Np, const int32_t *idx, const int32_t *inv_off, const int32_t *inv_list,
                           const BwdOut &out, hipStream_t st) {
  if (g.D != kD) return hipErrorInvalidValue;
  BwdArgs a = {};
  a.g = g;
  a.q = q;
  a.k = k;
  a.v = v;
  a.go = go;
  a.qd = qd;
  a.kd = kd;
  a.vd = vd;
  a.god = god;
  for (int i = 0; i < 4; ++i) a.work[i] = work[i];
  a.lse2 = lse2;
  a.dsum = dsum;
  a.Np = Np;
  a.idx = idx;
  a.inv_off = inv_off;
  a.inv_list = inv_list;
  a.out = out;
  for (int mode = 0; mode < 2; ++mode) {
    a.n_heads_sel = 0;
    for (int h = 0; h < g.H; ++h) {
      const bool is_topk = (g.topk[h >> 6] >> (h & 63)) & 1ull;
      if (is_topk == bool(mode)) a.heads[a.n_heads_sel++] = uint8_t(h);
    }
    if (a.n_heads_sel == 0) continue;
    const int BM = mode ? 64 : 128;
    a.tiles_per_head = (g.N + BM - 1) / BM;
    const unsigned grid = unsigned(a.tiles_per_head) * a.n_heads_sel * g.B;
    a.n_blocks = int(grid);
    if (mode) {
      attn_bwd_dq_kernel<2><<<grid, 128, size_t(g.k) * sizeof(int32_t), st>>>(a);
      attn_bwd_dkv_kernel<2, 0><<<grid, 128, size_t(g.nb) * sizeof(int32_t), st>>>(a);
    } else {
      attn_bwd_dq_kernel<4><<<grid, 256, 0, st>>>(a);
      attn_bwd_dkv_kernel<4, 1><<<grid, 256, 0, st>>>(a);
      attn_bwd_dkv_kernel<4, 2><<<grid, 256, 0, st>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace salad
