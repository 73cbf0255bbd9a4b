// Backward of the linear branch and of the per-head projection, bf16,
// d = 128 (rows in each head's working order, as in attn_bwd.hip).
//
// Forward (SALAD structured summary, paper.rainbus.top/paper/2601.16515,
// Prerequisites > Linear Attention and method steps 4-6): per (b, h), with
// a_n = relu(q_n), H = relu(K)^T V, Z = relu(K)^T 1, den_n = a_n . Z + eps,
// O_l = a_n H / den_n and out += s_b O_l W_p.  Given G = dL/dout (rows g_n)
// and M = H W_p, the chain rule gives (dO_l = s g W_p^T, so a_n H W_p g_n^T
// = a_n . (g_n M^T)):
//   gm_n  = g_n M^T,             t_n = a_n . gm_n,
//   dden_n = -s t_n / den_n^2,    dq_n += ((s / den_n) gm_n + dden_n Z) * [q_n > 0]
//   A     = sum_n (a_n / den_n)^T g_n,   Bz = sum_n dden_n a_n
//   dH    = s A W_p^T,   dZ = Bz,   dW_p += s H^T A,   dL/ds_b += <M, A>
//   dk_n += (dH v_n + dZ) * [k_n > 0],   dv_n += dH^T relu(k_n).
// A sample whose branch is dropped (s_b < drop_tau) is skipped throughout.
//
// Kernels here: lin_bwd_prep (M per head), lin_bwd_rows (gm and the
// split-N partial sums of A and Bz on MFMA), the split reduction (the
// forward's linear_reduce_kernel), lin_bwd_head (dH, dH^T as bf16, per-head
// dW_p and <M, A>) and lin_bwd_wp (dW_p summed over heads in a fixed
// order).  They run before the sparse-branch gradient kernels, whose
// epilogues add the per-row terms (dq from gm, den and dden; dk, dv from
// dH and dZ), so no gradient row is written twice.
#include "common.h"
#include "kernels.h"
#include "mfma_util.h"

namespace salad {

namespace {
constexpr int D = 128;

__device__ __forceinline__ bool dropped(const Geom &g, const float *s_gate, int b) {
  return s_gate[b] < g.drop_tau;
}

// Row operand offsets (row l32 of a 32-row block of a swizzled [.][128]
// tile, logical unit 2ks + hl) -- as in the attention kernels.
struct RowOp {
  int lane_off, x;
  __device__ __forceinline__ void init(int lane) {
    const int hl = lane >> 5, l32 = lane & 31, sw = kv_swz(l32);
    lane_off = l32 * D + 8 * (hl ^ (sw & 1));
    x = sw >> 1;
  }
  __device__ __forceinline__ int at(int blk32, int ks) const { return blk32 * 32 * D + lane_off + 16 * (ks ^ x); }
};

// Stage a [128][128] bf16 matrix into LDS with the unit swizzle (256 threads).
__device__ __forceinline__ void stage_swizzled(bf16_t *dst, const bf16_t *src, int t) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int u = t + 256 * i, row = u >> 4, unit = u & 15;
    *(u32x4 *)(dst + row * D + ((unit ^ kv_swz(row)) << 3)) = *(const u32x4 *)(src + row * D + unit * 8);
  }
}
}  // namespace

// M = H W_p (fp32 and bf16, row-major).  Grid (16, B*H); block blk owns rows
// 8 blk .. +7; thread t: row t/32, columns (t%32) + 32m.
__global__ void __launch_bounds__(256) lin_bwd_prep_kernel(Geom g, const float *__restrict__ hm,
                                                           const bf16_t *__restrict__ w_p,
                                                           const float *__restrict__ s_gate,
                                                           float *__restrict__ mf, bf16_t *__restrict__ mb) {
  __shared__ __attribute__((aligned(16))) bf16_t Ws[D * D];
  __shared__ float Hs[8 * D];
  const int blk = blockIdx.x, bh = blockIdx.y, b = bh / g.H, t = threadIdx.x;
  if (dropped(g, s_gate, b)) return;
  for (int e = t * 8; e < D * D; e += 256 * 8) *(u32x4 *)(Ws + e) = *(const u32x4 *)(w_p + e);
  const float *hr = hm + ((long long)bh * D + 8 * blk) * D;
  for (int e = t; e < 8 * D; e += 256) Hs[e] = hr[e];
  __syncthreads();
  const int ii = t >> 5, jg = t & 31;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int k = 0; k < D; ++k) {
    const float hv = Hs[ii * D + k];
#pragma unroll
    for (int m = 0; m < 4; ++m) o[m] = fmaf(hv, bf16_to_f32(Ws[k * D + jg + 32 * m]), o[m]);
  }
  const long long row = ((long long)bh * D + 8 * blk + ii) * D;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    mf[row + jg + 32 * m] = o[m];
    mb[row + jg + 32 * m] = f32_to_bf16(o[m]);
  }
}

// Per row gm and the split-N partials of A (128 x 128) and Bz (128).  With
// the forward's output given (outv.base non-NULL), also each row's
// D = dO . O_s for the sparse branch's backward, from
// O_s = out - s_b O_l W_p = out - s_b (a M) / den, whose dot with dO is
// dO . out - s_b t / den (t = a . gm, already at hand); dropped samples
// (out = O_s) only get D = dO . out.
// Grid (S, B*H), 256 threads; split s covers rows [s*chunk, (s+1)*chunk).
// A step handles 128 rows: wave w owns rows 32w + l32 (one per lane column)
// for gm^T = M g^T on MFMA (M rows from LDS, g rows as B operands) and the
// dot products; it then leaves a_n / den_n and g_n (bf16) in LDS, and
// each wave adds its 64 x 64 quadrant of A over the 128 rows with
// transposing reads.  Each step's rows (dO, q and out) are loaded into
// registers during the step before, so the global loads overlap the MFMA
// work (one wave per SIMD here: nothing else hides them).  Fixed order
// throughout.
__global__ void __launch_bounds__(256, 1) lin_bwd_rows_kernel(Geom g, const bf16_t *__restrict__ qw,
                                                              const bf16_t *__restrict__ gw,
                                                              const bf16_t *__restrict__ qd,
                                                              const bf16_t *__restrict__ god, HeadSet work,
                                                              const bf16_t *__restrict__ mb,
                                                              const float *__restrict__ zv,
                                                              const float *__restrict__ s_gate,
                                                              float *__restrict__ partial, int S, int chunk,
                                                              View outv, float *__restrict__ dsum, int Np) {
  constexpr int TT = 128;
  __shared__ __attribute__((aligned(1024))) bf16_t Ms[D * D];
  __shared__ __attribute__((aligned(1024))) bf16_t At[TT * D];
  __shared__ __attribute__((aligned(1024))) bf16_t Gt[TT * D];
  __shared__ __attribute__((aligned(16))) float Zs[D];
  __shared__ float wrow[TT];
  const int s = blockIdx.x, bh = blockIdx.y, b = bh / g.H;
  const int t = threadIdx.x, lane = t & 63, hl = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int n0 = s * chunk, n1 = min(g.N, n0 + chunk);
  const int h = bh % g.H;
  const bf16_t *outb = (const bf16_t *)outv.base;
  // this head's Q and dO rows: working copies (rows D apart) or, for heads
  // outside `work`, the boundary layout in place (rows H*D apart)
  const bool fw = bit(work.w, h);
  const long long hoff = fw ? (long long)bh * g.N * D : ((long long)b * g.N * g.H + h) * D;
  const bf16_t *q = (fw ? qw : qd) + hoff, *go = (fw ? gw : god) + hoff;
  const int rs = fw ? D : g.H * D;
  // dO . out over this lane's features f = 32db + 8r4 + 4hl + e of row n,
  // completed across the two half-waves (same row); dropped samples only
  auto go_out = [&](int n) __attribute__((always_inline)) {
    const bf16_t *gr = go + (long long)n * rs;
    const bf16_t *orow = outb + row_offset(g, outv, b, h, n);
    float acc = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int f = 32 * db + 8 * r4 + 4 * hl;
        const bf16x4 g4 = *(const bf16x4 *)(gr + f), o4 = *(const bf16x4 *)(orow + f);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fmaf(float(g4[e]), float(o4[e]), acc);
      }
    return acc + __shfl_xor(acc, 32);
  };
  if (dropped(g, s_gate, b)) {
    if (!outb) return;
    for (int base = n0; base < n1; base += 128) {
      const int n = base + 32 * w + l32;
      if (n >= n1) continue;  // both half-waves of a row skip together
      const float dv = go_out(n);
      if (hl == 0) dsum[(long long)bh * Np + n] = dv;
    }
    return;
  }
  const float sb = s_gate[b];
  stage_swizzled(Ms, mb + (long long)bh * D * D, t);
  if (t < D) Zs[t] = zv[(long long)bh * D + t];
  RowOp ro;
  ro.init(lane);
  // transposing-read offsets for the A reduction (rows as the k index):
  // row 8hl + 4r + jl/4 of a 16-row step, feature f0 + 4*(jl%4)
  const int i0 = (w >> 1) * 64, j0 = (w & 1) * 64;
  const int gq = lane >> 4, jl = lane & 15;
  int toff[2][2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int op = 0; op < 2; ++op) {
        const int row = 8 * hl + 4 * r + (jl >> 2);
        const int f = (op ? j0 : i0) + 32 * bi + 16 * (gq & 1) + 4 * (jl & 3);
        toff[op][bi][r] = row * D + (((f >> 3) ^ kv_swz(row)) << 3) + (f & 4);
      }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  float bz[4] = {0.f, 0.f, 0.f, 0.f};  // Bz[4(t%32) .. +3] over rows of group t/32
  __syncthreads();

  // one step's rows in registers: dO as B operands (features 16ks + 8hl + e)
  // and q in the accumulator layout (features 32db + 8r4 + 4hl + e)
  struct Rows {
    bf16x8 gf[8];
    bf16x4 qv[4][4];
  };
  auto load_rows = [&](int base, Rows &R) __attribute__((always_inline)) {
    const int n = base + 32 * w + l32;
    const long long nc = (long long)(n < n1 ? n : n0) * rs;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) R.gf[ks] = *(const bf16x8 *)(go + nc + (2 * ks + hl) * 8);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) R.qv[db][r4] = *(const bf16x4 *)(q + nc + 32 * db + 8 * r4 + 4 * hl);
  };
  auto step = [&](int base, Rows &R) __attribute__((always_inline)) {
    const int rl = 32 * w + l32, n = base + rl;
    const bool valid = n < n1;
    // this step's out row (dO layout: its dot with dO needs only matching
    // features), issued before the MFMAs that hide its latency
    bf16x8 of[8];
    if (outb) {
      const bf16_t *orow = outb + row_offset(g, outv, b, h, valid ? n : n0);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) of[ks] = *(const bf16x8 *)(orow + (2 * ks + hl) * 8);
    }
    if (!valid) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) R.gf[ks] = bf16x8{};
    }
    // gm^T[f][n] = sum_j M[f][j] g_n[j]
    f32x16 gm[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) gm[db] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int db = 0; db < 4; ++db) gm[db] = mfma_32x32x16(*(const bf16x8 *)(Ms + ro.at(db, ks)), R.gf[ks], gm[db]);
    // this lane's features f = 32db + 8r4 + 4hl + e
    float tp = 0.f, dp = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int f = 32 * db + 8 * r4 + 4 * hl;
        const f32x4 z4 = *(const f32x4 *)(Zs + f);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float av = fmaxf(float(R.qv[db][r4][e]), 0.f);
          tp = fmaf(av, gm[db][4 * r4 + e], tp);
          dp = fmaf(av, z4[e], dp);
        }
      }
    tp += __shfl_xor(tp, 32);
    dp += __shfl_xor(dp, 32);
    const float den = dp + g.eps;
    const float dden = -sb * tp / (den * den);
    const float inv_den = 1.f / den;
    if (outb) {
      typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
      float go_dot = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          go_dot = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{R.gf[ks][e], R.gf[ks][e + 1]},
                                                   bf16x2{of[ks][e], of[ks][e + 1]}, go_dot, false);
      go_dot += __shfl_xor(go_dot, 32);
      if (valid && hl == 0) dsum[(long long)bh * Np + n] = go_dot - sb * tp * inv_den;
    }
    const float a_scale = valid ? inv_den : 0.f;  // rows past the range add nothing
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int f = 32 * db + 8 * r4 + 4 * hl;
        bf16x4 ap;
#pragma unroll
        for (int e = 0; e < 4; ++e) ap[e] = (__bf16)(fmaxf(float(R.qv[db][r4][e]), 0.f) * a_scale);
        *(bf16x4 *)(At + rl * D + (((f >> 3) ^ kv_swz(rl)) << 3) + (f & 4)) = ap;
      }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      *(bf16x8 *)(Gt + rl * D + (((2 * ks + hl) ^ kv_swz(rl)) << 3)) = R.gf[ks];
    if (hl == 0) wrow[rl] = valid ? dden * den : 0.f;
    __syncthreads();
    // A[i][j] += sum_rows (a/den)[row][i] g[row][j]
#pragma unroll
    for (int ks = 0; ks < TT / 16; ++ks) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        const s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(At + 16 * ks * D + toff[0][bi][0]));
        const s16x4 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(At + 16 * ks * D + toff[0][bi][1]));
        const s16x4 q0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(Gt + 16 * ks * D + toff[1][bi][0]));
        const s16x4 q1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(Gt + 16 * ks * D + toff[1][bi][1]));
        typedef __attribute__((ext_vector_type(8))) short s16x8;
        const s16x8 a8 = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
        const s16x8 b8 = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
        av[bi] = *(const bf16x8 *)&a8;
        bv[bi] = *(const bf16x8 *)&b8;
      }
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = mfma_32x32x16(av[bi], bv[bj], acc[bi][bj]);
    }
    // Bz[f] += sum_rows (a/den)[row][f] * (dden den)[row]  (= dden a):
    // thread t takes features 4(t%32) .. +3 (one 8-byte read a row) over
    // the 16 rows of group t/32
    {
      const int f = 4 * (t & 31), r0 = (t >> 5) * 16;
#pragma unroll 4
      for (int rr = 0; rr < 16; ++rr) {
        const int row = r0 + rr;
        const bf16x4 a4 = *(const bf16x4 *)(At + row * D + (((f >> 3) ^ kv_swz(row)) << 3) + (f & 4));
        const float wv = wrow[row];
#pragma unroll
        for (int e = 0; e < 4; ++e) bz[e] = fmaf(float(a4[e]), wv, bz[e]);
      }
    }
    __syncthreads();  // At, Gt, wrow are refilled next step
  };
  // two named register sets, alternating: step on one while the other loads
  Rows R0, R1;
  if (n0 < n1) load_rows(n0, R0);
  for (int base = n0; base < n1; base += 2 * TT) {
    if (base + TT < n1) load_rows(base + TT, R1);
    step(base, R0);
    if (base + TT >= n1) break;
    if (base + 2 * TT < n1) load_rows(base + 2 * TT, R0);
    step(base + TT, R1);
  }

  float *out = partial + ((long long)bh * S + s) * (D * D + D);
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + 32 * bi + 8 * (r >> 2) + 4 * hl + (r & 3);
        const int j = j0 + 32 * bj + l32;
        out[i * D + j] = acc[bi][bj][r];
      }
  // the 8 row groups' partial sums, added in group order
  float *bzs = (float *)At;  // [8][128], At is free after the last step
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 4; ++e) bzs[(t >> 5) * D + 4 * (t & 31) + e] = bz[e];
  __syncthreads();
  if (t < D) {
    float acc_z = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc_z += bzs[i * D + t];
    out[D * D + t] = acc_z;
  }
}

// Per head, from the reduced A (fp32 [128][128]) and Bz: dH = s A W_p^T as
// bf16 row-major and transposed, the head's s H^T A (fp32) and 16 partial
// sums of <M, A>.  Grid (16, B*H); block blk owns rows 8blk..+7 of dH and of
// s H^T A; thread t: row t/32, columns (t%32) + 32m.
__global__ void __launch_bounds__(256) lin_bwd_head_kernel(Geom g, const float *__restrict__ a_red,
                                                           const float *__restrict__ hm,
                                                           const float *__restrict__ mf,
                                                           const bf16_t *__restrict__ w_p,
                                                           const float *__restrict__ s_gate,
                                                           bf16_t *__restrict__ dhb, bf16_t *__restrict__ dhtb,
                                                           float *__restrict__ dwp_h, float *__restrict__ ds_part) {
  __shared__ bf16_t wt[D * D];  // W_p^T: wt[k][j] = W_p[j][k]
  __shared__ float Hc[D * 8];   // H[k][8blk + c]
  __shared__ float red[256];
  const int blk = blockIdx.x, bh = blockIdx.y, b = bh / g.H, t = threadIdx.x;
  const int ii = t >> 5, jg = t & 31, i = 8 * blk + ii;
  const long long hbase = (long long)bh * D * D;
  if (dropped(g, s_gate, b)) {
    // no gradient through this sample's linear branch
#pragma unroll
    for (int m = 0; m < 4; ++m) dwp_h[hbase + (long long)i * D + jg + 32 * m] = 0.f;
    if (t == 0) ds_part[bh * 16 + blk] = 0.f;
    return;
  }
  for (int e = t; e < D * D; e += 256) {
    const int j = e >> 7, k = e & (D - 1);
    wt[k * D + j] = w_p[e];  // W_p[j][k] -> WpT[k][j]
  }
  for (int e = t; e < D * 8; e += 256) {
    const int k = e >> 3, c = e & 7;
    Hc[e] = hm[hbase + (long long)k * D + 8 * blk + c];
  }
  __syncthreads();
  const float sb = s_gate[b];
  const float *arow = a_red + hbase + (long long)i * D;
  float dh[4] = {0.f, 0.f, 0.f, 0.f}, dw[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k = 0; k < D; ++k) {
    const float av = arow[k];
    const float hv = Hc[k * 8 + ii];
    const float *ak = a_red + hbase + (long long)k * D;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int j = jg + 32 * m;
      dh[m] = fmaf(av, bf16_to_f32(wt[k * D + j]), dh[m]);
      dw[m] = fmaf(hv, ak[j], dw[m]);
    }
  }
  float dsp = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int j = jg + 32 * m;
    const float v = sb * dh[m];
    dhb[hbase + (long long)i * D + j] = f32_to_bf16(v);
    dhtb[hbase + (long long)j * D + i] = f32_to_bf16(v);
    dwp_h[hbase + (long long)i * D + j] = sb * dw[m];
    dsp = fmaf(mf[hbase + (long long)i * D + j], arow[j], dsp);
  }
  red[t] = dsp;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (t < st) red[t] += red[t + st];
    __syncthreads();
  }
  if (t == 0) ds_part[bh * 16 + blk] = red[0];
}

// dW_p = sum over (b, h) of the heads' s H^T A, in head order.
__global__ void __launch_bounds__(256) lin_bwd_wp_kernel(int BH, const float *__restrict__ dwp_h,
                                                         float *__restrict__ dw_p) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D * D) return;
  float acc = 0.f;
  for (int i = 0; i < BH; ++i) acc += dwp_h[(long long)i * D * D + e];
  dw_p[e] = acc;
}

hipError_t launch_linear_bwd(const Geom &g, const bf16_t *q, const bf16_t *go, const bf16_t *qd,
                             const bf16_t *god, const uint64_t work[4], const float *hm,
                             const float *zv, const bf16_t *w_p, const float *s_gate,
                             const LinBwdScratch &w, float *dw_p, View outv, float *dsum, int Np,
                             hipStream_t st) {
  if (g.D != D) return hipErrorInvalidValue;
  const int BH = g.B * g.H;
  // one workgroup per CU (LDS-bound) and one round of them: at most 256
  // workgroups, each over a longer row range (S never exceeds the split
  // count the partial-sum workspace is sized for)
  const int chunks = (g.N + 127) / 128;
  int S = 256 / BH;
  S = S < 1 ? 1 : (S > chunks ? chunks : S);
  if (S > linear_splits(g)) S = linear_splits(g);
  int chunk = (g.N + S - 1) / S;
  chunk = (chunk + 127) / 128 * 128;
  S = (g.N + chunk - 1) / chunk;
  lin_bwd_prep_kernel<<<dim3(16, BH), 256, 0, st>>>(g, hm, w_p, s_gate, w.mf, w.mb);
  HeadSet hs;
  for (int i = 0; i < 4; ++i) hs.w[i] = work[i];
  lin_bwd_rows_kernel<<<dim3(S, BH), 256, 0, st>>>(g, q, go, qd, god, hs, w.mb, zv, s_gate, w.partial, S, chunk,
                                                    outv, dsum, Np);
  hipError_t e = launch_linear_reduce(g, S, w.partial, w.a_red, w.bz, st);
  if (e != hipSuccess) return e;
  lin_bwd_head_kernel<<<dim3(16, BH), 256, 0, st>>>(g, w.a_red, hm, w.mf, w_p, s_gate, w.dhb, w.dhtb,
                                                    w.dwp_h, w.ds_part);
  lin_bwd_wp_kernel<<<(D * D + 255) / 256, 256, 0, st>>>(BH, w.dwp_h, dw_p);
  return hipGetLastError();
}

}  // namespace salad
