// Linear-attention branch: state H = relu(K)^T V, Z = relu(K)^T 1 and
// output O_l = relu(Q) H / (relu(Q) Z + eps).
//
// Source: SALAD structured summary (paper.rainbus.top/paper/2601.16515),
// Prerequisites > Linear Attention (kernel phi = ReLU, O(N d^2) cost) and
// method step 3 (the branch runs on the same Q, K, V as the sparse one).
//
// bf16 path (d = 128), on MFMA v_mfma_f32_32x32x16_bf16:
//   state: the contraction runs over tokens, the slow index of K and V;
//   64-token tiles sit in LDS row-major and transposing LDS reads
//   (ds_read_b64_tr_b16) deliver 4 consecutive tokens of a feature per
//   lane; the 4 waves each accumulate a 64x64 quadrant of H; the N tokens
//   are split over workgroups and the partial states are summed in a fixed
//   order by a second kernel (deterministic, no atomics).
//   apply: H is split into bf16 hi + lo halves (about 16 significant bits)
//   so the output keeps near-fp32 accuracy; relu(q) is exact in bf16.
// f32 path (d = 64 or 128): plain VALU loops.
#include "common.h"
#include "kernels.h"

namespace salad {

// MFMA operand layout (32x32x16 bf16): lane l supplies A[m = l%32][k = 8*(l/32) + e]
// and B[k = 8*(l/32) + e][n = l%32]; the 16 results of lane l are
// C[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32], r = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__global__ void linear_reduce_kernel(int D, int S, const float *__restrict__ partial,
                                     float *__restrict__ h, float *__restrict__ z);

__device__ __forceinline__ u32x4 relu_bf16x8(u32x4 v) {
  // clear each 16-bit half whose sign bit is set
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w = v[i];
    uint32_t lo = (w & 0x8000u) ? 0u : (w & 0xffffu);
    uint32_t hi = (w & 0x80000000u) ? 0u : (w & 0xffff0000u);
    v[i] = lo | hi;
  }
  return v;
}

// ---------------------------------------------------------------------------
// State, bf16, d = 128.  Grid (S, B*H); 256 threads; split s covers working
// rows [s*chunk, (s+1)*chunk).  Tiles of 64 tokens: thread t loads 16-byte
// chunk c = t%16 of rows t/16 + 16i (i < 4) of K and V -- each load
// instruction covers four whole 256-byte rows -- and, when kw_out / vw_out
// are given and the head is flagged in `copy`, stores them to those
// working-layout copies (the pass that already reads K and V produces the
// contiguous per-head copies the attention kernel streams for heads whose
// working order differs from the token order).  relu(K) and V go to LDS row-major; unit u of
// row j sits at u ^ lin_swz(j).  The MFMA operands, which need 4 consecutive
// tokens of one feature per lane, come from ds_read_b64_tr_b16: each 16-lane
// group reads 4 rows x 64 bytes, which lin_swz spreads over distinct banks.
// Wave w accumulates the 64x64 quadrant (i0, j0) = (64*(w/2), 64*(w%2)) of H.
// The loads of the tile after next are issued before the current tile's MFMAs
// (two tiles of rows in flight per thread).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lin_swz(int j) { return ((j & 3) << 2) | ((j >> 2) & 3); }

typedef __attribute__((ext_vector_type(4))) short s16x4_l;
typedef __attribute__((address_space(3))) s16x4_l lds_s16x4_l;

struct HeadMask {
  uint64_t w[4];
};

__global__ void __launch_bounds__(256, 2) linear_state_bf16_kernel(Geom g, View kv, View vv,
                                                                float *__restrict__ partial,
                                                                int S, int chunk,
                                                                bf16_t *__restrict__ kw_out,
                                                                bf16_t *__restrict__ vw_out,
                                                                HeadMask copy,
                                                                const float *__restrict__ s_gate) {
  constexpr int D = 128, TT = 64;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[TT * D];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[TT * D];
  const int s = blockIdx.x, bh = blockIdx.y, h = bh % g.H, b = bh / g.H;
  const int n0 = s * chunk, n1 = min(g.N, n0 + chunk);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int c = t & 15, rg = t >> 4;
  const bf16_t *kb = (const bf16_t *)kv.base;
  const bf16_t *vb = (const bf16_t *)vv.base;
  const long long wbase = (long long)bh * g.N * D;  // working-layout copy of this (b, h)
  if (!bit(copy.w, h)) kw_out = vw_out = nullptr;
  // Branch dropping: a dropped sample needs no linear state, only the
  // working copies of its temporal heads (the sparse branch reads them).
  if (s_gate && s_gate[b] < g.drop_tau) {
    if (!kw_out && !vw_out) return;
    for (int base = n0; base < n1; base += TT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = base + rg + 16 * i;
        if (n >= n1) continue;
        const long long w_at = wbase + (long long)n * D + c * 8;
        if (kw_out) *(u32x4 *)(kw_out + w_at) = *(const u32x4 *)(kb + row_offset(g, kv, b, h, n) + c * 8);
        if (vw_out) *(u32x4 *)(vw_out + w_at) = *(const u32x4 *)(vb + row_offset(g, vv, b, h, n) + c * 8);
      }
    }
    return;
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const int i0 = (w >> 1) * 64, j0 = (w & 1) * 64;
  const int hl = lane >> 5, gq = lane >> 4, jl = lane & 15;
  // lane-constant part of the transposing reads: row 8hl + 4r + jl/4,
  // feature f0 + 4*(jl%4) with f0 = base + 16*(gq%2)
  int toff[2][2][2];  // [operand A/B][block][r]
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int op = 0; op < 2; ++op) {
        const int row = 8 * hl + 4 * r + (jl >> 2);
        const int f = (op ? j0 : i0) + 32 * bi + 16 * (gq & 1) + 4 * (jl & 3);
        toff[op][bi][r] = row * D + (((f >> 3) ^ lin_swz(row)) << 3) + (f & 4);
      }

  // Two tiles of K and V rows in flight: the loads of tile i+2 are issued
  // while tile i's MFMAs run, with tile i+1 already in registers, so each
  // load has two tiles of work to land in.
  u32x4 kr0[4], vr0[4], kr1[4], vr1[4];
  auto load = [&](int base, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = base + rg + 16 * i;
      if (n < n1) {
        kr[i] = *(const u32x4 *)(kb + row_offset(g, kv, b, h, n) + c * 8);
        vr[i] = *(const u32x4 *)(vb + row_offset(g, vv, b, h, n) + c * 8);
      } else {
        kr[i] = u32x4{0, 0, 0, 0};
        vr[i] = u32x4{0, 0, 0, 0};
      }
    }
  };
  // working copies, relu(K), Z and the LDS tiles of the rows in kr / vr
  auto stage = [&](int base, const u32x4 (&kr)[4], const u32x4 (&vr)[4]) {
    __syncthreads();  // previous tile's operand reads are done
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rg + 16 * i, n = base + row;
      if (n < n1) {
        if (kw_out) *(u32x4 *)(kw_out + wbase + (long long)n * D + c * 8) = kr[i];
        if (vw_out) *(u32x4 *)(vw_out + wbase + (long long)n * D + c * 8) = vr[i];
      }
      const u32x4 rk = relu_bf16x8(kr[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        z[e] += bf16_to_f32(bf16_t((rk[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
      const int unit = c ^ lin_swz(row);
      *(u32x4 *)(Ks + row * D + unit * 8) = rk;
      *(u32x4 *)(Vs + row * D + unit * 8) = vr[i];
    }
    __syncthreads();
  };
  auto mma = [&]() {
#pragma unroll
    for (int ks = 0; ks < TT / 16; ++ks) {
      bf16x8 a[2], bb[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        const s16x4_l p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_l *)(Ks + 16 * ks * D + toff[0][bi][0]));
        const s16x4_l p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_l *)(Ks + 16 * ks * D + toff[0][bi][1]));
        const s16x4_l q0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_l *)(Vs + 16 * ks * D + toff[1][bi][0]));
        const s16x4_l q1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_l *)(Vs + 16 * ks * D + toff[1][bi][1]));
        typedef __attribute__((ext_vector_type(8))) short s16x8_l;
        s16x8_l av = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
        s16x8_l bv = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
        a[bi] = *(const bf16x8 *)&av;
        bb[bi] = *(const bf16x8 *)&bv;
      }
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = mfma32(a[bi], bb[bj], acc[bi][bj]);
    }
  };
  if (n0 < n1) load(n0, kr0, vr0);
  if (n0 + TT < n1) load(n0 + TT, kr1, vr1);
  for (int base = n0; base < n1; base += 2 * TT) {
    stage(base, kr0, vr0);
    if (base + 2 * TT < n1) load(base + 2 * TT, kr0, vr0);
    mma();
    if (base + TT >= n1) break;
    stage(base + TT, kr1, vr1);
    if (base + 3 * TT < n1) load(base + 3 * TT, kr1, vr1);
    mma();
  }

  float *out = partial + ((long long)bh * S + s) * (D * D + D);
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + 32 * bi + 8 * (r >> 2) + 4 * hl + (r & 3);
        const int j = j0 + 32 * bj + (lane & 31);
        out[i * D + j] = acc[bi][bj][r];
      }
  // Z: reduce the 16 row groups in a fixed order
  __syncthreads();
  float *zs = (float *)Ks;  // [16][128]
#pragma unroll
  for (int e = 0; e < 8; ++e) zs[rg * D + c * 8 + e] = z[e];
  __syncthreads();
  if (t < D) {
    float acc_z = 0.f;
    for (int i = 0; i < 16; ++i) acc_z += zs[i * D + t];
    out[D * D + t] = acc_z;
  }
}

// ---------------------------------------------------------------------------
// State, f32, d = 64 or 128.  Grid (S, B*H); 256 threads; thread t owns a
// TI x TI tile of H (TI = d/16) at rows TI*(t/16), columns TI*(t%16).
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) linear_state_f32_kernel(Geom g, View kv, View vv,
                                                               float *__restrict__ partial,
                                                               int S, int chunk) {
  constexpr int TT = 32, TI = D / 16;
  __shared__ float Ks[TT][D];
  __shared__ float Vs[TT][D];
  const int s = blockIdx.x, bh = blockIdx.y, h = bh % g.H, b = bh / g.H;
  const int n0 = s * chunk, n1 = min(g.N, n0 + chunk);
  const int t = threadIdx.x, ig = t >> 4, jg = t & 15;
  const float *kb = (const float *)kv.base;
  const float *vb = (const float *)vv.base;
  float acc[TI][TI];
  for (int a = 0; a < TI; ++a)
    for (int c = 0; c < TI; ++c) acc[a][c] = 0.f;
  float zacc = 0.f;
  for (int base = n0; base < n1; base += TT) {
    __syncthreads();
    for (int e = t; e < TT * D; e += 256) {
      const int r = e / D, col = e % D, n = base + r;
      float kval = 0.f, vval = 0.f;
      if (n < n1) {
        kval = fmaxf(kb[row_offset(g, kv, b, h, n) + col], 0.f);
        vval = vb[row_offset(g, vv, b, h, n) + col];
      }
      Ks[r][col] = kval;
      Vs[r][col] = vval;
    }
    __syncthreads();
    for (int r = 0; r < TT; ++r) {
      float kk[TI], vvv[TI];
      for (int a = 0; a < TI; ++a) kk[a] = Ks[r][ig * TI + a];
      for (int c = 0; c < TI; ++c) vvv[c] = Vs[r][jg * TI + c];
      for (int a = 0; a < TI; ++a)
        for (int c = 0; c < TI; ++c) acc[a][c] = fmaf(kk[a], vvv[c], acc[a][c]);
      if (t < D) zacc += Ks[r][t];
    }
  }
  float *out = partial + ((long long)bh * S + s) * (D * D + D);
  for (int a = 0; a < TI; ++a)
    for (int c = 0; c < TI; ++c) out[(ig * TI + a) * D + jg * TI + c] = acc[a][c];
  if (t < D) out[D * D + t] = zacc;
}

// Fixed-order sum of the S partial states: h[bh] = sum_s partial[bh][s].
__global__ void linear_reduce_kernel(int D, int S, const float *__restrict__ partial,
                                     float *__restrict__ h, float *__restrict__ z) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int per = D * D + D;
  if (e >= per) return;
  const float *p = partial + (long long)bh * S * per + e;
  float acc = 0.f;
#pragma unroll 8
  for (int s = 0; s < S; ++s) acc += p[(long long)s * per];
  if (e < D * D)
    h[(long long)bh * D * D + e] = acc;
  else
    z[(long long)bh * D + (e - D * D)] = acc;
}

// ---------------------------------------------------------------------------
// Finalize, d = 128 (fused layer): sum the split-N partial states of 8 rows
// of H (and 8 of Z) in a fixed order, keep them in LDS and fold the
// projection and the gate in: Hp[j][i] = bf16(s_b * (H W_p)[i][j]).
// Samples dropped by the branch threshold (s_b < drop_tau) are skipped.
// Grid (16, B*H), 1024 threads; block blk owns rows 8*blk..+7.  The kernel
// is bound by the latency of its loads, so the splits are spread over four
// thread groups: thread 256q + u sums the 16-byte unit u of the block's
// 1024 H elements (and, for u < 2, of its 8 Z elements) over the splits
// q, q+4, q+8, ... in order, and the four group sums are added in the order
// q = 0..3 through LDS.
// W_p is staged once per block as bf16 (16-byte loads); thread t < 256 then
// computes row t/32 at columns (t%32) + 32m, m < 4.  H and Z are also
// written out in fp32.
// FULL (full-width [C, C] projection, applied after the attention kernel
// by a GEMM over whole token rows): Hp = bf16(H^T), no W_p and no gate.
// ---------------------------------------------------------------------------
template <typename T, bool FULL>
__global__ void __launch_bounds__(1024) linear_finalize_kernel(Geom g, int S,
                                                              const float *__restrict__ partial,
                                                              const T *__restrict__ w_p,
                                                              const float *__restrict__ s_gate,
                                                              float *__restrict__ hm,
                                                              float *__restrict__ zv,
                                                              bf16_t *__restrict__ hp) {
  constexpr int D = 128, per = D * D + D;
  __shared__ __attribute__((aligned(16))) T Ws[FULL ? 8 : D * D];
  __shared__ __attribute__((aligned(16))) float Hs[8 * D];
  __shared__ f32x4 red[4][258];
  const int blk = blockIdx.x, bh = blockIdx.y, b = bh / g.H, t = threadIdx.x;
  if (s_gate[b] < g.drop_tau) return;  // dropped sample: no linear branch (its state was skipped)
  // stage W_p (16-byte chunks)
  constexpr int VEC = 16 / sizeof(T);
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  if constexpr (!FULL)
    for (int e = t * VEC; e < D * D; e += 1024 * VEC)
      *(u32x4 *)(Ws + e) = *(const u32x4 *)(w_p + e);
  // this block's 1024 H elements and 8 Z elements over the splits: group q
  // takes splits q, q+4, ...; then the groups in order
  {
    const int q = t >> 8, u = t & 255;
    const float *p = partial + (long long)bh * S * per;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, accz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int s = q; s < S; s += 4) {
      acc += *(const f32x4 *)(p + (long long)s * per + 8 * blk * D + 4 * u);
      if (u < 2) accz += *(const f32x4 *)(p + (long long)s * per + D * D + 8 * blk + 4 * u);
    }
    red[q][u] = acc;
    if (u < 2) red[q][256 + u] = accz;
  }
  __syncthreads();
  if (t < 258) {
    const f32x4 v = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
    if (t < 256) {
      *(f32x4 *)(Hs + 4 * t) = v;
      *(f32x4 *)(hm + ((long long)bh * D + 8 * blk) * D + 4 * t) = v;
    } else {
      *(f32x4 *)(zv + (long long)bh * D + 8 * blk + 4 * (t - 256)) = v;
    }
  }
  __syncthreads();
  if (t >= 256) return;
  const int ii = t >> 5, jg = t & 31;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (FULL) {
#pragma unroll
    for (int m = 0; m < 4; ++m) o[m] = Hs[ii * D + jg + 32 * m];
  } else {
#pragma unroll 8
    for (int k = 0; k < D; ++k) {
      const float hv = Hs[ii * D + k];
#pragma unroll
      for (int m = 0; m < 4; ++m) o[m] = fmaf(hv, io<T>::ld(Ws + k * D + jg + 32 * m), o[m]);
    }
  }
  const float sb = FULL ? 1.f : s_gate[b];
  bf16_t *dst = hp + (long long)bh * D * D;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const __bf16 v = (__bf16)(sb * o[m]);
    dst[(jg + 32 * m) * D + 8 * blk + ii] = *(const bf16_t *)&v;
  }
}

hipError_t launch_linear_finalize(const Geom &g, int bf16, const float *partial, const void *w_p,
                                  const float *s, float *h, bf16_t *hp, float *z, hipStream_t st) {
  if (g.D != 128) return hipErrorInvalidValue;
  const int S = linear_splits(g);
  dim3 grid(16, g.B * g.H);
  if (!w_p)  // full-width projection: the GEMM after the attention kernel applies W_p and s
    linear_finalize_kernel<bf16_t, true><<<grid, 1024, 0, st>>>(g, S, partial, nullptr, s, h, z, hp);
  else if (bf16)
    linear_finalize_kernel<bf16_t, false><<<grid, 1024, 0, st>>>(g, S, partial, (const bf16_t *)w_p, s, h, z, hp);
  else
    linear_finalize_kernel<float, false><<<grid, 1024, 0, st>>>(g, S, partial, (const float *)w_p, s, h, z, hp);
  return hipGetLastError();
}

// Partial states only (the fused layer finalizes them itself), optionally
// writing working-layout copies of K and V.
hipError_t launch_linear_partials(const Geom &g, View kv, View vv, float *partial, bf16_t *kw_out,
                                  bf16_t *vw_out, const uint64_t copy_heads[4], const float *s_gate,
                                  hipStream_t st) {
  const int S = linear_splits(g);
  int chunk = (g.N + S - 1) / S;
  chunk = (chunk + 127) / 128 * 128;
  HeadMask m;
  for (int i = 0; i < 4; ++i) m.w[i] = copy_heads[i];
  linear_state_bf16_kernel<<<dim3(S, g.B * g.H), 256, 0, st>>>(g, kv, vv, partial, S, chunk, kw_out,
                                                              vw_out, m, s_gate);
  return hipGetLastError();
}

hipError_t launch_linear_reduce(const Geom &g, int S, const float *partial, float *h, float *z,
                                hipStream_t st) {
  dim3 grid((g.D * g.D + g.D + 255) / 256, g.B * g.H);
  linear_reduce_kernel<<<grid, 256, 0, st>>>(g.D, S, partial, h, z);
  return hipGetLastError();
}

hipError_t launch_linear_state(const Geom &g, int bf16, View kv, View vv, float *partial, float *h,
                               float *z, hipStream_t st) {
  const int S = linear_splits(g);
  int chunk = (g.N + S - 1) / S;
  chunk = (chunk + 127) / 128 * 128;
  dim3 grid(S, g.B * g.H);
  if (bf16) {
    linear_state_bf16_kernel<<<grid, 256, 0, st>>>(g, kv, vv, partial, S, chunk, nullptr, nullptr,
                                                   HeadMask{}, nullptr);
  } else if (g.D == 128) {
    linear_state_f32_kernel<128><<<grid, 256, 0, st>>>(g, kv, vv, partial, S, chunk);
  } else {
    linear_state_f32_kernel<64><<<grid, 256, 0, st>>>(g, kv, vv, partial, S, chunk);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid2((g.D * g.D + g.D + 255) / 256, g.B * g.H);
  linear_reduce_kernel<<<grid2, 256, 0, st>>>(g.D, S, partial, h, z);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Apply, bf16, d = 128.  Grid (up to 1024/(B*H) workgroups, B*H), each over
// 128-token tiles tile, tile + gridDim.x, ... (the staged H is reused, and
// the next tile's Q rows load during this tile's MFMAs); 4 waves x 32
// tokens per tile.
// LDS holds H^T as bf16 hi and lo halves, [d_out][d_in], unit u of row j
// at u ^ (j & 15).  Per wave: C[d_out][token] = sum_i H^T[d_out][i] relu(q)[i].
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) linear_apply_bf16_kernel(Geom g, View qv, const float *__restrict__ hm,
                                                                const float *__restrict__ zv,
                                                                float *__restrict__ o_l) {
  constexpr int D = 128;
  __shared__ __attribute__((aligned(16))) bf16_t Hhi[D * D];
  __shared__ __attribute__((aligned(16))) bf16_t Hlo[D * D];
  __shared__ float Zs[D];
  const int bh = blockIdx.y, h = bh % g.H, b = bh / g.H;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, hl = lane >> 5, l32 = lane & 31;
  const float *H = hm + (long long)bh * D * D;
  // stage H^T: thread handles column j = t % 128 and units u = t/128 + 2*m;
  // all 64 loads are issued before the first conversion, so the staging
  // pays one L2 round trip, not eight
  {
    const int j = t & 127;
    float hv[8][8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[m][e] = H[((2 * m + (t >> 7)) * 8 + e) * D + j];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int u = 2 * m + (t >> 7);
      uint16_t his[8], los[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bf16_t hi = f32_to_bf16(hv[m][e]);
        his[e] = hi;
        los[e] = f32_to_bf16(hv[m][e] - bf16_to_f32(hi));
      }
      const int pu = u ^ (j & 15);
      *(bf16x8 *)(Hhi + j * D + pu * 8) = *(const bf16x8 *)his;
      *(bf16x8 *)(Hlo + j * D + pu * 8) = *(const bf16x8 *)los;
    }
    if (t < D) Zs[t] = zv[(long long)bh * D + t];
  }
  __syncthreads();
  // the staged H serves several 128-token tiles (tile, tile + gridDim.x, ...);
  // the next tile's Q rows are loaded before this tile's MFMAs
  const int n_tiles = (g.N + 127) / 128;
  const bf16_t *qb = (const bf16_t *)qv.base;
  u32x4 qn[8];
  auto load_q = [&](int tile) {
    const int p = tile * 128 + w * 32 + l32;
    const long long qoff = row_offset(g, qv, b, h, p < g.N ? p : g.N - 1);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qn[ks] = *(const u32x4 *)(qb + qoff + (2 * ks + hl) * 8);
  };
  if (int(blockIdx.x) < n_tiles) load_q(blockIdx.x);
  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int p = tile * 128 + w * 32 + l32;
    const bool valid = p < g.N;
    bf16x8 q[8];
    float den = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 raw = relu_bf16x8(qn[ks]);
      q[ks] = *(bf16x8 *)&raw;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t bits = (raw[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
        den = fmaf(bf16_to_f32(bf16_t(bits)), Zs[16 * ks + 8 * hl + e], den);
      }
    }
    if (tile + int(gridDim.x) < n_tiles) load_q(tile + gridDim.x);
    // add the other half-wave's partial denominator (lanes l and l^32)
    den += __shfl_xor(den, 32);
    den += g.eps;
    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int j = 32 * db + l32;
        const int pu = (2 * ks + hl) ^ (j & 15);
        const bf16x8 ahi = *(const bf16x8 *)(Hhi + j * D + pu * 8);
        const bf16x8 alo = *(const bf16x8 *)(Hlo + j * D + pu * 8);
        o[db] = mfma32(ahi, q[ks], o[db]);
        o[db] = mfma32(alo, q[ks], o[db]);
      }
    if (valid) {
      float *dst = o_l + (((long long)bh * g.N) + p) * D;
      const float inv = 1.0f / den;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 v = {o[db][4 * r4] * inv, o[db][4 * r4 + 1] * inv, o[db][4 * r4 + 2] * inv,
                     o[db][4 * r4 + 3] * inv};
          *(f32x4 *)(dst + 32 * db + 8 * r4 + 4 * hl) = v;
        }
    }
  }
}

// Apply, f32.  Grid (ceil(N/64), B*H); thread t: token t/4, columns 32*(t%4)..+31
// (d = 128) or 16*(t%4)..+15 (d = 64).  H staged in LDS (dynamic).
template <int D>
__global__ void __launch_bounds__(256) linear_apply_f32_kernel(Geom g, View qv, const float *__restrict__ hm,
                                                               const float *__restrict__ zv,
                                                               float *__restrict__ o_l) {
  extern __shared__ float Hs[];  // [D][D]
  constexpr int NC = D / 4;
  const int bh = blockIdx.y, h = bh % g.H, b = bh / g.H;
  const int t = threadIdx.x;
  for (int e = t; e < D * D; e += 256) Hs[e] = hm[(long long)bh * D * D + e];
  __syncthreads();
  const int p = blockIdx.x * 64 + (t >> 2), jc = (t & 3) * NC;
  if (p >= g.N) return;
  const float *q = (const float *)qv.base + row_offset(g, qv, b, h, p);
  const float *Z = zv + (long long)bh * D;
  float acc[NC];
  for (int j = 0; j < NC; ++j) acc[j] = 0.f;
  float den = 0.f;
  for (int i = 0; i < D; ++i) {
    const float qi = fmaxf(q[i], 0.f);
    den = fmaf(qi, Z[i], den);
    for (int j = 0; j < NC; ++j) acc[j] = fmaf(qi, Hs[i * D + jc + j], acc[j]);
  }
  den += g.eps;
  float *dst = o_l + ((long long)bh * g.N + p) * D + jc;
  for (int j = 0; j < NC; ++j) dst[j] = acc[j] / den;
}

hipError_t launch_linear_apply(const Geom &g, int bf16, View qv, const float *h, const float *z,
                               float *o_l, hipStream_t st) {
  if (bf16) {
    // about two rounds of workgroups (two per CU), each over several tiles
    const int tiles = (g.N + 127) / 128, per_head = 1024 / (g.B * g.H);
    dim3 grid(per_head < 1 ? 1 : (per_head < tiles ? per_head : tiles), g.B * g.H);
    linear_apply_bf16_kernel<<<grid, 256, 0, st>>>(g, qv, h, z, o_l);
  } else {
    dim3 grid((g.N + 63) / 64, g.B * g.H);
    const size_t lds = size_t(g.D) * g.D * sizeof(float);
    if (g.D == 128) {
      hipFuncSetAttribute((const void *)linear_apply_f32_kernel<128>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
      linear_apply_f32_kernel<128><<<grid, 256, lds, st>>>(g, qv, h, z, o_l);
    } else {
      linear_apply_f32_kernel<64><<<grid, 256, lds, st>>>(g, qv, h, z, o_l);
    }
  }
  return hipGetLastError();
}

}  // namespace salad
