// Linear-attention branch: state H = relu(K)^T V, Z = relu(K)^T 1 and
// output O_l = relu(Q) H / (relu(Q) Z + eps).
//
// Source: SALAD structured summary (paper.rainbus.top/paper/2601.16515),
// Prerequisites > Linear Attention (kernel phi = ReLU, O(N d^2) cost) and
// method step 3 (the branch runs on the same Q, K, V as the sparse one).
//
// bf16 path (d = 128), on MFMA v_mfma_f32_32x32x16_bf16:
//   state: the contraction runs over tokens, the slow index of K and V, so
//   each 128-token tile is written to LDS transposed ([d][token], XOR
//   swizzled) and the 4 waves each accumulate a 64x64 quadrant of H; the N
//   tokens are split over workgroups and the partial states are summed in a
//   fixed order by a second kernel (deterministic, no atomics).
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
// State, bf16, d = 128.  Grid (S, B*H); 256 threads.
// Tile: 128 tokens.  Load mapping: thread t reads 16-byte chunk c = t%16 of
// rows 8*(t/16) .. +7, so each load instruction covers 4 full 256-byte rows.
// LDS layout of Kt/Vt: row = feature (128), 16 units of 8 tokens; unit u of
// row rho is stored at u ^ swz(rho), swz(rho) = (rho ^ (rho >> 3)) & 15,
// which keeps both the transposed stores (rows 8 apart) and the MFMA operand
// reads (16 consecutive rows) on distinct 16-byte bank groups.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int kt_swz(int rho) { return (rho ^ (rho >> 3)) & 15; }

__global__ void __launch_bounds__(256) linear_state_bf16_kernel(Geom g, View kv, View vv,
                                                                float *__restrict__ partial,
                                                                int S, int chunk) {
  constexpr int D = 128, TT = 128;
  __shared__ __attribute__((aligned(16))) bf16_t Kt[D * TT];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[D * TT];
  const int s = blockIdx.x, bh = blockIdx.y, h = bh % g.H, b = bh / g.H;
  const int n0 = s * chunk, n1 = min(g.N, n0 + chunk);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int c = t & 15, rg = t >> 4;
  const bf16_t *kb = (const bf16_t *)kv.base;
  const bf16_t *vb = (const bf16_t *)vv.base;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const int i0 = (w >> 1) * 64, j0 = (w & 1) * 64;
  const int hl = lane >> 5, l32 = lane & 31;

  for (int base = n0; base < n1; base += TT) {
    u32x4 kr[8], vr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = base + rg * 8 + i;
      if (n < n1) {
        kr[i] = relu_bf16x8(*(const u32x4 *)(kb + row_offset(g, kv, b, h, n) + c * 8));
        vr[i] = *(const u32x4 *)(vb + row_offset(g, vv, b, h, n) + c * 8);
      } else {
        kr[i] = u32x4{0, 0, 0, 0};
        vr[i] = u32x4{0, 0, 0, 0};
      }
    }
    __syncthreads();  // previous tile's operand reads are done
    // transpose 8 rows x 8 features into 8 rows of Kt/Vt (one 16-byte unit each)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int rho = c * 8 + e;
      const int sh = (e & 1) * 16, word = e >> 1;
      u32x4 ko, vo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t k_lo = (kr[2 * i][word] >> sh) & 0xffffu, k_hi = (kr[2 * i + 1][word] >> sh) & 0xffffu;
        uint32_t v_lo = (vr[2 * i][word] >> sh) & 0xffffu, v_hi = (vr[2 * i + 1][word] >> sh) & 0xffffu;
        ko[i] = k_lo | (k_hi << 16);
        vo[i] = v_lo | (v_hi << 16);
        z[e] += bf16_to_f32(bf16_t(k_lo)) + bf16_to_f32(bf16_t(k_hi));
      }
      const int unit = rg ^ kt_swz(rho);
      *(u32x4 *)(Kt + rho * TT + unit * 8) = ko;
      *(u32x4 *)(Vt + rho * TT + unit * 8) = vo;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < TT / 16; ++ks) {
      bf16x8 a[2], bb[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        const int rho = i0 + 32 * bi + l32;
        a[bi] = *(const bf16x8 *)(Kt + rho * TT + ((2 * ks + hl) ^ kt_swz(rho)) * 8);
      }
#pragma unroll
      for (int bj = 0; bj < 2; ++bj) {
        const int rho = j0 + 32 * bj + l32;
        bb[bj] = *(const bf16x8 *)(Vt + rho * TT + ((2 * ks + hl) ^ kt_swz(rho)) * 8);
      }
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = mfma32(a[bi], bb[bj], acc[bi][bj]);
    }
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
  // Z: reduce the 16 row groups in a fixed order
  __syncthreads();
  float *zs = (float *)Kt;  // [16][128]
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
__global__ void __launch_bounds__(256) linear_reduce_kernel(int D, int S, const float *__restrict__ partial,
                                                            float *__restrict__ h, float *__restrict__ z) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int per = D * D + D;
  if (e >= per) return;
  const float *p = partial + (long long)bh * S * per + e;
  float acc = 0.f;
  for (int s = 0; s < S; ++s) acc += p[(long long)s * per];
  if (e < D * D)
    h[(long long)bh * D * D + e] = acc;
  else
    z[(long long)bh * D + (e - D * D)] = acc;
}

hipError_t launch_linear_state(const Geom &g, int bf16, View kv, View vv, float *partial, float *h,
                               float *z, hipStream_t st) {
  const int S = linear_splits(g);
  int chunk = (g.N + S - 1) / S;
  chunk = (chunk + 127) / 128 * 128;
  dim3 grid(S, g.B * g.H);
  if (bf16) {
    linear_state_bf16_kernel<<<grid, 256, 0, st>>>(g, kv, vv, partial, S, chunk);
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
// Apply, bf16, d = 128.  Grid (ceil(N/128), B*H); 4 waves x 32 tokens.
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
  // stage H^T: thread handles column j = t % 128 and units u = t/128 + 2*m
  {
    const int j = t & 127;
    for (int u = t >> 7; u < 16; u += 2) {
      bf16x8 hi8, lo8;
      uint16_t his[8], los[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = H[(u * 8 + e) * D + j];
        const bf16_t hi = f32_to_bf16(v);
        his[e] = hi;
        los[e] = f32_to_bf16(v - bf16_to_f32(hi));
      }
      hi8 = *(const bf16x8 *)his;
      lo8 = *(const bf16x8 *)los;
      const int pu = u ^ (j & 15);
      *(bf16x8 *)(Hhi + j * D + pu * 8) = hi8;
      *(bf16x8 *)(Hlo + j * D + pu * 8) = lo8;
    }
    if (t < D) Zs[t] = zv[(long long)bh * D + t];
  }
  __syncthreads();
  const int p = blockIdx.x * 128 + w * 32 + l32;
  const bool valid = p < g.N;
  const bf16_t *qb = (const bf16_t *)qv.base;
  const long long qoff = row_offset(g, qv, b, h, valid ? p : g.N - 1);
  bf16x8 q[8];
  float den = 0.f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x4 raw = relu_bf16x8(*(const u32x4 *)(qb + qoff + (2 * ks + hl) * 8));
    q[ks] = *(bf16x8 *)&raw;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t bits = (raw[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
      den = fmaf(bf16_to_f32(bf16_t(bits)), Zs[16 * ks + 8 * hl + e], den);
    }
  }
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
  if (!valid) return;
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
    dim3 grid((g.N + 127) / 128, g.B * g.H);
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
