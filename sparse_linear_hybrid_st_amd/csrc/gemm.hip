// Dense projections over whole token rows: the full-width [C, C] reading of
// the static projection W_p and the output projection W^O.
//
// Sources: SALAD structured summary (paper.rainbus.top/paper/2601.16515),
// method steps 4 (projection of the linear branch's output) and 7 (output
// projection).
//
// out[m, :] (+)= a[m, :] W for m < rows: a [rows, C], W [C, C], out [rows, C],
// all row-major; C a multiple of 128 for bf16 (head_dim 128), of 64 for f32.
//
// bf16: a hand-written MFMA GEMM on v_mfma_f32_32x32x16_bf16, fp32
// accumulation.  A workgroup of eight waves owns a 256 x 256 tile of out
// (the large tile keeps the L2 -> LDS traffic at 64 KB per 2 x 256 x 256 x 64
// flops) and walks K in stages of 64 through two LDS buffers (128 KB)
// filled by DMA (buffer_load ... lds) one stage ahead.  It computes the
// transposed tile out^T = W^T a^T: W's stage [64 k][256 n] is read
// transposed (ds_read_b64_tr_b16) as the MFMA A operand and a's stage
// [256 m][64 k] row-major as the B operand, so each lane ends with 4
// consecutive output columns of one row per register group and stores 8
// bytes at a time.  Wave w owns rows 64*(w%4) .. +63 and columns
// 128*(w/4) .. +127: 2 x 4 blocks of 32 x 32 (128 accumulators, two waves
// per SIMD).  (Four waves of 128 x 128, or stages of 32 in a ring of four,
// measured slower on the 480p projection.)
// f32 (the small fp32 workloads): an LDS-tiled fp32 loop.
#include <stdint.h>

#include "common.h"
#include "kernels.h"
#include "mfma_util.h"

namespace salad {

namespace {

constexpr int kGM = 256;  // rows of out per workgroup
constexpr int kGN = 256;  // columns of out per workgroup

// s_waitcnt immediate for "vmcnt <= n" (n < 64) with no wait on lgkmcnt or
// expcnt: vmcnt's low four bits sit in [3:0], its high two in [15:14].
constexpr int vmcnt_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// NWV waves (4: 2 x 2 waves of 128 x 128; 8: 4 x 2 waves of 64 x 128), K
// stages of KGK (32 or 64) in a ring of NST LDS buffers (2 or 4; 128 KB
// either way), filled NST - 1 stages ahead.
//
// a's stage [256 m][KGK k] bf16: rows of UA = KGK/8 16-byte units; unit u of
// row r sits at u ^ a_swz(r), a_swz(r) = (r / (16/UA)) mod UA, which puts
// the 16 rows a quarter-wave reads (one unit each) on 16 distinct 16-byte
// bank groups.
template <int NWV, int KGK, int NST>
__global__ void __launch_bounds__(64 * NWV, 1) gemm_bf16_kernel(const bf16_t *__restrict__ a,
                                                                   const bf16_t *__restrict__ w,
                                                                   bf16_t *__restrict__ out, int rows, int C,
                                                                   int accumulate, int n_tiles_n, int n_blocks) {
  constexpr int WM = NWV / 2;                    // row slots (the column halves are 2)
  constexpr int MB = kGM / WM / 32;              // 32-row blocks per wave
  constexpr int NB = 4;                          // 32-column blocks per wave
  constexpr int UA = KGK / 8;                    // 16-byte units per row of a's stage
  constexpr int RPA = 64 / UA;                   // rows of a per 1-KB DMA op
  constexpr int A_OPS = kGM * KGK * 2 / 1024 / NWV;  // 1-KB DMA ops per wave per stage
  constexpr int W_OPS = KGK * kGN * 2 / 1024 / NWV;
  constexpr int OPS = A_OPS + W_OPS;             // per wave per stage
  static_assert(A_OPS * NWV * 1024 == kGM * KGK * 2 && W_OPS * NWV * 1024 == KGK * kGN * 2, "DMA split");
  static_assert(NST == 2 || NST == 4, "ring");
  constexpr int SA = kGM * KGK, SW = KGK * kGN;  // elements per buffer
  __shared__ __attribute__((aligned(1024))) bf16_t A0[SA];
  __shared__ __attribute__((aligned(1024))) bf16_t A1[SA];
  __shared__ __attribute__((aligned(1024))) bf16_t A2[NST == 4 ? SA : 1];
  __shared__ __attribute__((aligned(1024))) bf16_t A3[NST == 4 ? SA : 1];
  __shared__ __attribute__((aligned(1024))) bf16_t W0[SW];
  __shared__ __attribute__((aligned(1024))) bf16_t W1[SW];
  __shared__ __attribute__((aligned(1024))) bf16_t W2[NST == 4 ? SW : 1];
  __shared__ __attribute__((aligned(1024))) bf16_t W3[NST == 4 ? SW : 1];
  auto a_swz = [](int r) { return (r / (16 / UA)) & (UA - 1); };

  const int t = threadIdx.x, lane = t & 63, hl = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wv % WM, wn = wv / WM;
  // XCD-aware order: consecutive tile numbers (the column tiles of one row
  // band next to each other) land on one XCD, so a band's rows stay in its L2
  const int tile = xcd_order(blockIdx.x, n_blocks);
  const int tm = tile / n_tiles_n, tn = tile % n_tiles_n;
  const int m0 = tm * kGM, n0 = tn * kGN;
  const int m_valid = min(kGM, rows - m0);

  // DMA descriptors: a's row band (256 rows from m0, of which m_valid
  // exist; the extent ends there) and the whole of W.  In the last row band
  // the rows past m_valid re-read row m_valid - 1 (finite data whose output
  // rows are never stored), with the whole address in the lane offset.
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a + (long long)m0 * C), 0, unsigned(m_valid) * unsigned(C) * 2u, 0x00020000);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)w, 0, unsigned(C) * unsigned(C) * 2u, 0x00020000);
  // a: op i of wave wv fills rows RPA*(i*NWV + wv) .. +RPA-1; lane l writes
  // physical unit l%UA of row l/UA, so it fetches logical unit (l%UA) ^
  // a_swz(row); a_swz(row) = (4*(i*NWV + wv) + l/16) mod UA does not depend
  // on i (NWV is even), so the lane's byte offset is one register and op i
  // adds a scalar RPA*i*NWV rows.
  const int a_unit = (lane % UA) ^ a_swz(RPA * wv + lane / UA);
  const int a_voff = ((RPA * wv + lane / UA) * C + a_unit * 8) * 2;
  // W: op i of wave wv fills k-rows 2*(i*NWV + wv) .. +1 (512-byte rows of
  // 32 units); lane l writes physical unit l%32 of k-row 2*(i*NWV + wv) +
  // l/32, fetching logical unit (l%32) ^ kv_swz(k-row).  The swizzle key
  // (k-row mod 16) depends on i at most through its parity, so the lane has
  // two byte offsets and op i adds a scalar 2*i*NWV k-rows.  When C is an
  // odd multiple of 128 the last column tile has 128 columns: its units
  // 16..31 re-read units 0..15, and the waves of the upper half (wn = 1)
  // store nothing.
  int w_voff[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int kr = 2 * (par * NWV + wv) + (lane >> 5);
    const int u = (lane & 31) ^ kv_swz(kr);
    w_voff[par] = ((kr - 2 * par * NWV) * C + n0 + ((n0 + kGN <= C ? u : (u & 15)) << 3)) * 2;
  }
  // The last stage computes from one buffer while the other (A0, W0: the
  // number of stages is even) is free.  Then each wave that stores copies
  // the old out values of its first 32-row block (32 rows x its 128
  // columns, 8 KB) into its own part of that buffer (waves 0-3 in A0, 4-7
  // in W0), so the read-modify-write below finds half of them in LDS
  // instead of waiting for HBM.  Row r of a copy holds its 16-byte unit u
  // at u ^ (r mod 16); rows past m_valid re-read row m_valid - 1 (never
  // stored).
  static_assert(NST != 2 || (NWV <= 8 && SA >= 4 * 4096 && SW >= 4 * 4096), "out copies fit the free buffer");
  const bool opf = accumulate && NST == 2 && n0 + 128 * wn < C;
  const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(out + (long long)m0 * C), 0, unsigned(m_valid) * unsigned(C) * 2u, 0x00020000);
  auto prefetch_out = [&](bf16_t *__restrict__ Ad, bf16_t *__restrict__ Wd) {
    bf16_t *reg = (wv < 4 ? Ad : Wd) + (wv & 3) * 4096;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 4 * i + (lane >> 4);
      const int u = (lane & 15) ^ (row & 15);
      const int grow = min(32 * MB * wm + row, m_valid - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ors, (lds_void *)(reg + 512 * i), 16,
                                               unsigned((grow * C + n0 + 128 * wn + u * 8) * 2), 0, 0, 0);
    }
  };
  auto issue = [&](int k0, bf16_t *__restrict__ Ad, bf16_t *__restrict__ Wd) {
#pragma unroll
    for (int i = 0; i < A_OPS; ++i) {
      unsigned off = unsigned(a_voff), so = unsigned(k0 + RPA * i * NWV * C) * 2u;
      if (m_valid < kGM) {
        const int row = RPA * (i * NWV + wv) + lane / UA;
        off = unsigned((min(row, m_valid - 1) * C + a_unit * 8) * 2);
        so = unsigned(k0) * 2u;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_void *)(Ad + (RPA * (i * NWV + wv)) * KGK), 16, off,
                                               so, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < W_OPS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_void *)(Wd + (2 * (i * NWV + wv)) * kGN), 16,
                                               unsigned(w_voff[i & 1]),
                                               unsigned(k0 + 2 * i * NWV) * unsigned(C) * 2u, 0, 0);
  };

  // Operand reads.  W^T (A operand) for column block nb and k-step kk:
  // transposing reads (ds_read_b64_tr_b16) of the k-major stage, as for the
  // attention kernel's V tile, with the k-rows in natural order: read r of
  // lane half hl covers k-rows 16kk + 8hl + 4r + (0..3), so element
  // e = 4r + e' of the operand is k = 16kk + 8hl + e, the order in which the
  // B operand (a's rows, 8 consecutive k per lane) arrives; a lane's column
  // is 128wn + 32nb + 16*(gq%2) + 4*(jl%4).  The swizzled unit of a column
  // depends on the block too, so each (nb, r) has its own lane offset; the
  // k-step adds 16 rows (a constant).
  const int gq = lane >> 4, jl = lane & 15;
  int w_rd[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int nc = 128 * wn + 32 * nb + 16 * (gq & 1) + 4 * (jl & 3);
      const int kr = 8 * hl + 4 * r + (jl >> 2);
      w_rd[nb][r] = kr * kGN + (((nc >> 3) ^ kv_swz(kr)) << 3) + (nc & 4);
    }
  // a (B operand) for row block mb and k-step kk: row 32*MB*wm + 32mb +
  // l32, logical unit 2kk + hl; the swizzle key depends on l32 only (the
  // blocks are 32 rows apart)
  const int a_rd = (32 * MB * wm + l32) * KGK;
  const int a_sw = a_swz(l32);

  f32x16 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x16{};

  auto compute = [&](const bf16_t *__restrict__ As, const bf16_t *__restrict__ Ws) {
#pragma unroll
    for (int kk = 0; kk < KGK / 16; ++kk) {
      typedef __attribute__((ext_vector_type(8))) short s16x8;
      bf16x8 wa[NB], ab[MB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(Ws + 16 * kk * kGN + w_rd[nb][0]));
        const s16x4 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(Ws + 16 * kk * kGN + w_rd[nb][1]));
        const s16x8 v = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
        wa[nb] = *(const bf16x8 *)&v;
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        ab[mb] = *(const bf16x8 *)(As + a_rd + 32 * mb * KGK + (((2 * kk + hl) ^ a_sw) << 3));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = mfma_32x32x16(wa[nb], ab[mb], acc[nb][mb]);
    }
  };

  // The ring, unrolled by its length so each step names its buffers
  // statically.  Before computing stage kt: wait until this wave's DMA of
  // stage kt has landed (its DMAs complete in issue order, so "at most the
  // later stages' ops outstanding" suffices), barrier (every wave's DMA
  // landed and every wave is done with stage kt-1's buffer), then start the
  // DMA of stage kt + NST - 1 into that buffer.  C is a multiple of 128, so
  // the number of stages n_k is a multiple of NST.
  const int n_k = C / KGK;
  auto step = [&](int kt, const bf16_t *__restrict__ As, const bf16_t *__restrict__ Ws, bf16_t *__restrict__ An,
                  bf16_t *__restrict__ Wn) {
    if (NST == 4 && kt + 2 < n_k)
      __builtin_amdgcn_s_waitcnt(vmcnt_wait(2 * OPS));
    else if (NST == 4 && kt + 1 < n_k)
      __builtin_amdgcn_s_waitcnt(vmcnt_wait(OPS));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    wg_barrier();
    if (kt + NST - 1 < n_k)
      issue((kt + NST - 1) * KGK, An, Wn);
    else if (NST == 2 && opf)
      prefetch_out(An, Wn);
    compute(As, Ws);
  };
  issue(0, A0, W0);
  if constexpr (NST == 4) {
    issue(KGK, A1, W1);
    issue(2 * KGK, A2, W2);
    for (int kt = 0; kt < n_k; kt += 4) {
      step(kt, A0, W0, A3, W3);
      step(kt + 1, A1, W1, A0, W0);
      step(kt + 2, A2, W2, A1, W1);
      step(kt + 3, A3, W3, A2, W2);
    }
  } else {
    for (int kt = 0; kt < n_k; kt += 2) {
      step(kt, A0, W0, A1, W1);
      step(kt + 1, A1, W1, A0, W0);
    }
  }

  // acc[nb][mb][4 r4 + e] = out[m][n] with m = m0 + 32*MB*wm + 32mb + l32
  // and n = n0 + 128wn + 32nb + 8r4 + 4hl + e: four consecutive columns per
  // store.  (The lane's row index passes through an empty asm so that the
  // store addresses are formed here, not hoisted above the K loop where they
  // would hold registers throughout.)
  if (n0 + 128 * wn >= C) return;
  int lr = l32;
  asm volatile("" : "+v"(lr));
  // Old values: the reads from HBM (blocks not copied to LDS) are issued
  // first, then the copied block is read from LDS, so those reads overlap
  // the LDS work.
  bf16x4 old[MB][NB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int mr = 32 * MB * wm + 32 * mb + lr;
    const bf16_t *orow = out + (long long)(m0 + min(mr, m_valid - 1)) * C + n0 + 128 * wn;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        old[mb][nb][r4] = bf16x4{};
        if (accumulate && !(opf && mb == 0)) old[mb][nb][r4] = *(const bf16x4 *)(orow + 32 * nb + 8 * r4 + 4 * hl);
      }
  }
  if (opf) {  // the copy made during the last stage
    const bf16_t *reg = (wv < 4 ? A0 : W0) + (wv & 3) * 4096;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        old[0][nb][r4] = *(const bf16x4 *)(reg + lr * 128 + (((4 * nb + r4) ^ (lr & 15)) << 3) + 4 * hl);
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int mr = 32 * MB * wm + 32 * mb + lr;
    if (mr >= m_valid) continue;
    bf16_t *orow = out + (long long)(m0 + mr) * C + n0 + 128 * wn;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[nb][mb][4 * r4 + e] + float(old[mb][nb][r4][e]));
        *(bf16x4 *)(orow + 32 * nb + 8 * r4 + 4 * hl) = v;
      }
    }
  }
}

constexpr int kGemmWaves = 8, kGemmK = 64, kGemmStages = 2;

// fp32: 64 x 64 tiles of out, K steps of 16 through LDS; thread (ty, tx)
// computes rows 4ty..+3 and columns tx + 16j, j < 4.
__global__ void __launch_bounds__(256) gemm_f32_kernel(const float *__restrict__ a,
                                                       const float *__restrict__ w,
                                                       float *__restrict__ out, int rows, int C,
                                                       int accumulate) {
  __shared__ float As[64][17];
  __shared__ float Ws[16][64];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < C; k0 += 16) {
    for (int e = t; e < 64 * 16; e += 256) {
      const int r = e >> 4, c = e & 15;
      As[r][c] = m0 + r < rows ? a[(long long)(m0 + r) * C + k0 + c] : 0.f;
      const int kr = e >> 6, nc = e & 63;
      Ws[kr][nc] = w[(long long)(k0 + kr) * C + n0 + nc];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(As[4 * ty + i][k], Ws[k][tx + 16 * j], acc[i][j]);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 4 * ty + i;
    if (m >= rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float *d = out + (long long)m * C + n0 + tx + 16 * j;
      *d = acc[i][j] + (accumulate ? *d : 0.f);
    }
  }
}

}  // namespace

const char *gemm_rows(int bf16, long long rows, int C, const void *a, const void *w, float beta,
                      void *out, hipStream_t st) {
  if (rows == 0) return nullptr;
  if (C <= 0 || C % (bf16 ? 128 : 64)) return "gemm: C must be a positive multiple of 128 (bf16) or 64 (f32)";
  if (rows >= (1ll << 31)) return "gemm: too many rows";
  if ((long long)C * C * 2 >= (1ll << 31)) return "gemm: C too large";
  const int acc = beta != 0.f;
  if (!bf16) {
    dim3 grid(C / 64, unsigned((rows + 63) / 64));
    gemm_f32_kernel<<<grid, 256, 0, st>>>((const float *)a, (const float *)w, (float *)out, int(rows), C, acc);
  } else {
    const int tn = (C + kGN - 1) / kGN;
    const long long tiles = (rows + kGM - 1) / kGM * tn;
    gemm_bf16_kernel<kGemmWaves, kGemmK, kGemmStages><<<unsigned(tiles), 64 * kGemmWaves, 0, st>>>(
        (const bf16_t *)a, (const bf16_t *)w, (bf16_t *)out, int(rows), C, acc, tn, int(tiles));
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? nullptr : hipGetErrorString(e);
}

}  // namespace salad
