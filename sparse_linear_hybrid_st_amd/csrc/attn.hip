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
//   * A workgroup of four waves owns a query tile: 128 queries of a window
//     head (each wave 32 queries over every key), or one 64-query block of
//     a Top-K head (two query groups of 32 times the two 32-key halves of
//     every key tile; the halves are merged after the last tile).  A wave
//     keeps its queries in registers as MFMA B operands.
//   * Key tiles of 64 rows are staged in LDS, double-buffered (two
//     workgroups per CU): K row-major (XOR-swizzled 16-byte units), read
//     transposed for V, so that both MFMA operand reads are contiguous.
//     The next tile's DMA is issued before the current tile's MFMAs.
//   * S^T = K Q^T puts one query per lane column, so the online softmax
//     (exp2, running sum, and the rare offset update) is lane-local except
//     for one exchange between the two half-waves; P^T then feeds
//     O^T += V^T P^T directly from
//     registers (the key order inside an MFMA k-step is free, so P needs no
//     shuffle).
//   * Window heads skip key tiles outside the window, and tiles that lie
//     wholly inside every query's window skip the mask.  Top-K heads walk
//     the selected block list.
// f32 path (d = 64 or 128): one thread per query walks its key set.
#include "common.h"
#include "kernels.h"
#include "mfma_util.h"

namespace salad {


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
struct AttnArgs {
  Geom g;
  View q;
  View k, v;             // K, V of the heads flagged in `work` (working copies)
  View kd, vd;           // K, V of the other heads (rows already in working order)
  uint64_t work[4];
  const int32_t *idx;
  float *o_s;            // staged: working layout fp32 output
  const bf16_t *hp;      // fused: [B*H][128][128] bf16, s_b * (H W_p)^T (H^T with out_l)
  const float *z;        // fused: [B*H][128] linear normaliser state
  const float *s_gate;   // fused: [B] gate values (branch dropping below g.drop_tau)
  View out;              // fused: output rows (boundary layout, scattered)
  View out_l;            // fused, full-width projection: s_b * O_l rows (base NULL otherwise)
  const bf16_t *go;      // backward prep: dL/dO_s, working layout [B*H][N][128] (heads in work)
  const bf16_t *god;     // backward prep: dL/dO_s, boundary layout [B,N,H,128] (other heads)
  float *lse2;           // backward prep: [B*H][lse_stride] log2 of each row's softmax normaliser;
                         // fused: optional [B*H][N] copy of the same for a later backward
  float *dsum;           // backward prep: [B*H][lse_stride] D = dO . O_s per row
  int lse_stride;        // backward prep: row stride of lse2 / dsum per head (>= N)
  int n_heads_sel;       // heads handled by this launch
  uint8_t heads[kMaxHeads];
  int tiles_per_head;    // query tiles per (b, head)
  int n_blocks;          // grid size (for the XCD-aware order)
};

// MODE 0: O_s to a.o_s (fp32, working layout).  MODE 1: fused layer
// epilogue (linear branch, projection, gate, scatter to token order).
// MODE 2: backward preparation -- per row, the log2-domain normaliser
// lse2 (P = exp2(scale*log2(e)*s - lse2)) and D = dO . O_s.
// TOPK: the heads of this launch are Top-K heads.  Key-split workgroups
// (Top-K heads): 64 queries, four waves as two query groups of 32 (qg) times
// the two 32-key halves of every key tile (kg); the halves of a query group
// are merged after the last tile.  Otherwise (window heads): 128 queries,
// wave w the query group w over every key of each tile.
template <int MODE, bool TOPK>
__global__ void __launch_bounds__(256, 2) attn_bf16_kernel(AttnArgs a) {
  constexpr bool FUSED = MODE == 1;
  constexpr bool KS = TOPK;
  constexpr int NW = 4;                          // waves per workgroup
  constexpr int BM = KS ? 64 : 128;              // queries per workgroup
  constexpr int NKB = KS ? 1 : 2;                // 32-key blocks of a tile per wave
  constexpr int TILE = kBN * kD;                 // elements per K or V tile
  constexpr int DMA_PER_WAVE = (TILE * 2 / 1024) / NW;  // 1-KB DMA ops per tensor per wave
  // Two named buffers per tensor (not one indexed array): with distinct LDS
  // objects the compiler can tell that the DMA into one buffer does not
  // feed the reads of the other, so it does not wait for the next tile's
  // DMA before computing on the current one.  64 KB per workgroup: two
  // workgroups (eight waves) share a CU.
  __shared__ __attribute__((aligned(1024))) bf16_t K0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16_t K1[TILE];
  __shared__ __attribute__((aligned(1024))) bf16_t V0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16_t V1[TILE];
  const Geom &g = a.g;
  // the wave index is uniform per wave; readfirstlane lets the compiler use
  // it as a scalar (the DMA destination in M0 must be wave-uniform)
  const int t = threadIdx.x, lane = t & 63, hl = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int qg = KS ? (w & 1) : w;   // query group of 32
  const int kg = KS ? (w >> 1) : 0;  // key half of each tile (key-split)
  const int kb0 = KS ? kg : 0;       // first 32-key block of a tile this wave takes

  const int tile = xcd_order(blockIdx.x, a.n_blocks);
  const int qt = tile % a.tiles_per_head;
  const int bhs = tile / a.tiles_per_head;
  const int h = a.heads[bhs % a.n_heads_sel];
  const int b = bhs / a.n_heads_sel;
  const int q0 = qt * BM;
  const int bh = b * g.H + h;

  // K and V of this head: from the working copies, or, for heads whose
  // working order is the token order, straight from the rows they already
  // occupy (the two views have the same form; the host checked both)
  const bool from_work = bit(a.work, h);
  const bf16_t *qbase = (const bf16_t *)a.q.base;
  const bf16_t *kbase = (const bf16_t *)(from_work ? a.k.base : a.kd.base);
  const bf16_t *vbase = (const bf16_t *)(from_work ? a.v.base : a.vd.base);
  const long long kv_sB = from_work ? a.k.sB : a.kd.sB;
  const long long kv_sH = from_work ? a.k.sH : a.kd.sH;

  // this wave's queries as MFMA B operands: lane -> query q0 + 32qg + l32,
  // features 16ks + 8hl + e
  const int pq = q0 + 32 * qg + l32;
  const long long q_off = row_offset(g, a.q, b, h, min(pq, g.N - 1));
  bf16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8 *)(qbase + q_off + (2 * ks + hl) * 8);

  int n_tiles, kt_first = 0;
  const int32_t *sel = nullptr;
  if (TOPK) {
    n_tiles = g.k;
    sel = a.idx + ((long long)bh * g.nb + q0 / g.block) * g.k;
  } else {
    const int lo = max(0, q0 - g.r);
    const int hi = min(g.N - 1, q0 + BM - 1 + g.r);
    kt_first = lo / kBN;
    n_tiles = hi / kBN - kt_first + 1;
  }
  const int wq_lo = q0 + 32 * qg, wq_hi = min(q0 + 32 * qg + 31, g.N - 1);

  // First key row of tile `it`.  An out-of-range block index (only possible
  // if idx was not produced by the selection) maps past the end, where every
  // row is masked.  Top-K workgroups first copy their block list to LDS, so
  // reading it inside the tile loop is an LDS read, not a global load whose
  // wait would also wait for the DMAs in flight.
  extern __shared__ int32_t sel_lds[];  // Top-K: g.k block start rows
  if (TOPK) {
    for (int j = t; j < n_tiles; j += NW * 64) {
      const int kb = sel[j];
      sel_lds[j] = (kb >= 0 && kb < g.nb) ? kb * g.block : g.N;
    }
    __syncthreads();
  }
  auto tile_start = [&](int it) -> int {
    if (!TOPK) return (kt_first + it) * kBN;
    return sel_lds[it];
  };
  // DMA one K and one V tile into a buffer: op i of wave w fills LDS rows
  // 4*(i*NW + w) .. +3; lane l writes physical unit l%16 of row l/16, so it
  // fetches logical unit (l%16) ^ kv_swz(row).  Rows of this (b, h) are in
  // working order, sN elements apart (checked on the host), so a lane's
  // address is a per-head base plus a lane-constant offset.
  // Rows past N (only in the last tile) re-read row N-1: finite data whose
  // keys are masked.
  // The DMAs are buffer loads: a descriptor per head (base, byte extent) in
  // SGPRs, the tile start as a scalar offset and a lane-constant byte
  // offset, so issuing a tile costs no per-lane address arithmetic.
  const int sN = int(from_work ? a.k.sN : a.kd.sN);
  const unsigned head_bytes = unsigned((long long)(g.N - 1) * sN * 2 + kD * 2);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(kbase + (long long)b * kv_sB + (long long)h * kv_sH), 0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(vbase + (long long)b * kv_sB + (long long)h * kv_sH), 0, head_bytes, 0x00020000);
  int dma_row[DMA_PER_WAVE], dma_off[DMA_PER_WAVE];  // row in tile, byte offset
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    dma_row[i] = 4 * (i * NW + w) + (lane >> 4);
    dma_off[i] = 2 * (dma_row[i] * sN + (((lane & 15) ^ kv_swz(dma_row[i])) << 3));
  }
  auto issue_tile = [&](int k0, bf16_t *__restrict__ Kd, bf16_t *__restrict__ Vd) {
    const bool tail = k0 + kBN > g.N;
    const unsigned soff = unsigned(k0) * unsigned(sN) * 2u;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      int off = dma_off[i];
      if (tail) off -= 2 * (k0 + dma_row[i] - min(k0 + dma_row[i], g.N - 1)) * sN;
      lds_void *kd = (lds_void *)(Kd + (4 * (i * NW + w)) * kD);
      lds_void *vd = (lds_void *)(Vd + (4 * (i * NW + w)) * kD);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, kd, 16, unsigned(off), soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, vd, 16, unsigned(off), soff, 0, 0);
    }
  };

  // Lane-constant LDS element offsets.  K operand (row kb*32 + l32, logical
  // unit 2ks + hl): the swizzle key depends on l32 only, so unit
  // (2ks + hl) ^ swz = 2 (ks ^ (swz >> 1)) + (hl ^ (swz & 1)).
  const int kswz = kv_swz(l32);
  const int k_lane = l32 * kD + 8 * (hl ^ (kswz & 1));
  const int k_x = kswz >> 1;
  // V^T operand, transposing read r of d-block db for k-step kk:
  // row = 32*(kk/2) + 16*(kk%2) + 8r + 4hl + jl/4 and
  // d = 32db + 16*(gq%2) + 4*(jl%4); its swizzle key depends on (lane, r).
  const int gq = lane >> 4, jl = lane & 15;
  int v_off[2][4];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int row = 8 * r + 4 * hl + (jl >> 2);
      const int d = 32 * db + 16 * (gq & 1) + 4 * (jl & 3);
      v_off[r][db] = row * kD + (((d >> 3) ^ kv_swz(row)) << 3) + (d & 4);
    }

  const float c2 = g.scale * 1.4426950408889634f;  // softmax scale * log2(e)
  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  // Running offset m_off (log2 units) of this lane's query: probabilities are
  // exp2(c2 * s - m_off).  l_run: this lane's partial row sum.  m_set_w:
  // the lanes whose offset has been taken from a real score (until then no
  // key has counted), kept as a wave mask so the per-block test below is
  // one compare and scalar logic.
  float m_off = 0.f, l_run = 0.f;
  unsigned long long m_set_w = 0ull;

  // One key tile: S^T = K Q^T (qk), online softmax (softmax), O^T += V^T
  // P^T (pv), over this wave's NKB blocks of 32 keys of the tile (blocks
  // kb0 .. kb0 + NKB - 1).  classify tells whether those keys hold any key
  // of this wave's queries and whether they need no mask.  Each phase takes
  // its LDS buffer as a restrict parameter, which lets the compiler tell its
  // reads apart from DMAs into the other buffers.
  auto classify = [&](int k0, bool &any, bool &full) {
    const int ku = k0 + 32 * kb0;                  // first key of this wave's part
    const int ke = ku + 32 * NKB;                  // one past its last
    const int k1 = min(ke, g.N) - 1;
    if (TOPK) {
      any = ku < g.N;
      full = ke <= g.N;
    } else {
      any = (ku <= wq_hi + g.r) && (k1 >= wq_lo - g.r) && (wq_lo <= wq_hi);
      full = (ke <= g.N) && (ku >= wq_hi - g.r) && (ke - 1 <= wq_lo + g.r);
    }
  };
  // S^T[key][query] = K Q^T per block of 32 keys (raw scores: products of
  // the stored values, accumulated in fp32).  kop: the K operand of block kb
  // of this wave's part of the tile for feature step ks.
  auto kop = [&](const bf16_t *__restrict__ Ks, int kb, int ks) -> bf16x8 {
    return *(const bf16x8 *)(Ks + (kb0 + kb) * 32 * kD + k_lane + 16 * (ks ^ k_x));
  };
  // K operands of feature steps 1..7 of block kb (step 0 starts the
  // accumulator; below), and their products.  The operands are read as a
  // batch, one phase before the products that use them, so no product
  // waits for its own LDS read.
  auto kread = [&](const bf16_t *__restrict__ Ks, int kb, bf16x8 (&ka)[7]) {
#pragma unroll
    for (int ks = 1; ks < 8; ++ks) ka[ks - 1] = kop(Ks, kb, ks);
  };
  auto qk_rest = [&](const bf16x8 (&ka)[7], f32x16 &s) {
#pragma unroll
    for (int ks = 1; ks < 8; ++ks) s = mfma_32x32x16(ka[ks - 1], qf[ks], s);
  };
  // Softmax.  Key j is kept
  // iff j < N and, for window heads, |pq - j| <= r, i.e. the unsigned value
  // pq - j + r is at most 2r (one subtract and one compare per score); the
  // mask is applied where the scores start (qk_first).
  // The offset m_off only has to bound the row's scores loosely: O and l
  // share it, so the final O / l is exact whatever its value.  Each lane
  // exponentiates its scores under the current offset (one FMA and one
  // exp2 per score: the scores stay exact products), packs them to bf16
  // for the PV product and sums them in fp32 (plain adds: the dot-product
  // instructions that could sum the packed pairs share the matrix unit's
  // issue and cost more than the adds).  A lane whose block sum exceeds 2^8
  // may hold a probability above 2^8 (every term is at most the sum); only then, or
  // while no offset has been taken, is the tile's true maximum formed,
  // combined with the other half-wave (which holds the other keys of the
  // same query, so both halves keep one offset), the offset raised to it, O
  // and l rescaled and the tile's probabilities recomputed.  So probabilities
  // stay below 2^8 (no overflow in fp32 sums or in bf16), and an ordinary
  // tile costs one FMA, one exp2, half a pack and one add per score.  (The test
  // is per block of 32 keys: with 16 scores per lane it bounds each one the
  // same way.)
  auto exp_pack = [&](const f32x16 &s, float shift, bf16x8 &p0, bf16x8 &p1) -> float {
    float x[16];
#pragma unroll
    for (int e = 0; e < 16; ++e)
      // v_exp_f32 directly: tiny results flush to 0; large ones (even inf)
      // are caught by the block-sum test below and recomputed
      x[e] = __builtin_amdgcn_exp2f(fmaf(s[e], c2, -shift));
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      bf16x8 pv;
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = (__bf16)x[8 * half + e];
      (half ? p1 : p0) = pv;
    }
    // the row sum in fp32 (a pairwise tree: v_add, not the dot-product
    // instructions, which share the matrix unit's issue)
#pragma unroll
    for (int w2 = 1; w2 < 16; w2 *= 2)
#pragma unroll
      for (int e = 0; e < 16; e += 2 * w2) x[e] += x[e + w2];
    return x[0];
  };
  // First feature step of every block.  The accumulator starts at 0; on
  // edge tiles a masked key's starts at -inf instead, which the products
  // (finite) leave at -inf, so the mask costs nothing after the scores
  // exist and the tile's VALU work needs no second, masked copy.
  auto qk_first = [&](const bf16_t *__restrict__ Ks, int k0, bool full, f32x16 (&s)[NKB]) {
    bf16x8 ka[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) ka[kb] = kop(Ks, kb, 0);
    if (full) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] = mfma_32x32x16(ka[kb], qf[0], f32x16{});
    } else {
      int jl = k0 + 4 * hl;                              // j = jl + c below
      // opaque to the optimiser: otherwise it carries the per-score
      // differences below across tiles as induction variables, updating
      // them on every tile although only edge tiles use them
      asm volatile("" : "+v"(jl));
      const unsigned wb = unsigned(pq - jl + g.r);        // pq - j + r = wb - c
      const int lim = g.N - jl;                          // j < N  <=>  c < lim
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        f32x16 init;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = (kb0 + kb) * 32 + 8 * (r >> 2) + (r & 3);
          // bitwise, not short-circuit: keeps the mask a select, not a branch
          const bool keep = (c < lim) & (TOPK | (wb - unsigned(c) <= unsigned(2 * g.r)));
          init[r] = keep ? 0.f : -INFINITY;
        }
        s[kb] = mfma_32x32x16(ka[kb], qf[0], init);
      }
    }
  };
  // Softmax of block kb of the tile, in place (its masked scores are -inf
  // already).  sched: scheduling hints for the straight-line code up to the
  // rare rescale branch.
  auto softmax = [&](int kb, f32x16 &s, bf16x8 &p0, bf16x8 &p1, auto sched) {
    float lt = exp_pack(s, m_off, p0, p1);
    const unsigned long long need_w = __ballot(!(lt <= 256.f)) | ~m_set_w;
    sched();
    if (need_w) {
      const bool need = (need_w >> lane) & 1ull, m_set = (m_set_w >> lane) & 1ull;
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = fmaf(mx, c2, -m_off);  // relative to the current offset (c2 > 0)
      // both half-waves of a query column agree on the maximum and on
      // whether to move the offset
      // (the swap of x with itself gives lanes 0-31's x in [0] and lanes
      // 32-63's in [1], on every lane)
      const unsigned um = __float_as_uint(mx), un = need ? 1u : 0u;
      const auto sm = __builtin_amdgcn_permlane32_swap(um, um, false, false);
      const auto sn = __builtin_amdgcn_permlane32_swap(un, un, false, false);
      const float mxa = fmaxf(__uint_as_float(sm[0]), __uint_as_float(sm[1]));
      const bool need_q = (sn[0] | sn[1]) != 0u;
      const float delta = (need_q && mxa != -INFINITY) ? mxa : 0.f;
      if (delta != 0.f) {
        const float alpha = m_set ? __builtin_amdgcn_exp2f(-delta) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        m_off += delta;
      }
      m_set_w |= __ballot(mxa != -INFINITY);
      if (__any(delta != 0.f)) lt = exp_pack(s, m_off, p0, p1);
    }
    l_run += lt;
  };
  // O^T[d][q] += V^T[d][keys] P^T[keys][q] over block kb of 32 keys.
  // k-step kk, half hl, element e = 4r + e' covers key
  // 32*(kk/2) + 8*(2*(kk%2) + r) + 4*hl + e' of this wave's part of the
  // tile (which starts at row 32*kb0); the matching V^T operand comes from
  // two transposing reads (r = 0, 1).  vread reads block kb's eight
  // operands (two k-steps x four d-blocks) as a batch ahead of pv.
  typedef __attribute__((ext_vector_type(8))) short s16x8;
  auto vread = [&](const bf16_t *__restrict__ Vs, int kb, s16x8 (&va)[8]) {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16_t *vk = Vs + 16 * (2 * kb0 + 2 * kb + k2) * kD;
        const s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vk + v_off[0][db]));
        const s16x4 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vk + v_off[1][db]));
        va[4 * k2 + db] = s16x8{p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      }
  };
  auto pv = [&](const s16x8 (&va)[8], const bf16x8 &p0, const bf16x8 &p1) {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        o[db] = mfma_32x32x16(*(const bf16x8 *)&va[4 * k2 + db], k2 ? p1 : p0, o[db]);
  };
  auto compute = [&](int k0, const bf16_t *__restrict__ Ks, const bf16_t *__restrict__ Vs) {
    bool any, full;
    classify(k0, any, full);
    if (!any) return;
    f32x16 s[NKB];
    bf16x8 pb[2 * NKB];
    qk_first(Ks, k0, full, s);
    bf16x8 ka[7];
    s16x8 va[8];
    kread(Ks, 0, ka);
    if constexpr (NKB == 2) {
      // Ordered so that each block's softmax (VALU) has independent MFMAs
      // to issue beside it, and every batch of operands is read one phase
      // ahead: block 0's products (block 1's K operands read meanwhile),
      // block 1's products with block 0's softmax (block 0's V operands
      // read meanwhile), block 0's PV products with block 1's softmax
      // (block 1's V operands read meanwhile), block 1's PV products.
      qk_rest(ka, s[0]);
      bf16x8 kb1[7];
      kread(Ks, 1, kb1);
      qk_rest(kb1, s[1]);
      vread(Vs, 0, va);
      softmax(0, s[0], pb[0], pb[1], [] {
        __builtin_amdgcn_sched_group_barrier(0x100, 7, 0);
#pragma unroll
        for (int i = 0; i < 7; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 7; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
        }
      });
      pv(va, pb[0], pb[1]);
      s16x8 vb[8];
      vread(Vs, 1, vb);
      softmax(1, s[1], pb[2], pb[3], [] {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        }
      });
      pv(vb, pb[2], pb[3]);
    } else {
      // block 0's products with its V operands read meanwhile, its
      // softmax, its PV products
      qk_rest(ka, s[0]);
      vread(Vs, 0, va);
      softmax(0, s[0], pb[0], pb[1], [] {
        __builtin_amdgcn_sched_group_barrier(0x100, 7, 0);
#pragma unroll
        for (int i = 0; i < 7; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      });
      pv(va, pb[0], pb[1]);
    }
  };

  // Tile starts are read before each DMA is issued and carried along, so no
  // global load (and its wait) sits between a DMA and the LDS reads.  Each
  // wave's DMAs complete in issue order, so "vmcnt <= n" means all but the
  // last n issued have landed; a barrier after such a wait makes every
  // wave's share visible.
  int k_cur = n_tiles > 0 ? tile_start(0) : 0;
  {
    // Double-buffered, unrolled by two so each half names its buffers
    // statically.  Before computing tile it: wait for this wave's DMA of
    // tile it (vmcnt 0), barrier (every wave's DMA landed and every wave is
    // done with the other buffer), then start the DMA of tile it+1.
    if (n_tiles > 0) issue_tile(k_cur, K0, V0);
    for (int it = 0; it < n_tiles; it += 2) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      const int k_nxt = it + 1 < n_tiles ? tile_start(it + 1) : 0;
      if (it + 1 < n_tiles) issue_tile(k_nxt, K1, V1);
      compute(k_cur, K0, V0);
      if (it + 1 >= n_tiles) break;
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      const int k_nn = it + 2 < n_tiles ? tile_start(it + 2) : 0;
      if (it + 2 < n_tiles) issue_tile(k_nn, K0, V0);
      compute(k_nxt, K1, V1);
      k_cur = k_nn;
    }
  }

  if constexpr (KS) {
    // Merge the key halves of each query group: the waves with kg = 1 hand
    // their offset, partial sums and O to the kg = 0 wave of the same query
    // group through LDS (the tile buffers are free now); O and l are scaled
    // to the larger offset.  A half that saw no key (no offset) adds nothing.
    __syncthreads();                       // every wave is done with the tile buffers
    bool m_set = (m_set_w >> lane) & 1ull;
    float *xo = (float *)(qg ? K1 : K0);  // [64 values][64 lanes]
    float *xm = (float *)V0 + qg * 192;    // [3][64 lanes]
    if (kg == 1) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(db * 16 + r) * 64 + lane] = o[db][r];
      xm[lane] = m_off;
      xm[64 + lane] = l_run;
      xm[128 + lane] = m_set ? 1.f : 0.f;
    }
    __syncthreads();
    if (kg == 0 && xm[128 + lane] != 0.f) {
      const float m_b = xm[lane], l_b = xm[64 + lane];
      const float m_new = m_set ? fmaxf(m_off, m_b) : m_b;
      const float a0 = m_set ? __builtin_amdgcn_exp2f(m_off - m_new) : 0.f;
      const float a1 = __builtin_amdgcn_exp2f(m_b - m_new);
      l_run = l_run * a0 + l_b * a1;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * a0 + xo[(db * 16 + r) * 64 + lane] * a1;
      m_off = m_new;
      m_set = true;
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;

  if constexpr (FUSED) {
    // For a later backward: each row's normaliser in log2 units ([B*H][N])
    if (a.lse2 && hl == 0 && kg == 0 && pq < g.N) a.lse2[(long long)bh * g.N + pq] = m_off + log2f(l_tot);
    // Branch dropping ([G] 2 C): a sample whose gate value is below the
    // threshold keeps only the sparse branch (its state was not computed).
    if (a.s_gate[b] < g.drop_tau) {
      if (kg != 0 || pq >= g.N) return;
      bf16_t *orow = (bf16_t *)a.out.base + row_offset(g, a.out, b, h, pq);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[db][4 * r4 + e] * inv);
          *(bf16x4 *)(orow + 32 * db + 8 * r4 + 4 * hl) = v;
        }
      if (a.out_l.base) {  // the projection GEMM then adds nothing to this row
        bf16_t *lrow = (bf16_t *)a.out_l.base + row_offset(g, a.out_l, b, h, pq);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) *(bf16x4 *)(lrow + 32 * db + 8 * r4 + 4 * hl) = bf16x4{};
      }
      return;
    }
    // Linear branch, projection, gate and combine for this wave's queries:
    //   out = O_s + relu(q) Hp / (relu(q) . Z + eps),  Hp = s_b (H W_p)^T
    // Hp rows 0..63 go to K0 and rows 64..127 to V0 (same swizzle as K);
    // every wave loads its share, the waves holding the queries use it.
    __syncthreads();  // every wave is done with the tile buffers
    const bf16_t *hsrc = a.hp + (long long)bh * kD * kD;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const int row = 4 * (i * NW + w) + (lane >> 4);
      const int u = (lane & 15) ^ kv_swz(row);
      __builtin_amdgcn_global_load_lds((const void *)(hsrc + row * kD + u * 8),
                                       (lds_void *)(K0 + (4 * (i * NW + w)) * kD), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void *)(hsrc + (64 + row) * kD + u * 8),
                                       (lds_void *)(V0 + (4 * (i * NW + w)) * kD), 16, 0, 0);
    }
    // relu(q) operands and the normaliser relu(q) . Z (this lane's 64 features
    // plus the other half-wave's)
    const float *zr = a.z + (long long)bh * kD;
    bf16x8 rq[8];
    float den = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const f32x4 z0 = *(const f32x4 *)(zr + 16 * ks + 8 * hl);
      const f32x4 z1 = *(const f32x4 *)(zr + 16 * ks + 8 * hl + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qv = fmaxf(float(qf[ks][e]), 0.f);
        rq[ks][e] = (__bf16)qv;  // exact: relu of a bf16 value
        den = fmaf(qv, e < 4 ? z0[e] : z1[e - 4], den);
      }
    }
    den += __shfl_xor(den, 32);
    const float inv_den = 1.f / (den + g.eps);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (kg != 0) return;
    f32x16 lin[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) lin[db] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16_t *hb = (db < 2 ? K0 : V0) + (db & 1) * 32 * kD;
        const bf16x8 ha = *(const bf16x8 *)(hb + k_lane + 16 * (ks ^ k_x));
        lin[db] = mfma_32x32x16(ha, rq[ks], lin[db]);
      }
    if (pq >= g.N) return;
    bf16_t *orow = (bf16_t *)a.out.base + row_offset(g, a.out, b, h, pq);
    if (a.out_l.base) {
      // full-width projection: O_s here, s_b * O_l to its own rows; a GEMM
      // over whole token rows adds (s_b O_l) W_p afterwards
      bf16_t *lrow = (bf16_t *)a.out_l.base + row_offset(g, a.out_l, b, h, pq);
      const float sl = a.s_gate[b] * inv_den;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          bf16x4 v, u;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = (__bf16)(o[db][4 * r4 + e] * inv);
            u[e] = (__bf16)(lin[db][4 * r4 + e] * sl);
          }
          *(bf16x4 *)(orow + 32 * db + 8 * r4 + 4 * hl) = v;
          *(bf16x4 *)(lrow + 32 * db + 8 * r4 + 4 * hl) = u;
        }
      return;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = (__bf16)(o[db][4 * r4 + e] * inv + lin[db][4 * r4 + e] * inv_den);
        *(bf16x4 *)(orow + 32 * db + 8 * r4 + 4 * hl) = v;
      }
    return;
  }

  if (kg != 0) return;
  if constexpr (MODE == 2) {
    // both half-waves of a query column return together, so the exchange
    // below sees its partner
    if (pq >= g.N) return;
    const bf16_t *grow = from_work ? a.go + ((long long)bh * g.N + pq) * kD
                                   : a.god + (((long long)b * g.N + pq) * g.H + h) * kD;
    float dp = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const bf16x4 gv = *(const bf16x4 *)(grow + 32 * db + 8 * r4 + 4 * hl);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp = fmaf(o[db][4 * r4 + e] * inv, float(gv[e]), dp);
      }
    dp += __shfl_xor(dp, 32);
    if (hl == 0) {
      const long long row = (long long)bh * a.lse_stride + pq;
      a.dsum[row] = dp;
      a.lse2[row] = m_off + log2f(l_tot);
    }
    return;
  }
  if (pq >= g.N) return;
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

namespace {
// One launch per head kind: window heads in 128-query tiles, Top-K heads one
// 64-query block per workgroup; four waves each.
template <int MODE>
hipError_t launch_bf16(AttnArgs a, hipStream_t st) {
  const Geom &g = a.g;
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
    if (mode)
      attn_bf16_kernel<MODE, true><<<grid, 256, size_t(g.k) * sizeof(int32_t), st>>>(a);
    else
      attn_bf16_kernel<MODE, false><<<grid, 256, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
}  // namespace

// The bf16 kernel streams K and V of one (b, h) as rows sN elements apart,
// with the same strides for both, and addresses a head's rows with 32-bit
// byte offsets.
static bool kv_streamable(const Geom &g, const View &kv, const View &vv) {
  return !kv.perm && !vv.perm && kv.sB == vv.sB && kv.sH == vv.sH && kv.sN == vv.sN &&
         kv.sN > 0 && kv.sN < (1ll << 20) && (long long)(g.N - 1) * kv.sN * 2 + kD * 2 < (1ll << 32);
}

bool kv_direct_ok(const Geom &g, View kd, View vd) { return kv_streamable(g, kd, vd); }

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
  if (!kv_streamable(g, kv, vv)) return hipErrorInvalidValue;
  AttnArgs a = {};
  a.g = g;
  a.q = qv;
  a.k = a.kd = kv;
  a.v = a.vd = vv;
  for (int i = 0; i < 4; ++i) a.work[i] = ~0ull;
  a.idx = idx;
  a.o_s = o_s;
  return launch_bf16<0>(a, st);
}

hipError_t launch_attn_bwd_prep(const Geom &g, View qv, View kw, View vw, View kd, View vd,
                                const uint64_t work[4], const int32_t *idx, const bf16_t *go,
                                const bf16_t *god, float *lse2, float *dsum, int stride, hipStream_t st) {
  bool any_work = false, any_direct = false;
  for (int h = 0; h < g.H; ++h) {
    const bool w = (work[h >> 6] >> (h & 63)) & 1ull;
    any_work |= w;
    any_direct |= !w;
  }
  if ((any_work && !kv_streamable(g, kw, vw)) || (any_direct && !kv_streamable(g, kd, vd)))
    return hipErrorInvalidValue;
  AttnArgs a = {};
  a.g = g;
  a.q = qv;
  a.k = kw;
  a.v = vw;
  a.kd = kd;
  a.vd = vd;
  for (int i = 0; i < 4; ++i) a.work[i] = work[i];
  a.idx = idx;
  a.go = go;
  a.god = god;
  a.lse2 = lse2;
  a.dsum = dsum;
  a.lse_stride = stride;
  return launch_bf16<2>(a, st);
}

hipError_t launch_attn_fused(const Geom &g, View qv, View kw, View vw, View kd, View vd,
                             const uint64_t work[4], const int32_t *idx, const bf16_t *hp,
                             const float *z, const float *s_gate, View outv, View outl, float *lse_out,
                             hipStream_t st) {
  bool any_work = false, any_direct = false;
  for (int h = 0; h < g.H; ++h) {
    const bool w = (work[h >> 6] >> (h & 63)) & 1ull;
    any_work |= w;
    any_direct |= !w;
  }
  if ((any_work && !kv_streamable(g, kw, vw)) || (any_direct && !kv_streamable(g, kd, vd)))
    return hipErrorInvalidValue;
  AttnArgs a = {};
  a.g = g;
  a.q = qv;
  a.k = kw;
  a.v = vw;
  a.kd = kd;
  a.vd = vd;
  for (int i = 0; i < 4; ++i) a.work[i] = work[i];
  a.idx = idx;
  a.hp = hp;
  a.z = z;
  a.s_gate = s_gate;
  a.out = outv;
  a.out_l = outl;
  a.lse2 = lse_out;
  return launch_bf16<1>(a, st);
}

}  // namespace salad
