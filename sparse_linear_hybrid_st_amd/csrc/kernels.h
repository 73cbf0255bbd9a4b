// Host-side launchers of the gfx950 kernels (one per stage of the layer).
// Every launcher enqueues on `st` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace salad {

// Workspace of the Top-K selection: block means of Q and K (fp64
// [B*H][nb][d] each) and the block scores (fp64 [B*H][nb][nb]).
inline size_t select_ws_bytes(const Geom &g) {
  const size_t BH = size_t(g.B) * g.H;
  return 2 * ((BH * g.nb * g.D * sizeof(double) + 255) & ~size_t(255)) +
         ((BH * g.nb * g.nb * sizeof(double) + 255) & ~size_t(255));
}

// File-scope device scratch of salad_linear_state_noalloc (noalloc.hip):
// this device's address of it (looked up on first use per device) and its
// fixed size in bytes.
hipError_t noalloc_scratch(void **out);
size_t noalloc_scratch_bytes();

// Token chunks per (b, h) used by the split-N linear-state reduction.
inline int linear_splits(const Geom &g) {
  // at most 512 workgroups (two per CU at the state kernel's register use),
  // so they all run in one round
  int chunks = (g.N + 127) / 128;
  int want = 512 / (g.B * g.H);
  return want < 1 ? 1 : (want > chunks ? chunks : want);
}

// The gate's token mean runs over tiles of (row chunk, column band): a band
// is 64 groups of 8 columns, a chunk kGateRows token rows.
constexpr int kGateRows = 64;
inline int gate_bands(const Geom &g) { return (g.H * g.D / 8 + 63) / 64; }
inline int gate_chunks(const Geom &g) { return (g.N + kGateRows - 1) / kGateRows; }

// Workspace bytes of the gate: one double per (sample, row chunk, band).
inline size_t gate_ws_bytes(const Geom &g) {
  return size_t(g.B) * gate_chunks(g) * gate_bands(g) * sizeof(double);
}

// RoPE (cos, sin) table in fp64: rope_table_entries(g) double2 entries.
int rope_table_entries(const Geom &g);
hipError_t launch_rope_table(const Geom &g, double2 *table, hipStream_t st);
// table: optional RoPE table (NULL: angles computed per element; same values).
// heads: optional set of heads to move (NULL: all).
hipError_t launch_permute(const Geom &g, int bf16, int rope, int inverse, const void *src,
                          void *dst, hipStream_t st, const double2 *table = nullptr,
                          const uint64_t *heads = nullptr);
// RoPE without reordering: src and dst both [B,N,H,d] (bf16 or f32).
hipError_t launch_rope_rows(const Geom &g, int bf16, const void *src, void *dst,
                            const double2 *table, hipStream_t st);
hipError_t launch_block_select(const Geom &g, int bf16, View qv, View kv, double *qbar,
                               double *kbar, double *scores, int32_t *idx, hipStream_t st);
// partial: [B*H][S][D*D + D] floats of workspace (S = linear_splits).
hipError_t launch_linear_state(const Geom &g, int bf16, View kv, View vv, float *partial,
                               float *h, float *z, hipStream_t st);
// Fused-layer pieces (bf16, d = 128).
// Also writes working-layout copies of K / V when kw_out / vw_out are non-null.
// kw_out / vw_out (working layout) receive the rows of the heads flagged
// in copy_heads.
// s_gate (device, nullable): samples with s_b < g.drop_tau skip the state
// and only write their copies.
hipError_t launch_linear_partials(const Geom &g, View kv, View vv, float *partial, bf16_t *kw_out,
                                  bf16_t *vw_out, const uint64_t copy_heads[4], const float *s_gate,
                                  hipStream_t st);
// h: [B*H][128][128] fp32 state (workspace); hp: [B*H][128][128] bf16 =
// s_b * (H W_p)^T, or H^T when w_p is NULL (full-width projection);
// z: [B*H][128] fp32.
hipError_t launch_linear_finalize(const Geom &g, int bf16, const float *partial, const void *w_p,
                                  const float *s, float *h, bf16_t *hp, float *z, hipStream_t st);
// Sparse attention with the linear branch, projection, gate and inverse
// permutation fused into the epilogue; out in the boundary layout.
// Heads flagged in `work` read K, V through kw, vw (working copies), the
// others through kd, vd (rows in working order where they already are).
// s_gate: samples with s_b < g.drop_tau skip the linear term (out = O_s).
// outl.base non-NULL (full-width projection, hp = H^T): out receives O_s
// and outl receives s_b * O_l (zero rows for dropped samples).  lse_out
// (nullable, [B*H][N] by working row): each row's softmax normaliser in
// log2 units, for a later backward.
hipError_t launch_attn_fused(const Geom &g, View qv, View kw, View vw, View kd, View vd,
                             const uint64_t work[4], const int32_t *idx, const bf16_t *hp,
                             const float *z, const float *s_gate, View outv, View outl, float *lse_out,
                             hipStream_t st);
// Backward preparation (bf16, d = 128): the forward sparse attention per
// row, reduced to lse2 (log2 of the softmax normaliser in units of
// scale*log2(e) scores) and D = dO . O_s; lse2 / dsum rows are `stride`
// apart per head.  K, V and dO of the heads in `work` come from working
// copies (kw, vw, go [B*H][N][128]), the other heads' in place (kd, vd, god
// in the boundary layout), as in launch_attn_fused.
hipError_t launch_attn_bwd_prep(const Geom &g, View qv, View kw, View vw, View kd, View vd,
                                const uint64_t work[4], const int32_t *idx, const bf16_t *go,
                                const bf16_t *god, float *lse2, float *dsum, int stride, hipStream_t st);
// ---- backward (bf16, d = 128) ------------------------------------------------
// Every backward kernel reads the rows of a head in `work` (the temporal
// heads) from working copies [B*H][N][128] and the other heads' rows in
// place from the boundary layout [B,N,H,128], where they already sit in
// their working order (the token order), H*128 elements apart.
// Fixed-order sum of S split partials [B*H][S][D*D + D] into h and z.
hipError_t launch_linear_reduce(const Geom &g, int S, const float *partial, float *h, float *z,
                                hipStream_t st);
// Top-K inverse lists: off [B*H][nb + 1] (per key block, the offset of its
// selecting query blocks in list [B*H][nb * k]).
hipError_t launch_topk_inverse(const Geom &g, const int32_t *idx, int32_t *off, int32_t *list,
                               hipStream_t st);
// Scratch of the linear-branch backward (sizes per B*H heads, d = 128):
// mf [D*D] fp32, mb [D*D] bf16, partial [S][D*D + D] fp32 (S =
// linear_splits), a_red [D*D] and bz [D] fp32, dhb, dhtb [D*D] bf16,
// dwp_h [D*D] fp32, ds_part [16] fp32.
struct LinBwdScratch {
  float *mf;
  bf16_t *mb;
  float *partial, *a_red, *bz;
  bf16_t *dhb, *dhtb;
  float *dwp_h, *ds_part;
};
// Linear-branch and projection gradients that need whole-head sums: M = H
// W_p (mb), A and Bz = dZ (bz), dH and dH^T (dhb, dhtb), dw_p [d][d] and
// ws.ds_part (16 partial sums of dL/ds per head; zero for dropped samples).
// outv.base non-NULL (the forward's output, boundary layout): also each
// working row's D = dO . O_s into dsum (rows Np apart per head).  Q and dO:
// q, go (working copies) for heads in `work`, qd, god (boundary) otherwise.
hipError_t launch_linear_bwd(const Geom &g, const bf16_t *q, const bf16_t *go, const bf16_t *qd,
                             const bf16_t *god, const uint64_t work[4], const float *hm,
                             const float *zv, const bf16_t *w_p, const float *s_gate,
                             const LinBwdScratch &w, float *dw_p, View outv, float *dsum, int Np,
                             hipStream_t st);
// dQ, dK, dV rows (bf16, boundary layout [B,N,H,d]) of the whole layer: the
// sparse branch's gradients plus, in the epilogues, the linear branch's per
// row terms (from M, Z, dH, dH^T, dZ and s; none for dropped samples) and
// the transposed RoPE rotation of dQ and dK (table non-NULL).  lse2 / dsum
// rows are Np apart per head.
struct BwdOut {
  const bf16_t *mb, *dhb, *dhtb;  // [B*H][128][128] bf16
  const float *zv, *dz;           // [B*H][128]
  const float *s_gate;            // [B]
  const double2 *rope_tab;        // NULL: no RoPE
  bf16_t *dq, *dk, *dv;           // boundary layout
};
// q, k, v, go: working copies of the heads in `work`; qd, kd, vd, god: the
// boundary layout (Q, K rotated when RoPE is on) for the other heads.
hipError_t launch_attn_bwd(const Geom &g, const bf16_t *q, const bf16_t *k, const bf16_t *v,
                           const bf16_t *go, const bf16_t *qd, const bf16_t *kd, const bf16_t *vd,
                           const bf16_t *god, const uint64_t work[4], const float *lse2, const float *dsum,
                           int Np, const int32_t *idx, const int32_t *inv_off, const int32_t *inv_list,
                           const BwdOut &out, hipStream_t st);
// Gate backward.  colsum: partial column sums of X [B][splits][C] fp32;
// final: ds_b = sum of the heads' partials, dt_b = ds_b s_b (1 - s_b) (0 for
// dropped samples or with s_override), dgate_w, dgate_b, optional ds_out;
// dx: dX[b, n, :] = dt_b w / N.
int gate_bwd_splits(const Geom &g);
hipError_t launch_gate_colsum(const Geom &g, const bf16_t *x, float *partial, hipStream_t st);
hipError_t launch_gate_bwd(const Geom &g, const float *ds_part, const float *s, int has_gate,
                           const float *colsum, float *dt, float *ds_out, float *dgate_w,
                           float *dgate_b, hipStream_t st);
hipError_t launch_gate_dx(const Geom &g, const float *dt, const bf16_t *w, bf16_t *dx, hipStream_t st);
// ---- window calibration --------------------------------------------------
constexpr int kMaxCalibRadii = 64;
struct CalibRadii {
  int n;
  int32_t r[kMaxCalibRadii];
};
// Row chunks per (b, h) of the error reduction; part holds 2 doubles per chunk.
int calib_splits(const Geom &g);
// err[bh] = ||ow - od||^2 / ||od||^2 over each (b, h)'s rows (fp32 working layout).
hipError_t launch_calib_err(const Geom &g, const float *od, const float *ow, double *part, double *err,
                            hipStream_t st);
// choice[h]: the first radius with max_b err[i][b][h] <= tau, else N - 1.
hipError_t launch_calib_choose(const Geom &g, const CalibRadii &radii, float tau, const double *err,
                               int32_t *choice, hipStream_t st);
// Whether the attention kernel can stream K, V rows through these views.
bool kv_direct_ok(const Geom &g, View kd, View vd);
hipError_t launch_linear_apply(const Geom &g, int bf16, View qv, const float *h, const float *z,
                               float *o_l, hipStream_t st);
// ws: gate_ws_bytes of workspace.
hipError_t launch_gate(const Geom &g, int bf16, const void *x, const void *w, float bias,
                       void *ws, float *s, hipStream_t st);
hipError_t launch_combine(const Geom &g, int bf16, const float *o_s, const float *o_l,
                          const void *w_p, const float *s, void *out, hipStream_t st);
hipError_t launch_sparse_attn(const Geom &g, int bf16, View qv, View kv, View vv,
                              const int32_t *idx, float *o_s, hipStream_t st);
// Staged full-width projection: out[b, pi_h(p), h, :] = o_s[b,h,p,:] and
// olt (same layout) = s_b * o_l[b,h,p,:] (zero for dropped samples).
hipError_t launch_split_full(const Geom &g, int bf16, const float *o_s, const float *o_l,
                             const float *s, void *out, void *olt, hipStream_t st);
// Row-major out[rows, C] = a[rows, C] W[C, C] + beta * out (one MFMA GEMM
// kernel for bf16, a tiled fp32 kernel for f32; float32 accumulation; C a
// multiple of 128 for bf16, of 64 for f32; beta 0 or 1).  a must not
// overlap out.
// Returns NULL on success, else a message.
const char *gemm_rows(int bf16, long long rows, int C, const void *a, const void *w, float beta,
                      void *out, hipStream_t st);

}  // namespace salad
