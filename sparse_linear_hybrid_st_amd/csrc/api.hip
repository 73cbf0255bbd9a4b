// C-ABI entry points: argument validation (before anything is enqueued),
// workspace carving and launch order.  See include/salad.h for the contract.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <string>

#include "../../include/salad.h"
#include "common.h"
#include "kernels.h"

using namespace salad;

namespace {

thread_local std::string g_err;

salad_status fail(salad_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

salad_status hip_status(hipError_t e, const char *where) {
  if (e == hipSuccess) return SALAD_OK;
  return fail(SALAD_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Info {
  Geom g;
  int bf16, rope, full;
  int any_topk, any_window;
  size_t esize;
};

salad_status validate(const salad_problem *p, Info *inf) {
  if (!p) return fail(SALAD_ERR_NULL, "problem is NULL");
  if (p->batch < 1) return fail(SALAD_ERR_SHAPE, "batch must be >= 1 (got %d)", p->batch);
  if (p->n_heads < 1 || p->n_heads > SALAD_MAX_HEADS)
    return fail(SALAD_ERR_SHAPE, "n_heads must be in [1, %d] (got %d)", SALAD_MAX_HEADS, p->n_heads);
  if (p->io_dtype != SALAD_F32 && p->io_dtype != SALAD_BF16)
    return fail(SALAD_ERR_SHAPE, "io_dtype must be SALAD_F32 or SALAD_BF16 (got %d)", p->io_dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(SALAD_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", p->head_dim);
  if (p->io_dtype == SALAD_BF16 && p->head_dim != 128)
    return fail(SALAD_ERR_UNSUPPORTED, "bf16 kernels are built for head_dim 128 only");
  if (p->grid_f < 1 || p->grid_h < 1 || p->grid_w < 1)
    return fail(SALAD_ERR_SHAPE, "grid dims must be >= 1");
  const long long N = (long long)p->grid_f * p->grid_h * p->grid_w;
  if (N > (1ll << 28)) return fail(SALAD_ERR_SHAPE, "N = F*Hg*Wg too large (%lld)", N);
  if ((long long)p->batch * p->n_heads * N * p->head_dim > (1ll << 40) ||
      (long long)p->batch * p->n_heads * N >= (1ll << 31))
    return fail(SALAD_ERR_SHAPE, "tensor too large (batch*n_heads*N must stay below 2^31 rows)");
  // the bf16 attention kernels address one head's K/V rows with 32-bit byte
  // offsets: N rows of 256 bytes in a contiguous working copy
  if (p->io_dtype == SALAD_BF16 && N * 128 * 2 > (1ll << 32) - 1)
    return fail(SALAD_ERR_UNSUPPORTED, "bf16 kernels take N < 2^24 tokens (got %lld)", N);
  Geom &g = inf->g;
  memset(&g, 0, sizeof g);
  g.B = p->batch;
  g.H = p->n_heads;
  g.D = p->head_dim;
  g.N = int(N);
  g.F = p->grid_f;
  g.Hg = p->grid_h;
  g.Wg = p->grid_w;
  inf->any_topk = inf->any_window = 0;
  for (int h = 0; h < g.H; ++h) {
    const int k = p->head_kind[h];
    if (k == SALAD_HEAD_TEMPORAL) g.temporal[h >> 6] |= 1ull << (h & 63);
    if (k == SALAD_HEAD_TOPK) g.topk[h >> 6] |= 1ull << (h & 63);
    if (k < 0 || k > 2) return fail(SALAD_ERR_SHAPE, "head_kind[%d] = %d is not a SALAD_HEAD_* value", h, k);
    if (k == SALAD_HEAD_TOPK) inf->any_topk = 1; else inf->any_window = 1;
  }
  if (inf->any_window && p->window_radius < 0)
    return fail(SALAD_ERR_SHAPE, "window_radius must be >= 0 (got %d)", p->window_radius);
  // a radius past N - 1 keeps the same keys as N - 1; clamping it keeps the
  // kernels' 32-bit window arithmetic (q0 + tile + r, 2r) in range
  g.r = p->window_radius < 0 ? 0 : (int)std::min<long long>(p->window_radius, N - 1);
  if (inf->any_topk) {
    if (p->block < 1) return fail(SALAD_ERR_SHAPE, "block must be >= 1 (got %d)", p->block);
    g.block = p->block;
    g.nb = int((N + p->block - 1) / p->block);
    if (p->topk < 1 || p->topk > g.nb)
      return fail(SALAD_ERR_SHAPE, "topk must be in [1, %d] (got %d)", g.nb, p->topk);
    g.k = p->topk;
    if (p->io_dtype == SALAD_BF16 && p->block != 64)
      return fail(SALAD_ERR_UNSUPPORTED, "bf16 Top-K kernels are built for block 64 only (got %d)", p->block);
    if (g.nb > 4096) return fail(SALAD_ERR_UNSUPPORTED, "more than 4096 key blocks (%d)", g.nb);
  } else {
    g.block = p->block > 0 ? p->block : 64;
    g.nb = int((N + g.block - 1) / g.block);
    g.k = p->topk;
  }
  g.scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / sqrtf(float(p->head_dim));
  g.eps = p->linear_eps;
  if (!std::isfinite(p->branch_drop_tau))
    return fail(SALAD_ERR_SHAPE, "branch_drop_tau must be finite");
  if (p->proj_mode != SALAD_PROJ_HEAD && p->proj_mode != SALAD_PROJ_FULL)
    return fail(SALAD_ERR_SHAPE, "proj_mode must be SALAD_PROJ_HEAD or SALAD_PROJ_FULL (got %d)", p->proj_mode);
  inf->full = p->proj_mode == SALAD_PROJ_FULL;
  g.drop_tau = p->branch_drop_tau;
  g.rope_base = p->rope_base;
  for (int i = 0; i < 3; ++i) g.rope_dims[i] = p->rope_dims[i];
  if (p->rope) {
    if (p->rope != 1) return fail(SALAD_ERR_SHAPE, "rope must be 0 or 1");
    int sum = 0;
    for (int i = 0; i < 3; ++i) {
      if (p->rope_dims[i] < 0 || (p->rope_dims[i] & 1))
        return fail(SALAD_ERR_SHAPE, "rope_dims must be even and >= 0");
      sum += p->rope_dims[i];
    }
    if (sum != p->head_dim) return fail(SALAD_ERR_SHAPE, "rope_dims must sum to head_dim");
    if (!(p->rope_base > 0.f)) return fail(SALAD_ERR_SHAPE, "rope_base must be > 0");
  }
  g.fdF = make_fastdiv(uint32_t(g.F));
  g.fdS = make_fastdiv(uint32_t(g.Hg * g.Wg));
  g.fdW = make_fastdiv(uint32_t(g.Wg));
  inf->bf16 = p->io_dtype == SALAD_BF16;
  inf->rope = p->rope;
  inf->esize = inf->bf16 ? 2 : 4;
  return SALAD_OK;
}

// Workspace plan.  Regions are 256-byte aligned.  The stage entry points use
// the first total_stage bytes.  salad_attn_forward adds, after that shared
// scratch: for bf16 (fused) the RoPE'd working Q/K (only with rope), the
// block selection, Hp and Z; for f32 (staged) working copies of Q/K/V, the
// selection, O_s, O_l, H and Z.  Both end with the gate values, the RoPE
// table and, for the full-width projection, s_b * O_l in token rows.
struct Plan {
  size_t wq, wk, wv, wkr, idx, o_s, o_l, h, z, s, hp, rope_tab, olt;
  size_t total_stage, total_forward;
};

size_t up(size_t x) { return (x + 255) & ~size_t(255); }

Plan plan(const Info &inf) {
  const Geom &g = inf.g;
  Plan pl = {};
  const size_t BH = size_t(g.B) * g.H;
  const size_t rows = BH * g.N;
  const size_t means = inf.any_topk ? up(select_ws_bytes(g)) : 0;
  const size_t lin = up(BH * linear_splits(g) * (size_t(g.D) * g.D + g.D) * sizeof(float));
  const size_t gate = up(gate_ws_bytes(g));
  pl.total_stage = means > lin ? (means > gate ? means : gate) : (lin > gate ? lin : gate);
  size_t off = pl.total_stage;
  const size_t idx_bytes = inf.any_topk ? up(BH * g.nb * g.k * sizeof(int32_t)) : 0;
  if (inf.bf16) {
    const bool rope = inf.rope != 0;
    pl.wq = off; off += rope ? up(rows * g.D * inf.esize) : 0;
    pl.wkr = off; off += rope ? up(rows * g.D * inf.esize) : 0;
    pl.wk = off; off += up(rows * g.D * inf.esize);
    pl.wv = off; off += up(rows * g.D * inf.esize);
    pl.idx = off; off += idx_bytes;
    pl.h = off; off += up(BH * g.D * g.D * sizeof(float));
    pl.hp = off; off += up(BH * g.D * g.D * sizeof(bf16_t));
    pl.z = off; off += up(BH * g.D * sizeof(float));
  } else {
    pl.wq = off; off += up(rows * g.D * inf.esize);
    pl.wk = off; off += up(rows * g.D * inf.esize);
    pl.wv = off; off += up(rows * g.D * inf.esize);
    pl.idx = off; off += idx_bytes;
    pl.o_s = off; off += up(rows * g.D * sizeof(float));
    pl.o_l = off; off += up(rows * g.D * sizeof(float));
    pl.h = off; off += up(BH * g.D * g.D * sizeof(float));
    pl.z = off; off += up(BH * g.D * sizeof(float));
  }
  pl.s = off; off += up(size_t(g.B) * sizeof(float));
  pl.rope_tab = off; off += inf.rope ? up(size_t(rope_table_entries(g)) * 16) : 0;
  pl.olt = off; off += inf.full ? up(rows * g.D * inf.esize) : 0;
  pl.total_forward = off;
  return pl;
}

#define CHECK(x)                       \
  do {                                 \
    salad_status _s = (x);             \
    if (_s != SALAD_OK) return _s;     \
  } while (0)

salad_status need(const void *ptr, const char *name) {
  if (!ptr) return fail(SALAD_ERR_NULL, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(SALAD_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return SALAD_OK;
}

salad_status need_ws(void *ws, size_t ws_bytes, size_t needed) {
  if (needed == 0) return SALAD_OK;
  if (!ws) return fail(SALAD_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", needed);
  if (!aligned16(ws)) return fail(SALAD_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (ws_bytes < needed)
    return fail(SALAD_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", ws_bytes, needed);
  return SALAD_OK;
}

// Boundary layout [B, N, H, d] read in each head's working order (temporal
// heads gather token st_token(p) for working row p).
View boundary_view(const Geom &g, const void *base) {
  View v;
  v.base = base;
  v.sB = (long long)g.N * g.H * g.D;
  v.sH = g.D;
  v.sN = (long long)g.H * g.D;
  v.perm = 1;
  return v;
}

// Carve the selection scratch: Q means, K means, scores (see select_ws_bytes).
void select_regions(const Geom &g, void *ws, double **qm, double **km, double **sc) {
  const size_t one = up(size_t(g.B) * g.H * g.nb * g.D * sizeof(double));
  char *w = (char *)ws;
  *qm = (double *)w;
  *km = (double *)(w + one);
  *sc = (double *)(w + 2 * one);
}

// Full-width projection ([S] step 4, [C, C] reading): out += olt W_p over
// the B*N token rows, where olt already holds s_b * O_l.
salad_status project_full(const Info &inf, const void *olt, const void *w_p, void *out, hipStream_t st) {
  const Geom &g = inf.g;
  if (const char *m = gemm_rows(inf.bf16, (long long)g.B * g.N, g.H * g.D, olt, w_p, 1.f, out, st))
    return fail(SALAD_ERR_HIP, "salad_attn_forward: projection GEMM: %s", m);
  return SALAD_OK;
}

View working_view(const Geom &g, const void *base) {
  View v;
  v.base = base;
  v.sB = (long long)g.H * g.N * g.D;
  v.sH = (long long)g.N * g.D;
  v.sN = g.D;
  v.perm = 0;
  return v;
}

// Optional caller-created events recorded around the sparse-branch kernels
// (the measurement variants of the forward and backward); NULL: none.
struct Marks {
  hipEvent_t begin = nullptr, end = nullptr;
};

hipError_t mark(hipEvent_t ev, hipStream_t st) { return ev ? hipEventRecord(ev, st) : hipSuccess; }

}  // namespace

extern "C" {

salad_status salad_workspace_size(const salad_problem *p, size_t *bytes) {
  Info inf;
  CHECK(validate(p, &inf));
  if (!bytes) return fail(SALAD_ERR_NULL, "bytes is NULL");
  *bytes = plan(inf).total_forward;
  return SALAD_OK;
}

salad_status salad_permute(const salad_problem *p, int apply_rope, int inverse, const void *src,
                           void *dst, hipStream_t stream) {
  Info inf;
  CHECK(validate(p, &inf));
  CHECK(need(src, "src"));
  CHECK(need(dst, "dst"));
  if (inverse && apply_rope) return fail(SALAD_ERR_SHAPE, "apply_rope needs inverse = 0");
  if (apply_rope && !p->rope) return fail(SALAD_ERR_SHAPE, "apply_rope needs problem->rope = 1 (dims, base)");
  if (src == dst) return fail(SALAD_ERR_SHAPE, "src and dst must not overlap");
  return hip_status(launch_permute(inf.g, inf.bf16, apply_rope, inverse, src, dst, stream), "salad_permute");
}

salad_status salad_block_select(const salad_problem *p, const void *qw, const void *kw, int32_t *idx,
                                double *qbar, double *kbar, void *ws, size_t ws_bytes,
                                hipStream_t stream) {
  Info inf;
  CHECK(validate(p, &inf));
  CHECK(need(qw, "qw"));
  CHECK(need(kw, "kw"));
  CHECK(need(idx, "idx"));
  if (!inf.any_topk) return fail(SALAD_ERR_SHAPE, "no Top-K head in the problem");
  const Geom &g = inf.g;
  CHECK(need_ws(ws, ws_bytes, up(select_ws_bytes(g))));
  if (qbar) CHECK(need(qbar, "qbar"));
  if (kbar) CHECK(need(kbar, "kbar"));
  double *qm, *km, *scores;
  select_regions(g, ws, &qm, &km, &scores);
  if (qbar) qm = qbar;
  if (kbar) km = kbar;
  return hip_status(launch_block_select(g, inf.bf16, working_view(g, qw), working_view(g, kw), qm, km,
                                        scores, idx, stream),
                    "salad_block_select");
}

salad_status salad_sparse_attn(const salad_problem *p, const void *qw, const void *kw, const void *vw,
                               const int32_t *idx, float *o_s, hipStream_t stream) {
  Info inf;
  CHECK(validate(p, &inf));
  CHECK(need(qw, "qw"));
  CHECK(need(kw, "kw"));
  CHECK(need(vw, "vw"));
  CHECK(need(o_s, "o_s"));
  if (inf.any_topk) CHECK(need(idx, "idx"));
  const Geom &g = inf.g;
  return hip_status(launch_sparse_attn(g, inf.bf16, working_view(g, qw), working_view(g, kw),
                                       working_view(g, vw), idx, o_s, stream),
                    "salad_sparse_attn");
}

salad_status salad_linear_state(const salad_problem *p, const void *kw, const void *vw, float *h,
                                float *z, void *ws, size_t ws_bytes, hipStream_t stream) {
  Info inf;
  CHECK(validate(p, &inf));
  CHECK(need(kw, "kw"));
  CHECK(need(vw, "vw"));
  CHECK(need(h, "h"));
  CHECK(need(z, "z"));
  const Geom &g = inf.g;
  const size_t needed = up(size_t(g.B) * g.H * linear_splits(g) * (size_t(g.D) * g.D + g.D) * sizeof(float));
  CHECK(need_ws(ws, ws_bytes, needed));
  return hip_status(launch_linear_state(g, inf.bf16, working_view(g, kw), working_view(g, vw),
                                        (float *)ws, h, z, stream),
                    "salad_linear_state");
}

salad_status salad_linear_state_noalloc(const salad_problem *p, const void *kw, const void *vw, float *h,
                                        float *z, hipStream_t stream) {
  Info inf;
  CHECK(validate(p, &inf));
  CHECK(need(kw, "kw"));
  CHECK(need(vw, "vw"));
  CHECK(need(h, "h"));
  CHECK(need(z, "z"));
  const Geom &g = inf.g;
  const size_t needed = up(size_t(g.B) * g.H * linear_splits(g) * (size_t(g.D) * g.D + g.D) * sizeof(float));
  if (needed > noalloc_scratch_bytes())
    return fail(SALAD_ERR_WORKSPACE,
                "salad_linear_state_noalloc: the split-N partial states need %zu bytes, more than the "
                "library's fixed %zu-byte device scratch (use salad_linear_state with a workspace)",
                needed, noalloc_scratch_bytes());
  void *scratch = nullptr;
  hipError_t e = noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "salad_linear_state_noalloc: scratch address");
  return hip_status(launch_linear_state(g, inf.bf16, working_view(g, kw), working_view(g, vw),
                                        (float *)scratch, h, z, stream),
                    "salad_linear_state_noalloc");
}

salad_status salad_linear_apply(const salad_problem *p, const void *qw, const float *h, const float *z,
                                float *o_l, hipStream_t stream) {
  Info inf;
  CHECK(validate(p, &inf));
  CHECK(need(qw, "qw"));
  CHECK(need(h, "h"));
  CHECK(need(z, "z"));
  CHECK(need(o_l, "o_l"));
  const Geom &g = inf.g;
  return hip_status(launch_linear_apply(g, inf.bf16, working_view(g, qw), h, z, o_l, stream),
                    "salad_linear_apply");
}

salad_status salad_gate(const salad_problem *p, const void *x, const void *w, float bias, float *s,
                        void *ws, size_t ws_bytes, hipStream_t stream) {
  Info inf;
  CHECK(validate(p, &inf));
  CHECK(need(x, "x"));
  CHECK(need(w, "w"));
  CHECK(need(s, "s"));
  const Geom &g = inf.g;
  const size_t needed = up(gate_ws_bytes(g));
  CHECK(need_ws(ws, ws_bytes, needed));
  return hip_status(launch_gate(g, inf.bf16, x, w, bias, ws, s, stream), "salad_gate");
}

salad_status salad_combine(const salad_problem *p, const float *o_s, const float *o_l, const void *w_p,
                           const float *s, void *out, hipStream_t stream) {
  Info inf;
  CHECK(validate(p, &inf));
  CHECK(need(o_s, "o_s"));
  CHECK(need(o_l, "o_l"));
  CHECK(need(w_p, "w_p"));
  CHECK(need(s, "s"));
  CHECK(need(out, "out"));
  if (inf.full)
    return fail(SALAD_ERR_UNSUPPORTED,
                "salad_combine applies the per-head projection only; the full-width projection runs in "
                "salad_attn_forward");
  return hip_status(launch_combine(inf.g, inf.bf16, o_s, o_l, w_p, s, out, stream), "salad_combine");
}

}  // extern "C"

namespace {

salad_status attn_forward(const salad_problem *p, const void *q, const void *k, const void *v, const void *x,
                          const void *w_p, const void *gate_w, float gate_b, const float *s_override, void *out,
                          float *s_out, int32_t *idx_out, float *lse_out, void *ws, size_t ws_bytes,
                          hipStream_t stream, Marks marks) {
  Info inf;
  CHECK(validate(p, &inf));
  CHECK(need(q, "q"));
  CHECK(need(k, "k"));
  CHECK(need(v, "v"));
  CHECK(need(w_p, "w_p"));
  CHECK(need(out, "out"));
  if (!s_override) {
    CHECK(need(x, "x"));
    CHECK(need(gate_w, "gate_w"));
  } else {
    CHECK(need(s_override, "s_override"));
  }
  if (s_out) CHECK(need(s_out, "s_out"));
  if (idx_out) CHECK(need(idx_out, "idx_out"));
  if (lse_out) {
    CHECK(need(lse_out, "lse_out"));
    if (!inf.bf16) return fail(SALAD_ERR_UNSUPPORTED, "lse_out needs bf16 storage (the backward is bf16 only)");
  }
  const Geom &g = inf.g;
  const Plan pl = plan(inf);
  CHECK(need_ws(ws, ws_bytes, pl.total_forward));
  char *w = (char *)ws;
  void *scratch = w;
  void *wq = w + pl.wq, *wk = w + pl.wk, *wv = w + pl.wv;
  int32_t *idx = idx_out ? idx_out : (int32_t *)(w + pl.idx);
  float *o_s = (float *)(w + pl.o_s), *o_l = (float *)(w + pl.o_l);
  float *hm = (float *)(w + pl.h), *zv = (float *)(w + pl.z);
  float *s = s_out ? s_out : (float *)(w + pl.s);

  hipError_t e;
  if (s_override) {
    if (s_out) {
      e = hipMemcpyAsync(s_out, s_override, sizeof(float) * g.B, hipMemcpyDeviceToDevice, stream);
      if (e != hipSuccess) return hip_status(e, "salad_attn_forward: copy s");
    } else {
      s = const_cast<float *>(s_override);
    }
  } else {
    e = launch_gate(g, inf.bf16, x, gate_w, gate_b, scratch, s, stream);
    if (e != hipSuccess) return hip_status(e, "salad_attn_forward: gate");
  }
  const int rope = p->rope;

  if (inf.bf16) {
    // Fused path.  Heads whose working order is the token order (spatial
    // and Top-K) are read in place: their rows of one (b, h) are already
    // contiguous and equally spaced in the [B,N,H,d] layout.  The
    // linear-state pass reads K and V in each head's working order and
    // writes contiguous working copies for the temporal heads only; Q is
    // gathered by the attention kernel itself.  With RoPE, Q and K are
    // rotated first, keeping their layout.  The linear branch, projection,
    // gate and inverse permutation run in the attention epilogue.
    View qv = boundary_view(g, q), kb = boundary_view(g, k), vb = boundary_view(g, v);
    if (rope) {
      double2 *tab = (double2 *)(w + pl.rope_tab);
      if ((e = launch_rope_table(g, tab, stream)) != hipSuccess ||
          (e = launch_rope_rows(g, 1, q, wq, tab, stream)) != hipSuccess ||
          (e = launch_rope_rows(g, 1, k, w + pl.wkr, tab, stream)) != hipSuccess)
        return hip_status(e, "salad_attn_forward: rope");
      qv = boundary_view(g, wq);
      kb = boundary_view(g, w + pl.wkr);
    }
    // in-place rows of non-temporal heads: the boundary views, whose token
    // gather is the identity for those heads
    View kd = kb, vd = vb;
    kd.perm = vd.perm = 0;
    uint64_t work[4];
    const bool direct = kv_direct_ok(g, kd, vd);
    for (int i = 0; i < 4; ++i) work[i] = direct ? g.temporal[i] : ~0ull;
    const View kw = working_view(g, wk), vw = working_view(g, wv);
    bf16_t *hp = (bf16_t *)(w + pl.hp);
    // full-width projection: the finalize leaves W_p and s to the GEMM below
    if ((e = launch_linear_partials(g, kb, vb, (float *)scratch, (bf16_t *)wk, (bf16_t *)wv, work, s,
                                    stream)) != hipSuccess ||
        (e = launch_linear_finalize(g, 1, (const float *)scratch, inf.full ? nullptr : w_p, s, hm, hp, zv,
                                    stream)) != hipSuccess)
      return hip_status(e, "salad_attn_forward: linear state");
    if (inf.any_topk) {
      // Top-K heads are never temporal: their working rows are the token rows
      double *qm, *km, *sc;
      select_regions(g, scratch, &qm, &km, &sc);
      e = launch_block_select(g, 1, qv, kb, qm, km, sc, idx, stream);
      if (e != hipSuccess) return hip_status(e, "salad_attn_forward: block select");
    }
    View outl = boundary_view(g, w + pl.olt);  // s_b * O_l rows (full-width projection only)
    if (!inf.full) outl.base = nullptr;
    if ((e = mark(marks.begin, stream)) != hipSuccess ||
        (e = launch_attn_fused(g, qv, kw, vw, kd, vd, work, idx, hp, zv, s, boundary_view(g, out), outl,
                               lse_out, stream)) != hipSuccess ||
        (e = mark(marks.end, stream)) != hipSuccess)
      return hip_status(e, "salad_attn_forward: attention");
    if (inf.full) return project_full(inf, w + pl.olt, w_p, out, stream);
    return SALAD_OK;
  }

  // f32: staged path through working copies
  double2 *tab = rope ? (double2 *)(w + pl.rope_tab) : nullptr;
  if (rope && (e = launch_rope_table(g, tab, stream)) != hipSuccess)
    return hip_status(e, "salad_attn_forward: rope");
  if ((e = launch_permute(g, inf.bf16, rope, 0, q, wq, stream, tab)) != hipSuccess ||
      (e = launch_permute(g, inf.bf16, rope, 0, k, wk, stream, tab)) != hipSuccess ||
      (e = launch_permute(g, inf.bf16, 0, 0, v, wv, stream)) != hipSuccess)
    return hip_status(e, "salad_attn_forward: permute");
  const View qv = working_view(g, wq), kv = working_view(g, wk), vv = working_view(g, wv);
  if (inf.any_topk) {
    double *qm, *km, *sc;
    select_regions(g, scratch, &qm, &km, &sc);
    e = launch_block_select(g, inf.bf16, qv, kv, qm, km, sc, idx, stream);
    if (e != hipSuccess) return hip_status(e, "salad_attn_forward: block select");
  }
  if ((e = mark(marks.begin, stream)) != hipSuccess ||
      (e = launch_sparse_attn(g, inf.bf16, qv, kv, vv, idx, o_s, stream)) != hipSuccess ||
      (e = mark(marks.end, stream)) != hipSuccess)
    return hip_status(e, "salad_attn_forward: sparse attention");
  if ((e = launch_linear_state(g, inf.bf16, kv, vv, (float *)scratch, hm, zv, stream)) != hipSuccess)
    return hip_status(e, "salad_attn_forward: linear state");
  if ((e = launch_linear_apply(g, inf.bf16, qv, hm, zv, o_l, stream)) != hipSuccess)
    return hip_status(e, "salad_attn_forward: linear apply");
  if (inf.full) {
    if ((e = launch_split_full(g, inf.bf16, o_s, o_l, s, out, w + pl.olt, stream)) != hipSuccess)
      return hip_status(e, "salad_attn_forward: split");
    return project_full(inf, w + pl.olt, w_p, out, stream);
  }
  if ((e = launch_combine(g, inf.bf16, o_s, o_l, w_p, s, out, stream)) != hipSuccess)
    return hip_status(e, "salad_attn_forward: combine");
  return SALAD_OK;
}

}  // namespace

extern "C" {

salad_status salad_attn_forward(const salad_problem *p, const void *q, const void *k, const void *v,
                                const void *x, const void *w_p, const void *gate_w, float gate_b,
                                const float *s_override, void *out, float *s_out, int32_t *idx_out,
                                float *lse_out, void *ws, size_t ws_bytes, hipStream_t stream) {
  return attn_forward(p, q, k, v, x, w_p, gate_w, gate_b, s_override, out, s_out, idx_out, lse_out, ws,
                      ws_bytes, stream, Marks());
}

salad_status salad_attn_forward_timed(const salad_problem *p, const void *q, const void *k, const void *v,
                                      const void *x, const void *w_p, const void *gate_w, float gate_b,
                                      const float *s_override, void *out, float *s_out, int32_t *idx_out,
                                      float *lse_out, void *ws, size_t ws_bytes, hipStream_t stream,
                                      hipEvent_t attn_begin, hipEvent_t attn_end) {
  Marks m;
  m.begin = attn_begin;
  m.end = attn_end;
  return attn_forward(p, q, k, v, x, w_p, gate_w, gate_b, s_override, out, s_out, idx_out, lse_out, ws,
                      ws_bytes, stream, m);
}

salad_status salad_output_projection(const salad_problem *p, const void *in, const void *w_o, void *out,
                                     hipStream_t stream) {
  Info inf;
  CHECK(validate(p, &inf));
  CHECK(need(in, "in"));
  CHECK(need(w_o, "w_o"));
  CHECK(need(out, "out"));
  const Geom &g = inf.g;
  const long long rows = (long long)g.B * g.N;
  const size_t bytes = size_t(rows) * g.H * g.D * inf.esize;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(in), b0 = reinterpret_cast<uintptr_t>(out);
  if (a0 < b0 + bytes && b0 < a0 + bytes) return fail(SALAD_ERR_SHAPE, "in and out must not overlap");
  if (const char *m = gemm_rows(inf.bf16, rows, g.H * g.D, in, w_o, 0.f, out, stream))
    return fail(SALAD_ERR_HIP, "salad_output_projection: %s", m);
  return SALAD_OK;
}

// ---- window calibration ---------------------------------------------------------

namespace {
struct CalibPlan {
  size_t od, ow, part, total;
};
CalibPlan calib_plan(const Info &inf) {
  const Geom &g = inf.g;
  const size_t rows = size_t(g.B) * g.H * g.N;
  CalibPlan pl;
  pl.od = 0;
  pl.ow = up(rows * g.D * sizeof(float));
  pl.part = pl.ow + up(rows * g.D * sizeof(float));
  pl.total = pl.part + up(size_t(g.B) * g.H * calib_splits(g) * 2 * sizeof(double));
  return pl;
}
}  // namespace

salad_status salad_calibrate_workspace_size(const salad_problem *p, size_t *bytes) {
  Info inf;
  CHECK(validate(p, &inf));
  if (!bytes) return fail(SALAD_ERR_NULL, "bytes is NULL");
  *bytes = calib_plan(inf).total;
  return SALAD_OK;
}

salad_status salad_window_calibrate(const salad_problem *p, const void *qw, const void *kw, const void *vw,
                                    const int32_t *radii, int n_radii, float tau, double *err,
                                    int32_t *choice, void *ws, size_t ws_bytes, hipStream_t stream) {
  Info inf;
  CHECK(validate(p, &inf));
  CHECK(need(qw, "qw"));
  CHECK(need(kw, "kw"));
  CHECK(need(vw, "vw"));
  CHECK(need(err, "err"));
  CHECK(need(choice, "choice"));
  if (!radii) return fail(SALAD_ERR_NULL, "radii is NULL");
  if (n_radii < 1 || n_radii > kMaxCalibRadii)
    return fail(SALAD_ERR_SHAPE, "n_radii must be in [1, %d] (got %d)", kMaxCalibRadii, n_radii);
  if (!(tau >= 0.f) || !std::isfinite(tau)) return fail(SALAD_ERR_SHAPE, "tau must be finite and >= 0");
  CalibRadii cr;
  cr.n = n_radii;
  for (int i = 0; i < n_radii; ++i) {
    if (radii[i] < 0 || (i > 0 && radii[i] <= radii[i - 1]))
      return fail(SALAD_ERR_SHAPE, "radii must be >= 0 and strictly ascending");
    cr.r[i] = radii[i];
  }
  const CalibPlan pl = calib_plan(inf);
  CHECK(need_ws(ws, ws_bytes, pl.total));
  // every head as a window head in its working order
  Geom g = inf.g;
  for (int i = 0; i < 4; ++i) g.topk[i] = 0;
  char *w = (char *)ws;
  float *od = (float *)(w + pl.od), *ow = (float *)(w + pl.ow);
  double *part = (double *)(w + pl.part);
  const View qv = working_view(g, qw), kv = working_view(g, kw), vv = working_view(g, vw);
  hipError_t e;
  g.r = g.N - 1;  // dense: every key in every query's window
  if ((e = launch_sparse_attn(g, inf.bf16, qv, kv, vv, nullptr, od, stream)) != hipSuccess)
    return hip_status(e, "salad_window_calibrate: dense attention");
  const size_t slice = size_t(g.B) * g.H;
  for (int i = 0; i < n_radii; ++i) {
    g.r = std::min(radii[i], g.N - 1);
    if ((e = launch_sparse_attn(g, inf.bf16, qv, kv, vv, nullptr, ow, stream)) != hipSuccess ||
        (e = launch_calib_err(g, od, ow, part, err + i * slice, stream)) != hipSuccess)
      return hip_status(e, "salad_window_calibrate: window attention");
  }
  g.r = inf.g.r;
  if ((e = launch_calib_choose(g, cr, tau, err, choice, stream)) != hipSuccess)
    return hip_status(e, "salad_window_calibrate: choice");
  return SALAD_OK;
}

// ---- backward -----------------------------------------------------------------

namespace {

// Backward workspace (bf16, d = 128).  Regions 256-byte aligned: a shared
// scratch (gate partials, then the linear-state and linear-backward split
// partials, and the Top-K means and scores in between), working copies of
// Q, K (rotated), V and dO, lse2 / D, the selection and its inverse lists,
// the per-head linear state and backward matrices, the gate's column sums
// and values, and the RoPE table.
struct BwdPlan {
  size_t wq, wk, wv, wg, wqr, wkr, lse, dsum, idx, inv_off, inv_list, h, z;
  size_t mf, mb, a_red, bz, dhb, dhtb, dwp_h, ds_part, colsum, s, dt, rope_tab;
  int Np;
  size_t total;
};

BwdPlan bwd_plan(const Info &inf) {
  const Geom &g = inf.g;
  BwdPlan pl = {};
  const size_t BH = size_t(g.B) * g.H, D = size_t(g.D);
  const size_t rows = BH * g.N;
  pl.Np = (g.N + 63) / 64 * 64;
  const size_t means = inf.any_topk ? up(select_ws_bytes(g)) : 0;
  const size_t lin = up(BH * linear_splits(g) * (D * D + D) * sizeof(float));
  const size_t gate = up(gate_ws_bytes(g));
  size_t off = std::max(means, std::max(lin, gate));
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += up(bytes);
    return at;
  };
  pl.wq = take(rows * D * 2);
  pl.wk = take(rows * D * 2);
  pl.wv = take(rows * D * 2);
  pl.wg = take(rows * D * 2);
  pl.wqr = take(inf.rope ? rows * D * 2 : 0);  // rotated Q, K in the boundary layout
  pl.wkr = take(inf.rope ? rows * D * 2 : 0);
  pl.lse = take(BH * pl.Np * sizeof(float));
  pl.dsum = take(BH * pl.Np * sizeof(float));
  pl.idx = take(inf.any_topk ? BH * g.nb * g.k * sizeof(int32_t) : 0);
  pl.inv_off = take(inf.any_topk ? BH * (g.nb + 1) * sizeof(int32_t) : 0);
  pl.inv_list = take(inf.any_topk ? BH * g.nb * g.k * sizeof(int32_t) : 0);
  pl.h = take(BH * D * D * sizeof(float));
  pl.z = take(BH * D * sizeof(float));
  pl.mf = take(BH * D * D * sizeof(float));
  pl.mb = take(BH * D * D * 2);
  pl.a_red = take(BH * D * D * sizeof(float));
  pl.bz = take(BH * D * sizeof(float));
  pl.dhb = take(BH * D * D * 2);
  pl.dhtb = take(BH * D * D * 2);
  pl.dwp_h = take(BH * D * D * sizeof(float));
  pl.ds_part = take(BH * 16 * sizeof(float));
  pl.colsum = take(size_t(g.B) * gate_bwd_splits(g) * g.H * D * sizeof(float));
  pl.s = take(size_t(g.B) * sizeof(float));
  pl.dt = take(size_t(g.B) * sizeof(float));
  pl.rope_tab = take(inf.rope ? size_t(rope_table_entries(g)) * 16 : 0);
  pl.total = off;
  return pl;
}

salad_status validate_backward(const salad_problem *p, Info *inf) {
  CHECK(validate(p, inf));
  if (!inf->bf16)
    return fail(SALAD_ERR_UNSUPPORTED, "salad_attn_backward is built for bf16 storage (d = 128) only");
  if (inf->full)
    return fail(SALAD_ERR_UNSUPPORTED, "salad_attn_backward supports the per-head projection (SALAD_PROJ_HEAD) only");
  return SALAD_OK;
}

}  // namespace

salad_status salad_backward_workspace_size(const salad_problem *p, size_t *bytes) {
  Info inf;
  CHECK(validate_backward(p, &inf));
  if (!bytes) return fail(SALAD_ERR_NULL, "bytes is NULL");
  *bytes = bwd_plan(inf).total;
  return SALAD_OK;
}

}  // extern "C"

namespace {

salad_status attn_backward(const salad_problem *p, const void *q, const void *k, const void *v, const void *x,
                           const void *w_p, const void *gate_w, float gate_b, const float *s_override,
                           const void *dout, const void *out_saved, const float *lse_saved, void *dq, void *dk,
                           void *dv, float *dw_p, void *dx, float *dgate_w, float *dgate_b, float *ds_out,
                           void *ws, size_t ws_bytes, hipStream_t stream, Marks marks) {
  Info inf;
  CHECK(validate_backward(p, &inf));
  CHECK(need(q, "q"));
  CHECK(need(k, "k"));
  CHECK(need(v, "v"));
  CHECK(need(w_p, "w_p"));
  CHECK(need(dout, "dout"));
  CHECK(need(dq, "dq"));
  CHECK(need(dk, "dk"));
  CHECK(need(dv, "dv"));
  CHECK(need(dw_p, "dw_p"));
  const int has_gate = s_override == nullptr;
  if (has_gate) {
    CHECK(need(x, "x"));
    CHECK(need(gate_w, "gate_w"));
    if (dx) CHECK(need(dx, "dx"));
    if (dgate_w) CHECK(need(dgate_w, "dgate_w"));
    if (dgate_b && (reinterpret_cast<uintptr_t>(dgate_b) & 3u))
      return fail(SALAD_ERR_ALIGN, "dgate_b is not 4-byte aligned");
  } else {
    CHECK(need(s_override, "s_override"));
  }
  if (ds_out) CHECK(need(ds_out, "ds_out"));
  const bool saved = out_saved || lse_saved;
  if (saved) {
    CHECK(need(out_saved, "out_saved"));
    CHECK(need(lse_saved, "lse_saved"));
  }
  const Geom &g = inf.g;
  const BwdPlan pl = bwd_plan(inf);
  CHECK(need_ws(ws, ws_bytes, pl.total));
  char *w = (char *)ws;
  void *scratch = w;
  bf16_t *wq = (bf16_t *)(w + pl.wq), *wk = (bf16_t *)(w + pl.wk), *wv = (bf16_t *)(w + pl.wv),
         *wg = (bf16_t *)(w + pl.wg);
  float *lse = (float *)(w + pl.lse), *dsum = (float *)(w + pl.dsum);
  int32_t *idx = (int32_t *)(w + pl.idx);
  float *hm = (float *)(w + pl.h), *zv = (float *)(w + pl.z);
  float *s = (float *)(w + pl.s);
  double2 *tab = inf.rope ? (double2 *)(w + pl.rope_tab) : nullptr;
  hipError_t e;

  // gate values (and X's column sums for dL/dw)
  if (has_gate) {
    if ((e = launch_gate(g, 1, x, gate_w, gate_b, scratch, s, stream)) != hipSuccess ||
        (e = launch_gate_colsum(g, (const bf16_t *)x, (float *)(w + pl.colsum), stream)) != hipSuccess)
      return hip_status(e, "salad_attn_backward: gate");
  } else if ((e = hipMemcpyAsync(s, s_override, sizeof(float) * g.B, hipMemcpyDeviceToDevice, stream)) !=
             hipSuccess) {
    return hip_status(e, "salad_attn_backward: copy s");
  }
  // Q and K rotated first (boundary layout) when RoPE is on.  Heads whose
  // working order is the token order are then read in place; the temporal
  // heads get working copies: Q and dO from the permute, K and V from the
  // linear-state pass, which reads every head's K and V anyway.
  const void *qsrc = q, *ksrc = k;
  if (inf.rope) {
    if ((e = launch_rope_table(g, tab, stream)) != hipSuccess ||
        (e = launch_rope_rows(g, 1, q, w + pl.wqr, tab, stream)) != hipSuccess ||
        (e = launch_rope_rows(g, 1, k, w + pl.wkr, tab, stream)) != hipSuccess)
      return hip_status(e, "salad_attn_backward: rope");
    qsrc = w + pl.wqr;
    ksrc = w + pl.wkr;
  }
  const View qb = boundary_view(g, qsrc), kb = boundary_view(g, ksrc), vb = boundary_view(g, v);
  View kd = kb, vd = vb;
  kd.perm = vd.perm = 0;
  uint64_t work[4];
  const bool direct = kv_direct_ok(g, kd, vd);
  for (int i = 0; i < 4; ++i) work[i] = direct ? g.temporal[i] : ~0ull;
  bool any_work = false;
  for (int i = 0; i < 4; ++i) any_work |= work[i] != 0;
  if (any_work && ((e = launch_permute(g, 1, 0, 0, qsrc, wq, stream, nullptr, work)) != hipSuccess ||
                   (e = launch_permute(g, 1, 0, 0, dout, wg, stream, nullptr, work)) != hipSuccess))
    return hip_status(e, "salad_attn_backward: permute");
  const View kv = working_view(g, wk), vv = working_view(g, wv);
  if ((e = launch_linear_partials(g, kb, vb, (float *)scratch, wk, wv, work, nullptr, stream)) != hipSuccess ||
      (e = launch_linear_reduce(g, linear_splits(g), (const float *)scratch, hm, zv, stream)) != hipSuccess)
    return hip_status(e, "salad_attn_backward: linear state");
  int32_t *inv_off = nullptr, *inv_list = nullptr;
  if (inf.any_topk) {
    // Top-K heads are never temporal: their working rows are the token rows
    double *qm, *km, *sc;
    select_regions(g, scratch, &qm, &km, &sc);
    inv_off = (int32_t *)(w + pl.inv_off);
    inv_list = (int32_t *)(w + pl.inv_list);
    if ((e = launch_block_select(g, 1, qb, kb, qm, km, sc, idx, stream)) != hipSuccess ||
        (e = launch_topk_inverse(g, idx, inv_off, inv_list, stream)) != hipSuccess)
      return hip_status(e, "salad_attn_backward: block select");
  }
  // linear branch and projection: whole-head sums (M, A, dZ, dH, dW_p, ds)
  LinBwdScratch lw;
  lw.mf = (float *)(w + pl.mf);
  lw.mb = (bf16_t *)(w + pl.mb);
  lw.partial = (float *)scratch;
  lw.a_red = (float *)(w + pl.a_red);
  lw.bz = (float *)(w + pl.bz);
  lw.dhb = (bf16_t *)(w + pl.dhb);
  lw.dhtb = (bf16_t *)(w + pl.dhtb);
  lw.dwp_h = (float *)(w + pl.dwp_h);
  lw.ds_part = (float *)(w + pl.ds_part);
  // with the forward's output and normalisers, D comes from the linear
  // pass and the normalisers are copied into the padded rows; otherwise the
  // forward's sparse branch is recomputed below
  View outv = boundary_view(g, out_saved);
  if (!saved) outv.base = nullptr;
  if (saved && (e = hipMemcpy2DAsync(lse, size_t(pl.Np) * sizeof(float), lse_saved, size_t(g.N) * sizeof(float),
                                     size_t(g.N) * sizeof(float), size_t(g.B) * g.H, hipMemcpyDeviceToDevice,
                                     stream)) != hipSuccess)
    return hip_status(e, "salad_attn_backward: copy lse");
  if ((e = launch_linear_bwd(g, wq, wg, (const bf16_t *)qsrc, (const bf16_t *)dout, work, hm, zv,
                             (const bf16_t *)w_p, s, lw, dw_p, outv, dsum, pl.Np, stream)) != hipSuccess)
    return hip_status(e, "salad_attn_backward: linear branch");
  // sparse branch (normalisers and D, then dQ and dK, dV, whose epilogues add
  // the linear branch's per-row terms and write the final rows)
  BwdOut bo;
  bo.mb = lw.mb;
  bo.dhb = lw.dhb;
  bo.dhtb = lw.dhtb;
  bo.zv = zv;
  bo.dz = lw.bz;
  bo.s_gate = s;
  bo.rope_tab = tab;
  bo.dq = (bf16_t *)dq;
  bo.dk = (bf16_t *)dk;
  bo.dv = (bf16_t *)dv;
  if ((!saved && (e = launch_attn_bwd_prep(g, qb, kv, vv, kd, vd, work, idx, wg, (const bf16_t *)dout, lse,
                                          dsum, pl.Np, stream)) != hipSuccess) ||
      (e = mark(marks.begin, stream)) != hipSuccess ||
      (e = launch_attn_bwd(g, wq, wk, wv, wg, (const bf16_t *)qsrc, (const bf16_t *)ksrc, (const bf16_t *)v,
                           (const bf16_t *)dout, work, lse, dsum, pl.Np, idx, inv_off, inv_list, bo, stream)) !=
          hipSuccess ||
      (e = mark(marks.end, stream)) != hipSuccess)
    return hip_status(e, "salad_attn_backward: sparse attention");
  // gate
  float *dt = (float *)(w + pl.dt);
  if ((e = launch_gate_bwd(g, lw.ds_part, s, has_gate, (const float *)(w + pl.colsum), dt, ds_out,
                           has_gate ? dgate_w : nullptr, has_gate ? dgate_b : nullptr, stream)) != hipSuccess ||
      (has_gate && dx && (e = launch_gate_dx(g, dt, (const bf16_t *)gate_w, (bf16_t *)dx, stream)) != hipSuccess))
    return hip_status(e, "salad_attn_backward: gate");
  return SALAD_OK;
}

}  // namespace

extern "C" {

salad_status salad_attn_backward(const salad_problem *p, const void *q, const void *k, const void *v,
                                 const void *x, const void *w_p, const void *gate_w, float gate_b,
                                 const float *s_override, const void *dout, const void *out_saved,
                                 const float *lse_saved, void *dq, void *dk, void *dv, float *dw_p, void *dx,
                                 float *dgate_w, float *dgate_b, float *ds_out, void *ws, size_t ws_bytes,
                                 hipStream_t stream) {
  return attn_backward(p, q, k, v, x, w_p, gate_w, gate_b, s_override, dout, out_saved, lse_saved, dq, dk, dv,
                       dw_p, dx, dgate_w, dgate_b, ds_out, ws, ws_bytes, stream, Marks());
}

salad_status salad_attn_backward_timed(const salad_problem *p, const void *q, const void *k, const void *v,
                                       const void *x, const void *w_p, const void *gate_w, float gate_b,
                                       const float *s_override, const void *dout, const void *out_saved,
                                       const float *lse_saved, void *dq, void *dk, void *dv, float *dw_p,
                                       void *dx, float *dgate_w, float *dgate_b, float *ds_out, void *ws,
                                       size_t ws_bytes, hipStream_t stream, hipEvent_t attn_begin,
                                       hipEvent_t attn_end) {
  Marks m;
  m.begin = attn_begin;
  m.end = attn_end;
  return attn_backward(p, q, k, v, x, w_p, gate_w, gate_b, s_override, dout, out_saved, lse_saved, dq, dk, dv,
                       dw_p, dx, dgate_w, dgate_b, ds_out, ws, ws_bytes, stream, m);
}

const char *salad_last_error(void) { return g_err.c_str(); }

}  // extern "C"
