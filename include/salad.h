/*
 * salad.h -- C ABI of the MI355X (gfx950) hybrid attention library.
 *
 * One attention layer of SALAD (arXiv 2601.16515): a high-sparsity branch
 * (sliding-window attention over head-wise token-permuted sequences, or
 * Top-K block-sparse attention) and a ReLU linear-attention branch on the
 * same Q/K/V, combined as  out = O_s + s * (O_l W_p)  with the gate
 * s = sigmoid(w . mean_tokens(X) + b).
 *
 * Sources, cited by tag and section:
 *  [S] "SALAD: Achieve High-Sparsity Attention via Efficient Linear
 *      Attention Tuning for Video Diffusion Transformer" -- structured
 *      summary, paper.rainbus.top/paper/2601.16515: Prerequisites >
 *      Sparse Attention, Linear Attention; Method step details, steps 1-8.
 *  [I] ijyty.com/news/870645 (sparse attention in video diffusion
 *      models): 1.1 ST sliding window and head-wise token re-ordering,
 *      1.2 Top-K block-sparse attention, 2.3 gate, 4.1 fixed gates.
 *  [A] news.axiwang.com/a/172924.html: section 六 (technical details).
 *  [G] gist.science/fr/paper/2601.16515: section 2 (Méthodologie).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Shapes: B batch, N = F*Hg*Wg tokens (frame-major: token
 *  n = f*Hg*Wg + y*Wg + x), H heads, d head dim (64 or 128), C = H*d.
 *  Boundary layout [B, N, H, d] row-major: one (token, head) row is d
 *  contiguous elements.  X is [B, N, C].
 *  Working layout [B, H, N, d]: row p of head h holds token pi_h(p), where
 *  pi_h is the identity for spatial and Top-K heads and, for temporal heads,
 *  pi(p) = (p mod F)*Hg*Wg + floor(p/F) (sites row-major, frames fastest;
 *  [I] 1.1).
 *  Storage type (io_dtype) applies to Q, K, V, X, W_p, gate w and out:
 *  SALAD_F32 (float) or SALAD_BF16 (bfloat16 bits, uint16).  Stage results
 *  O_s, O_l, H, Z and s are float32; block means are float64.
 *
 *  Ownership: every buffer is allocated and freed by the caller.  Device
 *  pointers must be 16-byte aligned and contiguous in the stated layout.
 *  Scratch memory comes only from the caller's workspace (ws, ws_bytes),
 *  sized by salad_workspace_size, and the library keeps no pointer after a
 *  call returns.  The library allocates no device memory and creates no
 *  handles or streams.
 *
 *  Execution: calls enqueue kernels on `stream` and return without
 *  synchronising.  Results are deterministic (no floating-point atomics).
 *
 *  Errors: every argument is validated before anything is enqueued.  On a
 *  non-OK status nothing was launched and no output was touched;
 *  salad_last_error() gives a thread-local message.  SALAD_ERR_HIP reports
 *  a failed launch; device faults surface at the caller's next sync.
 *  NaN/Inf inputs propagate.
 */
#ifndef SALAD_H
#define SALAD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SALAD_OK = 0,
  SALAD_ERR_NULL = 1,        /* a required pointer is NULL                   */
  SALAD_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes           */
  SALAD_ERR_UNSUPPORTED = 3, /* valid but not built (e.g. d not in {64,128}) */
  SALAD_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned      */
  SALAD_ERR_WORKSPACE = 5,   /* ws NULL or ws_bytes below the required size  */
  SALAD_ERR_HIP = 6          /* a kernel launch failed                       */
} salad_status;

typedef enum { SALAD_F32 = 0, SALAD_BF16 = 1 } salad_dtype;

enum { SALAD_HEAD_SPATIAL = 0, SALAD_HEAD_TEMPORAL = 1, SALAD_HEAD_TOPK = 2 };

/* Shape of the static projection W_p of the linear branch ([S] step 4):
 * one [d, d] matrix shared by the heads (each head's linear output row times
 * W_p), or one [C, C] matrix over a token's linear outputs concatenated in
 * head order (the reading that matches the extra parameter count of about
 * 5 % that [S] reports). */
enum { SALAD_PROJ_HEAD = 0, SALAD_PROJ_FULL = 1 };

#define SALAD_MAX_HEADS 256

/* The layer's problem statement ([S] method steps 2-6, [I] 1.1-1.2). */
typedef struct {
  int32_t batch;                      /* B >= 1                                   */
  int32_t n_heads;                    /* H in [1, SALAD_MAX_HEADS]                */
  int32_t head_dim;                   /* d in {64, 128}                           */
  int32_t grid_f, grid_h, grid_w;     /* latent F x Hg x Wg; N = F*Hg*Wg <= 2^28
                                         (bf16: N < 2^24), B*H*N < 2^31 rows,
                                         B*H*N*d <= 2^40                         */
  uint8_t head_kind[SALAD_MAX_HEADS]; /* per head: SALAD_HEAD_* (first H used)    */
  int32_t window_radius;              /* window heads keep key j iff |p-j| <= r;
                                         r >= N-1 acts as N-1 (dense)            */
  int32_t block;                      /* Top-K block size (queries and keys)      */
  int32_t topk;                       /* Top-K: key blocks kept per query block   */
  float softmax_scale;                /* <= 0 selects 1/sqrt(d)                   */
  float linear_eps;                   /* linear denominator guard (1e-6 typical)  */
  int32_t rope;                       /* 1: 3D RoPE on Q and K before both branches */
  int32_t rope_dims[3];               /* frame/height/width segment sizes, even, sum d */
  float rope_base;                    /* rotary base (10000)                      */
  int32_t io_dtype;                   /* salad_dtype                              */
  float branch_drop_tau;              /* post-tuning branch dropping ([G] 2 C, [S]
                                         step 8): a sample whose gate value s_b is
                                         below it keeps only the sparse branch
                                         (out = O_s) and its linear-branch work is
                                         skipped; 0 never drops (s_b > 0); finite */
  int32_t proj_mode;                  /* SALAD_PROJ_HEAD or SALAD_PROJ_FULL        */
} salad_problem;

/* Bytes of workspace that any entry point below except salad_attn_backward
 * and salad_window_calibrate may need for problem *p (the largest over
 * them); those two have their own sizes (salad_backward_workspace_size,
 * salad_calibrate_workspace_size).  Errors: NULL, SHAPE, UNSUPPORTED. */
salad_status salad_workspace_size(const salad_problem *p, size_t *bytes);

/* Head-wise token permutation ([I] 1.1), optionally with 3D RoPE ([S] step 3,
 * [A] 六).  inverse = 0: src [B,N,H,d] (boundary) -> dst [B,H,N,d] (working);
 * with apply_rope = 1 each row is rotated by its token's (f, y, x) position
 * before the store: pair (2i, 2i+1) of an axis segment of D dims turns by
 * pos * rope_base^(-2i/D), computed in float64 and rounded once to the
 * storage type.  inverse = 1: src working -> dst boundary (apply_rope must
 * be 0).  Element type: io_dtype.  src and dst must not overlap. */
salad_status salad_permute(const salad_problem *p, int apply_rope, int inverse,
                           const void *src, void *dst, hipStream_t stream);

/* Top-K block selection ([I] 1.2, first two steps).  For every Top-K head:
 * block means of the working Q and K over blocks of p->block rows (the last
 * block averages its valid rows), accumulated in float64; score of key block
 * kb for query block qb = qbar[qb] . kbar[kb] in float64; keep the p->topk
 * highest, equal scores resolved toward the lower block index; write them
 * ascending to idx [B, H, nb, topk] (int32, nb = ceil(N/block)).  Rows of
 * non-Top-K heads are not written.  qbar/kbar (float64 [B,H,nb,d]) also
 * receive the means when non-NULL.  The workspace (salad_workspace_size)
 * holds the means and the float64 block scores. */
salad_status salad_block_select(const salad_problem *p, const void *qw, const void *kw,
                                int32_t *idx, double *qbar, double *kbar,
                                void *ws, size_t ws_bytes, hipStream_t stream);

/* Sparse branch ([S] Prerequisites > Sparse Attention; [I] 1.1, 1.2):
 * o_s[b,h,p,:] = sum_{j in S(p)} softmax_j(scale * q_p . k_j) v_j over the
 * working rows, with S(p) = {j : |p-j| <= r} for window heads and the rows
 * of the key blocks idx[b,h,p/block,:] for Top-K heads.  qw, kw, vw working
 * layout in io_dtype; o_s float32 working layout.  idx may be NULL when no
 * head is Top-K. */
salad_status salad_sparse_attn(const salad_problem *p, const void *qw, const void *kw,
                               const void *vw, const int32_t *idx, float *o_s,
                               hipStream_t stream);

/* Linear-attention state ([S] Prerequisites > Linear Attention):
 * h[b,h] = relu(K)^T V  (float32 [B,H,d,d], h[i][j] = sum_n relu(k_n[i]) v_n[j])
 * and z[b,h] = relu(K)^T 1 (float32 [B,H,d]) over all N tokens.  kw, vw are
 * working layout (the sums ignore token order).  Split over N with a
 * fixed-order reduction through the workspace. */
salad_status salad_linear_state(const salad_problem *p, const void *kw, const void *vw,
                                float *h, float *z, void *ws, size_t ws_bytes,
                                hipStream_t stream);

/* salad_linear_state without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops and harnesses
 * that forbid allocation): identical arguments and results, except that the
 * split-N partial states live in a fixed 36 MiB device array inside the
 * library (one per GPU, kept until the process ends) instead of ws.  It
 * allocates nothing.  Problems whose partial states need more than 36 MiB
 * (B*H above about 570 at d = 128) are rejected with SALAD_ERR_WORKSPACE.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * device (other streams or threads) race and must be serialised by the
 * caller.  The first call on a device looks the array's address up
 * (SALAD_ERR_HIP if that fails).  Errors otherwise as salad_linear_state. */
salad_status salad_linear_state_noalloc(const salad_problem *p, const void *kw, const void *vw,
                                        float *h, float *z, hipStream_t stream);

/* Linear-attention output ([S] Prerequisites > Linear Attention):
 * o_l[b,h,p,:] = relu(q_p)^T H / (relu(q_p) . Z + linear_eps), working layout,
 * float32 out. */
salad_status salad_linear_apply(const salad_problem *p, const void *qw, const float *h,
                                const float *z, float *o_l, hipStream_t stream);

/* Gate ([S] step 5, [I] 2.3, [A] 六): s[b] = sigmoid(w . mean_n X[b,n,:] + bias),
 * X [B,N,C] and w [C] in io_dtype, s float32 [B] on the device. */
salad_status salad_gate(const salad_problem *p, const void *x, const void *w, float bias,
                        float *s, void *ws, size_t ws_bytes, hipStream_t stream);

/* Combine ([S] steps 4 and 6): out[b, pi_h(p), h, :] =
 * o_s[b,h,p,:] + s[b] * (o_l[b,h,p,:] W_p), W_p [d_in, d_out] row-major in
 * io_dtype, shared by all heads, no bias.  o_s, o_l float32 working layout;
 * s float32 [B] device; out boundary layout in io_dtype.  A sample with
 * s_b < p->branch_drop_tau gets out = O_s (branch dropping, [G] 2 C).
 * SALAD_PROJ_HEAD only (the full-width projection mixes heads and runs
 * inside salad_attn_forward); SALAD_ERR_UNSUPPORTED otherwise. */
salad_status salad_combine(const salad_problem *p, const float *o_s, const float *o_l,
                           const void *w_p, const float *s, void *out, hipStream_t stream);

/* Whole layer ([S] steps 2-6, and step 8 through p->branch_drop_tau): q, k,
 * v [B,N,H,d], x [B,N,C], w_p ([d,d] for SALAD_PROJ_HEAD, [C,C] for
 * SALAD_PROJ_FULL), gate_w [C] in io_dtype -> out [B,N,H,d] in io_dtype.
 * With SALAD_PROJ_FULL, out[b,n,:] = O_s[b,n,:] + s_b * (O_l[b,n,:] W_p) over
 * the token's C-wide rows; the [B*N, C] x [C, C] product runs as one GEMM
 * kernel (float32 accumulation) on `stream`, accumulating into out; the
 * workspace then also holds s_b * O_l in token rows (B*N*C io_dtype
 * elements, zero for dropped samples).
 * s_override (device float [B]) replaces the gate when non-NULL; s_out
 * (device float [B]) and idx_out ([B,H,nb,topk] int32, Top-K heads only)
 * receive the gate values (before any dropping) and the block selection
 * when non-NULL.  A sample with s_b < branch_drop_tau gets
 * out = O_s; the decision is taken on the device, so nothing synchronises.
 * lse_out (device float [B,H,N], optional, bf16 storage only): for each
 * working row of each head, log2 of its sparse-branch softmax normaliser
 * in units of scale*log2(e) scores, to be handed to salad_attn_backward
 * with out.  Workspace: salad_workspace_size. */
salad_status salad_attn_forward(const salad_problem *p, const void *q, const void *k,
                                const void *v, const void *x, const void *w_p,
                                const void *gate_w, float gate_b, const float *s_override,
                                void *out, float *s_out, int32_t *idx_out, float *lse_out,
                                void *ws, size_t ws_bytes, hipStream_t stream);

/* Backward of salad_attn_forward (head-wise projection, bf16 storage,
 * d = 128): the gradients of L = sum(dout * out) that fine-tuning the
 * layer needs ([S] steps 4-5 and the training configuration under
 * 复现评估; [G] 2 A-B).  The pages print no backward; it is the forward's
 * derivative, with these readings: the storage rounding of the rotated Q
 * and K passes gradients unchanged; relu'(0) = 0; the Top-K selection is
 * held fixed (recomputed from Q and K exactly as the forward does); a
 * sample with s_b < branch_drop_tau gets no gradient through its linear
 * branch, W_p or the gate; with s_override the gate is not differentiated.
 *
 * Inputs as for salad_attn_forward, plus dout [B,N,H,d] (bf16) and,
 * optionally, the forward's out and lse_out for the same inputs (out_saved,
 * lse_saved; both or neither): with them the sparse branch's normalisers
 * are reused and D = dO . O_s comes from out (O_s = out - s_b O_l W_p);
 * without them the forward's sparse branch is recomputed.  Outputs:
 * dq, dk, dv [B,N,H,d] bf16 (w.r.t. the unrotated Q, K); dw_p [d,d] float32;
 * when the gate is computed (s_override NULL): dx [B,N,C] bf16, dgate_w [C]
 * and dgate_b [1] float32, each optional (NULL: not written); ds_out [B]
 * float32 (optional): dL/ds_b.  Sums over rows and heads run in a fixed
 * order (no atomics): results are deterministic.  Workspace:
 * salad_backward_workspace_size.  Errors as above; SALAD_ERR_UNSUPPORTED for
 * f32 storage or SALAD_PROJ_FULL. */
salad_status salad_backward_workspace_size(const salad_problem *p, size_t *bytes);
salad_status salad_attn_backward(const salad_problem *p, const void *q, const void *k,
                                 const void *v, const void *x, const void *w_p,
                                 const void *gate_w, float gate_b, const float *s_override,
                                 const void *dout, const void *out_saved, const float *lse_saved,
                                 void *dq, void *dk, void *dv, float *dw_p, void *dx,
                                 float *dgate_w, float *dgate_b, float *ds_out, void *ws,
                                 size_t ws_bytes, hipStream_t stream);

/* Per-head window calibration ([I] 1.1): for every head of the problem,
 * evaluated as a window head in its working order (Top-K heads in token
 * order), the relative squared error of window attention against dense
 * attention for each candidate radius:
 *   err[i][b][h] = ||O_window(radii[i]) - O_dense||_F^2 / ||O_dense||_F^2
 * over the head's N rows of sample b (float64, device, [n_radii][B][H]),
 * and choice[h] (int32, device, [H]) = the smallest radii[i] with
 * max_b err[i][b][h] <= tau, or N - 1 (the dense window) when none is.
 * The batch entries are the calibration samples.  qw, kw, vw in working
 * layout, io_dtype.  radii: host array, 1 <= n_radii <= 64, strictly
 * ascending, >= 0 (radii past N - 1 act as N - 1).  tau >= 0 (the pages
 * use 2.0).  window_radius, block and topk of *p are ignored.  Workspace:
 * salad_calibrate_workspace_size.  Errors: NULL, ALIGN, SHAPE, WORKSPACE,
 * UNSUPPORTED, HIP. */
salad_status salad_calibrate_workspace_size(const salad_problem *p, size_t *bytes);
salad_status salad_window_calibrate(const salad_problem *p, const void *qw, const void *kw,
                                    const void *vw, const int32_t *radii, int n_radii, float tau,
                                    double *err, int32_t *choice, void *ws, size_t ws_bytes,
                                    hipStream_t stream);

/* Output projection ([S] step 7): out[b,n,:] = in[b,n,:] W_o, a row vector
 * times W_o [C, C] row-major, no bias; in, out [B, N, C] (equivalently
 * [B,N,H,d]) and W_o in io_dtype.  One GEMM kernel, float32 accumulation.
 * in and out must not overlap.  Errors: NULL, ALIGN, SHAPE, HIP. */
salad_status salad_output_projection(const salad_problem *p, const void *in, const void *w_o,
                                     void *out, hipStream_t stream);

/* Measurement variants of salad_attn_forward and salad_attn_backward, for
 * callers that time the sparse-branch kernels on their own stream (the
 * forward's attention kernel(s); the backward's dQ, then dK and dV kernels):
 * identical arguments and results, and in addition the caller-created
 * events attn_begin and attn_end (either may be NULL) are recorded on
 * `stream` immediately before the first and after the last of those
 * kernels.  The library keeps no state and creates or waits for no event.
 * Errors as for the plain calls; a failed event record is SALAD_ERR_HIP. */
salad_status salad_attn_forward_timed(const salad_problem *p, const void *q, const void *k,
                                      const void *v, const void *x, const void *w_p,
                                      const void *gate_w, float gate_b, const float *s_override,
                                      void *out, float *s_out, int32_t *idx_out, float *lse_out,
                                      void *ws, size_t ws_bytes, hipStream_t stream,
                                      hipEvent_t attn_begin, hipEvent_t attn_end);
salad_status salad_attn_backward_timed(const salad_problem *p, const void *q, const void *k,
                                       const void *v, const void *x, const void *w_p,
                                       const void *gate_w, float gate_b, const float *s_override,
                                       const void *dout, const void *out_saved,
                                       const float *lse_saved, void *dq, void *dk, void *dv,
                                       float *dw_p, void *dx, float *dgate_w, float *dgate_b,
                                       float *ds_out, void *ws, size_t ws_bytes,
                                       hipStream_t stream, hipEvent_t attn_begin,
                                       hipEvent_t attn_end);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *salad_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SALAD_H */
