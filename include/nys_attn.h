/*
 * nys_attn.h - C ABI of the MI355X (gfx950) Nystrom self-attention forward.
 *
 * Operation (review page "Nystromformer: A Nystrom-Based Algorithm for Approximating
 * Self-Attention", section "Proposed method"): for every (batch b, head h) with
 * Q, K, V in R^{n x d} and s = 1/sqrt(d),
 *
 *   Qt, Kt  = segment means of Q, K over m contiguous segments (token t in segment
 *             floor(t m / n): rows [ceil(j n / m), ceil((j+1) n / m)) form segment j)
 *   F       = softmax_row(s Q Kt^T)          (n x m)
 *   A_S     = softmax_row(s Qt Kt^T)         (m x m)
 *   Bbar    = softmax_row(s Qt K^T)          (m x n)
 *   Z       = pinv_iters steps of Z <- 1/4 Z (13I - X(15I - X(7I - X))), X = A_S Z,
 *             from Z_0 = A_S^T / (||A_S||_1 ||A_S||_inf)   (approximates A_S^+)
 *   out     = F (Z (Bbar V)) + dwconv(V)
 *
 * where dwconv(V)[t, :] = sum_{k<W} w[h][k] V[t + k - (W-1)/2, :] with V = 0 outside
 * [0, n) (a depthwise convolution along the sequence, one filter per head shared by
 * the d features). The n x n matrices are never formed: time and memory are linear in
 * n (page, "Main findings").
 *
 * Conventions for every entry point:
 *  - All functions return a status; nothing throws across this boundary. On failure,
 *    nys_attn_last_error() returns a thread-local description of the last error.
 *  - Arguments are validated on the host before any HIP call.
 *  - Device pointers are plain device addresses (hipMalloc or equivalent) on the
 *    device that was current when the plan was created. The caller owns every tensor.
 */
#ifndef NYS_ATTN_H
#define NYS_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque plan: holds the shapes and the device workspace of one problem size. */
typedef struct nys_attn_plan nys_attn_plan;

/* Element type of q, k, v and out. A C caller may pass any int; the library validates
 * it. Compiled as C++ the enum gets a fixed int underlying type (the same size and ABI
 * as the C enum), so every int value is a valid nys_dtype there as well. */
#ifdef __cplusplus
typedef enum nys_dtype_e : int { NYS_F32 = 0, NYS_BF16 = 1 } nys_dtype;
#else
typedef enum { NYS_F32 = 0, NYS_BF16 = 1 } nys_dtype;
#endif

typedef enum {
  NYS_OK = 0,
  NYS_E_ARG = 1,         /* invalid argument (null pointer, bad shape, misalignment) */
  NYS_E_UNSUPPORTED = 2, /* valid but not built: d not in {32,64,128}, m > 256, ...      */
  NYS_E_NOMEM = 3,       /* device workspace allocation failed                         */
  NYS_E_DEVICE = 4,      /* no HIP device, or the current device is not gfx950          */
  NYS_E_LAUNCH = 5       /* a kernel launch or a HIP runtime call failed                */
} nys_status;

/* Optional fp32 device buffers filled by nys_attn_forward_debug; each may be NULL.
 * Layouts (row-major, BH = B*H, heads in b-major order):
 *   q_land, k_land : [BH][m][d]   segment means Qt, Kt
 *   a_s, z         : [BH][m][m]   landmark kernel A_S and its iterative inverse Z
 *   w              : [BH][m][d]   Bbar V
 *   y              : [BH][m][d]   Z (Bbar V)
 *   attn           : [BH][n][d]   F Y, the attention part without the conv skip   */
typedef struct {
  float *q_land, *k_land, *a_s, *z, *w, *y, *attn;
} nys_attn_taps;

/* Create a plan for one problem size and allocate its device workspace on the current
 * device.
 *   B, H >= 0 (B*H == 0 is an empty problem: forward does nothing);
 *   n >= 1; 1 <= m <= 256, m <= n (m need not divide n);
 *   d in {32, 64, 128} (other positive d: NYS_E_UNSUPPORTED);
 *   conv_width odd, 1 <= conv_width <= 65;
 *   0 <= pinv_iters <= 100;  dtype NYS_F32 or NYS_BF16; n*d < 2^31; B*H < 2^23.
 * Shapes whose kernels need more LDS than the device offers (fp32 with d = 128 and
 * m > 96) are NYS_E_UNSUPPORTED.
 * On success *plan is set; on failure *plan = NULL (when plan itself is non-NULL).
 * Errors: NYS_E_ARG, NYS_E_UNSUPPORTED, NYS_E_DEVICE (no device / not gfx950, checked
 * after argument validation), NYS_E_NOMEM. */
nys_status nys_attn_create(nys_attn_plan **plan, int B, int H, int n, int d, int m,
                           int conv_width, int pinv_iters, nys_dtype dtype);

/* Enqueue one forward pass on `stream` (a hipStream_t; NULL = the default stream).
 *   q, k, v, out : device, [B][H][n][d] contiguous, d fastest, element type = dtype,
 *                  16-byte aligned; out must not overlap q, k or v.
 *   conv_w       : device, fp32 [H][conv_width], 16-byte aligned not required.
 * Asynchronous: returns after the launches; device faults surface at the caller's next
 * synchronisation. A plan serves one forward at a time (its workspace is shared):
 * forwards on one plan must be ordered on a stream. No NaN/Inf checks.
 * Errors: NYS_E_ARG (null/misaligned/overlapping pointers), NYS_E_LAUNCH. */
nys_status nys_attn_forward(nys_attn_plan *plan, const void *q, const void *k,
                            const void *v, const float *conv_w, void *out, void *stream);

/* nys_attn_forward plus copies of the intermediates into the non-NULL fields of
 * `taps` (layouts above). taps may be NULL. Same errors as nys_attn_forward. */
nys_status nys_attn_forward_debug(nys_attn_plan *plan, const void *q, const void *k,
                                  const void *v, const float *conv_w, void *out,
                                  void *stream, const nys_attn_taps *taps);

/* Forward of a padded batch with per-element valid lengths (padding masks / ragged
 * batches; the page does not define masking, this entry point takes the reading that a
 * padded element is the unpadded sequence):
 *   lengths : device, int32 [B], or NULL for all n. Entry b is the valid length L_b of
 *             batch element b, m <= L_b <= n; tokens [L_b, n) are padding.
 * For every head of element b, rows [0, L_b) of out are the forward of the unpadded
 * length-L_b sequence (segments by floor(t m / L_b); padding tokens are neither keys,
 * values, landmark members nor conv inputs, and their q, k, v rows are not read) and
 * rows [L_b, n) are written as zeros. Entries outside [m, n] are clamped into it on the
 * device so that no access leaves the tensors; their results are unspecified.
 * taps: as for nys_attn_forward_debug (may be NULL; rows past L_b of taps->attn are
 * zero, the landmark-sized taps are those of the unpadded sequence).
 * Other arguments and errors as nys_attn_forward. */
nys_status nys_attn_forward_varlen(nys_attn_plan *plan, const void *q, const void *k,
                                   const void *v, const float *conv_w, const int *lengths,
                                   void *out, void *stream, const nys_attn_taps *taps);

/* Allocation-free forward, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. It computes
 * exactly what nys_attn_forward computes for a plan of the same shape (same kernels, same
 * launch geometry), without a plan: the workspace is one static device array of
 * NYS_NOALLOC_SCRATCH_BYTES bytes per GPU, held by each GPU the library runs on until the
 * process ends. The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); it launches a small clearing kernel before the forward when m is not a
 * multiple of 32.
 *   B, H, n, d, m, conv_width, pinv_iters, dtype : as for nys_attn_create
 *   q, k, v, conv_w, out, stream                 : as for nys_attn_forward
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race and give undefined
 * results; calls ordered on one stream are safe. B*H == 0 does nothing.
 * Errors: NYS_E_ARG, NYS_E_UNSUPPORTED (as for nys_attn_create, and shapes whose workspace
 * exceeds NYS_NOALLOC_SCRATCH_BYTES: the five workloads of the benchmark fit), NYS_E_DEVICE
 * (no device / not gfx950 / the scratch symbol cannot be looked up), NYS_E_LAUNCH. */
#define NYS_NOALLOC_SCRATCH_BYTES (160u * 1024u * 1024u)
nys_status nys_attn_forward_noalloc(int B, int H, int n, int d, int m, int conv_width,
                                    int pinv_iters, nys_dtype dtype, const void *q,
                                    const void *k, const void *v, const float *conv_w,
                                    void *out, void *stream);

/* Backward pass: gradients of L = sum(out * dout) for the forward of this plan, i.e. the
 * derivative of the method of the Nystromformer review page ("Proposed method", bullets
 * M1..M6), including the alpha scaling of the pseudo-inverse start and the conv skip.
 *   q, k, v, conv_w, lengths : as for nys_attn_forward_varlen (lengths may be NULL)
 *   dout   : device [B][H][n][d] in the plan's dtype, the upstream gradient of out
 *   dq, dk, dv : device [B][H][n][d] in the plan's dtype, written (rows >= lengths[b] zero)
 *   dconv_w: device fp32 [H][conv_width], written (summed over the batch)
 * Every plan is supported. bf16 plans with m <= 64 run fused kernels that recompute the
 * forward's segment means and landmark context; the first call allocates their workspace
 * (about BH (2 n d + (2 iters + 1) mp^2 + 3 C mp d) * 4 bytes). fp32 plans and m > 64 run
 * the general path: batched fp32 products with the factors softmax(s Q Kt^T) and
 * softmax(s Qt K^T) held whole; its first call allocates about
 * BH (4 n mp + (iters + 13) mp^2 + 3 n d + 6 mp d) * 4 bytes (mp = m rounded up to 32;
 * linear in n). Setting NYS_BACKWARD=general selects the general path for any plan.
 * Neither needs a preceding forward. Preconditions: 16-byte aligned tensors; dq, dk, dv
 * distinct from each other and from q, k, v, dout; dconv_w distinct from conv_w;
 * B*H <= 65535 on the general path. Shares the plan workspace with nys_attn_forward:
 * one call at a time per plan.
 * Errors: NYS_E_ARG, NYS_E_UNSUPPORTED, NYS_E_NOMEM, NYS_E_LAUNCH. */
nys_status nys_attn_backward(nys_attn_plan *plan, const void *q, const void *k, const void *v,
                             const float *conv_w, const int *lengths, const void *dout,
                             void *dq, void *dk, void *dv, float *dconv_w, void *stream);

/* Projections around the attention core (Fastformer review page, "Proposed method": the
 * input embeddings become Q, K, V through linear projections per head), bf16 in and out,
 * fp32 accumulation. No plan: these are plain products on the given stream.
 *
 * nys_proj_qkv: for each head h, q[b][h] = x[b] Wq_h^T, k[b][h] = x[b] Wk_h^T,
 * v[b][h] = x[b] Wv_h^T, where Wq_h, Wk_h, Wv_h are the d rows of w_qkv starting at
 * h*d, (H + h)*d and (2H + h)*d.
 *   x     : device bf16 [B][n][d_model]
 *   w_qkv : device bf16 [3*H*d][d_model] ([out_features][in_features])
 *   q,k,v : device bf16 [B][H][n][d], written (the layout nys_attn_forward reads)
 * nys_proj_out: y[b][t][:] = concat_h(o[b][h][t][:]) w_o^T (head h at features h*d..).
 *   o     : device bf16 [B][H][n][d]
 *   w_o   : device bf16 [d_model][H*d]
 *   y     : device bf16 [B][n][d_model], written
 * Preconditions: B, H, n >= 1; d in {32, 64, 128}; d_model >= 64 and a multiple of 64;
 * H*d a multiple of 64; all pointers 16-byte aligned, outputs not overlapping inputs;
 * B*n*max(d_model, 3*H*d) < 2^31 and 3*H*d*d_model < 2^31 (NYS_E_UNSUPPORTED otherwise).
 * Asynchronous like nys_attn_forward.
 * Errors: NYS_E_ARG, NYS_E_UNSUPPORTED, NYS_E_DEVICE, NYS_E_LAUNCH. */
nys_status nys_proj_qkv(const void *x, const void *w_qkv, void *q, void *k, void *v, int B,
                        int H, int n, int d, int d_model, void *stream);
nys_status nys_proj_out(const void *o, const void *w_o, void *y, int B, int H, int n, int d,
                        int d_model, void *stream);

/* FLASH mixed-chunk attention (review page "Transformer Quality in Linear Time", "Proposed
 * method", third bullet), bf16 in and out, one output per head:
 *   out[t] = softmax over t' in chunk(t) (t' <= t if causal) of (s q_t . k_t') v_t'
 *          + s q_t (sum over covered keys u of k_u^T v_u) / (number of covered keys)
 * with s = 1/sqrt(d), chunk g = tokens [g*chunk, min((g+1)*chunk, n)), covered = all
 * tokens (causal = 0) or the tokens of the chunks before t's chunk (causal = 1; none for
 * the first chunk, whose global term is zero).
 *   q, k, v, out : device bf16 [B][H][n][d]; out written
 *   workspace    : device memory of at least nys_flash_workspace_bytes(...) bytes, owned
 *                  by the caller, 16-byte aligned, not overlapping the tensors
 * nys_flash_states fills the workspace from k and v (chunk sums K_g^T V_g, then the
 * scaled global sums); nys_flash_attend reads it and writes out; nys_flash_attention does
 * both. Preconditions: B, H, n >= 1; d in {32, 64, 128}; chunk in {64, 128, 256}; causal
 * in {0, 1}; B*H*n*d < 2^31. Asynchronous on the given stream.
 * Errors: NYS_E_ARG, NYS_E_UNSUPPORTED, NYS_E_DEVICE, NYS_E_LAUNCH. */
size_t nys_flash_workspace_bytes(int B, int H, int n, int d, int chunk, int causal);
nys_status nys_flash_states(const void *k, const void *v, int B, int H, int n, int d, int chunk,
                            int causal, void *workspace, size_t workspace_bytes, void *stream);
nys_status nys_flash_attend(const void *q, const void *k, const void *v, void *out, int B, int H,
                            int n, int d, int chunk, int causal, void *workspace,
                            size_t workspace_bytes, void *stream);
nys_status nys_flash_attention(const void *q, const void *k, const void *v, void *out, int B,
                               int H, int n, int d, int chunk, int causal, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Bytes of device workspace the plan owns (0 for a NULL plan). */
size_t nys_attn_workspace_bytes(const nys_attn_plan *plan);

/* Stage timing for benchmarks. After nys_attn_profile_enable(plan, max_calls), each of
 * the next max_calls forwards records HIP events around its NYS_ATTN_STAGES kernels on
 * the forward's stream: 0 segment means, 1 landmark kernel + pseudo-inverse, 2 landmark
 * context (split over n), 3 output (merge, Y = Z W, softmax times Y, conv skip).
 * nys_attn_profile_read waits for those events and writes, for call i, the durations in
 * milliseconds to stage_ms[NYS_ATTN_STAGES*i + 0..3]; *n_calls receives the number of
 * recorded calls (at most max_calls), after which recording restarts from zero.
 * Errors: NYS_E_ARG, NYS_E_LAUNCH. */
#define NYS_ATTN_STAGES 4
nys_status nys_attn_profile_enable(nys_attn_plan *plan, int max_calls);
nys_status nys_attn_profile_read(nys_attn_plan *plan, float *stage_ms, int max_calls,
                                 int *n_calls);

/* Wait for the device, then free the workspace and the plan. NULL-safe. */
void nys_attn_destroy(nys_attn_plan *plan);

/* Thread-local description of the last failure in this thread ("" if none). */
const char *nys_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NYS_ATTN_H */
