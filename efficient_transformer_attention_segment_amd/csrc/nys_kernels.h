// Kernel argument blocks and host launchers of the three stages of the forward pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nys {

// Stage 1: segment means of Q and K.
struct SegArgs {
  const int* lengths;  // [B] valid lengths, or nullptr (all n)
  int BH, H, n, m, mp;
  float* qt;       // [BH][mp][d]
  float* kt;       // [BH][mp][d]
  uint16_t* qt_hl; // [BH][2][mp][d] hi plane then lo plane
  uint16_t* kt_hl; // [BH][2][mp][d]
};

// Stage 2: landmark kernel + iterative pseudo-inverse (one block per head) and the
// landmark context split over n (BH * C blocks, partial softmax states). For mp <= 64 both
// run in one launch: blocks [0, npinv) form the pseudo-inverse, the rest the context.
struct CtxArgs {
  const void* k;
  const void* v;
  const int* lengths;     // [B] valid lengths, or nullptr (all n)
  const float* qt;        // [BH][mp][d]  landmarks Qt (fp32)
  const uint16_t* qt_hl;  // [BH][2][mp][d]
  const uint16_t* kt_hl;  // [BH][2][mp][d]
  float* a_s;             // [BH][mp][mp]  logits, then A_S
  float* z;               // [BH][mp][mp]  final Z (fp32)
  uint16_t* planes;       // [BH][kPlanes][mp][mp]  hi/lo bf16 operand planes
  float* own;             // [BH][2][mp][mp]  fp32 X, X^2 (global-memory pinv variant)
  float* alpha_part;      // [BH][mp/32][mp+1] per-strip column abs-sums, row max (mp > 64)
  uint16_t* z_hl;         // [BH][2][mp][mp]  final Z, row-major hi/lo
  float* part_w;          // [BH][C][d][mp]   per-chunk unnormalised (Bbar V)^T
  float* part_ml;         // [BH][C][2][mp]   per-chunk running max (log2 units), sum
  int uneven_ncu;         // 0: chunk c is [c * chunk, (c + 1) * chunk); else the CU count
                          // of the uneven split (see chunk_range in context.hip)
  int BH, H, n, d, m, mp, iters, chunk, C, LG, TG;
  int npinv;              // pseudo-inverse blocks at the front of the context grid (0 or BH)
  int ring_ni;            // bf16 context: 1 KiB LDS-DMA loads per wave per K or V tile
  int ring_stages;        // bf16 context: K/V tiles in the LDS ring (2..4)
  int fp32_out;           // 1: the in-LDS pseudo-inverse (mp <= 64) also stores the fp32
                          // A_S and Z for inspection; nothing downstream reads them
  float scale;            // 1/sqrt(d)
  float scale_log2e;      // log2(e)/sqrt(d)
};

// Valid length of head bh: lengths[bh / H] clamped into [m, n], or n.
__device__ __forceinline__ int valid_length(const int* lengths, int bh, int H, int n, int m) {
  if (lengths == nullptr) return n;
  const int L = lengths[bh / H];
  return L < m ? m : (L > n ? n : L);
}

// Number of hi/lo bf16 mp x mp planes per head in CtxArgs::planes.
constexpr int kPlanes = 18;

// Stage 3: merge of the partial states into W and Y = Z W (prologue of every block),
// then softmax(Q Kt^T s) Y plus the depthwise conv of V, stored in the I/O dtype;
// optionally the fp32 W, Y and attention part for inspection.
struct OutArgs {
  const void* q;
  const void* v;
  const int* lengths;     // [B] valid lengths, or nullptr (all n)
  const float* conv_w;    // [H][W]
  void* out;              // [BH][n][d]
  float* attn_tap;        // [BH][n][d] or nullptr
  float* w_tap;           // [BH][mp][d] or nullptr (written by each head's first block)
  float* y_tap;           // [BH][mp][d] or nullptr
  const float* kt;        // [BH][mp][d]      landmarks Kt (fp32)
  const uint16_t* kt_hl;  // [BH][2][mp][d]
  const uint16_t* z_hl;   // [BH][2][mp][mp]
  const float* part_w;    // [BH][C][d][mp]
  const float* part_ml;   // [BH][C][2][mp]
  uint16_t* yt;           // [BH][2][d][mp + 8] Y^T planes staged per head (the
                          // online-softmax variants; see output_stages_y)
  int BH, H, n, m, mp, W, half, tok_per_block, G, C;
  float scale_log2e;
};

// Backward pass (bf16 I/O, mp <= 64): gradients of sum(out * dout) with respect to q, k,
// v and the conv weights. The forward's segment-means and context kernels run first
// (SegArgs / CtxArgs of the plan); these kernels then use their workspace outputs.
struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* conv_w;      // [H][W]
  const int* lengths;       // [B] or nullptr
  uint16_t* dq;             // [BH][n][d] outputs
  uint16_t* dk;
  uint16_t* dv;
  float* dconv_w;           // [H][W] output
  // forward state
  const float* qt;          // [BH][mp][d] landmarks (fp32), rows >= m zero
  const float* kt;
  const uint16_t* qt_hl;    // [BH][2][mp][d]
  const uint16_t* kt_hl;
  const float* part_w;      // [BH][C][d][mp] context partial (Bbar V)^T
  const float* part_ml;     // [BH][C][2][mp] context partial max (log2 units), sum
  // backward workspace
  float* w;                 // [BH][mp][d]   W = B V (merged)
  float* stat;              // [BH][2][mp]   B's reference max (log2 units) and sum
  float* a_s;               // [BH][mp][mp]  A_S
  float* alpha;             // [BH][4]       alpha, max column sum, max row sum, pad
  int* amax;                // [BH][2]       argmax column, argmax row
  float* zs;                // [BH][T+1][mp][mp] iterates Z_0..Z_T
  float* xs;                // [BH][T][mp][mp]   X_k = A Z_k
  uint16_t* y_hl;           // [BH][2][mp][d]  Y = Z W
  uint16_t* ktT_hl;         // [BH][2][d][mp]  Kt^T
  uint16_t* qtT_hl;         // [BH][2][d][mp]  Qt^T
  float* part1;             // [BH][C][2][mp][d] pass-1 partials: F^T dO, dSF^T Q
  uint16_t* dw_hl;          // [BH][2][mp][d]  dW
  uint16_t* dwT_hl;         // [BH][2][d][mp]  dW^T
  float* db;                // [BH][mp]        D_B = rowsum(dW o W)
  float* dkt;               // [BH][mp][d]     dKt (complete)
  float* dqt;               // [BH][mp][d]     dQt from the A_S path
  float* part2;             // [BH][C][mp][d]  pass-2 partials: dSB K
  float* dq_part;           // [BH][n][d]      s dSF Kt
  float* dv_part;           // [BH][n][d]      B^T dW
  float* part_dw;           // [BH][C3][W]
  int B, H, BH, n, d, m, mp, W, iters, chunk, C, chunk3, C3;
  int fin_segs;  // rows of the final pass's per-segment table: segments one of its token
                 // tiles can meet (mp with per-sequence lengths, where segments can be short)
  float scale, scale_log2e;
};
hipError_t launch_backward(const BwdArgs& a, hipStream_t s);
hipError_t configure_backward();

// General backward (any m <= 256, fp32 or bf16 I/O): batched fp32 products over the
// heads with the factors F and B held whole (backward_general.hip). Workspace buffers are
// fp32 and per head: [n][mp] F, G1; [mp][n] Bm, G2; [mp][mp] A, P, Q1, R, Gz, Gn, dR, dX,
// dQ1, dP, dA; [T+1][mp][mp] Zs; [max(T,1)][mp][mp] Xs; [mp][d] Wc (= B V), Y, dY, dW, dQt, dKt;
// [n][d] dQ, dK, dV; [4] alpha; [2] amax (int); [ceil(n / dw_chunk)][W] dw_part.
struct GenBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* conv_w;
  const int* lengths;
  void* dq;
  void* dk;
  void* dv;
  float* dconv_w;
  const float* qt;  // [BH][mp][d] landmarks (segment-means kernel), rows >= m zero
  const float* kt;
  float *F, *G1, *Bm, *G2;
  float *A, *P, *Q1, *R, *Gz, *Gn, *dR, *dX, *dQ1, *dP, *dA;
  float *Zs, *Xs;
  float *Wc, *Y, *dY, *dW, *dQt, *dKt;
  float *dQ, *dK, *dV;
  float* alpha;
  int* amax;
  float* dw_part;
  float* ksplit;  // [nsplit][BH][mp][d] partial products of the token-dimension products
  int nsplit;     // most k-splits ksplit holds (1: no split)
  int B, H, BH, n, d, m, mp, W, iters, dw_chunk;
  float scale;
  bool bf16;
};
hipError_t launch_backward_general(const GenBwdArgs& a, hipStream_t s);

// FLASH mixed-chunk attention (bf16 I/O): chunk states, global sums, local + global.
struct FlashArgs {
  const uint16_t* q;        // [BH][n][d]
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;            // [BH][n][d]
  float* states;            // [BH][G][d][d]  (K_g^T V_g)^T
  uint16_t* mplanes;        // [BH][causal ? G : 1][2][d][d]  hi/lo of (s / n_g) M_g^T
  int BH, n, d, chunk, G, causal;
  float scale, scale_log2e;
};
hipError_t launch_flash_states(const FlashArgs& a, hipStream_t s);
hipError_t launch_flash_attend(const FlashArgs& a, hipStream_t s);
hipError_t configure_flash();

// Projections around the core (bf16): q, k, v = split_heads(x w_qkv^T) and
// y = concat_heads(o) w_o^T.
struct ProjArgs {
  const void* a;     // x [B n][D] (qkv) or o [B][H][n][d] (out)
  const void* w;     // w_qkv [3 H d][D] or w_o [D][H d]
  void* q;           // qkv outputs [B][H][n][d]
  void* k;
  void* v;
  void* y;           // out output [B n][D]
  int B, H, n, d, D;
};
hipError_t launch_qkv_proj(const ProjArgs& a, hipStream_t s);
hipError_t launch_out_proj(const ProjArgs& a, hipStream_t s);
size_t proj_lds_bytes();
hipError_t configure_proj();

hipError_t launch_segmeans(bool bf16, int d, const void* q, const void* k, const SegArgs& a,
                           hipStream_t s);
// Zero the landmark rows m..mp-1 of every head (fp32 means and hi/lo planes of Q and K).
hipError_t launch_clear_landmark_padding(int d, const SegArgs& a, hipStream_t s);
// Separate pseudo-inverse launch, used only when it is not fused (mp > 64).
hipError_t launch_pinv(int d, const CtxArgs& a, hipStream_t s);
hipError_t launch_context(bool bf16, int d, const CtxArgs& a, hipStream_t s);
hipError_t launch_output(bool bf16, int d, int conv_ksteps, const OutArgs& a, hipStream_t s);
// True when the output launch for this shape first merges the context states and forms
// Y = Z W once per head (into OutArgs::yt) instead of in every block's prologue.
bool output_stages_y(bool bf16, int d, int mp, int conv_ksteps, int C);
constexpr int kMaxChunks = 16;  // context chunks per head the output merge supports

// Dynamic LDS each launch needs (bytes), and one-time kernel attribute setup.
// pinv fused into the context launch?
inline bool context_fuses_pinv(int mp) { return mp <= 64; }
// LDS-DMA ring geometry of the bf16 context kernel (sets a.ring_ni, a.ring_stages).
void context_ring_geometry(int d, CtxArgs& a);
size_t context_lds_bytes(bool bf16, int d, const CtxArgs& a);
size_t output_lds_bytes(bool bf16, int d, int mp, int conv_ksteps, int C);
hipError_t configure_context(bool bf16, int d, int mp, size_t ctx_lds);
// Context blocks resident per CU at this LDS size (0 if the runtime cannot tell).
// Token groups per landmark group in a context block (block = 64 LG TG threads, at most
// 512, the kernel's launch bound; a step covers 32 TG tokens): four waves for m <= 64; two
// groups (8 waves, 64-token steps) at exactly four landmark groups, where 32-token steps
// left the block's loop dominated by its per-step barriers; one above.
constexpr int context_token_groups(int LG) { return LG == 4 ? 2 : (LG > 4 ? 1 : 4 / LG); }
int context_blocks_per_cu(bool bf16, int d, int mp, size_t ctx_lds);
// Output blocks resident per CU at this LDS size (0 if the runtime cannot tell).
int output_blocks_per_cu(bool bf16, int d, int ks, int mp, int m, int C, size_t lds);
// Tokens per step of one output block (32 per wave).
int output_step_tokens(bool bf16, int d, int mp, int conv_ksteps, int C);
hipError_t configure_output(bool bf16, int d, int conv_ksteps, size_t out_lds);

}  // namespace nys
