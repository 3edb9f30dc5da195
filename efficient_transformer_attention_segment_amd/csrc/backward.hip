// Backward pass of the Nystrom self-attention forward (Nystromformer review page,
// "Proposed method", bullets M1..M6): gradients of L = sum(out * dout) with respect to
// Q, K, V and the depthwise conv weights, bf16 I/O, m <= 64 (mp <= 64).
//
// Per (batch, head), with s = 1/sqrt(d), F = softmax(s Q Kt^T) (n x m),
// A = softmax(s Qt Kt^T) (m x m), B = softmax(s Qt K^T) (m x n), Z = the iterated
// pseudo-inverse of A, W = B V, Y = Z W, out = F Y + conv(V):
//
//   dY = F^T dO                 dF = dO Y^T,  dSF = F o (dF - rowsum(F o dF))
//   dQ += s dSF Kt              dKt += s dSF^T Q
//   dZ = dY W^T                 dW = Z^T dY
//   dA = reverse sweep of the iteration from dZ (plus the alpha term)
//   dSA = A o (dA - rowsum(A o dA));  dQt += s dSA Kt;  dKt += s dSA^T Qt
//   dB = dW V^T,  dSB = B o (dB - rowsum(B o dB)) with rowsum(B o dB) = rowsum(dW o W)
//   dV = B^T dW + conv^T(dO)    dK += s dSB^T Qt    dQt += s dSB K
//   dQ += dQt[seg(t)] / |seg|   dK += dKt[seg(t)] / |seg|  (segment means)
//   dw[k] = sum_t dO[t] . V[t + k - (W-1)/2]
//
// Kernels, in stream order after the forward's segment-means and context kernels
// (which leave Qt, Kt and the split-n partial states of B V in the workspace):
//   bwd_land_fwd_kernel   one block per head: merge W and B's softmax statistics,
//                         A, alpha, the iteration with every Z_k and X_k saved, Y = Z W
//   bwd_pass1_kernel      over tokens (Q, dO): dQ's first term, partial dY and dKt
//   bwd_land_bwd_kernel   one block per head: dZ, dW, the reverse sweep, dA, dSA, dQt,
//                         dKt, rowsum(dW o W)
//   bwd_pass2_kernel      over tokens (K, V): dK (complete), B^T dW, partial dQt
//   bwd_final_kernel      over tokens (dO, V): dQ and dV complete, partial dw
//   bwd_dw_kernel         dw summed over the batch and token chunks
//
// Token passes use v_mfma_f32_32x32x16_bf16 tiles whose operands are k-contiguous rows:
// token rows straight from HBM (bf16, exact), landmark-sized operands as hi/lo bf16
// planes (~17 significant bits), per-step transposed copies in LDS for the products
// that contract over tokens. The m x m steps run in fp32 on the VALU out of LDS.
#include "nys_common.h"
#include "nys_kernels.h"

namespace nys {

constexpr int kBwdThreads = 256;  // landmark-sized kernels and the final pass

// ------------------------------------------------------------------ fp32 block products
// C[M][N] = alpha op(A) op(B) + beta C on fp32 MFMA (v_mfma_f32_32x32x2_f32, products
// and sums in fp32). op(A) is A stored [M][K] (lda) or, with TA, A stored [K][M]; op(B)
// is B stored [K][N] (ldb) or, with TB, B stored [N][K]. Each wave forms whole 32 x 32
// output tiles; the two k-slots of the MFMA take the two halves of the k range, so a lane
// reads four consecutive k of a k-contiguous operand as one 16-byte load. M and N
// multiples of 32, K a multiple of 8, lda and ldb multiples of 4, A and B 16-byte
// aligned. C must not alias A or B; no barrier inside.
template <bool TA, bool TB>
__device__ void blk_mm(float* C, int ldc, const float* A, int lda, const float* B, int ldb,
                       int M, int N, int K, float alpha, float beta) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int r32 = lane & 31, kb = (lane >> 5) * (K / 2);
  const int tn = N / 32, tiles = (M / 32) * tn;
  for (int t = wave; t < tiles; t += nw) {
    const int i0 = 32 * (t / tn), j0 = 32 * (t % tn);
    f32x16 acc = zero16();
    for (int s = kb; s < kb + K / 2; s += 4) {
      f32x4 av, bv;
      if (TA) {
#pragma unroll
        for (int q = 0; q < 4; ++q) av[q] = A[(s + q) * lda + i0 + r32];
      } else {
        av = *reinterpret_cast<const f32x4*>(A + (i0 + r32) * lda + s);
      }
      if (TB) {
        bv = *reinterpret_cast<const f32x4*>(B + (j0 + r32) * ldb + s);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) bv[q] = B[(s + q) * ldb + j0 + r32];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[q], bv[q], acc, 0, 0, 0);
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float* p = C + acc_row(i0, rr, lane) * ldc + j0 + r32;
      *p = beta != 0.f ? alpha * acc[rr] + beta * *p : alpha * acc[rr];
    }
  }
}

// C = b C + a I over the MP x MP block, identity only on the first m diagonal entries.
__device__ void blk_eye(float* C, int ld, int MP, int m, float a, float b) {
  for (int e = threadIdx.x; e < MP * MP; e += blockDim.x) {
    const int i = e / MP, j = e % MP;
    C[i * ld + j] = b * C[i * ld + j] + ((i == j && i < m) ? a : 0.f);
  }
}

__device__ void blk_copy_out(float* dst, int ldd, const float* src, int lds_, int R, int Cc) {
  for (int e = threadIdx.x; e < R * Cc; e += blockDim.x) {
    const int i = e / Cc, j = e % Cc;
    dst[(size_t)i * ldd + j] = src[i * lds_ + j];
  }
}

__device__ void blk_copy_in(float* dst, int ldd, const float* src, int lds_, int R, int Cc) {
  for (int e = threadIdx.x; e < R * Cc; e += blockDim.x) {
    const int i = e / Cc, j = e % Cc;
    dst[i * ldd + j] = src[(size_t)i * lds_ + j];
  }
}

// dst[R][Cc] (ld ldd) = src[R][Cc] (ld lds_) as 16-byte pieces, every load of the copy
// issued before the first store (one memory latency per copy). R, Cc, ldd, lds_ multiples
// of 4 where needed, both pointers 16-byte aligned.
template <int R, int Cc>
__device__ __forceinline__ void blk_load4(float* dst, int ldd, const float* src, int lds_) {
  constexpr int N4 = R * Cc / 4, PER = (N4 + kBwdThreads - 1) / kBwdThreads;
  f32x4 v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = threadIdx.x + kBwdThreads * u;
    if (e < N4)
      v[u] = *reinterpret_cast<const f32x4*>(src + (size_t)(e / (Cc / 4)) * lds_ + 4 * (e % (Cc / 4)));
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = threadIdx.x + kBwdThreads * u;
    if (e < N4) *reinterpret_cast<f32x4*>(dst + (e / (Cc / 4)) * ldd + 4 * (e % (Cc / 4))) = v[u];
  }
}

// dst[R][Cc] = scale * sum over nc slabs (stride elements apart) of src[R][Cc] (ld Cc);
// the loads of one slab are issued together.
template <int R, int Cc>
__device__ __forceinline__ void blk_sum4(float* dst, int ldd, const float* src, size_t stride,
                                         int nc, float scale) {
  constexpr int N4 = R * Cc / 4, PER = (N4 + kBwdThreads - 1) / kBwdThreads;
  f32x4 acc[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nc; ++c)
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = threadIdx.x + kBwdThreads * u;
      if (e < N4) acc[u] += *reinterpret_cast<const f32x4*>(src + c * stride + 4 * (size_t)e);
    }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = threadIdx.x + kBwdThreads * u;
    if (e < N4)
      *reinterpret_cast<f32x4*>(dst + (e / (Cc / 4)) * ldd + 4 * (e % (Cc / 4))) = acc[u] * scale;
  }
}

// hi/lo planes of an fp32 matrix src [R][Cc] (ld lds_): row-major [R][Cc] or transposed
// [Cc][R] (plane stride R * Cc).
// With kPerm (transposed only), row i of src lands at column (i & ~15) | kslot_perm(i & 15):
// the k order in which accumulator registers feed the next product as its B operand.
template <bool kTrans, bool kPerm = false>
__device__ void blk_split_out(uint16_t* hl, const float* src, int lds_, int R, int Cc) {
  for (int e = threadIdx.x; e < R * Cc; e += blockDim.x) {
    const int i = kTrans ? e % R : e / Cc, j = kTrans ? e / R : e % Cc;
    uint16_t hi, lo;
    split1(src[(size_t)i * lds_ + j], hi, lo);
    const int ip = kPerm ? ((i & ~15) | kslot_perm(i & 15)) : i;
    const size_t o = kTrans ? (size_t)j * R + ip : (size_t)i * Cc + j;
    hl[o] = hi;
    hl[(size_t)R * Cc + o] = lo;
  }
}

// ------------------------------------------------------------------ MFMA row tiles
// acc += A[32 rows][0:K] B[0:K][32 cols]: lane (h, r32) passes the start of A row r32 and
// of B^T row r32 (k contiguous); AL / BL say whether a lo plane is present (otherwise the
// operand is exact bf16 and only the hi pointer is read).
template <int K, bool AL, bool BL>
__device__ __forceinline__ f32x16 mma_rows(f32x16 acc, const uint16_t* ahi, const uint16_t* alo,
                                           const uint16_t* bhi, const uint16_t* blo, int h) {
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 16) {
    const Pair8 x{ld8(ahi + k0 + 8 * h), AL ? ld8(alo + k0 + 8 * h) : zero8()};
    const Pair8 y{ld8(bhi + k0 + 8 * h), BL ? ld8(blo + k0 + 8 * h) : zero8()};
    acc = mfma_pair<AL, BL>(x, y, acc);
  }
  return acc;
}

// Same product with B given as a row-major tile bt[K][ldb] (k rows, output columns
// col0.. across), read with LDS transpose reads: lane 4j + q of each 16-lane group
// addresses row k + j, column col0 + 16 (group & 1) + 4q, and receives column
// col0 + lane % 32 at k-slots 8h .. 8h + 7. B is exact bf16.
template <int K, bool AL>
__device__ __forceinline__ f32x16 mma_rows_btr(f32x16 acc, const uint16_t* ahi,
                                               const uint16_t* alo, const uint16_t* bt, int ldb,
                                               int col0, int lane) {
  const int h = lane >> 5, trj = (lane & 15) >> 2;
  const int trc = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int kk = k0 + 8 * h;
    const Pair8 x{ld8(ahi + kk), AL ? ld8(alo + kk) : zero8()};
    const Pair8 y{lds_tr16x2(bt + (kk + trj) * ldb + trc, bt + (kk + 4 + trj) * ldb + trc),
                  zero8()};
    acc = mfma_pair<AL, false>(x, y, acc);
  }
  return acc;
}

// Token row held by accumulator register rr of lane half h (within a 32-row tile).
__device__ __forceinline__ int acc_r(int rr, int h) { return 8 * (rr >> 2) + 4 * h + (rr & 3); }

// Segment bounds in 32-bit unsigned arithmetic: L * m < 2^32 because n * d < 2^31,
// d >= 32 and m <= 64.
__device__ __forceinline__ int seg_start(int j, int L, int m) {
  return (int)(((unsigned)j * (unsigned)L + (unsigned)(m - 1)) / (unsigned)m);
}
__device__ __forceinline__ int seg_of(int t, int L, int m) {
  return (int)(((unsigned)t * (unsigned)m) / (unsigned)L);
}

// ======================================================================= L1
template <int D, int MP>
__global__ __launch_bounds__(kBwdThreads) void bwd_land_fwd_kernel(BwdArgs a) {
  extern __shared__ __align__(16) float smem[];
  constexpr int LM = MP + 4, LD = D + 4;  // 16-byte rows
  float* Am = smem;               // [MP][LM]
  float* Zb = Am + MP * LM;
  float* Xb = Zb + MP * LM;
  float* T1 = Xb + MP * LM;
  float* T2 = T1 + MP * LM;
  float* Wm = T2 + MP * LM;       // [MP][LD]
  float* Yb = Wm + MP * LD;       // [MP][LD]
  float* Qs = Wm;                 // Qt, Kt at the start (dead once A is formed)
  float* Ks = Yb;
  __shared__ float colsum[MP], rowsum[MP], sal;
  const int bh = blockIdx.x, m = a.m, tid = threadIdx.x;
  const float* qt = a.qt + (size_t)bh * MP * D;
  const float* kt = a.kt + (size_t)bh * MP * D;

  blk_split_out<true>(a.ktT_hl + (size_t)bh * 2 * D * MP, kt, D, MP, D);
  blk_split_out<true, true>(a.qtT_hl + (size_t)bh * 2 * D * MP, qt, D, MP, D);
  blk_load4<MP, D>(Qs, LD, qt, D);
  blk_load4<MP, D>(Ks, LD, kt, D);
  __syncthreads();
  blk_mm<false, true>(Am, LM, Qs, LD, Ks, LD, MP, MP, D, a.scale, 0.f);
  __syncthreads();
  if (tid < MP) {  // row softmax over the m landmarks; padding rows and columns zero
    const int i = tid;
    float* row = Am + i * LM;
    if (i < m) {
      float mx = kNegBig;
      for (int j = 0; j < m; ++j) mx = fmaxf(mx, row[j]);
      float sum = 0.f;
      for (int j = 0; j < m; ++j) {
        const float e = expf(row[j] - mx);
        row[j] = e;
        sum += e;
      }
      const float inv = 1.f / sum;
      for (int j = 0; j < m; ++j) row[j] *= inv;
    }
    for (int j = (i < m ? m : 0); j < MP; ++j) row[j] = 0.f;
  }
  __syncthreads();
  if (tid < MP) {
    float cs = 0.f, rs = 0.f;
    for (int i = 0; i < MP; ++i) cs += fabsf(Am[i * LM + tid]);
    for (int j = 0; j < MP; ++j) rs += fabsf(Am[tid * LM + j]);
    colsum[tid] = cs;
    rowsum[tid] = rs;
  }
  __syncthreads();
  if (tid == 0) {
    int jc = 0, ir = 0;
    for (int j = 1; j < m; ++j)
      if (colsum[j] > colsum[jc]) jc = j;
    for (int i = 1; i < m; ++i)
      if (rowsum[i] > rowsum[ir]) ir = i;
    const float c = colsum[jc], r = rowsum[ir];
    sal = 1.f / (c * r);
    a.alpha[4 * bh + 0] = sal;
    a.alpha[4 * bh + 1] = c;
    a.alpha[4 * bh + 2] = r;
    a.alpha[4 * bh + 3] = 0.f;
    a.amax[2 * bh + 0] = jc;
    a.amax[2 * bh + 1] = ir;
  }
  __syncthreads();
  const float al = sal;
  for (int e = tid; e < MP * MP; e += blockDim.x) {
    const int i = e / MP, j = e % MP;
    Zb[i * LM + j] = al * Am[j * LM + i];
  }
  __syncthreads();
  const size_t mm2 = (size_t)MP * MP;
  float* zs = a.zs + (size_t)bh * (a.iters + 1) * mm2;
  float* xs = a.xs + (size_t)bh * a.iters * mm2;
  blk_copy_out(zs, MP, Zb, LM, MP, MP);
  float* Z = Zb;
  float* Zn = T2;
  for (int it = 0; it < a.iters; ++it) {
    blk_mm<false, false>(Xb, LM, Am, LM, Z, LM, MP, MP, MP, 1.f, 0.f);
    __syncthreads();
    blk_copy_out(xs + it * mm2, MP, Xb, LM, MP, MP);
    for (int e = tid; e < MP * MP; e += blockDim.x) {
      const int i = e / MP, j = e % MP;
      T1[i * LM + j] = ((i == j && i < m) ? 7.f : 0.f) - Xb[i * LM + j];  // 7I - X
    }
    __syncthreads();
    blk_mm<false, false>(Zn, LM, Xb, LM, T1, LM, MP, MP, MP, -1.f, 0.f);  // -X(7I - X)
    __syncthreads();
    blk_eye(Zn, LM, MP, m, 15.f, 1.f);                        // 15I - X(7I - X)
    __syncthreads();
    blk_mm<false, false>(T1, LM, Xb, LM, Zn, LM, MP, MP, MP, -1.f, 0.f);
    __syncthreads();
    blk_eye(T1, LM, MP, m, 13.f, 1.f);                        // R = 13I - X(...)
    __syncthreads();
    blk_mm<false, false>(Zn, LM, Z, LM, T1, LM, MP, MP, MP, 0.25f, 0.f);
    __syncthreads();
    float* t = Z;
    Z = Zn;
    Zn = t;
    blk_copy_out(zs + (it + 1) * mm2, MP, Z, LM, MP, MP);
  }
  // W = merge of the context partial states (rows >= m zero) and B's statistics:
  // per landmark the merged reference max and sum, then W^T in 16-byte pieces
  const float* pw = a.part_w + (size_t)bh * a.C * D * MP;
  const float* pml = a.part_ml + (size_t)bh * a.C * 2 * MP;
  float* stat = a.stat + (size_t)bh * 2 * MP;
  float* cscale = T1;  // [C][MP] per-chunk weight exp2(ml_c - mx) / ls (T1 is free here)
  if (tid < MP) {
    const int j = tid;
    float mx = kNegBig, ls = 0.f;
    if (j < m) {
      for (int c = 0; c < a.C; ++c) mx = fmaxf(mx, pml[c * 2 * MP + j]);
      for (int c = 0; c < a.C; ++c) ls += fast_exp2(pml[c * 2 * MP + j] - mx) * pml[c * 2 * MP + MP + j];
      for (int c = 0; c < a.C; ++c) cscale[c * MP + j] = fast_exp2(pml[c * 2 * MP + j] - mx) / ls;
    } else {
      for (int c = 0; c < a.C; ++c) cscale[c * MP + j] = 0.f;
    }
    stat[j] = j < m ? mx : 0.f;
    stat[MP + j] = j < m ? ls : 1.f;
  }
  __syncthreads();
  {
    constexpr int N4 = D * MP / 4, PER = (N4 + kBwdThreads - 1) / kBwdThreads;
    f32x4 acc[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < a.C; ++c)
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int e = tid + kBwdThreads * u;  // feature e / (MP/4), landmarks 4 (e % (MP/4)) ..
        if (e < N4) {
          const f32x4 w4 = *reinterpret_cast<const f32x4*>(pw + (size_t)c * D * MP + 4 * (size_t)e);
          const f32x4 s4 = *reinterpret_cast<const f32x4*>(cscale + c * MP + 4 * (e % (MP / 4)));
          acc[u] += w4 * s4;
        }
      }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + kBwdThreads * u;
      if (e < N4) {
        const int f = e / (MP / 4), j0 = 4 * (e % (MP / 4));
#pragma unroll
        for (int q = 0; q < 4; ++q) Wm[(j0 + q) * LD + f] = acc[u][q];
      }
    }
  }
  __syncthreads();
  blk_copy_out(a.w + (size_t)bh * MP * D, D, Wm, LD, MP, D);
  blk_mm<false, false>(Yb, LD, Z, LM, Wm, LD, MP, D, MP, 1.f, 0.f);
  __syncthreads();
  blk_split_out<false>(a.y_hl + (size_t)bh * 2 * MP * D, Yb, LD, MP, D);
  blk_copy_out(a.a_s + (size_t)bh * mm2, MP, Am, LM, MP, MP);
}

// ======================================================================= pass 1
template <int D, int MP, int NW>
__global__ __launch_bounds__(64 * NW) void bwd_pass1_kernel(BwdArgs a) {
  constexpr int T = 32 * NW, LT = MP / 32, FT = D / 32;
  constexpr int NRED = 2 * LT * FT, RPW = (NRED + NW - 1) / NW;
  // LDS rows padded by 16 bytes: the transposed tile stores and the 16-byte row reads of
  // 32 lanes then spread over the banks instead of meeting in one
  constexpr int TP = T + 8, DP = D + 8, MPP = MP + 8;
  extern __shared__ __align__(16) char lds[];
  uint16_t* ft_hi = reinterpret_cast<uint16_t*>(lds);  // F^T   [MP][TP]
  uint16_t* ft_lo = ft_hi + MP * TP;
  uint16_t* st_hi = ft_lo + MP * TP;                    // dSF^T [MP][TP]
  uint16_t* st_lo = st_hi + MP * TP;
  uint16_t* qR = st_lo + MP * TP;                       // Q     [T][DP] (step's tokens)
  uint16_t* oR = qR + T * DP;                           // dO    [T][DP]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, r32 = lane & 31;
  uint16_t* ds_hi = oR + T * DP + wave * 2 * 32 * MPP;  // dSF   [32][MPP] per wave
  uint16_t* ds_lo = ds_hi + 32 * MPP;
  int bh, c;
  xcd_map(blockIdx.x, a.BH, a.C, bh, c);
  const int m = a.m, L = valid_length(a.lengths, bh, a.H, a.n, a.m);
  const int tb = c * a.chunk, te = min(tb + a.chunk, L);
  const uint16_t* q = a.q + (size_t)bh * a.n * D;
  const uint16_t* dO = a.dout + (size_t)bh * a.n * D;
  const uint16_t* kt_hi = a.kt_hl + (size_t)bh * 2 * MP * D;
  const uint16_t* kt_lo = kt_hi + MP * D;
  const uint16_t* y_hi = a.y_hl + (size_t)bh * 2 * MP * D;
  const uint16_t* y_lo = y_hi + MP * D;
  const uint16_t* kT_hi = a.ktT_hl + (size_t)bh * 2 * D * MP;
  const uint16_t* kT_lo = kT_hi + D * MP;
  float* dqp = a.dq_part + (size_t)bh * a.n * D;
  const float sl = a.scale_log2e;

  f32x16 red[RPW];
#pragma unroll
  for (int u = 0; u < RPW; ++u) red[u] = zero16();

  for (int t0 = tb; t0 < te; t0 += T) {
    const int tw = t0 + 32 * wave;
    // this wave's Q and dO rows, row-major (zeros past the chunk's valid end), staged for
    // the reduction at the end of the step
    Rows32<D> rq, ro;
    rq.load(q, tw, te, lane);
    ro.load(dO, tw, te, lane);
    // S = Q Kt^T and dF = dO Y^T for 32 tokens: lane = landmark, registers = tokens
    const int trow = min(tw + r32, L - 1);
    f32x16 sc[LT], df[LT];
#pragma unroll
    for (int lt = 0; lt < LT; ++lt) {
      const size_t kr = (size_t)(32 * lt + r32) * D;
      sc[lt] = mma_rows<D, false, true>(zero16(), q + (size_t)trow * D, nullptr, kt_hi + kr,
                                        kt_lo + kr, h);
      df[lt] = mma_rows<D, false, true>(zero16(), dO + (size_t)trow * D, nullptr, y_hi + kr,
                                        y_lo + kr, h);
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const bool tv = tw + acc_r(rr, h) < te;
      float x[LT], mx = kNegBig;
#pragma unroll
      for (int lt = 0; lt < LT; ++lt) {
        x[lt] = (32 * lt + r32 < m) ? sc[lt][rr] * sl : kNegBig;
        mx = fmaxf(mx, x[lt]);
      }
      mx = half_max(mx);
      float sum = 0.f;
#pragma unroll
      for (int lt = 0; lt < LT; ++lt) {
        x[lt] = (32 * lt + r32 < m) ? fast_exp2(x[lt] - mx) : 0.f;
        sum += x[lt];
      }
      const float inv = 1.f / half_sum(sum);
      float dsum = 0.f;
#pragma unroll
      for (int lt = 0; lt < LT; ++lt) {
        x[lt] *= inv;
        dsum += x[lt] * df[lt][rr];
      }
      dsum = half_sum(dsum);
#pragma unroll
      for (int lt = 0; lt < LT; ++lt) {
        const float f = tv ? x[lt] : 0.f;
        sc[lt][rr] = f;
        df[lt][rr] = tv ? f * (df[lt][rr] - dsum) : 0.f;
      }
    }
#pragma unroll
    for (int lt = 0; lt < LT; ++lt) {
      store_cols_hl(ft_hi, ft_lo, TP, 32 * wave, 32 * lt, sc[lt], lane);
      store_cols_hl(st_hi, st_lo, TP, 32 * wave, 32 * lt, df[lt], lane);
      store_rows_hl(ds_hi, ds_lo, MPP, 0, 32 * lt, df[lt], lane);
    }
    // dQ (first term) = s dSF Kt for the wave's 32 tokens
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      const size_t br = (size_t)(32 * ft + r32) * MP;
      const f32x16 acc = mma_rows<MP, true, true>(zero16(), ds_hi + r32 * MPP, ds_lo + r32 * MPP,
                                                  kT_hi + br, kT_lo + br, h);
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int tok = tw + acc_r(rr, h);
        if (tok < te) dqp[(size_t)tok * D + 32 * ft + r32] = a.scale * acc[rr];
      }
    }
    rq.store(qR + 32 * wave * DP, DP, tw, te, lane);
    ro.store(oR + 32 * wave * DP, DP, tw, te, lane);
    __syncthreads();
    // partial dY = F^T dO and dSF^T Q over the step's T tokens
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      const int ti = wave + NW * u;
      if (ti < NRED) {
        const int which = ti / (LT * FT), rem = ti % (LT * FT), at = rem / FT, bt = rem % FT;
        const uint16_t* ah = (which == 0 ? ft_hi : st_hi) + (32 * at + r32) * TP;
        const uint16_t* alo = (which == 0 ? ft_lo : st_lo) + (32 * at + r32) * TP;
        red[u] = mma_rows_btr<T, true>(red[u], ah, alo, which == 0 ? oR : qR, DP, 32 * bt, lane);
      }
    }
    __syncthreads();
  }
  float* part = a.part1 + ((size_t)bh * a.C + c) * 2 * MP * D;
#pragma unroll
  for (int u = 0; u < RPW; ++u) {
    const int ti = wave + NW * u;
    if (ti < NRED) {
      const int which = ti / (LT * FT), rem = ti % (LT * FT), at = rem / FT, bt = rem % FT;
      store_rows_f32(part + (size_t)which * MP * D, D, 32 * at, 32 * bt, red[u], lane);
    }
  }
}

// ======================================================================= L2
template <int D, int MP>
__global__ __launch_bounds__(kBwdThreads) void bwd_land_bwd_kernel(BwdArgs a) {
  extern __shared__ __align__(16) float smem[];
  constexpr int LM = MP + 4, LD = D + 4;  // 16-byte rows
  const int bh = blockIdx.x, m = a.m, tid = threadIdx.x;
  const size_t mm2 = (size_t)MP * MP;
  __shared__ float sred[kBwdThreads / 64];
  // phase 1: dY, W, Z_T -> dZ = dY W^T, dW = Z_T^T dY
  float* rdY = smem;                  // [MP][LD]
  float* rW = rdY + MP * LD;          // [MP][LD]
  float* rZ = rW + MP * LD;           // [MP][LM]
  float* rdZ = rZ + MP * LM;          // [MP][LM]
  float* rdW = rdZ + MP * LM;         // [MP][LD]
  const float* p1 = a.part1 + (size_t)bh * a.C * 2 * MP * D;
  blk_sum4<MP, D>(rdY, LD, p1, (size_t)2 * MP * D, a.C, 1.f);
  const float* wg = a.w + (size_t)bh * MP * D;
  blk_load4<MP, D>(rW, LD, wg, D);
  const float* zT = a.zs + ((size_t)bh * (a.iters + 1) + a.iters) * mm2;
  blk_load4<MP, MP>(rZ, LM, zT, MP);
  __syncthreads();
  blk_mm<false, true>(rdZ, LM, rdY, LD, rW, LD, MP, MP, D, 1.f, 0.f);
  blk_mm<true, false>(rdW, LD, rZ, LM, rdY, LD, MP, D, MP, 1.f, 0.f);
  __syncthreads();
  if (tid < MP) {
    float acc = 0.f;
    for (int f = 0; f < D; ++f) acc += rdW[tid * LD + f] * rW[tid * LD + f];
    a.db[(size_t)bh * MP + tid] = acc;
  }
  blk_split_out<false>(a.dw_hl + (size_t)bh * 2 * MP * D, rdW, LD, MP, D);
  blk_split_out<true, true>(a.dwT_hl + (size_t)bh * 2 * D * MP, rdW, LD, MP, D);
  // dZ into registers (the loop's buffers overlap phase 1)
  constexpr int PER = (MP * MP + kBwdThreads - 1) / kBwdThreads;
  float g0[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + kBwdThreads * u;
    g0[u] = e < MP * MP ? rdZ[(e / MP) * LM + e % MP] : 0.f;
  }
  __syncthreads();
  // phase 2: reverse sweep of the iteration
  float* Am = smem;
  float* dA = Am + MP * LM;
  float* G = dA + MP * LM;
  float* Xb = G + MP * LM;
  float* Zb = Xb + MP * LM;
  float* B1 = Zb + MP * LM;
  float* B2 = B1 + MP * LM;
  float* B3 = B2 + MP * LM;
  float* B4 = B3 + MP * LM;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + kBwdThreads * u;
    if (e < MP * MP) G[(e / MP) * LM + e % MP] = g0[u];
  }
  blk_load4<MP, MP>(Am, LM, a.a_s + (size_t)bh * mm2, MP);
  for (int e = tid; e < MP * LM; e += blockDim.x) dA[e] = 0.f;
  const float* zs = a.zs + (size_t)bh * (a.iters + 1) * mm2;
  const float* xs = a.xs + (size_t)bh * a.iters * mm2;
  for (int it = a.iters - 1; it >= 0; --it) {
    blk_load4<MP, MP>(Xb, LM, xs + it * mm2, MP);
    blk_load4<MP, MP>(Zb, LM, zs + it * mm2, MP);
    __syncthreads();
    for (int e = tid; e < MP * MP; e += blockDim.x) {  // P = 7I - X
      const int i = e / MP, j = e % MP;
      B1[i * LM + j] = ((i == j && i < m) ? 7.f : 0.f) - Xb[i * LM + j];
    }
    __syncthreads();
    blk_mm<false, false>(B2, LM, Xb, LM, B1, LM, MP, MP, MP, -1.f, 0.f);
    __syncthreads();
    blk_eye(B2, LM, MP, m, 15.f, 1.f);                          // Qm = 15I - X P
    __syncthreads();
    blk_mm<false, false>(B3, LM, Xb, LM, B2, LM, MP, MP, MP, -1.f, 0.f);
    __syncthreads();
    blk_eye(B3, LM, MP, m, 13.f, 1.f);                          // R = 13I - X Qm
    __syncthreads();
    blk_mm<false, true>(B4, LM, G, LM, B3, LM, MP, MP, MP, 0.25f, 0.f);   // G_new = G R^T / 4
    __syncthreads();
    blk_mm<true, false>(B3, LM, Zb, LM, G, LM, MP, MP, MP, 0.25f, 0.f);   // dR = Z^T G / 4
    __syncthreads();
    blk_mm<false, true>(G, LM, B3, LM, B2, LM, MP, MP, MP, -1.f, 0.f);    // dX = -dR Qm^T
    __syncthreads();
    blk_mm<true, false>(B2, LM, Xb, LM, B3, LM, MP, MP, MP, -1.f, 0.f);   // dQm = -X^T dR
    __syncthreads();
    blk_mm<false, true>(G, LM, B2, LM, B1, LM, MP, MP, MP, -1.f, 1.f);    // dX -= dQm P^T
    blk_mm<true, false>(B3, LM, Xb, LM, B2, LM, MP, MP, MP, -1.f, 0.f);   // dP = -X^T dQm
    __syncthreads();
    for (int e = tid; e < MP * MP; e += blockDim.x) {             // dX -= dP
      const int i = e / MP, j = e % MP;
      G[i * LM + j] -= B3[i * LM + j];
    }
    __syncthreads();
    blk_mm<false, true>(dA, LM, G, LM, Zb, LM, MP, MP, MP, 1.f, 1.f);     // dA += dX Z^T
    blk_mm<true, false>(B4, LM, Am, LM, G, LM, MP, MP, MP, 1.f, 1.f);     // G_new += A^T dX
    __syncthreads();
    float* t = G;
    G = B4;
    B4 = t;
  }
  // Z_0 = alpha A^T: dA += alpha G^T, d alpha = <G, A^T>, alpha = 1 / (c r)
  const float al = a.alpha[4 * bh], cmax = a.alpha[4 * bh + 1], rmax = a.alpha[4 * bh + 2];
  const int jc = a.amax[2 * bh], ir = a.amax[2 * bh + 1];
  float part = 0.f;
  for (int e = tid; e < MP * MP; e += blockDim.x) {
    const int i = e / MP, j = e % MP;
    part += G[i * LM + j] * Am[j * LM + i];
  }
  part = wave_sum(part);
  if ((tid & 63) == 0) sred[tid >> 6] = part;
  __syncthreads();
  float dal = 0.f;
#pragma unroll
  for (int w = 0; w < kBwdThreads / 64; ++w) dal += sred[w];
  for (int e = tid; e < MP * MP; e += blockDim.x) {
    const int i = e / MP, j = e % MP;
    float v = dA[i * LM + j] + al * G[j * LM + i];
    if (i < m && j < m) {
      if (j == jc) v -= dal * al / cmax;
      if (i == ir) v -= dal * al / rmax;
    }
    dA[i * LM + j] = v;
  }
  __syncthreads();
  // dSA = A o (dA - rowsum(A o dA)) into Xb
  if (tid < MP) {
    const int i = tid;
    float rs = 0.f;
    for (int j = 0; j < MP; ++j) rs += Am[i * LM + j] * dA[i * LM + j];
    for (int j = 0; j < MP; ++j)
      Xb[i * LM + j] = (i < m && j < m) ? Am[i * LM + j] * (dA[i * LM + j] - rs) : 0.f;
  }
  __syncthreads();
  // dQt (A_S path) = s dSA Kt -> global; dKt = s dSA^T Qt + s sum_c (dSF^T Q)_c
  blk_mm<false, false>(a.dqt + (size_t)bh * MP * D, D, Xb, LM, a.kt + (size_t)bh * MP * D, D,
                       MP, D, MP, a.scale, 0.f);
  float* rK = B1;  // [MP][LD] over B1.. (dead)
  blk_sum4<MP, D>(rK, LD, p1 + (size_t)MP * D, (size_t)2 * MP * D, a.C, a.scale);
  __syncthreads();
  blk_mm<true, false>(rK, LD, Xb, LM, a.qt + (size_t)bh * MP * D, D, MP, D, MP, a.scale, 1.f);
  __syncthreads();
  blk_copy_out(a.dkt + (size_t)bh * MP * D, D, rK, LD, MP, D);
}

// ======================================================================= pass 2
// Transposed orientation: S^T = Qt K^T and dB^T = dW V^T put each token on a lane and its
// landmarks in the accumulator registers (landmark 32 lt + 8 (r/4) + 4 h + r % 4 in
// register r of lane half h). B and dSB then feed dK^T = Qt^T dSB and dV^T = dW^T B as
// B operands straight from the registers; Qt^T and dW^T are stored with each group of 16
// landmarks in that register order (kslot_perm). Only dSB^T goes through LDS, for the
// reduction over tokens.
template <int D, int MP, int NW>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void bwd_pass2_kernel(BwdArgs a) {
  constexpr int T = 32 * NW, LT = MP / 32, FT = D / 32;
  constexpr int NRED = LT * FT, RPW = (NRED + NW - 1) / NW;
  constexpr int TP = T + 8, DP = D + 8;  // LDS rows padded by 16 bytes (bank spread)
  extern __shared__ __align__(16) char lds[];
  uint16_t* sT_hi = reinterpret_cast<uint16_t*>(lds);  // dSB [MP][TP] (landmark rows)
  uint16_t* sT_lo = sT_hi + MP * TP;
  uint16_t* kR = sT_lo + MP * TP;                       // K   [T][DP] (step's tokens)
  float* smx = reinterpret_cast<float*>(kR + T * DP);  // per landmark: max, 1/sum, D_B
  float* sinv = smx + MP;
  float* sdb = sinv + MP;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, r32 = lane & 31;
  int bh, c;
  xcd_map(blockIdx.x, a.BH, a.C, bh, c);
  const int m = a.m, L = valid_length(a.lengths, bh, a.H, a.n, a.m);
  const int tb = c * a.chunk, te = min(tb + a.chunk, L);
  const uint16_t* kk = a.k + (size_t)bh * a.n * D;
  const uint16_t* vv = a.v + (size_t)bh * a.n * D;
  const uint16_t* qt_hi = a.qt_hl + (size_t)bh * 2 * MP * D;
  const uint16_t* qt_lo = qt_hi + MP * D;
  const uint16_t* dw_hi = a.dw_hl + (size_t)bh * 2 * MP * D;
  const uint16_t* dw_lo = dw_hi + MP * D;
  const uint16_t* qT_hi = a.qtT_hl + (size_t)bh * 2 * D * MP;
  const uint16_t* qT_lo = qT_hi + D * MP;
  const uint16_t* wT_hi = a.dwT_hl + (size_t)bh * 2 * D * MP;
  const uint16_t* wT_lo = wT_hi + D * MP;
  const float* dkt = a.dkt + (size_t)bh * MP * D;
  uint16_t* dk = a.dk + (size_t)bh * a.n * D;
  float* dvp = a.dv_part + (size_t)bh * a.n * D;
  const float sl = a.scale_log2e;
  for (int j = threadIdx.x; j < MP; j += blockDim.x) {
    const float* stat = a.stat + (size_t)bh * 2 * MP;
    smx[j] = stat[j];
    sinv[j] = 1.f / stat[MP + j];
    sdb[j] = a.db[(size_t)bh * MP + j];
  }
  __syncthreads();
  f32x16 red[RPW];
#pragma unroll
  for (int u = 0; u < RPW; ++u) red[u] = zero16();

  for (int t0 = tb; t0 < te; t0 += T) {
    const int tw = t0 + 32 * wave, tok = tw + r32;  // the lane's token
    const bool tv = tok < te;
    Rows32<D> rk;  // the wave's K rows, staged for the reduction below
    rk.load(kk, tw, te, lane);
    const int trow = min(tok, L - 1);
    f32x16 sb[LT], db[LT];  // B and dSB: landmark rows, this lane's token
#pragma unroll
    for (int lt = 0; lt < LT; ++lt) {
      const size_t lr = (size_t)(32 * lt + r32) * D;
      sb[lt] = mma_rows<D, true, false>(zero16(), qt_hi + lr, qt_lo + lr, kk + (size_t)trow * D,
                                        nullptr, h);
      db[lt] = mma_rows<D, true, false>(zero16(), dw_hi + lr, dw_lo + lr, vv + (size_t)trow * D,
                                        nullptr, h);
    }
#pragma unroll
    for (int lt = 0; lt < LT; ++lt) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int j = 32 * lt + acc_r(rr, h);
        const bool v = tv && j < m;
        const float b = v ? fast_exp2(sb[lt][rr] * sl - smx[j]) * sinv[j] : 0.f;
        sb[lt][rr] = b;
        db[lt][rr] = v ? b * (db[lt][rr] - sdb[j]) : 0.f;
      }
      store_rows_hl(sT_hi, sT_lo, TP, 32 * lt, 32 * wave, db[lt], lane);
    }
    // B operands from the registers: k-step s covers landmarks 16 s .. 16 s + 15, held in
    // registers 8 (s % 2) .. 8 (s % 2) + 7 of tile s / 2
    Pair8 pb[2 * LT], pd[2 * LT];
#pragma unroll
    for (int s = 0; s < 2 * LT; ++s) {
      float x[8], y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = sb[s / 2][8 * (s % 2) + e];
        y[e] = db[s / 2][8 * (s % 2) + e];
      }
      pb[s] = split8(x);
      pd[s] = split8(y);
    }
    const int segj = seg_of(min(tok, L - 1), L, m);
    const float seginv = 1.f / (float)(seg_start(segj + 1, L, m) - seg_start(segj, L, m));
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      f32x16 gk = zero16(), gv = zero16();
#pragma unroll
      for (int s = 0; s < 2 * LT; ++s) {
        const size_t ar = (size_t)(32 * ft + r32) * MP + 16 * s + 8 * h;
        gk = mfma_pair<true, true>(Pair8{ld8(qT_hi + ar), ld8(qT_lo + ar)}, pd[s], gk);
        gv = mfma_pair<true, true>(Pair8{ld8(wT_hi + ar), ld8(wT_lo + ar)}, pb[s], gv);
      }
      if (tv) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int f0 = 32 * ft + 8 * g4 + 4 * h;
          const f32x4 kt4 = *reinterpret_cast<const f32x4*>(dkt + (size_t)segj * D + f0);
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = a.scale * gk[4 * g4 + e] + kt4[e] * seginv;
          const bf16x2 lo2 = bf16_rne2(x[0], x[1]), hi2 = bf16_rne2(x[2], x[3]);
          *reinterpret_cast<u32x2*>(dk + (size_t)tok * D + f0) =
              u32x2{__builtin_bit_cast(uint32_t, lo2), __builtin_bit_cast(uint32_t, hi2)};
          *reinterpret_cast<f32x4*>(dvp + (size_t)tok * D + f0) =
              f32x4{gv[4 * g4], gv[4 * g4 + 1], gv[4 * g4 + 2], gv[4 * g4 + 3]};
        }
      }
    }
    rk.store(kR + 32 * wave * DP, DP, tw, te, lane);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      const int ti = wave + NW * u;
      if (ti < NRED) {
        const int at = ti / FT, bt = ti % FT;
        red[u] = mma_rows_btr<T, true>(red[u], sT_hi + (32 * at + r32) * TP,
                                       sT_lo + (32 * at + r32) * TP, kR, DP, 32 * bt, lane);
      }
    }
    __syncthreads();
  }
  float* part = a.part2 + ((size_t)bh * a.C + c) * MP * D;
#pragma unroll
  for (int u = 0; u < RPW; ++u) {
    const int ti = wave + NW * u;
    if (ti < NRED) store_rows_f32(part, D, 32 * (ti / FT), 32 * (ti % FT), red[u], lane);
  }
  // padding rows of this chunk: dK = 0
  const int zb = max(tb, L), ze = min(tb + a.chunk, a.n);
  for (int e = threadIdx.x; e < (ze > zb ? (ze - zb) * D : 0); e += blockDim.x)
    dk[(size_t)zb * D + e] = 0;
}

// ======================================================================= final pass
constexpr int kFinTok = 128;  // tokens per block
constexpr int kFinRows = kFinTok + 64;  // staged rows: the tile, its halo and the
                                        // dw band's last column tile (zero past the halo)

template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_final_kernel(BwdArgs a) {
  extern __shared__ __align__(16) char lds[];
  const int W = a.W, half = (W - 1) / 2, R = kFinTok + W - 1, MP = a.mp, m = a.m;
  uint16_t* so = reinterpret_cast<uint16_t*>(lds);   // dO rows t0 - half .. [kFinRows][D]
  uint16_t* sv = so + kFinRows * D;                  // V rows  t0 - half .. [kFinRows][D]
  float* sq = reinterpret_cast<float*>(sv + kFinRows * D);  // dQt / |seg| per segment
  float* sw = sq + a.fin_segs * D;                   // conv taps [W]
  float* sdw = sw + 65;                              // dw sums [W]
  int* srow = reinterpret_cast<int*>(sdw + 4 * 65);  // per token: its dQt row offset
  int bh, c3;
  xcd_map(blockIdx.x, a.BH, a.C3, bh, c3);
  const int L = valid_length(a.lengths, bh, a.H, a.n, a.m), hh = bh % a.H;
  const int t0 = c3 * kFinTok, t1 = min(t0 + kFinTok, a.n), tv = min(t1, L);
  const uint16_t* dO = a.dout + (size_t)bh * a.n * D;
  const uint16_t* vv = a.v + (size_t)bh * a.n * D;
  // staged rows, zeros outside [0, L) and past R: loads from rows clamped into [0, L) in
  // batches of kSB per thread, every load of a batch in flight before its first LDS write
  // (a load under a condition compiles into a branch closed by a wait for everything)
  {
    constexpr int NST = (kFinRows * (D / 8) + kBwdThreads - 1) / kBwdThreads, kSB = 3;
#pragma unroll
    for (int u0 = 0; u0 < NST; u0 += kSB) {
      u32x4 ov[kSB], vw[kSB];
#pragma unroll
      for (int u = 0; u < kSB; ++u) {
        const int e = threadIdx.x + kBwdThreads * (u0 + u < NST ? u0 + u : 0);
        const int r = e / (D / 8), f8 = (e % (D / 8)) * 8, tok = t0 - half + r;
        const int tc = tok < 0 ? 0 : (tok < L ? tok : L - 1);
        ov[u] = *reinterpret_cast<const u32x4*>(dO + (size_t)tc * D + f8);
        vw[u] = *reinterpret_cast<const u32x4*>(vv + (size_t)tc * D + f8);
      }
#pragma unroll
      for (int u = 0; u < kSB; ++u) {
        const int e = threadIdx.x + kBwdThreads * (u0 + u);
        const int r = e / (D / 8), f8 = (e % (D / 8)) * 8, tok = t0 - half + r;
        asm volatile("" : "+v"(ov[u]), "+v"(vw[u]));
        const bool ok = r < R && tok >= 0 && tok < L;
        if (u0 + u < NST && e < kFinRows * (D / 8)) {
          *reinterpret_cast<u32x4*>(so + r * D + f8) = ok ? ov[u] : u32x4{0u, 0u, 0u, 0u};
          *reinterpret_cast<u32x4*>(sv + r * D + f8) = ok ? vw[u] : u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  }
  const int j0 = tv > t0 ? seg_of(t0, L, m) : 0;
  const int j1 = tv > t0 ? seg_of(tv - 1, L, m) : -1;
  const float* dqt = a.dqt + (size_t)bh * MP * D;
  const float* p2 = a.part2 + (size_t)bh * a.C * MP * D;
  for (int e = threadIdx.x; e < (j1 - j0 + 1) * D; e += blockDim.x) {
    const int j = j0 + e / D, f = e % D;
    // chunk partials summed in chunk order, four loads in flight at a time
    float acc = 0.f;
    int c = 0;
    for (; c + 4 <= a.C; c += 4) {
      float x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = p2[((size_t)(c + u) * MP + j) * D + f];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += x[u];
    }
    for (; c < a.C; ++c) acc += p2[((size_t)c * MP + j) * D + f];
    const float len = (float)(seg_start(j + 1, L, m) - seg_start(j, L, m));
    sq[(j - j0) * D + f] = (dqt[(size_t)j * D + f] + a.scale * acc) / len;
  }
  for (int k = threadIdx.x; k < W; k += blockDim.x) {
    sw[k] = a.conv_w[hh * W + k];
    sdw[k] = 0.f;
  }
  for (int i = threadIdx.x; i < kFinTok; i += blockDim.x)
    srow[i] = t0 + i < tv ? (seg_of(t0 + i, L, m) - j0) * D : 0;
  __syncthreads();
  const float* dqp = a.dq_part + (size_t)bh * a.n * D;
  const float* dvp = a.dv_part + (size_t)bh * a.n * D;
  uint16_t* dq = a.dq + (size_t)bh * a.n * D;
  uint16_t* dv = a.dv + (size_t)bh * a.n * D;
  // thread = (token i, features f0 .. f0 + 7): dQ and dV, 16-byte loads and stores; the
  // transposed conv reads one 16-byte dO run per tap
  constexpr int NE8 = kFinTok * (D / 8) / kBwdThreads;
  auto cvt8 = [](const float* x) {
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = __builtin_bit_cast(uint32_t, bf16_rne2(x[2 * e], x[2 * e + 1]));
    return r;
  };
#pragma unroll 2
  for (int u = 0; u < NE8; ++u) {
    const int e = threadIdx.x + kBwdThreads * u, i = e / (D / 8), f0 = (e % (D / 8)) * 8;
    const int t = t0 + i;
    if (t >= t1) continue;
    u32x4 oq{0u, 0u, 0u, 0u}, ov{0u, 0u, 0u, 0u};
    if (t < tv) {
      const f32x4 q0 = *reinterpret_cast<const f32x4*>(dqp + (size_t)t * D + f0);
      const f32x4 q1 = *reinterpret_cast<const f32x4*>(dqp + (size_t)t * D + f0 + 4);
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(dvp + (size_t)t * D + f0);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(dvp + (size_t)t * D + f0 + 4);
      const float* sqr = sq + srow[i] + f0;
      float xq[8], acc[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xq[q] = q0[q] + sqr[q];
        xq[4 + q] = q1[q] + sqr[4 + q];
        acc[q] = v0[q];
        acc[4 + q] = v1[q];
      }
      // d out[t'] / d V[t] = w[k] for t' = t - k + half: staged row i + 2 half - k
      const uint16_t* op = so + (i + 2 * half) * D + f0;
      for (int k = 0; k < W; ++k) {
        const bf16x8 r = ld8(op - k * D);
        const float wk = sw[k];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += wk * (float)r[q];  // exact widening
      }
      oq = cvt8(xq);
      ov = cvt8(acc);
    }
    *reinterpret_cast<u32x4*>(dq + (size_t)t * D + f0) = oq;
    *reinterpret_cast<u32x4*>(dv + (size_t)t * D + f0) = ov;
  }
  // dw[k] = sum over rows i < tv - t0 of G[i][i + k], G = dO_tile V_ext^T on MFMA (wave w:
  // rows 32 w .. 32 w + 31, the column tiles that meet the band 0 <= j - i < W)
  {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, r32 = lane & 31;
    const int nvalid = tv - t0;
    if (32 * wave < nvalid) {
      const int tj1 = wave + (30 + W) / 32;
      for (int tj = wave; tj <= tj1; ++tj) {
        f32x16 g = zero16();
        g = mma_rows<D, false, false>(g, so + (32 * wave + r32 + half) * D, nullptr,
                                      sv + (32 * tj + r32) * D, nullptr, h);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int i = 32 * wave + acc_r(rr, h), k = 32 * tj + r32 - i;
          if (k >= 0 && k < W && i < nvalid) atomicAdd(&sdw[k], g[rr]);
        }
      }
    }
  }
  __syncthreads();
  for (int k = threadIdx.x; k < W; k += blockDim.x)
    a.part_dw[((size_t)bh * a.C3 + c3) * W + k] = sdw[k];
}

__global__ __launch_bounds__(kBwdThreads) void bwd_dw_kernel(BwdArgs a) {
  __shared__ float sred[kBwdThreads / 64];
  const int hh = blockIdx.x / a.W, k = blockIdx.x % a.W;
  float s = 0.f;
  for (int e = threadIdx.x; e < a.B * a.C3; e += blockDim.x) {
    const int b = e / a.C3, c = e % a.C3;
    s += a.part_dw[(((size_t)b * a.H + hh) * a.C3 + c) * a.W + k];
  }
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) sred[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < kBwdThreads / 64; ++w) t += sred[w];
    a.dconv_w[hh * a.W + k] = t;
  }
}

// ======================================================================= host side
template <int D, int MP>
struct BwdShape {
  static constexpr int NW = D == 128 ? 2 : 4;
  static constexpr int T = 32 * NW;
  static constexpr size_t l1 = (5 * MP * (MP + 4) + 2 * MP * (D + 4)) * 4;
  static constexpr size_t l2a = 9 * MP * (MP + 4), l2b = 3 * MP * (D + 4) + 2 * MP * (MP + 4);
  static constexpr size_t l2 = (l2a > l2b ? l2a : l2b) * 4;
  static constexpr size_t p1 =
      ((size_t)4 * MP * (T + 8) + 2 * (D + 8) * T + NW * 2 * 32 * (MP + 8)) * 2;
  static constexpr size_t p2 = ((size_t)2 * MP * (T + 8) + (size_t)T * (D + 8)) * 2 + 3 * MP * 4;
  static constexpr size_t fin_bytes(int segs) {
    return (size_t)2 * kFinRows * D * 2 + ((size_t)segs * D + 65 + 4 * 65 + kFinTok) * 4;
  }
  static constexpr size_t fin = fin_bytes(MP);  // the most any plan asks for
};

template <int D, int MP>
static hipError_t configure_bwd_t() {
  using S = BwdShape<D, MP>;
  const void* fns[] = {reinterpret_cast<const void*>(&bwd_land_fwd_kernel<D, MP>),
                       reinterpret_cast<const void*>(&bwd_land_bwd_kernel<D, MP>),
                       reinterpret_cast<const void*>(&bwd_pass1_kernel<D, MP, S::NW>),
                       reinterpret_cast<const void*>(&bwd_pass2_kernel<D, MP, S::NW>),
                       reinterpret_cast<const void*>(&bwd_final_kernel<D>)};
  const size_t bytes[] = {S::l1, S::l2, S::p1, S::p2, S::fin};
  for (int i = 0; i < 5; ++i) {
    const hipError_t e = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)bytes[i]);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t configure_backward() {
  hipError_t e;
  if ((e = configure_bwd_t<32, 32>()) != hipSuccess) return e;
  if ((e = configure_bwd_t<32, 64>()) != hipSuccess) return e;
  if ((e = configure_bwd_t<64, 32>()) != hipSuccess) return e;
  if ((e = configure_bwd_t<64, 64>()) != hipSuccess) return e;
  if ((e = configure_bwd_t<128, 32>()) != hipSuccess) return e;
  return configure_bwd_t<128, 64>();
}

template <int D, int MP>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  using S = BwdShape<D, MP>;
  const int BH = a.BH;
  hipLaunchKernelGGL((bwd_land_fwd_kernel<D, MP>), dim3(BH), dim3(kBwdThreads), S::l1, s, a);
  hipLaunchKernelGGL((bwd_pass1_kernel<D, MP, S::NW>), dim3(BH * a.C), dim3(64 * S::NW), S::p1,
                     s, a);
  hipLaunchKernelGGL((bwd_land_bwd_kernel<D, MP>), dim3(BH), dim3(kBwdThreads), S::l2, s, a);
  hipLaunchKernelGGL((bwd_pass2_kernel<D, MP, S::NW>), dim3(BH * a.C), dim3(64 * S::NW), S::p2,
                     s, a);
  // the table holds only the segments a token tile can meet: with less LDS per block, three
  // blocks share a CU at d = 64
  hipLaunchKernelGGL((bwd_final_kernel<D>), dim3(BH * a.C3), dim3(kBwdThreads),
                     S::fin_bytes(a.fin_segs), s, a);
  hipLaunchKernelGGL(bwd_dw_kernel, dim3(a.H * a.W), dim3(kBwdThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_backward(const BwdArgs& a, hipStream_t s) {
  if (a.mp == 32) {
    if (a.d == 32) return launch_bwd_t<32, 32>(a, s);
    if (a.d == 64) return launch_bwd_t<64, 32>(a, s);
    return launch_bwd_t<128, 32>(a, s);
  }
  if (a.d == 32) return launch_bwd_t<32, 64>(a, s);
  if (a.d == 64) return launch_bwd_t<64, 64>(a, s);
  return launch_bwd_t<128, 64>(a, s);
}

}  // namespace nys
