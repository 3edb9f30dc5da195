// General backward pass of the Nystrom self-attention (Nystromformer review page,
// "Proposed method", bullets M1..M6): the gradients of L = sum(out * dout) for any shape
// the forward supports (m up to 256, fp32 or bf16 I/O, padded batches), as a sequence of
// batched fp32 products and small row and element kernels. The fused kernels of
// backward.hip cover bf16 with m <= 64; this path covers the rest.
//
// Per (batch, head) with valid length L, s = 1/sqrt(d), landmarks Qt, Kt from the
// forward's segment-means kernel:
//   F = softmax_row(s Q Kt^T) [n][mp]     A = softmax_row(s Qt Kt^T) [mp][mp]
//   B = softmax_row(s Qt K^T) [mp][n]     W = B V, Z_0 = alpha A^T, T steps of
//   X = A Z, P = 7I - X, Q1 = 15I - X P, R = 13I - X Q1, Z' = Z R / 4 (Z_k, X_k kept),
//   Y = Z_T W, then
//   dF = dO Y^T, dSF = F o (dF - rowsum(F o dF)), dQ = s dSF Kt, dKt = s dSF^T Q,
//   dY = F^T dO, dZ = dY W^T, dW = Z_T^T dY, the reverse sweep through the steps to dA,
//   the alpha term, dSA = A o (dA - rowsum(A o dA)), dQt = s dSA Kt, dKt += s dSA^T Qt,
//   dB = dW V^T, dSB = B o (dB - rowsum(B o dB)), dK = s dSB^T Qt, dQt += s dSB K,
//   dV = B^T dW + conv^T(dO), dQ += dQt[seg(t)] / |seg|, dK += dKt[seg(t)] / |seg|,
//   dw[k] = sum_t dO[t] . V[t + k - (W-1)/2].
// F and B are held whole (n x mp per head: memory linear in n). Rows and columns of
// token index t >= L are zero everywhere; padding rows of q, k, v and dout are not read.
#include "nys_common.h"
#include "nys_kernels.h"

namespace nys {

// ------------------------------------------------------------------ batched product
// C[b] = alpha op(A[b]) op(B[b]) + beta C[b] + diag I (diagonal entries i = j < diag_n),
// C fp32 M x N (ldc), op(A) M x K: A stored [M][K] (lda) or, with TA, [K][M]; op(B)
// K x N: B stored [K][N] (ldb) or, with TB, [N][K]. Element types float or bf16 bits.
// 64 x 64 output tiles per block, 32-deep k slabs staged in LDS (the next slab loaded into
// registers meanwhile), each wave forming a 32 x 32 quarter on fp32 MFMA
// (v_mfma_f32_32x32x2_f32).
// Token masking (mask bits: 1 = M, 2 = N, 4 = K is a token dimension): indices at or
// past the batch entry's valid length read as zero (those memory rows are never read)
// and C entries in masked rows / columns are written as zero.
struct GemmArgs {
  const void* A;
  const void* B;
  float* C;
  long long sA, sB, sC;  // batch strides in elements
  int lda, ldb, ldc;
  int M, N, K;
  float alpha, beta, diag;
  int diag_n;
  int mask;
  const int* lengths;
  int H, n, m;
  // split over K (nsplit > 1): block z covers batch entry z % nbatch and k range
  // [kchunk (z / nbatch), + kchunk), writing its raw partial product to part
  // [nsplit][nbatch][M][N]; split_reduce_kernel then forms C
  float* part;
  int nsplit, kchunk, nbatch;
};

template <typename T>
__device__ __forceinline__ float ld_elem(const T* p);
template <>
__device__ __forceinline__ float ld_elem<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p) {
  return __uint_as_float((uint32_t)*p << 16);
}

// Four consecutive elements as floats in one load (8 bytes of bf16 or 16 of fp32); p
// aligned to four elements.
template <typename T>
__device__ __forceinline__ f32x4 ld4f(const T* p) {
  if constexpr (sizeof(T) == 2) {
    const u32x2 u = *reinterpret_cast<const u32x2*>(p);
    return f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u),
                 __uint_as_float(u[1] << 16), __uint_as_float(u[1] & 0xffff0000u)};
  } else {
    return *reinterpret_cast<const f32x4*>(p);
  }
}

constexpr int kGT = 64, kGK = 32, kGS = kGT + 4;
constexpr int kSplitBlocks = 1024, kSplitMin = 512;  // split-K targets (see Runner::gemm)

template <typename TAe, typename TBe, bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  __shared__ __align__(16) float As[kGK][kGS];
  __shared__ __align__(16) float Bs[kGK][kGS];
  const int split = g.nsplit > 1 ? (int)blockIdx.z / g.nbatch : 0;
  const int b = g.nsplit > 1 ? (int)blockIdx.z % g.nbatch : (int)blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r32 = lane & 31;
  const int wr = wave >> 1, wc = wave & 1;  // this wave's 32 x 32 quarter of the tile
  const int row0 = blockIdx.y * kGT, col0 = blockIdx.x * kGT;
  const int L = valid_length(g.lengths, b, g.H, g.n, g.m);
  const int lm = (g.mask & 1) ? min(g.M, L) : g.M;
  const int ln = (g.mask & 2) ? min(g.N, L) : g.N;
  const int lk0 = (g.mask & 4) ? min(g.K, L) : g.K;
  const int kbeg = split * g.kchunk;
  const int lk = g.nsplit > 1 ? min(lk0, kbeg + g.kchunk) : lk0;
  const TAe* A = static_cast<const TAe*>(g.A) + (size_t)b * g.sA;
  const TBe* B = static_cast<const TBe*>(g.B) + (size_t)b * g.sB;
  f32x16 acc = zero16();
  // the next slab's elements are loaded into registers while the current one is used
  // each thread fetches runs of four elements along the operand's stored contiguous
  // index (one vector load when all four are in range, else element by element)
  constexpr int U4 = kGT * kGK / 1024;
  f32x4 ra[U4], rb[U4];
  // Interior slabs (every run in range, 4-element aligned runs) load without conditions;
  // edge slabs take the element-wise path. A load under a condition compiles into a branch
  // that the compiler closes with a wait for everything in flight, so a slab loaded that
  // way takes several memory round trips.
  const bool runs_aligned =
      ((g.lda | g.ldb) & 3) == 0 && (reinterpret_cast<uintptr_t>(A) & (4 * sizeof(TAe) - 1)) == 0 &&
      (reinterpret_cast<uintptr_t>(B) & (4 * sizeof(TBe) - 1)) == 0;
  const bool tile_in = runs_aligned && row0 + kGT <= lm && col0 + kGT <= ln;
  auto run4 = [](const auto* p, bool all, int nvalid) {
    if (all && (reinterpret_cast<uintptr_t>(p) & (4 * sizeof(*p) - 1)) == 0) return ld4f(p);
    f32x4 x{0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < nvalid; ++q) x[q] = ld_elem(p + q);
    return x;
  };
  auto fetch = [&](int k0) {
    if (tile_in && k0 + kGK <= lk) {
#pragma unroll
      for (int u = 0; u < U4; ++u) {
        const int e = 4 * (tid + 256 * u);
        const int ai = TA ? e % kGT : e / kGK, ak = TA ? e / kGT : e % kGK;
        const int i = row0 + ai, k = k0 + ak;
        ra[u] = ld4f(TA ? A + (size_t)k * g.lda + i : A + (size_t)i * g.lda + k);
        const int bk = TB ? e % kGK : e / kGT, bj = TB ? e / kGK : e % kGT;
        const int jj = col0 + bj, kb = k0 + bk;
        rb[u] = ld4f(TB ? B + (size_t)jj * g.ldb + kb : B + (size_t)kb * g.ldb + jj);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < U4; ++u) {
      const int e = 4 * (tid + 256 * u);
      // A tile: 64 rows x kGK k
      const int ai = TA ? e % kGT : e / kGK, ak = TA ? e / kGT : e % kGK;
      const int i = row0 + ai, k = k0 + ak;
      if (TA) {  // run over i at fixed k
        const int nv = k < lk ? max(0, min(4, lm - i)) : 0;
        ra[u] = nv > 0 ? run4(A + (size_t)k * g.lda + i, nv == 4, nv) : f32x4{0.f, 0.f, 0.f, 0.f};
      } else {  // run over k at fixed i
        const int nv = i < lm ? max(0, min(4, lk - k)) : 0;
        ra[u] = nv > 0 ? run4(A + (size_t)i * g.lda + k, nv == 4, nv) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // B tile: kGK k x 64 columns
      const int bk = TB ? e % kGK : e / kGT, bj = TB ? e / kGK : e % kGT;
      const int jj = col0 + bj, kb = k0 + bk;
      if (TB) {  // run over k at fixed column
        const int nv = jj < ln ? max(0, min(4, lk - kb)) : 0;
        rb[u] = nv > 0 ? run4(B + (size_t)jj * g.ldb + kb, nv == 4, nv) : f32x4{0.f, 0.f, 0.f, 0.f};
      } else {  // run over columns at fixed k
        const int nv = kb < lk ? max(0, min(4, ln - jj)) : 0;
        rb[u] = nv > 0 ? run4(B + (size_t)kb * g.ldb + jj, nv == 4, nv) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  const int kstart = g.nsplit > 1 ? kbeg : 0;
  if (kstart < lk) fetch(kstart);
  for (int k0 = kstart; k0 < lk; k0 += kGK) {
#pragma unroll
    for (int u = 0; u < U4; ++u) {
      const int e = 4 * (tid + 256 * u);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (TA) As[e / kGT][e % kGT + q] = ra[u][q];
        else As[e % kGK + q][e / kGK] = ra[u][q];
        if (TB) Bs[e % kGK + q][e / kGK] = rb[u][q];
        else Bs[e / kGT][e % kGT + q] = rb[u][q];
      }
    }
    __syncthreads();
    if (k0 + kGK < lk) fetch(k0 + kGK);
    // fp32 MFMA over the slab: lane half h takes k-slot h of each pair of k
#pragma unroll
    for (int kk = 0; kk < kGK; kk += 2) {
      const float av = As[kk + (lane >> 5)][32 * wr + r32];
      const float bv = Bs[kk + (lane >> 5)][32 * wc + r32];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  const int j = col0 + 32 * wc + r32;  // the lane's column; rows from acc_row
  if (g.nsplit > 1) {  // raw partial; the reduction applies the epilogue
    float* P = g.part + ((size_t)split * g.nbatch + b) * g.M * g.N;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int i = acc_row(row0 + 32 * wr, rr, lane);
      if (i < g.M && j < g.N) P[(size_t)i * g.N + j] = acc[rr];
    }
    return;
  }
  float* C = g.C + (size_t)b * g.sC;
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int i = acc_row(row0 + 32 * wr, rr, lane);
    if (i >= g.M || j >= g.N) continue;
    float* p = C + (size_t)i * g.ldc + j;
    float v = g.alpha * acc[rr];
    if (g.beta != 0.f) v += g.beta * *p;
    if (i == j && i < g.diag_n) v += g.diag;
    if (i >= lm || j >= ln) v = 0.f;
    *p = v;
  }
}

// C = alpha sum_s part[s] + beta C + diag I for a product split over K, the splits added
// in a fixed order (one thread per element of C).
__global__ __launch_bounds__(256) void split_reduce_kernel(GemmArgs g) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long mn = (long long)g.M * g.N;
  if (e >= mn * g.nbatch) return;
  const int b = (int)(e / mn), r = (int)(e % mn), i = r / g.N, j = r % g.N;
  const int L = valid_length(g.lengths, b, g.H, g.n, g.m);
  const int lm = (g.mask & 1) ? min(g.M, L) : g.M;
  const int ln = (g.mask & 2) ? min(g.N, L) : g.N;
  float v = 0.f;
  for (int sp = 0; sp < g.nsplit; ++sp) v += g.part[((size_t)sp * g.nbatch + b) * mn + r];
  float* p = g.C + (size_t)b * g.sC + (size_t)i * g.ldc + j;
  v *= g.alpha;
  if (g.beta != 0.f) v += g.beta * *p;
  if (i == j && i < g.diag_n) v += g.diag;
  if (i >= lm || j >= ln) v = 0.f;
  *p = v;
}

// ------------------------------------------------------------------ row kernels
// Valid extent of a row/column dimension: 0 = all, 1 = the m landmarks, 2 = the batch
// entry's valid length.
__device__ __forceinline__ int extent(int mode, int full, int m, int L) {
  return mode == 0 ? full : (mode == 1 ? min(full, m) : min(full, L));
}

struct RowArgs {
  float* X;        // [batch][rows][cols] (ld = cols)
  const float* P;  // softmax probabilities (dsoftmax only)
  int rows, cols, rmode, cmode;
  float scale;
  const int* lengths;
  int H, n, m;
};

// In place: X <- softmax over the valid columns of scale * X, per valid row; everything
// else zero. One wave per row.
__global__ __launch_bounds__(256) void row_softmax_kernel(RowArgs a, int nrows_total) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= nrows_total) return;
  const int b = (int)(row / a.rows), r = (int)(row % a.rows);
  const int L = valid_length(a.lengths, b, a.H, a.n, a.m);
  const int vr = extent(a.rmode, a.rows, a.m, L), vc = extent(a.cmode, a.cols, a.m, L);
  float* x = a.X + (size_t)row * a.cols;
  if (a.cols % 4 != 0) {  // rows not 16-byte aligned: one element per lane and access
    if (r >= vr) {
      for (int j = lane; j < a.cols; j += 64) x[j] = 0.f;
      return;
    }
    float mx = kNegBig;
    for (int j = lane; j < vc; j += 64) mx = fmaxf(mx, a.scale * x[j]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int j = lane; j < vc; j += 64) sum += expf(a.scale * x[j] - mx);
    const float inv = 1.f / wave_sum(sum);
    for (int j = lane; j < a.cols; j += 64) x[j] = j < vc ? expf(a.scale * x[j] - mx) * inv : 0.f;
    return;
  }
  if (r >= vr) {
    for (int j = 4 * lane; j < a.cols; j += 256)
      *reinterpret_cast<f32x4*>(x + j) = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  // four consecutive columns per lane and access (cols is a multiple of 4)
  float mx = kNegBig;
  for (int j = 4 * lane; j < vc; j += 256) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(x + j);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (j + q < vc) mx = fmaxf(mx, a.scale * v[q]);
  }
  mx = wave_max(mx);
  float sum = 0.f;
  for (int j = 4 * lane; j < vc; j += 256) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(x + j);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (j + q < vc) sum += expf(a.scale * v[q] - mx);
  }
  const float inv = 1.f / wave_sum(sum);
  for (int j = 4 * lane; j < a.cols; j += 256) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(x + j);
    f32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = j + q < vc ? expf(a.scale * v[q] - mx) * inv : 0.f;
    *reinterpret_cast<f32x4*>(x + j) = o;
  }
}

// In place on the upstream gradient dP of a row softmax P: X <- P o (X - rowsum(P o X)),
// zero outside the valid rows and columns. One wave per row.
__global__ __launch_bounds__(256) void row_dsoftmax_kernel(RowArgs a, int nrows_total) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= nrows_total) return;
  const int b = (int)(row / a.rows), r = (int)(row % a.rows);
  const int L = valid_length(a.lengths, b, a.H, a.n, a.m);
  const int vr = extent(a.rmode, a.rows, a.m, L), vc = extent(a.cmode, a.cols, a.m, L);
  float* x = a.X + (size_t)row * a.cols;
  const float* p = a.P + (size_t)row * a.cols;
  if (a.cols % 4 != 0) {  // rows not 16-byte aligned: one element per lane and access
    if (r >= vr) {
      for (int j = lane; j < a.cols; j += 64) x[j] = 0.f;
      return;
    }
    float dot = 0.f;
    for (int j = lane; j < vc; j += 64) dot += p[j] * x[j];
    dot = wave_sum(dot);
    for (int j = lane; j < a.cols; j += 64) x[j] = j < vc ? p[j] * (x[j] - dot) : 0.f;
    return;
  }
  if (r >= vr) {
    for (int j = 4 * lane; j < a.cols; j += 256)
      *reinterpret_cast<f32x4*>(x + j) = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  float dot = 0.f;
  for (int j = 4 * lane; j < vc; j += 256) {
    const f32x4 pv = *reinterpret_cast<const f32x4*>(p + j), xv = *reinterpret_cast<const f32x4*>(x + j);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (j + q < vc) dot += pv[q] * xv[q];
  }
  dot = wave_sum(dot);
  for (int j = 4 * lane; j < a.cols; j += 256) {
    const f32x4 pv = *reinterpret_cast<const f32x4*>(p + j), xv = *reinterpret_cast<const f32x4*>(x + j);
    f32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = j + q < vc ? pv[q] * (xv[q] - dot) : 0.f;
    *reinterpret_cast<f32x4*>(x + j) = o;
  }
}

// ------------------------------------------------------------------ landmark kernels
// alpha = 1 / (max column abs-sum * max row abs-sum) of A (m x m valid part of mp x mp),
// the maximising column jc and row ir (first index on ties), and Z_0 = alpha A^T.
// One block per head.
__global__ __launch_bounds__(256) void alpha_z0_kernel(const float* A, float* Z0, float* alpha,
                                                       int* amax, int mp, int m,
                                                       long long sZ0) {
  __shared__ float colsum[256], rowsum[256];
  __shared__ float sal;
  const int b = blockIdx.x, tid = threadIdx.x;
  const float* a = A + (size_t)b * mp * mp;
  if (tid < m) {
    float cs = 0.f, rs = 0.f;
    for (int i = 0; i < m; ++i) cs += fabsf(a[(size_t)i * mp + tid]);
    for (int j = 0; j < m; ++j) rs += fabsf(a[(size_t)tid * mp + j]);
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
    alpha[4 * b + 0] = sal;
    alpha[4 * b + 1] = c;
    alpha[4 * b + 2] = r;
    alpha[4 * b + 3] = 0.f;
    amax[2 * b + 0] = jc;
    amax[2 * b + 1] = ir;
  }
  __syncthreads();
  float* z = Z0 + (size_t)b * sZ0;
  for (int e = tid; e < mp * mp; e += blockDim.x) {
    const int i = e / mp, j = e % mp;
    z[e] = sal * a[(size_t)j * mp + i];
  }
}

// Gradient through Z_0 = alpha A^T and alpha = 1 / (c r), c = colsum_jc(|A|),
// r = rowsum_ir(|A|): dA += alpha G0^T, d(alpha) = sum G0 o A^T,
// dA[:, jc] -= d(alpha) alpha / c * sign(A[:, jc]), dA[ir, :] -= d(alpha) alpha / r * sign.
// One block per head; dA [mp][mp] updated in place.
__global__ __launch_bounds__(256) void alpha_backward_kernel(const float* A, const float* G0,
                                                             long long sG0, float* dA,
                                                             const float* alpha, const int* amax,
                                                             int mp, int m) {
  __shared__ float red[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  const float* a = A + (size_t)b * mp * mp;
  const float* g = G0 + (size_t)b * sG0;
  float* da = dA + (size_t)b * mp * mp;
  const float al = alpha[4 * b], c = alpha[4 * b + 1], r = alpha[4 * b + 2];
  const int jc = amax[2 * b], ir = amax[2 * b + 1];
  float part = 0.f;
  for (int e = tid; e < mp * mp; e += blockDim.x) {
    const int i = e / mp, j = e % mp;
    part += g[e] * a[(size_t)j * mp + i];
  }
  part = wave_sum(part);
  if ((tid & 63) == 0) red[tid >> 6] = part;
  __syncthreads();
  const float dal = red[0] + red[1] + red[2] + red[3];
  for (int e = tid; e < mp * mp; e += blockDim.x) {
    const int i = e / mp, j = e % mp;
    float v = da[e] + al * g[(size_t)j * mp + i];
    const float aij = a[e];
    const float sg = aij > 0.f ? 1.f : (aij < 0.f ? -1.f : 0.f);
    if (j == jc && i < m) v -= dal * al / c * sg;
    if (i == ir && j < m) v -= dal * al / r * sg;
    da[e] = v;
  }
}

// Y = -X (elementwise copy with negation) plus k I on the first m diagonal entries, on
// mp x mp matrices of `batch` heads (for P = 7I - X).
__global__ __launch_bounds__(256) void eye_minus_kernel(float* Y, const float* X, long long sY,
                                                        long long sX, int mp, int m, float k,
                                                        int batch) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long long)batch * mp * mp) return;
  const int b = (int)(e / ((long long)mp * mp)), w = (int)(e % ((long long)mp * mp));
  const int i = w / mp, j = w % mp;
  Y[(size_t)b * sY + w] = ((i == j && i < m) ? k : 0.f) - X[(size_t)b * sX + w];
}

// Y += alpha X elementwise on `count` floats.
__global__ __launch_bounds__(256) void axpy_kernel(float* Y, const float* X, float alpha,
                                                   long long count) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e < count) Y[e] += alpha * X[e];
}

// ------------------------------------------------------------------ token kernels
// dX[t] += dXt[seg(t)] / |seg(t)| for t < L (segment means backward), rows [BH][n][d].
__global__ __launch_bounds__(256) void segment_scatter_kernel(float* dX, const float* dXt,
                                                              int n, int d, int mp, int m,
                                                              const int* lengths, int H) {
  const int b = blockIdx.y;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;  // four features each
  const int L = valid_length(lengths, b, H, n, m);
  if (e >= (long long)L * (d / 4)) return;
  const int t = (int)(e / (d / 4)), f = (int)(e % (d / 4)) * 4;
  const int j = (int)(((long long)t * m) / L);
  const int start = (int)(((long long)j * L + m - 1) / m);
  const int end = (int)(((long long)(j + 1) * L + m - 1) / m);
  const float inv = 1.f / (float)(end - start);
  f32x4* px = reinterpret_cast<f32x4*>(dX + ((size_t)b * n + t) * d + f);
  const f32x4 g = *reinterpret_cast<const f32x4*>(dXt + ((size_t)b * mp + j) * d + f);
  *px += g * inv;
}

// Eight consecutive elements of a token row as floats (bf16 bits or fp32), one or two
// 16-byte loads; p 16-byte aligned (bf16) or 32-byte aligned (fp32).
template <typename T>
__device__ __forceinline__ void ld8f(const T* p, float* x) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[2 * q] = __uint_as_float(u[q] << 16);
      x[2 * q + 1] = __uint_as_float(u[q] & 0xffff0000u);
    }
  } else {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(p), hi = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[q] = lo[q];
      x[4 + q] = hi[q];
    }
  }
}

constexpr int kMaxConvW = 65;  // widest conv the plan accepts

// Tokens per thread in the conv kernels: a thread reads the W + kConvTok - 1 rows its
// kConvTok tokens need once, and every tap index below is a compile-time function of two
// unrolled loop counters.
constexpr int kConvTok = 4;

// dV[t] += sum_k w[k] dO[t - k + half] over the valid rows (the conv's transpose); one
// thread per kConvTok consecutive tokens x eight consecutive features. Row j of the
// thread's window is dO[t0 - half + j]; it meets token t0 + r through tap r - j + 2 half.
template <typename T>
__global__ __launch_bounds__(256) void conv_transpose_kernel(float* dV, const T* dO,
                                                             const float* w, int n, int d,
                                                             int W, int H, int m,
                                                             const int* lengths) {
  const int b = blockIdx.y;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const int L = valid_length(lengths, b, H, n, m);
  const int groups = (L + kConvTok - 1) / kConvTok;
  if (e >= (long long)groups * (d / 8)) return;
  const int t0 = (int)(e / (d / 8)) * kConvTok, f0 = (int)(e % (d / 8)) * 8, half = (W - 1) / 2;
  const float* wh = w + (size_t)(b % H) * W;
  const T* o = dO + (size_t)b * n * d + f0;
  float acc[kConvTok][8] = {};
#pragma unroll
  for (int j = 0; j < kMaxConvW + kConvTok - 1; ++j) {
    const int src = t0 - half + j;
    if (j < W + kConvTok - 1 && src >= 0 && src < L) {
      float x[8];
      ld8f(o + (size_t)src * d, x);
#pragma unroll
      for (int r = 0; r < kConvTok; ++r) {
        const int k = r - j + 2 * half;  // tap joining row j to token t0 + r
        if (k >= 0 && k < W) {
          const float wk = wh[k];
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[r][q] += wk * x[q];
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kConvTok; ++r) {
    if (t0 + r >= L) break;
    f32x4* p = reinterpret_cast<f32x4*>(dV + ((size_t)b * n + t0 + r) * d + f0);
    p[0] += f32x4{acc[r][0], acc[r][1], acc[r][2], acc[r][3]};
    p[1] += f32x4{acc[r][4], acc[r][5], acc[r][6], acc[r][7]};
  }
}

// Partial conv-weight gradient of one (head, token chunk): part[b][chunk][k] =
// sum over the chunk's valid t of dO[t] . V[t + k - half] (V zero outside [0, L)). One
// thread per kConvTok consecutive tokens x eight consecutive features; row j of the
// thread's V window is V[t0 - half + j], which meets token t0 + r through tap j - r, so the
// per-tap sums stay in registers.
template <typename T>
__global__ __launch_bounds__(256) void dw_partial_kernel(float* part, const T* dO, const T* V,
                                                         int n, int d, int W, int H, int m,
                                                         const int* lengths, int chunk,
                                                         int nchunks) {
  __shared__ float red[4][kMaxConvW + 7];
  const int b = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int L = valid_length(lengths, b, H, n, m);
  const int t0c = c * chunk, t1 = min(t0c + chunk, L), half = (W - 1) / 2;
  const T* o = dO + (size_t)b * n * d;
  const T* v = V + (size_t)b * n * d;
  float acc[kMaxConvW];
#pragma unroll
  for (int k = 0; k < kMaxConvW; ++k) acc[k] = 0.f;
  const int groups = (max(0, t1 - t0c) + kConvTok - 1) / kConvTok;
  for (long long e = tid; e < (long long)groups * (d / 8); e += 256) {
    const int t0 = t0c + (int)(e / (d / 8)) * kConvTok, f0 = (int)(e % (d / 8)) * 8;
    float go[kConvTok][8];
#pragma unroll
    for (int r = 0; r < kConvTok; ++r) {
      if (t0 + r < t1) {
        ld8f(o + (size_t)(t0 + r) * d + f0, go[r]);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) go[r][q] = 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxConvW + kConvTok - 1; ++j) {
      const int src = t0 - half + j;
      if (j < W + kConvTok - 1 && src >= 0 && src < L) {
        float x[8];
        ld8f(v + (size_t)src * d + f0, x);
#pragma unroll
        for (int r = 0; r < kConvTok; ++r) {
          const int k = j - r;  // compile-time: tap joining token t0 + r to row j
          if (k >= 0 && k < kMaxConvW && k < W) {
            float s8 = 0.f;
#pragma unroll
            for (int q = 0; q < 8; ++q) s8 += go[r][q] * x[q];
            acc[k] += s8;
          }
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxConvW; ++k) {
    if (k < W) {
      const float s = wave_sum(acc[k]);
      if ((tid & 63) == 0) red[tid >> 6][k] = s;
    }
  }
  __syncthreads();
  if (tid < W)
    part[((size_t)b * nchunks + c) * W + tid] = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
}

// dw[h][k] = sum over batch entries of head h and chunks of the partials (fixed order).
__global__ __launch_bounds__(128) void dw_reduce_kernel(float* dw, const float* part, int B, int H,
                                                        int W, int nchunks) {
  const int h = blockIdx.x, k = threadIdx.x;
  if (k >= W) return;
  float s = 0.f;
  for (int bb = 0; bb < B; ++bb)
    for (int c = 0; c < nchunks; ++c) s += part[(((size_t)bb * H + h) * nchunks + c) * W + k];
  dw[(size_t)h * W + k] = s;
}

// out[b][t][:] = src (fp32) in the I/O type for t < L, zero on padding rows.
template <typename T>
__global__ __launch_bounds__(256) void store_grad_kernel(T* out, const float* src, int n, int d,
                                                         int H, int m, const int* lengths) {
  const int b = blockIdx.y;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;  // four elements each
  if (e >= (long long)n * d / 4) return;
  const int L = valid_length(lengths, b, H, n, m);
  const size_t o = (size_t)b * n * d + 4 * e;
  const f32x4 v = (4 * e) / d < L ? *reinterpret_cast<const f32x4*>(src + o) : f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4*>(out + o) = v;
  } else {
    const bf16x2 lo = bf16_rne2(v[0], v[1]), hi = bf16_rne2(v[2], v[3]);
    *reinterpret_cast<u32x2*>(out + o) =
        u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  }
}

// Zero `count` floats.
__global__ __launch_bounds__(256) void zero_kernel(float* p, long long count) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e < count) p[e] = 0.f;
}

// ------------------------------------------------------------------ host sequence
namespace {

struct Runner {
  const GenBwdArgs& a;
  hipStream_t s;
  hipError_t err = hipSuccess;

  // C = alpha op(A) op(B) + beta C + diag I, batched over the BH heads
  template <typename TAe, typename TBe, bool TA, bool TB>
  void gemm(const TAe* A, long long sA, int lda, const TBe* B, long long sB, int ldb, float* C,
            long long sC, int ldc, int M, int N, int K, float alpha, float beta, int mask,
            float diag = 0.f, int diag_n = 0) {
    if (err != hipSuccess) return;
    GemmArgs g{A, B, C, sA, sB, sC, lda, ldb, ldc, M, N, K, alpha, beta, diag, diag_n, mask,
               a.lengths, a.H, a.n, a.m, nullptr, 1, 0, a.BH};
    // products over the token dimension have few output tiles per head and a long k loop:
    // split k so that about kSplitBlocks blocks share it (at least kSplitMin tokens each)
    const int tiles = ((N + kGT - 1) / kGT) * ((M + kGT - 1) / kGT);
    if ((mask & 4) && a.nsplit > 1 && (long long)M * N <= (long long)a.mp * a.d) {
      const int want = (kSplitBlocks + tiles * a.BH - 1) / (tiles * a.BH);
      const int sp = std::min({a.nsplit, want, std::max(1, K / kSplitMin)});
      if (sp > 1) {
        g.nsplit = sp;
        g.kchunk = (K + sp - 1) / sp;
        g.kchunk = (g.kchunk + kGK - 1) / kGK * kGK;
        g.part = a.ksplit;
      }
    }
    const dim3 grid((N + kGT - 1) / kGT, (M + kGT - 1) / kGT, a.BH * g.nsplit);
    hipLaunchKernelGGL((gemm_kernel<TAe, TBe, TA, TB>), grid, dim3(256), 0, s, g);
    err = hipGetLastError();
    if (err == hipSuccess && g.nsplit > 1) {
      const long long total = (long long)a.BH * M * N;
      hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                         s, g);
      err = hipGetLastError();
    }
  }
  void softmax(float* X, int rows, int cols, int rmode, int cmode, float scale) {
    if (err != hipSuccess) return;
    RowArgs r{X, nullptr, rows, cols, rmode, cmode, scale, a.lengths, a.H, a.n, a.m};
    const long long total = (long long)a.BH * rows;
    hipLaunchKernelGGL(row_softmax_kernel, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, s, r,
                       (int)total);
    err = hipGetLastError();
  }
  void dsoftmax(float* X, const float* P, int rows, int cols, int rmode, int cmode) {
    if (err != hipSuccess) return;
    RowArgs r{X, P, rows, cols, rmode, cmode, 1.f, a.lengths, a.H, a.n, a.m};
    const long long total = (long long)a.BH * rows;
    hipLaunchKernelGGL(row_dsoftmax_kernel, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, s, r,
                       (int)total);
    err = hipGetLastError();
  }
  void axpy(float* Y, const float* X, float alpha, long long count) {
    if (err != hipSuccess) return;
    hipLaunchKernelGGL(axpy_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, Y, X,
                       alpha, count);
    err = hipGetLastError();
  }
};

template <typename T>
hipError_t run(const GenBwdArgs& a, hipStream_t s) {
  Runner r{a, s};
  const int BH = a.BH, n = a.n, d = a.d, mp = a.mp, m = a.m, T_ = a.iters;
  const long long nd = (long long)n * d, nm = (long long)n * mp, md = (long long)mp * d,
                  mm = (long long)mp * mp;
  const float sc = a.scale;
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  const T* dO = static_cast<const T*>(a.dout);
  constexpr int kM = 1, kN = 2, kK = 4;  // token-dimension masks
  // ---- forward recomputation (landmarks qt, kt come from the segment-means kernel)
  // F = softmax_row(s Q Kt^T): rows = tokens, columns = landmarks
  r.gemm<T, float, false, true>(q, nd, d, a.kt, md, d, a.F, nm, mp, n, mp, d, 1.f, 0.f, kM);
  r.softmax(a.F, n, mp, 2, 1, sc);
  // A = softmax_row(s Qt Kt^T)
  r.gemm<float, float, false, true>(a.qt, md, d, a.kt, md, d, a.A, mm, mp, mp, mp, d, 1.f, 0.f, 0);
  r.softmax(a.A, mp, mp, 1, 1, sc);
  // B = softmax_row(s Qt K^T): rows = landmarks, columns = tokens
  r.gemm<float, T, false, true>(a.qt, md, d, k, nd, d, a.Bm, nm, n, mp, n, d, 1.f, 0.f, kN);
  r.softmax(a.Bm, mp, n, 1, 2, sc);
  // W = B V
  r.gemm<float, T, false, false>(a.Bm, nm, n, v, nd, d, a.Wc, md, d, mp, d, n, 1.f, 0.f, kK);
  // alpha, Z_0 = alpha A^T, then the iteration with every Z_k and X_k kept
  const long long zst = (long long)(T_ + 1) * mm, xst = (long long)std::max(T_, 1) * mm;
  if (r.err == hipSuccess) {
    hipLaunchKernelGGL(alpha_z0_kernel, dim3(BH), dim3(256), 0, s, a.A, a.Zs, a.alpha, a.amax, mp,
                       m, zst);
    r.err = hipGetLastError();
  }
  for (int it = 0; it < T_; ++it) {
    float* Z = a.Zs + it * mm;
    float* X = a.Xs + it * mm;
    r.gemm<float, float, false, false>(a.A, mm, mp, Z, zst, mp, X, xst, mp, mp, mp, mp, 1.f, 0.f, 0);
    if (r.err == hipSuccess) {  // P = 7I - X
      hipLaunchKernelGGL(eye_minus_kernel, dim3((unsigned)((BH * mm + 255) / 256)), dim3(256), 0, s,
                         a.P, X, mm, xst, mp, m, 7.f, BH);
      r.err = hipGetLastError();
    }
    // Q1 = 15I - X P, R = 13I - X Q1, Z' = Z R / 4
    r.gemm<float, float, false, false>(X, xst, mp, a.P, mm, mp, a.Q1, mm, mp, mp, mp, mp, -1.f, 0.f,
                                       0, 15.f, m);
    r.gemm<float, float, false, false>(X, xst, mp, a.Q1, mm, mp, a.R, mm, mp, mp, mp, mp, -1.f, 0.f,
                                       0, 13.f, m);
    r.gemm<float, float, false, false>(Z, zst, mp, a.R, mm, mp, Z + mm, zst, mp, mp, mp, mp, 0.25f,
                                       0.f, 0);
  }
  const float* ZT = a.Zs + (long long)T_ * mm;
  // Y = Z_T W
  r.gemm<float, float, false, false>(ZT, zst, mp, a.Wc, md, d, a.Y, md, d, mp, d, mp, 1.f, 0.f, 0);

  // ---- backward
  // dF = dO Y^T (into G1), dSF = F o (dF - rowsum(F o dF))
  r.gemm<T, float, false, true>(dO, nd, d, a.Y, md, d, a.G1, nm, mp, n, mp, d, 1.f, 0.f, kM);
  r.dsoftmax(a.G1, a.F, n, mp, 2, 1);
  // dQ = s dSF Kt; dKt = s dSF^T Q; dY = F^T dO
  r.gemm<float, float, false, false>(a.G1, nm, mp, a.kt, md, d, a.dQ, nd, d, n, d, mp, sc, 0.f, kM);
  r.gemm<float, T, true, false>(a.G1, nm, mp, q, nd, d, a.dKt, md, d, mp, d, n, sc, 0.f, kK);
  r.gemm<float, T, true, false>(a.F, nm, mp, dO, nd, d, a.dY, md, d, mp, d, n, 1.f, 0.f, kK);
  // dZ_T = dY W^T, dW = Z_T^T dY
  float* G = a.Gz;  // running dZ_{k+1}
  r.gemm<float, float, false, true>(a.dY, md, d, a.Wc, md, d, G, mm, mp, mp, mp, d, 1.f, 0.f, 0);
  r.gemm<float, float, true, false>(ZT, zst, mp, a.dY, md, d, a.dW, md, d, mp, d, mp, 1.f, 0.f, 0);
  // reverse sweep: dA accumulates dX Z_k^T over the steps (the first step overwrites it);
  // G becomes dZ_k
  if (T_ == 0 && r.err == hipSuccess) {
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((BH * mm + 255) / 256)), dim3(256), 0, s, a.dA,
                       (long long)BH * mm);
    r.err = hipGetLastError();
  }
  float* Gn = a.Gn;
  for (int it = T_ - 1; it >= 0; --it) {
    const float* Z = a.Zs + it * mm;
    const float* X = a.Xs + it * mm;
    // recompute P, Q1, R of this step
    if (r.err == hipSuccess) {
      hipLaunchKernelGGL(eye_minus_kernel, dim3((unsigned)((BH * mm + 255) / 256)), dim3(256), 0, s,
                         a.P, X, mm, xst, mp, m, 7.f, BH);
      r.err = hipGetLastError();
    }
    r.gemm<float, float, false, false>(X, xst, mp, a.P, mm, mp, a.Q1, mm, mp, mp, mp, mp, -1.f, 0.f,
                                       0, 15.f, m);
    r.gemm<float, float, false, false>(X, xst, mp, a.Q1, mm, mp, a.R, mm, mp, mp, mp, mp, -1.f, 0.f,
                                       0, 13.f, m);
    // Z' = Z R / 4: dZk = G R^T / 4, dR = Z^T G / 4
    r.gemm<float, float, false, true>(G, mm, mp, a.R, mm, mp, Gn, mm, mp, mp, mp, mp, 0.25f, 0.f, 0);
    r.gemm<float, float, true, false>(Z, zst, mp, G, mm, mp, a.dR, mm, mp, mp, mp, mp, 0.25f, 0.f, 0);
    // R = 13I - X Q1: dX = -dR Q1^T, dQ1 = -X^T dR
    r.gemm<float, float, false, true>(a.dR, mm, mp, a.Q1, mm, mp, a.dX, mm, mp, mp, mp, mp, -1.f, 0.f, 0);
    r.gemm<float, float, true, false>(X, xst, mp, a.dR, mm, mp, a.dQ1, mm, mp, mp, mp, mp, -1.f, 0.f, 0);
    // Q1 = 15I - X P: dX -= dQ1 P^T, dP = -X^T dQ1
    r.gemm<float, float, false, true>(a.dQ1, mm, mp, a.P, mm, mp, a.dX, mm, mp, mp, mp, mp, -1.f, 1.f, 0);
    r.gemm<float, float, true, false>(X, xst, mp, a.dQ1, mm, mp, a.dP, mm, mp, mp, mp, mp, -1.f, 0.f, 0);
    // P = 7I - X: dX -= dP
    r.axpy(a.dX, a.dP, -1.f, (long long)BH * mm);
    // X = A Z: dA += dX Z^T, dZk += A^T dX
    r.gemm<float, float, false, true>(a.dX, mm, mp, Z, zst, mp, a.dA, mm, mp, mp, mp, mp, 1.f,
                                      it == T_ - 1 ? 0.f : 1.f, 0);
    r.gemm<float, float, true, false>(a.A, mm, mp, a.dX, mm, mp, Gn, mm, mp, mp, mp, mp, 1.f, 1.f, 0);
    float* t = G;
    G = Gn;
    Gn = t;
  }
  // Z_0 = alpha A^T and the alpha term
  if (r.err == hipSuccess) {
    hipLaunchKernelGGL(alpha_backward_kernel, dim3(BH), dim3(256), 0, s, a.A, G, mm, a.dA, a.alpha,
                       a.amax, mp, m);
    r.err = hipGetLastError();
  }
  // dSA = A o (dA - rowsum(A o dA)); dQt = s dSA Kt; dKt += s dSA^T Qt
  r.dsoftmax(a.dA, a.A, mp, mp, 1, 1);
  r.gemm<float, float, false, false>(a.dA, mm, mp, a.kt, md, d, a.dQt, md, d, mp, d, mp, sc, 0.f, 0);
  r.gemm<float, float, true, false>(a.dA, mm, mp, a.qt, md, d, a.dKt, md, d, mp, d, mp, sc, 1.f, 0);
  // dB = dW V^T (into G2), dSB = B o (dB - rowsum(B o dB))
  r.gemm<float, T, false, true>(a.dW, md, d, v, nd, d, a.G2, nm, n, mp, n, d, 1.f, 0.f, kN);
  r.dsoftmax(a.G2, a.Bm, mp, n, 1, 2);
  // dK = s dSB^T Qt; dQt += s dSB K; dV = B^T dW
  r.gemm<float, float, true, false>(a.G2, nm, n, a.qt, md, d, a.dK, nd, d, n, d, mp, sc, 0.f, kM);
  r.gemm<float, T, false, false>(a.G2, nm, n, k, nd, d, a.dQt, md, d, mp, d, n, sc, 1.f, kK);
  r.gemm<float, float, true, false>(a.Bm, nm, n, a.dW, md, d, a.dV, nd, d, n, d, mp, 1.f, 0.f, kM);
  if (r.err != hipSuccess) return r.err;
  // segment means: dQ += dQt[seg] / |seg|, dK += dKt[seg] / |seg|
  const dim3 tok((unsigned)((nd + 255) / 256), BH);
  const dim3 tok4((unsigned)((nd / 4 + 255) / 256), BH);
  hipLaunchKernelGGL(segment_scatter_kernel, tok4, dim3(256), 0, s, a.dQ, a.dQt, n, d, mp, m,
                     a.lengths, a.H);
  hipLaunchKernelGGL(segment_scatter_kernel, tok4, dim3(256), 0, s, a.dK, a.dKt, n, d, mp, m,
                     a.lengths, a.H);
  // conv skip: dV += conv^T(dO); dw
  const dim3 tokc((unsigned)(((n + kConvTok - 1) / kConvTok * (long long)(d / 8) + 255) / 256), BH);
  hipLaunchKernelGGL((conv_transpose_kernel<T>), tokc, dim3(256), 0, s, a.dV, dO, a.conv_w, n, d,
                     a.W, a.H, m, a.lengths);
  const int nch = (n + a.dw_chunk - 1) / a.dw_chunk;
  hipLaunchKernelGGL((dw_partial_kernel<T>), dim3(nch, BH), dim3(256), 0, s, a.dw_part, dO, v, n,
                     d, a.W, a.H, m, a.lengths, a.dw_chunk, nch);
  hipLaunchKernelGGL(dw_reduce_kernel, dim3(a.H), dim3(128), 0, s, a.dconv_w, a.dw_part, a.B, a.H,
                     a.W, nch);
  // outputs in the I/O type, padding rows zero
  hipLaunchKernelGGL((store_grad_kernel<T>), tok4, dim3(256), 0, s, static_cast<T*>(a.dq), a.dQ,
                     n, d, a.H, m, a.lengths);
  hipLaunchKernelGGL((store_grad_kernel<T>), tok4, dim3(256), 0, s, static_cast<T*>(a.dk), a.dK,
                     n, d, a.H, m, a.lengths);
  hipLaunchKernelGGL((store_grad_kernel<T>), tok4, dim3(256), 0, s, static_cast<T*>(a.dv), a.dV,
                     n, d, a.H, m, a.lengths);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_general(const GenBwdArgs& a, hipStream_t s) {
  return a.bf16 ? run<uint16_t>(a, s) : run<float>(a, s);
}

}  // namespace nys
