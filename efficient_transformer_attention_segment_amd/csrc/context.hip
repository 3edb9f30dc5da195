// Stage 2 of the forward pass (Nystromformer review page, "Proposed method"):
//
//  * pinv_kernel   one block per head: A_S = softmax_row(s Qt Kt^T), the scaling
//                  alpha = 1/(||A_S||_1 ||A_S||_inf), Z_0 = alpha A_S^T, then `iters`
//                  steps of Z <- 1/4 Z (13I - X(15I - X(7I - X))), X = A_S Z, every
//                  m x m product on MFMA. For mp <= 64 all operand planes live in LDS
//                  (4 waves); larger mp keeps them in global memory (16 waves).
//  * flash_kernel  BH * C blocks: the right factor softmax_row(s Qt K^T) V, computed
//                  without forming the m x n matrix: each block streams one chunk of K/V
//                  tiles, keeps a running max / sum per landmark (online softmax over n)
//                  and an unnormalised m x d accumulator; it writes that partial state
//                  (feature-major, so the merge reads it as W^T).
//
// Blocks never exchange data inside a kernel: on MI355X each XCD has its own L2, and a
// device-scope hand-off costs an L2 write-back plus invalidate per block. The output
// stage merges the C partial states (fixed chunk order, log-sum-exp rescaling) and
// forms Y = Z W in its prologue.
#include "nys_common.h"
#include "nys_kernels.h"

namespace nys {

// Store the transpose in fp32: element (i, j) goes to p[j][i].
__device__ __forceinline__ void store_cols_f32(float* p, int ld, int row0, int col0,
                                               const f32x16& v, int lane) {
  const int j = col0 + (lane & 31);
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<f32x4*>(p + (size_t)j * ld + row0 + 8 * g + 4 * (lane >> 5)) =
        f32x4{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
}

__device__ __forceinline__ float block_max(float x, float* red, int tid, int nw) {
  x = wave_max(x);
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = x;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; ++i) r = fmaxf(r, red[i]);
  return r;
}

// ------------------------------------------------------------------ pinv
// Plane pairs (hi, lo) per head. In LDS mode they are LDS arrays, otherwise a slice of
// CtxArgs::planes. Z and the X^2/T plane are updated in place: every wave first computes
// all of its tiles into registers, the block synchronises, then the tiles are written.
// LDS variant: 12 planes. Global variant adds a second Z pair and a separate T pair.
enum { kPA = 0, kPZr = 2, kPZc = 4, kPXr = 6, kPXc = 8, kPX2T = 10, kLdsPlanes = 12,
       kGZr1 = 12, kGZc1 = 14, kGT = 16 };
static_assert(kPlanes == 18, "plane count");

template <bool kLds, int TPW>
__device__ __forceinline__ void pinv_body(const CtxArgs& a, int bh, uint16_t* pl, float* red,
                                          float* red_part, float* red_col) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthreads = blockDim.x, nw = nthreads >> 6;
  const int mp = a.mp, m = a.m, nt = mp / 32, ntiles = nt * nt;
  const size_t P = (size_t)mp * mp;
  const int dd = a.d;
  float* A = a.a_s + (size_t)bh * P;
  float* own = a.own + (size_t)bh * 2 * P;  // fp32 X, X^2 (global variant only)
  auto plane = [&](int idx) { return pl + (size_t)idx * P; };

  // 1. logits Qt Kt^T (both landmark sets as hi/lo planes, K = d), scaled to log2
  //    units, held in registers: tile t = wave + nw*u of the mp x mp matrix.
  constexpr int TPW0 = kLds ? 1 : 4;  // tiles per wave for mp <= 64 / mp <= 256
  f32x16 at[TPW0];
  {
    const uint16_t* qh = a.qt_hl + (size_t)bh * 2 * mp * dd;
    const uint16_t* kh = a.kt_hl + (size_t)bh * 2 * mp * dd;
#pragma unroll
    for (int u = 0; u < TPW0; ++u) {
      const int t = wave + nw * u;
      if (t < ntiles)
        at[u] = gemm_tile(qh, qh + (size_t)mp * dd, dd, kh, kh + (size_t)mp * dd, dd,
                          32 * (t / nt), 32 * (t % nt), dd, lane) * a.scale_log2e;
    }
  }
  // 2. row softmax over the m real landmarks (padded rows/columns become 0): per-tile
  //    half-wave reductions, combined across column tiles through LDS partials
  //    part[row][tile column].
  const int r32 = lane & 31;
#pragma unroll
  for (int u = 0; u < TPW0; ++u) {
    const int t = wave + nw * u;
    if (t < ntiles) {
      const int row0 = 32 * (t / nt), tj = t % nt, j = 32 * tj + r32;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float mx = half_max(j < m ? at[u][rr] : kNegBig);
        if (r32 == 0) red_part[acc_row(row0, rr, lane) * nt + tj] = mx;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < TPW0; ++u) {
    const int t = wave + nw * u;
    if (t < ntiles) {
      const int row0 = 32 * (t / nt), tj = t % nt, j = 32 * tj + r32;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int i = acc_row(row0, rr, lane);
        float mx = kNegBig;
        for (int c = 0; c < nt; ++c) mx = fmaxf(mx, red_part[i * nt + c]);
        at[u][rr] = (i < m && j < m) ? fast_exp2(at[u][rr] - mx) : 0.f;
      }
    }
  }
  __syncthreads();  // every wave has read the maxima before the sums overwrite them
#pragma unroll
  for (int u = 0; u < TPW0; ++u) {
    const int t = wave + nw * u;
    if (t < ntiles) {
      const int row0 = 32 * (t / nt), tj = t % nt;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float sm = half_sum(at[u][rr]);
        if (r32 == 0) red_part[acc_row(row0, rr, lane) * nt + tj] = sm;
      }
    }
  }
  __syncthreads();
  // normalise; then abs row sums (partials again) and abs column sums (per row tile)
#pragma unroll
  for (int u = 0; u < TPW0; ++u) {
    const int t = wave + nw * u;
    if (t < ntiles) {
      const int row0 = 32 * (t / nt);
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int i = acc_row(row0, rr, lane);
        float sum = 0.f;
        for (int c = 0; c < nt; ++c) sum += red_part[i * nt + c];
        at[u][rr] = i < m ? at[u][rr] / sum : 0.f;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < TPW0; ++u) {
    const int t = wave + nw * u;
    if (t < ntiles) {
      const int ti = t / nt, tj = t % nt, row0 = 32 * ti;
      float cs = 0.f;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float rs = half_sum(fabsf(at[u][rr]));
        if (r32 == 0) red_part[acc_row(row0, rr, lane) * nt + tj] = rs;
        cs += fabsf(at[u][rr]);
      }
      cs += __shfl_xor(cs, 32);
      if (lane < 32) red_col[ti * mp + 32 * tj + r32] = cs;
    }
  }
  __syncthreads();
  float rmax = 0.f, cmax = 0.f;
  for (int i = tid; i < m; i += nthreads) {
    float rs = 0.f, cs = 0.f;
    for (int c = 0; c < nt; ++c) {
      rs += red_part[i * nt + c];
      cs += red_col[c * mp + i];
    }
    rmax = fmaxf(rmax, rs);
    cmax = fmaxf(cmax, cs);
  }
  rmax = block_max(rmax, red, tid, nw);
  cmax = block_max(cmax, red + 16, tid, nw);
  const float alpha = 1.0f / (cmax * rmax);
  // 3. A_S (fp32 copy for inspection, hi/lo operand plane) and Z_0 = alpha A_S^T, stored
  //    row-major (kPZr) and transposed (kPZc, i.e. alpha A_S row-major)
#pragma unroll
  for (int u = 0; u < TPW0; ++u) {
    const int t = wave + nw * u;
    if (t < ntiles) {
      const int row0 = 32 * (t / nt), col0 = 32 * (t % nt);
      store_rows_f32(A, mp, row0, col0, at[u], lane);
      store_rows_hl(plane(kPA), plane(kPA + 1), mp, row0, col0, at[u], lane);
      const f32x16 zv = at[u] * alpha;
      store_rows_hl(plane(kPZc), plane(kPZc + 1), mp, row0, col0, zv, lane);
      store_cols_hl(plane(kPZr), plane(kPZr + 1), mp, row0, col0, zv, lane);
      if (a.iters == 0) store_cols_f32(a.z + (size_t)bh * P, mp, row0, col0, zv, lane);
    }
  }
  __syncthreads();

  // 5. iterations. Each wave owns tiles t = wave + nw*u.
  if constexpr (kLds) {
    // mp <= 64: one tile per wave. Z and the X^2/T plane are updated in place: the
    // products are held in registers across a barrier before they are written.
    static_assert(TPW == 1, "LDS variant holds one tile per wave");
    const int t = wave;
    const bool mine = t < ntiles;
    const int row0 = 32 * (t / nt), col0 = 32 * (t % nt);
    const int j = col0 + (lane & 31);
    for (int it = 0; it < a.iters; ++it) {
      f32x16 x, x2, acc;
      if (mine) {  // X = A Z
        x = gemm_tile(plane(kPA), plane(kPA + 1), mp, plane(kPZc), plane(kPZc + 1), mp, row0,
                      col0, mp, lane);
        store_rows_hl(plane(kPXr), plane(kPXr + 1), mp, row0, col0, x, lane);
        store_cols_hl(plane(kPXc), plane(kPXc + 1), mp, row0, col0, x, lane);
      }
      __syncthreads();
      if (mine) {  // X^2 = X X
        x2 = gemm_tile(plane(kPXr), plane(kPXr + 1), mp, plane(kPXc), plane(kPXc + 1), mp, row0,
                       col0, mp, lane);
        store_cols_hl(plane(kPX2T), plane(kPX2T + 1), mp, row0, col0, x2, lane);
      }
      __syncthreads();
      if (mine)  // X^3 = X X^2
        acc = gemm_tile(plane(kPXr), plane(kPXr + 1), mp, plane(kPX2T), plane(kPX2T + 1), mp,
                        row0, col0, mp, lane);
      __syncthreads();
      if (mine) {  // T = 13I - 15X + 7X^2 - X^3  (= 13I - X(15I - X(7I - X)))
        f32x16 tv;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const float diag = (acc_row(row0, rr, lane) == j) ? 13.f : 0.f;
          tv[rr] = diag - 15.f * x[rr] + 7.f * x2[rr] - acc[rr];
        }
        store_cols_hl(plane(kPX2T), plane(kPX2T + 1), mp, row0, col0, tv, lane);
      }
      __syncthreads();
      if (mine)  // Z T
        acc = gemm_tile(plane(kPZr), plane(kPZr + 1), mp, plane(kPX2T), plane(kPX2T + 1), mp,
                        row0, col0, mp, lane);
      __syncthreads();
      if (mine) {  // Z <- Z T / 4
        const f32x16 zv = acc * 0.25f;
        store_rows_hl(plane(kPZr), plane(kPZr + 1), mp, row0, col0, zv, lane);
        store_cols_hl(plane(kPZc), plane(kPZc + 1), mp, row0, col0, zv, lane);
        if (it == a.iters - 1) store_rows_f32(a.z + (size_t)bh * P, mp, row0, col0, zv, lane);
      }
      __syncthreads();
    }
  } else {
    // mp > 64: planes in global memory; Z and T get separate (ping-pong) planes so every
    // product is written as soon as it is formed. fp32 X, X^2 of the own tiles go to
    // per-head scratch and are read back by the same wave.
    for (int it = 0; it < a.iters; ++it) {
      const int zr = (it & 1) ? kGZr1 : kPZr, zc = (it & 1) ? kGZc1 : kPZc;
      const int zr_n = (it & 1) ? kPZr : kGZr1, zc_n = (it & 1) ? kPZc : kGZc1;
#pragma unroll 1
      for (int t = wave; t < ntiles; t += nw) {  // X = A Z
        const int row0 = 32 * (t / nt), col0 = 32 * (t % nt);
        const f32x16 x = gemm_tile(plane(kPA), plane(kPA + 1), mp, plane(zc), plane(zc + 1), mp,
                                   row0, col0, mp, lane);
        store_rows_hl(plane(kPXr), plane(kPXr + 1), mp, row0, col0, x, lane);
        store_cols_hl(plane(kPXc), plane(kPXc + 1), mp, row0, col0, x, lane);
        store_rows_f32(own, mp, row0, col0, x, lane);
      }
      __syncthreads();
#pragma unroll 1
      for (int t = wave; t < ntiles; t += nw) {  // X^2 = X X
        const int row0 = 32 * (t / nt), col0 = 32 * (t % nt);
        const f32x16 x2 = gemm_tile(plane(kPXr), plane(kPXr + 1), mp, plane(kPXc),
                                    plane(kPXc + 1), mp, row0, col0, mp, lane);
        store_cols_hl(plane(kPX2T), plane(kPX2T + 1), mp, row0, col0, x2, lane);
        store_rows_f32(own + P, mp, row0, col0, x2, lane);
      }
      __syncthreads();
#pragma unroll 1
      for (int t = wave; t < ntiles; t += nw) {  // T = 13I - 15X + 7X^2 - X X^2
        const int row0 = 32 * (t / nt), col0 = 32 * (t % nt);
        const int j = col0 + (lane & 31);
        const f32x16 x3 = gemm_tile(plane(kPXr), plane(kPXr + 1), mp, plane(kPX2T),
                                    plane(kPX2T + 1), mp, row0, col0, mp, lane);
        f32x16 tv;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const size_t o = (size_t)acc_row(row0, rr, lane) * mp + j;
          const float diag = (acc_row(row0, rr, lane) == j) ? 13.f : 0.f;
          tv[rr] = diag - 15.f * own[o] + 7.f * own[P + o] - x3[rr];
        }
        store_cols_hl(plane(kGT), plane(kGT + 1), mp, row0, col0, tv, lane);
      }
      __syncthreads();
#pragma unroll 1
      for (int t = wave; t < ntiles; t += nw) {  // Z <- Z T / 4
        const int row0 = 32 * (t / nt), col0 = 32 * (t % nt);
        const f32x16 zv = gemm_tile(plane(zr), plane(zr + 1), mp, plane(kGT), plane(kGT + 1), mp,
                                    row0, col0, mp, lane) * 0.25f;
        store_rows_hl(plane(zr_n), plane(zr_n + 1), mp, row0, col0, zv, lane);
        store_cols_hl(plane(zc_n), plane(zc_n + 1), mp, row0, col0, zv, lane);
        if (it == a.iters - 1) store_rows_f32(a.z + (size_t)bh * P, mp, row0, col0, zv, lane);
      }
      __syncthreads();
    }
  }
  // 6. hand Z (row-major hi/lo) to the Y = Z W product of the output stage
  {
    const int zfin = kLds ? kPZr : ((a.iters & 1) ? kGZr1 : kPZr);
    uint16_t* dst = a.z_hl + (size_t)bh * 2 * P;
    const int n8 = (int)(P / 8);
    for (int e = tid; e < 2 * n8; e += nthreads) {
      const int which = e / n8, off = (e % n8) * 8;
      st8(dst + (size_t)which * P + off, ld8(plane(zfin + which) + off));
    }
  }
}

// ------------------------------------------------------------------ pinv, mp <= 64
// Compile-time specialisation for MP in {32, 64}: one 32x32 tile per wave (waves beyond
// the tile count only join the barriers), every loop unrolled, all operand planes in LDS.
// Z and the X^2/T plane are updated in place, so results are held in registers across
// the barrier that precedes their store.
template <int MP, int D>
__global__ __launch_bounds__(256) void pinv_lds_kernel(CtxArgs a) {
  constexpr int NT = MP / 32, NTILES = NT * NT, KD = D / 16, KM = MP / 16;
  constexpr int P = MP * MP;
  // LDS plane rows padded by 16 bytes: a 32-lane operand fetch then touches every bank
  // once instead of a few banks many times
  constexpr int LD = MP + 8, PL = MP * LD;
  extern __shared__ __align__(16) char lds[];
  __shared__ float red_part[MP * NT];  // [row][column tile]
  __shared__ float red_col[NT * MP];   // [row tile][column]
  __shared__ float red[16];
  uint16_t* pl = reinterpret_cast<uint16_t*>(lds);
  auto plane = [&](int idx) { return pl + idx * PL; };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r32 = lane & 31;
  const int bh = blockIdx.x, m = a.m;
  const bool mine = wave < NTILES;
  const int row0 = 32 * (wave / NT), tj = wave % NT, col0 = 32 * tj;
  const int jcol = col0 + r32;

  // 1. scaled logits (log2 units)
  f32x16 at = zero16();
  if (mine) {
    const uint16_t* qh = a.qt_hl + (size_t)bh * 2 * MP * D;
    const uint16_t* kh = a.kt_hl + (size_t)bh * 2 * MP * D;
    at = gemm_tile_k<KD>(qh, qh + MP * D, D, kh, kh + MP * D, D, row0, col0, lane) * a.scale_log2e;
  }
  // 2. row softmax over the m real landmarks (padded rows/columns become 0)
  if (mine) {
    float mx[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) mx[rr] = half_max(jcol < m ? at[rr] : kNegBig);
    if (r32 == 0)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) red_part[acc_row(row0, rr, lane) * NT + tj] = mx[rr];
  }
  __syncthreads();
  if (mine) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int i = acc_row(row0, rr, lane);
      float mx = red_part[i * NT];
#pragma unroll
      for (int c = 1; c < NT; ++c) mx = fmaxf(mx, red_part[i * NT + c]);
      at[rr] = (i < m && jcol < m) ? fast_exp2(at[rr] - mx) : 0.f;
    }
  }
  __syncthreads();
  if (mine) {
    float sm[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) sm[rr] = half_sum(at[rr]);
    if (r32 == 0)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) red_part[acc_row(row0, rr, lane) * NT + tj] = sm[rr];
  }
  __syncthreads();
  if (mine) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int i = acc_row(row0, rr, lane);
      float sm = red_part[i * NT];
#pragma unroll
      for (int c = 1; c < NT; ++c) sm += red_part[i * NT + c];
      at[rr] = i < m ? at[rr] * (1.f / sm) : 0.f;
    }
  }
  __syncthreads();
  // abs row sums (partials per column tile) and abs column sums (per row tile)
  if (mine) {
    float rs[16], cs = 0.f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      rs[rr] = half_sum(fabsf(at[rr]));
      cs += fabsf(at[rr]);
    }
    cs += __shfl_xor(cs, 32);
    if (r32 == 0)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) red_part[acc_row(row0, rr, lane) * NT + tj] = rs[rr];
    if (lane < 32) red_col[(row0 / 32) * MP + jcol] = cs;
  }
  __syncthreads();
  float rmax = 0.f, cmax = 0.f;
  if (tid < m) {
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      rmax += red_part[tid * NT + c];
      cmax += red_col[c * MP + tid];
    }
  }
  rmax = wave_max(rmax);
  cmax = wave_max(cmax);
  if (lane == 0) {
    red[wave] = rmax;
    red[8 + wave] = cmax;
  }
  __syncthreads();
  rmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  cmax = fmaxf(fmaxf(red[8], red[9]), fmaxf(red[10], red[11]));
  const float alpha = 1.0f / (cmax * rmax);
  // 3. A_S (fp32 copy), its operand plane, Z_0 = alpha A_S^T (row-major and transposed)
  if (mine) {
    store_rows_f32(a.a_s + (size_t)bh * P, MP, row0, col0, at, lane);
    store_rows_hl(plane(kPA), plane(kPA + 1), LD, row0, col0, at, lane);
    const f32x16 zv = at * alpha;
    store_rows_hl(plane(kPZc), plane(kPZc + 1), LD, row0, col0, zv, lane);
    store_cols_hl(plane(kPZr), plane(kPZr + 1), LD, row0, col0, zv, lane);
    if (a.iters == 0) store_cols_f32(a.z + (size_t)bh * P, MP, row0, col0, zv, lane);
  }
  __syncthreads();
  // 4. iterations
  for (int it = 0; it < a.iters; ++it) {
    f32x16 x, x2, acc;
    if (mine) {  // X = A Z
      x = gemm_tile_k<KM>(plane(kPA), plane(kPA + 1), LD, plane(kPZc), plane(kPZc + 1), LD,
                          row0, col0, lane);
      store_rows_hl(plane(kPXr), plane(kPXr + 1), LD, row0, col0, x, lane);
      store_cols_hl(plane(kPXc), plane(kPXc + 1), LD, row0, col0, x, lane);
    }
    __syncthreads();
    if (mine) {  // X^2 = X X
      x2 = gemm_tile_k<KM>(plane(kPXr), plane(kPXr + 1), LD, plane(kPXc), plane(kPXc + 1), LD,
                           row0, col0, lane);
      store_cols_hl(plane(kPX2T), plane(kPX2T + 1), LD, row0, col0, x2, lane);
    }
    __syncthreads();
    if (mine)  // X^3 = X X^2
      acc = gemm_tile_k<KM>(plane(kPXr), plane(kPXr + 1), LD, plane(kPX2T), plane(kPX2T + 1), LD, row0, col0, lane);
    __syncthreads();
    if (mine) {  // T = 13I - 15X + 7X^2 - X^3  (= 13I - X(15I - X(7I - X)))
      f32x16 tv;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float diag = (acc_row(row0, rr, lane) == jcol) ? 13.f : 0.f;
        tv[rr] = diag - 15.f * x[rr] + 7.f * x2[rr] - acc[rr];
      }
      store_cols_hl(plane(kPX2T), plane(kPX2T + 1), LD, row0, col0, tv, lane);
    }
    __syncthreads();
    if (mine)  // Z T
      acc = gemm_tile_k<KM>(plane(kPZr), plane(kPZr + 1), LD, plane(kPX2T), plane(kPX2T + 1), LD, row0, col0, lane);
    __syncthreads();
    if (mine) {  // Z <- Z T / 4
      const f32x16 zv = acc * 0.25f;
      store_rows_hl(plane(kPZr), plane(kPZr + 1), LD, row0, col0, zv, lane);
      store_cols_hl(plane(kPZc), plane(kPZc + 1), LD, row0, col0, zv, lane);
      if (it == a.iters - 1) store_rows_f32(a.z + (size_t)bh * P, MP, row0, col0, zv, lane);
    }
    __syncthreads();
  }
  // 5. Z (row-major hi/lo, unpadded) for the output stage
  uint16_t* dst = a.z_hl + (size_t)bh * 2 * P;
  for (int e = tid; e < 2 * P / 8; e += 256) {
    const int which = e / (P / 8), r = (e % (P / 8)) / (MP / 8), c8 = (e % (MP / 8)) * 8;
    st8(dst + (size_t)which * P + r * MP + c8, ld8(plane(kPZr + which) + r * LD + c8));
  }
}

template <bool kLds, int TPW, int D>
__global__ __launch_bounds__(kLds ? 256 : 1024) void pinv_kernel(CtxArgs a) {
  extern __shared__ __align__(16) char lds[];
  __shared__ float red[32];
  __shared__ float red_part[256 * 8];  // [row][column tile] partial max / sums
  __shared__ float red_col[8 * 256];   // [row tile][column] partial column sums
  const int bh = blockIdx.x;
  uint16_t* pl = kLds ? reinterpret_cast<uint16_t*>(lds)
                      : a.planes + (size_t)bh * kPlanes * a.mp * a.mp;
  pinv_body<kLds, TPW>(a, bh, pl, red, red_part, red_col);
}

// ------------------------------------------------------------------ flash
// NCH: 8-element V chunks each thread stages per step (D / (16 * LG), rounded up).
template <typename Tin, int D, int NCH>
__global__ __launch_bounds__(512) void flash_kernel(CtxArgs a) {
  extern __shared__ __align__(16) char lds[];
  constexpr bool kS = Input<Tin>::kSplit;
  constexpr int KD = D / 16;       // k-steps over features
  constexpr int FT = D / 32;       // feature tiles of the accumulator
  constexpr int VR = D + 8;        // LDS row stride (elements) of the row-major V tile
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nthreads = blockDim.x;
  const int r32 = lane & 31, h = lane >> 5;
  const int LG = a.LG, TG = a.TG, g = wave % LG, tg = wave / LG;
  const int mp = a.mp;
  int bh, c;
  xcd_map(blockIdx.x, a.BH, a.C, bh, c);
  const int c0 = c * a.chunk, c1 = min(a.n, c0 + a.chunk);
  const Tin* K = static_cast<const Tin*>(a.k) + (size_t)bh * a.n * D;
  const Tin* V = static_cast<const Tin*>(a.v) + (size_t)bh * a.n * D;

  // landmark operand, with s*log2(e) folded in so the scores come out in log2 units
  Pair8 qb[KD];
  {
    const float* qs = a.qt + ((size_t)bh * mp + 32 * g + r32) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < KD; ++s) {
      const f32x4 u0 = *reinterpret_cast<const f32x4*>(qs + 16 * s);
      const f32x4 u1 = *reinterpret_cast<const f32x4*>(qs + 16 * s + 4);
      float x[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x[q] = u0[q] * a.scale_log2e;
        x[4 + q] = u1[q] * a.scale_log2e;
      }
      qb[s] = split8(x);
    }
  }
  f32x16 wacc[FT];
#pragma unroll
  for (int f = 0; f < FT; ++f) wacc[f] = zero16();
  float M = kNegBig, L = 0.f;

  const int step = 32 * TG;
  const int nchunks = step * (D / 8);
  uint16_t* vt = reinterpret_cast<uint16_t*>(lds);  // [step][VR] V rows (hi)
  uint16_t* vt_lo = vt + (size_t)step * VR;          // fp32 input only
  // transposed-read addressing (see lds_tr16): lane 4j + q of each 16-lane group points
  // at token row j, feature column 16*(group & 1) + 4q of the feature tile
  const int trj = (lane & 15) >> 2;
  const int trcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  auto load_v = [&](int base, Chunk<Tin>* vc) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int qi = tid + nthreads * u;
      const int row = qi / (D / 8), cf = qi % (D / 8), tok = base + row;
      vc[u].load(V + (size_t)tok * D + cf * 8, qi < nchunks && tok < a.n);
    }
  };
  auto store_v = [&](const Chunk<Tin>* vc) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int qi = tid + nthreads * u;
      if (qi < nchunks) {
        const int row = qi / (D / 8), cf = qi % (D / 8);
        vc[u].store(vt + (size_t)row * VR + cf * 8, vt_lo + (size_t)row * VR + cf * 8);
      }
    }
  };
  auto load_k = [&](int base, Pair8* ka) {
    const int tok = base + 32 * tg + r32;
#pragma unroll
    for (int s = 0; s < KD; ++s)
      ka[s] = Input<Tin>::load8(K + (size_t)tok * D + 16 * s + 8 * h, tok < a.n);
  };

  Chunk<Tin> vc[NCH];
  Pair8 ka[KD];
  load_v(c0, vc);
  load_k(c0, ka);
  store_v(vc);
  __syncthreads();
  for (int base = c0; base < c1; base += step) {
    const bool more = base + step < c1;
    Pair8 kn[KD];
    if (more) {  // next step's K and V, in flight during this step's products
      load_v(base + step, vc);
      load_k(base + step, kn);
    }
    // scores (log2 units): rows = 32 tokens, columns = 32 landmarks
    f32x16 S = zero16();
#pragma unroll
    for (int s = 0; s < KD; ++s) S = mfma_pair<kS, true>(ka[s], qb[s], S);

    // online softmax over tokens per landmark; only the chunk's last step can be partial
    const bool partial = base + 32 * tg + 32 > c1;
    float mx = kNegBig;
    if (!partial) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, S[rr]);
    } else {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int tok = base + 32 * tg + 8 * (rr >> 2) + 4 * h + (rr & 3);
        if (tok >= c1) S[rr] = kNegBig;
        mx = fmaxf(mx, S[rr]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // lazy rescaling: keep the reference maximum while every lane's new maximum stays
    // within 2^8 of it (probabilities then stay <= 256); the state (M, L, acc) is exact
    // for any reference point
    if (__any(mx > M + 8.f)) {
      const float mn = fmaxf(M, mx);
      const float corr = fast_exp2(M - mn);
      L *= corr;
#pragma unroll
      for (int f = 0; f < FT; ++f) wacc[f] *= corr;
      M = mn;
    }
    float p[16];
    float ps = 0.f;
    if (!partial) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        p[rr] = fast_exp2(S[rr] - M);
        ps += p[rr];
      }
    } else {  // masked tokens contribute exactly 0 (M may still be the -1e30 start value)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        p[rr] = S[rr] > 0.5f * kNegBig ? fast_exp2(S[rr] - M) : 0.f;
        ps += p[rr];
      }
    }
    L += ps;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const Pair8 pb = split8(&p[8 * s2]);
      const size_t r0 = (size_t)(32 * tg + 16 * s2 + 4 * h + trj) * VR + trcol;
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        const size_t o = r0 + 32 * f;
        Pair8 va;
        va.hi = lds_tr16x2(vt + o, vt + o + 8 * VR);
        va.lo = kS ? lds_tr16x2(vt_lo + o, vt_lo + o + 8 * VR) : zero8();
        wacc[f] = mfma_pair<kS, true>(va, pb, wacc[f]);
      }
    }
    if (more) {
      __syncthreads();  // every wave is done with this step's V tile
      store_v(vc);
#pragma unroll
      for (int s = 0; s < KD; ++s) ka[s] = kn[s];
      __syncthreads();
    }
  }
  L += __shfl_xor(L, 32);

  // merge the TG token groups of each landmark group (fixed order)
  __syncthreads();
  float* mb = reinterpret_cast<float*>(lds);
  const int slot_floats = FT * 16 * 64 + 128;
  if (tg > 0) {
    float* sb = mb + (size_t)(g * (TG - 1) + tg - 1) * slot_floats;
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sb[(f * 16 + rr) * 64 + lane] = wacc[f][rr];
    sb[FT * 16 * 64 + lane] = M;
    sb[FT * 16 * 64 + 64 + lane] = L;
  }
  __syncthreads();
  if (tg == 0) {
    for (int o = 1; o < TG; ++o) {
      const float* sb = mb + (size_t)(g * (TG - 1) + o - 1) * slot_floats;
      const float mo = sb[FT * 16 * 64 + lane], lo = sb[FT * 16 * 64 + 64 + lane];
      const float mn = fmaxf(M, mo);
      const float ca = fast_exp2(M - mn), cb = fast_exp2(mo - mn);
      L = L * ca + lo * cb;
      M = mn;
#pragma unroll
      for (int f = 0; f < FT; ++f)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          wacc[f][rr] = wacc[f][rr] * ca + sb[(f * 16 + rr) * 64 + lane] * cb;
    }
    // partial W^T: [feature][landmark], 32 consecutive landmarks per register
    const int lm = 32 * g + r32;
    float* pw = a.part_w + ((size_t)bh * a.C + c) * D * mp + lm;
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr)
        pw[(size_t)(32 * f + acc_row(0, rr, lane)) * mp] = wacc[f][rr];
    if (h == 0) {
      float* pm = a.part_ml + ((size_t)bh * a.C + c) * 2 * mp;
      pm[lm] = M;
      pm[mp + lm] = L;
    }
  }
}

// ------------------------------------------------------------------ host side
static bool pinv_in_lds(int mp) { return mp <= 64; }

size_t context_lds_bytes(bool bf16, int d, int mp, int LG, int TG) {
  const size_t vbytes = (bf16 ? 1 : 2) * (size_t)(32 * TG) * (d + 8) * 2;
  const size_t mbytes = (size_t)LG * (TG - 1) * ((d / 32) * 16 * 64 + 128) * 4;
  return vbytes > mbytes ? vbytes : mbytes;
}

static size_t pinv_lds_bytes(int mp) {
  return pinv_in_lds(mp) ? (size_t)kLdsPlanes * mp * (mp + 8) * 2 : 0;
}

template <int D>
static hipError_t launch_pinv_t(const CtxArgs& a, hipStream_t s) {
  if (a.mp == 32)
    hipLaunchKernelGGL((pinv_lds_kernel<32, D>), dim3(a.BH), dim3(256), pinv_lds_bytes(32), s, a);
  else if (a.mp == 64)
    hipLaunchKernelGGL((pinv_lds_kernel<64, D>), dim3(a.BH), dim3(256), pinv_lds_bytes(64), s, a);
  else
    hipLaunchKernelGGL((pinv_kernel<false, 4, D>), dim3(a.BH), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pinv(int d, const CtxArgs& a, hipStream_t s) {
  if (d == 32) return launch_pinv_t<32>(a, s);
  if (d == 64) return launch_pinv_t<64>(a, s);
  return launch_pinv_t<128>(a, s);
}

static int flash_nch(int d, int LG) {
  const int n = (d + 16 * LG - 1) / (16 * LG);
  return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : 8;
}

template <typename Tin, int D>
static hipError_t launch_flash_t(const CtxArgs& a, hipStream_t s) {
  const size_t flds = context_lds_bytes(Input<Tin>::kSplit == false, D, a.mp, a.LG, a.TG);
  const dim3 grid(a.BH * a.C), block(64 * a.LG * a.TG);
  switch (flash_nch(D, a.LG)) {
    case 1: hipLaunchKernelGGL((flash_kernel<Tin, D, 1>), grid, block, flds, s, a); break;
    case 2: hipLaunchKernelGGL((flash_kernel<Tin, D, 2>), grid, block, flds, s, a); break;
    case 4: hipLaunchKernelGGL((flash_kernel<Tin, D, 4>), grid, block, flds, s, a); break;
    default: hipLaunchKernelGGL((flash_kernel<Tin, D, 8>), grid, block, flds, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_flash(bool bf16, int d, const CtxArgs& a, hipStream_t s) {
  if (bf16) {
    if (d == 32) return launch_flash_t<uint16_t, 32>(a, s);
    if (d == 64) return launch_flash_t<uint16_t, 64>(a, s);
    return launch_flash_t<uint16_t, 128>(a, s);
  }
  if (d == 32) return launch_flash_t<float, 32>(a, s);
  if (d == 64) return launch_flash_t<float, 64>(a, s);
  return launch_flash_t<float, 128>(a, s);
}

template <int D>
static hipError_t set_pinv_attr() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&pinv_lds_kernel<64, D>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)pinv_lds_bytes(64));
}

template <typename Tin, int D>
static hipError_t set_flash_attr(size_t bytes) {
  const void* fns[] = {reinterpret_cast<const void*>(&flash_kernel<Tin, D, 1>),
                       reinterpret_cast<const void*>(&flash_kernel<Tin, D, 2>),
                       reinterpret_cast<const void*>(&flash_kernel<Tin, D, 4>),
                       reinterpret_cast<const void*>(&flash_kernel<Tin, D, 8>)};
  for (const void* f : fns) {
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t configure_context(bool bf16, int d, size_t flash_lds) {
  hipError_t e;
  if (d == 32) e = set_pinv_attr<32>();
  else if (d == 64) e = set_pinv_attr<64>();
  else e = set_pinv_attr<128>();
  if (e != hipSuccess) return e;
  if (bf16) {
    if (d == 32) return set_flash_attr<uint16_t, 32>(flash_lds);
    if (d == 64) return set_flash_attr<uint16_t, 64>(flash_lds);
    return set_flash_attr<uint16_t, 128>(flash_lds);
  }
  if (d == 32) return set_flash_attr<float, 32>(flash_lds);
  if (d == 64) return set_flash_attr<float, 64>(flash_lds);
  return set_flash_attr<float, 128>(flash_lds);
}

}  // namespace nys
