// Stage 2 of the forward pass (Nystromformer review page, "Proposed method"):
//
//  * pseudo-inverse   one block per head: A_S = softmax_row(s Qt Kt^T), the scaling
//                     alpha = 1/(||A_S||_1 ||A_S||_inf), Z_0 = alpha A_S^T, then `iters`
//                     steps of Z <- 1/4 Z (13I - X(15I - X(7I - X))), X = A_S Z, every
//                     m x m product on MFMA. For mp <= 64 the operand planes live in LDS
//                     (4 waves) and these blocks ride at the front of the context launch;
//                     larger mp keeps them in global memory: pinv_global_kernel (16
//                     waves per head) forms A_S and Z_0, then every product of the
//                     iteration is its own launch over all heads (pinv_phase_kernel).
//  * landmark context BH * C blocks: the right factor softmax_row(s Qt K^T) V, computed
//                     without forming the m x n matrix: each block streams one chunk of
//                     K/V tiles, keeps a running max / sum per landmark (online softmax
//                     over n) and an unnormalised m x d accumulator; it writes that
//                     partial state (feature-major, so the merge reads it as W^T).
//
// The two need only the segment means, so one launch overlaps the latency-bound
// pseudo-inverse with the bandwidth-bound context stream. Blocks never exchange data
// inside a kernel: on MI355X each XCD has its own L2, and a device-scope hand-off costs
// an L2 write-back plus invalidate per block. The output stage merges the C partial
// states (fixed chunk order, log-sum-exp rescaling) and forms Y = Z W in its prologue.
#include <algorithm>

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
// Variant for 64 < mp <= 256 (one block of 16 waves per head, up to four tiles per wave):
// hi/lo operand planes in a slice of CtxArgs::planes, 18 of them (row- and column-major
// copies, double-buffered where one launch reads a matrix while another of its waves
// writes the next one, so that no plane is read and rewritten by one launch). The
// multi-launch iteration (pinv_phase_kernel) uses kPZc, Z_0's columns, for the odd
// iterations' X rows once X_0 is formed, and kPX2r for X^2 rows.
enum { kPA = 0, kPZr = 2, kPZc = 4, kPXr = 6, kPXc = 8, kPX2T = 10, kGZr1 = 12, kPX2r = 14,
       kGT = 16, kPXr1 = kPZc };
static_assert(kPlanes == 18, "plane count");

template <int TPW>
__device__ __forceinline__ void pinv_body(const CtxArgs& a, int bh, uint16_t* pl, float* red,
                                          float* red_part, float* red_col) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthreads = blockDim.x, nw = nthreads >> 6;
  const int mp = a.mp, m = a.m, nt = mp / 32, ntiles = nt * nt;
  const size_t P = (size_t)mp * mp;
  const int dd = a.d;
  float* A = a.a_s + (size_t)bh * P;
  auto plane = [&](int idx) { return pl + (size_t)idx * P; };

  // 1. logits Qt Kt^T (both landmark sets as hi/lo planes, K = d), scaled to log2
  //    units, held in registers: tile t = wave + nw*u of the mp x mp matrix.
  constexpr int TPW0 = 4;  // tiles per wave (mp <= 256, 16 waves)
  f32x16 at[TPW0];
  {
    const uint16_t* qh = a.qt_hl + (size_t)bh * 2 * mp * dd;
    const uint16_t* kh = a.kt_hl + (size_t)bh * 2 * mp * dd;
#pragma unroll
    for (int u = 0; u < TPW0; ++u) {
      const int t = wave + nw * u;
      if (t < ntiles)
        at[u] = gemm_tile_rt(qh, qh + (size_t)mp * dd, dd, kh, kh + (size_t)mp * dd, dd,
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

  // 5. the iterations run as separate launches (pinv_phase_kernel); with none, hand Z_0
  //    (row-major hi/lo) to the output stage here
  if (a.iters == 0) {
    uint16_t* dst = a.z_hl + (size_t)bh * 2 * P;
    const int n8 = (int)(P / 8);
    for (int e = tid; e < 2 * n8; e += nthreads) {
      const int which = e / n8, off = (e % n8) * 8;
      st8(dst + (size_t)which * P + off, ld8(plane(kPZr + which) + off));
    }
  }
}

// First step for mp > 64 when the iteration runs (iters > 0), one block per 32-row strip
// of A_S (nt = mp / 32 waves, wave w forms the tile in column strip w): the scaled logits,
// the row softmax, A_S in fp32 (for the taps) and as hi/lo row planes, and the unscaled
// row and column planes of A_S that Z_0 = alpha A_S^T is built from. alpha needs every
// strip's column sums, so each strip stores its partial column abs-sums and its largest
// row abs-sum; the first iteration's X = A Z_0 and Z_1 = Z_0 T / 4 apply alpha to their
// products (pinv_alpha).
__global__ __launch_bounds__(512) void pinv_strip_kernel(CtxArgs a) {
  __shared__ float red_part[32 * 8];  // [row of the strip][column tile]
  __shared__ float red_rows[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r32 = lane & 31;
  const int mp = a.mp, m = a.m, nt = mp / 32, dd = a.d;
  int bh, strip;
  xcd_map(blockIdx.x, a.BH, nt, bh, strip);
  const size_t P = (size_t)mp * mp;
  const int row0 = 32 * strip, col0 = 32 * wave, j = col0 + r32;
  uint16_t* pl = a.planes + (size_t)bh * kPlanes * P;
  auto plane = [&](int idx) { return pl + (size_t)idx * P; };
  const uint16_t* qh = a.qt_hl + (size_t)bh * 2 * mp * dd;
  const uint16_t* kh = a.kt_hl + (size_t)bh * 2 * mp * dd;
  f32x16 at = gemm_tile_rt(qh, qh + (size_t)mp * dd, dd, kh, kh + (size_t)mp * dd, dd, row0,
                           col0, dd, lane) * a.scale_log2e;
  auto lrow = [&](int rr) { return acc_row(0, rr, lane); };  // row within the strip
  // row maxima over the m real columns: half-wave, then across the column tiles
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const float mx = half_max(j < m ? at[rr] : kNegBig);
    if (r32 == 0) red_part[lrow(rr) * nt + wave] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int i = row0 + lrow(rr);
    float mx = kNegBig;
    for (int c = 0; c < nt; ++c) mx = fmaxf(mx, red_part[lrow(rr) * nt + c]);
    at[rr] = (i < m && j < m) ? fast_exp2(at[rr] - mx) : 0.f;
  }
  __syncthreads();  // every wave has read the maxima before the sums overwrite them
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const float sm = half_sum(at[rr]);
    if (r32 == 0) red_part[lrow(rr) * nt + wave] = sm;
  }
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    float sum = 0.f;
    for (int c = 0; c < nt; ++c) sum += red_part[lrow(rr) * nt + c];
    at[rr] = row0 + lrow(rr) < m ? at[rr] / sum : 0.f;
  }
  __syncthreads();
  // abs row sums (partials per column tile) and this strip's abs column sums
  float cs = 0.f;
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const float rs = half_sum(fabsf(at[rr]));
    if (r32 == 0) red_part[lrow(rr) * nt + wave] = rs;
    cs += fabsf(at[rr]);
  }
  cs += __shfl_xor(cs, 32);
  float* part = a.alpha_part + ((size_t)bh * nt + strip) * (mp + 1);
  if (lane < 32) part[j] = cs;
  __syncthreads();
  if (wave == 0) {
    float rmax = 0.f;
    if (lane < 32 && row0 + lane < m) {
      float rs = 0.f;
      for (int c = 0; c < nt; ++c) rs += red_part[lane * nt + c];
      rmax = rs;
    }
    rmax = wave_max(rmax);
    if (lane == 0) part[mp] = rmax;
  }
  // A_S (fp32 copy for inspection, hi/lo rows) and the unscaled Z_0 planes, fragment-major
  store_rows_f32(a.a_s + (size_t)bh * P, mp, row0, col0, at, lane);
  store_rows_hl_frag(plane(kPA), plane(kPA + 1), mp, row0, col0, at, lane);
  store_rows_hl_frag(plane(kPZc), plane(kPZc + 1), mp, row0, col0, at, lane);
  store_cols_hl_frag(plane(kPZr), plane(kPZr + 1), mp, row0, col0, at, lane);
}

// alpha = 1 / (max column abs-sum * max row abs-sum) of head bh's A_S, from the partial
// sums pinv_strip_kernel left (one wave, every lane gets the value).
__device__ __forceinline__ float pinv_alpha(const CtxArgs& a, int bh, int lane) {
  const int mp = a.mp, nt = mp / 32;
  const float* part = a.alpha_part + (size_t)bh * nt * (mp + 1);
  float cmax = 0.f, rmax = 0.f;
  for (int j = lane; j < a.m; j += 64) {
    float cs = 0.f;
    for (int s = 0; s < nt; ++s) cs += part[(size_t)s * (mp + 1) + j];
    cmax = fmaxf(cmax, cs);
  }
  if (lane < nt) rmax = part[(size_t)lane * (mp + 1) + mp];
  return 1.0f / (wave_max(cmax) * wave_max(rmax));
}

// The iteration for every head at once (mp > 64): one wave per 32 x 32 output tile,
// operands read from the head's planes in global memory (they stay in the XCD's L2: a
// head's tiles run on one XCD). The planes written by the strip kernel and by these
// launches are fragment-major (frag_off), so every operand load reads whole cache lines;
// only the final Z leaves row-major. Launch boundaries order the steps, so the m x m
// products of a head spread over many CUs instead of one.
// X = A Z is mostly carried along instead of being formed again from each Z: with
// T_k = 13I - 15X_k + 7X_k^2 - X_k^3, Z_{k+1} = Z_k T_k / 4 gives
// X_{k+1} = A Z_{k+1} = (13X_k - 15X_k^2 + 7X_k^3 - X_k^4) / 4, a polynomial in X_k. The X
// chain then takes two dependent launches per iteration, and each Z product runs beside
// the next iteration's X^2 (the same iterates as forming X = A Z every time, up to
// rounding). Carried X drifts from A Z by rounding that the iteration no longer corrects
// (max error of Z 1e-2 of its RMS on clustered inputs, against 3e-4 with X formed from
// Z every time), so X is formed again as A Z at the refresh iterations (pinv_refresh:
// the last one and every second one before it, down to half of the count), which brings
// the error back to the level of the plain iteration.
//   PH 0:  X_k = A Z_k (k = 0, or a refresh) -> X rows and columns (hi/lo), fp32 X
//   PH 1:  X_k^2 = X_k X_k -> X^2 rows and columns (hi/lo), fp32 X^2; with kWithZ the
//          second half of the grid forms Z_k = Z_{k-1} T_{k-1} / 4 -> Z rows; kZOnly
//          (before a refresh) forms only Z_k, as rows and as columns (into the X^2 row
//          planes, free until X_k^2)
//   PH 2:  X^3 = X X^2 and T_k -> T columns (hi/lo); with kMore also X^4 = X^2 X^2 and
//          X_{k+1} -> X rows (other set) and columns, fp32 X
//   PH 3:  Z_I = Z_{I-1} T_{I-1} / 4 -> fp32 Z and the row-major hi/lo copy
// Z_0's planes are unscaled (A_S^T): X_0 and Z_1 take alpha on their products.
enum { kWithZ = 1, kZOnly = 2, kMore = 1, kRefresh = 1 };

__host__ __device__ constexpr bool pinv_refresh(int k, int iters) {
  return k >= 1 && 2 * k >= iters && (iters - 1 - k) % 2 == 0;
}

template <int PH, int KS>
__global__ __launch_bounds__(64) void pinv_phase_kernel(CtxArgs a, int it, int flags) {
  __shared__ float st[32 * kStageLd];
  const int lane = threadIdx.x;
  constexpr int mp = 16 * KS, nt = mp / 32;
  const int per = a.BH * nt * nt;
  // PH 1: the Z product (second half of the grid, or all of it)
  const int half = (PH == 1 && ((flags & kZOnly) || (int)blockIdx.x >= per)) ? 1 : 0;
  const int bx = (PH == 1 && !(flags & kZOnly)) ? (int)blockIdx.x - half * per : (int)blockIdx.x;
  int bh, t;
  xcd_map(bx, a.BH, nt * nt, bh, t);
  const size_t P = (size_t)mp * mp;
  const int row0 = 32 * (t / nt), col0 = 32 * (t % nt);
  uint16_t* pl = a.planes + (size_t)bh * kPlanes * P;
  auto plane = [&](int idx) { return pl + (size_t)idx * P; };
  auto xrows = [&](int k) { return (k & 1) ? kPXr1 : kPXr; };
  auto zrows = [&](int k) { return (k & 1) ? kGZr1 : kPZr; };
  float* own = a.own + (size_t)bh * 2 * P;
  if constexpr (PH == 0) {
    const bool refresh = flags & kRefresh;  // Z_k's columns sit in the X^2 row planes
    const int zc = refresh ? kPX2r : kPZc, xr = xrows(it);
    f32x16 x = gemm_tile_frag<KS>(plane(kPA), plane(kPA + 1), plane(zc), plane(zc + 1), row0,
                                  col0, lane);
    if (!refresh) x *= pinv_alpha(a, bh, lane);
    stage_tile(st, x, lane);
    stage_store_frag<false>(plane(xr), plane(xr + 1), mp, row0, col0, st, lane);
    stage_store_frag<true>(plane(kPXc), plane(kPXc + 1), mp, row0, col0, st, lane);
    stage_store_f32(own, mp, row0, col0, st, lane);
  } else if constexpr (PH == 1) {
    if (half == 0) {
      const int xr = xrows(it);
      const f32x16 x2 = gemm_tile_frag<KS>(plane(xr), plane(xr + 1), plane(kPXc),
                                           plane(kPXc + 1), row0, col0, lane);
      stage_tile(st, x2, lane);
      stage_store_frag<false>(plane(kPX2r), plane(kPX2r + 1), mp, row0, col0, st, lane);
      stage_store_frag<true>(plane(kPX2T), plane(kPX2T + 1), mp, row0, col0, st, lane);
      stage_store_f32(own + P, mp, row0, col0, st, lane);
    } else {
      const int zr = zrows(it - 1), zr_n = zrows(it);
      const f32x16 zv = gemm_tile_frag<KS>(plane(zr), plane(zr + 1), plane(kGT),
                                           plane(kGT + 1), row0, col0, lane) *
                        (it == 1 ? 0.25f * pinv_alpha(a, bh, lane) : 0.25f);
      stage_tile(st, zv, lane);
      stage_store_frag<false>(plane(zr_n), plane(zr_n + 1), mp, row0, col0, st, lane);
      if (flags & kZOnly)
        stage_store_frag<true>(plane(kPX2r), plane(kPX2r + 1), mp, row0, col0, st, lane);
    }
  } else if constexpr (PH == 2) {
    const int j = col0 + (lane & 31), xr = xrows(it);
    const bool more = flags & kMore;
    f32x16 x3, x4 = zero16();
    if (more)  // X^3 and X^4 share the columns of X^2
      gemm_tile_frag2<KS>(plane(xr), plane(xr + 1), plane(kPX2r), plane(kPX2r + 1), plane(kPX2T),
                          plane(kPX2T + 1), row0, col0, lane, x3, x4);
    else
      x3 = gemm_tile_frag<KS>(plane(xr), plane(xr + 1), plane(kPX2T), plane(kPX2T + 1), row0,
                              col0, lane);
    f32x16 tv, xn;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const size_t o = (size_t)acc_row(row0, rr, lane) * mp + j;
      const float diag = (acc_row(row0, rr, lane) == j) ? 13.f : 0.f;
      const float x = own[o], x2 = own[P + o];
      tv[rr] = diag - 15.f * x + 7.f * x2 - x3[rr];
      xn[rr] = 0.25f * (13.f * x - 15.f * x2 + 7.f * x3[rr] - x4[rr]);
    }
    stage_tile(st, tv, lane);
    stage_store_frag<true>(plane(kGT), plane(kGT + 1), mp, row0, col0, st, lane);
    if (more) {
      __syncthreads();  // the staging tile is read out before it takes X_{k+1}
      const int xr_n = xrows(it + 1);
      stage_tile(st, xn, lane);
      stage_store_frag<false>(plane(xr_n), plane(xr_n + 1), mp, row0, col0, st, lane);
      stage_store_frag<true>(plane(kPXc), plane(kPXc + 1), mp, row0, col0, st, lane);
      stage_store_f32(own, mp, row0, col0, st, lane);
    }
  } else {
    const int zr = zrows(a.iters - 1);
    const f32x16 zv = gemm_tile_frag<KS>(plane(zr), plane(zr + 1), plane(kGT), plane(kGT + 1),
                                         row0, col0, lane) *
                      (a.iters == 1 ? 0.25f * pinv_alpha(a, bh, lane) : 0.25f);
    stage_tile(st, zv, lane);
    uint16_t* dst = a.z_hl + (size_t)bh * 2 * P;
    stage_store_rows_hl(dst, dst + P, mp, row0, col0, st, lane);
    stage_store_f32(a.z + (size_t)bh * P, mp, row0, col0, st, lane);
  }
}

// ------------------------------------------------------------------ pinv, mp <= 64
// Compile-time specialisation for MP in {32, 64}: one 32x32 tile per wave (waves beyond
// the tile count only join the barriers), every loop unrolled, operand planes in LDS.
//
// Every m x m matrix lives in LDS once, row-major (hi and lo planes), with the 16-byte
// chunks of each row permuted (swz_off). A product C = A B is formed transposed on MFMA
// (C^T = B^T A^T): rows of A are read as 16-byte runs, columns of B with LDS transpose
// reads, and the result comes out one row of C per lane (16 values in four runs of four
// columns), which is stored as 8-byte row runs.
template <int MP>
__device__ __forceinline__ int swz(int r, int c) {
  return swz_off<MP / 8>(r, c);
}

// Column of register rr in the row-per-lane layout of a tile at column col0.
__device__ __forceinline__ int row_tile_col(int col0, int rr, int lane) {
  return col0 + 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
}

// MFMA B operand of C = A B from rows row0..row0+31 of A: lane l holds row row0 + l % 32,
// k-slots 16 s + 8 (l / 32) + e of k-step s.
template <int MP>
__device__ __forceinline__ void load_row_operand(const uint16_t* ahi, const uint16_t* alo,
                                                 int row0, int lane, Pair8* bo) {
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int s = 0; s < MP / 16; ++s) {
    const int k0 = 16 * s + 8 * h;
    bo[s] = Pair8{ld8(ahi + swz<MP>(row0 + r, k0)), ld8(alo + swz<MP>(row0 + r, k0))};
  }
}

// C[row0:+32, col0:+32] of C = A B for MP x MP planes, row-per-lane layout: lane l holds
// row row0 + l % 32, register rr column row_tile_col(col0, rr, l). bo: rows of A from
// load_row_operand.
template <int MP>
__device__ __forceinline__ f32x16 prod_rows_op(const Pair8* bo, const uint16_t* bhi,
                                               const uint16_t* blo, int col0, int lane) {
  constexpr int KS = MP / 16;
  const int h = lane >> 5;
  // transposed reads: lane 4j + q of each 16-lane group addresses row k0 + j, column
  // col0 + 16 * (group & 1) + 4q; the result lane then holds column col0 + lane % 32
  const int trj = (lane & 15) >> 2, trc = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  Pair8 ao[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int k0 = 16 * s + 8 * h;
    ao[s].hi = lds_tr16x2(bhi + swz<MP>(k0 + trj, trc), bhi + swz<MP>(k0 + 4 + trj, trc));
    ao[s].lo = lds_tr16x2(blo + swz<MP>(k0 + trj, trc), blo + swz<MP>(k0 + 4 + trj, trc));
  }
  f32x16 acc = zero16();
#pragma unroll
  for (int s = 0; s < KS; ++s) acc = mfma_pair<true, true>(ao[s], bo[s], acc);
  return acc;
}

template <int MP>
__device__ __forceinline__ f32x16 prod_rows(const uint16_t* ahi, const uint16_t* alo,
                                            const uint16_t* bhi, const uint16_t* blo,
                                            int row0, int col0, int lane) {
  Pair8 bo[MP / 16];
  load_row_operand<MP>(ahi, alo, row0, lane, bo);
  return prod_rows_op<MP>(bo, bhi, blo, col0, lane);
}

// Store a row-per-lane tile into swizzled hi/lo planes (four 8-byte runs per plane).
template <int MP>
__device__ __forceinline__ void store_row_tile(uint16_t* hi, uint16_t* lo, int row0, int col0,
                                               const f32x16& v, int lane) {
  const int i = row0 + (lane & 31), h = lane >> 5;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint16_t a[4], b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split1(v[4 * g + e], a[e], b[e]);
    const int o = swz<MP>(i, col0 + 8 * g + 4 * h);
    *reinterpret_cast<u32x2*>(hi + o) =
        u32x2{(uint32_t)a[0] | ((uint32_t)a[1] << 16), (uint32_t)a[2] | ((uint32_t)a[3] << 16)};
    *reinterpret_cast<u32x2*>(lo + o) =
        u32x2{(uint32_t)b[0] | ((uint32_t)b[1] << 16), (uint32_t)b[2] | ((uint32_t)b[3] << 16)};
  }
}

// Row-per-lane tile to a row-major fp32 matrix in global memory (ld = MP).
template <int MP>
__device__ __forceinline__ void store_row_tile_f32(float* p, int row0, int col0, const f32x16& v,
                                                   int lane) {
  float* q = p + (size_t)(row0 + (lane & 31)) * MP + col0 + 4 * (lane >> 5);
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<f32x4*>(q + 8 * g) = f32x4{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
}

// LDS planes (hi, lo pairs) for Z, X and X^2 / T; the iteration rotates their roles.
// A_S passes through the third pair once on its way into registers.
enum { kQZ = 0, kQX = 2, kQT = 4, kQPlanes = 6 };

template <int MP>
constexpr size_t pinv_lds_planes_bytes() { return (size_t)kQPlanes * MP * MP * 2; }

template <int MP, int D>
__device__ __forceinline__ void pinv_lds_body(const CtxArgs& a, int bh, uint16_t* pl,
                                              float* red_part, float* red_col, float* red) {
  constexpr int NT = MP / 32, NTILES = NT * NT, KD = D / 16;
  constexpr int P = MP * MP;
  auto plane = [&](int idx) { return pl + idx * P; };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r32 = lane & 31, h = lane >> 5;
  const int m = a.m;
  const bool mine = wave < NTILES;
  const int row0 = 32 * (wave / NT), ti = wave / NT, tj = wave % NT, col0 = 32 * tj;
  const int irow = row0 + r32;  // the row this lane holds

  // 1. scaled logits (log2 units), row-per-lane: the product Kt Qt^T read transposed
  f32x16 at = zero16();
  if (mine) {
    const uint16_t* qh = a.qt_hl + (size_t)bh * 2 * MP * D;
    const uint16_t* kh = a.kt_hl + (size_t)bh * 2 * MP * D;
    at = gemm_tile_k<KD>(kh, kh + MP * D, D, qh, qh + MP * D, D, col0, row0, lane) * a.scale_log2e;
  }
  // 2. row softmax over the m real landmarks (padded rows/columns become 0) and
  // alpha = 1 / (max column abs-sum * max row abs-sum), with two barriers. A lane holds
  // 16 of its row's columns in the tile, its partner lane (l ^ 32) the other 16. Each
  // tile leaves its row maximum and its sum of exponentials relative to that maximum;
  // the row's softmax combines the NT partials, each rescaled by exp(mx_c - M).
  float mloc = kNegBig;
  if (mine) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
      if (row_tile_col(col0, rr, lane) < m) mloc = fmaxf(mloc, at[rr]);
    mloc = halves_max(mloc);
    float sloc = 0.f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      at[rr] = row_tile_col(col0, rr, lane) < m ? fast_exp2(at[rr] - mloc) : 0.f;
      sloc += at[rr];
    }
    sloc = halves_sum(sloc);
    if (h == 0) {
      red_part[2 * (irow * NT + tj)] = mloc;
      red_part[2 * (irow * NT + tj) + 1] = sloc;
    }
  }
  __syncthreads();  // every tile's row partials are in
  float rsum = 0.f;  // this row's abs-sum: the entries are positive, so sum * (1 / sum)
  if (mine) {
    float M = kNegBig;
#pragma unroll
    for (int c = 0; c < NT; ++c) M = fmaxf(M, red_part[2 * (irow * NT + c)]);
    float S = 0.f;
#pragma unroll
    for (int c = 0; c < NT; ++c)
      S += red_part[2 * (irow * NT + c) + 1] * fast_exp2(red_part[2 * (irow * NT + c)] - M);
    const float inv = irow < m ? 1.f / S : 0.f;
    const float sc = fast_exp2(mloc - M) * inv;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) at[rr] *= sc;
    rsum = S * inv;
    // abs column sums of this tile over its 32 rows, all formed before any is stored
    // (lanes 31 and 63 hold them)
    float cs[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) cs[rr] = half_sum_upper(at[rr]);
    if (r32 == 31) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) red_col[ti * MP + row_tile_col(col0, rr, lane)] = cs[rr];
    }
  }
  const float rmax_w = wave_max_dpp(rsum);
  if (lane == 0) red[wave] = rmax_w;
  __syncthreads();  // column partials and every wave's largest row sum are in
  // every wave forms alpha itself: lane j sums column j's partials (MP <= 64)
  float csum = 0.f;
  if (lane < m) {
#pragma unroll
    for (int c = 0; c < NT; ++c) csum += red_col[c * MP + lane];
  }
  const float cmax = wave_max_dpp(csum);
  const float rmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float alpha = 1.0f / (cmax * rmax);
  // 3. A_S (operand planes; the fp32 copy only on inspection calls), Z_0 = alpha A_S^T
  if (mine) {
    if (a.fp32_out) store_row_tile_f32<MP>(a.a_s + (size_t)bh * P, row0, col0, at, lane);
    store_row_tile<MP>(plane(kQT), plane(kQT + 1), row0, col0, at, lane);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {  // element (i, j) of A goes to Z_0[j][i]
      const int j = row_tile_col(col0, rr, lane);
      uint16_t hb, lb;
      const float zv = alpha * at[rr];
      split1(zv, hb, lb);
      plane(kQZ)[swz<MP>(j, irow)] = hb;
      plane(kQZ + 1)[swz<MP>(j, irow)] = lb;
      if (a.iters == 0 && a.fp32_out) a.z[(size_t)bh * P + (size_t)j * MP + irow] = zv;
    }
  }
  __syncthreads();
  // the wave's rows of A_S stay in registers for every X = A Z (the T planes that held
  // them are first rewritten after the barrier that follows the first X)
  constexpr int KM = MP / 16;
  Pair8 abo[KM];
  if (mine) load_row_operand<MP>(plane(kQT), plane(kQT + 1), row0, lane, abo);
  // 4. iterations Z <- 1/4 Z (13I - 15X + 7X^2 - X^3), X = A Z. The three plane pairs
  // rotate roles (pz holds Z, px receives X, pt X^2): once X = A Z is formed, each wave's
  // rows of Z sit in registers, so T = 13I - 15X + 7X^2 - X^3 can overwrite the Z planes
  // and the new Z the X planes, four barriers per iteration.
  int pz = kQZ, px = kQX, pt = kQT;
  for (int it = 0; it < a.iters; ++it) {
    f32x16 u;  // 13I - 15X + 7X^2, formed once X^2 is known
    Pair8 zrows[KM];
    if (mine) {  // X = A Z; this wave's rows of Z kept for Z T
      load_row_operand<MP>(plane(pz), plane(pz + 1), row0, lane, zrows);
      u = prod_rows_op<MP>(abo, plane(pz), plane(pz + 1), col0, lane);
      store_row_tile<MP>(plane(px), plane(px + 1), row0, col0, u, lane);
    }
    __syncthreads();
    if (mine) {  // X^2 = X X
      const f32x16 x2 =
          prod_rows<MP>(plane(px), plane(px + 1), plane(px), plane(px + 1), row0, col0, lane);
      store_row_tile<MP>(plane(pt), plane(pt + 1), row0, col0, x2, lane);
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float diag = (irow == row_tile_col(col0, rr, lane)) ? 13.f : 0.f;
        u[rr] = diag - 15.f * u[rr] + 7.f * x2[rr];
      }
    }
    __syncthreads();
    if (mine) {  // X^3 = X X^2, then T = 13I - 15X + 7X^2 - X^3 into the Z planes
      const f32x16 x3 =
          prod_rows<MP>(plane(px), plane(px + 1), plane(pt), plane(pt + 1), row0, col0, lane);
      store_row_tile<MP>(plane(pz), plane(pz + 1), row0, col0, u - x3, lane);
    }
    __syncthreads();
    if (mine) {  // Z <- Z T / 4, into the X planes
      const f32x16 zv = prod_rows_op<MP>(zrows, plane(pz), plane(pz + 1), col0, lane) * 0.25f;
      store_row_tile<MP>(plane(px), plane(px + 1), row0, col0, zv, lane);
      if (it == a.iters - 1 && a.fp32_out)
        store_row_tile_f32<MP>(a.z + (size_t)bh * P, row0, col0, zv, lane);
    }
    __syncthreads();
    const int nz = px;
    px = pt;
    pt = pz;
    pz = nz;
  }
  // 5. Z (row-major hi/lo, unpermuted) for the output stage
  uint16_t* dst = a.z_hl + (size_t)bh * 2 * P;
  for (int e = tid; e < 2 * P / 8; e += blockDim.x) {
    const int which = e / (P / 8), r = (e % (P / 8)) / (MP / 8), c8 = (e % (MP / 8)) * 8;
    st8(dst + (size_t)which * P + r * MP + c8, ld8(plane(pz + which) + swz<MP>(r, c8)));
  }
}


template <int D>
__global__ __launch_bounds__(1024) void pinv_global_kernel(CtxArgs a) {
  __shared__ float red[32];
  __shared__ float red_part[256 * 8];  // [row][column tile] partial max / sums
  __shared__ float red_col[8 * 256];   // [row tile][column] partial column sums
  const int bh = blockIdx.x;
  pinv_body<4>(a, bh, a.planes + (size_t)bh * kPlanes * a.mp * a.mp, red, red_part, red_col);
}

// Head, chunk and token range [c0, c1) of context block blk (without the pseudo-inverse
// blocks), the range cut at the head's valid length (an empty chunk leaves M = -inf,
// L = 0). Even split: blocks are mapped to (head, chunk) by xcd_map and chunk c is
// [c chunk, (c + 1) chunk). Uneven split (uneven_ncu > 0, chosen on the host when the
// fused pseudo-inverse blocks share CUs with context blocks): blocks are chunk-major
// (block c BH + bh of the context range) and land round-robin on uneven_ncu CUs after the
// npinv pseudo-inverse blocks; a context block on a CU that also holds a pseudo-inverse
// block runs at about 0.7 of the speed of the others, so each head's tokens are split in
// proportion to those weights over its chunks, in whole steps of 32 TG tokens.
__device__ __forceinline__ void context_block(const CtxArgs& a, int blk, int& bh, int& c,
                                              int& c0, int& c1) {
  if (a.uneven_ncu == 0) {
    xcd_map(blk, a.BH, a.C, bh, c);
    c0 = c * a.chunk;
    c1 = c0 + a.chunk;
  } else {
    bh = blk % a.BH;
    c = blk / a.BH;
    const int ncu = a.uneven_ncu, step = 32 * a.TG, nsteps = (a.n + step - 1) / step;
    auto weight = [&](int cc) {
      const long long b = (long long)a.npinv + (long long)cc * a.BH + bh;
      return (b >= ncu && (int)(b % ncu) < a.npinv) ? 0.7 : 1.0;
    };
    double total = 0.0;
    for (int cc = 0; cc < a.C; ++cc) total += weight(cc);
    double cum = 0.0;
    int start = 0;
    c0 = c1 = 0;
    for (int cc = 0; cc <= c; ++cc) {
      cum += weight(cc);
      const int end = cc == a.C - 1
                          ? a.n
                          : min(a.n, step * (int)llround((double)nsteps * cum / total));
      c0 = min(start, end);
      c1 = end;
      start = max(start, end);
    }
  }
  c1 = min(valid_length(a.lengths, bh, a.H, a.n, a.m), c1);
}

// Merge the TG token groups of each landmark group (fixed order) and write the block's
// partial state: W^T [feature][landmark] unnormalised, running max (log2 units) and sum.
// mb: LDS scratch of LG * (TG - 1) slots; the caller synchronises before reusing LDS.
template <int D>
__device__ __forceinline__ void flash_store_partial(const CtxArgs& a, int bh, int c,
                                                    f32x16* wacc, float M, float L, float* mb) {
  constexpr int FT = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r32 = lane & 31, h = lane >> 5;
  const int LG = a.LG, TG = a.TG, g = wave % LG, tg = wave / LG, mp = a.mp;
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

// ------------------------------------------------------------------ context, fp32
// Register staging (fp32 inputs are split into hi/lo bf16 tiles on the way to LDS).
// NCH: 8-element V chunks each thread stages per step (D / (16 * LG), rounded up).
template <typename Tin, int D, int NCH>
__device__ __forceinline__ void flash_reg_body(const CtxArgs& a, int blk, char* lds) {
  constexpr bool kS = Input<Tin>::kSplit;
  constexpr int KD = D / 16;       // k-steps over features
  constexpr int FT = D / 32;       // feature tiles of the accumulator
  constexpr int VR = D + 8;        // LDS row stride (elements) of the row-major V tile
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nthreads = blockDim.x;
  const int r32 = lane & 31, h = lane >> 5;
  const int LG = a.LG, TG = a.TG, g = wave % LG, tg = wave / LG;
  const int mp = a.mp;
  int bh, c, c0, c1;
  context_block(a, blk, bh, c, c0, c1);
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
      vc[u].load(V + (size_t)tok * D + cf * 8, qi < nchunks && tok < c1);
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
      ka[s] = Input<Tin>::load8(K + (size_t)tok * D + 16 * s + 8 * h, tok < c1);
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
      for (int f = 0; f < FT; ++f) scale_in_place(wacc[f], corr);
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
  __syncthreads();  // LDS becomes the merge buffer
  flash_store_partial<D>(a, bh, c, wacc, M, L, reinterpret_cast<float*>(lds));
}

// ------------------------------------------------------------------ context, bf16
// K and V tiles of `step` tokens stream through a ring of ring_stages LDS slots filled
// by LDS-DMA (no registers held for data in flight): while tile t is consumed, tiles
// t+1 .. t+stages-1 are in flight. Each tile is row-major with permuted 16-byte chunks
// (swz_off); a wave's DMA instruction i covers slots [64 (i W + wave), +64) of the tile,
// slot s holding row s / CPR, chunk (s % CPR) ^ key. Slots past the tile's real chunks
// (and rows past the chunk end) load a valid row of the head whose values are masked.
template <int D>
__device__ __forceinline__ void flash_ring_body(const CtxArgs& a, int blk, char* lds) {
  constexpr int KD = D / 16;       // k-steps over features
  constexpr int FT = D / 32;       // feature tiles of the accumulator
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  // the wave index read into a scalar register: everything derived from it (the wave's
  // landmark and token groups, LDS destinations, the partial-step test) stays scalar
  const int tid = threadIdx.x, lane = tid & 63, nw = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, h = lane >> 5;
  const int LG = a.LG, TG = a.TG, g = wave % LG, tg = wave / LG;
  const int mp = a.mp;
  int bh, c, c0, c1;
  context_block(a, blk, bh, c, c0, c1);
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + (size_t)bh * a.n * D;
  const uint16_t* V = static_cast<const uint16_t*>(a.v) + (size_t)bh * a.n * D;

  const int step = 32 * TG;
  const int NI = a.ring_ni, S = a.ring_stages;
  const int tile_elems = nw * NI * 512;  // 1 KiB (512 bf16) per wave instruction
  const int real = step * CPR;
  const int nsteps = c1 > c0 ? (c1 - c0 + step - 1) / step : 0;
  uint16_t* ring = reinterpret_cast<uint16_t*>(lds);
  // Instruction i of a wave moves 16-byte chunk s = 64 (i nw + wave) + lane of the step:
  // row s / CPR, chunk (s % CPR) ^ chunk_key(row). The key repeats every 8 rows, so when
  // an instruction covers a multiple of 8 rows (RI), the lane's chunk is the same for
  // every i and its source offset grows by RI rows per instruction.
  const int RI = 64 * nw / CPR;
  const bool uniform_rows = RI % 8 == 0 && real == NI * 64 * nw;
  const int r0 = (64 * wave + lane) / CPR;
  const uint32_t lane_bytes = 2u * (uint32_t)(r0 * D + 8 * ((lane % CPR) ^ chunk_key<CPR>(r0)));
  const uint32_t inst_bytes = 2u * (uint32_t)(RI * D);
  auto issue = [&](int t, int slot) {
    const int base = c0 + t * step;
    uint16_t* dk = ring + (size_t)slot * 2 * tile_elems;
    uint16_t* dv = dk + tile_elems;
    if (uniform_rows && base + step <= c1) {  // a whole step: no row is clamped
      const uint16_t* kb = K + (size_t)base * D;
      const uint16_t* vb = V + (size_t)base * D;
      for (int i = 0; i < NI; ++i) {
        const int b = i * nw + wave;
        dma16_s(kb, lane_bytes + i * inst_bytes, dk + 512 * b);
        dma16_s(vb, lane_bytes + i * inst_bytes, dv + 512 * b);
      }
      return;
    }
    for (int i = 0; i < NI; ++i) {
      const int b = i * nw + wave, s = 64 * b + lane;
      const int r = s / CPR, ch = (s % CPR) ^ chunk_key<CPR>(r);
      const int tok = (s < real && base + r < c1) ? base + r : c0;
      const size_t off = (size_t)tok * D + 8 * ch;
      dma16(K + off, dk + 512 * b);
      dma16(V + off, dv + 512 * b);
    }
  };

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
  // ring prologue after the landmark operand's loads: those few loads then return before
  // the K/V flood of every block (context stage at n = 4096, m = 64: 35.8-35.9 -> 35.2-35.3
  // us on one box, against the ring first)
  for (int t = 0; t < S - 1 && t < nsteps; ++t) issue(t, t);
  f32x16 wacc[FT];
#pragma unroll
  for (int f = 0; f < FT; ++f) wacc[f] = zero16();
  float M = kNegBig, L = 0.f;
  // transposed-read addressing (see lds_tr16): lane 4j + q of each 16-lane group points
  // at token row j, feature column 16*(group & 1) + 4q of the feature tile
  const int trj = (lane & 15) >> 2;
  const int trcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int krow = 32 * tg + r32;

  int cslot = 0, islot = S - 1;  // ring slots of tile t and of tile t + S - 1
  for (int t = 0; t < nsteps; ++t) {
    // tile t is complete once only the DMA of later tiles is outstanding (any other
    // younger load only makes the count conservative)
    wait_dma_barrier(2 * NI * min(nsteps - 1 - t, S - 2));
    if (t + S - 1 < nsteps) issue(t + S - 1, islot);  // refills the slot consumed at t - 1
    islot = islot + 1 == S ? 0 : islot + 1;
    const int base = c0 + t * step;
    const uint16_t* kt = ring + (size_t)cslot * 2 * tile_elems;
    const uint16_t* vt = kt + tile_elems;
    cslot = cslot + 1 == S ? 0 : cslot + 1;

    // scores (log2 units): rows = 32 tokens, columns = 32 landmarks
    f32x16 Sc = zero16();
#pragma unroll
    for (int s = 0; s < KD; ++s) {
      const Pair8 ka{ld8(kt + swz_off<CPR>(krow, 16 * s + 8 * h)), zero8()};
      Sc = mfma_pair<false, true>(ka, qb[s], Sc);
    }
    // online softmax over tokens per landmark; only the chunk's last step can be partial
    const bool partial = base + 32 * tg + 32 > c1;
    float mx = kNegBig;
    if (!partial) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, Sc[rr]);
    } else {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int tok = base + 32 * tg + 8 * (rr >> 2) + 4 * h + (rr & 3);
        if (tok >= c1) Sc[rr] = kNegBig;
        mx = fmaxf(mx, Sc[rr]);
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
      for (int f = 0; f < FT; ++f) scale_in_place(wacc[f], corr);
      M = mn;
    }
    float p[16];
    float ps = 0.f;
    if (!partial) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        p[rr] = fast_exp2(Sc[rr] - M);
        ps += p[rr];
      }
    } else {  // masked tokens contribute exactly 0 (M may still be the -1e30 start value)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        p[rr] = Sc[rr] > 0.5f * kNegBig ? fast_exp2(Sc[rr] - M) : 0.f;
        ps += p[rr];
      }
    }
    L += ps;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const Pair8 pb = split8(&p[8 * s2]);
      const int row = 32 * tg + 16 * s2 + 4 * h + trj;
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        const int col = 32 * f + trcol;
        const Pair8 va{lds_tr16x2(vt + swz_off<CPR>(row, col), vt + swz_off<CPR>(row + 8, col)),
                       zero8()};
        wacc[f] = mfma_pair<false, true>(va, pb, wacc[f]);
      }
    }
  }
  L += __shfl_xor(L, 32);
  __syncthreads();  // ring drained (the last wait was for everything); LDS becomes scratch
  flash_store_partial<D>(a, bh, c, wacc, M, L, reinterpret_cast<float*>(lds));
}

// ------------------------------------------------------------------ context launch
// MP > 0: blocks [0, BH) run the pseudo-inverse of their head (mp = MP), the rest the
// landmark context; MP == 0: context blocks only. NCH applies to fp32 inputs.
// Occupancy target: three 4-wave blocks per CU for bf16 with d <= 64 (their LDS is 48 KiB),
// else two (fused) or one 8-wave block.
template <typename Tin, int D>
constexpr int context_min_blocks(int mp) {
  return mp == 0 ? 1 : (!Input<Tin>::kSplit && D <= 64) ? 3 : 2;
}

template <typename Tin, int D, int MP, int NCH>
__global__ __launch_bounds__(MP > 0 ? 256 : 512, (context_min_blocks<Tin, D>(MP)))
void context_kernel(CtxArgs a) {
  extern __shared__ __align__(16) char lds[];
  int blk = blockIdx.x;
  if constexpr (MP > 0) {
    __shared__ float red_part[2 * MP * (MP / 32)];  // [row][column tile][max, sum]
    __shared__ float red_col[(MP / 32) * MP];   // [row tile][column]
    __shared__ float red[16];
    if (blk < a.npinv) {
      pinv_lds_body<MP, D>(a, blk, reinterpret_cast<uint16_t*>(lds), red_part, red_col, red);
      return;
    }
    blk -= a.npinv;
  }
  if constexpr (Input<Tin>::kSplit) flash_reg_body<Tin, D, NCH>(a, blk, lds);
  else flash_ring_body<D>(a, blk, lds);
}

// ------------------------------------------------------------------ host side
static bool pinv_in_lds(int mp) { return mp <= 64; }

static size_t pinv_lds_bytes(int mp) {
  return pinv_in_lds(mp) ? (size_t)kQPlanes * mp * mp * 2 : 0;
}

void context_ring_geometry(int d, CtxArgs& a) {
  const int nw = a.LG * a.TG, step = 32 * a.TG, chunks = step * (d / 8);
  a.ring_ni = (chunks + 64 * nw - 1) / (64 * nw);
  const size_t stage = (size_t)2 * nw * a.ring_ni * 1024;
  // 48 KiB (the fused pseudo-inverse's planes at m = 64) keeps three blocks per CU
  const size_t budget = std::max<size_t>(48 * 1024, pinv_lds_bytes(a.mp));
  a.ring_stages = (int)std::min<size_t>(4, std::max<size_t>(2, budget / stage));
}

size_t context_lds_bytes(bool bf16, int d, const CtxArgs& a) {
  const int LG = a.LG, TG = a.TG;
  size_t main;
  if (bf16) {
    main = (size_t)a.ring_stages * 2 * (LG * TG) * a.ring_ni * 1024;
  } else {
    main = (size_t)2 * (32 * TG) * (d + 8) * 2;
  }
  const size_t merge = (size_t)LG * (TG - 1) * ((d / 32) * 16 * 64 + 128) * 4;
  const size_t pinv = context_fuses_pinv(a.mp) ? pinv_lds_bytes(a.mp) : 0;
  return std::max({main, merge, pinv});
}

template <int D>
static hipError_t launch_pinv_t(const CtxArgs& a, hipStream_t s) {
  if (a.iters == 0) {  // no iteration: the per-head kernel also hands Z_0 over
    hipLaunchKernelGGL((pinv_global_kernel<D>), dim3(a.BH), dim3(1024), 0, s, a);
    return hipGetLastError();
  }
  const int nt = a.mp / 32;
  hipLaunchKernelGGL(pinv_strip_kernel, dim3(a.BH * nt), dim3(64 * nt), 0, s, a);
  hipError_t e = hipGetLastError();
  const int tiles = (a.mp / 32) * (a.mp / 32);
  const dim3 grid(a.BH * tiles), block(64);
  if (e != hipSuccess) return e;
  switch (a.mp) {
#define NYS_PHASES(MP)                                                                   \
  case MP:                                                                               \
    hipLaunchKernelGGL((pinv_phase_kernel<0, MP / 16>), grid, block, 0, s, a, 0, 0);     \
    for (int it = 0; it < a.iters; ++it) {                                               \
      const bool re = pinv_refresh(it, a.iters), next_re = pinv_refresh(it + 1, a.iters); \
      if (re) {                                                                          \
        hipLaunchKernelGGL((pinv_phase_kernel<1, MP / 16>), grid, block, 0, s, a, it,    \
                           (int)kZOnly);                                                 \
        hipLaunchKernelGGL((pinv_phase_kernel<0, MP / 16>), grid, block, 0, s, a, it,    \
                           (int)kRefresh);                                               \
      }                                                                                  \
      const bool with_z = it > 0 && !re;                                                 \
      hipLaunchKernelGGL((pinv_phase_kernel<1, MP / 16>), dim3(grid.x * (with_z ? 2 : 1)), \
                         block, 0, s, a, it, with_z ? (int)kWithZ : 0);                  \
      const bool more = it + 1 < a.iters && !next_re;                                    \
      hipLaunchKernelGGL((pinv_phase_kernel<2, MP / 16>), grid, block, 0, s, a, it,      \
                         more ? (int)kMore : 0);                                         \
    }                                                                                    \
    hipLaunchKernelGGL((pinv_phase_kernel<3, MP / 16>), grid, block, 0, s, a, a.iters, 0); \
    break;
    NYS_PHASES(96) NYS_PHASES(128) NYS_PHASES(160) NYS_PHASES(192) NYS_PHASES(224)
    NYS_PHASES(256)
#undef NYS_PHASES
    default: return hipErrorInvalidValue;
  }
  if (e == hipSuccess) e = hipGetLastError();
  return e;
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

// Every kernel instance a (dtype, d) pair can launch: MP in {32, 64, 0} for the fused
// pseudo-inverse, NCH for fp32 staging.
template <typename Tin, int D>
static const void* context_fn(int mp, int LG) {
  if constexpr (!Input<Tin>::kSplit) {
    if (mp == 32) return reinterpret_cast<const void*>(&context_kernel<Tin, D, 32, 1>);
    if (mp == 64) return reinterpret_cast<const void*>(&context_kernel<Tin, D, 64, 1>);
    return reinterpret_cast<const void*>(&context_kernel<Tin, D, 0, 1>);
  } else {
#define NYS_NCH(MP)                                                                     \
  switch (flash_nch(D, LG)) {                                                           \
    case 1: return reinterpret_cast<const void*>(&context_kernel<Tin, D, MP, 1>);       \
    case 2: return reinterpret_cast<const void*>(&context_kernel<Tin, D, MP, 2>);       \
    case 4: return reinterpret_cast<const void*>(&context_kernel<Tin, D, MP, 4>);       \
    default: return reinterpret_cast<const void*>(&context_kernel<Tin, D, MP, 8>);      \
  }
    if (mp == 32) { NYS_NCH(32) }
    if (mp == 64) { NYS_NCH(64) }
    NYS_NCH(0)
#undef NYS_NCH
  }
}

static const void* context_fn(bool bf16, int d, int mp, int LG) {
  if (bf16) {
    if (d == 32) return context_fn<uint16_t, 32>(mp, LG);
    if (d == 64) return context_fn<uint16_t, 64>(mp, LG);
    return context_fn<uint16_t, 128>(mp, LG);
  }
  if (d == 32) return context_fn<float, 32>(mp, LG);
  if (d == 64) return context_fn<float, 64>(mp, LG);
  return context_fn<float, 128>(mp, LG);
}

hipError_t launch_context(bool bf16, int d, const CtxArgs& a, hipStream_t s) {
  const void* fn = context_fn(bf16, d, a.mp, a.LG);
  if (64 * a.LG * a.TG > (a.npinv > 0 ? 256 : 512)) return hipErrorInvalidConfiguration;
  const dim3 grid(a.npinv + a.BH * a.C), block(64 * a.LG * a.TG);
  void* args[] = {const_cast<CtxArgs*>(&a)};
  return hipLaunchKernel(fn, grid, block, args, context_lds_bytes(bf16, d, a), s);
}

int context_blocks_per_cu(bool bf16, int d, int mp, size_t ctx_lds) {
  const int LG = mp / 32, TG = context_token_groups(LG);
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, context_fn(bf16, d, mp, LG), 64 * LG * TG,
                                                   ctx_lds) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return nb;
}

hipError_t configure_context(bool bf16, int d, int mp, size_t ctx_lds) {
  const int LG = mp / 32;
  return hipFuncSetAttribute(context_fn(bf16, d, mp, LG),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)ctx_lds);
}

}  // namespace nys
