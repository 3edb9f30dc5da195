// Segment-means landmarks (Nystromformer review page, "Proposed method": landmarks are
// the means of contiguous token segments, an O(n) step).
//
// Segment j of a head with valid length L (n, or the padded batch's length) is rows
// [ceil(j L / m), ceil((j+1) L / m)): token t belongs to segment floor(t m / L).
//
// One wave owns one (matrix in {Q, K}, head, segment j) and streams the segment's
// contiguous rows: lane L reads 16-byte chunk L % CPR of row L / CPR + RPW * it, so each
// load instruction covers RPW whole consecutive rows (1 KiB contiguous), and the loads of
// eight iterations are in flight together. Each lane sums its rows in fp32; lanes that
// share a chunk are then combined with a butterfly over the row bits of the lane index.
//
// Outputs per head: fp32 means [mp][d] (rows m..mp-1 are left untouched; the workspace
// keeps them zero) and the same values as hi/lo bf16 planes [2][mp][d] for the MFMA
// stages.
#include "nys_common.h"
#include "nys_kernels.h"

namespace nys {

// Wave-uniform index arithmetic: the wave index through readfirstlane, so the task split and
// the segment bounds run on scalar registers, in 32 bits (divisions by a runtime value in
// 64 bits on vector registers cost a few hundred instructions before a wave's first load).
// First row of segment j of m over L rows: ceil(j L / m); the 64-bit form only when m n
// reaches 2^32.
__device__ __forceinline__ int seg_first(int j, int L, int m, bool wide) {
  if (wide) return (int)(((long long)j * L + m - 1) / m);
  return (int)(((unsigned)j * (unsigned)L + (unsigned)(m - 1)) / (unsigned)m);
}
__device__ __forceinline__ bool seg_wide(const SegArgs& a) {
  return (unsigned long long)a.m * (unsigned long long)a.n >= (1ull << 32);
}

template <typename Tin, int D>
__global__ __launch_bounds__(256) void segmeans_kernel(const Tin* __restrict__ q,
                                                       const Tin* __restrict__ k,
                                                       SegArgs a) {
  constexpr int EPC = 16 / sizeof(Tin);  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;           // chunks per row
  constexpr int RPW = 64 / CPR;          // rows per wave load
  static_assert(CPR >= 1 && CPR <= 64 && (64 % CPR) == 0, "row must tile a wave");
  const int lane = threadIdx.x & 63;
  const unsigned task = blockIdx.x * 4u + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (task >= 2u * (unsigned)a.BH * (unsigned)a.m) return;  // whole waves only; no barrier
  const int j = (int)(task % (unsigned)a.m);
  const int bh = (int)((task / (unsigned)a.m) % (unsigned)a.BH);
  const int which = (int)(task / ((unsigned)a.m * (unsigned)a.BH));
  const int c = lane % CPR, r0 = lane / CPR;
  const int L = valid_length(a.lengths, bh, a.H, a.n, a.m);
  const bool wide = seg_wide(a);
  const int start = seg_first(j, L, a.m, wide);
  const int rows = seg_first(j + 1, L, a.m, wide) - start;

  const Tin* src = (which ? k : q) + ((size_t)bh * a.n + start) * D + c * EPC;
  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
  const int nit = (rows + RPW - 1) / RPW;
#pragma unroll 8
  for (int it = 0; it < nit; ++it) {
    const int r = r0 + RPW * it;
    float x[8];
    if constexpr (EPC == 8) {
      Input<Tin>::load_raw(src + (size_t)r * D, r < rows, x);
    } else {
      const f32x4 v = r < rows ? *reinterpret_cast<const f32x4*>(src + (size_t)r * D)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = v[e];
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] += x[e];
  }
  // lanes c, c + CPR, c + 2 CPR, ... hold partial sums of the same chunk
#pragma unroll
  for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] += __shfl_xor(acc[e], o);
  if (lane >= CPR) return;

  const float inv_l = 1.0f / (float)rows;
  float mean[8];
#pragma unroll
  for (int e = 0; e < EPC; ++e) mean[e] = acc[e] * inv_l;
  float* dst = (which ? a.kt : a.qt) + ((size_t)bh * a.mp + j) * D + c * EPC;
  uint16_t* hl = (which ? a.kt_hl : a.qt_hl) + (size_t)bh * 2 * a.mp * D + (size_t)j * D + c * EPC;
  *reinterpret_cast<f32x4*>(dst) = f32x4{mean[0], mean[1], mean[2], mean[3]};
  if constexpr (EPC == 8) {
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{mean[4], mean[5], mean[6], mean[7]};
    const Pair8 p = split8(mean);
    st8(hl, p.hi);
    st8(hl + (size_t)a.mp * D, p.lo);
  } else {
    uint16_t hb[4], lb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split1(mean[e], hb[e], lb[e]);
    *reinterpret_cast<u32x2*>(hl) =
        u32x2{(uint32_t)hb[0] | ((uint32_t)hb[1] << 16), (uint32_t)hb[2] | ((uint32_t)hb[3] << 16)};
    *reinterpret_cast<u32x2*>(hl + (size_t)a.mp * D) =
        u32x2{(uint32_t)lb[0] | ((uint32_t)lb[1] << 16), (uint32_t)lb[2] | ((uint32_t)lb[3] << 16)};
  }
}

// Short segments (at most one load instruction's RPW rows each): one wave takes SPW
// consecutive segments of one (matrix, head), so SPW loads are in flight per wave instead
// of one. Requires m % SPW == 0. Two segments per wave measured best (B=32 H=12 n=512
// d=64 m=64: 23 us with one, 16.5 with two, 18.4 with four, 20.6 with eight).
template <typename Tin, int D, int SPW>
__global__ __launch_bounds__(256) void segmeans_short_kernel(const Tin* __restrict__ q,
                                                             const Tin* __restrict__ k,
                                                             SegArgs a) {
  constexpr int EPC = 16 / sizeof(Tin);
  constexpr int CPR = D / EPC;
  static_assert(CPR >= 1 && CPR <= 64 && (64 % CPR) == 0, "row must tile a wave");
  const int lane = threadIdx.x & 63;
  const unsigned groups = (unsigned)(a.m / SPW);
  const unsigned task = blockIdx.x * 4u + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (task >= 2u * (unsigned)a.BH * groups) return;  // whole waves only; no barrier
  const int j0 = (int)(task % groups) * SPW;
  const int bh = (int)((task / groups) % (unsigned)a.BH);
  const int which = (int)(task / (groups * (unsigned)a.BH));
  const int c = lane % CPR, r = lane / CPR;
  const int L = valid_length(a.lengths, bh, a.H, a.n, a.m);
  const bool wide = seg_wide(a);
  const Tin* base = (which ? k : q) + (size_t)bh * a.n * D + c * EPC;
  float x[SPW][8];
  int rows[SPW];
#pragma unroll
  for (int g = 0; g < SPW; ++g) {
    const int j = j0 + g;
    const int start = seg_first(j, L, a.m, wide);
    rows[g] = seg_first(j + 1, L, a.m, wide) - start;
    const Tin* src = base + (size_t)(start + r) * D;
    if constexpr (EPC == 8) {
      Input<Tin>::load_raw(src, r < rows[g], x[g]);
    } else {
      const f32x4 v = r < rows[g] ? *reinterpret_cast<const f32x4*>(src) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) x[g][e] = v[e];
    }
  }
#pragma unroll
  for (int g = 0; g < SPW; ++g) {
#pragma unroll
    for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < EPC; ++e) x[g][e] += __shfl_xor(x[g][e], o);
    if (lane < CPR) {
      const int j = j0 + g;
      const float inv_l = 1.0f / (float)rows[g];
      float mean[8];
#pragma unroll
      for (int e = 0; e < EPC; ++e) mean[e] = x[g][e] * inv_l;
      float* dst = (which ? a.kt : a.qt) + ((size_t)bh * a.mp + j) * D + c * EPC;
      uint16_t* hl =
          (which ? a.kt_hl : a.qt_hl) + (size_t)bh * 2 * a.mp * D + (size_t)j * D + c * EPC;
      *reinterpret_cast<f32x4*>(dst) = f32x4{mean[0], mean[1], mean[2], mean[3]};
      if constexpr (EPC == 8) {
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{mean[4], mean[5], mean[6], mean[7]};
        const Pair8 p = split8(mean);
        st8(hl, p.hi);
        st8(hl + (size_t)a.mp * D, p.lo);
      } else {
        uint16_t hb[4], lb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split1(mean[e], hb[e], lb[e]);
        *reinterpret_cast<u32x2*>(hl) = u32x2{(uint32_t)hb[0] | ((uint32_t)hb[1] << 16),
                                              (uint32_t)hb[2] | ((uint32_t)hb[3] << 16)};
        *reinterpret_cast<u32x2*>(hl + (size_t)a.mp * D) =
            u32x2{(uint32_t)lb[0] | ((uint32_t)lb[1] << 16), (uint32_t)lb[2] | ((uint32_t)lb[3] << 16)};
      }
    }
  }
}

// Long segments (more than 64 rows): one block of WPS (2, 4 or 8) waves per (matrix, head,
// segment).
// Wave w streams rows w, w + WPS, ... in whole-row loads as above (so every wave moves about
// 64 rows, not one wave the whole segment), and the waves' chunk sums are added through LDS.
template <typename Tin, int D, int WPS>
__global__ __launch_bounds__(64 * WPS) void segmeans_split_kernel(const Tin* __restrict__ q,
                                                                  const Tin* __restrict__ k,
                                                                  SegArgs a) {
  constexpr int EPC = 16 / sizeof(Tin), CPR = D / EPC, RPW = 64 / CPR;
  __shared__ float part[WPS][CPR][EPC];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned task = blockIdx.x;  // (matrix, head, segment)
  const int j = (int)(task % (unsigned)a.m);
  const int bh = (int)((task / (unsigned)a.m) % (unsigned)a.BH);
  const int which = (int)(task / ((unsigned)a.m * (unsigned)a.BH));
  const int c = lane % CPR, r0 = lane / CPR;
  const int L = valid_length(a.lengths, bh, a.H, a.n, a.m);
  const bool wide = seg_wide(a);
  const int start = seg_first(j, L, a.m, wide);
  const int rows = seg_first(j + 1, L, a.m, wide) - start;
  const Tin* src = (which ? k : q) + ((size_t)bh * a.n + start) * D + c * EPC;
  float acc[8];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
  const int nit = (rows + RPW * WPS - 1) / (RPW * WPS);
#pragma unroll 8
  for (int it = 0; it < nit; ++it) {
    const int r = r0 + RPW * (wave + WPS * it);
    float x[8];
    if constexpr (EPC == 8) {
      Input<Tin>::load_raw(src + (size_t)r * D, r < rows, x);
    } else {
      const f32x4 v = r < rows ? *reinterpret_cast<const f32x4*>(src + (size_t)r * D)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = v[e];
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] += x[e];
  }
#pragma unroll
  for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] += __shfl_xor(acc[e], o);
  if (lane < CPR)
#pragma unroll
    for (int e = 0; e < EPC; ++e) part[wave][lane][e] = acc[e];
  __syncthreads();
  if (wave != 0 || lane >= CPR) return;
  float mean[8];
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < WPS; ++w) sum += part[w][lane][e];  // fixed order
    mean[e] = sum / (float)rows;
  }
  float* dst = (which ? a.kt : a.qt) + ((size_t)bh * a.mp + j) * D + c * EPC;
  uint16_t* hl = (which ? a.kt_hl : a.qt_hl) + (size_t)bh * 2 * a.mp * D + (size_t)j * D + c * EPC;
  *reinterpret_cast<f32x4*>(dst) = f32x4{mean[0], mean[1], mean[2], mean[3]};
  if constexpr (EPC == 8) {
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{mean[4], mean[5], mean[6], mean[7]};
    const Pair8 p = split8(mean);
    st8(hl, p.hi);
    st8(hl + (size_t)a.mp * D, p.lo);
  } else {
    uint16_t hb[4], lb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split1(mean[e], hb[e], lb[e]);
    *reinterpret_cast<u32x2*>(hl) =
        u32x2{(uint32_t)hb[0] | ((uint32_t)hb[1] << 16), (uint32_t)hb[2] | ((uint32_t)hb[3] << 16)};
    *reinterpret_cast<u32x2*>(hl + (size_t)a.mp * D) =
        u32x2{(uint32_t)lb[0] | ((uint32_t)lb[1] << 16), (uint32_t)lb[2] | ((uint32_t)lb[3] << 16)};
  }
}

template <typename Tin, int D>
static hipError_t launch_segmeans_t(const void* q, const void* k, const SegArgs& a,
                                    hipStream_t s) {
  const int lmax = (a.n + a.m - 1) / a.m;  // longest segment
  if (lmax > 256) {
    hipLaunchKernelGGL((segmeans_split_kernel<Tin, D, 8>), dim3((unsigned)(2LL * a.BH * a.m)),
                       dim3(512), 0, s, static_cast<const Tin*>(q), static_cast<const Tin*>(k), a);
    return hipGetLastError();
  }
  if (lmax > 128) {
    hipLaunchKernelGGL((segmeans_split_kernel<Tin, D, 4>), dim3((unsigned)(2LL * a.BH * a.m)),
                       dim3(256), 0, s, static_cast<const Tin*>(q), static_cast<const Tin*>(k), a);
    return hipGetLastError();
  }
  if (lmax > 64) {
    hipLaunchKernelGGL((segmeans_split_kernel<Tin, D, 2>), dim3((unsigned)(2LL * a.BH * a.m)),
                       dim3(128), 0, s, static_cast<const Tin*>(q), static_cast<const Tin*>(k), a);
    return hipGetLastError();
  }
  constexpr int RPW = 64 / (D / (16 / (int)sizeof(Tin)));  // rows per load instruction
  if (lmax <= RPW && a.m % 2 == 0) {
    const long long waves = 2LL * a.BH * (a.m / 2);  // one per 2 segments
    hipLaunchKernelGGL((segmeans_short_kernel<Tin, D, 2>), dim3((unsigned)((waves + 3) / 4)),
                       dim3(256), 0, s, static_cast<const Tin*>(q), static_cast<const Tin*>(k), a);
    return hipGetLastError();
  }
  const long long waves = 2LL * a.BH * a.m;  // one per (matrix, head, segment)
  const int blocks = (int)((waves + 3) / 4);
  hipLaunchKernelGGL((segmeans_kernel<Tin, D>), dim3(blocks), dim3(256), 0, s,
                     static_cast<const Tin*>(q), static_cast<const Tin*>(k), a);
  return hipGetLastError();
}

// Landmark rows m..mp-1 of head blockIdx.x set to zero: fp32 means of Q and K and both
// hi/lo planes of each (a plan's workspace keeps them zero from its creation; a reused
// scratch buffer does not).
__global__ __launch_bounds__(256) void clear_landmark_padding_kernel(SegArgs a, int d) {
  const size_t bh = blockIdx.x;
  const int per = (a.mp - a.m) * d;
  for (int e = threadIdx.x; e < per; e += blockDim.x) {
    const size_t off = (size_t)a.m * d + e;  // row m + e / d, column e % d
    a.qt[bh * a.mp * d + off] = 0.f;
    a.kt[bh * a.mp * d + off] = 0.f;
    for (int plane = 0; plane < 2; ++plane) {
      const size_t o = (bh * 2 + plane) * a.mp * d + off;
      a.qt_hl[o] = 0;
      a.kt_hl[o] = 0;
    }
  }
}

hipError_t launch_clear_landmark_padding(int d, const SegArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(clear_landmark_padding_kernel, dim3((unsigned)a.BH), dim3(256), 0, s, a, d);
  return hipGetLastError();
}

hipError_t launch_segmeans(bool bf16, int d, const void* q, const void* k, const SegArgs& a,
                           hipStream_t s) {
  if (bf16) {
    if (d == 32) return launch_segmeans_t<uint16_t, 32>(q, k, a, s);
    if (d == 64) return launch_segmeans_t<uint16_t, 64>(q, k, a, s);
    return launch_segmeans_t<uint16_t, 128>(q, k, a, s);
  }
  if (d == 32) return launch_segmeans_t<float, 32>(q, k, a, s);
  if (d == 64) return launch_segmeans_t<float, 64>(q, k, a, s);
  return launch_segmeans_t<float, 128>(q, k, a, s);
}

}  // namespace nys
