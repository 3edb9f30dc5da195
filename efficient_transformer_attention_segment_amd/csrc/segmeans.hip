// Segment-means landmarks (Nystromformer review page, "Proposed method": landmarks are
// the means of contiguous token segments, an O(n) step).
//
// One thread owns one (matrix in {Q, K}, head, segment j, 8-feature chunk) and sums the
// l = n/m rows of its segment in fp32 with 16-byte loads. Consecutive threads take
// consecutive chunks of a row, so each load instruction of a wave reads whole 128-byte
// row pieces of several segments; there is no cross-thread reduction.
//
// Outputs per head: fp32 means [mp][d] (rows m..mp-1 are left untouched; the workspace
// keeps them zero) and the same values as hi/lo bf16 planes [2][mp][d] for the MFMA
// stages.
#include "nys_common.h"
#include "nys_kernels.h"

namespace nys {

template <typename Tin, int D>
__global__ __launch_bounds__(256) void segmeans_kernel(const Tin* __restrict__ q,
                                                       const Tin* __restrict__ k,
                                                       SegArgs a) {
  constexpr int kChunks = D / 8;
  const long long g = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = 2LL * a.BH * a.m * kChunks;
  if (g >= total) return;
  const int c = (int)(g % kChunks);
  long long rest = g / kChunks;
  const int j = (int)(rest % a.m);
  rest /= a.m;
  const int bh = (int)(rest % a.BH);
  const int which = (int)(rest / a.BH);

  const Tin* src = (which ? k : q) + (size_t)bh * a.n * D + (size_t)j * a.l * D + c * 8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll 8
  for (int r = 0; r < a.l; ++r) {
    float x[8];
    Input<Tin>::load_raw(src + (size_t)r * D, true, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += x[e];
  }
  const float inv_l = 1.0f / (float)a.l;
  float mean[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mean[e] = acc[e] * inv_l;

  float* dst = (which ? a.kt : a.qt) + ((size_t)bh * a.mp + j) * D + c * 8;
  *reinterpret_cast<f32x4*>(dst) = f32x4{mean[0], mean[1], mean[2], mean[3]};
  *reinterpret_cast<f32x4*>(dst + 4) = f32x4{mean[4], mean[5], mean[6], mean[7]};

  Pair8 p = split8(mean);
  uint16_t* hl = (which ? a.kt_hl : a.qt_hl) + (size_t)bh * 2 * a.mp * D + (size_t)j * D + c * 8;
  st8(hl, p.hi);
  st8(hl + (size_t)a.mp * D, p.lo);
}

template <typename Tin, int D>
static hipError_t launch_segmeans_t(const void* q, const void* k, const SegArgs& a,
                                    hipStream_t s) {
  const long long total = 2LL * a.BH * a.m * (D / 8);
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL((segmeans_kernel<Tin, D>), dim3(blocks), dim3(256), 0, s,
                     static_cast<const Tin*>(q), static_cast<const Tin*>(k), a);
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
