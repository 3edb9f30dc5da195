// Projections around the Nystrom core (Fastformer review page, "Proposed method": the
// input embeddings become Q, K, V through linear projections per head; the heads'
// outputs are concatenated and projected back to the model width):
//
//   qkv_proj_kernel  [Q | K | V] = X W_qkv^T, X [B n][D], W_qkv [3 H d][D]; the store
//                    splits the 3 H d output features into q, k, v [B][H][n][d]
//   out_proj_kernel  Y = concat_h(O_h) W_o^T, O [B][H][n][d] gathered by the A-tile
//                    loader, W_o [D][H d], Y [B n][D]
//
// Both are C = A B^T with A [M][K] and B [N][K] row-major (k contiguous), bf16 in,
// fp32 accumulate, bf16 out. A block computes a 128 (N) x 128 (M) tile of C^T with 4
// waves (64 x 64 each, 2 x 2 MFMA tiles of v_mfma_f32_32x32x16_bf16), over k-slabs of
// 64. A and B slabs stream through a two-slot LDS ring filled by LDS DMA (one slab in
// flight while the other is multiplied), rows stored with the chunk permutation of
// swz_off so both operand fetches are 16-byte runs without bank conflicts. The C^T
// orientation gives every lane four runs of four consecutive output features of one
// token: 8-byte stores.
#include "nys_common.h"
#include "nys_kernels.h"

namespace nys {

constexpr int kPBM = 128, kPBN = 128, kPBK = 64;  // tile sizes (M, N, K)
constexpr int kPSlab = kPBM * kPBK;               // bf16 elements per A or B slab

// Source of A-row r's 16-byte chunk at k-offset kk (elements) for the two kernels.
struct ARowsQkv {
  const uint16_t* x;
  int M, K;
  __device__ __forceinline__ const uint16_t* at(int m, int kk) const {
    return x + (size_t)m * K + kk;
  }
};
struct ARowsOut {  // row m = token (b, t), column k = head h = k / d, feature k % d
  const uint16_t* o;
  int n, H, d;
  __device__ __forceinline__ const uint16_t* at(int m, int kk) const {
    const int b = m / n, t = m - b * n, h = kk / d, f = kk - h * d;
    return o + (((size_t)b * H + h) * n + t) * d + f;
  }
};

// C^T[n][m] for the block's tile; returns acc[tn][tm] for the wave (rows n = 64 wn +
// 32 tn + 8 (r/4) + 4 (lane/32) + r%4, column m = 64 wm + 32 tm + lane % 32 of the tile).
template <typename ARows>
__device__ __forceinline__ void proj_tile(const ARows& arows, const uint16_t* w, int M, int N,
                                          int K, int m0, int n0, uint16_t* ring,
                                          f32x16 (&acc)[2][2]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, r32 = lane & 31;
  const int wn = wave & 1, wm = wave >> 1;
  const int nslab = K / kPBK;
  // DMA: 1024 chunks per slab = 16 wave instructions; wave w issues slots 64 (4 i + w)
  auto issue = [&](int t) {
    uint16_t* sa = ring + (size_t)(t & 1) * 2 * kPSlab;
    uint16_t* sb = sa + kPSlab;
    const int k0 = t * kPBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int blk = 4 * i + wave, s = 64 * blk + lane;
      const int r = s >> 3, c = (s & 7) ^ chunk_key<8>(r);
      const int m = min(m0 + r, M - 1), nn = min(n0 + r, N - 1);
      dma16(arows.at(m, k0 + 8 * c), sa + 512 * blk);
      dma16(w + (size_t)nn * K + k0 + 8 * c, sb + 512 * blk);
    }
  };
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = zero16();
  issue(0);
  for (int t = 0; t < nslab; ++t) {
    wait_dma_barrier(0);  // slab t is in LDS; every wave is done with slab t - 1
    if (t + 1 < nslab) issue(t + 1);
    const uint16_t* sa = ring + (size_t)(t & 1) * 2 * kPSlab;
    const uint16_t* sb = sa + kPSlab;
#pragma unroll
    for (int s = 0; s < kPBK / 16; ++s) {
      bf16x8 wa[2], xb[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        wa[u] = ld8(sb + swz_off<8>(64 * wn + 32 * u + r32, 16 * s + 8 * h));
        xb[u] = ld8(sa + swz_off<8>(64 * wm + 32 * u + r32, 16 * s + 8 * h));
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma(wa[a], xb[b], acc[a][b]);
    }
  }
}

// Four consecutive features of one token as 8 bytes of bf16 (RNE).
__device__ __forceinline__ u32x2 pack4(const f32x16& v, int g) {
  const bf16x2 p = bf16_rne2(v[4 * g], v[4 * g + 1]);
  const bf16x2 q = bf16_rne2(v[4 * g + 2], v[4 * g + 3]);
  return u32x2{__builtin_bit_cast(uint32_t, p), __builtin_bit_cast(uint32_t, q)};
}

__global__ __launch_bounds__(256, 2) void qkv_proj_kernel(ProjArgs a) {
  extern __shared__ __align__(16) char lds[];
  const int M = a.B * a.n, N = 3 * a.H * a.d, K = a.D;
  int mb, nb;
  xcd_map(blockIdx.x, (M + kPBM - 1) / kPBM, (N + kPBN - 1) / kPBN, mb, nb);
  const int m0 = mb * kPBM, n0 = nb * kPBN;
  f32x16 acc[2][2];
  proj_tile(ARowsQkv{static_cast<const uint16_t*>(a.a), M, K}, static_cast<const uint16_t*>(a.w),
            M, N, K, m0, n0, reinterpret_cast<uint16_t*>(lds), acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5;
  const int wn = wave & 1, wm = wave >> 1;
  const int HD = a.H * a.d;
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) {
    const int m = m0 + 64 * wm + 32 * tm + (lane & 31);
    if (m >= M) continue;
    const int b = m / a.n, t = m - b * a.n;
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nn = n0 + 64 * wn + 32 * tn + 8 * g + 4 * h;  // 4 features, one head
        if (nn >= N) continue;
        const int which = nn / HD, hd = (nn - which * HD) / a.d, f = nn - which * HD - hd * a.d;
        uint16_t* dst = static_cast<uint16_t*>(which == 0 ? a.q : which == 1 ? a.k : a.v) +
                        (((size_t)b * a.H + hd) * a.n + t) * a.d + f;
        *reinterpret_cast<u32x2*>(dst) = pack4(acc[tn][tm], g);
      }
  }
}

__global__ __launch_bounds__(256, 2) void out_proj_kernel(ProjArgs a) {
  extern __shared__ __align__(16) char lds[];
  const int M = a.B * a.n, N = a.D, K = a.H * a.d;
  int mb, nb;
  xcd_map(blockIdx.x, (M + kPBM - 1) / kPBM, (N + kPBN - 1) / kPBN, mb, nb);
  const int m0 = mb * kPBM, n0 = nb * kPBN;
  f32x16 acc[2][2];
  proj_tile(ARowsOut{static_cast<const uint16_t*>(a.a), a.n, a.H, a.d},
            static_cast<const uint16_t*>(a.w), M, N, K, m0, n0,
            reinterpret_cast<uint16_t*>(lds), acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5;
  const int wn = wave & 1, wm = wave >> 1;
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) {
    const int m = m0 + 64 * wm + 32 * tm + (lane & 31);
    if (m >= M) continue;
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nn = n0 + 64 * wn + 32 * tn + 8 * g + 4 * h;
        if (nn >= N) continue;
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.y) + (size_t)m * N + nn) =
            pack4(acc[tn][tm], g);
      }
  }
}

size_t proj_lds_bytes() { return (size_t)2 * 2 * kPSlab * 2; }

hipError_t configure_proj() {
  const int bytes = (int)proj_lds_bytes();
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&qkv_proj_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&out_proj_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t launch_qkv_proj(const ProjArgs& a, hipStream_t s) {
  const int M = a.B * a.n, N = 3 * a.H * a.d;
  const dim3 grid(((M + kPBM - 1) / kPBM) * ((N + kPBN - 1) / kPBN));
  hipLaunchKernelGGL(qkv_proj_kernel, grid, dim3(256), proj_lds_bytes(), s, a);
  return hipGetLastError();
}

hipError_t launch_out_proj(const ProjArgs& a, hipStream_t s) {
  const int M = a.B * a.n, N = a.D;
  const dim3 grid(((M + kPBM - 1) / kPBM) * ((N + kPBN - 1) / kPBN));
  hipLaunchKernelGGL(out_proj_kernel, grid, dim3(256), proj_lds_bytes(), s, a);
  return hipGetLastError();
}

}  // namespace nys
