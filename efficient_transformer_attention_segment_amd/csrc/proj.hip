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
// fp32 accumulate, bf16 out. A block computes a 256 (N) x 256 (M) tile of C^T; each of
// its 4 waves owns 128 x 128 (4 x 4 tiles of v_mfma_f32_32x32x16_bf16), so a k-step of
// 16 costs 8 operand fetches of 1 KiB per wave for 16 MFMAs. k-slabs of 32 for A and B
// stream through a four-stage LDS ring filled by LDS DMA (three slabs in flight), rows
// stored with the chunk permutation of swz_off so the operand fetches are 16-byte runs
// without bank conflicts. The result tile is staged in LDS as bf16 and written with
// 16-byte stores that fill whole cache lines (the MFMA fragments alone would give 8-byte
// pieces of 32 rows per instruction, which halves the store bandwidth). Rows past M or N
// are clamped on load and skipped on store.
#include "nys_common.h"
#include "nys_kernels.h"

namespace nys {

// Block tile 256 (N) x 256 (M); 4 waves in a 2 x 2 grid, 128 x 128 each (4 x 4 MFMA
// tiles, 256 fp32 accumulators per lane, held in AGPRs). k-slabs of 32 through a ring of
// four stages (32 KiB each: A and B 256 x 32 bf16), so three slabs are in flight while
// one is multiplied. One block per CU (128 KiB of LDS).
constexpr int kPBM = 256, kPBN = 256, kPBK = 32, kPStages = 4;
constexpr int kPSlab = kPBM * kPBK;     // bf16 elements per A (or B) slab
constexpr int kPDmaPerSlab = 8;         // DMA instructions per wave per stage (A + B)

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

using ProjAcc = f32x16[4][4];
// Operand fragments of one slab for one wave: [k-step][W tiles 0-3, X tiles 0-3].
using ProjFrag = bf16x8[kPBK / 16][8];

// All 16 ds_read_b128 of one slab for the wave (issued back to back; the MFMAs that use
// them come later).
__device__ __forceinline__ void proj_read_slab(const uint16_t* sa, const uint16_t* sb, int wn,
                                               int wm, int r32, int h, ProjFrag& f) {
#pragma unroll
  for (int s = 0; s < kPBK / 16; ++s)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f[s][u] = ld8(sb + swz_off<4>(128 * wn + 32 * u + r32, 16 * s + 8 * h));
      f[s][4 + u] = ld8(sa + swz_off<4>(128 * wm + 32 * u + r32, 16 * s + 8 * h));
    }
}

__device__ __forceinline__ void proj_mfma_step(const bf16x8 (&f)[8], ProjAcc& acc) {
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = mfma(f[a], f[4 + b], acc[a][b]);
}

// C^T[n][m] for the block's tile; acc[tn][tm] holds, for the wave, rows n = 128 wn +
// 32 tn + 8 (r/4) + 4 (lane/32) + r%4 and column m = 128 wm + 32 tm + lane % 32.
//
// Schedule of slab t: MFMAs of its first k-step; wait for slab t + 1's DMA and barrier
// (every wave has read slab t into registers by then, so its stage is free); DMA of slab
// t + 4 into that stage; reads of slab t + 1 into the other fragment set; MFMAs of slab
// t's second k-step. Up to three slabs are in flight and the next slab's fragment reads
// overlap the current MFMAs.
template <typename ARows>
__device__ __forceinline__ void proj_tile(const ARows& arows, const uint16_t* w, int M, int N,
                                          int K, int m0, int n0, uint16_t* ring, ProjAcc& acc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, r32 = lane & 31;
  const int wn = wave & 1, wm = wave >> 1;
  const int nslab = K / kPBK;
  // one stage: 2 x 1024 16-byte chunks = 32 wave instructions, 8 per wave; slot s of an
  // operand holds row s / 4, stored chunk s % 4 (logical chunk (s % 4) ^ key(row))
  auto stage = [&](int t) { return ring + (size_t)(t % kPStages) * 2 * kPSlab; };
  auto issue = [&](int t) {
    uint16_t* sa = stage(t);
    uint16_t* sb = sa + kPSlab;
    // blocks start at different k-slabs (by their slot on the XCD) so that concurrent
    // blocks do not all read the same column window of the 2-byte * K row stride
    const int k0 = ((t + (int)(blockIdx.x >> 3)) % nslab) * kPBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int blk = 4 * i + wave, s = 64 * blk + lane;
      const int r = s >> 2, c = (s & 3) ^ chunk_key<4>(r);
      const int m = min(m0 + r, M - 1), nn = min(n0 + r, N - 1);
      dma16(arows.at(m, k0 + 8 * c), sa + 512 * blk);
      dma16(w + (size_t)nn * K + k0 + 8 * c, sb + 512 * blk);
    }
  };
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = zero16();
#pragma unroll
  for (int t = 0; t < kPStages; ++t)
    if (t < nslab) issue(t);
  // slab 0 landed once at most the younger slabs' DMAs are outstanding
  wait_dma_barrier(kPDmaPerSlab * min(nslab - 1, kPStages - 1));
  ProjFrag f0, f1;
  proj_read_slab(stage(0), stage(0) + kPSlab, wn, wm, r32, h, f0);
  for (int t = 0; t < nslab; t += 2) {  // nslab is even (K is a multiple of 64)
    proj_mfma_step(f0[0], acc);
    wait_lds_dma_barrier(kPDmaPerSlab * min(nslab - 2 - t, kPStages - 2));
    if (t + kPStages < nslab) issue(t + kPStages);
    proj_read_slab(stage(t + 1), stage(t + 1) + kPSlab, wn, wm, r32, h, f1);
    proj_mfma_step(f0[1], acc);
    proj_mfma_step(f1[0], acc);
    if (t + 2 < nslab) {
      wait_lds_dma_barrier(kPDmaPerSlab * min(nslab - 3 - t, kPStages - 2));
      if (t + 1 + kPStages < nslab) issue(t + 1 + kPStages);
      proj_read_slab(stage(t + 2), stage(t + 2) + kPSlab, wn, wm, r32, h, f0);
    }
    proj_mfma_step(f1[1], acc);
  }
}

// Epilogue staging: the bf16 C tile as [256 tokens][256 features] in LDS (128 KiB, the
// ring's space once the main loop is done), 16-byte chunk c of token row m stored at chunk
// c ^ (m & 15). The fragment writes (8 bytes, 32 tokens per instruction) and the 16-byte
// row reads then spread over all banks.
__device__ __forceinline__ int stage_off(int m, int chunk) {
  return m * (kPBN / 8) * 16 + ((chunk ^ (m & 15)) << 4);
}

__device__ __forceinline__ void proj_stage_tile(const ProjAcc& acc, char* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5;
  const int wn = wave & 1, wm = wave >> 1;
  __syncthreads();  // every wave is done reading the ring
#pragma unroll
  for (int tm = 0; tm < 4; ++tm) {
    const int m = 128 * wm + 32 * tm + (lane & 31);
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& v = acc[tn][tm];
        const bf16x2 p = bf16_rne2(v[4 * g], v[4 * g + 1]);
        const bf16x2 q = bf16_rne2(v[4 * g + 2], v[4 * g + 3]);
        const int chunk = 16 * wn + 4 * tn + g;  // features 8 chunk .. 8 chunk + 7
        *reinterpret_cast<u32x2*>(lds + stage_off(m, chunk) + 8 * h) =
            u32x2{__builtin_bit_cast(uint32_t, p), __builtin_bit_cast(uint32_t, q)};
      }
  }
  __syncthreads();
}

// Store pass over the staged tile: thread t handles chunk t % 32 of tokens t / 32 + 8 i,
// so each wave instruction writes whole 16-byte chunks of two tokens' feature rows.
template <typename Dst>
__device__ __forceinline__ void proj_store_tile(const char* lds, int m0, int n0, int M, int N,
                                                const Dst& dst) {
  const int chunk = threadIdx.x & 31, r = threadIdx.x >> 5;
  const int nn = n0 + 8 * chunk;
  if (nn >= N) return;
#pragma unroll 4
  for (int i = 0; i < kPBM / 8; ++i) {
    const int m = r + 8 * i;
    if (m0 + m >= M) break;
    const u32x4 v = *reinterpret_cast<const u32x4*>(lds + stage_off(m, chunk));
    *reinterpret_cast<u32x4*>(dst(m0 + m, nn)) = v;
  }
}

struct DstQkv {  // feature nn of token m -> q, k or v [B][H][n][d]
  uint16_t *q, *k, *v;
  int n, H, d, HD;
  __device__ __forceinline__ uint16_t* operator()(int m, int nn) const {
    const int b = m / n, t = m - b * n, which = nn / HD, rem = nn - which * HD;
    const int hd = rem / d, f = rem - hd * d;
    return (which == 0 ? q : which == 1 ? k : v) + (((size_t)b * H + hd) * n + t) * d + f;
  }
};
struct DstRows {  // y [M][N]
  uint16_t* y;
  int N;
  __device__ __forceinline__ uint16_t* operator()(int m, int nn) const {
    return y + (size_t)m * N + nn;
  }
};

__global__ __launch_bounds__(256, 1) void qkv_proj_kernel(ProjArgs a) {
  extern __shared__ __align__(16) char lds[];
  const int M = a.B * a.n, N = 3 * a.H * a.d, K = a.D;
  int mb, nb;
  xcd_map(blockIdx.x, (M + kPBM - 1) / kPBM, (N + kPBN - 1) / kPBN, mb, nb);
  const int m0 = mb * kPBM, n0 = nb * kPBN;
  ProjAcc acc;
  proj_tile(ARowsQkv{static_cast<const uint16_t*>(a.a), M, K}, static_cast<const uint16_t*>(a.w),
            M, N, K, m0, n0, reinterpret_cast<uint16_t*>(lds), acc);
  proj_stage_tile(acc, lds);
  proj_store_tile(lds, m0, n0, M, N,
                  DstQkv{static_cast<uint16_t*>(a.q), static_cast<uint16_t*>(a.k),
                         static_cast<uint16_t*>(a.v), a.n, a.H, a.d, a.H * a.d});
}

__global__ __launch_bounds__(256, 1) void out_proj_kernel(ProjArgs a) {
  extern __shared__ __align__(16) char lds[];
  const int M = a.B * a.n, N = a.D, K = a.H * a.d;
  int mb, nb;
  xcd_map(blockIdx.x, (M + kPBM - 1) / kPBM, (N + kPBN - 1) / kPBN, mb, nb);
  const int m0 = mb * kPBM, n0 = nb * kPBN;
  ProjAcc acc;
  proj_tile(ARowsOut{static_cast<const uint16_t*>(a.a), a.n, a.H, a.d},
            static_cast<const uint16_t*>(a.w), M, N, K, m0, n0,
            reinterpret_cast<uint16_t*>(lds), acc);
  proj_stage_tile(acc, lds);
  proj_store_tile(lds, m0, n0, M, N, DstRows{static_cast<uint16_t*>(a.y), N});
}

size_t proj_lds_bytes() { return (size_t)kPStages * 2 * kPSlab * 2; }

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
