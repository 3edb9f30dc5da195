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
// fp32 accumulate, bf16 out. A block computes a 128 (N) x 256 (M) tile of C^T; each of
// its 4 waves owns 64 x 128 (2 x 4 tiles of v_mfma_f32_32x32x16_bf16), so a k-step of
// 16 costs 6 operand fetches of 1 KiB per wave for 8 MFMAs. k-slabs of 32 for A and B
// stream through a three-stage LDS ring filled by LDS DMA, rows stored with the chunk
// permutation of swz_off so the operand fetches are 16-byte runs without bank conflicts.
// Two blocks share a CU (72 KiB of LDS and 128 accumulators per lane each), so one
// block's ring wait and result stores overlap the other's MFMAs. The result tile is staged
// in LDS as bf16 and written with 16-byte stores that fill whole cache lines (the MFMA
// fragments alone would give 8-byte pieces of 32 rows per instruction, which halves the
// store bandwidth). Rows past M or N are clamped on load and skipped on store.
#include "nys_common.h"
#include "nys_kernels.h"

namespace nys {

// Block tile 128 (N) x 256 (M); 4 waves in a 2 x 2 grid, 64 x 128 each (2 x 4 MFMA tiles,
// 128 fp32 accumulators per lane, held in AGPRs). k-slabs of 32 through a ring of three
// stages (24 KiB each: A 256 x 32 and B 128 x 32 bf16). Two blocks per CU.
constexpr int kPBM = 256, kPBN = 128, kPBK = 32, kPStages = 3;
constexpr int kPSlabA = kPBM * kPBK, kPSlabB = kPBN * kPBK;  // bf16 elements per slab
constexpr int kPStage = kPSlabA + kPSlabB;
constexpr int kPDmaPerSlab = 6;  // DMA instructions per wave per stage (4 A + 2 B)

// A-row sources of the two kernels, split for the DMA's saddr form: a wave-uniform base
// per 32-wide k-slab (k0) and a per-lane byte offset of row m, chunk kc (k0 + 8 kc .. +7)
// that is the same for every slab. Byte offsets fit 32 bits (tensors stay below 2^31
// elements).
struct ARowsQkv {  // x [M][K]
  const uint16_t* x;
  int K;
  __device__ __forceinline__ const uint16_t* slab(int k0) const { return x + k0; }
  __device__ __forceinline__ uint32_t lane_bytes(int m, int kc) const {
    return 2u * ((uint32_t)m * (uint32_t)K + 8u * (uint32_t)kc);
  }
};
struct ARowsOut {  // row m = token (b, t), column k = head k / d, feature k % d
  const uint16_t* o;
  int n, H, d;
  // a 32-wide slab lies in one head (d is a multiple of 32): head k0 / d, features from k0 % d
  __device__ __forceinline__ const uint16_t* slab(int k0) const {
    return o + (size_t)(k0 / d) * n * d + (k0 % d);
  }
  __device__ __forceinline__ uint32_t lane_bytes(int m, int kc) const {
    const int b = m / n, t = m - b * n;
    return 2u * ((uint32_t)((b * H * n + t) * d) + 8u * (uint32_t)kc);
  }
};

using ProjAcc = f32x16[2][4];
// Operand fragments of one k-step for one wave: W tiles 0-1, X tiles 0-3.
using ProjFrag = bf16x8[6];

// The six ds_read_b128 of k-step s (0 or 1) of a slab for the wave.
__device__ __forceinline__ void proj_read_step(const uint16_t* sa, const uint16_t* sb, int s,
                                               int wn, int wm, int r32, int h, ProjFrag& f) {
#pragma unroll
  for (int u = 0; u < 2; ++u) f[u] = ld8(sb + swz_off<4>(64 * wn + 32 * u + r32, 16 * s + 8 * h));
#pragma unroll
  for (int u = 0; u < 4; ++u)
    f[2 + u] = ld8(sa + swz_off<4>(128 * wm + 32 * u + r32, 16 * s + 8 * h));
}

__device__ __forceinline__ void proj_mfma_step(const ProjFrag& f, ProjAcc& acc) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = mfma(f[a], f[2 + b], acc[a][b]);
}

// Wait until at most n of this wave's loads are outstanding and its LDS reads have
// returned, then a workgroup barrier (n: 0, 6 or 12).
__device__ __forceinline__ void proj_ring_barrier(int n) {
  switch (n) {
    case 12: asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
  }
}

// C^T[n][m] for the block's tile; acc[tn][tm] holds, for the wave, rows n = 64 wn +
// 32 tn + 8 (r/4) + 4 (lane/32) + r%4 and column m = 128 wm + 32 tm + lane % 32.
//
// Schedule of slab t (fragments of its first k-step already in registers): read its
// second k-step; MFMAs of the first; wait for slab t + 1's DMA and barrier (every wave has
// read slab t by then, so its stage is free); DMA of slab t + 3 into that stage; read the
// first k-step of slab t + 1; MFMAs of slab t's second k-step. Two slabs are in flight
// beyond the one being multiplied, and every fragment read overlaps MFMAs.
template <typename ARows>
__device__ __forceinline__ void proj_tile(const ARows& arows, const uint16_t* w, int M, int N,
                                          int K, int m0, int n0, uint16_t* ring, ProjAcc& acc) {
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, r32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const int nslab = K / kPBK;
  // one stage: A 1024 and B 512 16-byte chunks = 24 wave instructions, 6 per wave; slot s
  // of an operand holds row s / 4, stored chunk s % 4 (logical chunk (s % 4) ^ key(row))
  auto stage = [&](int t) { return ring + (size_t)(t % kPStages) * kPStage; };
  // the lane's six DMA sources as byte offsets from the slab bases (rows clamped at M, N)
  uint32_t aoff[4], boff[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = 64 * (4 * i + wave) + lane, r = s >> 2, c = (s & 3) ^ chunk_key<4>(r);
    aoff[i] = arows.lane_bytes(min(m0 + r, M - 1), c);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int s = 64 * (4 * i + wave) + lane, r = s >> 2, c = (s & 3) ^ chunk_key<4>(r);
    boff[i] = 2u * ((uint32_t)min(n0 + r, N - 1) * (uint32_t)K + 8u * (uint32_t)c);
  }
  auto issue = [&](int t) {
    uint16_t* sa = stage(t);
    uint16_t* sb = sa + kPSlabA;
    // blocks start at different k-slabs (by their slot on the XCD) so that concurrent
    // blocks do not all read the same column window of the 2-byte * K row stride
    const int k0 = ((t + (int)(blockIdx.x >> 3)) % nslab) * kPBK;
    const uint16_t* abase = arows.slab(k0);
    const uint16_t* bbase = w + k0;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16_s(abase, aoff[i], sa + 512 * (4 * i + wave));
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16_s(bbase, boff[i], sb + 512 * (4 * i + wave));
  };
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = zero16();
#pragma unroll
  for (int t = 0; t < kPStages; ++t)
    if (t < nslab) issue(t);
  // slab 0 landed once at most the younger slabs' DMAs are outstanding
  proj_ring_barrier(kPDmaPerSlab * min(nslab - 1, kPStages - 1));
  ProjFrag fa, fb;
  proj_read_step(stage(0), stage(0) + kPSlabA, 0, wn, wm, r32, h, fa);
  for (int t = 0; t < nslab; ++t) {
    proj_read_step(stage(t), stage(t) + kPSlabA, 1, wn, wm, r32, h, fb);
    proj_mfma_step(fa, acc);
    if (t + 1 < nslab) {
      proj_ring_barrier(kPDmaPerSlab * min(nslab - 2 - t, kPStages - 2));
      if (t + kPStages < nslab) issue(t + kPStages);
      proj_read_step(stage(t + 1), stage(t + 1) + kPSlabA, 0, wn, wm, r32, h, fa);
    }
    proj_mfma_step(fb, acc);
  }
}

// Epilogue staging: the bf16 C tile as [256 tokens][128 features] in LDS (64 KiB, the
// ring's space once the main loop is done), 16-byte chunk c of token row m stored at chunk
// c ^ (m & 15). The fragment writes (8 bytes, 32 tokens per instruction) and the 16-byte
// row reads then spread over all banks.
__device__ __forceinline__ int stage_off(int m, int chunk) {
  return m * (kPBN / 8) * 16 + ((chunk ^ (m & 15)) << 4);
}

__device__ __forceinline__ void proj_stage_tile(const ProjAcc& acc, char* lds) {
  const int lane = threadIdx.x & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  __syncthreads();  // every wave is done reading the ring
#pragma unroll
  for (int tm = 0; tm < 4; ++tm) {
    const int m = 128 * wm + 32 * tm + (lane & 31);
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& v = acc[tn][tm];
        const bf16x2 p = bf16_rne2(v[4 * g], v[4 * g + 1]);
        const bf16x2 q = bf16_rne2(v[4 * g + 2], v[4 * g + 3]);
        const int chunk = 8 * wn + 4 * tn + g;  // features 8 chunk .. 8 chunk + 7
        *reinterpret_cast<u32x2*>(lds + stage_off(m, chunk) + 8 * h) =
            u32x2{__builtin_bit_cast(uint32_t, p), __builtin_bit_cast(uint32_t, q)};
      }
  }
  __syncthreads();
}

// Store pass over the staged tile: thread t handles chunk t % 16 of tokens t / 16 + 16 i,
// so each wave instruction writes whole 16-byte chunks of four tokens' feature rows.
template <typename Dst>
__device__ __forceinline__ void proj_store_tile(const char* lds, int m0, int n0, int M, int N,
                                                const Dst& dst) {
  const int chunk = threadIdx.x & 15, r = threadIdx.x >> 4;
  const int nn = n0 + 8 * chunk;
  if (nn >= N) return;
  const int rows = min(kPBM, M - m0);
  if (dst.linear(m0, rows)) {  // rows m0 + r + 16 i sit at a fixed stride: one address
    uint16_t* p = dst(m0 + r, nn);
    const size_t step = (size_t)16 * dst.row_stride();
#pragma unroll 4
    for (int i = 0; i < kPBM / 16; ++i) {
      if (r + 16 * i >= rows) break;
      const u32x4 v = *reinterpret_cast<const u32x4*>(lds + stage_off(r + 16 * i, chunk));
      *reinterpret_cast<u32x4*>(p + i * step) = v;
    }
    return;
  }
#pragma unroll 4
  for (int i = 0; i < kPBM / 16; ++i) {
    const int m = r + 16 * i;
    if (m >= rows) break;
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
  // tokens m0 .. m0 + rows - 1 of one batch element: consecutive rows d apart
  __device__ __forceinline__ bool linear(int m0, int rows) const {
    return m0 / n == (m0 + rows - 1) / n;
  }
  __device__ __forceinline__ int row_stride() const { return d; }
};
struct DstRows {  // y [M][N]
  uint16_t* y;
  int N;
  __device__ __forceinline__ uint16_t* operator()(int m, int nn) const {
    return y + (size_t)m * N + nn;
  }
  __device__ __forceinline__ bool linear(int, int) const { return true; }
  __device__ __forceinline__ int row_stride() const { return N; }
};

__global__ __launch_bounds__(256, 2) void qkv_proj_kernel(ProjArgs a) {
  extern __shared__ __align__(16) char lds[];
  const int M = a.B * a.n, N = 3 * a.H * a.d, K = a.D;
  int mb, nb;
  xcd_map(blockIdx.x, (M + kPBM - 1) / kPBM, (N + kPBN - 1) / kPBN, mb, nb);
  const int m0 = mb * kPBM, n0 = nb * kPBN;
  ProjAcc acc;
  proj_tile(ARowsQkv{static_cast<const uint16_t*>(a.a), K}, static_cast<const uint16_t*>(a.w),
            M, N, K, m0, n0, reinterpret_cast<uint16_t*>(lds), acc);
  proj_stage_tile(acc, lds);
  proj_store_tile(lds, m0, n0, M, N,
                  DstQkv{static_cast<uint16_t*>(a.q), static_cast<uint16_t*>(a.k),
                         static_cast<uint16_t*>(a.v), a.n, a.H, a.d, a.H * a.d});
}

__global__ __launch_bounds__(256, 2) void out_proj_kernel(ProjArgs a) {
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

size_t proj_lds_bytes() {
  static_assert((size_t)kPBM * kPBN * 2 <= (size_t)kPStages * kPStage * 2, "staging fits the ring");
  return (size_t)kPStages * kPStage * 2;
}

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
