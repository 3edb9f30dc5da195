// FLASH mixed-chunk attention (review page "Transformer Quality in Linear Time",
// "Proposed method", third bullet): the sequence is cut into non-overlapping chunks of
// c tokens; inside a chunk, softmax attention (quadratic in c); across chunks, a linear
// attention with identity features, averaged over the keys it covers; the two summed.
// Per (batch, head), s = 1/sqrt(d), chunk g = tokens [g c, min((g+1) c, n)):
//
//   out[t] = softmax_{t' in chunk(t), t' <= t if causal}(s Q_t . K_t') V_t'
//          + s Q_t M_g / n_g,   M_g = sum over covered chunks of S_j,  S_j = K_j^T V_j
//
// covered = every chunk (non-causal) or the chunks before g (causal; n_g = g c, and
// chunk 0 has no global term).
//
//   flash_state_kernel   one block per (head, chunk): S_g^T = V_g^T K_g (d x d, fp32) on
//                        MFMA, the chunk staged row-major in LDS and read transposed
//   flash_scan_kernel    one block per head: the global sums, scaled by s / n_g and
//                        stored as hi/lo bf16 planes of M^T (one per head, or one per
//                        chunk when causal)
//   flash_attend_kernel  one block per (head, chunk), one wave per 32 queries: local
//                        attention with an online softmax over 32-key tiles (scores on
//                        MFMA with queries across lanes and keys in registers, P kept in
//                        registers as hi/lo bf16, V row-major in LDS read transposed),
//                        then + Q M_g, bf16 store
#include "nys_common.h"
#include "nys_kernels.h"

namespace nys {

__device__ __forceinline__ int fl_row(int rr, int h) { return 8 * (rr >> 2) + 4 * h + (rr & 3); }

// Eight k values (rows k .. k + 7 of a row-major bf16 tile with row stride ld) of column
// col0 + lane % 32, as an MFMA operand: LDS transpose reads, lane 4j + q of each 16-lane
// group addressing row k + j, column col0 + 16 (group & 1) + 4q.
__device__ __forceinline__ bf16x8 fl_tr8(const uint16_t* tile, int ld, int k, int col0, int lane) {
  const int trj = (lane & 15) >> 2, trc = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  return lds_tr16x2(tile + (k + trj) * ld + trc, tile + (k + 4 + trj) * ld + trc);
}

// Rows [t0, t0 + C) of NM row-major bf16 [n][D] matrices into LDS (row strides ld[]),
// zeros at and past t1 (> t0). Each thread's loads go out in batches of kB, every load of
// a batch in flight before its first LDS write, from rows clamped below t1: a load under a
// condition compiles into a branch that the compiler closes with a wait for everything in
// flight, so the rows would arrive one memory round trip at a time.
template <int D, int C, int NTH, int NM>
__device__ __forceinline__ void stage_chunk_rows(const uint16_t* const (&src)[NM],
                                                 uint16_t* const (&dst)[NM], const int (&ld)[NM],
                                                 int t0, int t1) {
  constexpr int TOT = C * (D / 8), PER = (TOT + NTH - 1) / NTH, kB = 4;
#pragma unroll
  for (int u0 = 0; u0 < PER; u0 += kB) {
    u32x4 x[kB][NM];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int e0 = threadIdx.x + NTH * (u0 + u), e = e0 < TOT ? e0 : 0;
      const int i = e / (D / 8), f8 = (e % (D / 8)) * 8, t = min(t0 + i, t1 - 1);
#pragma unroll
      for (int mt = 0; mt < NM; ++mt)
        x[u][mt] = *reinterpret_cast<const u32x4*>(src[mt] + (size_t)t * D + f8);
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int e = threadIdx.x + NTH * (u0 + u);
      const int i = e / (D / 8), f8 = (e % (D / 8)) * 8;
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) {
        asm volatile("" : "+v"(x[u][mt]));  // the select stays here, not next to the load
        if (u0 + u < PER && e < TOT)
          *reinterpret_cast<u32x4*>(dst[mt] + i * ld[mt] + f8) =
              t0 + i < t1 ? x[u][mt] : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
}

// ------------------------------------------------------------------ chunk states
// S_g^T = V_g^T K_g: the chunk's K and V rows are staged row-major (16-byte writes) and
// both operands, which contract over tokens, come from LDS transpose reads.
template <int D, int C>
__global__ __launch_bounds__(256) void flash_state_kernel(FlashArgs a) {
  extern __shared__ __align__(16) char lds[];
  uint16_t* kS = reinterpret_cast<uint16_t*>(lds);  // K [C][D]
  uint16_t* vS = kS + C * D;                          // V [C][D]
  int bh, g;
  xcd_map(blockIdx.x, a.BH, a.G, bh, g);
  const int t0 = g * C, t1 = min(t0 + C, a.n);
  const uint16_t* k = a.k + (size_t)bh * a.n * D;
  const uint16_t* v = a.v + (size_t)bh * a.n * D;
  stage_chunk_rows<D, C, 256, 2>({k, v}, {kS, vS}, {D, D}, t0, t1);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5;
  constexpr int FT = D / 32;
  float* st = a.states + ((size_t)bh * a.G + g) * D * D;
  for (int tile = wave; tile < FT * FT; tile += 4) {
    const int ti = tile / FT, tj = tile % FT;
    f32x16 acc = zero16();
#pragma unroll 4
    for (int k0 = 0; k0 < C; k0 += 16) {
      const int kk = k0 + 8 * h;
      acc = mfma(fl_tr8(vS, D, kk, 32 * ti, lane), fl_tr8(kS, D, kk, 32 * tj, lane), acc);
    }
    store_rows_f32(st, D, 32 * ti, 32 * tj, acc, lane);
  }
}

// ------------------------------------------------------------------ global sums
template <int D>
__global__ __launch_bounds__(256) void flash_scan_kernel(FlashArgs a) {
  const int bh = blockIdx.x;
  const float* st = a.states + (size_t)bh * a.G * D * D;
  constexpr int PER = D * D / 256;
  float run[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) run[u] = 0.f;
  if (!a.causal) {
    for (int g = 0; g < a.G; ++g)
#pragma unroll
      for (int u = 0; u < PER; ++u) run[u] += st[(size_t)g * D * D + threadIdx.x + 256 * u];
  }
  const int nplanes = a.causal ? a.G : 1;
  for (int g = 0; g < nplanes; ++g) {
    const int ncov = a.causal ? g * a.chunk : a.n;
    const float sc = ncov > 0 ? a.scale / (float)ncov : 0.f;
    uint16_t* pl = a.mplanes + ((size_t)bh * nplanes + g) * 2 * D * D;
#pragma unroll
    for (int u = 0; u < PER; ++u) {  // run holds M^T row-major (the states are S_g^T)
      const int e = threadIdx.x + 256 * u;
      uint16_t hi, lo;
      split1(run[u] * sc, hi, lo);
      pl[e] = hi;
      pl[D * D + e] = lo;
    }
    if (a.causal)
#pragma unroll
      for (int u = 0; u < PER; ++u) run[u] += st[(size_t)g * D * D + threadIdx.x + 256 * u];
  }
}

// ------------------------------------------------------------------ local + global
// One wave per 32 queries, in the transposed orientation: S^T = K Q^T puts each query on
// a lane and its keys in the accumulator registers (key 8 (r/4) + 4 h + r % 4 of the
// tile in register r of lane half h), so the online max and sum need one exchange with
// the other half per tile. P stays in registers and is the B operand of
// O^T += V^T P^T directly: for k-step s, registers 8 s .. 8 s + 7 hold keys
// 16 s + 4 h + (0..3) and 16 s + 8 + 4 h + (0..3), so the A operand reads V^T in that key
// order -- two 4-row transpose reads of the row-major V tile at rows 16 s + 4 h and
// 16 s + 8 + 4 h.
// K rows go through LDS too when the block then still fits twice per CU (80 KiB);
// otherwise every wave reads its keys from L2.
template <int D, int C>
struct FlashAttendLds {
  static constexpr int LK = D + 8;  // padded K rows: 16-byte reads of 8 rows spread banks
  static constexpr bool k_in_lds = (size_t)C * D * 2 + (size_t)C * LK * 2 <= 80 * 1024;
  static constexpr size_t bytes = (size_t)C * D * 2 + (k_in_lds ? (size_t)C * LK * 2 : 0);
};

template <int D, int C>
__global__ __launch_bounds__(2 * C) void flash_attend_kernel(FlashArgs a) {
  constexpr int FT = D / 32, LK = FlashAttendLds<D, C>::LK;
  constexpr bool kKL = FlashAttendLds<D, C>::k_in_lds;
  extern __shared__ __align__(16) char lds[];
  uint16_t* vS = reinterpret_cast<uint16_t*>(lds);   // V [C][D] (row-major)
  uint16_t* kS = vS + C * D;                          // K [C][LK] when kKL
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, r32 = lane & 31;
  int bh, g;
  xcd_map(blockIdx.x, a.BH, a.G, bh, g);
  const int t0 = g * C, t1 = min(t0 + C, a.n);
  const uint16_t* q = a.q + (size_t)bh * a.n * D;
  const uint16_t* k = a.k + (size_t)bh * a.n * D;
  const uint16_t* v = a.v + (size_t)bh * a.n * D;
  if constexpr (kKL) stage_chunk_rows<D, C, 2 * C, 2>({v, k}, {vS, kS}, {D, LK}, t0, t1);
  else stage_chunk_rows<D, C, 2 * C, 1>({v}, {vS}, {D}, t0, t1);
  __syncthreads();
  const int q0 = t0 + 32 * wave;  // this wave's first query
  if (q0 >= t1) return;           // no barrier follows
  const int qi = q0 + r32;        // the lane's query
  const int qrow = min(qi, t1 - 1);
  bf16x8 qb[D / 16];              // B operand: query qrow, features 16 s + 8 h ..
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qb[s] = ld8(q + (size_t)qrow * D + 16 * s + 8 * h);
  f32x16 o[FT];                   // O^T: features 32 f + row, this lane's query
#pragma unroll
  for (int f = 0; f < FT; ++f) o[f] = zero16();
  float mrow = kNegBig, lrow = 0.f;
  const float sl = a.scale_log2e;
  const int trj = (lane & 15) >> 2, trc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int ntile = a.causal ? wave + 1 : (t1 - t0 + 31) / 32;
  for (int kt = 0; kt < ntile; ++kt) {
    const int k0 = t0 + 32 * kt;
    const uint16_t* krow = kKL ? kS + (32 * kt + r32) * LK           // A operand: key rows
                               : k + (size_t)min(k0 + r32, t1 - 1) * D;
    f32x16 sc = zero16();
#pragma unroll
    for (int s = 0; s < D / 16; ++s) sc = mfma(ld8(krow + 16 * s + 8 * h), qb[s], sc);
    // no key past the chunk's end and, causal, none after any of the wave's queries: no
    // masks (the scale is positive, so the maximum is taken on the raw scores)
    const bool full = k0 + 32 <= t1 && (!a.causal || k0 + 31 <= q0);
    float mx = kNegBig;
    if (full) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, sc[rr]);
    } else {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int key = k0 + fl_row(rr, h);
        if (!(key < t1 && (!a.causal || key <= qi))) sc[rr] = kNegBig;
        mx = fmaxf(mx, sc[rr]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    mx = mx > 0.5f * kNegBig ? mx * sl : kNegBig;
    // lazy rescaling: the reference maximum moves only when some lane's maximum passes it
    // by more than 8 (log2 units; probabilities stay <= 256); exact for any reference
    if (__any(mx > mrow + 8.f)) {
      const float mn = fmaxf(mrow, mx), corr = fast_exp2(mrow - mn);
      lrow *= corr;
#pragma unroll
      for (int f = 0; f < FT; ++f) scale_in_place(o[f], corr);
      mrow = mn;
    }
    float ps = 0.f, pe[16];
    if (full) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        pe[rr] = fast_exp2(fmaf(sc[rr], sl, -mrow));
        ps += pe[rr];
      }
    } else {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        pe[rr] = sc[rr] > 0.5f * kNegBig ? fast_exp2(fmaf(sc[rr], sl, -mrow)) : 0.f;
        ps += pe[rr];
      }
    }
    Pair8 pb[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) pb[s2] = split8(pe + 8 * s2);
    ps += __shfl_xor(ps, 32);
    lrow += ps;
#pragma unroll
    for (int f = 0; f < FT; ++f) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const uint16_t* base = vS + 32 * f + trc;
        const int r0 = 32 * kt + 16 * s2 + 4 * h + trj;
        const bf16x8 va = lds_tr16x2(base + r0 * D, base + (r0 + 8) * D);
        o[f] = mfma_pair<false, true>(Pair8{va, zero8()}, pb[s2], o[f]);
      }
    }
  }
  // + (M^T Q^T) from the planes (already scaled by s / n_g), then the bf16 store
  const uint16_t* pl = a.mplanes + ((size_t)bh * (a.causal ? a.G : 1) + (a.causal ? g : 0)) *
                                       2 * D * D;
  uint16_t* out = a.out + (size_t)bh * a.n * D;
  const float inv = 1.f / lrow;
#pragma unroll
  for (int f = 0; f < FT; ++f) {
    f32x16 gl = zero16();
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const uint16_t* row = pl + (size_t)(32 * f + r32) * D + 16 * s + 8 * h;
      gl = mfma_pair<true, false>(Pair8{ld8(row), ld8(row + D * D)}, Pair8{qb[s], zero8()}, gl);
    }
    if (qi < t1) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = o[f][4 * g4 + e] * inv + gl[4 * g4 + e];
        const bf16x2 lo2 = bf16_rne2(x[0], x[1]), hi2 = bf16_rne2(x[2], x[3]);
        *reinterpret_cast<u32x2*>(out + (size_t)qi * D + 32 * f + 8 * g4 + 4 * h) =
            u32x2{__builtin_bit_cast(uint32_t, lo2), __builtin_bit_cast(uint32_t, hi2)};
      }
    }
  }
}

// ------------------------------------------------------------------ host side
template <int D, int C>
struct FlashShape {
  static constexpr size_t state_lds = (size_t)2 * C * D * 2;
  static constexpr size_t attend_lds = FlashAttendLds<D, C>::bytes;
};

template <int D, int C>
static hipError_t flash_cfg_t() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&flash_state_kernel<D, C>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)FlashShape<D, C>::state_lds);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&flash_attend_kernel<D, C>),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)FlashShape<D, C>::attend_lds);
}

hipError_t configure_flash() {
  hipError_t e = hipSuccess;
#define NYS_FLASH_CFG(D, C) \
  if ((e = flash_cfg_t<D, C>()) != hipSuccess) return e;
  NYS_FLASH_CFG(32, 64) NYS_FLASH_CFG(32, 128) NYS_FLASH_CFG(32, 256)
  NYS_FLASH_CFG(64, 64) NYS_FLASH_CFG(64, 128) NYS_FLASH_CFG(64, 256)
  NYS_FLASH_CFG(128, 64) NYS_FLASH_CFG(128, 128) NYS_FLASH_CFG(128, 256)
#undef NYS_FLASH_CFG
  return e;
}

template <int D, int C>
static hipError_t flash_states_t(const FlashArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((flash_state_kernel<D, C>), dim3(a.BH * a.G), dim3(256),
                     (FlashShape<D, C>::state_lds), s, a);
  hipLaunchKernelGGL((flash_scan_kernel<D>), dim3(a.BH), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, int C>
static hipError_t flash_attend_t(const FlashArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((flash_attend_kernel<D, C>), dim3(a.BH * a.G), dim3(2 * C),
                     (FlashShape<D, C>::attend_lds), s, a);
  return hipGetLastError();
}

template <template <int, int> class Op>
static hipError_t flash_dispatch(const FlashArgs& a, hipStream_t s) {
  switch (a.d * 1000 + a.chunk) {
    case 32064: return Op<32, 64>::run(a, s);
    case 32128: return Op<32, 128>::run(a, s);
    case 32256: return Op<32, 256>::run(a, s);
    case 64064: return Op<64, 64>::run(a, s);
    case 64128: return Op<64, 128>::run(a, s);
    case 64256: return Op<64, 256>::run(a, s);
    case 128064: return Op<128, 64>::run(a, s);
    case 128128: return Op<128, 128>::run(a, s);
    case 128256: return Op<128, 256>::run(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int C>
struct FlashStatesOp {
  static hipError_t run(const FlashArgs& a, hipStream_t s) { return flash_states_t<D, C>(a, s); }
};
template <int D, int C>
struct FlashAttendOp {
  static hipError_t run(const FlashArgs& a, hipStream_t s) { return flash_attend_t<D, C>(a, s); }
};

hipError_t launch_flash_states(const FlashArgs& a, hipStream_t s) {
  return flash_dispatch<FlashStatesOp>(a, s);
}
hipError_t launch_flash_attend(const FlashArgs& a, hipStream_t s) {
  return flash_dispatch<FlashAttendOp>(a, s);
}

}  // namespace nys
