// Device helpers shared by the Nystrom attention kernels. CDNA4 (gfx950) only.
//
// Matrix products use the wave64 MFMA v_mfma_f32_32x32x16_bf16 (fp32 accumulate).
// Operand layout of that instruction, as used throughout:
//   A (32 x 16): lane l holds row (l % 32), k-slots (l / 32, e) for e = 0..7
//   B (16 x 32): lane l holds column (l % 32), k-slots (l / 32, e)
//   C (32 x 32): lane l, register r holds row 8*(r/4) + 4*(l/32) + (r%4), column l % 32
// A and B map k-slot (l/32, e) to the same k, so any consistent assignment of logical k
// indices to the slots of both operands gives the same contraction. The kernels use that
// freedom to feed an accumulator straight back in as an operand (see kslot_perm).
//
// Values that need more than bf16's 8-bit mantissa are carried as a bf16 pair
// hi = bf16(x), lo = bf16(x - hi) (about 17 significant bits); a product of two such
// values is formed as hi*hi + hi*lo + lo*hi with fp32 accumulation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nys {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

struct Pair8 {  // an MFMA operand as a hi/lo bf16 pair
  bf16x8 hi, lo;
};

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// c += a * b for hi/lo pairs; kA / kB say whether a / b carry a nonzero lo part.
template <bool kA, bool kB>
__device__ __forceinline__ f32x16 mfma_pair(const Pair8& a, const Pair8& b, f32x16 c) {
  if constexpr (kA) c = mfma(a.lo, b.hi, c);
  if constexpr (kB) c = mfma(a.hi, b.lo, c);
  return mfma(a.hi, b.hi, c);
}

// v *= s with every element scaled in its own register: a plain multiply inside a
// rarely taken branch lets the register allocator place the scaled accumulator elsewhere
// and copy it back on every loop iteration. The compiler's hazard checks do not look
// inside asm, so the wait states are explicit. The leading s_nop reads v[0] and s, so the
// MFMA that wrote v and the v_exp that produced s both come before it: it covers the
// MFMA-result and transcendental-result read hazards. The trailing one reads v[15], the
// last element scaled, so the next MFMA that accumulates into v comes after it: it covers
// the VALU-write to MFMA-read hazard. (Tying the whole vector instead brings the copies
// back.)
__device__ __forceinline__ void scale_in_place(f32x16& v, float s) {
  asm volatile("s_nop 15" : "+v"(v[0]), "+v"(s));
#pragma unroll
  for (int i = 0; i < 16; ++i) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(v[i]) : "v"(s));
  asm volatile("s_nop 4" : "+v"(v[15]));
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 zero8() {
  return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Round-to-nearest-even fp32 -> bf16 (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ __bf16 bf16_rne(float x) { return (__bf16)x; }

// Two values per conversion instruction (v_cvt_pk_bf16_f32 takes a pair).
__device__ __forceinline__ bf16x2 bf16_rne2(float a, float b) {
  return __builtin_convertvector(f32x2{a, b}, bf16x2);
}

__device__ __forceinline__ Pair8 split8(const float* x) {
  Pair8 p;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const bf16x2 h = bf16_rne2(x[e], x[e + 1]);
    const f32x2 hf = __builtin_convertvector(h, f32x2);
    const bf16x2 l = bf16_rne2(x[e] - hf[0], x[e + 1] - hf[1]);
    p.hi[e] = h[0];
    p.hi[e + 1] = h[1];
    p.lo[e] = l[0];
    p.lo[e + 1] = l[1];
  }
  return p;
}

__device__ __forceinline__ void split1(float x, uint16_t& hi, uint16_t& lo) {
  __bf16 h = bf16_rne(x);
  __bf16 l = bf16_rne(x - (float)h);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, l);
}

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void st8(uint16_t* p, const bf16x8& v) {
  *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(u32x4, v);
}

// LDS transpose read (ds_read_b64_tr_b16). Within each 16-lane group, lane k = 4j + q
// supplies the address of four consecutive 16-bit elements; result lane 4q + c receives
// element c of the lanes 4*0+q, 4*1+q, 4*2+q, 4*3+q, i.e. with lane 4j + q pointing at
// row T + j, column F(q) of a row-major tile, lane 4q + c gets rows T..T+3 of column
// F(q) + c: four consecutive k values of one operand row.
typedef __attribute__((ext_vector_type(4))) short s16x4;
__device__ __forceinline__ u32x2 lds_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uint16_t*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Eight k values as two transposed reads (k 0..3 from p0, k 4..7 from p1).
__device__ __forceinline__ bf16x8 lds_tr16x2(const uint16_t* p0, const uint16_t* p1) {
  const u32x2 a = lds_tr16(p0), b = lds_tr16(p1);
  return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

// Eight consecutive input elements as an MFMA operand. bf16 inputs are exact in the hi
// part; fp32 inputs are split into hi/lo. Out-of-range rows read as zero.
template <typename Tin>
struct Input;

template <>
struct Input<uint16_t> {
  static constexpr bool kSplit = false;
  __device__ __forceinline__ static Pair8 load8(const uint16_t* p, bool valid) {
    Pair8 r;
    r.hi = valid ? ld8(p) : zero8();
    r.lo = zero8();
    return r;
  }
  __device__ __forceinline__ static void load_raw(const uint16_t* p, bool valid, float* out8) {
    u32x4 u = valid ? *reinterpret_cast<const u32x4*>(p) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out8[2 * i] = __uint_as_float(u[i] << 16);
      out8[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
};

template <>
struct Input<float> {
  static constexpr bool kSplit = true;
  __device__ __forceinline__ static Pair8 load8(const float* p, bool valid) {
    float x[8];
    load_raw(p, valid, x);
    return split8(x);
  }
  __device__ __forceinline__ static void load_raw(const float* p, bool valid, float* out8) {
    f32x4 a = valid ? *reinterpret_cast<const f32x4*>(p) : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 b = valid ? *reinterpret_cast<const f32x4*>(p + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out8[i] = a[i];
      out8[4 + i] = b[i];
    }
  }
};

// Staging of eight consecutive input elements into a row-major bf16 LDS tile (fp32
// inputs are split into a hi tile and a lo tile).
template <typename Tin>
struct Chunk;

template <>
struct Chunk<uint16_t> {
  u32x4 v;
  __device__ __forceinline__ void load(const uint16_t* p, bool valid) {
    v = valid ? *reinterpret_cast<const u32x4*>(p) : u32x4{0u, 0u, 0u, 0u};
  }
  __device__ __forceinline__ void store(uint16_t* hi, uint16_t* /*lo*/) const {
    *reinterpret_cast<u32x4*>(hi) = v;
  }
};

template <>
struct Chunk<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p, bool valid) {
    a = valid ? *reinterpret_cast<const f32x4*>(p) : f32x4{0.f, 0.f, 0.f, 0.f};
    b = valid ? *reinterpret_cast<const f32x4*>(p + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void store(uint16_t* hi, uint16_t* lo) const {
    float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    const Pair8 p = split8(x);
    st8(hi, p.hi);
    st8(lo, p.lo);
  }
};

// 32 consecutive rows of a row-major bf16 [n][D] matrix, staged into LDS by one wave in two
// phases: load() issues every load, each from a row clamped into [0, end) (end >= 1), and
// store() writes them, zeros for rows at or past end. A load under a condition compiles
// into a branch that the compiler closes with a wait for everything in flight, so staging
// rows one conditional load at a time costs a memory round trip per load.
template <int D>
struct Rows32 {
  static constexpr int NL = D / 16;  // 16-byte chunks per lane
  u32x4 v[NL];
  __device__ __forceinline__ void load(const uint16_t* src, int t0, int end, int lane) {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int idx = lane + 64 * u, i = idx / (D / 8), f8 = (idx % (D / 8)) * 8;
      const int t = t0 + i < end ? t0 + i : end - 1;
      v[u] = *reinterpret_cast<const u32x4*>(src + (size_t)t * D + f8);
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst, int ldr, int t0, int end, int lane) {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int idx = lane + 64 * u, i = idx / (D / 8), f8 = (idx % (D / 8)) * 8;
      asm volatile("" : "+v"(v[u]));  // the select stays here, not next to the load
      const u32x4 x = t0 + i < end ? v[u] : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(dst + (size_t)i * ldr + f8) = x;
    }
  }
};

// Position of logical index t inside a 16-wide k-step when an accumulator's rows are
// reused as the k dimension of the next product. Accumulator register r of lane half h
// holds row 8*(r/4) + 4*h + (r%4); read as eight k-slots per half for one 16-row step,
// slot (h, e) then carries row 8*(e/4) + 4*h + (e%4). Storing the other operand with
// rows permuted by this map (swap bits 2 and 3 of the index) lines both up.
__device__ __forceinline__ int kslot_perm(int t) {
  return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane moves within 16-lane rows (VALU, no LDS round trip).
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xb1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4e;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;  // rotate right by 4 within the row
constexpr int kDppRowRor8 = 0x128;  // rotate right by 8 within the row

// Max / sum over the 32 lanes of a half-wave (lanes 0-31 or 32-63): four DPP steps
// reduce each 16-lane row, one exchange combines the two rows.
__device__ __forceinline__ float half_max(float x) {
  x = fmaxf(x, dpp_mov<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_mov<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_mov<kDppRowRor4>(x));
  x = fmaxf(x, dpp_mov<kDppRowRor8>(x));
  return fmaxf(x, __shfl_xor(x, 16));
}

__device__ __forceinline__ float half_sum(float x) {
  x += dpp_mov<kDppQuadXor1>(x);
  x += dpp_mov<kDppQuadXor2>(x);
  x += dpp_mov<kDppRowRor4>(x);
  x += dpp_mov<kDppRowRor8>(x);
  return x + __shfl_xor(x, 16);
}

// Row broadcasts (gfx9 DPP): lane 15 of each row into the next row, lane 31 into rows 2
// and 3; the row mask picks the rows written, the others keep `old`.
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_bcast(float old, float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), kCtrl, kRowMask, 0xf, false));
}

// Sum over the 32 lanes of a half-wave with DPP steps only, valid in the half's upper
// row: lanes 16-31 hold the sum of lanes 0-31, lanes 48-63 that of lanes 32-63.
__device__ __forceinline__ float half_sum_upper(float x) {
  x += dpp_mov<kDppQuadXor1>(x);
  x += dpp_mov<kDppQuadXor2>(x);
  x += dpp_mov<kDppRowRor4>(x);
  x += dpp_mov<kDppRowRor8>(x);
  return x + dpp_bcast<kDppRowBcast15, 0xa>(0.f, x);
}

// Max over all 64 lanes, in every lane: DPP row reductions, two row broadcasts that
// leave the maximum in lane 63, and a read of that lane.
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = fmaxf(x, dpp_mov<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_mov<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_mov<kDppRowRor4>(x));
  x = fmaxf(x, dpp_mov<kDppRowRor8>(x));
  x = fmaxf(x, dpp_bcast<kDppRowBcast15, 0xa>(x, x));
  x = fmaxf(x, dpp_bcast<kDppRowBcast31, 0xc>(x, x));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// x[l] combined with x[l ^ 32] (the other half-wave) through v_permlane32_swap, the same
// value in both lanes of a pair: the swap leaves (x[l], x[l ^ 32]) in every lane, in an
// order that depends on the half, and both combinations are symmetric.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------- LDS-DMA staging
// global_load_lds_dwordx4: every lane moves 16 bytes from its own global address to LDS
// at (M0 base) + 16 * lane, so one wave instruction fills 1 KiB of LDS contiguously and
// any permutation of 16-byte chunks is free on the global side. Issued through inline
// asm: the caller tracks completion itself with wait_dma_barrier. dst_lds must be
// wave-uniform.
__device__ __forceinline__ void dma16(const void* src, void* dst_lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst_lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0)
               : "memory", "m0");
}

// Same DMA with a wave-uniform base in SGPRs and a 32-bit per-lane byte offset: no 64-bit
// address arithmetic per lane. sbase must be wave-uniform.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, void* dst_lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst_lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(m0)
               : "memory", "m0");
}

// Wait until at most n vector-memory loads of this wave are outstanding, then a
// workgroup barrier. Loads complete in issue order, so when the n youngest loads are
// the DMA of later tiles, every older tile is in LDS; after the barrier that holds for
// every wave's share. No compiler fence is involved: the "memory" clobber keeps LDS
// accesses on their side of it. n is wave-uniform and at most 32.
template <int N>
__device__ __forceinline__ void wait_vm_barrier_n() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_dma_barrier(int n) {
  switch (n) {
#define NYS_WAIT_CASE(N) case N: wait_vm_barrier_n<N>(); break;
    NYS_WAIT_CASE(1) NYS_WAIT_CASE(2) NYS_WAIT_CASE(3) NYS_WAIT_CASE(4) NYS_WAIT_CASE(5)
    NYS_WAIT_CASE(6) NYS_WAIT_CASE(7) NYS_WAIT_CASE(8) NYS_WAIT_CASE(10) NYS_WAIT_CASE(12)
    NYS_WAIT_CASE(14) NYS_WAIT_CASE(16) NYS_WAIT_CASE(20) NYS_WAIT_CASE(24) NYS_WAIT_CASE(28)
    NYS_WAIT_CASE(32)
#undef NYS_WAIT_CASE
    default: wait_vm_barrier_n<0>(); break;  // any other count: wait for everything
  }
}

// As wait_dma_barrier, and also wait for this wave's outstanding LDS reads first, so
// that after the barrier no wave still reads the stage a following DMA may overwrite.
// n is 0, 8, 16 or 24.
template <int N>
__device__ __forceinline__ void wait_vm_lds_barrier_n() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds_dma_barrier(int n) {
  switch (n) {
    case 8: wait_vm_lds_barrier_n<8>(); break;
    case 16: wait_vm_lds_barrier_n<16>(); break;
    case 24: wait_vm_lds_barrier_n<24>(); break;
    default: wait_vm_lds_barrier_n<0>(); break;
  }
}

// 16-byte chunk permutation of row-major bf16 tiles with cpr chunks per row (4, 8 or
// 16): chunk c of row r is stored at chunk c ^ chunk_key(r). With it, eight consecutive
// rows read at one chunk (16-byte operand fetches) hit eight distinct 16-byte bank
// groups, and four consecutive rows read at one aligned 32-byte column pair (transposed
// reads) hit four distinct 32-byte bank groups.
template <int CPR>
__device__ __forceinline__ int chunk_key(int r) {
  static_assert(CPR == 4 || CPR == 8 || CPR == 16, "chunks per row");
  if constexpr (CPR == 4) return 2 * ((r >> 1) & 1) + ((r >> 2) & 1);
  else return 2 * (r & 3) + ((r >> 2) & 1);
}

// Element offset of (r, c) in a permuted row-major tile of CPR chunks per row.
template <int CPR>
__device__ __forceinline__ int swz_off(int r, int c) {
  return r * (8 * CPR) + (((c >> 3) ^ chunk_key<CPR>(r)) << 3) + (c & 7);
}

// Map a linear block index to (head, part) so that all parts of one head run on the
// same XCD (blocks are dispatched round-robin over the 8 XCDs) and share its L2.
__device__ __forceinline__ void xcd_map(int b, int heads, int parts, int& head, int& part) {
  if ((heads & 7) == 0) {
    const int x = b & 7, slot = b >> 3;
    head = x + 8 * (slot / parts);
    part = slot % parts;
  } else {
    head = b / parts;
    part = b % parts;
  }
}

// ---------------------------------------------------------------- 32x32 tile helpers
// acc(32x32) = A[row0:+32, 0:K] * B[0:K, col0:+32] with A given as row-major hi/lo
// planes (leading dimension lda) and B given through its transpose, i.e. planes holding
// B^T row-major (ldb), so both operands are read as 16-byte runs along k.
__device__ __forceinline__ f32x16 gemm_tile(const uint16_t* ahi, const uint16_t* alo, int lda,
                                            const uint16_t* bhi, const uint16_t* blo, int ldb,
                                            int row0, int col0, int K, int lane) {
  const int r = lane & 31, h = lane >> 5;
  const size_t oa = (size_t)(row0 + r) * lda + 8 * h;
  const size_t ob = (size_t)(col0 + r) * ldb + 8 * h;
  f32x16 acc = zero16();
#pragma unroll 8
  for (int k0 = 0; k0 < K; k0 += 16) {
    Pair8 a{ld8(ahi + oa + k0), ld8(alo + oa + k0)};
    Pair8 b{ld8(bhi + ob + k0), ld8(blo + ob + k0)};
    acc = mfma_pair<true, true>(a, b, acc);
  }
  return acc;
}

// Same product with a compile-time number of 16-wide k-steps: every operand load is
// issued before the first MFMA, so one memory latency covers the whole tile.
template <int KSTEPS>
__device__ __forceinline__ f32x16 gemm_tile_k(const uint16_t* ahi, const uint16_t* alo, int lda,
                                              const uint16_t* bhi, const uint16_t* blo, int ldb,
                                              int row0, int col0, int lane) {
  const int r = lane & 31, h = lane >> 5;
  const size_t oa = (size_t)(row0 + r) * lda + 8 * h;
  const size_t ob = (size_t)(col0 + r) * ldb + 8 * h;
  Pair8 a[KSTEPS], b[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    a[s] = Pair8{ld8(ahi + oa + 16 * s), ld8(alo + oa + 16 * s)};
    b[s] = Pair8{ld8(bhi + ob + 16 * s), ld8(blo + ob + 16 * s)};
  }
  // keep the scheduler from sinking loads next to their MFMAs (it would to save registers,
  // and each group of loads would then cost a memory latency of its own)
  __builtin_amdgcn_sched_barrier(0);
  f32x16 acc = zero16();
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) acc = mfma_pair<true, true>(a[s], b[s], acc);
  return acc;
}

// Software-pipelined tile products with a compile-time depth of KS 16-wide k-steps: the
// operands of the next PF k-steps are in flight while the current one is multiplied, so a
// deep product costs about one memory latency instead of one per k-step (a loop over a
// runtime depth waits for every k-step's loads before its MFMAs). A and B^T as row-major
// hi/lo planes (lda, ldb), as in gemm_tile.
template <int KS, int PF = 4>
__device__ __forceinline__ f32x16 gemm_tile_p(const uint16_t* ahi, const uint16_t* alo, int lda,
                                              const uint16_t* bhi, const uint16_t* blo, int ldb,
                                              int row0, int col0, int lane) {
  constexpr int R = PF < KS ? PF : KS;
  const int r = lane & 31, h = lane >> 5;
  const size_t oa = (size_t)(row0 + r) * lda + 8 * h;
  const size_t ob = (size_t)(col0 + r) * ldb + 8 * h;
  Pair8 a[R], b[R];
#pragma unroll
  for (int s = 0; s < R; ++s) {
    a[s] = Pair8{ld8(ahi + oa + 16 * s), ld8(alo + oa + 16 * s)};
    b[s] = Pair8{ld8(bhi + ob + 16 * s), ld8(blo + ob + 16 * s)};
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x16 acc = zero16();
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    acc = mfma_pair<true, true>(a[s % R], b[s % R], acc);
    if (s + R < KS) {
      a[s % R] = Pair8{ld8(ahi + oa + 16 * (s + R)), ld8(alo + oa + 16 * (s + R))};
      b[s % R] = Pair8{ld8(bhi + ob + 16 * (s + R)), ld8(blo + ob + 16 * (s + R))};
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the refill ahead of the next k-steps
  }
  return acc;
}

// gemm_tile with a runtime depth K (a multiple of 32, at most 256), dispatched to the
// pipelined product of that depth.
__device__ __forceinline__ f32x16 gemm_tile_rt(const uint16_t* ahi, const uint16_t* alo, int lda,
                                               const uint16_t* bhi, const uint16_t* blo, int ldb,
                                               int row0, int col0, int K, int lane) {
  switch (K >> 4) {
#define NYS_GT_CASE(N) \
    case N: return gemm_tile_p<N>(ahi, alo, lda, bhi, blo, ldb, row0, col0, lane);
    NYS_GT_CASE(2) NYS_GT_CASE(4) NYS_GT_CASE(6) NYS_GT_CASE(8) NYS_GT_CASE(10)
    NYS_GT_CASE(12) NYS_GT_CASE(14)
#undef NYS_GT_CASE
    default: return gemm_tile_p<16>(ahi, alo, lda, bhi, blo, ldb, row0, col0, lane);
  }
}

// Element (i, j) held by register rr of an accumulator tile at (row0, col0).
__device__ __forceinline__ int acc_row(int row0, int rr, int lane) {
  return row0 + 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
}

__device__ __forceinline__ void store_rows_hl(uint16_t* hi, uint16_t* lo, int ld, int row0,
                                              int col0, const f32x16& v, int lane) {
  const int j = col0 + (lane & 31);
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    uint16_t a, b;
    split1(v[rr], a, b);
    const size_t o = (size_t)acc_row(row0, rr, lane) * ld + j;
    hi[o] = a;
    lo[o] = b;
  }
}

// Store the transpose: element (i, j) goes to [j][i]; rows come in runs of four.
__device__ __forceinline__ void store_cols_hl(uint16_t* hi, uint16_t* lo, int ld, int row0,
                                              int col0, const f32x16& v, int lane) {
  const int j = col0 + (lane & 31);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint16_t a[4], b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split1(v[4 * g + e], a[e], b[e]);
    const size_t o = (size_t)j * ld + row0 + 8 * g + 4 * (lane >> 5);
    *reinterpret_cast<u32x2*>(hi + o) =
        u32x2{(uint32_t)a[0] | ((uint32_t)a[1] << 16), (uint32_t)a[2] | ((uint32_t)a[3] << 16)};
    *reinterpret_cast<u32x2*>(lo + o) =
        u32x2{(uint32_t)b[0] | ((uint32_t)b[1] << 16), (uint32_t)b[2] | ((uint32_t)b[3] << 16)};
  }
}

// Fragment-major operand planes (ld x ld, ld a multiple of 32). Element (r, c) sits in
// the 1 KiB block of row block r / 32 and k-step c / 16, at the slot of the lane that
// takes it as an MFMA operand (lane r % 32 + 32 ((c % 16) / 8), element c % 8). One
// operand load of a k-step then reads a whole contiguous block: eight full 128-byte
// lines instead of 32-byte pieces of 32 lines.
__device__ __forceinline__ size_t frag_off(int r, int c, int ld) {
  return ((size_t)(r >> 5) * (ld >> 4) + (c >> 4)) * 512 + ((r & 31) + 32 * ((c >> 3) & 1)) * 8 +
         (c & 7);
}

// C = A B^T tile at (row0, col0) with A and B^T both in fragment-major planes of depth
// 16 KS, software-pipelined like gemm_tile_p (PF k-steps of operands in flight).
template <int KS, int PF = 4>
__device__ __forceinline__ f32x16 gemm_tile_frag(const uint16_t* ahi, const uint16_t* alo,
                                                 const uint16_t* bhi, const uint16_t* blo,
                                                 int row0, int col0, int lane) {
  constexpr int R = PF < KS ? PF : KS;
  const size_t oa = (size_t)(row0 >> 5) * KS * 512 + 8 * lane;
  const size_t ob = (size_t)(col0 >> 5) * KS * 512 + 8 * lane;
  Pair8 a[R], b[R];
#pragma unroll
  for (int s = 0; s < R; ++s) {
    a[s] = Pair8{ld8(ahi + oa + 512 * s), ld8(alo + oa + 512 * s)};
    b[s] = Pair8{ld8(bhi + ob + 512 * s), ld8(blo + ob + 512 * s)};
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x16 acc = zero16();
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    acc = mfma_pair<true, true>(a[s % R], b[s % R], acc);
    if (s + R < KS) {
      a[s % R] = Pair8{ld8(ahi + oa + 512 * (s + R)), ld8(alo + oa + 512 * (s + R))};
      b[s % R] = Pair8{ld8(bhi + ob + 512 * (s + R)), ld8(blo + ob + 512 * (s + R))};
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the refill ahead of the next k-steps
  }
  return acc;
}

// Two tiles at (row0, col0) that share the right operand: C1 = A1 B^T and C2 = A2 B^T, each
// B fragment loaded once for both products (pipelined like gemm_tile_frag).
template <int KS, int PF = 4>
__device__ __forceinline__ void gemm_tile_frag2(const uint16_t* a1hi, const uint16_t* a1lo,
                                                const uint16_t* a2hi, const uint16_t* a2lo,
                                                const uint16_t* bhi, const uint16_t* blo,
                                                int row0, int col0, int lane, f32x16& c1,
                                                f32x16& c2) {
  constexpr int R = PF < KS ? PF : KS;
  const size_t oa = (size_t)(row0 >> 5) * KS * 512 + 8 * lane;
  const size_t ob = (size_t)(col0 >> 5) * KS * 512 + 8 * lane;
  Pair8 x[R], y[R], b[R];
#pragma unroll
  for (int s = 0; s < R; ++s) {
    x[s] = Pair8{ld8(a1hi + oa + 512 * s), ld8(a1lo + oa + 512 * s)};
    y[s] = Pair8{ld8(a2hi + oa + 512 * s), ld8(a2lo + oa + 512 * s)};
    b[s] = Pair8{ld8(bhi + ob + 512 * s), ld8(blo + ob + 512 * s)};
  }
  __builtin_amdgcn_sched_barrier(0);
  c1 = zero16();
  c2 = zero16();
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    c1 = mfma_pair<true, true>(x[s % R], b[s % R], c1);
    c2 = mfma_pair<true, true>(y[s % R], b[s % R], c2);
    if (s + R < KS) {
      x[s % R] = Pair8{ld8(a1hi + oa + 512 * (s + R)), ld8(a1lo + oa + 512 * (s + R))};
      y[s % R] = Pair8{ld8(a2hi + oa + 512 * (s + R)), ld8(a2lo + oa + 512 * (s + R))};
      b[s % R] = Pair8{ld8(bhi + ob + 512 * (s + R)), ld8(blo + ob + 512 * (s + R))};
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// store_rows_hl / store_cols_hl into fragment-major planes of width ld.
__device__ __forceinline__ void store_rows_hl_frag(uint16_t* hi, uint16_t* lo, int ld, int row0,
                                                   int col0, const f32x16& v, int lane) {
  const int j = col0 + (lane & 31);
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    uint16_t a, b;
    split1(v[rr], a, b);
    const size_t o = frag_off(acc_row(row0, rr, lane), j, ld);
    hi[o] = a;
    lo[o] = b;
  }
}

__device__ __forceinline__ void store_cols_hl_frag(uint16_t* hi, uint16_t* lo, int ld, int row0,
                                                   int col0, const f32x16& v, int lane) {
  const int j = col0 + (lane & 31);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint16_t a[4], b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split1(v[4 * g + e], a[e], b[e]);
    // columns row0 + 8g + 4h .. +3 of row j: four consecutive slots of one lane's chunk
    const size_t o = frag_off(j, row0 + 8 * g + 4 * (lane >> 5), ld);
    *reinterpret_cast<u32x2*>(hi + o) =
        u32x2{(uint32_t)a[0] | ((uint32_t)a[1] << 16), (uint32_t)a[2] | ((uint32_t)a[3] << 16)};
    *reinterpret_cast<u32x2*>(lo + o) =
        u32x2{(uint32_t)b[0] | ((uint32_t)b[1] << 16), (uint32_t)b[2] | ((uint32_t)b[3] << 16)};
  }
}

// ---------------------------------------------------------------- staged tile stores
// A wave's 32x32 accumulator tile parked in LDS (fp32, [32][33]: the pad keeps column reads
// conflict-free), so that its stores leave as 16-byte runs: 8 consecutive k values of one
// fragment-major row or column (two bf16 planes), or 4 consecutive columns of a row-major
// fp32 matrix, instead of one 2- or 4-byte store per element. The caller's wave owns `st`
// (32 * 33 floats) and separates successive uses of it with a wave barrier.
constexpr int kStageLd = 33;

__device__ __forceinline__ void stage_tile(float* st, const f32x16& v, int lane) {
  const int c = lane & 31;
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) st[acc_row(0, rr, lane) * kStageLd + c] = v[rr];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the tile is in LDS for every lane
}

// Rows (transpose = false) or columns (true) of the staged tile at (row0, col0) into the
// fragment-major hi/lo planes of width ld (frag_off): per 16-wide k-step one 16-byte run
// per lane and plane.
template <bool kCols>
__device__ __forceinline__ void stage_store_frag(uint16_t* hi, uint16_t* lo, int ld, int row0,
                                                 int col0, const float* st, int lane) {
  const int r = lane & 31, half = lane >> 5;
#pragma unroll
  for (int s = 0; s < 2; ++s) {  // the two k-steps the 32-wide tile spans
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = 16 * s + 8 * half + e;
      x[e] = kCols ? st[k * kStageLd + r] : st[r * kStageLd + k];
    }
    const Pair8 p = split8(x);
    // row (col0 + r, k from row0) for columns, (row0 + r, k from col0) for rows
    const size_t o = kCols ? frag_off(col0 + r, row0 + 16 * s + 8 * half, ld)
                           : frag_off(row0 + r, col0 + 16 * s + 8 * half, ld);
    st8(hi + o, p.hi);
    st8(lo + o, p.lo);
  }
}

// The staged tile into a row-major fp32 matrix (ld) or row-major hi/lo bf16 planes:
// 16-byte runs of 4 (fp32) or 8 (bf16) consecutive columns.
__device__ __forceinline__ void stage_store_f32(float* p, int ld, int row0, int col0,
                                                const float* st, int lane) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = 8 * it + (lane >> 3), c4 = 4 * (lane & 7);
    const float* q = st + row * kStageLd + c4;
    *reinterpret_cast<f32x4*>(p + (size_t)(row0 + row) * ld + col0 + c4) =
        f32x4{q[0], q[1], q[2], q[3]};
  }
}

__device__ __forceinline__ void stage_store_rows_hl(uint16_t* hi, uint16_t* lo, int ld, int row0,
                                                    int col0, const float* st, int lane) {
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int row = 16 * it + (lane >> 2), c8 = 8 * (lane & 3);
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = st[row * kStageLd + c8 + e];
    const Pair8 pr = split8(x);
    const size_t o = (size_t)(row0 + row) * ld + col0 + c8;
    st8(hi + o, pr.hi);
    st8(lo + o, pr.lo);
  }
}

__device__ __forceinline__ void store_rows_f32(float* p, int ld, int row0, int col0,
                                               const f32x16& v, int lane) {
  const int j = col0 + (lane & 31);
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) p[(size_t)acc_row(row0, rr, lane) * ld + j] = v[rr];
}

}  // namespace nys
