// Stage 3 of the forward pass (Nystromformer review page, "Proposed method": the output
// is the Nystrom form applied to V, plus a skip connection through a depthwise
// convolution of V):
//
//   out[t] = softmax_j(s q_t . kt_j) Y[j]  +  sum_k w[h][k] V[t + k - (W-1)/2]
//
// Prologue of every block (4 waves, one head): merge the C partial states of the
// landmark context (per landmark, weights exp2(M_c - M*) / sum_c exp2(M_c - M*) L_c,
// fixed chunk order) into W^T in LDS, form Y = Z W on MFMA and keep Y^T (hi/lo bf16,
// landmark index permuted to match the score registers) in LDS; stage Kt (hi/lo, with
// s*log2(e) folded in) and the conv filter's MFMA operand in LDS.
//
// The block then walks a contiguous token range of its head in steps of 128 tokens;
// each wave owns 32 tokens per step. Per wave and step:
//  * scores S^T = Kt Q^T (landmarks x tokens) on MFMA, Q read straight into the B
//    operand;
//  * softmax over the landmarks. Each lane holds one token, so the normaliser is
//    lane-local plus one exchange with the partner half-wave. With at most two landmark
//    tiles (NT = 1, 2) all scores stay in registers: max, exponentials, sum, then the
//    probabilities scaled by 1/sum feed the product directly (no accumulator
//    rescaling). Larger m runs an online softmax over landmark tiles (NT = 0);
//  * O^T += Y^T P^T on MFMA, P fed straight from the score registers (hi/lo bf16);
//  * the convolution as a banded product O^T += V_ext^T T^T on MFMA, with the filter
//    expanded per lane into the B operand once per block; V is staged row-major in LDS
//    with its halo (16-byte writes) and read feature-major with LDS transpose reads;
//    the next step's V rows and Q are loaded into registers while this step computes;
//  * bf16 (RNE) or fp32 store: each lane writes d/2 contiguous features of its token.
#include "nys_common.h"
#include "nys_kernels.h"

namespace nys {

// Feature carried by A-operand row i of output feature tile f: chosen so that a lane's
// 16 accumulator registers of tile f are 16 consecutive features.
template <int D>
__device__ __forceinline__ int out_feature(int f, int i) {
  return (D / 2) * ((i >> 2) & 1) + 16 * f + 4 * (i >> 3) + (i & 3);
}

// Landmark index held by score register rr of landmark tile lt.
__device__ __forceinline__ int score_landmark(int lt, int rr, int h) {
  return 32 * lt + 8 * (rr >> 2) + 4 * h + (rr & 3);
}

// NT: landmark tiles handled with all scores in registers (1 or 2), or 0 for the
// online softmax over a runtime number of tiles. kFull: m == 32 * NT (no masking).
template <typename Tin, int D, int KS, bool kKtLds, int NT, bool kFull>
__global__ __launch_bounds__(256) void output_kernel(OutArgs a) {
  extern __shared__ __align__(16) char lds[];
  constexpr bool kS = Input<Tin>::kSplit;
  constexpr int KD = D / 16, FT = D / 32;
  constexpr int EXT = 96 + 16 * KS;  // staged V rows per 128-token step (with halo)
  constexpr int VR = D + 8;          // LDS row stride (elements) of the row-major V tile
  constexpr int KR = D + 8;          // LDS row stride of the Kt planes
  constexpr int NCH = (EXT * (D / 8) + 255) / 256;  // 8-element V chunks per thread
  static_assert(NT == 0 || kKtLds, "register-resident softmax expects Kt in LDS");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, h = lane >> 5;
  const int mp = NT > 0 ? 32 * NT : a.mp;
  const int YS = mp + 8;
  int bh, grp;
  xcd_map(blockIdx.x, a.BH, a.G, bh, grp);
  const int head = bh % a.H;
  const int t_begin = grp * a.tok_per_block;
  const int t_end = min(a.n, t_begin + a.tok_per_block);
  // scores in log2 units: folded into Kt when it is staged (NT > 0), else applied here
  const float score_scale = NT > 0 ? 1.f : a.scale_log2e;

  uint16_t* yl = reinterpret_cast<uint16_t*>(lds);     // [2][D][YS]  Y^T hi, lo
  uint16_t* wl = yl + (size_t)2 * D * YS;              // [KS][2][64][8] conv B operand
  // region used first by the prologue (W^T planes, chunk weights), then by the main
  // loop (Kt planes when kKtLds, V rows)
  uint16_t* un = wl + (size_t)KS * 2 * 64 * 8;
  uint16_t* wtl = un;                                  // [2][D][YS]  W^T hi, lo
  float* wgt = reinterpret_cast<float*>(un + (size_t)2 * D * YS);  // [C][mp]
  uint16_t* kl = un;                                   // [2][mp][KR] Kt hi, lo
  uint16_t* vt = kl + (kKtLds ? (size_t)2 * mp * KR : 0);  // [EXT][VR] V rows (hi)
  uint16_t* vt_lo = vt + (size_t)EXT * VR;             // V rows lo (fp32 input only)
  const bool taps = grp == 0;

  {
    // chunk weights per landmark
    const int C = a.C;
    const float* pml = a.part_ml + (size_t)bh * C * 2 * mp;
    for (int j = tid; j < mp; j += 256) {
      if (j >= a.m) {
        for (int c = 0; c < C; ++c) wgt[c * mp + j] = 0.f;
        continue;
      }
      float ms = kNegBig;
      for (int c0 = 0; c0 < C; c0 += 8) {
        float mv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) mv[u] = (c0 + u < C) ? pml[(size_t)(2 * (c0 + u)) * mp + j] : kNegBig;
#pragma unroll
        for (int u = 0; u < 8; ++u) ms = fmaxf(ms, mv[u]);
      }
      float den = 0.f;
      for (int c0 = 0; c0 < C; c0 += 8) {
        float ev[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const bool ok = c0 + u < C;
          ev[u] = ok ? fast_exp2(pml[(size_t)(2 * (c0 + u)) * mp + j] - ms) : 0.f;
          if (ok) wgt[(c0 + u) * mp + j] = ev[u];
          den += ev[u] * (ok ? pml[(size_t)(2 * (c0 + u) + 1) * mp + j] : 0.f);
        }
      }
      const float inv = 1.f / den;
      for (int c = 0; c < C; ++c) wgt[c * mp + j] *= inv;
    }
    // conv filter as the B operand of the banded product (identical for every wave)
    if (tid < 64) {
      const float* w = a.conv_w + (size_t)head * a.W;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = 16 * s + 8 * h + e - r32;
          x[e] = (k >= 0 && k < a.W) ? w[k] : 0.f;
        }
        const Pair8 p = split8(x);
        st8(wl + ((size_t)(2 * s) * 64 + lane) * 8, p.hi);
        st8(wl + ((size_t)(2 * s + 1) * 64 + lane) * 8, p.lo);
      }
    }
    __syncthreads();
    // W^T[f][j] = sum_c wgt[c][j] * partial_c^T[f][j], four landmarks per thread
    const float* pw = a.part_w + (size_t)bh * C * D * mp;
    for (int e = tid; e < D * mp / 4; e += 256) {
      const int f = e / (mp / 4), j = (e % (mp / 4)) * 4;
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
      for (int c0 = 0; c0 < C; c0 += 8) {
        f32x4 pv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          pv[u] = (c0 + u < C) ? *reinterpret_cast<const f32x4*>(pw + ((size_t)(c0 + u) * D + f) * mp + j)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (c0 + u < C) acc += *reinterpret_cast<const f32x4*>(wgt + (c0 + u) * mp + j) * pv[u];
      }
      uint16_t hb[4], lb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) split1(acc[q], hb[q], lb[q]);
      *reinterpret_cast<u32x2*>(wtl + (size_t)f * YS + j) =
          u32x2{(uint32_t)hb[0] | ((uint32_t)hb[1] << 16), (uint32_t)hb[2] | ((uint32_t)hb[3] << 16)};
      *reinterpret_cast<u32x2*>(wtl + (size_t)D * YS + (size_t)f * YS + j) =
          u32x2{(uint32_t)lb[0] | ((uint32_t)lb[1] << 16), (uint32_t)lb[2] | ((uint32_t)lb[3] << 16)};
      if (taps && a.w_tap != nullptr)
#pragma unroll
        for (int q = 0; q < 4; ++q) a.w_tap[((size_t)bh * mp + j + q) * D + f] = acc[q];
    }
    __syncthreads();
    // Y = Z W: A operand Z rows (global hi/lo), B operand W read along landmarks (W^T)
    const size_t P = (size_t)mp * mp;
    const uint16_t* zr = a.z_hl + (size_t)bh * 2 * P;
    const int ntj = D / 32, ntiles = (mp / 32) * ntj;
    for (int t = wave; t < ntiles; t += 4) {
      const int row0 = 32 * (t / ntj), col0 = 32 * (t % ntj);
      const f32x16 yv = gemm_tile(zr, zr + P, mp, wtl, wtl + (size_t)D * YS, YS, row0, col0, mp, lane);
      const int f = col0 + r32;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int i = acc_row(row0, rr, lane);
        const int ip = (i & ~15) | kslot_perm(i & 15);
        uint16_t hb, lb;
        split1(yv[rr], hb, lb);
        yl[(size_t)f * YS + ip] = hb;
        yl[(size_t)D * YS + (size_t)f * YS + ip] = lb;
        if (taps && a.y_tap != nullptr) a.y_tap[((size_t)bh * mp + i) * D + f] = yv[rr];
      }
    }
    __syncthreads();
    if constexpr (kKtLds) {
      if constexpr (NT > 0) {  // from the fp32 landmarks, scaled to log2 units, then split
        const float* ksrc = a.kt + (size_t)bh * mp * D;
        for (int e = tid; e < mp * (D / 8); e += 256) {
          const int row = e / (D / 8), c8 = (e % (D / 8)) * 8;
          const f32x4 u0 = *reinterpret_cast<const f32x4*>(ksrc + (size_t)row * D + c8);
          const f32x4 u1 = *reinterpret_cast<const f32x4*>(ksrc + (size_t)row * D + c8 + 4);
          float x[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            x[q] = u0[q] * a.scale_log2e;
            x[4 + q] = u1[q] * a.scale_log2e;
          }
          const Pair8 p = split8(x);
          st8(kl + (size_t)row * KR + c8, p.hi);
          st8(kl + (size_t)mp * KR + (size_t)row * KR + c8, p.lo);
        }
      } else {
        const uint16_t* ksrc = a.kt_hl + (size_t)bh * 2 * mp * D;
        for (int e = tid; e < 2 * mp * (D / 8); e += 256) {
          const int row = e / (D / 8), c8 = (e % (D / 8)) * 8;
          st8(kl + (size_t)row * KR + c8, ld8(ksrc + (size_t)row * D + c8));
        }
      }
    }
  }
  const uint16_t* khl = a.kt_hl + (size_t)bh * 2 * mp * D;
  const Tin* Q = static_cast<const Tin*>(a.q) + (size_t)bh * a.n * D;
  const Tin* V = static_cast<const Tin*>(a.v) + (size_t)bh * a.n * D;
  // transposed-read addressing of the conv operand (see lds_tr16): lane k = 4j + q of
  // each 16-lane group points at row j, column F(q) of the feature tile
  const int trj = (lane & 15) >> 2, trq = lane & 3;
  const int trcol = (D / 2) * (trq & 1) + 8 * ((lane >> 4) & 1) + 4 * (trq >> 1);

  auto load_v = [&](int T0, Chunk<Tin>* vc) {
    const int e0 = T0 - a.half;
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int qi = tid + 256 * u;
      const int row = qi / (D / 8), cf = qi % (D / 8), tok = e0 + row;
      vc[u].load(V + (size_t)tok * D + cf * 8, qi < EXT * (D / 8) && tok >= 0 && tok < a.n);
    }
  };
  auto store_v = [&](const Chunk<Tin>* vc) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int qi = tid + 256 * u;
      if (qi < EXT * (D / 8)) {
        const int row = qi / (D / 8), cf = qi % (D / 8);
        vc[u].store(vt + (size_t)row * VR + cf * 8, vt_lo + (size_t)row * VR + cf * 8);
      }
    }
  };
  auto load_q = [&](int T0, Pair8* qb) {
    const int tq = T0 + 32 * wave + r32;
#pragma unroll
    for (int s = 0; s < KD; ++s)
      qb[s] = Input<Tin>::load8(Q + (size_t)tq * D + 16 * s + 8 * h, tq < t_end);
  };
  // scores of landmark tile lt (landmarks x tokens)
  auto scores = [&](int lt, const Pair8* qb) -> f32x16 {
    f32x16 S = zero16();
    if constexpr (kKtLds) {
      const uint16_t* kp = kl + (size_t)(32 * lt + r32) * KR + 8 * h;
#pragma unroll
      for (int s = 0; s < KD; ++s) {
        const Pair8 ka{ld8(kp + 16 * s), ld8(kp + (size_t)mp * KR + 16 * s)};
        S = mfma_pair<true, kS>(ka, qb[s], S);
      }
    } else {
      const uint16_t* kp = khl + (size_t)(32 * lt + r32) * D + 8 * h;
      Pair8 ka[KD];
#pragma unroll
      for (int s = 0; s < KD; ++s) ka[s] = Pair8{ld8(kp + 16 * s), ld8(kp + (size_t)mp * D + 16 * s)};
#pragma unroll
      for (int s = 0; s < KD; ++s) S = mfma_pair<true, kS>(ka[s], qb[s], S);
    }
    return S;
  };
  // O^T += Y^T P^T for the 16 landmarks of k-step 2*lt + s2 (P values p[0..7])
  auto add_py = [&](f32x16* oacc, int lt, int s2, const float* p) {
    const Pair8 pb = split8(p);
#pragma unroll
    for (int f = 0; f < FT; ++f) {
      const uint16_t* yp = yl + (size_t)out_feature<D>(f, r32) * YS + 32 * lt + 16 * s2 + 8 * h;
      const Pair8 ya{ld8(yp), ld8(yp + (size_t)D * YS)};
      oacc[f] = mfma_pair<true, true>(ya, pb, oacc[f]);
    }
  };

  Chunk<Tin> vc[NCH];
  Pair8 qb[KD];
  load_v(t_begin, vc);
  load_q(t_begin, qb);
  __syncthreads();  // prologue done with the region the V tile reuses
  store_v(vc);
  __syncthreads();

  for (int T0 = t_begin; T0 < t_end; T0 += 128) {
    const bool more = T0 + 128 < t_end;
    Pair8 qn[KD];
    if (more) {  // next step's V rows and Q, in flight during this step's products
      load_v(T0 + 128, vc);
      load_q(T0 + 128, qn);
    }
    const int tq = T0 + 32 * wave + r32;
    const bool qok = tq < t_end;

    f32x16 oacc[FT];
#pragma unroll
    for (int f = 0; f < FT; ++f) oacc[f] = zero16();
    if constexpr (NT > 0) {
      // all scores in registers: max, exponentials, sum, then normalised P
      f32x16 S[NT];
#pragma unroll
      for (int lt = 0; lt < NT; ++lt) S[lt] = scores(lt, qb);
      float mx = kNegBig;
#pragma unroll
      for (int lt = 0; lt < NT; ++lt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          if (kFull || score_landmark(lt, rr, h) < a.m) mx = fmaxf(mx, S[lt][rr]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      float ps = 0.f;
#pragma unroll
      for (int lt = 0; lt < NT; ++lt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const float e = (kFull || score_landmark(lt, rr, h) < a.m) ? fast_exp2(S[lt][rr] - mx) : 0.f;
          S[lt][rr] = e;
          ps += e;
        }
      ps += __shfl_xor(ps, 32);
      const float inv = 1.f / ps;
#pragma unroll
      for (int lt = 0; lt < NT; ++lt)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = S[lt][8 * s2 + e] * inv;
          add_py(oacc, lt, s2, p);
        }
    } else {
      float M = kNegBig, L = 0.f;
      for (int lt = 0; lt < mp / 32; ++lt) {
        const f32x16 S = scores(lt, qb);
        float x[16];
        float mx = kNegBig;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          x[rr] = S[rr] * score_scale;
          if (score_landmark(lt, rr, h) < a.m) mx = fmaxf(mx, x[rr]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(M, mx);
        const float corr = fast_exp2(M - mn);
        float p[16];
        float ps = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          p[rr] = score_landmark(lt, rr, h) < a.m ? fast_exp2(x[rr] - mn) : 0.f;
          ps += p[rr];
        }
        L = L * corr + ps;
        M = mn;
#pragma unroll
        for (int f = 0; f < FT; ++f) oacc[f] *= corr;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) add_py(oacc, lt, s2, &p[8 * s2]);
      }
      L += __shfl_xor(L, 32);
      const float inv = 1.f / L;
#pragma unroll
      for (int f = 0; f < FT; ++f) oacc[f] *= inv;
    }

    if (a.attn_tap != nullptr && qok) {
      float* tp = a.attn_tap + ((size_t)bh * a.n + tq) * D + (D / 2) * h;
#pragma unroll
      for (int f = 0; f < FT; ++f)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(tp + 16 * f + 4 * q4) =
              f32x4{oacc[f][4 * q4], oacc[f][4 * q4 + 1], oacc[f][4 * q4 + 2], oacc[f][4 * q4 + 3]};
    }

    // conv: A operand V_ext^T (features x ext tokens) by transposed reads of the V rows
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const Pair8 wb{ld8(wl + ((size_t)(2 * s) * 64 + lane) * 8),
                     ld8(wl + ((size_t)(2 * s + 1) * 64 + lane) * 8)};
      const size_t r0 = (size_t)(32 * wave + 16 * s + 8 * h + trj) * VR + trcol;
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        Pair8 va;
        va.hi = lds_tr16x2(vt + r0 + 16 * f, vt + r0 + 16 * f + 4 * VR);
        va.lo = kS ? lds_tr16x2(vt_lo + r0 + 16 * f, vt_lo + r0 + 16 * f + 4 * VR) : zero8();
        oacc[f] = mfma_pair<kS, true>(va, wb, oacc[f]);
      }
    }

    if (qok) {
      if constexpr (kS) {
        float* op = static_cast<float*>(a.out) + ((size_t)bh * a.n + tq) * D + (D / 2) * h;
#pragma unroll
        for (int f = 0; f < FT; ++f)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<f32x4*>(op + 16 * f + 4 * q4) = f32x4{
                oacc[f][4 * q4], oacc[f][4 * q4 + 1], oacc[f][4 * q4 + 2], oacc[f][4 * q4 + 3]};
      } else {
        uint16_t* op = static_cast<uint16_t*>(a.out) + ((size_t)bh * a.n + tq) * D + (D / 2) * h;
#pragma unroll
        for (int f = 0; f < FT; ++f) {
          bf16x8 lo8, hi8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            lo8[e] = bf16_rne(oacc[f][e]);
            hi8[e] = bf16_rne(oacc[f][8 + e]);
          }
          st8(op + 16 * f, lo8);
          st8(op + 16 * f + 8, hi8);
        }
      }
    }
    if (more) {
      __syncthreads();  // every wave is done with this step's V tile
      store_v(vc);
#pragma unroll
      for (int s = 0; s < KD; ++s) qb[s] = qn[s];
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ host side
// LDS budget of one block; Kt goes to LDS only when everything fits in 160 KiB.
constexpr size_t kLdsLimit = 160 * 1024;

static size_t lds_bytes(bool bf16, int d, int mp, int conv_ksteps, int C, bool kt_lds) {
  const size_t ext = 96 + 16 * (size_t)conv_ksteps;
  const size_t yl = (size_t)2 * d * (mp + 8) * 2;
  const size_t wl = (size_t)conv_ksteps * 2 * 64 * 8 * 2;
  const size_t prologue = yl + (size_t)C * mp * 4;
  const size_t main = ((kt_lds ? (size_t)2 * mp * (d + 8) : 0) +
                       (bf16 ? 1 : 2) * ext * (size_t)(d + 8)) * 2;
  return yl + wl + (prologue > main ? prologue : main);
}

static bool kt_in_lds(bool bf16, int d, int mp, int conv_ksteps, int C) {
  return lds_bytes(bf16, d, mp, conv_ksteps, C, true) <= kLdsLimit;
}

size_t output_lds_bytes(bool bf16, int d, int mp, int conv_ksteps, int C) {
  return lds_bytes(bf16, d, mp, conv_ksteps, C, kt_in_lds(bf16, d, mp, conv_ksteps, C));
}

// Kernel variant for a shape: register-resident softmax for m <= 64 with the usual
// conv width (k-steps 4), online softmax otherwise.
template <typename Tin, int D, int KS>
static const void* pick_kernel(const OutArgs& a, bool kt_lds) {
  if constexpr (KS == 4) {
    if (a.mp <= 64 && kt_lds) {
      const bool full = a.m == a.mp;
      if (a.mp == 32)
        return full ? reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 1, true>)
                    : reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 1, false>);
      return full ? reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 2, true>)
                  : reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 2, false>);
    }
  }
  return kt_lds ? reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 0, false>)
                : reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, false, 0, false>);
}

template <typename Tin, int D, int KS>
static hipError_t launch_t(const OutArgs& a, hipStream_t s) {
  constexpr bool kBf16 = !Input<Tin>::kSplit;
  const size_t lds = output_lds_bytes(kBf16, D, a.mp, KS, a.C);
  const void* fn = pick_kernel<Tin, D, KS>(a, kt_in_lds(kBf16, D, a.mp, KS, a.C));
  void* args[] = {const_cast<OutArgs*>(&a)};
  return hipLaunchKernel(fn, dim3(a.BH * a.G), dim3(256), args, lds, s);
}

template <typename Tin, int D>
static hipError_t launch_ks(int ks, const OutArgs& a, hipStream_t s) {
  if (ks == 2) return launch_t<Tin, D, 2>(a, s);
  if (ks == 4) return launch_t<Tin, D, 4>(a, s);
  return launch_t<Tin, D, 6>(a, s);
}

hipError_t launch_output(bool bf16, int d, int ks, const OutArgs& a, hipStream_t s) {
  if (bf16) {
    if (d == 32) return launch_ks<uint16_t, 32>(ks, a, s);
    if (d == 64) return launch_ks<uint16_t, 64>(ks, a, s);
    return launch_ks<uint16_t, 128>(ks, a, s);
  }
  if (d == 32) return launch_ks<float, 32>(ks, a, s);
  if (d == 64) return launch_ks<float, 64>(ks, a, s);
  return launch_ks<float, 128>(ks, a, s);
}

template <typename Tin, int D, int KS>
static hipError_t attr_t(size_t bytes) {
  const void* fns[6] = {
      reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 0, false>),
      reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, false, 0, false>)};
  int nf = 2;
  if constexpr (KS == 4) {
    fns[nf++] = reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 1, true>);
    fns[nf++] = reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 1, false>);
    fns[nf++] = reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 2, true>);
    fns[nf++] = reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 2, false>);
  }
  for (int i = 0; i < nf; ++i) {
    const hipError_t e =
        hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename Tin, int D>
static hipError_t attr_ks(int ks, size_t bytes) {
  if (ks == 2) return attr_t<Tin, D, 2>(bytes);
  if (ks == 4) return attr_t<Tin, D, 4>(bytes);
  return attr_t<Tin, D, 6>(bytes);
}

hipError_t configure_output(bool bf16, int d, int ks, size_t bytes) {
  if (bf16) {
    if (d == 32) return attr_ks<uint16_t, 32>(ks, bytes);
    if (d == 64) return attr_ks<uint16_t, 64>(ks, bytes);
    return attr_ks<uint16_t, 128>(ks, bytes);
  }
  if (d == 32) return attr_ks<float, 32>(ks, bytes);
  if (d == 64) return attr_ks<float, 64>(ks, bytes);
  return attr_ks<float, 128>(ks, bytes);
}

}  // namespace nys
