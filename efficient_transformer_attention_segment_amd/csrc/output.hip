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
// s*log2(e) folded in) and the conv filter's MFMA operand in LDS. All of its global
// loads (chunk states, partials, Z, Kt, the first V rows and Q) are issued before any
// is used, so the set-up costs about one memory round trip.
//
// The block then walks a contiguous token range of its head in steps of 32 tokens per
// wave (4 waves, or 8 for the online-softmax shapes where one block fills the LDS).
// Per wave and step:
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
//  * store: fp32 lanes write d/2 contiguous features of their token; bf16 (RNE) rows
//    pass through the wave's slice of the V tile and leave as whole 128-byte lines,
//    with non-temporal stores.
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

// Landmark tiles whose Kt lo plane a lane can hold in registers (128 VGPRs at most).
template <int D>
constexpr int split_tiles() {
  return 16384 / (32 * D) < 8 ? 16384 / (32 * D) : 8;
}

// NT: landmark tiles handled with all scores in registers (1 or 2), or 0 for the
// online softmax over a runtime number of tiles. kFull: m == 32 * NT (no masking).
// NW: waves per block (4, or 8 where one block fills a CU's LDS); a step covers 32 NW
// tokens. kKtSplit (bf16 online-softmax shapes whose Kt does not fit beside Y^T): Kt is
// the same for every step, so its hi plane is kept in LDS (staged after Y is formed, in
// the region the W^T merge used) and each lane keeps its fragments of the lo plane in
// registers for the whole block, instead of reading Kt from L2 every step. (Scores on the
// hi plane alone, Kt rounded to bf16, were faster but lost 0.1 of the attention's scale on
// clustered inputs at m = 256 and at d = 128.)
template <typename Tin, int D, int KS, bool kKtLds, int NT, bool kFull, int NW, bool kKtSplit>
__global__ __launch_bounds__(64 * NW) void output_kernel(OutArgs a) {
  extern __shared__ __align__(16) char lds[];
  constexpr bool kS = Input<Tin>::kSplit;
  constexpr int KD = D / 16, FT = D / 32;
  constexpr int NTH = 64 * NW, STEP = 32 * NW;
  constexpr int EXT = STEP - 32 + 16 * KS;  // staged V rows per step (with halo)
  constexpr int VR = D + 8;          // LDS row stride (elements) of the row-major V tile
  constexpr int KR = D + 8;          // LDS row stride of the Kt planes
  constexpr int NCH = (EXT * (D / 8) + NTH - 1) / NTH;  // 8-element V chunks per thread
  static_assert(32 * NW * D <= EXT * VR, "output rows are staged in the V tile");
  static_assert(NT == 0 || kKtLds, "register-resident softmax expects Kt in LDS");
  static_assert(!kKtSplit || (NT == 0 && !kKtLds && NW == 4 && !kS),
                "split Kt: bf16 online-softmax shapes with 4-wave blocks");
  constexpr int kMaxT = kKtSplit ? split_tiles<D>() : 1;  // landmark tiles held (split Kt)
  // the wave index in a scalar register keeps the per-wave row tests scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, h = lane >> 5;
  const int mp = NT > 0 ? 32 * NT : a.mp;
  const int YS = mp + 8;
  int bh, grp;
  xcd_map(blockIdx.x, a.BH, a.G, bh, grp);
  const int head = bh % a.H;
  const int t_begin = grp * a.tok_per_block;
  const int t_end = min(a.n, t_begin + a.tok_per_block);
  // tokens at or past the head's valid length are padding: not read (the conv sees
  // zeros there), written as zeros
  const int t_valid_v = valid_length(a.lengths, bh, a.H, a.n, a.m);
  const int t_valid = min(t_end, t_valid_v);
  if (t_begin >= t_valid) {
    constexpr int EPV = 16 / sizeof(Tin);  // elements per 16-byte store
    Tin* o = static_cast<Tin*>(a.out) + ((size_t)bh * a.n + t_begin) * D;
    for (int e = threadIdx.x; e < (t_end - t_begin) * (D / EPV); e += NTH)
      *reinterpret_cast<u32x4*>(o + (size_t)e * EPV) = u32x4{0u, 0u, 0u, 0u};
    if (a.attn_tap != nullptr) {
      float* tp = a.attn_tap + ((size_t)bh * a.n + t_begin) * D;
      for (int e = threadIdx.x; e < (t_end - t_begin) * (D / 4); e += NTH)
        *reinterpret_cast<f32x4*>(tp + (size_t)e * 4) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  // scores in log2 units: folded into Kt when it is staged (NT > 0), else applied here
  const float score_scale = NT > 0 ? 1.f : a.scale_log2e;

  uint16_t* yl = reinterpret_cast<uint16_t*>(lds);     // [2][D][YS]  Y^T hi, lo
  uint16_t* wl = yl + (size_t)2 * D * YS;              // [KS][2][64][8] conv B operand
  uint16_t* kl = wl + (size_t)KS * 2 * 64 * 8;         // [2][mp][KR] Kt hi, lo (kKtLds)
  // region used first by the prologue (W^T planes, chunk weights), then by the V rows
  uint16_t* un = kl + (kKtLds ? (size_t)2 * mp * KR : 0);
  uint16_t* wtl = un;                                  // [2][D][YS]  W^T hi, lo
  float* wgt = reinterpret_cast<float*>(un + (size_t)2 * D * YS);  // [C][mp]
  uint16_t* ksp = un;                                  // [mp][KR] Kt hi (kKtSplit)
  uint16_t* vt = un + (kKtSplit ? (size_t)mp * KR : 0);  // [EXT][VR] V rows (hi)
  uint16_t* vt_lo = vt + (size_t)EXT * VR;             // V rows lo (fp32 input only)
  const bool taps = grp == 0;
  const int C = a.C;

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
      const int qi = tid + NTH * u;
      const int row = qi / (D / 8), cf = qi % (D / 8), tok = e0 + row;
      vc[u].load(V + (size_t)tok * D + cf * 8, qi < EXT * (D / 8) && tok >= 0 && tok < t_valid_v);
    }
  };
  auto store_v = [&](const Chunk<Tin>* vc) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int qi = tid + NTH * u;
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
      qb[s] = Input<Tin>::load8(Q + (size_t)tq * D + 16 * s + 8 * h, tq < t_valid);
  };
  // scores of landmark tile lt (landmarks x tokens)
  bf16x8 klo[kMaxT][KD];  // this lane's Kt lo fragments (kKtSplit)
  auto scores = [&](int lt, const Pair8* qb) -> f32x16 {
    f32x16 S = zero16();
    if constexpr (kKtSplit) {
      const uint16_t* kp = ksp + (size_t)(32 * lt + r32) * KR + 8 * h;
#pragma unroll
      for (int s = 0; s < KD; ++s) S = mfma_pair<true, false>(Pair8{ld8(kp + 16 * s), klo[lt][s]}, qb[s], S);
    } else if constexpr (kKtLds) {
      const uint16_t* kp = kl + (size_t)(32 * lt + r32) * KR + 8 * h;
#pragma unroll
      for (int s = 0; s < KD; ++s) {
        const Pair8 ka{ld8(kp + 16 * s), ld8(kp + (size_t)mp * KR + 16 * s)};
        S = mfma_pair<true, kS>(ka, qb[s], S);
      }
    } else {
      // Kt from L2, loaded in groups of KG k-steps (all at once unless registers are
      // short: two waves per SIMD at d = 128)
      constexpr int KG = (NW == 8 && D > 64) ? KD / 2 : KD;
      const uint16_t* kp = khl + (size_t)(32 * lt + r32) * D + 8 * h;
#pragma unroll
      for (int g = 0; g < KD; g += KG) {
        Pair8 ka[KG];
#pragma unroll
        for (int s = 0; s < KG; ++s)
          ka[s] = Pair8{ld8(kp + 16 * (g + s)), ld8(kp + (size_t)mp * D + 16 * (g + s))};
#pragma unroll
        for (int s = 0; s < KG; ++s) S = mfma_pair<true, kS>(ka[s], qb[g + s], S);
      }
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

  // ---- prologue. Every global load is issued before any of it is used, so the whole
  // set-up costs about one memory round trip. The landmark operands go first and the
  // first V rows and Q after them: loads retire in order, so the merge below waits only
  // for the landmark data while the token rows are still arriving.
  // Online-softmax shapes (NT = 0): the head's Y^T planes were formed once for the head
  // (output_ystage_kernel) in this LDS image's layout; LDS-DMA copies them straight in,
  // 1 KiB per wave instruction, completed before the token loop.
  if constexpr (NT == 0) {
    const uint16_t* ys = a.yt + (size_t)bh * 2 * D * YS;
    for (int b = wave; b < D * YS / 256; b += NW) dma16(ys + 512 * b + 8 * lane, yl + 512 * b);
  }
  Chunk<Tin> vc[NCH];
  Pair8 qb[KD];
  float wt0 = 0.f, wt1 = 0.f;  // conv taps `lane` and `lane + 64` of this head (wave 0)
  if (tid < 64) {
    const float* w = a.conv_w + (size_t)head * a.W;
    // clamped reads: the operand below takes only taps below W from these lanes
    wt0 = w[lane < a.W ? lane : a.W - 1];
    wt1 = w[lane + 64 < a.W ? lane + 64 : a.W - 1];
  }
  constexpr int kCB = 4;  // chunk states per load batch
  const float* pml = a.part_ml + (size_t)bh * C * 2 * mp;
  const float* pw = a.part_w + (size_t)bh * C * D * mp;
  const uint16_t* zr = a.z_hl + (size_t)bh * 2 * mp * mp;
  const size_t P = (size_t)mp * mp;
  const int ntj = D / 32, ntiles = (mp / 32) * ntj;
  // Running max / sum of landmark tid in the first kCB chunks. No prologue load sits
  // under a condition: the compiler turns one into a branch whose zero-filled registers it
  // guards with a wait for every load issued so far, so the set-up would take several
  // memory round trips. Slots past C repeat chunk C - 1 (zero weight below; its maximum is
  // already among the others); slots past an element count load in bounds, unused.
  float cm[kCB], cl[kCB];
  if (NT > 0 && tid < mp) {
#pragma unroll
    for (int c = 0; c < kCB; ++c) {
      const int cc = c < C ? c : C - 1;
      cm[c] = pml[(size_t)(2 * cc) * mp + tid];
      cl[c] = pml[(size_t)(2 * cc + 1) * mp + tid];
    }
  }
  // register-resident softmax shapes (mp = 32 NT): partial W^T of the first kCB chunks
  // (UP float4 outputs per thread), Z rows of the wave's Y tiles, the thread's Kt share
  constexpr int UP = NT > 0 ? (D * 8 * NT + NTH - 1) / NTH : 1;
  constexpr int TPY = NT > 0 ? (NT * (D / 32) + NW - 1) / NW : 1;
  constexpr int KM = NT > 0 ? 2 * NT : 1;
  constexpr int KU = NT > 0 ? (4 * NT * D + NTH - 1) / NTH : 1;
  f32x4 pv[UP][kCB];
  Pair8 za[TPY][KM];
  f32x4 kx[KU][2];
  if constexpr (NT > 0) {
#pragma unroll
    for (int u = 0; u < UP; ++u) {
      const int e0 = tid + NTH * u, e = e0 < D * mp / 4 ? e0 : 0;
      const int f = e / (mp / 4), j = (e % (mp / 4)) * 4;
#pragma unroll
      for (int c = 0; c < kCB; ++c) {
        const int cc = c < C ? c : C - 1;
        pv[u][c] = *reinterpret_cast<const f32x4*>(pw + ((size_t)cc * D + f) * mp + j);
      }
    }
#pragma unroll
    for (int u = 0; u < TPY; ++u) {
      const int t = wave + NW * u, tc = t < ntiles ? t : ntiles - 1;
      const int row0 = 32 * (tc / ntj);
#pragma unroll
      for (int s = 0; s < KM; ++s) {
        const size_t o = (size_t)(row0 + r32) * mp + 16 * s + 8 * h;
        za[u][s] = Pair8{ld8(zr + o), ld8(zr + P + o)};
      }
    }
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int e0 = tid + NTH * u, e = e0 < mp * (D / 8) ? e0 : 0;
      const int row = e / (D / 8), c8 = (e % (D / 8)) * 8;
      const float* ks = a.kt + ((size_t)bh * mp + row) * D + c8;
      kx[u][0] = *reinterpret_cast<const f32x4*>(ks);
      kx[u][1] = *reinterpret_cast<const f32x4*>(ks + 4);
    }
  }

  // split Kt: the lane's lo fragments, and a share of the hi rows to stage after Y
  constexpr int KHS = kKtSplit ? (kMaxT * 32 * (D / 8) + NTH - 1) / NTH : 1;
  bf16x8 khs[KHS];
  if constexpr (kKtSplit) {
#pragma unroll
    for (int lt = 0; lt < kMaxT; ++lt)
#pragma unroll
      for (int s = 0; s < KD; ++s)
        klo[lt][s] = ld8(khl + (size_t)mp * D + (size_t)(32 * (32 * lt < mp ? lt : 0) + r32) * D +
                         16 * s + 8 * h);  // tiles past mp load tile 0, unused
#pragma unroll
    for (int u = 0; u < KHS; ++u) {
      const int e = tid + NTH * u, row = e / (D / 8), c8 = (e % (D / 8)) * 8;
      khs[u] = ld8(khl + (size_t)(row < mp ? row : mp - 1) * D + c8);
    }
  }

  load_v(t_begin, vc);
  load_q(t_begin, qb);

  // chunk weights per landmark: exp2(M_c - M*) / sum_c exp2(M_c - M*) L_c
  if (NT > 0 && tid < mp) {
    const int j = tid;
    if (j >= a.m) {
      for (int c = 0; c < C; ++c) wgt[c * mp + j] = 0.f;
    } else if (C <= kCB) {
      float ms = kNegBig;
#pragma unroll
      for (int c = 0; c < kCB; ++c) ms = fmaxf(ms, cm[c]);
      float den = 0.f;
#pragma unroll
      for (int c = 0; c < kCB; ++c) {
        cm[c] = c < C ? fast_exp2(cm[c] - ms) : 0.f;
        den += cm[c] * cl[c];
      }
      const float inv = 1.f / den;
#pragma unroll
      for (int c = 0; c < kCB; ++c)
        if (c < C) wgt[c * mp + j] = cm[c] * inv;
    } else {
      float ms = kNegBig;
      for (int c = 0; c < C; ++c) ms = fmaxf(ms, pml[(size_t)(2 * c) * mp + j]);
      float den = 0.f;
      for (int c = 0; c < C; ++c) {
        const float ev = fast_exp2(pml[(size_t)(2 * c) * mp + j] - ms);
        wgt[c * mp + j] = ev;
        den += ev * pml[(size_t)(2 * c + 1) * mp + j];
      }
      const float inv = 1.f / den;
      for (int c = 0; c < C; ++c) wgt[c * mp + j] *= inv;
    }
  }
  // conv filter as the B operand of the banded product (identical for every wave)
  if (tid < 64) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {  // tap k from the lane that loaded it
        const int k = 16 * s + 8 * h + e - r32;
        const float v0 = __shfl(wt0, k & 63), v1 = __shfl(wt1, k & 63);
        x[e] = (k >= 0 && k < a.W) ? (k < 64 ? v0 : v1) : 0.f;
      }
      const Pair8 p = split8(x);
      st8(wl + ((size_t)(2 * s) * 64 + lane) * 8, p.hi);
      st8(wl + ((size_t)(2 * s + 1) * 64 + lane) * 8, p.lo);
    }
  }
  // Kt planes: from the fp32 landmarks scaled to log2 units (NT > 0), else the hi/lo copy
  if constexpr (kKtLds) {
    if constexpr (NT > 0) {
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int e = tid + NTH * u, row = e / (D / 8), c8 = (e % (D / 8)) * 8;
        if (e < mp * (D / 8)) {
          float x[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            x[q] = kx[u][0][q] * a.scale_log2e;
            x[4 + q] = kx[u][1][q] * a.scale_log2e;
          }
          const Pair8 p = split8(x);
          st8(kl + (size_t)row * KR + c8, p.hi);
          st8(kl + (size_t)mp * KR + (size_t)row * KR + c8, p.lo);
        }
      }
    } else {
      const uint16_t* ksrc = a.kt_hl + (size_t)bh * 2 * mp * D;
      for (int e = tid; e < 2 * mp * (D / 8); e += NTH) {
        const int row = e / (D / 8), c8 = (e % (D / 8)) * 8;
        st8(kl + (size_t)row * KR + c8, ld8(ksrc + (size_t)row * D + c8));
      }
    }
  }
  __syncthreads();
  // W^T[f][j] = sum_c wgt[c][j] * partial_c^T[f][j], four landmarks per thread
  auto put_w = [&](int f, int j, const f32x4& acc) {
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
  };
  auto merge_rest = [&](int f, int j, f32x4 acc, int cfrom) {  // chunks cfrom.. C-1
    for (int c0 = cfrom; c0 < C; c0 += kCB) {
      f32x4 v[kCB];
#pragma unroll
      for (int u = 0; u < kCB; ++u)
        v[u] = c0 + u < C ? *reinterpret_cast<const f32x4*>(pw + ((size_t)(c0 + u) * D + f) * mp + j)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < kCB; ++u)
        if (c0 + u < C) acc += *reinterpret_cast<const f32x4*>(wgt + (c0 + u) * mp + j) * v[u];
    }
    return acc;
  };
  if constexpr (NT > 0) {
#pragma unroll
    for (int u = 0; u < UP; ++u) {
      const int e = tid + NTH * u, f = e / (mp / 4), j = (e % (mp / 4)) * 4;
      if (e < D * mp / 4) {
        f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kCB; ++c)
          if (c < C) acc += *reinterpret_cast<const f32x4*>(wgt + c * mp + j) * pv[u][c];
        if (C > kCB) acc = merge_rest(f, j, acc, kCB);
        put_w(f, j, acc);
      }
    }
  }
  __syncthreads();
  // Y = Z W: A operand Z rows (global hi/lo), B operand W read along landmarks (W^T);
  // stored as Y^T with landmark i at (i & ~15) | kslot_perm(i & 15)
  auto put_y = [&](int row0, int col0, const f32x16& yv) {
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
  };
  if constexpr (NT > 0) {
#pragma unroll
    for (int u = 0; u < TPY; ++u) {
      const int t = wave + NW * u;
      if (t < ntiles) {
        const int row0 = 32 * (t / ntj), col0 = 32 * (t % ntj);
        const size_t ob = (size_t)(col0 + r32) * YS + 8 * h;
        f32x16 yv = zero16();
#pragma unroll
        for (int s = 0; s < KM; ++s) {
          const Pair8 b{ld8(wtl + ob + 16 * s), ld8(wtl + (size_t)D * YS + ob + 16 * s)};
          yv = mfma_pair<true, true>(za[u][s], b, yv);
        }
        put_y(row0, col0, yv);
      }
    }
  }
  __syncthreads();  // the V rows (and the split Kt hi rows) take over the W^T region
  if constexpr (kKtSplit) {
#pragma unroll
    for (int u = 0; u < KHS; ++u) {
      const int e = tid + NTH * u, row = e / (D / 8), c8 = (e % (D / 8)) * 8;
      if (row < mp) st8(ksp + (size_t)row * KR + c8, khs[u]);
    }
  }
  store_v(vc);
  if constexpr (NT == 0) wait_dma_barrier(0);  // every wave's share of the Y^T image landed
  __syncthreads();

  for (int T0 = t_begin; T0 < t_end; T0 += STEP) {
    const bool more = T0 + STEP < t_end;
    // next step's V rows and Q, in flight during this step's products (Q only where the
    // registers allow: not with two waves per SIMD at d = 128)
    constexpr bool kQPre = !(NW == 8 && D > 64);
    Pair8 qn[kQPre ? KD : 1];
    if (more) {
      load_v(T0 + STEP, vc);
      if constexpr (kQPre) load_q(T0 + STEP, qn);
    }
    const int tq = T0 + 32 * wave + r32;
    const bool qok = tq < t_end;
    const bool cut = t_valid < t_end;        // block-uniform
    const bool qpad = cut && tq >= t_valid;  // padding row of a cut block

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
      const float inv = __builtin_amdgcn_rcpf(ps);  // ps >= 1 (the maximum contributes 1)
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
      auto online_tile = [&](int lt) {
        const f32x16 S = scores(lt, qb);
        // without a register prefetch, the next step's Q goes into qb as soon as the
        // last scores are formed, in flight during the products below
        if constexpr (!kQPre)
          if (more && lt == mp / 32 - 1) load_q(T0 + STEP, qb);
        const bool full = 32 * lt + 32 <= a.m;  // no padded landmark in this tile
        float mx = kNegBig;
        if (full) {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, S[rr]);
        } else {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            if (score_landmark(lt, rr, h) < a.m) mx = fmaxf(mx, S[rr]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * score_scale;  // the scale is positive
        // lazy rescaling: the reference maximum M moves only when some lane's maximum
        // passes it by more than 8 (probabilities then stay <= 256); the state (M, L,
        // acc) is exact for any reference point
        if (__any(mx > M + 8.f)) {
          const float mn = fmaxf(M, mx);
          const float corr = fast_exp2(M - mn);
          L *= corr;
#pragma unroll
          for (int f = 0; f < FT; ++f) oacc[f] *= corr;
          M = mn;
        }
        float p[16];
        float ps = 0.f;
        if (full) {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            p[rr] = fast_exp2(fmaf(S[rr], score_scale, -M));
            ps += p[rr];
          }
        } else {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            p[rr] = score_landmark(lt, rr, h) < a.m ? fast_exp2(fmaf(S[rr], score_scale, -M)) : 0.f;
            ps += p[rr];
          }
        }
        L += ps;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) add_py(oacc, lt, s2, &p[8 * s2]);
      };
      if constexpr (kKtSplit) {
#pragma unroll
        for (int lt = 0; lt < kMaxT; ++lt)
          if (32 * lt < mp) online_tile(lt);
      } else {
        for (int lt = 0; lt < mp / 32; ++lt) online_tile(lt);
      }
      L += __shfl_xor(L, 32);
      const float inv = __builtin_amdgcn_rcpf(L);  // L >= 1 (the maximum contributes 1)
#pragma unroll
      for (int f = 0; f < FT; ++f) oacc[f] *= inv;
    }

    // only a cut block has padding rows; the empty asm keeps this a scalar branch (the
    // compiler would otherwise turn the zeroing into selects that every block runs)
    if (cut) {
      asm volatile("");
      if (qpad)
#pragma unroll
        for (int f = 0; f < FT; ++f) oacc[f] = zero16();
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

    if (cut) {
      asm volatile("");
      if (qpad)
#pragma unroll
        for (int f = 0; f < FT; ++f) oacc[f] = zero16();
    }
    if constexpr (kS) {
      if (qok) {
        float* op = static_cast<float*>(a.out) + ((size_t)bh * a.n + tq) * D + (D / 2) * h;
#pragma unroll
        for (int f = 0; f < FT; ++f)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<f32x4*>(op + 16 * f + 4 * q4) = f32x4{
                oacc[f][4 * q4], oacc[f][4 * q4 + 1], oacc[f][4 * q4 + 2], oacc[f][4 * q4 + 3]};
      }
    } else {
      // bf16: a lane holds half a row, so direct stores would fill each 128-byte line a
      // quarter per instruction. The wave's 32 rows are staged in its own slice of the V
      // tile (free once every wave's conv reads are done; 16-byte chunk c of row r sits
      // at chunk c ^ (r % CPR)) and written back as whole consecutive rows.
      constexpr int CPR = D / 8;
      __syncthreads();  // every wave has finished its conv reads of the V tile
      uint16_t* ow = vt + (size_t)wave * 32 * D;
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        bf16x8 lo8, hi8;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 a2 = bf16_rne2(oacc[f][e], oacc[f][e + 1]);
          const bf16x2 b2 = bf16_rne2(oacc[f][8 + e], oacc[f][9 + e]);
          lo8[e] = a2[0];
          lo8[e + 1] = a2[1];
          hi8[e] = b2[0];
          hi8[e + 1] = b2[1];
        }
        const int c0 = (CPR / 2) * h + 2 * f;  // chunk of features (D/2) h + 16 f
        st8(ow + r32 * D + 8 * (c0 ^ (r32 % CPR)), lo8);
        st8(ow + r32 * D + 8 * ((c0 + 1) ^ (r32 % CPR)), hi8);
      }
      // The output is not read again by this forward: non-temporal stores keep it from
      // displacing Q, K and V in the memory-side cache, whose dirty lines would otherwise
      // be written back during the next kernels' reads.
      uint16_t* ob = static_cast<uint16_t*>(a.out) + ((size_t)bh * a.n + T0 + 32 * wave) * D;
#pragma unroll
      for (int i = 0; i < CPR / 2; ++i) {
        const int row = i * (64 / CPR) + lane / CPR, c = lane % CPR;
        const bf16x8 v = ld8(ow + row * D + 8 * (c ^ (row % CPR)));
        if (T0 + 32 * wave + row < t_end)
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v),
                                      reinterpret_cast<u32x4*>(ob + (size_t)row * D + 8 * c));
      }
    }
    if (more) {
      __syncthreads();  // every wave is done with this step's V tile
      store_v(vc);
#pragma unroll
      for (int s = 0; s < KD; ++s) {
        if constexpr (kQPre) qb[s] = qn[s];
      }
      __syncthreads();
    }
  }
}

// Y^T staging for the online-softmax variants (NT = 0), once per head instead of in
// every output block: block (head, feature tile of 32) merges the C partial context
// states into W^T rows f0 .. f0+31 (chunk weights exp2(M_c - M*) / sum_c exp2(M_c - M*) L_c
// per landmark, chunks in fixed order), then each wave forms one 32-landmark row tile of
// Y = Z W on MFMA and writes it as the output kernel's LDS image of Y^T: [2][D][mp + 8]
// hi/lo bf16 with landmark i at (i & ~15) | kslot_perm(i & 15).
template <int D>
__global__ __launch_bounds__(512) void output_ystage_kernel(OutArgs a) {
  __shared__ __align__(16) float wgt[kMaxChunks * 256];      // [C][mp]
  __shared__ __align__(16) uint16_t wt[2 * 32 * (256 + 8)];  // W^T rows of the tile, hi/lo
  const int mp = a.mp, YS = mp + 8, C = a.C;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nth = blockDim.x;
  const int bh = blockIdx.x / (D / 32), f0 = 32 * (blockIdx.x % (D / 32));
  const float* pml = a.part_ml + (size_t)bh * C * 2 * mp;
  const float* pw = a.part_w + (size_t)bh * C * D * mp;
  // chunk weights of landmark j (thread j): every chunk's (max, sum) loaded at once
  if (tid < mp) {
    const int j = tid;
    float cm[kMaxChunks], cl[kMaxChunks];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      cm[c] = c < C ? pml[(size_t)(2 * c) * mp + j] : kNegBig;
      cl[c] = c < C ? pml[(size_t)(2 * c + 1) * mp + j] : 0.f;
    }
    float ms = kNegBig;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) ms = fmaxf(ms, cm[c]);
    float den = 0.f;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      cm[c] = c < C ? fast_exp2(cm[c] - ms) : 0.f;
      den += cm[c] * cl[c];
    }
    const float inv = j < a.m ? 1.f / den : 0.f;  // padded landmarks weigh nothing
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
      if (c < C) wgt[c * mp + j] = cm[c] * inv;
  }
  __syncthreads();
  // W^T[f][j] = sum_c wgt[c][j] partial_c[f][j]: four landmarks per output, all C chunk
  // loads of an output in flight together
  for (int e = tid; e < 32 * (mp / 4); e += nth) {
    const int fl = e / (mp / 4), j = (e % (mp / 4)) * 4, f = f0 + fl;
    f32x4 v[kMaxChunks];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
      v[c] = c < C ? *reinterpret_cast<const f32x4*>(pw + ((size_t)c * D + f) * mp + j)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
      if (c < C) acc += *reinterpret_cast<const f32x4*>(wgt + c * mp + j) * v[c];
    uint16_t hb[4], lb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) split1(acc[q], hb[q], lb[q]);
    *reinterpret_cast<u32x2*>(wt + (size_t)fl * YS + j) =
        u32x2{(uint32_t)hb[0] | ((uint32_t)hb[1] << 16), (uint32_t)hb[2] | ((uint32_t)hb[3] << 16)};
    *reinterpret_cast<u32x2*>(wt + (size_t)32 * YS + (size_t)fl * YS + j) =
        u32x2{(uint32_t)lb[0] | ((uint32_t)lb[1] << 16), (uint32_t)lb[2] | ((uint32_t)lb[3] << 16)};
    if (a.w_tap != nullptr)  // each feature tile writes its own columns
#pragma unroll
      for (int q = 0; q < 4; ++q) a.w_tap[((size_t)bh * mp + j + q) * D + f] = acc[q];
  }
  __syncthreads();
  // Y rows 32 wave .. + 31, columns f0 .. f0 + 31: A = Z rows (hi/lo), B read along the
  // landmarks from the W^T planes
  const int row0 = 32 * wave;
  if (row0 >= mp) return;
  const uint16_t* zr = a.z_hl + (size_t)bh * 2 * mp * mp;
  const f32x16 yv = gemm_tile_rt(zr, zr + (size_t)mp * mp, mp, wt, wt + (size_t)32 * YS, YS,
                                 row0, 0, mp, lane);
  uint16_t* yt = a.yt + (size_t)bh * 2 * D * YS;
  const int f = f0 + (lane & 31);
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int i = acc_row(row0, rr, lane);
    const int ip = (i & ~15) | kslot_perm(i & 15);
    uint16_t hb, lb;
    split1(yv[rr], hb, lb);
    yt[(size_t)f * YS + ip] = hb;
    yt[(size_t)D * YS + (size_t)f * YS + ip] = lb;
    if (a.y_tap != nullptr) a.y_tap[((size_t)bh * mp + i) * D + f] = yv[rr];
  }
}

// ------------------------------------------------------------------ host side
// LDS budget of one block; Kt goes to LDS only when everything fits in 160 KiB.
constexpr size_t kLdsLimit = 160 * 1024;

// Where Kt lives for the scores: the whole hi/lo copy in LDS, split (hi plane in LDS,
// lo plane in registers), or read from L2 every step.
enum class KtPlace { kLds, kSplit, kL2 };

// A block's LDS. ypre: an online-softmax variant, whose Y^T is staged per head (no W^T
// merge region).
static size_t lds_bytes(bool bf16, int d, int mp, int conv_ksteps, int C, KtPlace kt, int nw,
                        bool ypre) {
  const size_t ext = 32 * (size_t)nw - 32 + 16 * (size_t)conv_ksteps;
  const size_t yl = (size_t)2 * d * (mp + 8) * 2;
  const size_t wl = (size_t)conv_ksteps * 2 * 64 * 8 * 2;
  const size_t kl = kt == KtPlace::kLds ? (size_t)2 * mp * (d + 8) * 2 : 0;
  const size_t wtl = ypre ? 0 : (size_t)2 * d * (mp + 8) * 2 + (size_t)C * mp * 4;  // W^T + chunk weights
  // after the prologue: the split Kt hi rows, then the V rows
  const size_t vt = (kt == KtPlace::kSplit ? (size_t)mp * (d + 8) * 2 : 0) +
                    (bf16 ? 1 : 2) * ext * (size_t)(d + 8) * 2;
  return yl + wl + kl + (wtl > vt ? wtl : vt);
}

static int split_tiles_host(int d) { return std::min(8, 16384 / (32 * d)); }

struct OutShape {
  KtPlace kt;
  int nw;
  size_t lds;
  bool ypre;  // online softmax (NT = 0): Y^T staged per head by output_ystage_kernel
};

// Kernel shape for a problem. m <= 64 with the usual conv width (k-steps 4) and Kt in LDS
// runs the register-resident softmax, whose blocks merge the context states and form Y
// themselves (cheap at that size). Every other shape runs the online softmax over
// landmark tiles on Y^T staged once per head. Waves per block: those shapes usually fill
// a CU's LDS with one block. Where Kt fits beside Y^T the block takes 8 waves and
// 256-token steps if the larger V tile still fits (and registers allow two waves per
// SIMD: bf16, d <= 64). Where it does not fit, bf16 shapes hold Kt split (hi plane in
// LDS, lo plane in registers) in a 4-wave block, whose one wave per SIMD has the whole
// register file; fp32 shapes read Kt from L2.
static OutShape out_shape(bool bf16, int d, int mp, int ks, int C) {
  if (ks == 4 && mp <= 64 && lds_bytes(bf16, d, mp, ks, C, KtPlace::kLds, 4, false) <= kLdsLimit)
    return {KtPlace::kLds, 4, lds_bytes(bf16, d, mp, ks, C, KtPlace::kLds, 4, false), false};
  auto lds = [&](KtPlace kt, int nw) { return lds_bytes(bf16, d, mp, ks, C, kt, nw, true); };
  if (lds(KtPlace::kLds, 4) <= kLdsLimit) {
    int nw = 4;
    if (bf16 && mp > 64 && 2 * lds(KtPlace::kLds, 4) > kLdsLimit && lds(KtPlace::kLds, 8) <= kLdsLimit)
      nw = 8;
    return {KtPlace::kLds, nw, lds(KtPlace::kLds, nw), true};
  }
  if (bf16 && mp > 64 && mp / 32 <= split_tiles_host(d) &&
      lds(KtPlace::kSplit, 4) <= kLdsLimit)
    return {KtPlace::kSplit, 4, lds(KtPlace::kSplit, 4), true};
  int nw = 4;
  if (bf16 && mp > 64 && 2 * lds(KtPlace::kL2, 4) > kLdsLimit && lds(KtPlace::kL2, 8) <= kLdsLimit)
    nw = 8;
  return {KtPlace::kL2, nw, lds(KtPlace::kL2, nw), true};
}

bool output_stages_y(bool bf16, int d, int mp, int conv_ksteps, int C) {
  return out_shape(bf16, d, mp, conv_ksteps, C).ypre;
}

size_t output_lds_bytes(bool bf16, int d, int mp, int conv_ksteps, int C) {
  return out_shape(bf16, d, mp, conv_ksteps, C).lds;
}

int output_step_tokens(bool bf16, int d, int mp, int conv_ksteps, int C) {
  return 32 * out_shape(bf16, d, mp, conv_ksteps, C).nw;
}

// Kernel variant for a shape: register-resident softmax for m <= 64 with the usual
// conv width (k-steps 4), online softmax otherwise.
template <typename Tin, int D, int KS>
static const void* pick_kernel(const OutArgs& a, const OutShape& sh) {
  const bool kt_lds = sh.kt == KtPlace::kLds;
  if constexpr (KS == 4) {
    if (!sh.ypre) {  // register-resident softmax: mp <= 64, Kt in LDS
      const bool full = a.m == a.mp;
      if (a.mp == 32)
        return full ? reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 1, true, 4, false>)
                    : reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 1, false, 4, false>);
      return full ? reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 2, true, 4, false>)
                  : reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 2, false, 4, false>);
    }
  }
  if constexpr (!Input<Tin>::kSplit) {
    if (sh.kt == KtPlace::kSplit)
      return reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, false, 0, false, 4, true>);
    if (sh.nw == 8)
      return kt_lds ? reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 0, false, 8, false>)
                    : reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, false, 0, false, 8, false>);
  }
  return kt_lds ? reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 0, false, 4, false>)
                : reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, false, 0, false, 4, false>);
}

template <typename Tin, int D, int KS>
static int blocks_per_cu_t(int mp, int m, int C, size_t lds) {
  constexpr bool kBf16 = !Input<Tin>::kSplit;
  OutArgs a{};
  a.mp = mp;
  a.m = m;
  a.C = C;
  const OutShape sh = out_shape(kBf16, D, mp, KS, C);
  const void* fn = pick_kernel<Tin, D, KS>(a, sh);
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, 64 * sh.nw, lds) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return nb;
}

template <typename Tin, int D>
static int blocks_per_cu_ks(int ks, int mp, int m, int C, size_t lds) {
  if (ks == 2) return blocks_per_cu_t<Tin, D, 2>(mp, m, C, lds);
  if (ks == 4) return blocks_per_cu_t<Tin, D, 4>(mp, m, C, lds);
  return blocks_per_cu_t<Tin, D, 6>(mp, m, C, lds);
}

int output_blocks_per_cu(bool bf16, int d, int ks, int mp, int m, int C, size_t lds) {
  if (bf16) {
    if (d == 32) return blocks_per_cu_ks<uint16_t, 32>(ks, mp, m, C, lds);
    if (d == 64) return blocks_per_cu_ks<uint16_t, 64>(ks, mp, m, C, lds);
    return blocks_per_cu_ks<uint16_t, 128>(ks, mp, m, C, lds);
  }
  if (d == 32) return blocks_per_cu_ks<float, 32>(ks, mp, m, C, lds);
  if (d == 64) return blocks_per_cu_ks<float, 64>(ks, mp, m, C, lds);
  return blocks_per_cu_ks<float, 128>(ks, mp, m, C, lds);
}

template <typename Tin, int D, int KS>
static hipError_t launch_t(const OutArgs& a, hipStream_t s) {
  constexpr bool kBf16 = !Input<Tin>::kSplit;
  const OutShape sh = out_shape(kBf16, D, a.mp, KS, a.C);
  const void* fn = pick_kernel<Tin, D, KS>(a, sh);
  void* args[] = {const_cast<OutArgs*>(&a)};
  if (sh.ypre) {
    if (a.C > kMaxChunks || a.mp > 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL(output_ystage_kernel<D>, dim3(a.BH * (D / 32)), dim3(64 * (a.mp / 32)), 0,
                       s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipLaunchKernel(fn, dim3(a.BH * a.G), dim3(64 * sh.nw), args, sh.lds, s);
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
  const void* fns[9] = {
      reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 0, false, 4, false>),
      reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, false, 0, false, 4, false>)};
  int nf = 2;
  if constexpr (KS == 4) {
    fns[nf++] = reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 1, true, 4, false>);
    fns[nf++] = reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 1, false, 4, false>);
    fns[nf++] = reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 2, true, 4, false>);
    fns[nf++] = reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 2, false, 4, false>);
  }
  if constexpr (!Input<Tin>::kSplit) {
    fns[nf++] = reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, true, 0, false, 8, false>);
    fns[nf++] = reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, false, 0, false, 8, false>);
    fns[nf++] = reinterpret_cast<const void*>(&output_kernel<Tin, D, KS, false, 0, false, 4, true>);
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
