// Host side of the C ABI declared in include/nys_attn.h: argument validation (before
// any HIP call), device check, workspace sizing and carving, the launch sequence on the
// caller's stream (segment means, pseudo-inverse, landmark context, output), debug taps,
// stage timing, the backward pass and the projections.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <mutex>
#include <cstdint>
#include <cstdlib>
#include <new>
#include <cstring>
#include <string>
#include <vector>

#include "nys_attn.h"
#include "nys_kernels.h"

namespace {

thread_local std::string g_err;

nys_status fail(nys_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

constexpr int kStages = 4;  // segment means, pseudo-inverse, landmark context, output
const char* const kStageName[kStages] = {"segment means", "pseudo-inverse", "landmark context",
                                         "output"};

// Debug switches, read from the environment at each call (debugging only; none of them
// changes a result):
//   NYS_FAULT=alloc   nys_attn_create fails as if the workspace allocation had failed
//   NYS_FAULT=launch  forward and backward fail as if a kernel launch had failed, before
//                     anything is enqueued
//   NYS_DEBUG_SYNC=1  forward and backward wait for the stream after every launch and
//                     name the stage whose kernel failed (slow; localises device faults)
//   NYS_LOG=1         nys_attn_create prints the plan (tiles, grids, workspace) to stderr
bool env_is(const char* name, const char* value) {
  const char* e = std::getenv(name);
  return e != nullptr && std::strcmp(e, value) == 0;
}
bool env_on(const char* name) {
  const char* e = std::getenv(name);
  return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }
long long round_up(long long a, long long b) { return ((a + b - 1) / b) * b; }

// Whether the context chunks are split unevenly (the split itself is computed per block
// on the device, context_block in context.hip). Workgroups of one launch are placed
// round-robin over the CUs (block b on CU b mod ncu while they all fit at once: measured
// with per-block clocks), so a context block b >= ncu with b mod ncu < npinv runs next to
// a pseudo-inverse block and progresses at about 0.7 of the speed of the others. With the
// uneven split the context blocks are taken chunk-major (block npinv + c BH + bh holds
// chunk c of head bh; with BH a multiple of 8 a head's blocks still share one XCD), so
// every head has chunks on both kinds of CU, and each head's tokens are split in
// proportion to those speeds. False (uniform chunks, head-major blocks) when the launch
// does not fit in one round of resident blocks or no context block shares a CU.
bool uneven_chunks(int BH, int C, int npinv, int ncu, int slots_per_cu) {
  const long long blocks = (long long)npinv + (long long)BH * C;
  if (npinv <= 0 || npinv >= ncu || C < 2 || (BH & 7) != 0 ||
      blocks > (long long)slots_per_cu * ncu || blocks <= ncu)
    return false;
  for (long long b = npinv; b < blocks; ++b)
    if (b >= ncu && (int)(b % ncu) < npinv) return true;
  return false;
}

}  // namespace

// Byte offsets of the workspace's sub-buffers (256-byte aligned).
struct WsLayout {
  size_t qt, kt, qhl, khl, as, z, pl, own, apart, zhl, pw, pml, w, y, yt;
};

struct nys_attn_plan {
  int B, H, n, d, m, mp, W, half, iters, ks;
  nys_dtype dtype;
  int BH, chunk, C, LG, TG, tok_per_block, G;
  bool fused;  // pseudo-inverse blocks ride in the context launch (mp <= 64)
  int device;
  char* ws;
  size_t ws_bytes;
  WsLayout lay;
  bool debug_taps;  // the workspace holds the fp32 W and Y tap buffers
  nys::SegArgs seg;
  nys::CtxArgs ctx;
  nys::OutArgs out;
  int prof_max, prof_count;
  std::vector<hipEvent_t> prof_ev;  // kStages + 1 per recorded call
  char* bws;                        // backward workspace (first backward call), or null
  size_t bws_bytes;
  nys::BwdArgs bwd;
  char* gws;                        // general-backward workspace (first such call), or null
  size_t gws_bytes;
  nys::GenBwdArgs gen;
};

static nys_status validate_shape(int B, int H, int n, int d, int m, int W, int iters,
                                 nys_dtype dtype) {
  if (B < 0 || H < 0) return fail(NYS_E_ARG, "B and H must be >= 0");
  if (n < 1) return fail(NYS_E_ARG, "n must be >= 1");
  if (m < 1 || m > n) return fail(NYS_E_ARG, "need 1 <= m <= n");
  if (m > 256) return fail(NYS_E_UNSUPPORTED, "m > 256 is not built");
  if (d < 1) return fail(NYS_E_ARG, "d must be >= 1");
  if (d != 32 && d != 64 && d != 128) return fail(NYS_E_UNSUPPORTED, "d must be 32, 64 or 128");
  if (W < 1 || (W % 2) == 0) return fail(NYS_E_ARG, "conv_width must be odd and >= 1");
  if (W > 65) return fail(NYS_E_UNSUPPORTED, "conv_width > 65 is not built");
  if (iters < 0 || iters > 100) return fail(NYS_E_ARG, "pinv_iters must be in [0, 100]");
  if (dtype != NYS_F32 && dtype != NYS_BF16) return fail(NYS_E_ARG, "unknown dtype");
  if ((long long)n * d >= (1LL << 31)) return fail(NYS_E_UNSUPPORTED, "n*d must be < 2^31");
  // 2 B H m segment tasks are counted in 32 bits (m <= 256)
  if ((long long)B * H >= (1LL << 23)) return fail(NYS_E_UNSUPPORTED, "B*H must be < 2^23");
  return NYS_OK;
}

// Current device, checked to be a gfx950 part; its properties in *prop.
static nys_status current_device(int* dev, hipDeviceProp_t* prop) {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return fail(NYS_E_DEVICE, "no HIP device available");
  }
  if (hipGetDevice(dev) != hipSuccess) return fail(NYS_E_DEVICE, "hipGetDevice failed");
  if (hipGetDeviceProperties(prop, *dev) != hipSuccess)
    return fail(NYS_E_DEVICE, "hipGetDeviceProperties failed");
  if (std::strncmp(prop->gcnArchName, "gfx950", 6) != 0)
    return fail(NYS_E_DEVICE, std::string("device is ") + prop->gcnArchName + ", need gfx950");
  return NYS_OK;
}

// Everything of a plan but its workspace pointers: shapes, tiling, launch geometry (from
// the device's CU count and the runtime's occupancy figures), kernel LDS limits and the
// workspace layout (p->lay, p->ws_bytes). debug_taps: reserve the fp32 W and Y buffers
// that nys_attn_forward_debug fills. Allocates nothing.
static nys_status plan_init(nys_attn_plan* p, int B, int H, int n, int d, int m,
                            int conv_width, int pinv_iters, nys_dtype dtype, int dev,
                            const hipDeviceProp_t& prop, bool debug_taps) {
  p->B = B; p->H = H; p->n = n; p->d = d; p->m = m; p->W = conv_width;
  p->half = (conv_width - 1) / 2; p->iters = pinv_iters; p->dtype = dtype;
  p->device = dev;
  p->BH = B * H;
  p->mp = (int)round_up(m, 32);
  p->LG = p->mp / 32;
  p->TG = nys::context_token_groups(p->LG);
  const int step = 32 * p->TG;
  const long long work = (long long)p->BH * n;
  p->fused = nys::context_fuses_pinv(p->mp);
  p->ks = (p->half == 0) ? 2 : (p->half <= 16 ? 4 : 6);
  const bool bf16 = dtype == NYS_BF16;

  nys::CtxArgs& c = p->ctx;
  std::memset(&c, 0, sizeof(c));
  c.BH = p->BH; c.H = H; c.n = n; c.d = d; c.m = m; c.mp = p->mp; c.iters = pinv_iters;
  c.LG = p->LG; c.TG = p->TG;
  c.npinv = p->fused ? p->BH : 0;
  nys::context_ring_geometry(d, c);
  const size_t ctx_lds = nys::context_lds_bytes(bf16, d, c);
  const size_t max_lds = (size_t)prop.sharedMemPerBlock;
  if (ctx_lds > max_lds) return fail(NYS_E_UNSUPPORTED, "shape needs more LDS than the device offers");
  if (nys::configure_context(bf16, d, p->mp, ctx_lds) != hipSuccess) {
    (void)hipGetLastError();
    return fail(NYS_E_LAUNCH, "could not set kernel LDS limits");
  }
  // Context blocks: about one resident round of them next to the fused pseudo-inverse
  // blocks (the runtime's occupancy figure; three per CU if it cannot tell), at most 16
  // chunks per head (bounds the merge), and, with the fused pseudo-inverse, at most 4
  // when that still fills half the slots: the output prologue loads the chunk states of
  // four chunks in one batch.
  const int ctx_per_cu = nys::context_blocks_per_cu(bf16, d, p->mp, ctx_lds);
  const long long slots =
      (long long)(ctx_per_cu > 0 ? ctx_per_cu : 3) * std::max(1, prop.multiProcessorCount);
  const long long target = std::max<long long>(slots / 2, slots - (p->fused ? p->BH : 0));
  const long long heads = std::max(1, p->BH);  // B*H == 0 is an empty problem
  long long nc = std::min<long long>(16, std::max<long long>(1, (target + heads - 1) / heads));
  if (p->fused && nc > 4 && 4LL * heads >= target / 2) nc = 4;
  p->chunk = (int)round_up(std::max<long long>(step, ((long long)n + nc - 1) / nc), step);
  p->chunk = (int)std::min<long long>(p->chunk, round_up(n, step));
  p->C = ceil_div(n, p->chunk);
  if (p->C > nys::kMaxChunks) return fail(NYS_E_UNSUPPORTED, "too many context chunks");
  c.chunk = p->chunk; c.C = p->C;
  const size_t out_lds = nys::output_lds_bytes(bf16, d, p->mp, p->ks, p->C);
  if (out_lds > max_lds) return fail(NYS_E_UNSUPPORTED, "shape needs more LDS than the device offers");
  if (nys::configure_output(bf16, d, p->ks, out_lds) != hipSuccess) {
    (void)hipGetLastError();
    return fail(NYS_E_LAUNCH, "could not set kernel LDS limits");
  }
  // Output blocks: one resident round of them (the prologue of every block merges the
  // context states and forms Y, so a second round repeats it); 512 slots when the
  // runtime cannot tell the occupancy.
  {
    const int per_cu = nys::output_blocks_per_cu(bf16, d, p->ks, p->mp, m, p->C, out_lds);
    const long long slots =
        per_cu > 0 ? (long long)per_cu * std::max(1, prop.multiProcessorCount) : 512;
    const int stp = nys::output_step_tokens(bf16, d, p->mp, p->ks, p->C);
    p->tok_per_block = (int)round_up(std::max<long long>(stp, (work + slots - 1) / slots), stp);
    p->tok_per_block = (int)std::min<long long>(p->tok_per_block, round_up(n, stp));
    p->G = ceil_div(n, p->tok_per_block);
    // the same number of blocks per head with their tokens balanced (512 tokens in blocks of
    // 384 would leave one block a third of the other's work)
    p->tok_per_block = (int)round_up(ceil_div(n, p->G), stp);
    p->G = ceil_div(n, p->tok_per_block);
  }
  const bool uneven = p->fused && uneven_chunks(p->BH, p->C, p->BH, prop.multiProcessorCount,
                                                ctx_per_cu);
  c.uneven_ncu = uneven ? prop.multiProcessorCount : 0;
  c.scale = 1.0f / std::sqrt((float)d);
  c.scale_log2e = (float)(1.4426950408889634 / std::sqrt((double)d));

  // workspace layout
  const size_t BHs = (size_t)p->BH, mp = (size_t)p->mp, dd = (size_t)d;
  const size_t P = mp * mp;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  WsLayout& L = p->lay;
  L.qt = take(BHs * mp * dd * 4); L.kt = take(BHs * mp * dd * 4);
  L.qhl = take(BHs * 2 * mp * dd * 2); L.khl = take(BHs * 2 * mp * dd * 2);
  L.as = take(BHs * P * 4); L.z = take(BHs * P * 4);
  L.pl = take(p->mp > 64 ? BHs * nys::kPlanes * P * 2 : 0);
  L.own = take(p->mp > 64 ? BHs * 2 * P * 4 : 0);
  L.apart = take(p->mp > 64 ? BHs * (mp / 32) * (mp + 1) * 4 : 0);
  L.zhl = take(BHs * 2 * P * 2);
  L.pw = take(BHs * p->C * mp * dd * 4); L.pml = take(BHs * p->C * 2 * mp * 4);
  L.yt = take(nys::output_stages_y(bf16, d, p->mp, p->ks, p->C) ? BHs * 2 * dd * (mp + 8) * 2 : 0);
  L.w = take(debug_taps ? BHs * mp * dd * 4 : 0);
  L.y = take(debug_taps ? BHs * mp * dd * 4 : 0);
  p->ws_bytes = off;
  p->ws = nullptr;
  p->debug_taps = debug_taps;

  nys::OutArgs& o = p->out;
  std::memset(&o, 0, sizeof(o));
  o.BH = p->BH; o.H = H; o.n = n; o.m = m; o.mp = p->mp; o.W = conv_width; o.half = p->half;
  o.tok_per_block = p->tok_per_block; o.G = p->G; o.C = p->C;
  o.scale_log2e = c.scale_log2e;

  if (env_on("NYS_LOG"))
    std::fprintf(stderr,
                 "[nys_attn] plan B=%d H=%d n=%d d=%d m=%d (mp %d) W=%d iters=%d %s: "
                 "pseudo-inverse %s; context %d chunks of %d tokens (%s), %d blocks of %d "
                 "threads, %zu B LDS; output %d blocks per head of %d tokens, %zu B LDS; "
                 "workspace %zu B\n",
                 B, H, n, d, m, p->mp, conv_width, pinv_iters, bf16 ? "bf16" : "fp32",
                 p->fused ? "in the context launch" : "separate launches", p->C, p->chunk,
                 uneven ? "uneven split" : "even split", c.npinv + p->BH * p->C,
                 64 * p->LG * p->TG, ctx_lds, p->G, p->tok_per_block, out_lds, p->ws_bytes);
  p->prof_max = 0;
  p->prof_count = 0;
  p->bws = nullptr;
  p->bws_bytes = 0;
  std::memset(&p->bwd, 0, sizeof(p->bwd));
  p->gws = nullptr;
  p->gws_bytes = 0;
  std::memset(&p->gen, 0, sizeof(p->gen));
  return NYS_OK;
}

// Point the plan's kernel arguments at a workspace laid out by plan_init.
static void plan_bind(nys_attn_plan* p, char* ws) {
  p->ws = ws;
  const WsLayout& L = p->lay;
  auto F = [&](size_t o) { return reinterpret_cast<float*>(ws + o); };
  auto U = [&](size_t o) { return reinterpret_cast<uint16_t*>(ws + o); };
  p->seg = nys::SegArgs{nullptr, p->BH, p->H, p->n, p->m, p->mp, F(L.qt), F(L.kt), U(L.qhl),
                        U(L.khl)};
  nys::CtxArgs& c = p->ctx;
  c.qt = F(L.qt); c.qt_hl = U(L.qhl); c.kt_hl = U(L.khl);
  c.a_s = F(L.as); c.z = F(L.z); c.planes = U(L.pl); c.own = F(L.own);
  c.alpha_part = F(L.apart); c.z_hl = U(L.zhl);
  c.part_w = F(L.pw); c.part_ml = F(L.pml);
  nys::OutArgs& o = p->out;
  o.kt = F(L.kt); o.kt_hl = U(L.khl); o.z_hl = U(L.zhl); o.part_w = F(L.pw); o.part_ml = F(L.pml);
  o.yt = U(L.yt);
  o.w_tap = p->debug_taps ? F(L.w) : nullptr;  // enabled per call (debug forwards only)
  o.y_tap = p->debug_taps ? F(L.y) : nullptr;
}

extern "C" nys_status nys_attn_create(nys_attn_plan** plan, int B, int H, int n, int d, int m,
                                      int conv_width, int pinv_iters, nys_dtype dtype) {
  if (plan == nullptr) return fail(NYS_E_ARG, "plan out-pointer is NULL");
  *plan = nullptr;
  nys_status st = validate_shape(B, H, n, d, m, conv_width, pinv_iters, dtype);
  if (st != NYS_OK) return st;
  int dev = 0;
  hipDeviceProp_t prop;
  if ((st = current_device(&dev, &prop)) != NYS_OK) return st;

  nys_attn_plan* p = new (std::nothrow) nys_attn_plan();
  if (p == nullptr) return fail(NYS_E_NOMEM, "host allocation failed");
  if ((st = plan_init(p, B, H, n, d, m, conv_width, pinv_iters, dtype, dev, prop, true)) !=
      NYS_OK) {
    delete p;
    return st;
  }
  if (env_is("NYS_FAULT", "alloc")) {
    delete p;
    return fail(NYS_E_NOMEM, "workspace allocation failed (NYS_FAULT=alloc)");
  }
  char* ws = nullptr;
  if (p->ws_bytes > 0) {
    if (hipMalloc(reinterpret_cast<void**>(&ws), p->ws_bytes) != hipSuccess) {
      (void)hipGetLastError();
      delete p;
      return fail(NYS_E_NOMEM, "workspace allocation failed");
    }
    // zero once: landmark rows m..mp-1 stay zero for the plan's lifetime
    if (hipMemset(ws, 0, p->ws_bytes) != hipSuccess) {
      (void)hipFree(ws);
      delete p;
      return fail(NYS_E_LAUNCH, "workspace set-up failed");
    }
  }
  plan_bind(p, ws);
  *plan = p;
  g_err.clear();
  return NYS_OK;
}

static bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

static nys_status forward_impl(nys_attn_plan* p, const void* q, const void* k, const void* v,
                               const float* conv_w, const int* lengths, void* out, void* stream,
                               const nys_attn_taps* taps) {
  if (p == nullptr) return fail(NYS_E_ARG, "plan is NULL");
  if (p->BH == 0) return NYS_OK;
  if (!q || !k || !v || !out || !conv_w) return fail(NYS_E_ARG, "NULL tensor pointer");
  auto misaligned = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; };
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out))
    return fail(NYS_E_ARG, "q, k, v and out must be 16-byte aligned");
  const size_t bytes = (size_t)p->BH * p->n * p->d * (p->dtype == NYS_BF16 ? 2 : 4);
  if (ranges_overlap(out, bytes, q, bytes) || ranges_overlap(out, bytes, k, bytes) ||
      ranges_overlap(out, bytes, v, bytes))
    return fail(NYS_E_ARG, "out overlaps q, k or v");
  if (taps && taps->attn && misaligned(taps->attn))
    return fail(NYS_E_ARG, "taps->attn must be 16-byte aligned");

  if (env_is("NYS_FAULT", "launch"))
    return fail(NYS_E_LAUNCH, "kernel launch failed (NYS_FAULT=launch)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = p->dtype == NYS_BF16;
  const bool dsync = env_on("NYS_DEBUG_SYNC");
  const bool prof = p->prof_count < p->prof_max;
  hipEvent_t* ev = prof ? &p->prof_ev[(kStages + 1) * p->prof_count] : nullptr;
  auto chk = [&](hipError_t e, const char* what) -> bool {
    if (e != hipSuccess) {
      g_err = std::string(what) + ": " + hipGetErrorString(e);
      return false;
    }
    return true;
  };
  // stage i's launch(es) are enqueued: record its end marker, and with NYS_DEBUG_SYNC
  // wait for them and name the stage if its kernel failed
  auto mark = [&](int i) {
    if (dsync && i > 0) {
      const hipError_t e = hipStreamSynchronize(s);
      if (e != hipSuccess) {
        g_err = std::string(kStageName[i - 1]) + " kernel failed: " + hipGetErrorString(e);
        return false;
      }
    }
    return !prof || chk(hipEventRecord(ev[i], s), "event record");
  };
  nys::SegArgs sg = p->seg;
  sg.lengths = lengths;
  nys::CtxArgs c = p->ctx;
  c.k = k;
  c.v = v;
  c.lengths = lengths;
  nys::OutArgs o = p->out;
  o.q = q;
  o.v = v;
  o.conv_w = conv_w;
  o.lengths = lengths;
  o.out = out;
  o.attn_tap = taps ? taps->attn : nullptr;
  c.fp32_out = taps && (taps->a_s || taps->z);
  if (!taps || (!taps->w && !taps->y)) o.w_tap = o.y_tap = nullptr;
  if (!mark(0) || !chk(nys::launch_segmeans(bf16, p->d, q, k, sg, s), "segment means launch") ||
      !mark(1) || (!p->fused && !chk(nys::launch_pinv(p->d, c, s), "pseudo-inverse launch")) ||
      !mark(2) || !chk(nys::launch_context(bf16, p->d, c, s), "landmark context launch") ||
      !mark(3) || !chk(nys::launch_output(bf16, p->d, p->ks, o, s), "output launch") ||
      !mark(4))
    return NYS_E_LAUNCH;
  if (prof) p->prof_count++;

  if (taps) {
    const size_t mp = p->mp, m = p->m, dd = p->d, BH = p->BH;
    auto copy_md = [&](float* dst, const float* src) {
      if (!dst) return true;
      return chk(hipMemcpy2DAsync(dst, m * dd * 4, src, mp * dd * 4, m * dd * 4, BH,
                                  hipMemcpyDeviceToDevice, s),
                 "tap copy");
    };
    auto copy_mm = [&](float* dst, const float* src) {
      if (!dst) return true;
      for (size_t b = 0; b < BH; ++b)
        if (!chk(hipMemcpy2DAsync(dst + b * m * m, m * 4, src + b * mp * mp, mp * 4, m * 4, m,
                                  hipMemcpyDeviceToDevice, s),
                 "tap copy"))
          return false;
      return true;
    };
    if (!copy_md(taps->q_land, p->seg.qt) || !copy_md(taps->k_land, p->seg.kt) ||
        !copy_md(taps->w, p->out.w_tap) || !copy_md(taps->y, p->out.y_tap) ||
        !copy_mm(taps->a_s, p->ctx.a_s) || !copy_mm(taps->z, p->ctx.z))
      return NYS_E_LAUNCH;
  }
  return NYS_OK;
}

extern "C" nys_status nys_attn_forward(nys_attn_plan* plan, const void* q, const void* k,
                                       const void* v, const float* conv_w, void* out,
                                       void* stream) {
  return forward_impl(plan, q, k, v, conv_w, nullptr, out, stream, nullptr);
}

extern "C" nys_status nys_attn_forward_debug(nys_attn_plan* plan, const void* q, const void* k,
                                             const void* v, const float* conv_w, void* out,
                                             void* stream, const nys_attn_taps* taps) {
  return forward_impl(plan, q, k, v, conv_w, nullptr, out, stream, taps);
}

extern "C" nys_status nys_attn_forward_varlen(nys_attn_plan* plan, const void* q, const void* k,
                                              const void* v, const float* conv_w,
                                              const int* lengths, void* out, void* stream,
                                              const nys_attn_taps* taps) {
  return forward_impl(plan, q, k, v, conv_w, lengths, out, stream, taps);
}

// ------------------------------------------------------------------ allocation-free forward
// The workspace of nys_attn_forward_noalloc: one static device array per GPU, held for
// the life of the process. In host code `scratch` names a host-side stand-in, never the
// device memory: its device address comes from hipGetSymbolAddress, once per device.
static constexpr size_t kScratchBytes = (size_t)NYS_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
struct NoallocDevice {
  bool ready;
  hipDeviceProp_t prop;
  char* scratch;  // device address of this device's copy of `scratch`
};
constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
NoallocDevice g_noalloc[kMaxDevices];
}  // namespace

// Properties and scratch address of the current device, looked up on its first call.
static nys_status noalloc_device(int* dev, const NoallocDevice** out) {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return fail(NYS_E_DEVICE, "no HIP device available");
  }
  if (hipGetDevice(dev) != hipSuccess) return fail(NYS_E_DEVICE, "hipGetDevice failed");
  if (*dev < 0 || *dev >= kMaxDevices) return fail(NYS_E_DEVICE, "device index out of range");
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  NoallocDevice& nd = g_noalloc[*dev];
  if (!nd.ready) {
    int d2 = 0;
    nys_status st = current_device(&d2, &nd.prop);
    if (st != NYS_OK) return st;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return fail(NYS_E_DEVICE, std::string("scratch symbol lookup failed: ") +
                                    hipGetErrorString(e));
    }
    nd.scratch = static_cast<char*>(ptr);
    nd.ready = true;
  }
  *out = &nd;
  return NYS_OK;
}

extern "C" nys_status nys_attn_forward_noalloc(int B, int H, int n, int d, int m, int conv_width,
                                               int pinv_iters, nys_dtype dtype, const void* q,
                                               const void* k, const void* v,
                                               const float* conv_w, void* out, void* stream) {
  nys_status st = validate_shape(B, H, n, d, m, conv_width, pinv_iters, dtype);
  if (st != NYS_OK) return st;
  if (B * H == 0) return NYS_OK;
  int dev = 0;
  const NoallocDevice* nd = nullptr;
  if ((st = noalloc_device(&dev, &nd)) != NYS_OK) return st;
  nys_attn_plan p{};
  if ((st = plan_init(&p, B, H, n, d, m, conv_width, pinv_iters, dtype, dev, nd->prop, false)) !=
      NYS_OK)
    return st;
  if (p.ws_bytes > kScratchBytes)
    return fail(NYS_E_UNSUPPORTED, "shape needs " + std::to_string(p.ws_bytes) +
                                       " bytes of workspace; the static scratch of the "
                                       "allocation-free forward holds " +
                                       std::to_string(kScratchBytes));
  plan_bind(&p, nd->scratch);
  // Landmark rows m..mp-1 must read as zero; the scratch keeps whatever an earlier call
  // left there, so they are cleared before the forward (a kernel, not a memset).
  if (p.mp > p.m) {
    const hipError_t e = nys::launch_clear_landmark_padding(p.d, p.seg,
                                                            static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
      return fail(NYS_E_LAUNCH, std::string("landmark padding clear: ") + hipGetErrorString(e));
  }
  return forward_impl(&p, q, k, v, conv_w, nullptr, out, stream, nullptr);
}

extern "C" size_t nys_attn_workspace_bytes(const nys_attn_plan* plan) {
  return plan ? plan->ws_bytes : 0;
}

extern "C" nys_status nys_attn_profile_enable(nys_attn_plan* p, int max_calls) {
  if (p == nullptr || max_calls < 0 || max_calls > 100000)
    return fail(NYS_E_ARG, "profile_enable: bad plan or max_calls");
  for (hipEvent_t e : p->prof_ev) (void)hipEventDestroy(e);
  p->prof_ev.clear();
  p->prof_ev.resize((kStages + 1) * (size_t)max_calls);
  // Device-scope release: the markers sit between kernels of one stream, so no
  // system-scope fence is needed; with one, every marker costs microseconds of GPU time
  // that would be counted in the neighbouring stages.
  for (auto& e : p->prof_ev)
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
      p->prof_max = 0;
      return fail(NYS_E_LAUNCH, "event creation failed");
    }
  p->prof_max = max_calls;
  p->prof_count = 0;
  return NYS_OK;
}

extern "C" nys_status nys_attn_profile_read(nys_attn_plan* p, float* stage_ms, int max_calls,
                                            int* n_calls) {
  if (p == nullptr || n_calls == nullptr || (stage_ms == nullptr && max_calls > 0))
    return fail(NYS_E_ARG, "profile_read: NULL argument");
  const int n = std::min(p->prof_count, max_calls);
  for (int i = 0; i < n; ++i) {
    hipEvent_t* ev = &p->prof_ev[(kStages + 1) * i];
    if (hipEventSynchronize(ev[kStages]) != hipSuccess)
      return fail(NYS_E_LAUNCH, "event sync failed");
    for (int j = 0; j < kStages; ++j) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, ev[j], ev[j + 1]) != hipSuccess)
        return fail(NYS_E_LAUNCH, "event elapsed failed");
      stage_ms[kStages * i + j] = ms;
    }
  }
  *n_calls = n;
  p->prof_count = 0;
  return NYS_OK;
}

extern "C" void nys_attn_destroy(nys_attn_plan* p) {
  if (p == nullptr) return;
  (void)hipDeviceSynchronize();
  for (hipEvent_t e : p->prof_ev) (void)hipEventDestroy(e);
  if (p->ws) (void)hipFree(p->ws);
  if (p->bws) (void)hipFree(p->bws);
  if (p->gws) (void)hipFree(p->gws);
  delete p;
}

// ------------------------------------------------------------------ backward
static constexpr int kFinalTokens = 128;  // tokens per block of the final backward pass

// Carves (or, with base == nullptr, sizes) the backward workspace into p->bwd.
static size_t carve_backward(nys_attn_plan* p, char* base) {
  const size_t BHs = (size_t)p->BH, mp = (size_t)p->mp, dd = (size_t)p->d;
  const size_t P = mp * mp, T = (size_t)p->iters, C = (size_t)p->C;
  const int C3 = ceil_div(p->n, kFinalTokens);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return base ? base + o : nullptr;
  };
  nys::BwdArgs& b = p->bwd;
  b.w = reinterpret_cast<float*>(take(BHs * mp * dd * 4));
  b.stat = reinterpret_cast<float*>(take(BHs * 2 * mp * 4));
  b.a_s = reinterpret_cast<float*>(take(BHs * P * 4));
  b.alpha = reinterpret_cast<float*>(take(BHs * 4 * 4));
  b.amax = reinterpret_cast<int*>(take(BHs * 2 * 4));
  b.zs = reinterpret_cast<float*>(take(BHs * (T + 1) * P * 4));
  b.xs = reinterpret_cast<float*>(take(BHs * T * P * 4));
  b.y_hl = reinterpret_cast<uint16_t*>(take(BHs * 2 * mp * dd * 2));
  b.ktT_hl = reinterpret_cast<uint16_t*>(take(BHs * 2 * dd * mp * 2));
  b.qtT_hl = reinterpret_cast<uint16_t*>(take(BHs * 2 * dd * mp * 2));
  b.part1 = reinterpret_cast<float*>(take(BHs * C * 2 * mp * dd * 4));
  b.dw_hl = reinterpret_cast<uint16_t*>(take(BHs * 2 * mp * dd * 2));
  b.dwT_hl = reinterpret_cast<uint16_t*>(take(BHs * 2 * dd * mp * 2));
  b.db = reinterpret_cast<float*>(take(BHs * mp * 4));
  b.dkt = reinterpret_cast<float*>(take(BHs * mp * dd * 4));
  b.dqt = reinterpret_cast<float*>(take(BHs * mp * dd * 4));
  b.part2 = reinterpret_cast<float*>(take(BHs * C * mp * dd * 4));
  b.dq_part = reinterpret_cast<float*>(take(BHs * p->n * dd * 4));
  b.dv_part = reinterpret_cast<float*>(take(BHs * p->n * dd * 4));
  b.part_dw = reinterpret_cast<float*>(take(BHs * C3 * p->W * 4));
  b.B = p->B; b.H = p->H; b.BH = p->BH; b.n = p->n; b.d = p->d; b.m = p->m; b.mp = p->mp;
  b.W = p->W; b.iters = p->iters; b.chunk = p->chunk; b.C = p->C;
  b.chunk3 = kFinalTokens; b.C3 = C3;
  b.scale = p->ctx.scale;
  b.scale_log2e = p->ctx.scale_log2e;
  return off;
}

static nys_status backward_setup(nys_attn_plan* p) {
  static std::once_flag once;
  static hipError_t cfg = hipSuccess;
  std::call_once(once, [] { cfg = nys::configure_backward(); });
  if (cfg != hipSuccess) {
    (void)hipGetLastError();
    return fail(NYS_E_LAUNCH, "could not set backward kernel LDS limits");
  }
  if (p->bws) return NYS_OK;
  const size_t bytes = carve_backward(p, nullptr);
  if (hipMalloc(reinterpret_cast<void**>(&p->bws), bytes) != hipSuccess) {
    (void)hipGetLastError();
    p->bws = nullptr;
    return fail(NYS_E_NOMEM, "backward workspace allocation failed");
  }
  p->bws_bytes = bytes;
  carve_backward(p, p->bws);
  const nys::SegArgs& sg = p->seg;
  nys::BwdArgs& b = p->bwd;
  b.qt = sg.qt; b.kt = sg.kt; b.qt_hl = sg.qt_hl; b.kt_hl = sg.kt_hl;
  b.part_w = p->ctx.part_w; b.part_ml = p->ctx.part_ml;
  return NYS_OK;
}

// Tokens per block of the general backward's conv-weight partial sums.
static constexpr int kDwChunk = 256;

// Carves (or, with base == nullptr, sizes) the general-backward workspace into p->gen.
static size_t carve_general(nys_attn_plan* p, char* base) {
  const size_t BHs = (size_t)p->BH, mp = (size_t)p->mp, dd = (size_t)p->d, n = (size_t)p->n;
  const size_t mm = mp * mp, T = (size_t)p->iters;
  const size_t nch = (n + kDwChunk - 1) / kDwChunk;
  size_t off = 0;
  auto take = [&](size_t floats) {
    size_t o = off;
    off = align256(off + floats * 4);
    return base ? reinterpret_cast<float*>(base + o) : nullptr;
  };
  nys::GenBwdArgs& g = p->gen;
  g.F = take(BHs * n * mp); g.G1 = take(BHs * n * mp);
  g.Bm = take(BHs * mp * n); g.G2 = take(BHs * mp * n);
  for (float** t : {&g.A, &g.P, &g.Q1, &g.R, &g.Gz, &g.Gn, &g.dR, &g.dX, &g.dQ1, &g.dP, &g.dA})
    *t = take(BHs * mm);
  g.Zs = take(BHs * (T + 1) * mm);
  g.Xs = take(BHs * std::max<size_t>(T, 1) * mm);
  for (float** t : {&g.Wc, &g.Y, &g.dY, &g.dW, &g.dQt, &g.dKt}) *t = take(BHs * mp * dd);
  for (float** t : {&g.dQ, &g.dK, &g.dV}) *t = take(BHs * n * dd);
  g.alpha = take(BHs * 4);
  g.amax = reinterpret_cast<int*>(take(BHs * 2));
  g.dw_part = take(BHs * nch * p->W);
  // split-K scratch: up to 32 splits of at least 512 tokens, while B*H*splits fits a grid z
  g.nsplit = (int)std::max<size_t>(1, std::min<size_t>({32, n / 512, 65535 / std::max<size_t>(BHs, 1)}));
  g.ksplit = take(g.nsplit > 1 ? (size_t)g.nsplit * BHs * mp * dd : 0);
  g.B = p->B; g.H = p->H; g.BH = p->BH; g.n = p->n; g.d = p->d; g.m = p->m; g.mp = p->mp;
  g.W = p->W; g.iters = p->iters; g.dw_chunk = kDwChunk;
  g.scale = p->ctx.scale;
  g.bf16 = p->dtype == NYS_BF16;
  g.qt = p->seg.qt;
  g.kt = p->seg.kt;
  return off;
}

static nys_status general_setup(nys_attn_plan* p) {
  if (p->gws) return NYS_OK;
  if (p->BH > 65535) return fail(NYS_E_UNSUPPORTED, "backward: B*H > 65535");
  const size_t bytes = carve_general(p, nullptr);
  if (hipMalloc(reinterpret_cast<void**>(&p->gws), bytes) != hipSuccess) {
    (void)hipGetLastError();
    p->gws = nullptr;
    return fail(NYS_E_NOMEM, "backward workspace allocation failed");
  }
  p->gws_bytes = bytes;
  carve_general(p, p->gws);
  return NYS_OK;
}

extern "C" nys_status nys_attn_backward(nys_attn_plan* p, const void* q, const void* k,
                                        const void* v, const float* conv_w, const int* lengths,
                                        const void* dout, void* dq, void* dk, void* dv,
                                        float* dconv_w, void* stream) {
  if (p == nullptr) return fail(NYS_E_ARG, "plan is NULL");
  if (!q || !k || !v || !conv_w || !dout || !dq || !dk || !dv || !dconv_w)
    return fail(NYS_E_ARG, "NULL tensor pointer");
  for (const void* t : {q, k, v, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if ((reinterpret_cast<uintptr_t>(t) & 15u) != 0)
      return fail(NYS_E_ARG, "q, k, v, dout, dq, dk and dv must be 16-byte aligned");
  const size_t bytes = (size_t)p->BH * p->n * p->d * (p->dtype == NYS_BF16 ? 2 : 4);
  const void* outs[] = {dq, dk, dv};
  const void* ins[] = {q, k, v, dout};
  for (int i = 0; i < 3; ++i) {
    for (const void* in : ins)
      if (ranges_overlap(outs[i], bytes, in, bytes))
        return fail(NYS_E_ARG, "dq, dk, dv must not overlap q, k, v or dout");
    for (int j = 0; j < i; ++j)
      if (ranges_overlap(outs[i], bytes, outs[j], bytes))
        return fail(NYS_E_ARG, "dq, dk and dv must not overlap each other");
  }
  const size_t wbytes = (size_t)p->H * p->W * 4;
  if (ranges_overlap(dconv_w, wbytes, conv_w, wbytes))
    return fail(NYS_E_ARG, "dconv_w must not overlap conv_w");
  if (env_is("NYS_FAULT", "launch"))
    return fail(NYS_E_LAUNCH, "kernel launch failed (NYS_FAULT=launch)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->BH == 0) {
    if (hipMemsetAsync(dconv_w, 0, wbytes, s) != hipSuccess)
      return fail(NYS_E_LAUNCH, "dconv_w clear failed");
    return NYS_OK;
  }
  // the fused kernels cover bf16 with m <= 64; everything else (and NYS_BACKWARD=general)
  // takes the general path
  const bool general = p->dtype != NYS_BF16 || p->mp > 64 || env_is("NYS_BACKWARD", "general");
  const bool dsync = env_on("NYS_DEBUG_SYNC");
  if (general) {
    nys_status st = general_setup(p);
    if (st != NYS_OK) return st;
    nys::SegArgs sg = p->seg;
    sg.lengths = lengths;
    nys::GenBwdArgs g = p->gen;
    g.q = q; g.k = k; g.v = v; g.dout = dout; g.conv_w = conv_w; g.lengths = lengths;
    g.dq = dq; g.dk = dk; g.dv = dv; g.dconv_w = dconv_w;
    hipError_t e = nys::launch_segmeans(p->dtype == NYS_BF16, p->d, q, k, sg, s);
    if (e == hipSuccess && dsync) e = hipStreamSynchronize(s);
    if (e != hipSuccess)
      return fail(NYS_E_LAUNCH, std::string("backward: segment means: ") + hipGetErrorString(e));
    e = nys::launch_backward_general(g, s);
    if (e == hipSuccess && dsync) e = hipStreamSynchronize(s);
    if (e != hipSuccess)
      return fail(NYS_E_LAUNCH, std::string("backward: general kernels: ") + hipGetErrorString(e));
    return NYS_OK;
  }
  nys_status st = backward_setup(p);
  if (st != NYS_OK) return st;
  nys::SegArgs sg = p->seg;
  sg.lengths = lengths;
  nys::CtxArgs c = p->ctx;
  c.k = k;
  c.v = v;
  c.lengths = lengths;
  nys::BwdArgs b = p->bwd;
  b.q = static_cast<const uint16_t*>(q);
  b.k = static_cast<const uint16_t*>(k);
  b.v = static_cast<const uint16_t*>(v);
  b.dout = static_cast<const uint16_t*>(dout);
  b.conv_w = conv_w;
  b.lengths = lengths;
  b.dq = static_cast<uint16_t*>(dq);
  b.dk = static_cast<uint16_t*>(dk);
  b.dv = static_cast<uint16_t*>(dv);
  b.dconv_w = dconv_w;
  // Segments a final-pass tile of kFinalTokens tokens can meet: with every sequence of
  // length n, segments hold at least floor(n / m) tokens, so at most
  // kFinalTokens / floor(n / m) + 2; with per-sequence lengths a segment can be a single
  // token, so all of them.
  {
    const int per = p->n / p->m;
    b.fin_segs = (lengths == nullptr && per >= 1)
                     ? std::min(p->mp, kFinalTokens / per + 2)
                     : p->mp;
  }
  const char* what = "";
  hipError_t e = hipSuccess;
  // one stage's launch result (and, with NYS_DEBUG_SYNC, its completion)
  auto stage = [&](const char* name, hipError_t le) {
    what = name;
    e = le;
    if (e == hipSuccess && dsync) e = hipStreamSynchronize(s);
    return e == hipSuccess;
  };
  if (stage("segment means", nys::launch_segmeans(true, p->d, q, k, sg, s)) &&
      (p->fused || stage("pseudo-inverse", nys::launch_pinv(p->d, c, s))) &&
      stage("landmark context", nys::launch_context(true, p->d, c, s)) &&
      stage("gradient kernels", nys::launch_backward(b, s)))
    return NYS_OK;
  return fail(NYS_E_LAUNCH, std::string("backward: ") + what + ": " + hipGetErrorString(e));
}

// ------------------------------------------------------------------ projections
static nys_status proj_checks(int B, int H, int n, int d, int d_model) {
  if (B < 1 || H < 1 || n < 1) return fail(NYS_E_ARG, "B, H and n must be >= 1");
  if (d < 1 || d_model < 1) return fail(NYS_E_ARG, "d and d_model must be >= 1");
  if (d != 32 && d != 64 && d != 128) return fail(NYS_E_UNSUPPORTED, "d must be 32, 64 or 128");
  if (d_model % 64 != 0) return fail(NYS_E_UNSUPPORTED, "d_model must be a multiple of 64");
  if ((H * d) % 64 != 0) return fail(NYS_E_UNSUPPORTED, "H*d must be a multiple of 64");
  const long long wide = std::max<long long>(d_model, 3LL * H * d);
  if ((long long)B * n * wide >= (1LL << 31)) return fail(NYS_E_UNSUPPORTED, "tensor too large");
  if (3LL * H * d * d_model >= (1LL << 31)) return fail(NYS_E_UNSUPPORTED, "weights too large");
  return NYS_OK;
}

static nys_status proj_device() {
  static std::once_flag once;
  static nys_status status = NYS_OK;
  static std::string why;
  std::call_once(once, [] {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
      (void)hipGetLastError();
      status = NYS_E_DEVICE;
      why = "no HIP device available";
      return;
    }
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
        std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      status = NYS_E_DEVICE;
      why = "device is not gfx950";
      return;
    }
    if (nys::configure_proj() != hipSuccess) {
      (void)hipGetLastError();
      status = NYS_E_LAUNCH;
      why = "could not set projection kernel LDS limits";
    }
  });
  return status == NYS_OK ? NYS_OK : fail(status, why);
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

extern "C" nys_status nys_proj_qkv(const void* x, const void* w_qkv, void* q, void* k, void* v,
                                   int B, int H, int n, int d, int d_model, void* stream) {
  nys_status st = proj_checks(B, H, n, d, d_model);
  if (st != NYS_OK) return st;
  if (!x || !w_qkv || !q || !k || !v) return fail(NYS_E_ARG, "NULL tensor pointer");
  if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(NYS_E_ARG, "tensors must be 16-byte aligned");
  const size_t xb = (size_t)B * n * d_model * 2, hb = (size_t)B * H * n * d * 2;
  for (const void* o : {q, k, v})
    if (ranges_overlap(o, hb, x, xb) || ranges_overlap(o, hb, w_qkv, (size_t)3 * H * d * d_model * 2))
      return fail(NYS_E_ARG, "q, k, v must not overlap x or w_qkv");
  if ((st = proj_device()) != NYS_OK) return st;
  const nys::ProjArgs a{x, w_qkv, q, k, v, nullptr, B, H, n, d, d_model};
  const hipError_t e = nys::launch_qkv_proj(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(NYS_E_LAUNCH, std::string("qkv projection launch: ") + hipGetErrorString(e));
  return NYS_OK;
}

extern "C" nys_status nys_proj_out(const void* o, const void* w_o, void* y, int B, int H, int n,
                                   int d, int d_model, void* stream) {
  nys_status st = proj_checks(B, H, n, d, d_model);
  if (st != NYS_OK) return st;
  if (!o || !w_o || !y) return fail(NYS_E_ARG, "NULL tensor pointer");
  if (!aligned16(o) || !aligned16(w_o) || !aligned16(y))
    return fail(NYS_E_ARG, "tensors must be 16-byte aligned");
  const size_t yb = (size_t)B * n * d_model * 2;
  if (ranges_overlap(y, yb, o, (size_t)B * H * n * d * 2) ||
      ranges_overlap(y, yb, w_o, (size_t)d_model * H * d * 2))
    return fail(NYS_E_ARG, "y must not overlap o or w_o");
  if ((st = proj_device()) != NYS_OK) return st;
  const nys::ProjArgs a{o, w_o, nullptr, nullptr, nullptr, y, B, H, n, d, d_model};
  const hipError_t e = nys::launch_out_proj(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(NYS_E_LAUNCH, std::string("output projection launch: ") + hipGetErrorString(e));
  return NYS_OK;
}

// ------------------------------------------------------------------ FLASH mixed chunks
static size_t flash_layout(int B, int H, int n, int d, int chunk, int causal, size_t* planes_off) {
  const size_t BH = (size_t)B * H, G = (size_t)ceil_div(n, chunk);
  const size_t states = align256(BH * G * d * d * 4);
  if (planes_off) *planes_off = states;
  return states + align256(BH * (causal ? G : 1) * 2 * d * d * 2);
}

static nys_status flash_checks(int B, int H, int n, int d, int chunk, int causal) {
  if (B < 1 || H < 1 || n < 1) return fail(NYS_E_ARG, "B, H and n must be >= 1");
  if (causal != 0 && causal != 1) return fail(NYS_E_ARG, "causal must be 0 or 1");
  if (chunk < 1) return fail(NYS_E_ARG, "chunk must be >= 1");
  if (d != 32 && d != 64 && d != 128) return fail(NYS_E_UNSUPPORTED, "d must be 32, 64 or 128");
  if (chunk != 64 && chunk != 128 && chunk != 256)
    return fail(NYS_E_UNSUPPORTED, "chunk must be 64, 128 or 256");
  if ((long long)B * H * n * d >= (1LL << 31)) return fail(NYS_E_UNSUPPORTED, "tensor too large");
  return NYS_OK;
}

static nys_status flash_device() {
  static std::once_flag once;
  static nys_status status = NYS_OK;
  static std::string why;
  std::call_once(once, [] {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
      (void)hipGetLastError();
      status = NYS_E_DEVICE;
      why = "no HIP device available";
      return;
    }
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
        std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      status = NYS_E_DEVICE;
      why = "device is not gfx950";
      return;
    }
    if (nys::configure_flash() != hipSuccess) {
      (void)hipGetLastError();
      status = NYS_E_LAUNCH;
      why = "could not set mixed-chunk kernel LDS limits";
    }
  });
  return status == NYS_OK ? NYS_OK : fail(status, why);
}

extern "C" size_t nys_flash_workspace_bytes(int B, int H, int n, int d, int chunk, int causal) {
  if (flash_checks(B, H, n, d, chunk, causal) != NYS_OK) return 0;
  return flash_layout(B, H, n, d, chunk, causal, nullptr);
}

// phase: 1 = chunk states and global sums, 2 = attention, 3 = both
static nys_status flash_run(int phase, const void* q, const void* k, const void* v, void* out,
                            int B, int H, int n, int d, int chunk, int causal, void* ws,
                            size_t ws_bytes, void* stream) {
  nys_status st = flash_checks(B, H, n, d, chunk, causal);
  if (st != NYS_OK) return st;
  if (!k || !v || !ws || ((phase & 2) && (!q || !out))) return fail(NYS_E_ARG, "NULL pointer");
  for (const void* t : {q, k, v, (const void*)out, (const void*)ws})
    if (t && (reinterpret_cast<uintptr_t>(t) & 15u) != 0)
      return fail(NYS_E_ARG, "tensors and workspace must be 16-byte aligned");
  size_t poff = 0;
  const size_t need = flash_layout(B, H, n, d, chunk, causal, &poff);
  if (ws_bytes < need) return fail(NYS_E_ARG, "workspace too small");
  const size_t bytes = (size_t)B * H * n * d * 2;
  if (phase & 2)
    for (const void* in : {q, k, v})
      if (ranges_overlap(out, bytes, in, bytes) || ranges_overlap(out, bytes, ws, need))
        return fail(NYS_E_ARG, "out must not overlap q, k, v or the workspace");
  for (const void* in : {q, k, v})
    if (in && ranges_overlap(ws, need, in, bytes))
      return fail(NYS_E_ARG, "workspace must not overlap q, k or v");
  if ((st = flash_device()) != NYS_OK) return st;
  nys::FlashArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  a.states = reinterpret_cast<float*>(ws);
  a.mplanes = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + poff);
  a.BH = B * H; a.n = n; a.d = d; a.chunk = chunk; a.G = ceil_div(n, chunk); a.causal = causal;
  a.scale = 1.0f / std::sqrt((float)d);
  a.scale_log2e = (float)(1.4426950408889634 / std::sqrt((double)d));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (phase & 1) e = nys::launch_flash_states(a, s);
  if (e == hipSuccess && (phase & 2)) e = nys::launch_flash_attend(a, s);
  if (e != hipSuccess) return fail(NYS_E_LAUNCH, std::string("mixed-chunk launch: ") + hipGetErrorString(e));
  return NYS_OK;
}

extern "C" nys_status nys_flash_states(const void* k, const void* v, int B, int H, int n, int d,
                                       int chunk, int causal, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return flash_run(1, nullptr, k, v, nullptr, B, H, n, d, chunk, causal, workspace,
                   workspace_bytes, stream);
}

extern "C" nys_status nys_flash_attend(const void* q, const void* k, const void* v, void* out,
                                       int B, int H, int n, int d, int chunk, int causal,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  return flash_run(2, q, k, v, out, B, H, n, d, chunk, causal, workspace, workspace_bytes,
                   stream);
}

extern "C" nys_status nys_flash_attention(const void* q, const void* k, const void* v, void* out,
                                          int B, int H, int n, int d, int chunk, int causal,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  return flash_run(3, q, k, v, out, B, H, n, d, chunk, causal, workspace, workspace_bytes,
                   stream);
}

extern "C" const char* nys_attn_last_error(void) { return g_err.c_str(); }
