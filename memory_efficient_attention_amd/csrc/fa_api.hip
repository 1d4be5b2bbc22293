// C ABI: argument validation, workspace layout and kernel dispatch.
//
// Every refusal is decided on the host before any HIP call ("typed refusals,
// never silent fallbacks": mlx-train-perf 0.5.1 README, "If you maintain a
// trainer"), so a refused call launches nothing.  The library allocates no
// memory; the caller passes a workspace sized by fa_workspace_bytes().
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>

#include "fa.h"
#include "fa_internal.h"

#define FA_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kAlign = 256;
constexpr int kMinTile = 32;   // tables are sized for the smallest tile, so any tile config fits

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Layout {
  size_t flag = 0, delta = 0, nls = 0, qtab = 0, ktab = 0, qwork = 0, kwork = 0, total = 0;
};

bool shape_ok(int B, int H, int N) {
  if (B < 1 || H < 1 || N < 1 || N > FA_MAX_N) return false;
  const long long rows = (long long)B * H * N;
  return rows <= INT_MAX;   // B*H*ceil(N/32) workgroups and B*H*N rows fit in int
}

Layout layout(int B, int H, int N, bool has_seg, bool for_bwd) {
  Layout L;
  if (!for_bwd && !has_seg) return L;   // plain forward needs no workspace
  size_t off = kAlign;                  // flag word(s)
  if (for_bwd) {
    const size_t vec = align_up((size_t)B * H * N * sizeof(float));
    L.delta = off;
    off += vec;
    L.nls = off;
    off += vec;
  }
  if (has_seg) {
    const size_t tiles = (size_t)B * ((N + kMinTile - 1) / kMinTile);
    const size_t tab = align_up(tiles * sizeof(int2)), work = align_up(tiles * sizeof(int4));
    L.qtab = off;
    off += tab;
    L.ktab = off;
    off += tab;
    L.qwork = off;
    off += work;
    L.kwork = off;
    off += work;
  }
  L.total = off;
  return L;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Per-device "is gfx950" cache: 0 unknown, 1 yes, 2 no.
std::mutex g_mu;
signed char g_dev_ok[64];
int g_dev_cus[64];   // compute units of each checked device
void* g_scratch_ptr[64];   // device address of `scratch` on each device, once looked up

fa_status device_ok() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return FA_ERR_DEVICE;
  }
  if (dev < 64) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_dev_ok[dev] == 1) return FA_OK;
    if (g_dev_ok[dev] == 2) return FA_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return FA_ERR_DEVICE;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_dev_cus[dev] = prop.multiProcessorCount;
    g_dev_ok[dev] = ok ? 1 : 2;
  }
  return ok ? FA_OK : FA_ERR_DEVICE;
}

// Compute units of the current device once device_ok() has passed (0 if
// unknown, which turns the one-round balancing off).
int device_cus() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 0;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  return g_dev_cus[dev];
}

// Mirrored 32-row blocks (mirror_block in the kernels) for a dense causal
// launch of `wgs` workgroups of `nw` waves over N rows on a device of `cus`
// compute units, when the blocks tile N exactly: the number of rounds of the
// CUs the grid needs (1 or 2), else 0.  Up to two rounds the heaviest
// workgroups set the step time (the two-team dK/dV kernel gains at one round
// only); on larger grids the heaviest-first order packs unequal workgroups as
// well or better.
int use_mirror(bool dense, int causal, int N, int nw, long long wgs, long long cus) {
  if (!dense || !causal || N % (nw * 32) != 0 || cus <= 0 || wgs > 2 * cus) return 0;
  return wgs <= cus ? 1 : 2;
}

fa_status common_checks(int B, int H, int Hkv, int N, int D, fa_dtype dtype, float scale) {
  if (!shape_ok(B, H, N) || Hkv < 1 || H % Hkv != 0) return FA_ERR_SHAPE;
  if (D != 64 && D != 96 && D != 128) return FA_ERR_HEAD_DIM;
  if (dtype != FA_BF16 && dtype != FA_FP32) return FA_ERR_DTYPE;
  // one head's (N, D) matrix is addressed with 32-bit byte offsets
  if ((long long)N * D * (dtype == FA_FP32 ? 4 : 2) >= (1LL << 31)) return FA_ERR_SHAPE;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
  return FA_OK;
}

float log2e_scale(float scale) { return (float)((double)scale * 1.4426950408889634); }

}  // namespace

FA_API size_t fa_workspace_bytes(int B, int H, int N, int D, int has_seg, int for_bwd) {
  if (!shape_ok(B, H, N) || (D != 64 && D != 96 && D != 128)) return 0;
  return layout(B, H, N, has_seg != 0, for_bwd != 0).total;
}

FA_API fa_status fa_fwd(const void* q, const void* k, const void* v, const int32_t* seg, float scale,
                        int causal, void* o, float* lse, int B, int H, int Hkv, int N, int D,
                        fa_dtype dtype, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (fa_status st = common_checks(B, H, Hkv, N, D, dtype, scale)) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(seg, 4))
    return FA_ERR_ALIGN;
  const Layout L = layout(B, H, N, seg != nullptr, false);
  if (L.total > 0) {
    if (!ws || ws_bytes < L.total) return FA_ERR_WORKSPACE;
    if (!aligned(ws, kAlign)) return FA_ERR_ALIGN;
  }
  if (fa_status st = device_ok()) return st;
  (void)hipGetLastError();

  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  const int dt = dtype == FA_BF16 ? 0 : 1;
  fa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.seg = seg;
  p.work = seg ? (const int4*)(w + L.qwork) : nullptr;
  p.B = B;
  p.H = H;
  p.G = H / Hkv;
  p.N = N;
  const int nw = fa::tile_config(seg != nullptr, Hkv != H).nw_q;
  const int bm = nw * 32;   // queries per workgroup
  p.nqt = (N + bm - 1) / bm;
  p.mirror = use_mirror(seg == nullptr, causal, N, nw, (long long)B * H * p.nqt, device_cus());
  p.scale = scale;
  p.c = log2e_scale(scale);
  if (seg) {
    fa::TableJobs tj{};
    fa::OrderJobs oj{};
    tj.j[0] = {(int2*)(w + L.qtab), bm, fa::KEY_TILE, 0};
    oj.j[0] = {(const int2*)(w + L.qtab), p.nqt, (int4*)(w + L.qwork), 1};
    if (fa::launch_schedule(seg, B, N, causal != 0, tj, oj, 1, (int32_t*)(w + L.flag), s) != hipSuccess)
      return FA_ERR_HIP;
  }
  if (fa::launch_fwd(p, dt, D, causal != 0, nw, s) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

// Backward workspace of fa_bwd_noalloc: a fixed array in device memory,
// one copy per GPU, alive until the process ends.  Host code never uses its
// name as an address (on the host the name is only a stand-in); the device
// address comes from hipGetSymbolAddress, per device.
static __device__ __attribute__((aligned(256))) char scratch[FA_NOALLOC_MAX_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up on the first
// call there and kept; nullptr if the lookup fails.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

bool record(void* const* events, int i, hipStream_t s) {
  if (!events || !events[i]) return true;
  return hipEventRecord((hipEvent_t)events[i], s) == hipSuccess;
}

fa_status bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dO,
                   const float* lse, const int32_t* seg, float scale, int causal, void* dq, void* dk,
                   void* dv, int B, int H, int Hkv, int N, int D, fa_dtype dtype, void* ws,
                   size_t ws_bytes, void* stream, void* const* events) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  if (fa_status st = common_checks(B, H, Hkv, N, D, dtype, scale)) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dO, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(seg, 4))
    return FA_ERR_ALIGN;
  const Layout L = layout(B, H, N, seg != nullptr, true);
  if (!ws || ws_bytes < L.total) return FA_ERR_WORKSPACE;
  if (!aligned(ws, kAlign)) return FA_ERR_ALIGN;
  if (fa_status st = device_ok()) return st;
  (void)hipGetLastError();

  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  const int dt = dtype == FA_BF16 ? 0 : 1;
  float* delta = (float*)(w + L.delta);
  float* nls = (float*)(w + L.nls);

  const fa::TileConfig cfg = fa::tile_config(seg != nullptr, Hkv != H);
  const int nw = cfg.nw_q, nw_kv = cfg.nw_kv;
  const int bt = nw * 32;   // queries per dQ workgroup
  const int ntiles = (N + bt - 1) / bt;
  const int ntiles_kv = (N + nw_kv * 32 - 1) / (nw_kv * 32);
  if (seg) {
    // query tiles of dQ (and the segment-order check), key tiles of dK/dV
    fa::TableJobs tj{};
    fa::OrderJobs oj{};
    tj.j[0] = {(int2*)(w + L.qtab), bt, fa::KEY_TILE, 0};
    tj.j[1] = {(int2*)(w + L.ktab), nw_kv * 32, fa::QRY_TILE, 1};
    oj.j[0] = {(const int2*)(w + L.qtab), ntiles, (int4*)(w + L.qwork), 1};
    oj.j[1] = {(const int2*)(w + L.ktab), ntiles_kv, (int4*)(w + L.kwork), 0};
    if (fa::launch_schedule(seg, B, N, causal != 0, tj, oj, 2, (int32_t*)(w + L.flag), s) != hipSuccess)
      return FA_ERR_HIP;
  }

  fa::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.dO = dO;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.o = o;
  p.lse = lse;
  p.nls = nls;
  p.delta = delta;
  p.seg = seg;
  p.B = B;
  p.H = H;
  p.G = H / Hkv;
  p.N = N;
  p.scale = scale;
  p.c = log2e_scale(scale);
  const int cus = device_cus();

  // dQ first: it also writes -D_i and -LSE / scale for its rows, which
  // dK/dV then reads
  if (!record(events, 0, s)) return FA_ERR_HIP;
  p.work = seg ? (const int4*)(w + L.qwork) : nullptr;
  p.ntiles = ntiles;
  p.mirror = use_mirror(seg == nullptr, causal, N, nw, (long long)B * H * ntiles, cus);
  if (fa::launch_bwd_dq(p, dt, D, causal != 0, nw, s) != hipSuccess) return FA_ERR_HIP;

  if (!record(events, 1, s)) return FA_ERR_HIP;
  p.work = seg ? (const int4*)(w + L.kwork) : nullptr;
  p.ntiles = ntiles_kv;
  // (the kernel applies it to ungrouped heads and two-team workgroups)
  p.mirror = use_mirror(seg == nullptr, causal, N, nw_kv, (long long)B * Hkv * ntiles_kv, cus);
  if (fa::launch_bwd_dkdv(p, dt, D, causal != 0, nw_kv, s) != hipSuccess) return FA_ERR_HIP;
  if (!record(events, 2, s)) return FA_ERR_HIP;
  return FA_OK;
}

}  // namespace

FA_API fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                        const float* lse, const int32_t* seg, float scale, int causal, void* dq, void* dk,
                        void* dv, int B, int H, int Hkv, int N, int D, fa_dtype dtype, void* ws,
                        size_t ws_bytes, void* stream) {
  return bwd_impl(q, k, v, o, dO, lse, seg, scale, causal, dq, dk, dv, B, H, Hkv, N, D, dtype, ws, ws_bytes,
                  stream, nullptr);
}

FA_API fa_status fa_bwd_timed(const void* q, const void* k, const void* v, const void* o, const void* dO,
                              const float* lse, const int32_t* seg, float scale, int causal, void* dq,
                              void* dk, void* dv, int B, int H, int Hkv, int N, int D, fa_dtype dtype,
                              void* ws, size_t ws_bytes, void* stream, void* const* events) {
  return bwd_impl(q, k, v, o, dO, lse, seg, scale, causal, dq, dk, dv, B, H, Hkv, N, D, dtype, ws, ws_bytes,
                  stream, events);
}

FA_API fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                                const float* lse, const int32_t* seg, float scale, int causal, void* dq,
                                void* dk, void* dv, int B, int H, int Hkv, int N, int D, fa_dtype dtype,
                                void* stream) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  if (fa_status st = common_checks(B, H, Hkv, N, D, dtype, scale)) return st;
  if (layout(B, H, N, seg != nullptr, true).total > FA_NOALLOC_MAX_BYTES) return FA_ERR_SCRATCH;
  if (fa_status st = device_ok()) return st;
  void* ws = device_scratch();
  if (!ws) return FA_ERR_HIP;
  return bwd_impl(q, k, v, o, dO, lse, seg, scale, causal, dq, dk, dv, B, H, Hkv, N, D, dtype, ws,
                  FA_NOALLOC_MAX_BYTES, stream, nullptr);
}

// ---------------------------------------------------------------- linear cross-entropy
namespace {

struct LceLayout {
  size_t part = 0, dz = 0, dh32 = 0, total = 0;
};

fa_status lce_checks(int N, int V, int D, fa_dtype dtype) {
  if (N < 1 || V < 1 || D < 1) return FA_ERR_SHAPE;
  if (D % 256 != 0) return FA_ERR_SHAPE;
  const long long lim = 1LL << 30;
  if ((long long)V * D >= lim || (long long)N * D >= lim || (long long)N * FA_LCE_VOCAB_CHUNK >= lim)
    return FA_ERR_SHAPE;
  if (dtype != FA_BF16) return FA_ERR_DTYPE;
  return FA_OK;
}

LceLayout lce_layout(int N, int V, int D, bool for_bwd) {
  LceLayout L;
  if (!for_bwd) {
    L.part = 0;
    L.total = align_up((size_t)((V + 255) / 256) * N * 2 * sizeof(float));
    return L;
  }
  L.dz = 0;
  size_t off = align_up((size_t)N * FA_LCE_VOCAB_CHUNK * 2);
  L.dh32 = off;
  if (V > FA_LCE_VOCAB_CHUNK) off += align_up((size_t)N * D * sizeof(float));
  L.total = off;
  return L;
}

}  // namespace

FA_API size_t fa_lce_workspace_bytes(int N, int V, int D, int for_bwd) {
  if (lce_checks(N, V, D, FA_BF16) != FA_OK) return 0;
  return lce_layout(N, V, D, for_bwd != 0).total;
}

FA_API fa_status fa_lce_fwd(const void* h, const void* w, const int32_t* targets, float* nll, float* lse,
                            float* tlogit, int N, int V, int D, fa_dtype dtype, void* ws, size_t ws_bytes,
                            void* stream) {
  if (!h || !w || !targets || !nll || !lse || !tlogit) return FA_ERR_NULL;
  if (fa_status st = lce_checks(N, V, D, dtype)) return st;
  if (!aligned(h, 16) || !aligned(w, 16) || !aligned(targets, 4) || !aligned(nll, 4) || !aligned(lse, 4) ||
      !aligned(tlogit, 4))
    return FA_ERR_ALIGN;
  const LceLayout L = lce_layout(N, V, D, false);
  if (!ws || ws_bytes < L.total) return FA_ERR_WORKSPACE;
  if (!aligned(ws, kAlign)) return FA_ERR_ALIGN;
  if (fa_status st = device_ok()) return st;
  (void)hipGetLastError();
  fa::LceParams p{};
  p.h = h;
  p.w = w;
  p.targets = targets;
  p.nll = nll;
  p.lse = lse;
  p.tlogit = tlogit;
  p.part = (float*)((char*)ws + L.part);
  p.N = N;
  p.V = V;
  p.D = D;
  return fa::launch_lce_fwd(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

FA_API fa_status fa_lce_bwd(const void* h, const void* w, const int32_t* targets, const float* lse,
                            const float* dnll, void* dh, void* dw, int N, int V, int D, fa_dtype dtype,
                            void* ws, size_t ws_bytes, void* stream) {
  if (!h || !w || !targets || !lse || !dnll || !dh) return FA_ERR_NULL;
  if (fa_status st = lce_checks(N, V, D, dtype)) return st;
  if (!aligned(h, 16) || !aligned(w, 16) || !aligned(dh, 16) || !aligned(dw, 16) || !aligned(targets, 4) ||
      !aligned(lse, 4) || !aligned(dnll, 4))
    return FA_ERR_ALIGN;
  const LceLayout L = lce_layout(N, V, D, true);
  if (!ws || ws_bytes < L.total) return FA_ERR_WORKSPACE;
  if (!aligned(ws, kAlign)) return FA_ERR_ALIGN;
  if (fa_status st = device_ok()) return st;
  (void)hipGetLastError();
  fa::LceParams p{};
  p.h = h;
  p.w = w;
  p.targets = targets;
  p.lse_in = lse;
  p.dnll = dnll;
  p.dz = (char*)ws + L.dz;
  p.dh32 = (float*)((char*)ws + L.dh32);
  p.dh = dh;
  p.dw = dw;
  p.N = N;
  p.V = V;
  p.D = D;
  return fa::launch_lce_bwd(p, FA_LCE_VOCAB_CHUNK, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

FA_API fa_status fa_check_seg(const int32_t* host_seg, int B, int N) {
  if (!host_seg) return FA_ERR_NULL;
  if (B < 1 || N < 1 || N > FA_MAX_N) return FA_ERR_SHAPE;
  for (long long b = 0; b < B; ++b) {
    const int32_t* r = host_seg + b * N;
    for (int i = 0; i + 1 < N; ++i)
      if (r[i] > r[i + 1]) return FA_ERR_SEG;
  }
  return FA_OK;
}

FA_API const char* fa_status_string(fa_status status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H or N out of range";
    case FA_ERR_HEAD_DIM: return "head_dim must be 64, 96 or 128";
    case FA_ERR_DTYPE: return "dtype must be bf16 or fp32";
    case FA_ERR_WORKSPACE: return "workspace missing or smaller than fa_workspace_bytes()";
    case FA_ERR_ALIGN: return "pointer misaligned (tensors 16 B, lse/seg 4 B, workspace 256 B)";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_SEG: return "segment ids decrease along a row";
    case FA_ERR_HIP: return "HIP launch failed";
    case FA_ERR_DEVICE: return "current device is not a gfx950 GPU";
    case FA_ERR_SCRATCH: return "shape needs more workspace than fa_bwd_noalloc's static scratch (FA_NOALLOC_MAX_BYTES)";
  }
  return "unknown status";
}
