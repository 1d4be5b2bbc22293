// Host<->kernel parameter blocks, tile sizes and launcher declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Tile sizes.  A workgroup of NW waves owns NW x 32 queries (forward, dQ)
// or keys (dK/dV); the forward and dQ walk key tiles of KEY_TILE keys, dK/dV
// walks query tiles of QRY_TILE queries.  Every wave does the same
// arithmetic in the same order whatever NW is, so the choice of NW never
// changes a result bit.  Dense (causal or full) calls use WAVES_DENSE waves,
// whose one staged tile feeds the most waves; packed calls use WAVES_PACKED,
// whose smaller workgroups track short segments more closely and keep two
// workgroups per CU in flight.
constexpr int WAVES_DENSE = 8;
constexpr int WAVES_PACKED = 4;
constexpr int KEY_TILE = 64;
constexpr int QRY_TILE = 32;
// Waves per SIMD the attention kernels are compiled for (their register
// budget is 512 / this per lane).
constexpr int WAVES_PER_EU = 2;
// Load pipeline depth of every attention kernel: one tile staged ahead of
// the one in use.  Measured on MI355X, deeper rings gain nothing here
// (within 1 %), and the dK/dV kernel, at the 256-register limit, spills
// with three stages.
constexpr int STAGES = 2;
// Two tiles per ring slot in the 8-wave bf16 kernels of dense calls: key
// tiles in the forward and dQ (KSUB), query tiles in multi-head dK/dV
// (QSUB).
constexpr int KSUB_DENSE = 2;
constexpr int QSUB_DENSE = 2;
constexpr int LDS_PER_CU = 163840;
constexpr int WAVES_PER_CU = 4 * WAVES_PER_EU;

// Tile configuration by call mode: waves per workgroup of the forward and
// dQ (nw_q) and of dK/dV (nw_kv).  Where the mlx-train-perf README ("Turning
// it on", "Training packed") calibrates its kernels with a host-synced timing
// probe cached per batch size and sequence bucket, this is a fixed table,
// measured offline on MI355X: calls are deterministic and capturable, and no
// probe runs.  Every wave does the same arithmetic whatever the entry, so a
// packed call with a single segment gives the causal call's bits.
//   dense (causal or full), multi-head: 8 / 8 waves
//   packed:                             4 / 4 waves (short segments, many
//                                       small workgroups per CU)
//   dense, grouped-query heads:         8 / 4 waves (two-team dK/dV for even
//                                       groups: 8-wave workgroups of 128 keys)
// The key is the mode, not the size: A/B runs of 4- against 8-wave
// workgroups for every class at several sizes (2k to 64k rows, head_dim 64
// to 128) found no size at which the other choice wins by more than noise,
// and a size-keyed choice of key-tile length is ruled out because the host
// cannot tell a packed call's segment lengths (they are device data) while a
// single-segment packed call must keep the causal call's tile order.
struct TileConfig {
  int nw_q, nw_kv;
};
constexpr TileConfig tile_config(bool packed, bool grouped) {
  return {packed ? WAVES_PACKED : WAVES_DENSE, packed || grouped ? WAVES_PACKED : WAVES_DENSE};
}

// Stages a kernel of NW waves uses: the requested depth, reduced to what
// fits its share of the CU's LDS (WAVES_PER_CU / NW workgroups share a CU)
// at `per_stage` bytes per stage (fp32 tiles are twice as large).
constexpr int stages_for(int requested, int per_stage, int nw) {
  const int share = LDS_PER_CU / (WAVES_PER_CU >= nw ? WAVES_PER_CU / nw : 1);
  const int fit = share / per_stage;
  // two stages at least, even if that leaves fewer workgroups per CU
  return requested < fit ? requested : (fit > 2 ? fit : 2);
}

// Online softmax with a lazily moved reference: probabilities are taken
// against a per-row reference that moves only when a row's partial sum of
// unnormalised probabilities in one tile reaches this bound (so every
// probability stays below it) or the row has no reference yet.
constexpr float GROW_LIMIT = 65536.f;

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* seg;    // (B, N) or null
  // packed only: {b, query tile, first key tile, last key tile} per query
  // tile, longest first; workgroup w runs head w % H of entry w / H
  const int4* work;
  int B, H, N, nqt;
  int G;                 // query heads per key/value head (H / Hkv)
  int mirror;            // dense causal: mirrored 32-row blocks (mirror_block)
                         // when nonzero; the grid's rounds of CUs (1 or 2)
  float scale;           // softmax scale
  float c;               // scale * log2(e)
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dO;
  void* dq;
  void* dk;
  void* dv;
  const void* o;         // the forward's output (dQ: D_i = dO_i . O_i)
  const float* lse;      // the forward's log-sum-exp (dQ)
  float* nls;            // -LSE / scale (B, H, N): written by dQ, read by dK/dV
  float* delta;          // -D_i = -dO_i . O_i (B, H, N): written by dQ, read by dK/dV
  const int32_t* seg;
  // packed only, longest first: dQ {b, query tile, first, last key tile};
  // dK/dV {b, key tile, first, last query tile}; workgroup w runs head
  // w % H of entry w / H
  const int4* work;
  int B, H, N, ntiles;
  int G;                 // query heads per key/value head (H / Hkv)
  int mirror;            // as in FwdParams
  float scale, c;
};

// Causal grids of one or two rounds of the chip's CUs last as long as their
// heaviest workgroups (last query tile, or first key tile).  There,
// workgroup t of a head (of nt, nt * NW * 32 = N rows) gives its first NW / 2
// waves the 32-row blocks t NW / 2 + w and the others the mirrored blocks
// from the far end, so all workgroups carry the same visible work.  Every row
// is still walked in the same order.
__device__ __forceinline__ int mirror_block(int t, int w, int nw, int nt) {
  const int half = nw / 2, x = t * half + w % half;
  return w < half ? x : nt * nw - 1 - x;
}

// Fused linear cross-entropy (bf16 H (N, D), W (V, D)).
struct LceParams {
  const void* h;
  const void* w;
  const int32_t* targets;
  float* nll;            // forward outputs (N,)
  float* lse;
  float* tlogit;
  float* part;           // forward workspace: (ceil(V / 256), N) float2 partial (max, sum)
  const float* lse_in;   // backward inputs (N,)
  const float* dnll;
  void* dz;              // backward workspace: (N, VC) bf16
  float* dh32;           // backward workspace: (N, D) fp32 accumulator (several chunks)
  void* dh;              // (N, D) bf16
  void* dw;              // (V, D) bf16 or null
  int N, V, D;
};
hipError_t launch_lce_fwd(const LceParams& p, hipStream_t s);
hipError_t launch_lce_bwd(const LceParams& p, int vc, hipStream_t s);

// Launchers (defined next to their kernels).  dtype: 0 bf16, 1 fp32; nw:
// waves per workgroup, WAVES_DENSE or WAVES_PACKED.
hipError_t launch_fwd(const FwdParams& p, int dtype, int D, bool causal, int nw, hipStream_t s);
hipError_t launch_bwd_dq(const BwdParams& p, int dtype, int D, bool causal, int nw, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdParams& p, int dtype, int D, bool causal, int nw, hipStream_t s);

// Calls f(type_c<T>, int_c<D>, bool_c<CAUSAL>, int_c<NW>) for the runtime
// (dtype, D, causal, nw), so each launcher names its kernel template once.
template <typename T> struct type_c { using type = T; };
template <int V> struct int_c { static constexpr int value = V; };
template <bool V> struct bool_c { static constexpr bool value = V; };
template <typename F>
hipError_t dispatch(int dtype, int D, bool causal, int nw, F&& f) {
  auto by_nw = [&](auto t, auto d, auto c) {
    return nw == WAVES_PACKED ? f(t, d, c, int_c<WAVES_PACKED>{}) : f(t, d, c, int_c<WAVES_DENSE>{});
  };
  auto by_causal = [&](auto t, auto d) {
    return causal ? by_nw(t, d, bool_c<true>{}) : by_nw(t, d, bool_c<false>{});
  };
  auto by_d = [&](auto t) {
    if (D == 128) return by_causal(t, int_c<128>{});
    return D == 96 ? by_causal(t, int_c<96>{}) : by_causal(t, int_c<64>{});
  };
  return dtype == 0 ? by_d(type_c<__bf16>{}) : by_d(type_c<float>{});
}
// Packed-row schedule (fa_sched.hip): for one or two jobs in one pair of
// launches, per-tile visible ranges from segment ids, then a longest-first
// work list {b, tile, first, last} per table.
struct TableJob {
  int2* tab;     // out: B x ceil(N / tile) {first, last}
  int tile;      // rows per tile of this table (queries, or keys if `keys`)
  int other;     // rows per tile of the ranges (keys, or queries if `keys`)
  int keys;      // 0: query tiles -> key-tile ranges; 1: key tiles -> query-tile ranges
};
struct OrderJob {
  const int2* tab;   // a table of B x nt tiles
  int nt;
  int4* work;        // out: B x nt entries, longest range first
  int check;         // also raise flag[0] if a row's ids decrease (one job at most)
};
struct TableJobs {
  TableJob j[2];
};
struct OrderJobs {
  OrderJob j[2];
};
hipError_t launch_schedule(const int32_t* seg, int B, int N, bool causal, const TableJobs& tables,
                           const OrderJobs& orders, int njobs, int32_t* flag, hipStream_t s);

}  // namespace fa
