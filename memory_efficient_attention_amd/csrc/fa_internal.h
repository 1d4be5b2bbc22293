// Host<->kernel parameter blocks, tile sizes and launcher declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Tile sizes.  Forward: one workgroup owns FWD_WAVES waves x FWD_QBW blocks
// of 32 queries and walks key tiles of KEY_TILE keys; each K / V fragment
// read from LDS feeds FWD_QBW MFMAs.  dQ: DQ_WAVES waves x 32 queries, same
// key tiles.  dK/dV: DKV_WAVES waves x 32 keys, walking query tiles of
// QRY_TILE queries.  Each can be overridden at build time with
// -DFA_<NAME>=value for tuning.
#ifndef FA_FWD_WAVES
#define FA_FWD_WAVES 8
#endif
#ifndef FA_FWD_QBW
#define FA_FWD_QBW 1
#endif
#ifndef FA_DQ_WAVES
#define FA_DQ_WAVES 8
#endif
#ifndef FA_KEY_TILE
#define FA_KEY_TILE 64
#endif
#ifndef FA_DKV_WAVES
#define FA_DKV_WAVES 8
#endif
#ifndef FA_QRY_TILE
#define FA_QRY_TILE 32
#endif
// Waves per SIMD each kernel is compiled for (its register budget is 512 /
// this): the register-blocked forward needs one wave per SIMD, dQ and dK/dV
// run two.
#ifndef FA_FWD_WPE
#define FA_FWD_WPE (FA_FWD_QBW > 1 ? 1 : 2)
#endif
#ifndef FA_WAVES_PER_EU
#define FA_WAVES_PER_EU 2
#endif
constexpr int FWD_WAVES = FA_FWD_WAVES;
constexpr int FWD_QBW = FA_FWD_QBW;
constexpr int FWD_BM = FWD_WAVES * 32 * FWD_QBW;
constexpr int DQ_WAVES = FA_DQ_WAVES;
constexpr int DQ_BM = DQ_WAVES * 32;
constexpr int KEY_TILE = FA_KEY_TILE;
constexpr int DKV_WAVES = FA_DKV_WAVES;
constexpr int DKV_BN = DKV_WAVES * 32;
constexpr int QRY_TILE = FA_QRY_TILE;

// Online-softmax reference max: moved only when a row's max exceeds it by
// more than this many powers of two, so the O accumulator is rescaled rarely;
// unnormalised probabilities stay below 2^RESCALE_LOG2.
constexpr float RESCALE_LOG2 = 8.f;

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* seg;    // (B, N) or null
  const int2* qtab;      // per query tile: [first, last] key tile (packed only)
  int B, H, N, nqt;
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
  const float* lse2;     // log2-domain LSE (B, H, N)
  const float* delta;    // -D_i = -dO_i . O_i (B, H, N)
  const int32_t* seg;
  const int2* tab;       // dQ: per query tile key-tile range; dK/dV: per key tile query-tile range
  int B, H, N, ntiles;
  float scale, c;
};

struct PreParams {
  const void* o;
  const void* dO;
  const float* lse;
  float* delta;
  float* lse2;
  long long rows;
};

// Launchers (defined next to their kernels).  dtype: 0 bf16, 1 fp32.
hipError_t launch_fwd(const FwdParams& p, int dtype, int D, bool causal, hipStream_t s);
hipError_t launch_bwd_pre(const PreParams& p, int dtype, int D, hipStream_t s);
hipError_t launch_bwd_dq(const BwdParams& p, int dtype, int D, bool causal, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdParams& p, int dtype, int D, bool causal, hipStream_t s);
// Per-tile range tables from segment ids (see fa_sched.hip).
hipError_t launch_qtile_table(const int32_t* seg, int B, int N, int tq, int tk, bool causal,
                              int2* tab, hipStream_t s);
hipError_t launch_ktile_table(const int32_t* seg, int B, int N, int tk, int tq, bool causal,
                              int2* tab, hipStream_t s);
hipError_t launch_seg_check(const int32_t* seg, int B, int N, int32_t* flag, hipStream_t s);

}  // namespace fa
