// Fused linear cross-entropy: the loss layer of a language model without the
// (N, V) logits tensor.
//
// What is computed follows the mlx-train-perf README, section "The fused
// cross-entropy loss": for hidden states H (N, D), a dense head W (V, D) and
// targets t, the forward regenerates the logits Z = H W^T tile by tile and
// returns three N-length arrays, the per-token NLL, log-sum-exp and target
// logit; the backward recomputes the tiles it needs instead of reading a
// stored matrix (README, section "Implementations": the backward the kernel
// forward pairs with processes the vocabulary in fixed tiles).  With upstream
// per-token gradients g, dZ = g (softmax(Z) - onehot(t)), dH = dZ W and
// dW = dZ^T H.
//
// All products run on one MFMA GEMM core: a workgroup of 8 waves computes a
// 256 x 256 tile C = A B (C rows "M", columns "N") with the contraction
// streamed through LDS in K-slices of TK = 64, each wave a 64 x 128 block
// (2 x 4 MFMA tiles of 32 x 32).  Accumulators use the MFMA layout with lane = N
// column, so per-column statistics (a token's log-sum-exp) stay in a lane
// pair.  Operands come from LDS either along rows (a 256 x TK slice of a
// row-major matrix whose rows are the M or N index) or transposed (a TK x 256
// slice whose rows are the K index), matching k-slot orders pairwise:
//   forward and dZ:  Z^T  = W   H^T    (A rows of W, B rows of H)
//   dH:              dH^T = W^T dZ^T   (A transposed W, B rows of dZ)
//   dW:              dW^T = H^T dZ     (A transposed H, B transposed dZ)
// The transposed read delivers a lane's 8 k-slots of a 16-wide step in the
// order {4h..4h+3, 8+4h..8+4h+3} (h = lane / 32).  dZ is an intermediate of
// our own, so it is stored with the two middle 4-column groups of every 16
// swapped (dz_pos): a plain 16-byte row read of it then yields exactly that
// order, and dH pairs it with transposed W without a split read.
// The backward walks the vocabulary in chunks of VC: per chunk, dZ for all
// tokens is written to a workspace (N x VC bf16), then dH accumulates in an
// fp32 workspace and dW of the chunk's vocabulary rows is written out.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

// Per-wave block WM x WN (MB x NB MFMA tiles of 32 x 32): 64 x 128, 8 waves
// at 2 per SIMD.  (128 x 128 blocks at one wave per SIMD, with 2/3 of the
// LDS reads per MFMA, measured 4 % slower.)  The contraction is staged in
// slices of TK = 64 through a ring of 2 stages.
constexpr int TM = 256, TN = 256, TK = 64;   // contraction slice per stage
constexpr int WM = 64, WN = 128;
constexpr int MB = WM / 32, NB = WN / 32;
constexpr int WAVES_M = TM / WM, WAVES_N = TN / WN, NWV = WAVES_M * WAVES_N;
constexpr int WPE = NWV >= 8 ? 2 : 1;          // waves per SIMD the registers allow
constexpr int LCE_STAGES = 2;
static_assert(WM == 64 || WM == 128, "per-wave block");
static_assert(LCE_STAGES >= 2 && LCE_STAGES <= 4, "stage ring");
static_assert(TK == 32 || TK == 64, "contraction slice");
using LRow = Layout<bf16, TK, false>;     // 256 rows x TK elements
using LCol = Layout<bf16, TM, true>;      // TK rows x 256 elements (transposed reads)
using StRow = Stager<bf16, TM, TK, NWV, false>;
using StCol = Stager<bf16, TK, TM, NWV, true>;
constexpr int ROW_TILE = LRow::bytes(TM);
constexpr int COL_TILE = LCol::bytes(TK);
constexpr int TILE_MAX = ROW_TILE > COL_TILE ? ROW_TILE : COL_TILE;
static_assert(TM == TN, "square C tiles");

// Grouped order of a (mt x nt) grid of C tiles: runs of 8 M tiles sweep all
// N tiles, so the workgroups resident on one XCD at a time share their
// operand slices in its L2.  `L` comes through xcd_remap.
__device__ __forceinline__ void tile_of(int L, int mt, int nt, int& tm, int& tn) {
  constexpr int GM = 8;
  const int group = L / (GM * nt);
  const int first = group * GM;
  const int gm = min(mt - first, GM);
  const int r = L - group * GM * nt;
  tm = first + r % gm;
  tn = r / gm;
}

enum Operand { ROWS, COLS };

// Complete this wave's LDS reads.  A barrier does not wait for them, and the
// LDS unit orders them only against other LDS instructions, not against the
// direct global->LDS loads another wave issues after the barrier; the GEMM
// loop carries fragments read from a stage buffer across the barrier that
// frees that buffer, so it drains them first.
__device__ __forceinline__ void lds_drain() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Storage position of dZ column j within its chunk: bits 2 and 3 swapped
// (an involution, so it also maps a stored position back to its column).
__device__ __forceinline__ int dz_pos(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }

// The GEMM core.  A (M x K) and B (K x N) are staged per K-slice by
// stage_a(tile, k0) / stage_b(tile, k0) and read as `OA` / `OB` operands;
// acc[mb][nb] is the wave's MB x NB block of 32 x 32 tiles.  The ring holds
// LCE_STAGES K-slices; slice s + LCE_STAGES - 1 is issued halfway through
// slice s, into slice s - 1's buffer (free since the barrier).  Every slice
// ends at a workgroup barrier, where both waves of a SIMD stop together; so
// the MFMAs of each slice's last 16-wide step are issued only after the next
// barrier, where they keep the matrix unit busy while the new slice's first
// fragments come from LDS.  The order of the MFMAs on each accumulator is
// unchanged.
template <Operand OA, Operand OB, typename SA, typename SB>
__device__ __forceinline__ void gemm_tile(FA_LDS char* smem, int nk, SA&& stage_a, SB&& stage_b,
                                          f32x16 (&acc)[MB][NB], int wave, int lane) {
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  // load instructions per wave per slice, at least (both tiles' stagers deal
  // round-robin as one set)
  constexpr int LPT = (StRow::NINST > StCol::NINST ? StCol::NINST : StRow::NINST) * 2 / NWV;
  constexpr int KS = TK / 16;
  const int rbase = LRow::row_base(lane);
  const int cbase = LCol::col_base(lane);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x16{};
  auto stage = [&](int s, int buf) {
    stage_a(smem + buf * 2 * TILE_MAX, s * TK);
    stage_b(smem + buf * 2 * TILE_MAX + TILE_MAX, s * TK);
  };
  auto read = [&](const FA_LDS char* ta, const FA_LDS char* tb, int ks, bf16x8 (&a)[MB], bf16x8 (&b)[NB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if constexpr (OA == ROWS) a[mb] = frag_row<bf16, TK, false>(ta, rbase, WM * wm + 32 * mb, ks);
      else a[mb] = frag_col<bf16, TM>(ta, cbase, 16 * ks, WM * wm + 32 * mb);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (OB == ROWS) b[nb] = frag_row<bf16, TK, false>(tb, rbase, WN * wn + 32 * nb, ks);
      else b[nb] = frag_col<bf16, TN>(tb, cbase, 16 * ks, WN * wn + 32 * nb);
    }
  };
  auto mmas = [&](const bf16x8 (&a)[MB], const bf16x8 (&b)[NB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) mma(acc[mb][nb], a[mb], b[nb]);
  };
#pragma unroll
  for (int s = 0; s < LCE_STAGES - 1; ++s)
    if (s < nk) stage(s, s);
  bf16x8 pa[MB], pb[NB];   // the previous slice's last step, not yet multiplied
  int buf = 0;
  for (int s = 0; s < nk; ++s) {
    // slices s + 1 .. s + LCE_STAGES - 2 may stay in flight
    wait_tiles<LPT, LCE_STAGES - 2>(min(nk - 1 - s, LCE_STAGES - 2));
    lds_drain();   // pa / pb were read from the buffer this barrier frees
    __syncthreads();
    // The next slice's loads go out halfway through this slice's steps (its
    // buffer is free since the barrier): issued at the barrier, every wave's
    // loads left together with its first fragment reads (forward 5 % and
    // backward 3-4 % slower, measured); at the last step, too late.
    const bool more = s + LCE_STAGES - 1 < nk;
    const int nbuf = buf == 0 ? LCE_STAGES - 1 : buf - 1;
    const FA_LDS char* ta = smem + buf * 2 * TILE_MAX;
    const FA_LDS char* tb = ta + TILE_MAX;
    buf = buf + 1 == LCE_STAGES ? 0 : buf + 1;
    bf16x8 a[MB], b[NB];
    read(ta, tb, 0, a, b);
    if (s > 0) mmas(pa, pb);
#pragma unroll
    for (int ks = 1; ks < KS; ++ks) {
      if (ks == KS / 2 && more) stage(s + LCE_STAGES - 1, nbuf);
      bf16x8 a2[MB], b2[NB];
      read(ta, tb, ks, a2, b2);
      mmas(a, b);
      // the next step's fragment reads one after each of this step's MFMAs
      // (the compiler's own order waited for them right before use:
      // forward 1 % and backward 1 % slower, measured)
#pragma unroll
      for (int i = 0; i < MB * NB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < MB + NB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) a[mb] = a2[mb];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) b[nb] = b2[nb];
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) pa[mb] = a[mb];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) pb[nb] = b[nb];
  }
  if (nk > 0) mmas(pa, pb);
  __syncthreads();   // the staging buffers may be reused by the epilogue
}

}  // namespace

// ---------------------------------------------------------------- forward
// One workgroup per (vocabulary tile vt, token tile tt): Z^T for 256 vocabulary
// rows x 256 tokens over the full hidden size, then per token the tile's max
// and exp-sum (log2 domain) into part[vt][token], and the target logit where
// the tile holds it.
__global__ void __launch_bounds__(NWV * 64, WPE) lce_fwd_kernel(const LceParams p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * LCE_STAGES * TILE_MAX];
  FA_LDS char* smem = (FA_LDS char*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  const int nvt = (p.V + TM - 1) / TM, ntt = (p.N + TN - 1) / TN;
  int vt, tt;
  tile_of(xcd_remap(blockIdx.x, nvt * ntt), nvt, ntt, vt, tt);
  const int v0 = vt * TM, t0 = tt * TN;
  const int ld = p.D * 2;

  StRow sa, sb;
  sa.init(wave, lane);
  sb.init(wave, lane, StRow::NINST);
  f32x16 acc[MB][NB];
  gemm_tile<ROWS, ROWS>(
      smem, p.D / TK,
      [&](FA_LDS char* t, int k0) { sa.issue_block(t, p.w, v0, p.V, ld, k0 * 2); },
      [&](FA_LDS char* t, int k0) { sb.issue_block(t, p.h, t0, p.N, ld, k0 * 2); }, acc, wave, lane);

  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  float* stat = (float*)smem_raw;   // [WAVES_M][256 tokens][2]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int tl = WN * wn + 32 * nb + col;   // token within the tile
    const int tok = t0 + tl;
    const int tgt = tok < p.N ? p.targets[tok] : -1;
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = v0 + WM * wm + 32 * mb + 8 * (r >> 2) + 4 * h + (r & 3);
        const float z = acc[mb][nb][r];
        if (v == tgt) p.tlogit[tok] = z;
        mx = v < p.V ? fmaxf(mx, z) : mx;
      }
    mx = fmaxf(mx, other_half(mx));
    float sum = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = v0 + WM * wm + 32 * mb + 8 * (r >> 2) + 4 * h + (r & 3);
        sum += v < p.V ? exp2_fast((acc[mb][nb][r] - mx) * kLog2e) : 0.f;
      }
    sum += other_half(sum);
    if (h == 0) {
      stat[(wm * TN + tl) * 2] = mx * kLog2e;
      stat[(wm * TN + tl) * 2 + 1] = sum;
    }
  }
  __syncthreads();
  if (tid < TN && t0 + tid < p.N) {
    float m2 = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES_M; ++w) m2 = fmaxf(m2, stat[(w * TN + tid) * 2]);
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES_M; ++w) s += stat[(w * TN + tid) * 2 + 1] * exp2_fast(stat[(w * TN + tid) * 2] - m2);
    float2* part = (float2*)p.part + (size_t)vt * p.N + t0 + tid;
    *part = make_float2(m2, s);
  }
}

// Per token: combine the vocabulary tiles' (max, sum) into the log-sum-exp,
// then NLL = LSE - target logit.  A workgroup takes 64 tokens (one per lane);
// its 8 waves split the vocabulary tiles round-robin, each folding its share
// online, and wave 0 folds the 8 results.
constexpr int RED_TOK = 64, RED_WAVES = 8;
__global__ void __launch_bounds__(RED_WAVES * 64) lce_reduce_kernel(const LceParams p) {
  __shared__ float2 stat[RED_WAVES][RED_TOK];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tok = blockIdx.x * RED_TOK + lane;
  const int nvt = (p.V + TM - 1) / TM;
  float m = -INFINITY, s = 0.f;
  if (tok < p.N) {
    const float2* part = (const float2*)p.part + tok;
    for (int vt = wave; vt < nvt; vt += RED_WAVES) {
      const float2 q = part[(size_t)vt * p.N];
      const float mn = fmaxf(m, q.x);
      s = s * exp2_fast(m - mn) + q.y * exp2_fast(q.x - mn);
      m = mn;
    }
  }
  stat[wave][lane] = make_float2(m, s);
  __syncthreads();
  if (wave != 0 || tok >= p.N) return;
  float m2 = -INFINITY;
#pragma unroll
  for (int w = 0; w < RED_WAVES; ++w) m2 = fmaxf(m2, stat[w][lane].x);
  float s2 = 0.f;
#pragma unroll
  for (int w = 0; w < RED_WAVES; ++w) s2 += stat[w][lane].y * exp2_fast(stat[w][lane].x - m2);
  const float lse = (m2 + log2_fast(s2)) * kLn2;
  p.lse[tok] = lse;
  // a target outside [0, V) was never captured: report NaN, not stale memory
  const int tgt = p.targets[tok];
  const float tz = (tgt >= 0 && tgt < p.V) ? p.tlogit[tok] : __builtin_nanf("");
  p.tlogit[tok] = tz;
  p.nll[tok] = lse - tz;
}

// ---------------------------------------------------------------- backward
// dZ of vocabulary chunk [c0, c0 + VC): one workgroup per (vocabulary tile,
// token tile) of the chunk, Z^T recomputed as in the forward, then
// dZ = g (exp(Z - LSE) - [v = t]) stored as bf16 to dz[token][dz_pos(v - c0)]
// (zeros past V, so the following products see none of those columns).
__global__ void __launch_bounds__(NWV * 64, WPE) lce_dz_kernel(const LceParams p, int c0, int vc, int kvalid) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * LCE_STAGES * TILE_MAX];
  FA_LDS char* smem = (FA_LDS char*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  const int nvt = (kvalid + TM - 1) / TM, ntt = (p.N + TN - 1) / TN;
  int vt, tt;
  tile_of(xcd_remap(blockIdx.x, nvt * ntt), nvt, ntt, vt, tt);
  const int v0 = c0 + vt * TM, t0 = tt * TN;
  const int ld = p.D * 2;

  StRow sa, sb;
  sa.init(wave, lane);
  sb.init(wave, lane, StRow::NINST);
  f32x16 acc[MB][NB];
  gemm_tile<ROWS, ROWS>(
      smem, p.D / TK,
      [&](FA_LDS char* t, int k0) { sa.issue_block(t, p.w, v0, p.V, ld, k0 * 2); },
      [&](FA_LDS char* t, int k0) { sb.issue_block(t, p.h, t0, p.N, ld, k0 * 2); }, acc, wave, lane);

  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int tok = t0 + WN * wn + 32 * nb + col;
    if (tok >= p.N) continue;
    const int tgt = p.targets[tok];
    const float nl2 = -p.lse_in[tok] * kLog2e;
    const float g = p.dnll[tok];
    bf16* row = (bf16*)p.dz + (size_t)tok * vc;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int v = v0 + WM * wm + 32 * mb + 8 * j + 4 * h;   // first of 4 consecutive
        f32x4 d;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pz = exp2_fast(fmaf(acc[mb][nb][4 * j + i], kLog2e, nl2));
          d[i] = v + i < p.V ? g * (pz - (v + i == tgt ? 1.f : 0.f)) : 0.f;
        }
        // v - c0 is a multiple of 4, and dz_pos keeps 4-aligned runs together
        if (v - c0 < vc) *(bf16x4*)(row + dz_pos(v - c0)) = __builtin_convertvector(d, bf16x4);
      }
  }
}

// dH^T (D x N) += W^T dZ^T over the chunk: one workgroup per (hidden tile,
// token tile).  `mode`: 0 the only chunk (write dh), 1 first (write the fp32
// accumulator), 2 middle (accumulate), 3 last (accumulate and write dh).
__global__ void __launch_bounds__(NWV * 64, WPE) lce_dh_kernel(const LceParams p, int c0, int vc,
                                                              int kvalid, int mode) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * LCE_STAGES * TILE_MAX];
  FA_LDS char* smem = (FA_LDS char*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  const int ndt = p.D / TM, ntt = (p.N + TN - 1) / TN;
  int dt, tt;
  tile_of(xcd_remap(blockIdx.x, ndt * ntt), ndt, ntt, dt, tt);
  const int d0 = dt * TM, t0 = tt * TN;

  StCol sa;
  StRow sb;
  sa.init(wave, lane);
  sb.init(wave, lane, StCol::NINST);
  f32x16 acc[MB][NB];
  gemm_tile<COLS, ROWS>(
      smem, (kvalid + TK - 1) / TK,
      // W rows c0 + k0 .. + TK - 1 (rows past V read as zeros), hidden columns d0 .. d0 + 255
      [&](FA_LDS char* t, int k0) { sa.issue_block(t, p.w, c0 + k0, p.V, p.D * 2, d0 * 2); },
      // dZ rows t0 .. t0 + 255, chunk positions k0 .. k0 + TK - 1
      [&](FA_LDS char* t, int k0) { sb.issue_block(t, p.dz, t0, p.N, vc * 2, k0 * 2); }, acc, wave, lane);

  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int tok = t0 + WN * wn + 32 * nb + col;
    if (tok >= p.N) continue;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = d0 + WM * wm + 32 * mb + 8 * j + 4 * h;
        const size_t e = (size_t)tok * p.D + d;
        f32x4 x = {acc[mb][nb][4 * j], acc[mb][nb][4 * j + 1], acc[mb][nb][4 * j + 2], acc[mb][nb][4 * j + 3]};
        if (mode >= 2) x += *(const f32x4*)(p.dh32 + e);
        if (mode == 1 || mode == 2) *(f32x4*)(p.dh32 + e) = x;
        else *(bf16x4*)((bf16*)p.dh + e) = __builtin_convertvector(x, bf16x4);
      }
  }
}

// dW^T (D x VC) = H^T dZ over all tokens for the chunk's vocabulary rows: one
// workgroup per (hidden tile, vocabulary tile of the chunk).
__global__ void __launch_bounds__(NWV * 64, WPE) lce_dw_kernel(const LceParams p, int c0, int vc, int kvalid) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * LCE_STAGES * TILE_MAX];
  FA_LDS char* smem = (FA_LDS char*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  const int ndt = p.D / TM, nvt = (kvalid + TN - 1) / TN;
  int dt, vt;
  tile_of(xcd_remap(blockIdx.x, ndt * nvt), ndt, nvt, dt, vt);
  const int d0 = dt * TM, vl0 = vt * TN;   // vl: column of the chunk

  StCol sa, sb;
  sa.init(wave, lane);
  sb.init(wave, lane, StCol::NINST);
  f32x16 acc[MB][NB];
  gemm_tile<COLS, COLS>(
      smem, (p.N + TK - 1) / TK,
      // H rows k0 .. k0 + TK - 1 (tokens; rows past N read as zeros), hidden columns d0 ..
      [&](FA_LDS char* t, int k0) { sa.issue_block(t, p.h, k0, p.N, p.D * 2, d0 * 2); },
      // dZ rows k0 .. k0 + TK - 1, chunk positions vl0 .. vl0 + 255
      [&](FA_LDS char* t, int k0) { sb.issue_block(t, p.dz, k0, p.N, vc * 2, vl0 * 2); }, acc, wave, lane);

  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    // this lane's output column is stored dZ position pc, i.e. vocabulary row c0 + dz_pos(pc)
    const int pc = vl0 + WN * wn + 32 * nb + col;
    const int v = c0 + dz_pos(pc);
    if (v >= p.V || pc >= vc) continue;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = d0 + WM * wm + 32 * mb + 8 * j + 4 * h;
        f32x4 x = {acc[mb][nb][4 * j], acc[mb][nb][4 * j + 1], acc[mb][nb][4 * j + 2], acc[mb][nb][4 * j + 3]};
        *(bf16x4*)((bf16*)p.dw + (size_t)v * p.D + d) = __builtin_convertvector(x, bf16x4);
      }
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_lce_fwd(const LceParams& p, hipStream_t s) {
  const int nvt = (p.V + TM - 1) / TM, ntt = (p.N + TN - 1) / TN;
  hipLaunchKernelGGL(lce_fwd_kernel, dim3((unsigned)(nvt * ntt)), dim3(NWV * 64), 0, s, p);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(lce_reduce_kernel, dim3((unsigned)((p.N + RED_TOK - 1) / RED_TOK)), dim3(RED_WAVES * 64), 0,
                     s, p);
  return hipGetLastError();
}

hipError_t launch_lce_bwd(const LceParams& p, int vc, hipStream_t s) {
  const int ntt = (p.N + TN - 1) / TN, ndt = p.D / TM;
  const int nchunks = (p.V + vc - 1) / vc;
  for (int c = 0; c < nchunks; ++c) {
    const int c0 = c * vc;
    // the last chunk may be partial: only the 256-column tiles holding valid
    // vocabulary rows are computed (dZ columns past V inside such a tile are
    // written as zeros, and dh reads no further than that tile)
    const int kvalid = min(vc, p.V - c0);
    const int nvt = (kvalid + TM - 1) / TM;
    hipLaunchKernelGGL(lce_dz_kernel, dim3((unsigned)(nvt * ntt)), dim3(NWV * 64), 0, s, p, c0, vc, kvalid);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    const int mode = nchunks == 1 ? 0 : (c == 0 ? 1 : (c + 1 == nchunks ? 3 : 2));
    hipLaunchKernelGGL(lce_dh_kernel, dim3((unsigned)(ndt * ntt)), dim3(NWV * 64), 0, s, p, c0, vc, kvalid,
                       mode);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    if (p.dw) {
      hipLaunchKernelGGL(lce_dw_kernel, dim3((unsigned)(ndt * nvt)), dim3(NWV * 64), 0, s, p, c0, vc, kvalid);
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
  }
  return hipSuccess;
}

}  // namespace fa
