// Backward kernels: dQ (with the per-row preprocess), then dK/dV.
//
// The backward keeps O(N) state and recomputes the probability tiles from Q,
// K and the saved log-sum-exp (mlx-train-perf 0.5.1 README, section
// "Flash-attention training path"), with causal and packed block-diagonal
// masking (changelog "Added": PACKED variants of the dQ and dK/dV kernels;
// README "Sequence packing": the dK/dV pass bounds its query walk at each key
// block's segment end rather than masking cross-segment work after computing
// it).  With P = exp(scale Q K^T - LSE) and dP = dO V^T, the softmax
// Jacobian gives dS = P * (dP - D) with D_i = sum_j P_ij dP_ij = dO_i . O_i;
// then dQ = scale dS K, dK = scale dS^T Q and dV = P^T dO.
//
// No atomics: dQ is accumulated in registers over key tiles by the workgroup
// owning a query tile, dK and dV over query tiles by the workgroup owning a
// key tile, so results are deterministic run to run.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

// ---------------------------------------------------------------- dQ
// One workgroup = NW waves x 32 queries; walks the key tiles the query tile can
// see.  It runs first in the backward and also does the row preprocess for
// its queries: D_i = dO_i . O_i (O as stored), and writes -D_i and -LSE_i /
// scale, negated so that the dK/dV kernel can start its dP and S
// accumulators from them (dP - D_i and S - LSE / scale come straight out of
// the MFMAs).  Per tile: S^T = K Q^T and dP^T = V dO^T (Q^T, dO^T held in registers),
// P^T and dS^T in registers, dQ^T += K^T dS^T with K^T through the transposing
// LDS read of the K tile.
//
// KSUB = 2 (8-wave bf16 workgroups): each ring slot holds two key tiles,
// walked one after the other with the same registers, so a wave does twice
// the MFMAs per barrier; the MFMA order on every accumulator is unchanged.
template <typename T, int D, bool CAUSAL, int NW, int KSUB = 1>
__global__ void __launch_bounds__(NW * 64, WAVES_PER_EU) dq_kernel(const BwdParams p) {
  constexpr int BM = NW * 32, BN = KEY_TILE;
  constexpr int KS = D / 16, DB = D / 32, KB = BN / 32;
  static_assert(KSUB == 1 || (KSUB == 2 && NW == 8 && sizeof(T) == 2), "two-tile slots: 8-wave bf16");
  constexpr int SR = KSUB * BN;   // key rows per ring slot
  // K is read along rows and transposed (DUAL), V only along rows.
  using LK = Layout<T, D, true>;
  using LV = Layout<T, D, false>;
  using StK = Stager<T, SR, D, NW, true>;
  using StV = Stager<T, SR, D, NW, false>;
  constexpr int TK = LK::bytes(SR), TV = LV::bytes(SR);
  constexpr int S = sizeof(T) == 2 ? stages_for(STAGES, TK + TV + SR * 4, NW) : 2;
  static_assert(S >= 2 && S * (TK + TV + SR * 4) <= LDS_PER_CU, "K/V stages must fit in LDS");
  constexpr int LPT = (StK::NINST + StV::NINST) / NW;
  // layout: K[S] | V[S] | seg[S]
  __shared__ __attribute__((aligned(1024))) char smem_raw[S * (TK + TV + SR * 4)];
  FA_LDS char* smem = (FA_LDS char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  const int N = p.N;
  const int nqt = p.ntiles;

  // (batch, head, query tile) and key-tile range, as in the forward.  Two-
  // tile instances are launched for dense calls only, so they carry no
  // packed code.
  const bool packed = KSUB == 1 && p.seg != nullptr;
  int bh, b, kt_lo = 0, kt_hi, qw0;
  if (packed) {
    const int4 wk = p.work[blockIdx.x / p.H];
    b = wk.x;
    qw0 = wk.y * BM + wave * 32;
    kt_lo = wk.z;
    kt_hi = wk.w;
    bh = b * p.H + (int)(blockIdx.x % p.H);
  } else {
    const int Lw = xcd_remap(blockIdx.x, p.B * p.H * nqt);
    bh = Lw / nqt;
    b = bh / p.H;
    if (CAUSAL && p.mirror) {
      const int t = Lw - bh * nqt;
      qw0 = 32 * mirror_block(t, wave, NW, nqt);
      kt_hi = (32 * (nqt * NW - t * (NW / 2)) - 1) / BN;
    } else {
      const int qt = nqt - 1 - (Lw - bh * nqt);
      qw0 = qt * BM + wave * 32;
      kt_hi = ((CAUSAL ? min(qt * BM + BM, N) : N) - 1) / BN;
    }
  }
  const size_t off = (size_t)bh * N * D;
  const size_t offkv = (size_t)(bh / p.G) * N * D;   // its key/value head
  const T* gq = (const T*)p.q + off;
  const T* gk = (const T*)p.k + offkv;
  const T* gv = (const T*)p.v + offkv;
  const T* gdo = (const T*)p.dO + off;
  const int32_t* seg = packed ? p.seg + (size_t)b * N : nullptr;

  const int qi = qw0 + col;
  const int qc = min(qi, N - 1);
  const int qlast = min(qw0 + 31, N - 1);

  frag_t<T> qf[KS], dof[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = gfrag_row<T, D>(gq, qc, 2 * ks + h);
    dof[ks] = gfrag_row<T, D>(gdo, qc, 2 * ks + h);
  }
  // D_i from the lane's half of the row (the same 8-element chunks as its dO
  // fragments) and the other half's lane
  const T* go = (const T*)p.o + off;
  float dsum = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const frag_t<T> of = gfrag_row<T, D>(go, qc, 2 * ks + h);
#pragma unroll
    for (int e = 0; e < 8; ++e) dsum = fmaf((float)of[e], (float)dof[ks][e], dsum);
  }
  dsum += other_half(dsum);
  const float nls = -p.lse[(size_t)bh * N + qc] / p.scale;
  const float nlse2 = p.c * nls;   // -LSE log2(e)
  const float ndlt = -dsum;        // -D_i
  if (h == 0 && qi < N) {
    p.nls[(size_t)bh * N + qi] = nls;
    p.delta[(size_t)bh * N + qi] = ndlt;
  }
  int segq = 0, segq_first = 0, segq_last = 0;
  if (packed) {
    segq = seg[qc];
    segq_first = seg[min(qw0, N - 1)];
    segq_last = seg[qlast];
  }
  const float c = p.c;

  StK stk;
  StV stv;
  stk.init(wave, lane);
  stv.init(wave, lane, StK::NINST);
  const int kbase_r = LK::row_base(lane);
  const int vbase_r = LV::row_base(lane);
  const int cbase = LK::col_base(lane);

  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqacc[db] = f32x16{};

  // ring slot j holds key tiles kt_lo + KSUB j .. + KSUB - 1
  const int nst = (kt_hi - kt_lo + KSUB) / KSUB;
  auto stage = [&](int j, int buf) {
    const int r0 = (kt_lo + KSUB * j) * BN;
    stk.issue(smem + buf * TK, gk, r0, N);
    stv.issue(smem + S * TK + buf * TV, gv, r0, N);
    if (packed) stage_vec<SR>(smem + S * (TK + TV) + buf * SR * 4, seg, r0, N, wave, NW - 1, lane);
  };

  // Ring of S stages, as in the forward.
#pragma unroll
  for (int i = 0; i < S - 1; ++i)
    if (i < nst) stage(i, i);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    settle(qf[ks]);
    settle(dof[ks]);
  }
  settle(nlse2);
  settle(ndlt);
  settle(segq);
  settle(segq_first);
  settle(segq_last);
  for (int js = 0; js < nst; ++js) {
    const int buf = js % S;
    wait_tiles<LPT, S - 2>(nst - 1 - js);
    __syncthreads();
    // With two tiles per slot the next slot's loads go out at the second
    // tile (see the sub loop); with one, right after the barrier.
    const bool more = js + S - 1 < nst;
    const int nbuf = buf == 0 ? S - 1 : buf - 1;
    if (KSUB == 1 && more) stage(js + S - 1, nbuf);

    const FA_LDS char* Ks = smem + buf * TK;
    const FA_LDS char* Vs = smem + S * TK + buf * TV;
    const FA_LDS int* segs = (const FA_LDS int*)(smem + S * (TK + TV) + buf * SR * 4);
#pragma unroll
    for (int sub = 0; sub < KSUB; ++sub) {
    // Issued here, the loads do not crowd the first tile's fragment reads
    // at the moment every wave leaves the barrier (measured faster); the
    // slot they fill was released by that barrier.
    if (KSUB == 2 && sub == 1 && more) stage(js + S - 1, nbuf);
    const int kt = kt_lo + KSUB * js + sub;
    if (kt > kt_hi) break;
    const int rs = BN * sub;   // first row of this key tile in the slot
    const FA_LDS int* segk = segs + rs;
    const int k0 = kt * BN;
    const int klast = min(k0 + BN, N) - 1;

    bool skip = qw0 >= N;
    if (CAUSAL) skip = skip || k0 > qlast;
    bool full = (k0 + BN <= N) && (!CAUSAL || k0 + BN - 1 <= qw0);
    if (packed) {
      const int sk0 = segk[0], skl = segk[klast - k0];
      skip = skip || skl < segq_first || (!CAUSAL && sk0 > segq_last);
      full = full && (min(sk0, segq_first) == max(skl, segq_last));
    }
    if (skip) continue;

    f32x16 sacc[KB], dpacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      sacc[kb] = f32x16{};
      dpacc[kb] = f32x16{};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        mma(sacc[kb], frag_row<T, D, true>(Ks, kbase_r, rs + 32 * kb, ks), qf[ks]);
        mma(dpacc[kb], frag_row<T, D, false>(Vs, vbase_r, rs + 32 * kb, ks), dof[ks]);
      }
    }

    if (!full) {
      // Element 4j + i of block kb is key k0 + 4h + c with c = 32kb + 8j + i
      // a compile-time constant: key < N and (causal) key <= qi become one
      // compare of c against a per-lane bound; packed rows add the segment
      // test on a branch of their own.
      const int L = (CAUSAL ? min(qi, N - 1) : N - 1) - (k0 + 4 * h);
      if (packed) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const i32x4 sk = *(const FA_LDS i32x4*)(segk + 32 * kb + 8 * j + 4 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (!(32 * kb + 8 * j + i <= L && sk[i] == segq)) sacc[kb][4 * j + i] = -INFINITY;
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!(32 * kb + 8 * (r >> 2) + (r & 3) <= L)) sacc[kb][r] = -INFINITY;
      }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = exp2_fast(fmaf(sacc[kb][r], c, nlse2));
        sacc[kb][r] = pv * (dpacc[kb][r] + ndlt);
      }

    frag_t<T> dsf[KB][2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      dsf[kb][0] = acc_frag<T>(sacc[kb], 0);
      dsf[kb][1] = acc_frag<T>(sacc[kb], 1);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          mma(dqacc[db], frag_col<T, D>(Ks, cbase, rs + 32 * kb + 16 * kc, 32 * db), dsf[kb][kc]);
    }
  }

  if (qi < N) store_rows<T, D>((T*)p.dq + off, qi, dqacc, p.scale, lane);
}

// ---------------------------------------------------------------- dK / dV
// One workgroup = NW waves x 32 keys; walks the query tiles that can see the
// key tile.  Per tile: S = Q K^T and dP = dO V^T (K^T, V^T held in registers;
// the accumulator columns are keys, rows queries), P and dS in registers,
// dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T through the transposing
// LDS read.
// TEAMS = 2 (grouped-query heads, an even group size G): the workgroup's
// waves form two teams of NW / 2 that own the same keys; team t walks query
// heads t G / 2 .. (t + 1) G / 2 - 1 of the group, both teams in step (equal
// trip counts, shared barriers), and team 1 adds its dK and dV into team 0's
// through LDS at the end.  That gives grouped heads full-occupancy
// workgroups of equal halves instead of few long, half-occupied ones.
//
// QSUB = 2 (dense multi-head calls, 8 waves): each ring slot holds two query
// tiles, walked one after the other with the same registers, so a wave does
// twice the MFMAs per barrier.  The order of the MFMAs on every accumulator
// is unchanged.
template <typename T, int D, bool CAUSAL, int NW, int TEAMS = 1, int QSUB = 1>
__global__ void __launch_bounds__(NW * 64, WAVES_PER_EU) dkdv_kernel(const BwdParams p) {
  constexpr int KW = NW / TEAMS;   // waves along the keys
  constexpr int BNK = KW * 32, BMQ = QRY_TILE;
  constexpr int KS = D / 16, DB = D / 32, QB = BMQ / 32;
  constexpr int SR = QSUB * BMQ;   // query rows per ring slot
  using L = Layout<T, D>;
  using St = Stager<T, SR, D, NW>;
  constexpr int TILE = L::bytes(SR);
  constexpr int VEC = SR * 4;
  constexpr int PER_STAGE = TEAMS * (2 * TILE + 2 * VEC) + VEC;
  constexpr int S = sizeof(T) == 2 ? stages_for(STAGES, PER_STAGE, NW) : 2;
  static_assert(S >= 2 && S * PER_STAGE <= LDS_PER_CU, "Q/dO stages must fit in LDS");
  static_assert(TEAMS == 1 || (TEAMS == 2 && sizeof(T) == 2 && NW == 8), "teams: bf16, 8 waves");
  static_assert(TEAMS == 1 || S * PER_STAGE >= KW * 32 * D * 4, "team reduction reuses the ring");
  // The 2 TEAMS Q and dO tiles of a stage share one stager's per-lane
  // offsets when one tile's instructions already reach every wave; otherwise
  // (D < 128, 8 waves) each further tile's stager continues the round-robin
  // so that every wave has a load to count.
  constexpr bool SHARE = St::NINST >= NW;
  constexpr int LPT = SHARE ? 2 * TEAMS * (St::NINST / NW) : 2 * TEAMS * St::NINST / NW;
  __shared__ __attribute__((aligned(1024))) char smem_raw[S * PER_STAGE];
  FA_LDS char* smem = (FA_LDS char*)smem_raw;
  // layout: Q[S][TEAMS] | dO[S][TEAMS] | nls[S][TEAMS] | delta[S][TEAMS] | seg[S]
  constexpr int OFF_DO = S * TEAMS * TILE, OFF_NLS = 2 * S * TEAMS * TILE;
  constexpr int OFF_DLS = OFF_NLS + S * TEAMS * VEC, OFF_SEG = OFF_DLS + S * TEAMS * VEC;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Teams: waves {0, 1, 4, 5} form team 0 and {2, 3, 6, 7} team 1, so that
  // each SIMD (waves w and w + 4) holds key waves kw and kw + 2 of one team.
  // With mirrored key blocks those are one early and one late block.
  const int team = TEAMS == 1 ? 0 : (wave >> 1) & 1;
  const int kwave = TEAMS == 1 ? wave : (wave & 1) | ((wave >> 2) << 1);
  const int h = lane >> 5, col = lane & 31;
  const int N = p.N;
  const int nkt = p.ntiles;

  // (batch, key/value head, key tile) and query-tile range.  Packed: the
  // longest-first work list.  Dense: XCD-contiguous heads, key tile 0 (for
  // causal, seen by the most queries) first.  The workgroup walks the query
  // tiles of each of the key/value head's G query heads in turn and sums
  // their contributions to dK and dV in its registers.
  // Two-tile instances are launched for dense calls only (no packed code).
  const bool packed = QSUB == 1 && p.seg != nullptr;
  const int G = p.G, Hkv = p.H / G;
  int bg, b, qt_lo, qt_hi, kw0;
  if (packed) {
    const int4 wk = p.work[blockIdx.x / Hkv];
    b = wk.x;
    kw0 = wk.y * BNK + kwave * 32;
    qt_lo = wk.z;
    qt_hi = wk.w;
    bg = b * Hkv + (int)(blockIdx.x % Hkv);
  } else if (CAUSAL && (TEAMS == 2 ? p.mirror == 1 : G == 1 && p.mirror != 0)) {
    // mirrored key blocks (see mirror_block) over the key waves, the same in
    // both teams (one round of workgroups only: at two, the heaviest-first
    // order already pairs heavy and light teams); the walk starts at the
    // workgroup's first key.  The one-team kernel of grouped heads keeps its
    // own heavy/light pairing.
    const int Lw = xcd_remap(blockIdx.x, p.B * Hkv * nkt);
    bg = Lw / nkt;
    const int l = Lw - bg * nkt;
    kw0 = 32 * mirror_block(l, kwave, KW, nkt);
    b = bg / Hkv;
    qt_lo = 32 * l * (KW / 2) / BMQ;
    qt_hi = (N - 1) / BMQ;
  } else {
    const int Lw = xcd_remap(blockIdx.x, p.B * Hkv * nkt);
    bg = Lw / nkt;
    const int l = Lw - bg * nkt;
    // With grouped heads and one team there are few, long workgroups, all
    // resident at once, so a head's first key tiles (heaviest under causal
    // masking) are dispatched in ascending and its second half in descending
    // order: the two workgroups a CU receives pair a heavy tile with a light
    // one.  Teams fill a CU with one workgroup; heaviest first then.
    const int half = (nkt + 1) / 2;
    const int kt = (TEAMS == 1 && G > 1 && l >= half) ? nkt - 1 - (l - half) : l;
    kw0 = kt * BNK + kwave * 32;
    b = bg / Hkv;
    qt_lo = CAUSAL ? kt * BNK / BMQ : 0;
    qt_hi = (N - 1) / BMQ;
  }
  const size_t offkv = (size_t)bg * N * D;
  const size_t bh0 = (size_t)bg * G;   // first query head of the group
  const T* gk = (const T*)p.k + offkv;
  const T* gv = (const T*)p.v + offkv;
  const int32_t* seg = packed ? p.seg + (size_t)b * N : nullptr;
  // iteration it covers query head bh0 + team GT + it / nqs, query tiles
  // qt_lo + QSUB (it % nqs) .. + QSUB - 1 (GT = G / TEAMS heads per team)
  const int GT = G / TEAMS;
  const int nq = qt_hi - qt_lo + 1;
  const int nqs = (nq + QSUB - 1) / QSUB;
  const int nit = nq > 0 ? GT * nqs : 0;

  const int kj = kw0 + col;
  const int kc_ = min(kj, N - 1);
  const int klast = min(kw0 + 31, N - 1);

  frag_t<T> kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = gfrag_row<T, D>(gk, kc_, 2 * ks + h);
    vf[ks] = gfrag_row<T, D>(gv, kc_, 2 * ks + h);
  }
  int segk = 0, segk_first = 0, segk_last = 0;
  if (packed) {
    segk = seg[kc_];
    segk_first = seg[min(kw0, N - 1)];
    segk_last = seg[klast];
  }
  const float c = p.c;

  St stq, stdo;
  stq.init(wave, lane);
  if constexpr (!SHARE) stdo.init(wave, lane, St::NINST);
  St stq2, stdo2;   // team 1's tiles, continuing the round-robin
  if constexpr (TEAMS == 2 && !SHARE) {
    stq2.init(wave, lane, 2 * St::NINST);
    stdo2.init(wave, lane, 3 * St::NINST);
  }
  const int rbase = L::row_base(lane);
  const int cbase = L::col_base(lane);
  // seed value of this lane, relative to the slot's -LSE/scale vector: row
  // col of it (lanes 0-31) or of the -D_i vector (lanes 32-63)
  const int seed_base = (h ? OFF_DLS - OFF_NLS : 0) + 4 * col;

  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }

  auto stage = [&](int it, int buf) {
    const int hj = it / nqs;
    const int r0 = (qt_lo + (it - hj * nqs) * QSUB) * BMQ;
#pragma unroll
    for (int t = 0; t < TEAMS; ++t) {
      const size_t bh = bh0 + t * GT + hj;
      const int slot = buf * TEAMS + t;
      (SHARE || t == 0 ? stq : stq2).issue(smem + slot * TILE, (const T*)p.q + bh * N * D, r0, N);
      (SHARE ? stq : (t == 0 ? stdo : stdo2)).issue(smem + OFF_DO + slot * TILE, (const T*)p.dO + bh * N * D, r0, N);
      stage_vec<SR>(smem + OFF_NLS + slot * VEC, p.nls + bh * N, r0, N, wave, (2 * t) % NW, lane);
      stage_vec<SR>(smem + OFF_DLS + slot * VEC, p.delta + bh * N, r0, N, wave, (2 * t + 1) % NW, lane);
    }
    if (packed) stage_vec<SR>(smem + OFF_SEG + buf * VEC, seg, r0, N, wave, (2 * TEAMS) % NW, lane);
  };

  // Ring of S stages, as in the forward.
#pragma unroll
  for (int i = 0; i < S - 1; ++i)
    if (i < nit) stage(i, i);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    settle(kf[ks]);
    settle(vf[ks]);
  }
  settle(segk);
  settle(segk_first);
  settle(segk_last);
  for (int it = 0; it < nit; ++it) {
    const int buf = it % S;
    wait_tiles<LPT, S - 2>(nit - 1 - it);
    __syncthreads();
    const bool more = it + S - 1 < nit;
    const int nbuf = buf == 0 ? S - 1 : buf - 1;
    if (QSUB == 1 && more) stage(it + S - 1, nbuf);   // two-tile slots: at the second tile

    const int slot = buf * TEAMS + team;
    const FA_LDS char* Qs = smem + slot * TILE;
    const FA_LDS char* dOs = smem + OFF_DO + slot * TILE;
    const FA_LDS float* nls = (const FA_LDS float*)(smem + OFF_NLS + slot * VEC);
    const FA_LDS int* sqs = (const FA_LDS int*)(smem + OFF_SEG + buf * VEC);
    const int qtb = qt_lo + (it % nqs) * QSUB;
#pragma unroll
    for (int sub = 0; sub < QSUB; ++sub) {
    if (QSUB == 2 && sub == 1 && more) stage(it + S - 1, nbuf);   // as in dQ
    const int qt = qtb + sub;
    if (qt > qt_hi) break;
    const int rs = 32 * QB * sub;   // first row of this query tile in the slot
    const int q0 = qt * BMQ;
    const int qlast = min(q0 + BMQ, N) - 1;

    bool skip = kw0 >= N;
    if (CAUSAL) skip = skip || qlast < kw0;
    bool full = (q0 + BMQ <= N) && (kw0 + 31 < N) && (!CAUSAL || q0 >= kw0 + 31);
    if (packed) {
      const int sq0 = sqs[rs], sql = sqs[rs + qlast - q0];
      skip = skip || sq0 > segk_last || (!CAUSAL && sql < segk_first);
      full = full && (min(sq0, segk_first) == max(sql, segk_last));
    }
    if (skip) continue;

    // S - LSE / scale = Q K^T - LSE / scale and dP - D = dO V^T - D, block by
    // block: the accumulators start from the negated per-row values dQ
    // wrote, so the MFMAs deliver both differences directly.  The start
    // values come from one seeding MFMA (seed_rows): lane col reads -LSE/scale
    // of query row col (lanes 0-31) or -D_i of it (lanes 32-63), 4 bytes a
    // lane, where broadcasting the 16 rows a lane's accumulator spans would
    // read 128 bytes a lane from LDS per tile.
    f32x16 sacc[QB], dpacc[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      seed_rows(sacc[qb], dpacc[qb], *(const FA_LDS float*)((const FA_LDS char*)nls + seed_base + (rs + 32 * qb) * 4));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        mma(sacc[qb], frag_row<T, D>(Qs, rbase, rs + 32 * qb, ks), kf[ks]);
        mma(dpacc[qb], frag_row<T, D>(dOs, rbase, rs + 32 * qb, ks), vf[ks]);
      }
    }

    if (!full) {
      // Accumulator element 4j + i of block qb: query q0 + 4h + c with
      // c = 32qb + 8j + i a compile-time constant, key kj.  Visible iff
      // kj < N, (causal) q >= kj and q < N: one compare of c against a
      // per-lane lower bound, a second one only in the tile that holds row
      // N - 1, and the segment test on a branch of packed rows.
      const int A = kj < N ? (CAUSAL ? kj : 0) - (q0 + 4 * h) : (1 << 30);   // c >= A
      if (packed) {
        const int Bq = N - 1 - (q0 + 4 * h);   // c <= Bq
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const i32x4 sq = *(const FA_LDS i32x4*)(sqs + rs + 32 * qb + 8 * j + 4 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int cc = 32 * qb + 8 * j + i;
              if (!(cc >= A && cc <= Bq && sq[i] == segk)) sacc[qb][4 * j + i] = -INFINITY;
            }
          }
      } else if (q0 + BMQ > N) {   // the tile holding row N - 1
        const int Bq = N - 1 - (q0 + 4 * h);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int cc = 32 * qb + 8 * (r >> 2) + (r & 3);
            if (!(cc >= A && cc <= Bq)) sacc[qb][r] = -INFINITY;
          }
      } else {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!(32 * qb + 8 * (r >> 2) + (r & 3) >= A)) sacc[qb][r] = -INFINITY;
      }
    }

    // Per block: P = exp2(c (S - LSE / scale)), dS = P (dP - D); then
    // dV^T += dO^T P and dK^T += Q^T dS.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = exp2_fast(sacc[qb][r] * c);
        sacc[qb][r] = pv;
        dpacc[qb][r] = pv * dpacc[qb][r];
      }
      frag_t<T> pf[2], dsf[2];
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        pf[kc] = acc_frag<T>(sacc[qb], kc);
        dsf[kc] = acc_frag<T>(dpacc[qb], kc);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          mma(dvacc[db], frag_col<T, D>(dOs, cbase, rs + 32 * qb + 16 * kc, 32 * db), pf[kc]);
          mma(dkacc[db], frag_col<T, D>(Qs, cbase, rs + 32 * qb + 16 * kc, 32 * db), dsf[kc]);
        }
      // bf16: each of these MFMAs takes its A fragment from two transposing
      // LDS reads; have them issued one MFMA ahead.  Left to itself the
      // compiler waits for each pair just before its MFMA (lgkmcnt(0) every
      // time).  Only the issue order changes, so the results do not.
      if constexpr (sizeof(T) == 2) {
        constexpr int NM = DB * 4;
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          if (i + 1 < NM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      }
    }
    }
  }

  if constexpr (TEAMS == 2) {
    // team 0 += team 1, dK then dV, through the (now idle) ring: one fp32
    // value per (key wave, accumulator element, lane), lane-contiguous
    float* red = (float*)smem_raw;
    auto exchange = [&](f32x16 (&acc)[DB]) {
      __syncthreads();
      if (team == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) red[((kwave * DB + db) * 16 + r) * 64 + lane] = acc[db][r];
      }
      __syncthreads();
      if (team == 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] += red[((kwave * DB + db) * 16 + r) * 64 + lane];
      }
    };
    exchange(dkacc);
    exchange(dvacc);
    if (team == 1) return;
  }
  if (kj < N) {
    store_rows<T, D>((T*)p.dk + offkv, kj, dkacc, p.scale, lane);
    store_rows<T, D>((T*)p.dv + offkv, kj, dvacc, 1.f, lane);
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_bwd_dq(const BwdParams& p, int dtype, int D, bool causal, int nw, hipStream_t s) {
  return dispatch(dtype, D, causal, nw, [&](auto t, auto d, auto c, auto w) {
    using T = typename decltype(t)::type;
    constexpr int DD = decltype(d)::value, NW = decltype(w)::value;
    constexpr bool C = decltype(c)::value;
    const long long total = (long long)p.B * p.H * p.ntiles;
    constexpr int KS2 = (NW == 8 && sizeof(T) == 2) ? KSUB_DENSE : 1;
    if (KS2 > 1 && p.seg == nullptr)
      hipLaunchKernelGGL((dq_kernel<T, DD, C, NW, KS2>), dim3((unsigned)total), dim3(NW * 64), 0, s, p);
    else
      hipLaunchKernelGGL((dq_kernel<T, DD, C, NW, 1>), dim3((unsigned)total), dim3(NW * 64), 0, s, p);
    return hipGetLastError();
  });
}

hipError_t launch_bwd_dkdv(const BwdParams& p, int dtype, int D, bool causal, int nw, hipStream_t s) {
  // grouped heads, bf16, 4 key waves and an even group: two teams, for
  // dense and packed calls alike, so that a group's dK/dV sums its heads in
  // the same order either way and a single-segment packed call keeps the
  // causal call's bits
  if (nw == 4 && p.G > 1 && p.G % 2 == 0 && dtype == 0) {
    const long long total = (long long)p.B * (p.H / p.G) * p.ntiles;
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3((unsigned)total), dim3(8 * 64), 0, s, p);
      return hipGetLastError();
    };
    if (D == 128) return causal ? go(dkdv_kernel<bf16, 128, true, 8, 2>) : go(dkdv_kernel<bf16, 128, false, 8, 2>);
    if (D == 96) return causal ? go(dkdv_kernel<bf16, 96, true, 8, 2>) : go(dkdv_kernel<bf16, 96, false, 8, 2>);
    return causal ? go(dkdv_kernel<bf16, 64, true, 8, 2>) : go(dkdv_kernel<bf16, 64, false, 8, 2>);
  }
  return dispatch(dtype, D, causal, nw, [&](auto t, auto d, auto c, auto w) {
    using T = typename decltype(t)::type;
    constexpr int DD = decltype(d)::value, NW = decltype(w)::value;
    constexpr bool C = decltype(c)::value;
    const long long total = (long long)p.B * (p.H / p.G) * p.ntiles;
    // 8-wave dK/dV workgroups are dense multi-head ones (packed and grouped
    // calls use 4): two query tiles per ring slot for bf16
    constexpr int QS = (NW == 8 && sizeof(T) == 2) ? QSUB_DENSE : 1;
    if (QS > 1 && p.seg == nullptr)
      hipLaunchKernelGGL((dkdv_kernel<T, DD, C, NW, 1, QS>), dim3((unsigned)total), dim3(NW * 64), 0, s, p);
    else
      hipLaunchKernelGGL((dkdv_kernel<T, DD, C, NW, 1, 1>), dim3((unsigned)total), dim3(NW * 64), 0, s, p);
    return hipGetLastError();
  });
}

}  // namespace fa
