// Forward kernel: O and the per-row log-sum-exp, never an (N, N) matrix.
//
// What is computed follows the mlx-train-perf 0.5.1 README, section
// "Flash-attention training path": the forward keeps only the attention
// output and the log-sum-exp as saved state.  Masking is causal and, for
// packed rows, block-diagonal by segment id (same README, "Sequence packing";
// changelog "Added": the PACKED forward variant).
//
// One workgroup = NW waves of one (batch, head).  Each wave owns 32
// queries and computes S^T = K Q^T for a 64-key tile (32x32 MFMA tiles), so
// the softmax statistics of a query live in one lane pair (l, l+32).  Q^T
// stays in registers for the whole key walk; K and V tiles come through a
// ring of LDS stages filled by direct global->LDS loads.  O^T += V^T P^T
// takes P^T straight from the accumulator and V^T from the V tile through
// the transposing LDS read.
//
// Causal / packed structure is used at wave granularity: key tiles no query
// of a wave can see are skipped, tiles every query sees skip the
// per-element mask.  Probabilities are taken against a per-row reference
// that moves rarely (see GROW_LIMIT), so the O rescale is a rare,
// wave-uniform branch.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

//
// KSUB = 2 (8-wave bf16 workgroups of dense calls): each ring slot holds two
// key tiles, so a wave does twice the MFMAs per barrier, and the first
// tile's P V MFMAs are issued together with the second tile's softmax (see
// the slot body).  Every operation on every row happens in the same order as
// with one tile per slot.
template <typename T, int D, bool CAUSAL, int NW, int KSUB = 1>
__global__ void __launch_bounds__(NW * 64, WAVES_PER_EU) fwd_kernel(const FwdParams p) {
  constexpr int BM = NW * 32, BN = KEY_TILE;
  constexpr int KS = D / 16, DB = D / 32, KB = BN / 32;
  static_assert(KSUB == 1 || (KSUB == 2 && NW == 8 && sizeof(T) == 2), "two-tile slots: 8-wave bf16");
  constexpr int SR = KSUB * BN;   // key rows per ring slot
  // K is read only along rows (row-only layout), V only transposed (DUAL).
  using LK = Layout<T, D, false>;
  using LV = Layout<T, D, true>;
  using StK = Stager<T, SR, D, NW, false>;
  using StV = Stager<T, SR, D, NW, true>;
  constexpr int TK = LK::bytes(SR), TV = LV::bytes(SR);
  constexpr int S = sizeof(T) == 2 ? stages_for(STAGES, TK + TV + SR * 4, NW) : 2;
  static_assert(S >= 2 && S * (TK + TV + SR * 4) <= LDS_PER_CU, "K/V stages must fit in LDS");
  constexpr int LPT = (StK::NINST + StV::NINST) / NW;   // loads per wave per slot, at least
  // layout: K[S] | V[S] | seg[S]
  __shared__ __attribute__((aligned(1024))) char smem_raw[S * (TK + TV + SR * 4)];
  FA_LDS char* smem = (FA_LDS char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  const int N = p.N;

  // Which (batch, head, query tile), and the key tiles to walk.  Packed: the
  // longest-first work list.  Dense: each XCD takes a contiguous range of
  // heads, the last (for causal, longest) query tiles first.
  // two-tile instances are launched for dense calls only (no packed code)
  const bool packed = KSUB == 1 && p.seg != nullptr;
  // (mirrored blocks: see mirror_block)
  int bh, b, kt_lo = 0, kt_hi, qw0;
  if (packed) {
    const int4 wk = p.work[blockIdx.x / p.H];
    b = wk.x;
    qw0 = wk.y * BM + wave * 32;
    kt_lo = wk.z;
    kt_hi = wk.w;
    bh = b * p.H + (int)(blockIdx.x % p.H);
  } else {
    const int Lw = xcd_remap(blockIdx.x, p.B * p.H * p.nqt);
    bh = Lw / p.nqt;
    b = bh / p.H;
    if (CAUSAL && p.mirror) {
      const int t = Lw - bh * p.nqt;
      qw0 = 32 * mirror_block(t, wave, NW, p.nqt);
      kt_hi = (32 * (p.nqt * NW - t * (NW / 2)) - 1) / BN;
    } else {
      const int qt = p.nqt - 1 - (Lw - bh * p.nqt);
      qw0 = qt * BM + wave * 32;
      kt_hi = ((CAUSAL ? min(qt * BM + BM, N) : N) - 1) / BN;
    }
  }
  // q and o rows of head bh; k and v of its key/value head (grouped-query
  // heads form contiguous runs of G)
  const size_t off = (size_t)bh * N * D;
  const size_t offkv = (size_t)(bh / p.G) * N * D;
  const T* gq = (const T*)p.q + off;
  const T* gk = (const T*)p.k + offkv;
  const T* gv = (const T*)p.v + offkv;
  const int32_t* seg = packed ? p.seg + (size_t)b * N : nullptr;

  // The wave owns queries qw0 .. qw0 + 31; lane l holds query qw0 + l % 32.
  const int qi = qw0 + col;
  const int qc = min(qi, N - 1);
  const int qlast = min(qw0 + 31, N - 1);

  frag_t<T> qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = gfrag_row<T, D>(gq, qc, 2 * ks + h);
  int segq = 0, segq_first = 0, segq_last = 0;
  if (packed) {
    segq = seg[qc];
    segq_first = seg[min(qw0, N - 1)];
    segq_last = seg[qlast];
  }

  StK stk;
  StV stv;
  stk.init(wave, lane);
  stv.init(wave, lane, StK::NINST);
  const int rbase = LK::row_base(lane);
  const int cbase = LV::col_base(lane);

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  // msc: the row's reference (scores times c, log2 units; -inf until the row
  // has seen a visible key); lsum: this lane's half of the row sum.
  float msc = -INFINITY, lsum = 0.f;
  const float c = p.c;

  // ring slot j holds key tiles kt_lo + KSUB j .. + KSUB - 1
  const int nst = (kt_hi - kt_lo + KSUB) / KSUB;
  auto stage = [&](int j, int buf) {
    const int r0 = (kt_lo + KSUB * j) * BN;
    stk.issue(smem + buf * TK, gk, r0, N);
    stv.issue(smem + S * TK + buf * TV, gv, r0, N);
    if (packed) stage_vec<SR>(smem + S * (TK + TV) + buf * SR * 4, seg, r0, N, wave, NW - 1, lane);
  };
  // Ring of S stages: slots j + 1 .. j + S - 2 stay in flight while slot j
  // is used; the barrier after the wait also tells every wave that the
  // buffer of slot j - 1 is free for slot j + S - 1.
#pragma unroll
  for (int i = 0; i < S - 1; ++i)
    if (i < nst) stage(i, i);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) settle(qf[ks]);
  settle(segq);
  settle(segq_first);
  settle(segq_last);

  // ---- two-tile slot body (dense calls).  Probabilities overwrite their
  // scores in place, so a tile's probabilities cost no second register block;
  // a tile that takes the rare path has its scores recomputed from LDS first
  // (same MFMAs in the same order, so the same values).  The registers saved
  // let a wave issue the first tile's P V MFMAs in one block with the second
  // tile's exponentials, so its matrix and vector work overlap.  (Issuing
  // the second tile's scores with the first tile's softmax as well needs two
  // score blocks at once: it spills at head_dim 128 and measured 3-5 %
  // slower at 96 and 64.)
  auto scores = [&](f32x16 (&s)[KB], const FA_LDS char* Ks_, int rs) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) mma(s[kb], frag_row<T, D, false>(Ks_, rbase, rs + 32 * kb, ks), qf[ks]);
    }
  };
  auto mask_dense = [&](f32x16 (&s)[KB], int k0) {
    const int L = (CAUSAL ? min(qi, N - 1) : N - 1) - (k0 + 4 * h);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (!(32 * kb + 8 * (r >> 2) + (r & 3) <= L)) s[kb][r] = -INFINITY;
  };
  // probabilities against the current reference, in place; returns the
  // lane's partial row sum
  auto optimistic = [&](f32x16 (&s)[KB], float (&ls)[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) ls[r] = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2_fast(fmaf(s[kb][r], c, -msc));
        s[kb][r] = e;
        ls[r & 3] += e;
      }
    return (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };
  // the rare path on the tile's scores: move the references, rescale O and
  // the sums, probabilities in place
  auto rare = [&](f32x16 (&s)[KB], float (&ls)[4]) {
    float tm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tm[r & 3] = fmaxf(tm[r & 3], s[kb][r]);
    float tmax = fmaxf(fmaxf(tm[0], tm[1]), fmaxf(tm[2], tm[3]));
    tmax = fmaxf(tmax, other_half(tmax));
    const float tsc = tmax * c;
    const bool grow = tsc > msc;
    const float alpha = grow ? exp2_fast(msc - tsc) : 1.f;
    msc = grow ? tsc : msc;
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    const float mref = (msc == -INFINITY) ? 0.f : msc;
#pragma unroll
    for (int r = 0; r < 4; ++r) ls[r] = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2_fast(fmaf(s[kb][r], c, -mref));
        s[kb][r] = e;
        ls[r & 3] += e;
      }
  };
  auto to_frags = [&](const f32x16 (&s)[KB], frag_t<T> (&pf)[KB][2]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      pf[kb][0] = acc_frag<T>(s[kb], 0);
      pf[kb][1] = acc_frag<T>(s[kb], 1);
    }
  };
  auto pv = [&](const frag_t<T> (&pf)[KB][2], const FA_LDS char* Vs_, int rs) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          mma(oacc[db], frag_col<T, D>(Vs_, cbase, rs + 32 * kb + 16 * kc, 32 * db), pf[kb][kc]);
  };
  // Interleave of one overlapped block: NM MFMAs, each with its RD LDS
  // fragment reads issued a step ahead, and the vector work spread between
  // them, so few fragments are in flight at once.
  auto interleave = [&](auto nm, auto rd) {
    constexpr int NM = decltype(nm)::value, RD = decltype(rd)::value;
    __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + 1 < NM) __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
  };
  // slot of key tiles kt0 and kt0 + 1 (the second may lie past kt_hi)
  auto slot2 = [&](const FA_LDS char* Ks_, const FA_LDS char* Vs_, int kt0) {
    const int ka = kt0 * BN, kb1 = ka + BN;
    if (qw0 >= N || (CAUSAL && ka > qlast)) return;   // the second tile is invisible too
    const bool has1 = kt0 + 1 <= kt_hi && !(CAUSAL && kb1 > qlast);
    const bool full0 = (ka + BN <= N) && (!CAUSAL || ka + BN - 1 <= qw0);
    const bool full1 = (kb1 + BN <= N) && (!CAUSAL || kb1 + BN - 1 <= qw0);
    f32x16 s0[KB], s1[KB];
    float ls0[4], ls1[4];
    scores(s0, Ks_, 0);
    if (!full0) mask_dense(s0, ka);
    // first tile's softmax (a row with no reference yet takes the rare path
    // directly)
    const bool fresh = __builtin_amdgcn_ballot_w64(msc == -INFINITY) != 0;
    if (fresh) {
      rare(s0, ls0);
    } else {
      const float lpart = optimistic(s0, ls0);
      if (__builtin_amdgcn_ballot_w64(!(lpart < GROW_LIMIT)) != 0) {
        scores(s0, Ks_, 0);
        if (!full0) mask_dense(s0, ka);
        rare(s0, ls0);
      }
    }
    lsum += (ls0[0] + ls0[1]) + (ls0[2] + ls0[3]);
    frag_t<T> pf0[KB][2];
    to_frags(s0, pf0);
    if (!has1) {
      pv(pf0, Vs_, 0);
      return;
    }
    // first tile's P V with the second tile's softmax alongside; a row
    // without a reference cannot remain here (the first tile gave every row
    // one), and any overflow sends the tile down the rare path
    scores(s1, Ks_, BN);
    if (!full1) mask_dense(s1, kb1);
    pv(pf0, Vs_, 0);
    const float lpart1 = optimistic(s1, ls1);
    interleave(int_c<DB * KB * 2>{}, int_c<2>{});
    if (__builtin_amdgcn_ballot_w64(!(lpart1 < GROW_LIMIT)) != 0) {
      scores(s1, Ks_, BN);
      if (!full1) mask_dense(s1, kb1);
      rare(s1, ls1);
    }
    lsum += (ls1[0] + ls1[1]) + (ls1[2] + ls1[3]);
    frag_t<T> pf1[KB][2];
    to_frags(s1, pf1);
    pv(pf1, Vs_, BN);
  };

  for (int js = 0; js < nst; ++js) {
    const int buf = js % S;
    wait_tiles<LPT, S - 2>(nst - 1 - js);
    __syncthreads();
    if (js + S - 1 < nst) stage(js + S - 1, buf == 0 ? S - 1 : buf - 1);

    const FA_LDS char* Ks = smem + buf * TK;
    const FA_LDS char* Vs = smem + S * TK + buf * TV;
    const FA_LDS int* segs = (const FA_LDS int*)(smem + S * (TK + TV) + buf * SR * 4);
    if constexpr (KSUB == 2) {
      slot2(Ks, Vs, kt_lo + 2 * js);
      continue;
    }
#pragma unroll
    for (int sub = 0; sub < KSUB; ++sub) {
    const int kt = kt_lo + KSUB * js + sub;
    if (kt > kt_hi) break;
    const int rs = BN * sub;   // first row of this key tile in the slot
    const FA_LDS int* segk = segs + rs;
    const int k0 = kt * BN;
    const int klast = min(k0 + BN, N) - 1;

    // Wave-level tile class: nothing visible (skip), everything visible
    // (no mask), or mixed.
    bool skip = qw0 >= N;
    if (CAUSAL) skip = skip || k0 > qlast;
    bool full = (k0 + BN <= N) && (!CAUSAL || k0 + BN - 1 <= qw0);
    if (packed) {
      const int sk0 = segk[0], skl = segk[klast - k0];
      skip = skip || skl < segq_first || (!CAUSAL && sk0 > segq_last);
      full = full && (min(sk0, segq_first) == max(skl, segq_last));
    }
    if (skip) continue;

    // S^T = K Q^T, one 32-key block per accumulator.
    f32x16 sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) mma(sacc[kb], frag_row<T, D, false>(Ks, rbase, rs + 32 * kb, ks), qf[ks]);
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

    // Probabilities against the current reference; a row whose partial sum
    // reaches GROW_LIMIT (an overflow to inf included) or that has no
    // reference yet sends the wave down the rare path, which moves the
    // references to the tile's row maxima, rescales O and the sums, and
    // recomputes the probabilities.  Both lanes of a row see the same row
    // max, so they take the same decisions.
    // A wave with a row that has no reference yet (its first visible tile)
    // takes the rare path anyway, so it skips the optimistic pass.
    float ptile[KB][16];
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
    bool trigger = __builtin_amdgcn_ballot_w64(msc == -INFINITY) != 0;
    if (!trigger) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = exp2_fast(fmaf(sacc[kb][r], c, -msc));
          ptile[kb][r] = e;
          ls[r & 3] += e;
        }
      const float lpart = (ls[0] + ls[1]) + (ls[2] + ls[3]);
      trigger = __builtin_amdgcn_ballot_w64(!(lpart < GROW_LIMIT)) != 0;
    }
    if (trigger) {
      float tm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tm[r & 3] = fmaxf(tm[r & 3], sacc[kb][r]);
      float tmax = fmaxf(fmaxf(tm[0], tm[1]), fmaxf(tm[2], tm[3]));
      tmax = fmaxf(tmax, other_half(tmax));
      const float tsc = tmax * c;
      const bool grow = tsc > msc;
      // alpha is 0 on a row's first visible tile (msc = -inf), 1 if kept.
      const float alpha = grow ? exp2_fast(msc - tsc) : 1.f;
      msc = grow ? tsc : msc;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      const float mref = (msc == -INFINITY) ? 0.f : msc;
#pragma unroll
      for (int r = 0; r < 4; ++r) ls[r] = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = exp2_fast(fmaf(sacc[kb][r], c, -mref));
          ptile[kb][r] = e;
          ls[r & 3] += e;
        }
    }
    lsum += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    frag_t<T> pf[KB][2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x16 e;
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = ptile[kb][r];
      pf[kb][0] = acc_frag<T>(e, 0);
      pf[kb][1] = acc_frag<T>(e, 1);
    }

    // O^T += V^T P^T.
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          mma(oacc[db], frag_col<T, D>(Vs, cbase, rs + 32 * kb + 16 * kc, 32 * db), pf[kb][kc]);
    }
  }

  const float lt = lsum + other_half(lsum);
  if (qi < N) {
    store_rows<T, D>((T*)p.o + off, qi, oacc, 1.f / lt, lane);
    if (h == 0) p.lse[(size_t)bh * N + qi] = (msc + log2_fast(lt)) * kLn2;
  }
}

hipError_t launch_fwd(const FwdParams& p, int dtype, int D, bool causal, int nw, hipStream_t s) {
  return dispatch(dtype, D, causal, nw, [&](auto t, auto d, auto c, auto w) {
    using T = typename decltype(t)::type;
    constexpr int DD = decltype(d)::value, NW = decltype(w)::value;
    constexpr bool C = decltype(c)::value;
    const long long total = (long long)p.B * p.H * p.nqt;
    // 8-wave bf16 workgroups of dense calls take two key tiles per slot
    constexpr int KS2 = (NW == 8 && sizeof(T) == 2) ? KSUB_DENSE : 1;
    if (KS2 > 1 && p.seg == nullptr)
      hipLaunchKernelGGL((fwd_kernel<T, DD, C, NW, KS2>), dim3((unsigned)total), dim3(NW * 64), 0, s, p);
    else
      hipLaunchKernelGGL((fwd_kernel<T, DD, C, NW, 1>), dim3((unsigned)total), dim3(NW * 64), 0, s, p);
    return hipGetLastError();
  });
}

}  // namespace fa
