// Forward kernel: O and the per-row log-sum-exp, never an (N, N) matrix.
//
// What is computed follows the mlx-train-perf 0.5.1 README, section
// "Flash-attention training path": the forward keeps only the attention
// output and the log-sum-exp as saved state.  Masking is causal and, for
// packed rows, block-diagonal by segment id (same README, "Sequence packing";
// changelog "Added": the PACKED forward variant).
//
// One workgroup = FWD_WAVES waves of one (batch, head).  Each wave owns
// FWD_QBW blocks of 32 queries and computes S^T = K Q^T for a 64-key tile
// (32x32 MFMA tiles), so the softmax statistics of a query live in one lane
// pair (l, l+32); every K and V^T fragment read from LDS feeds FWD_QBW MFMAs.  Q^T stays in registers for the whole key walk; K and V tiles are
// double-buffered in LDS with direct global->LDS loads.  O^T += V^T P^T takes
// P^T straight from the accumulator and V^T from the V tile through the
// transposing LDS read.  Causal / packed structure is used at wave
// granularity: key tiles no query of a wave can see are skipped, tiles every
// query sees fully skip the per-element mask.  The running reference max
// moves only when a row's max grows by more than 2^RESCALE_LOG2, so the O
// rescale is a rare, wave-uniform branch.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(FWD_WAVES * 64, FA_FWD_WPE) fwd_kernel(const FwdParams p) {
  constexpr int NW = FWD_WAVES, QBW = FWD_QBW, QW = 32 * QBW, BM = FWD_BM, BN = KEY_TILE;
  constexpr int KS = D / 16, DB = D / 32, KB = BN / 32;
  // K is read only along rows (row-only layout), V only transposed (DUAL).
  using LK = Layout<T, D, false>;
  using LV = Layout<T, D, true>;
  using StK = Stager<T, BN, D, NW, false>;
  using StV = Stager<T, BN, D, NW, true>;
  constexpr int TK = LK::bytes(BN), TV = LV::bytes(BN);
  // layout: K[2] | V[2] | seg[2]
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * TK + 2 * TV + 2 * BN * 4];
  FA_LDS char* smem = (FA_LDS char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  const int N = p.N;

  const int total = p.B * p.H * p.nqt;
  const int Lw = xcd_remap(blockIdx.x, total);
  const int bh = Lw / p.nqt;
  const int qt = p.nqt - 1 - (Lw - bh * p.nqt);   // longest query tiles first
  const int b = bh / p.H;
  const size_t off = (size_t)bh * N * D;
  const T* gq = (const T*)p.q + off;
  const T* gk = (const T*)p.k + off;
  const T* gv = (const T*)p.v + off;
  const int32_t* seg = p.seg ? p.seg + (size_t)b * N : nullptr;
  const bool packed = seg != nullptr;

  // The wave owns queries qw0 .. qw0 + QW - 1, in QBW blocks of 32; lane l
  // holds query qw0 + 32 qb + l % 32 of block qb.
  const int q0 = qt * BM;
  const int qw0 = q0 + wave * QW;
  const int qlast = min(qw0 + QW - 1, N - 1);

  int kt_lo = 0, kt_hi;
  if (packed) {
    const int2 r = p.qtab[(size_t)b * p.nqt + qt];
    kt_lo = r.x;
    kt_hi = r.y;
  } else {
    kt_hi = ((CAUSAL ? min(q0 + BM, N) : N) - 1) / BN;
  }

  frag_t<T> qf[QBW][KS];
  int segq[QBW];
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const int qc = min(qw0 + 32 * qb + col, N - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[qb][ks] = gfrag_row<T, D>(gq, qc, 2 * ks + h);
    segq[qb] = packed ? seg[qc] : 0;
  }
  int segq_first = 0, segq_last = 0;
  if (packed) {
    segq_first = seg[min(qw0, N - 1)];
    segq_last = seg[qlast];
  }

  StK stk;
  StV stv;
  stk.init(wave, lane);
  stv.init(wave, lane);
  const int rbase = LK::row_base(lane);
  const int cbase = LV::col_base(lane);

  f32x16 oacc[QBW][DB];
  float msc[QBW], lsum[QBW];   // reference max (times c, log2 units), lane's half of the row sum
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qb][db] = f32x16{};
    msc[qb] = -INFINITY;
    lsum[qb] = 0.f;
  }
  const float c = p.c;

  auto stage = [&](int kt, int buf) {
    stk.issue(smem + buf * TK, gk, kt * BN, N, wave);
    stv.issue(smem + 2 * TK + buf * TV, gv, kt * BN, N, wave);
    if (packed) stage_vec<BN>(smem + 2 * TK + 2 * TV + buf * BN * 4, seg, kt * BN, N, wave, NW - 1, lane);
  };

  if (kt_lo <= kt_hi) stage(kt_lo, 0);
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int buf = (kt - kt_lo) & 1;
    wait_loads();
    __syncthreads();
    if (kt < kt_hi) stage(kt + 1, buf ^ 1);

    const FA_LDS char* Ks = smem + buf * TK;
    const FA_LDS char* Vs = smem + 2 * TK + buf * TV;
    const FA_LDS int* segk = (const FA_LDS int*)(smem + 2 * TK + 2 * TV + buf * BN * 4);
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

    // S^T = K Q^T, key block by key block (so that block 0's softmax can run
    // under block 1's MFMAs); each K fragment feeds the QBW query blocks.
    f32x16 sacc[QBW][KB];
    prio_hi();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) sacc[qb][kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const frag_t<T> a = frag_row<T, D, false>(Ks, rbase, 32 * kb, ks);
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb) mma(sacc[qb][kb], a, qf[qb][ks]);
      }
    }
    prio_lo();

    if (!full) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kr = 32 * kb + 8 * j + 4 * h;
          i32x4 sk = packed ? *(const FA_LDS i32x4*)(segk + kr) : i32x4{0, 0, 0, 0};
#pragma unroll
          for (int qb = 0; qb < QBW; ++qb) {
            const int qi = qw0 + 32 * qb + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = k0 + kr + i;
              const bool vis = key < N && (!CAUSAL || key <= qi) && (!packed || sk[i] == segq[qb]);
              if (!vis) sacc[qb][kb][4 * j + i] = -INFINITY;
            }
          }
        }
      }
    }

    // Online softmax in base 2 with a lazily moved reference max.  The
    // probabilities are computed against the current reference first; only
    // when some row's max outgrows it by 2^RESCALE_LOG2 (rare) is the
    // reference moved, O and the sum rescaled, and the tile's probabilities
    // recomputed.  Both lanes of a pair hold the same query and take the same
    // decisions; row max and row sum run as 4 independent chains.
    float ptile[QBW][KB][16];
    float ls[QBW][4];
    bool grow[QBW];
    float tsc[QBW];
    bool any_grow = false;
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      const float mref = (msc[qb] == -INFINITY) ? 0.f : msc[qb];
      float tm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int r = 0; r < 4; ++r) ls[qb][r] = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float sv = sacc[qb][kb][r];
          tm[r & 3] = fmaxf(tm[r & 3], sv);
          const float e = exp2_fast(fmaf(sv, c, -mref));
          ptile[qb][kb][r] = e;
          ls[qb][r & 3] += e;
        }
      float tmax = fmaxf(fmaxf(tm[0], tm[1]), fmaxf(tm[2], tm[3]));
      tmax = fmaxf(tmax, other_half(tmax));
      tsc[qb] = tmax * c;
      grow[qb] = tsc[qb] > msc[qb] + RESCALE_LOG2;
      any_grow = any_grow || grow[qb];
    }
    if (__builtin_amdgcn_ballot_w64(any_grow) != 0) {
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) {
        // alpha is 1 for rows that keep their reference (also when it is
        // still -inf: no visible key yet), 0 for a row's first visible tile.
        const float alpha = grow[qb] ? exp2_fast(msc[qb] - tsc[qb]) : 1.f;
        msc[qb] = grow[qb] ? tsc[qb] : msc[qb];
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
        const float mref = (msc[qb] == -INFINITY) ? 0.f : msc[qb];
#pragma unroll
        for (int r = 0; r < 4; ++r) ls[qb][r] = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = exp2_fast(fmaf(sacc[qb][kb][r], c, -mref));
            ptile[qb][kb][r] = e;
            ls[qb][r & 3] += e;
          }
      }
    }
    frag_t<T> pf[QBW][KB][2];
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      lsum[qb] += (ls[qb][0] + ls[qb][1]) + (ls[qb][2] + ls[qb][3]);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        f32x16 e;
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = ptile[qb][kb][r];
        pf[qb][kb][0] = acc_frag<T>(e, 0);
        pf[qb][kb][1] = acc_frag<T>(e, 1);
      }
    }

    // O^T += V^T P^T: each V^T fragment feeds the QBW query blocks.
    prio_hi();
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const frag_t<T> a = frag_col<T, D>(Vs, cbase, 32 * kb + 16 * kc, 32 * db);
#pragma unroll
          for (int qb = 0; qb < QBW; ++qb) mma(oacc[qb][db], a, pf[qb][kb][kc]);
        }
    prio_lo();
  }

#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const float lt = lsum[qb] + other_half(lsum[qb]);
    const int qi = qw0 + 32 * qb + col;
    if (qi < N) {
      store_rows<T, D>((T*)p.o + off, qi, oacc[qb], 1.f / lt, lane);
      if (h == 0) p.lse[(size_t)bh * N + qi] = (msc[qb] + log2_fast(lt)) * kLn2;
    }
  }
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t s) {
  const long long total = (long long)p.B * p.H * p.nqt;
  hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL>), dim3((unsigned)total), dim3(FWD_WAVES * 64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, int dtype, int D, bool causal, hipStream_t s) {
  if (dtype == 0) {
    if (D == 128) return causal ? launch_fwd_t<bf16, 128, true>(p, s) : launch_fwd_t<bf16, 128, false>(p, s);
    return causal ? launch_fwd_t<bf16, 64, true>(p, s) : launch_fwd_t<bf16, 64, false>(p, s);
  }
  if (D == 128) return causal ? launch_fwd_t<float, 128, true>(p, s) : launch_fwd_t<float, 128, false>(p, s);
  return causal ? launch_fwd_t<float, 64, true>(p, s) : launch_fwd_t<float, 64, false>(p, s);
}

}  // namespace fa
