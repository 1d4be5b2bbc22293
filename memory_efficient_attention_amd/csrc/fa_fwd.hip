// Forward kernel: O and the per-row log-sum-exp, never an (N, N) matrix.
//
// What is computed follows the mlx-train-perf 0.5.1 README, section
// "Flash-attention training path": the forward keeps only the attention
// output and the log-sum-exp as saved state.  Masking is causal and, for
// packed rows, block-diagonal by segment id (same README, "Sequence packing";
// changelog "Added": the PACKED forward variant).
//
// One workgroup = 8 waves = 256 queries of one (batch, head).  Each wave owns
// 32 queries and computes S^T = K Q^T for a 64-key tile (two 32x32 MFMA
// tiles), so the softmax statistics of a query live in one lane pair (l,
// l+32).  Q^T stays in registers for the whole key walk; K and V tiles are
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
__global__ void __launch_bounds__(FWD_WAVES * 64) fwd_kernel(const FwdParams p) {
  constexpr int NW = FWD_WAVES, BM = FWD_BM, BN = KEY_TILE;
  constexpr int KS = D / 16, DB = D / 32, KB = BN / 32;
  using L = Layout<T, D>;
  using St = Stager<T, BN, D, NW>;
  constexpr int TILE = L::bytes(BN);
  __shared__ __attribute__((aligned(1024))) char smem_raw[4 * TILE + 2 * BN * 4];
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

  const int q0 = qt * BM;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + col;
  const int qc = min(qi, N - 1);
  const int qlast = min(qw0 + 31, N - 1);

  int kt_lo = 0, kt_hi;
  if (packed) {
    const int2 r = p.qtab[(size_t)b * p.nqt + qt];
    kt_lo = r.x;
    kt_hi = r.y;
  } else {
    kt_hi = ((CAUSAL ? min(q0 + BM, N) : N) - 1) / BN;
  }

  frag_t<T> qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = gfrag_row<T, D>(gq, qc, 2 * ks + h);
  int segq = 0, segq_first = 0, segq_last = 0;
  if (packed) {
    segq = seg[qc];
    segq_first = seg[min(qw0, N - 1)];
    segq_last = seg[qlast];
  }

  St st;
  st.init(wave, lane);
  const int rbase = L::row_base(lane);
  const int cbase = L::col_base(lane);

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float msc = -INFINITY;   // reference max of the row, times c (log2 units)
  float lsum = 0.f;        // this lane's half of the row sum, relative to msc
  const float c = p.c;

  auto stage = [&](int kt, int buf) {
    st.issue(smem + buf * TILE, gk, kt * BN, N, wave);
    st.issue(smem + (2 + buf) * TILE, gv, kt * BN, N, wave);
    if (packed) stage_vec<BN>(smem + 4 * TILE + buf * BN * 4, seg, kt * BN, N, wave, NW - 1, lane);
  };

  if (kt_lo <= kt_hi) stage(kt_lo, 0);
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int buf = (kt - kt_lo) & 1;
    wait_loads();
    __syncthreads();
    if (kt < kt_hi) stage(kt + 1, buf ^ 1);

    const FA_LDS char* Ks = smem + buf * TILE;
    const FA_LDS char* Vs = smem + (2 + buf) * TILE;
    const FA_LDS int* segk = (const FA_LDS int*)(smem + 4 * TILE + buf * BN * 4);
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

    // S^T = K Q^T for the wave's 32 queries.
    f32x16 sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) mma(sacc[kb], frag_row<T, D>(Ks, rbase, 32 * kb, ks), qf[ks]);
    }

    if (!full) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kr = 32 * kb + 8 * j + 4 * h;
          i32x4 sk = packed ? *(const FA_LDS i32x4*)(segk + kr) : i32x4{0, 0, 0, 0};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = k0 + kr + i;
            const bool vis = key < N && (!CAUSAL || key <= qi) && (!packed || sk[i] == segq);
            if (!vis) sacc[kb][4 * j + i] = -INFINITY;
          }
        }
      }
    }

    // Online softmax in base 2 with a lazily moved reference max.  Both lanes
    // of a pair hold the same query and take the same decisions.
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[kb][r]);
    tmax = fmaxf(tmax, other_half(tmax));
    const float tsc = tmax * c;
    const bool grow = tsc > msc + RESCALE_LOG2;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      // alpha is 1 for rows that keep their reference (also when it is still
      // -inf: no visible key yet), and 0 for a row's first visible tile.
      const float alpha = grow ? exp2_fast(msc - tsc) : 1.f;
      msc = grow ? tsc : msc;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const float mref = (msc == -INFINITY) ? 0.f : msc;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2_fast(fmaf(sacc[kb][r], c, -mref));
        sacc[kb][r] = e;
        lsum += e;
      }

    // O^T += V^T P^T.
    frag_t<T> pf[KB][2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      pf[kb][0] = acc_frag<T>(sacc[kb], 0);
      pf[kb][1] = acc_frag<T>(sacc[kb], 1);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          mma(oacc[db], frag_col<T, D>(Vs, cbase, 32 * kb + 16 * kc, 32 * db), pf[kb][kc]);
  }

  const float lt = lsum + other_half(lsum);
  if (qi < N) {
    store_rows<T, D>((T*)p.o + off, qi, oacc, 1.f / lt, lane);
    if (h == 0) p.lse[(size_t)bh * N + qi] = (msc + log2_fast(lt)) * kLn2;
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
