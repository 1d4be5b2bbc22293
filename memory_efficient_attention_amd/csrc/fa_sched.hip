// Segment-aware tile schedule for packed rows.
//
// A packed row carries a per-token segment id (mlx-train-perf changelog,
// "Added": block-diagonal causal masking from an O(N) per-token segment id),
// and a token sees another only inside its own segment (0.5.1 README,
// "Sequence packing").  With contiguous segments the keys query i can see form
// the interval [start(i), i] (causal) or [start(i), end(i) - 1], and the
// queries that can see key j form [j, end(j) - 1] (causal) or
// [start(j), end(j) - 1].  These kernels turn those intervals into per-tile
// ranges so the attention kernels walk only tiles that hold a visible pair:
// the forward and dQ skip cross-segment key blocks, and dK/dV bounds its query
// walk at each key block's segment end (README, "Sequence packing", 0.5.0).
//
// start/end come from binary search on the row, valid because ids are
// non-decreasing; rows that violate this get clamped, in-range tables (and
// the order kernel raises the workspace flag).  Workgroups then take the
// tiles longest first, so the heaviest (long-segment) tiles do not start
// last and stretch the launch.
#include "fa_internal.h"

namespace fa {

// first index in [0, n) whose id is >= v
__device__ __forceinline__ int first_at_least(const int32_t* s, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// first index in [0, n) whose id is > v
__device__ __forceinline__ int first_above(const int32_t* s, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s[mid] <= v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// For each query tile of tq rows: the first and last key tile (of tk keys)
// holding a key some query of the tile can see.
__global__ void __launch_bounds__(256) qtile_table_kernel(const int32_t* seg, int B, int N, int tq,
                                                          int tk, int causal, int2* tab) {
  const int ntiles = (N + tq - 1) / tq;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)B * ntiles) return;
  const int b = (int)(t / ntiles), qt = (int)(t % ntiles);
  const int32_t* s = seg + (size_t)b * N;
  const int q0 = qt * tq, q1 = min(q0 + tq, N) - 1;
  int lo = first_at_least(s, N, s[q0]);
  int hi = causal ? q1 : first_above(s, N, s[q1]) - 1;
  lo = clampi(lo, 0, N - 1);
  hi = clampi(hi, 0, N - 1);
  tab[t] = make_int2(lo / tk, hi / tk);
}

// For each key tile of tk keys: the first and last query tile (of tq rows)
// holding a query that can see some key of the tile.
__global__ void __launch_bounds__(256) ktile_table_kernel(const int32_t* seg, int B, int N, int tk,
                                                          int tq, int causal, int2* tab) {
  const int ntiles = (N + tk - 1) / tk;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)B * ntiles) return;
  const int b = (int)(t / ntiles), kt = (int)(t % ntiles);
  const int32_t* s = seg + (size_t)b * N;
  const int k0 = kt * tk, k1 = min(k0 + tk, N) - 1;
  int lo = causal ? k0 : first_at_least(s, N, s[k0]);
  int hi = first_above(s, N, s[k1]) - 1;
  lo = clampi(lo, 0, N - 1);
  hi = clampi(hi, 0, N - 1);
  tab[t] = make_int2(lo / tq, hi / tq);
}

// Longest-first work list from a range table of n = B * nt tiles: work[k] =
// {b, tile, first, last} with k ordered by descending range length (clamped
// to 255 tiles), by a counting sort in LDS.  Ties come out in any order; the
// order only decides which workgroup starts first, never what a workgroup
// computes.  With seg given, also flag[0] = 1 if some row's ids decrease,
// else 0.  One workgroup.
__global__ void __launch_bounds__(1024) order_kernel(const int2* tab, int n, int nt, int4* work,
                                                     const int32_t* seg, int B, int N, int32_t* flag) {
  constexpr int NB = 256;
  __shared__ int cnt[NB];
  const int tid = threadIdx.x;
  for (int i = tid; i < NB; i += 1024) cnt[i] = 0;
  __syncthreads();
  auto bucket = [&](int i) {
    const int2 r = tab[i];
    return NB - 1 - clampi(r.y - r.x + 1, 0, NB - 1);   // longest first
  };
  for (int i = tid; i < n; i += 1024) atomicAdd(&cnt[bucket(i)], 1);
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int k = 0; k < NB; ++k) {
      const int c = cnt[k];
      cnt[k] = acc;
      acc += c;
    }
  }
  __syncthreads();
  for (int i = tid; i < n; i += 1024) {
    const int2 r = tab[i];
    work[atomicAdd(&cnt[bucket(i)], 1)] = make_int4(i / nt, i % nt, r.x, r.y);
  }
  if (seg) {
    int bad = 0;
    const long long m = (long long)B * N;
    for (long long i = tid; i < m; i += 1024) {
      if ((i % N) != N - 1 && seg[i] > seg[i + 1]) bad = 1;
    }
    bad = __syncthreads_or(bad);
    if (tid == 0) flag[0] = bad ? 1 : 0;
  }
}

hipError_t launch_qtile_table(const int32_t* seg, int B, int N, int tq, int tk, bool causal,
                              int2* tab, hipStream_t s) {
  const long long n = (long long)B * ((N + tq - 1) / tq);
  hipLaunchKernelGGL(qtile_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, seg, B, N,
                     tq, tk, causal ? 1 : 0, tab);
  return hipGetLastError();
}

hipError_t launch_ktile_table(const int32_t* seg, int B, int N, int tk, int tq, bool causal,
                              int2* tab, hipStream_t s) {
  const long long n = (long long)B * ((N + tk - 1) / tk);
  hipLaunchKernelGGL(ktile_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, seg, B, N,
                     tk, tq, causal ? 1 : 0, tab);
  return hipGetLastError();
}

hipError_t launch_tile_order(const int2* tab, int B, int nt, int4* work, const int32_t* check_seg, int N,
                             int32_t* flag, hipStream_t s) {
  hipLaunchKernelGGL(order_kernel, dim3(1), dim3(1024), 0, s, tab, B * nt, nt, work, check_seg, B, N, flag);
  return hipGetLastError();
}

}  // namespace fa
