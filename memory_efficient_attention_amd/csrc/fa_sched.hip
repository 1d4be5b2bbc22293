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

// The visible range of tile `it` of batch row b for one table job: a
// query-tile job (keys = 0) gives the first and last tile of `other` keys
// holding a key some query of the tile can see; a key-tile job (keys = 1)
// the first and last tile of `other` queries holding a query that can see
// some key of the tile.
__device__ int2 tile_range(const int32_t* seg, int N, int causal, const TableJob& J, int b, int it) {
  const int32_t* s = seg + (size_t)b * N;
  const int r0 = it * J.tile, r1 = min(r0 + J.tile, N) - 1;
  int lo, hi;
  if (J.keys) {
    lo = causal ? r0 : first_at_least(s, N, s[r0]);
    hi = first_above(s, N, s[r1]) - 1;
  } else {
    lo = first_at_least(s, N, s[r0]);
    hi = causal ? r1 : first_above(s, N, s[r1]) - 1;
  }
  lo = clampi(lo, 0, N - 1);
  hi = clampi(hi, 0, N - 1);
  return make_int2(lo / J.other, hi / J.other);
}

// Per-tile visible ranges, for one or two tables in one launch (blockIdx.y
// selects the job), one thread per tile.
__global__ void __launch_bounds__(256) table_kernel(const int32_t* seg, int B, int N, int causal,
                                                    TableJobs jobs) {
  const TableJob J = jobs.j[blockIdx.y];
  const int ntiles = (N + J.tile - 1) / J.tile;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)B * ntiles) return;
  J.tab[t] = tile_range(seg, N, causal, J, (int)(t / ntiles), (int)(t % ntiles));
}

// Longest-first work list from a range table of n = B * nt tiles: work[k] =
// {b, tile, first, last} with k ordered by descending range length (clamped
// to 255 tiles), by a counting sort in LDS.  Ties come out in any order; the
// order only decides which workgroup starts first, never what a workgroup
// computes.  A job with `check` set also writes flag[0] = 1 if some row's
// ids decrease, else 0.  One workgroup per job.  With `fused` (every job has
// at most ORDER_THREADS tiles) thread i computes tile i's range itself, so
// the table launch is skipped; larger jobs read the table_kernel's output.
constexpr int ORDER_THREADS = 1024;
__global__ void __launch_bounds__(ORDER_THREADS) order_kernel(const int32_t* seg, int B, int N, int causal,
                                                              int32_t* flag, OrderJobs jobs, TableJobs tables,
                                                              int fused) {
  constexpr int NB = 256;
  __shared__ int cnt[NB];
  __shared__ int wsum[NB / 64];
  const OrderJob J = jobs.j[blockIdx.x];
  const int n = B * J.nt;
  const int tid = threadIdx.x;
  int2 mine = make_int2(0, -1);
  if (fused && tid < n) mine = tile_range(seg, N, causal, tables.j[blockIdx.x], tid / J.nt, tid % J.nt);
  for (int i = tid; i < NB; i += ORDER_THREADS) cnt[i] = 0;
  __syncthreads();
  // fused: i is always this thread's own tile (n <= ORDER_THREADS)
  auto range = [&](int i) { return fused ? mine : J.tab[i]; };
  auto bucket = [&](int i) {
    const int2 r = range(i);
    return NB - 1 - clampi(r.y - r.x + 1, 0, NB - 1);   // longest first
  };
  for (int i = tid; i < n; i += ORDER_THREADS) atomicAdd(&cnt[bucket(i)], 1);
  __syncthreads();
  // exclusive prefix sum of the bucket counts: a shuffle scan within each of
  // the first NB / 64 waves, then the preceding waves' totals
  int own = 0, incl = 0;
  if (tid < NB) {
    own = cnt[tid];
    incl = own;
    const int lane = tid & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    if (lane == 63) wsum[tid >> 6] = incl;
  }
  __syncthreads();
  if (tid < NB) {
    int base = 0;
    for (int w = 0; w < (tid >> 6); ++w) base += wsum[w];
    cnt[tid] = base + incl - own;
  }
  __syncthreads();
  for (int i = tid; i < n; i += ORDER_THREADS) {
    const int2 r = range(i);
    J.work[atomicAdd(&cnt[bucket(i)], 1)] = make_int4(i / J.nt, i % J.nt, r.x, r.y);
  }
  if (J.check) {
    int bad = 0;
    const long long m = (long long)B * N;
    for (long long i = tid; i < m; i += ORDER_THREADS) {
      if ((i % N) != N - 1 && seg[i] > seg[i + 1]) bad = 1;
    }
    bad = __syncthreads_or(bad);
    if (tid == 0) flag[0] = bad ? 1 : 0;
  }
}

hipError_t launch_schedule(const int32_t* seg, int B, int N, bool causal, const TableJobs& tables,
                           const OrderJobs& orders, int njobs, int32_t* flag, hipStream_t s) {
  long long n = 0;
  for (int j = 0; j < njobs; ++j) {
    const long long nj = (long long)B * ((N + tables.j[j].tile - 1) / tables.j[j].tile);
    n = nj > n ? nj : n;
  }
  // small schedules (one tile per thread of the order kernel) take one
  // launch instead of two
  const int fused = n <= ORDER_THREADS ? 1 : 0;
  if (!fused) {
    hipLaunchKernelGGL(table_kernel, dim3((unsigned)((n + 255) / 256), (unsigned)njobs), dim3(256), 0, s, seg,
                       B, N, causal ? 1 : 0, tables);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  hipLaunchKernelGGL(order_kernel, dim3((unsigned)njobs), dim3(ORDER_THREADS), 0, s, seg, B, N, causal ? 1 : 0,
                     flag, orders, tables, fused);
  return hipGetLastError();
}

}  // namespace fa
