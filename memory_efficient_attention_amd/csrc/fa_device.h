// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// Matrix products use the 32x32 MFMA tile (v_mfma_f32_32x32x16_bf16 for bf16,
// eight v_mfma_f32_32x32x2_f32 for fp32).  Its fp32 accumulator layout puts,
// in lane l, column l%32 and rows 8*j + 4*(l/32) + i (j, i in 0..3) at
// acc[4*j + i].  Operands are 8-element fragments per lane: an A fragment
// holds row l%32 and a B fragment column l%32, both at k-slots 8*(l/32)..+7.
//
// The kernels contract over the sequence dimension with the probability or
// dS tile as the B operand taken straight from a previous product's
// accumulator: the 16 accumulator rows 16*kc + {8j+4h+i : j in {2kc, 2kc+1}}
// that lane l holds for k-chunk kc are acc[8*kc .. 8*kc+7], and that set of
// rows is used as the lane's 8 k-slots.  The other operand must then present
// the same rows in the same order: frag_col() below does that from a
// row-major LDS tile with the gfx950 transposing LDS read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct Frag;
template <> struct Frag<bf16> { using type = bf16x8; };
template <> struct Frag<float> { using type = f32x8; };
template <typename T> using frag_t = typename Frag<T>::type;

// ---------------------------------------------------------------- MFMA
__device__ __forceinline__ void mma(f32x16& acc, bf16x8 a, bf16x8 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& acc, f32x8 a, f32x8 b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], acc, 0, 0, 0);
}

// acc[8*kc .. 8*kc+7] as a B fragment (round to nearest even for bf16).
template <typename T> __device__ __forceinline__ frag_t<T> acc_frag(const f32x16& acc, int kc);
template <> __device__ __forceinline__ bf16x8 acc_frag<bf16>(const f32x16& acc, int kc) {
  f32x8 x;
#pragma unroll
  for (int s = 0; s < 8; ++s) x[s] = acc[8 * kc + s];
  return __builtin_convertvector(x, bf16x8);
}
template <> __device__ __forceinline__ f32x8 acc_frag<float>(const f32x16& acc, int kc) {
  f32x8 x;
#pragma unroll
  for (int s = 0; s < 8; ++s) x[s] = acc[8 * kc + s];
  return x;
}

// ---------------------------------------------------------------- math
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float other_half(float x) { return __shfl_xor(x, 32); }

// ---------------------------------------------------------------- LDS tiles
// A tile holds ROWS rows of D elements, row-major, rows packed back to back
// (row stride D * sizeof(T) bytes).  For bf16 the 16-byte chunks of a row
// are permuted by an XOR with swz(row) so that both read patterns used here
// hit 64 distinct banks: 16 lanes reading one chunk column of 16 consecutive
// rows (frag_row), and 32 lanes reading 4 rows x 4 chunks (frag_col).
template <typename T, int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (sizeof(T) != 2) {
    return 0;
  } else if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    static_assert(D == 64, "head_dim");
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  }
}

template <typename T, int D>
__device__ __forceinline__ uint32_t tile_off(int row, int chunk) {
  return (uint32_t)(row * D * (int)sizeof(T) + ((chunk ^ swz<T, D>(row)) << 4));
}

// Issue direct global->LDS loads of rows [row0, row0 + ROWS) of a (N, D)
// matrix into a tile.  Rows >= N read row N - 1 (finite data the masks
// discard).  Each wave instruction fills 64 consecutive 16-byte LDS chunks;
// the swizzle is applied by choosing which global chunk each lane fetches.
template <typename T, int ROWS, int D, int NT>
__device__ __forceinline__ void stage_tile(FA_LDS char* tile, const T* g, int row0, int N,
                                           int wave, int lane) {
  constexpr int CPR = D * (int)sizeof(T) / 16;
  constexpr int CHUNKS = ROWS * CPR;
  static_assert(CHUNKS % 64 == 0, "tile must be a whole number of wave loads");
  constexpr int WAVES = NT / 64;
#pragma unroll
  for (int base = 0; base < CHUNKS; base += NT) {
    const int wbase = base + wave * 64;
    if (CHUNKS % NT == 0 || wbase < CHUNKS) {
      const int P = wbase + lane;
      const int r = P / CPR;
      const int c = (P % CPR) ^ swz<T, D>(r);
      const int gr = min(row0 + r, N - 1);
      const char* src = (const char*)(g + (size_t)gr * D) + (c << 4);
      __builtin_amdgcn_global_load_lds(src, (FA_LDS void*)(tile + wbase * 16), 16, 0, 0);
    }
  }
  (void)WAVES;
}

// Direct global->LDS load of ROWS consecutive 4-byte values (row0 + i, i <
// ROWS, clamped to N - 1) by wave `wave_id` of the workgroup.
template <int ROWS>
__device__ __forceinline__ void stage_vec(FA_LDS char* dst, const void* g, int row0, int N,
                                          int wave, int wave_id, int lane) {
  static_assert(ROWS % 64 == 0 || ROWS < 64, "vector tile");
#pragma unroll
  for (int base = 0; base < ROWS; base += 64) {
    if (wave == wave_id && base + lane < ROWS) {
      const int gr = min(row0 + base + lane, N - 1);
      __builtin_amdgcn_global_load_lds((const char*)g + (size_t)gr * 4,
                                       (FA_LDS void*)(dst + base * 4), 4, 0, 0);
    }
  }
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 8 consecutive elements of `row` starting at column 8 * c8 (A/B fragment
// along D).
template <typename T, int D>
__device__ __forceinline__ frag_t<T> frag_row(const FA_LDS char* tile, int row, int c8) {
  if constexpr (sizeof(T) == 2) {
    return *(const FA_LDS bf16x8*)(tile + tile_off<T, D>(row, c8));
  } else {
    const FA_LDS f32x4* p = (const FA_LDS f32x4*)(tile + tile_off<T, D>(row, 2 * c8));
    f32x4 a = p[0], b = p[1];
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

// Transposed fragment: for lane l (h = l/32) the elements
//   tile[kbase + 4h + s][col0 + l%32]      for s = 0..3, then
//   tile[kbase + 8 + 4h + s][col0 + l%32]  for s = 0..3,
// i.e. the A operand whose k-slots match acc_frag(acc, kc) of a product whose
// accumulator rows are tile rows kbase .. kbase + 15.
//
// bf16 uses ds_read_b64_tr_b16: within each 16-lane group, lane i receives
// element i%4 of the 8 bytes fetched by lanes 4r + i/4 (r = 0..3).  So lane
// 16g + 4r + c fetches row kbase + 4h + r at columns
// col0 + 16(g%2) + 4c .. +3, and lane 16g + i ends up with column
// col0 + 16(g%2) + i of rows kbase + 4h + 0..3.
template <typename T, int D>
__device__ __forceinline__ frag_t<T> frag_col(const FA_LDS char* tile, int kbase, int col0, int lane) {
  const int h = lane >> 5;
  if constexpr (sizeof(T) == 2) {
    const int g = lane >> 4, r = (lane >> 2) & 3, c = lane & 3;
    const int e = col0 + 16 * (g & 1) + 4 * c;
    const int row1 = kbase + 4 * h + r, row2 = row1 + 8;
    const uint32_t off1 = tile_off<T, D>(row1, e >> 3) + ((e & 4) << 1);
    const uint32_t off2 = tile_off<T, D>(row2, e >> 3) + ((e & 4) << 1);
    s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(tile + off1));
    s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(tile + off2));
    bf16x4 xb = __builtin_bit_cast(bf16x4, x), yb = __builtin_bit_cast(bf16x4, y);
    return bf16x8{xb[0], xb[1], xb[2], xb[3], yb[0], yb[1], yb[2], yb[3]};
  } else {
    const int col = col0 + (lane & 31);
    f32x8 out;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int row = kbase + (s < 4 ? 4 * h + s : 8 + 4 * h + (s - 4));
      out[s] = *(const FA_LDS float*)(tile + row * D * 4 + col * 4);
    }
    return out;
  }
}

// 8 consecutive elements of a row of a (N, D) global matrix at column 8 * c8.
template <typename T, int D>
__device__ __forceinline__ frag_t<T> gfrag_row(const T* g, int row, int c8) {
  return *(const frag_t<T>*)(g + (size_t)row * D + 8 * c8);
}

// Store a (D x 32) accumulator set acc[db] (rows d, column = sequence index
// `row` of lane l%32) scaled by `f` into a (N, D) row-major global matrix.
template <typename T, int D>
__device__ __forceinline__ void store_rows(T* g, int row, const f32x16* acc, float f, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * db + 8 * j + 4 * h;
      f32x4 x = {acc[db][4 * j] * f, acc[db][4 * j + 1] * f, acc[db][4 * j + 2] * f,
                 acc[db][4 * j + 3] * f};
      if constexpr (sizeof(T) == 2) {
        *(bf16x4*)(g + (size_t)row * D + d) = __builtin_convertvector(x, bf16x4);
      } else {
        *(f32x4*)(g + (size_t)row * D + d) = x;
      }
    }
  }
}

// Workgroup index -> logical work index.  Workgroups are dealt round-robin to
// the 8 XCDs (each with its own L2); this gives each XCD a contiguous range of
// logical indices so that the tiles of one head run on one XCD.
__device__ __forceinline__ int xcd_remap(int p, int total) {
  if (total % 8 != 0) return p;
  return (p % 8) * (total / 8) + p / 8;
}

}  // namespace fa
