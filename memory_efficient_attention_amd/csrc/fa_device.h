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
typedef float f32x32 __attribute__((ext_vector_type(32)));
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

// Two accumulators seeded with per-row values in one instruction: the
// two-block fp32 MFMA (v_mfma_f32_32x32x1_2b_f32) forms, per block b, the
// outer product of a 32-row column (lane 32b + i holds row i) with a 32-wide
// row, into registers 16b .. 16b + 15 in the accumulator layout above.  With
// the row all ones, lane i < 32 passing x_i and lane 32 + i passing y_i,
// block 0 holds x_i in every column of row i and block 1 holds y_i: each lane
// needs only its own row's value, not the 16 rows its accumulator spans.
__device__ __forceinline__ void seed_rows(f32x16& a, f32x16& b, float v) {
  const f32x32 r = __builtin_amdgcn_mfma_f32_32x32x1f32(v, 1.0f, f32x32{}, 0, 0, 0);
  a = __builtin_shufflevector(r, r, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
  b = __builtin_shufflevector(r, r, 16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26, 27, 28, 29, 30, 31);
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
// A tile holds ROWS rows of D elements; rows sit in groups of 4, consecutive
// rows of a group S1 bytes apart, groups S4 bytes apart.  Two bf16 layouts,
// both free of bank conflicts with 64 four-byte banks:
//  * DUAL (tiles read both along rows and transposed): S1 = row + 64 bytes,
//    S4 = 4 * S1 + 16.  16 lanes reading the same 16-byte chunk of 16
//    consecutive rows (frag_row) start on 16 distinct 4-bank groups, and 32
//    lanes reading 4 consecutive rows x 64 bytes (frag_col) start 16 banks
//    apart.
//  * row-only (frag_row only): S1 = row + 16 bytes, S4 = 4 * S1, i.e. a plain
//    padded stride; 26 % smaller than DUAL at D = 128.
//  * D = 96: S1 = row, S4 = 4 * row + 16 for both (checked the same way).
// Every fragment address is a per-lane base plus a compile-time offset.  fp32
// tiles (small shapes only) are packed without padding.
template <typename T, int D, bool DUAL = true>
struct Layout {
  static constexpr int ROW = D * (int)sizeof(T);
  // D = 96 (192-byte rows) and D = 32 (64-byte rows, the K-slices of the
  // loss GEMMs): S1 = row, S4 = 4 * row + 16 serves every read pattern
  // without conflicts, so both tile kinds use it.
  static constexpr bool TIGHT = D == 96 || D == 32;
  static constexpr int PAD1 = TIGHT ? 0 : (DUAL ? 64 : 16);
  static constexpr int PAD4 = TIGHT || DUAL ? 16 : 0;
  static constexpr int S1 = sizeof(T) == 2 ? ROW + PAD1 : ROW;
  static constexpr int S4 = sizeof(T) == 2 ? 4 * S1 + PAD4 : 4 * S1;
  static constexpr int bytes(int rows) { return (rows / 4) * S4; }
  // byte offset of a row; linear in (row / 4, row % 4), so off(a + b) =
  // off(a) + off(b) whenever a is a multiple of 4
  __device__ static constexpr int off(int row) { return (row >> 2) * S4 + (row & 3) * S1; }
  // frag_row lane base: row lane % 32, 8-element chunk parity lane / 32
  __device__ static int row_base(int lane) { return off(lane & 31) + (lane >> 5) * 8 * (int)sizeof(T); }
  // frag_col lane base (see frag_col); DUAL tiles only
  __device__ static int col_base(int lane) {
    static_assert(DUAL, "transposed reads need the DUAL layout");
    const int h = lane >> 5;
    if constexpr (sizeof(T) == 2) {
      const int g = lane >> 4, r = (lane >> 2) & 3, c = lane & 3;
      return h * S4 + r * S1 + (16 * (g & 1) + 4 * c) * 2;
    } else {
      return h * S4 + (lane & 31) * 4;
    }
  }
};

// Direct global->LDS staging of ROWS rows of a (N, D) matrix into a tile.
// Each wave instruction fills 64 consecutive 16-byte LDS chunks; the lanes
// whose chunk is padding stay idle.  init() precomputes, per lane and per
// instruction, the source byte offset relative to the tile's first row.  The
// loads are buffer loads whose range is the matrix itself (N * row bytes), so
// rows >= N of a tail tile read as zeros without any clamping.
//
// The direct-to-LDS loads are issued from inline assembly.  Issued through
// the compiler builtins, they make the compiler wait for every outstanding
// LDS load before each transposing LDS read (it cannot tell which buffer the
// read touches), which serialises the next tile's loads with the current
// tile's math.  The kernels instead wait explicitly: s_waitcnt vmcnt(n) with
// n = the loads issued for the tiles still in flight behind the one needed,
// then a workgroup barrier.  Hidden from the compiler, these loads can only
// make its own vmcnt waits (for register loads) stricter, never looser.
// M0 carries the LDS address.  M0 is a register the compiler reserves (it
// cannot be declared clobbered), so these loads rely on nothing else in the
// kernels reading or writing M0; tests/test_isa_m0.py checks exactly that on
// the built code objects, so a compiler that starts using M0 fails the test
// suite instead of corrupting loads.  The compiler cannot see the hazards of
// these instructions, so each waits 5 states after its M0 write, which also
// covers an SGPR operand (descriptor, address) just written by a VALU op.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* g, int bytes) {
  const unsigned long long a = (unsigned long long)g;
  // raw buffer: base, stride 0, num_records = bytes, 32-bit data format
  return i32x4{(int)(unsigned)a, (int)((unsigned)(a >> 32) & 0xffffu), bytes, 0x00020000};
}
__device__ __forceinline__ void buffer_lds16(i32x4 rsrc, FA_LDS char* lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"((unsigned)(size_t)lds), "v"(voff), "s"(rsrc) : "memory");
}
__device__ __forceinline__ void global_lds4(const void* src, FA_LDS char* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dword %1, off"
               :: "s"((unsigned)(size_t)lds), "v"(src) : "memory");
}

template <typename T, int ROWS, int D, int NW, bool DUAL = true>
struct Stager {
  using L = Layout<T, D, DUAL>;
  static constexpr int CS1 = L::S1 / 16, CS4 = L::S4 / 16, CROW = L::ROW / 16;
  static constexpr int NCH = (ROWS / 4) * CS4;
  static constexpr int NINST = (NCH + 63) / 64;
  static constexpr int PER = (NINST + NW - 1) / NW;
  int rank;   // this wave's position in the round-robin deal of instructions
  int lane;

  static constexpr bool lane_active(int P) {
    return P < NCH && (P % CS4) / CS1 < 4 && (P % CS4) % CS1 < CROW;
  }
  // Every instruction has an active lane, so no wave ever skips one of its
  // loads (the explicit vmcnt waits count them).
  static constexpr bool every_inst_active() {
    for (int inst = 0; inst < NINST; ++inst) {
      bool any = false;
      for (int l = 0; l < 64; ++l) any = any || lane_active(inst * 64 + l);
      if (!any) return false;
    }
    return true;
  }
  static_assert(every_inst_active(), "a staging instruction would have no active lane");

  // Instruction i goes to wave (first + i) % NW.  Stagers of one tile that
  // start where the previous one ended deal their instructions round-robin as
  // a single set, so every wave issues at least floor(total / NW) of them.
  __device__ void init(int wave, int lane_, int first = 0) {
    rank = (wave - first % NW + NW) % NW;
    lane = lane_;
  }

  // g: the (N, D) matrix of this (batch, head); N * ROW < 2^31.  Each lane's
  // source offset is recomputed here (constant divisions only) rather than
  // kept in registers across the tile walk.
  __device__ void issue(FA_LDS char* tile, const T* g, int row0, int N) const {
    issue_block(tile, g, row0, N, L::ROW, 0);
  }
  // Rows row0 .. row0 + ROWS - 1, bytes col_byte0 .. col_byte0 + ROW - 1 of
  // each, of a row-major matrix of `nrows` rows, `ld_bytes` apart
  // (nrows * ld_bytes < 2^31); rows past nrows read as zeros.
  __device__ void issue_block(FA_LDS char* tile, const void* g, int row0, int nrows, int ld_bytes,
                              int col_byte0) const {
    const i32x4 rsrc = buffer_rsrc(g, nrows * ld_bytes);
    const int base = row0 * ld_bytes + col_byte0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int inst = k * NW + rank;
      const int P = inst * 64 + lane;
      const int grp = P / CS4, w = P % CS4, r = w / CS1, c = w % CS1;
      if (inst < NINST && lane_active(P))
        buffer_lds16(rsrc, tile + inst * 1024, base + (4 * grp + r) * ld_bytes + c * 16);
    }
  }
};

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
      global_lds4((const char*)g + (size_t)gr * 4, dst + base * 4);
    }
  }
}

// Makes the compiler complete, at this point, the register loads that
// produced x.  It places its vmcnt waits at first use; a first use inside the
// tile loop would be re-checked on every iteration with a wait that also
// drains the staged tiles in flight.
template <typename X>
__device__ __forceinline__ void settle(const X& x) {
  asm volatile("" :: "v"(x));
}
__device__ __forceinline__ void settle(const f32x8& x) {
  settle(f32x4{x[0], x[1], x[2], x[3]});
  settle(f32x4{x[4], x[5], x[6], x[7]});
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void wait_loads() { wait_vm<0>(); }

// Wait until the loads of the oldest staged tile have landed while `ahead`
// newer tiles (at most MAXA), PER load instructions each per wave, may still
// be in flight.  Loads complete in issue order.
template <int PER, int MAXA>
__device__ __forceinline__ void wait_tiles(int ahead) {
  if constexpr (MAXA >= 3) {
    if (ahead >= 3) return wait_vm<3 * PER>();
  }
  if constexpr (MAXA >= 2) {
    if (ahead >= 2) return wait_vm<2 * PER>();
  }
  if constexpr (MAXA >= 1) {
    if (ahead >= 1) return wait_vm<PER>();
  }
  wait_vm<0>();
}

// A/B fragment along D: 8 consecutive elements of tile row rb + lane % 32 at
// column 8 * (2 * ks + lane / 32); rb is a multiple of 4, `base` =
// Layout::row_base(lane).
template <typename T, int D, bool DUAL = true>
__device__ __forceinline__ frag_t<T> frag_row(const FA_LDS char* tile, int base, int rb, int ks) {
  using L = Layout<T, D, DUAL>;
  const FA_LDS char* p = tile + base + L::off(rb) + ks * 16 * (int)sizeof(T);
  if constexpr (sizeof(T) == 2) {
    return *(const FA_LDS bf16x8*)p;
  } else {
    const FA_LDS f32x4* q = (const FA_LDS f32x4*)p;
    f32x4 a = q[0], b = q[1];
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

// Transposed fragment: for lane l (h = l/32) the elements
//   tile[kbase + 4h + s][col0 + l%32]      for s = 0..3, then
//   tile[kbase + 8 + 4h + s][col0 + l%32]  for s = 0..3,
// i.e. the A operand whose k-slots match acc_frag(acc, kc) of a product whose
// accumulator rows are tile rows kbase .. kbase + 15 (kbase a multiple of 16;
// `base` = Layout::col_base(lane)).
//
// bf16 uses ds_read_b64_tr_b16: within each 16-lane group, lane i receives
// element i%4 of the 8 bytes fetched by lanes 4r + i/4 (r = 0..3).  So lane
// 16g + 4r + c fetches row kbase + 4h + r at columns
// col0 + 16(g%2) + 4c .. +3, and lane 16g + i ends up with column
// col0 + 16(g%2) + i of rows kbase + 4h + 0..3.
template <typename T, int D>
__device__ __forceinline__ frag_t<T> frag_col(const FA_LDS char* tile, int base, int kbase, int col0) {
  using L = Layout<T, D>;
  const FA_LDS char* p = tile + base + L::off(kbase) + col0 * (int)sizeof(T);
  if constexpr (sizeof(T) == 2) {
    s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)p);
    s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(p + 2 * L::S4));
    bf16x4 xb = __builtin_bit_cast(bf16x4, x), yb = __builtin_bit_cast(bf16x4, y);
    return bf16x8{xb[0], xb[1], xb[2], xb[3], yb[0], yb[1], yb[2], yb[3]};
  } else {
    f32x8 out;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      out[s] = *(const FA_LDS float*)(p + (s >= 4 ? 2 * L::S4 : 0) + (s & 3) * L::S1);
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
