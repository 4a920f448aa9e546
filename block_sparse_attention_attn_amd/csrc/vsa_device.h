// vsa_device.h -- device-side building blocks shared by the gfx950 kernels of the 64-token
// block-sparse attention library: vector types, MFMA wrappers, the LDS tile swizzles, the
// transposing LDS read and the global->LDS copy.
//
// Lane layouts (verified on gfx950 with an in-bounds probe):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] B[16x32]
//     A: lane l holds A[m = l%32][k = 8*(l/32) + j], j = 0..7 (8 bf16)
//     B: lane l holds B[k = 8*(l/32) + j][n = l%32]
//     D: lane l holds D[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32], i = 0..15 (16 fp32)
//   v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] B[32x16]
//     A: lane l holds A[m = l%16][k = 8*(l/16) + j]; B: B[k = 8*(l/16) + j][n = l%16]
//     D: lane l holds D[m = 4*(l/16) + i][n = l%16], i = 0..3
//   ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives element j (j = 0..3) as
//     element i%4 of the 8 bytes addressed by lane 4*j + i/4 of the group. So when lanes
//     4r..4r+3 address the 16 contiguous bf16 of row r (r = 0..3), lane i gets column i of that
//     4 x 16 block: a transposed read.
//   global_load_lds_dwordx4: lane l's 16 bytes land at LDS base + 16*l.
//
// The contraction index of an MFMA may be permuted freely as long as A and B use the same
// permutation; the kernels use that to feed a D fragment straight back as an operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vsa {

constexpr int BLOCK = 64;      // tokens per sparse block
constexpr int HEAD_DIM = 128;  // head dimension

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef _Float16 f16;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;

#define VSA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Two transposed 8-byte LDS reads joined into one 8-element MFMA operand.
__device__ __forceinline__ bf16x8 join(s16x4 lo, s16x4 hi) {
  union {
    s16x4 h[2];
    bf16x8 v;
  } u;
  u.h[0] = lo;
  u.h[1] = hi;
  return u.v;
}

__device__ __forceinline__ f16x8 join_f16(s16x4 lo, s16x4 hi) {
  union {
    s16x4 h[2];
    f16x8 v;
  } u;
  u.h[0] = lo;
  u.h[1] = hi;
  return u.v;
}

__device__ __forceinline__ s16x4 lds_read_tr(const VSA_LDS void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((VSA_LDS s16x4*)p);
}

// Max and sum of a lane's value with the value of lane l ^ 32, through v_permlane32_swap (a VALU
// lane swap, no LDS traffic): swapping a register with itself leaves the values of lanes l % 32
// and 32 + l % 32 in the two halves of the result, in that order for both lanes of the pair, so
// the two lanes get bitwise equal results.
__device__ __forceinline__ float pair_max32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Eight fp32 values to one bf16x8 operand, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4,
                                        float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (bf16)a0;
  r[1] = (bf16)a1;
  r[2] = (bf16)a2;
  r[3] = (bf16)a3;
  r[4] = (bf16)a4;
  r[5] = (bf16)a5;
  r[6] = (bf16)a6;
  r[7] = (bf16)a7;
  return r;
}

// Eight fp32 values to one f16x8 operand, round-to-nearest-even (v_cvt_pk_f16_f32).
__device__ __forceinline__ f16x8 pack8_f16(float a0, float a1, float a2, float a3, float a4,
                                           float a5, float a6, float a7) {
  f16x8 r;
  r[0] = (f16)a0;
  r[1] = (f16)a1;
  r[2] = (f16)a2;
  r[3] = (f16)a3;
  r[4] = (f16)a4;
  r[5] = (f16)a5;
  r[6] = (f16)a6;
  r[7] = (f16)a7;
  return r;
}

// floor(log2(x)) - top for a non-negative fp32 value given by its bits (the largest |value| of a
// tile or head, as an integer max over bit patterns keeps it): the power-of-two exponent e with
// x * 2^-e in [2^top, 2^(top+1)). 0 for x = 0 and for inf/NaN (those propagate either way).
__device__ __forceinline__ int f16_exponent(uint32_t amax_bits, int top) {
  const int ex = (int)((amax_bits >> 23) & 0xFF);
  if (ex == 255 || amax_bits == 0) return 0;
  // floor(log2(max)) for normal and subnormal fp32 values
  const int l2 = ex > 0 ? ex - 127 : -118 - __builtin_clz(amax_bits & 0x7FFFFF);
  return l2 - top;
}
// The exponent that brings a head's largest |value| into [2^14, 2^15): an fp16 copy x * 2^-e then
// holds every bf16 value of magnitude >= 2^-28 * max exactly (8 significant bits in fp16's normal
// range).
__device__ __forceinline__ int f16_head_exponent(uint32_t amax_bits) {
  return f16_exponent(amax_bits, 14);
}
// bf16 -> fp32 -> times 2^-e -> fp16 (round to nearest even): exact for values that land in fp16's
// normal range after the scaling.
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(bf16x8 x, int e) {
  f16x8 y;
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = (f16)__builtin_ldexpf((float)x[k], -e);
  return y;
}
// The largest |x| of a bf16x8 as fp32 bits (sign cleared, shifted into fp32 position).
__device__ __forceinline__ uint32_t absmax_bits8(bf16x8 x) {
  union {
    bf16x8 b;
    uint32_t u[4];
  } r;
  r.b = x;
  uint32_t m = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) m = max(m, max(r.u[e] & 0x7FFFu, (r.u[e] >> 16) & 0x7FFFu));
  return m << 16;
}

// ---------------------------------------------------------------------------------------------
// LDS tile formats
// ---------------------------------------------------------------------------------------------
// A [64 rows][128] tile of 16-bit values (Q, dO, K, V in bf16 or fp16) occupies 16 KiB = 64 rows x 16 chunks of 16 bytes; a
// row is exactly the 64 banks x 4 bytes of LDS, so the bank group of a chunk is its slot in the
// row. Chunk cc of row r is stored at chunk slot r*16 + (cc ^ swz128(r)) with
// swz128(r) = ((r >> 2) & 3) | ((r & 3) << 2), a swap of the row's two low bit pairs:
//   * 16 lanes reading the same chunk of 16 aligned rows (an MFMA operand read, ds_read_b128)
//     see swz128 take all 16 values: 16 different bank groups;
//   * 32 lanes of a transposed read (ds_read_b64_tr_b16) cover 4 aligned rows x 4 aligned chunks:
//     the chunk's low bits XOR a row constant, its high bits XOR the row's low bits, so the 16
//     (row, chunk) pairs land in 16 different bank groups.
__device__ __forceinline__ int swz128(int r) { return ((r >> 2) & 3) | ((r & 3) << 2); }
__device__ __forceinline__ int tile_byte(int r, int cc) {  // byte offset of chunk cc of row r
  return (r * 16 + (cc ^ swz128(r))) * 16;
}
// Byte offset of element (r, c) (c = column 0..127, a multiple of 4 for 8-byte accesses).
__device__ __forceinline__ int tile_elem_byte(int r, int c) {
  return tile_byte(r, c >> 3) + (c & 7) * 2;
}

// s_waitcnt immediate that waits until at most `n` vector memory operations are outstanding
// (gfx9 encoding: vmcnt low bits [3:0], high bits [15:14]; expcnt and lgkmcnt left at max).
constexpr int waitcnt_vm(int n) { return ((n >> 4) << 14) | (0xF << 8) | (7 << 4) | (n & 15); }

// Read-only metadata (index lists, counts, block sizes) through the constant address space, so
// the compiler issues scalar loads: they count against lgkmcnt, not vmcnt, and a read of a list
// entry never waits for the vector memory traffic (atomics, prefetches) in flight.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p, size_t i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

// One global -> LDS DMA of 16 bytes per lane (global_load_lds_dwordx4): lane l's bytes land at
// LDS byte address lds_base + 16*l. Issued through inline assembly so the compiler does not track
// it; callers wait with an explicit s_waitcnt vmcnt before a barrier that publishes the tile.
// M0 (the LDS base the DMA reads) is saved and restored around the DMA, since the compiler does
// not allow it on a clobber list. An LDS DMA that reads M0 must not directly follow the write of
// M0: the s_nop is the one wait state that gfx9-family parts require in between.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  const uint32_t base = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(base)
      : "memory");
}

// Work id of the calling workgroup in an XCD-aware launch of 8 * items_per_xcd workgroups. The
// dispatcher sends workgroup b to XCD b % 8, each XCD taking its workgroups in order, so XCD x
// runs local indices li = b / 8 = 0, 1, ... . With one round XCD x runs the contiguous work ids
// [x * items_per_xcd, (x + 1) * items_per_xcd): one slice of the (head-major) item list, so an
// XCD's L2 sees few heads. With R rounds the item list is cut into 8R slices of C =
// items_per_xcd / R ids and XCD x runs slice 8r + x in round r (8r + (x ^ 1) in odd rounds, so an
// XCD pair alternates the first and second halves of a head): at any time the eight XCDs share
// fewer heads, whose tiles then stay in the memory-side cache (MALL) that all XCDs share.
__device__ __forceinline__ int xcd_work_id(int items_per_xcd, int rounds) {
  const int x = blockIdx.x & 7, li = blockIdx.x >> 3;
  if (rounds <= 1) return x * items_per_xcd + li;
  const int c = items_per_xcd / rounds;
  const int r = li / c, j = li - r * c;
  return (8 * r + ((r & 1) ? (x ^ 1) : x)) * c + j;
}

// Index of the calling wave inside its workgroup, as a value the compiler knows to be uniform.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// The same DMA with a uniform 64-bit base (SGPRs) and a per-lane 32-bit byte offset, so issuing it
// costs no vector address arithmetic.
__device__ __forceinline__ void dma16_sb(const void* base_ptr, uint32_t voff, uint32_t lds_base) {
  const uint32_t lb = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_base);
  // readfirstlane returns a signed int: go through uint32_t so the low half is zero-extended
  const uint64_t b = (uint64_t)(uintptr_t)base_ptr;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(lb)
      : "memory");
}

__device__ __forceinline__ uint64_t uniform_u64(const void* p) {
  // readfirstlane returns a signed int: go through uint32_t so each half is zero-extended
  const uint64_t b = (uint64_t)(uintptr_t)p;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}
__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// Tile DMA with one M0 write per tile. A [64][128] 16-bit tile is 16 slices of 1 KiB (4 rows
// each); wave w of four copies slices 4w .. 4w+3, whose LDS destinations are consecutive KiB.
// global_load_lds adds its immediate offset to both the global and the LDS address, so M0 is set
// once to the wave's first slice and the four DMAs carry offsets 0, 1024, 2048, 3072; the
// per-lane global offsets (tile_offsets_wave) have the matching 1024 * i taken off.
__device__ __forceinline__ void tile_offsets_wave(uint32_t* off, int lane, int w) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = (4 * w + i) * 64 + lane;  // 16-byte chunk slot this lane fills
    const int r = slot >> 4;
    const int cc = (slot & 15) ^ swz128(r);
    off[i] = (uint32_t)((r * HEAD_DIM + cc * 8) * 2 - 1024 * i);  // >= 0: row r >= 16w + 4i
  }
}

// This wave's four slices of two tiles (ga -> lds_a, gb -> lds_b; the LDS addresses include the
// wave's 4w KiB) in one asm block: eight vector memory operations. Every write of M0 is followed
// by one wait state before the DMA that reads it; M0 is restored.
__device__ __forceinline__ void dma_tile_pair(const void* ga, const void* gb, const uint32_t* off,
                                              uint32_t lds_a, uint32_t lds_b) {
  const uint64_t a = uniform_u64(ga), b = uniform_u64(gb);
  const uint32_t la = uniform_u32(lds_a), lb = uniform_u32(lds_b);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %7\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %5\n\t"
      "global_load_lds_dwordx4 %2, %5 offset:1024\n\t"
      "global_load_lds_dwordx4 %3, %5 offset:2048\n\t"
      "global_load_lds_dwordx4 %4, %5 offset:3072\n\t"
      "s_mov_b32 m0, %8\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %6\n\t"
      "global_load_lds_dwordx4 %2, %6 offset:1024\n\t"
      "global_load_lds_dwordx4 %3, %6 offset:2048\n\t"
      "global_load_lds_dwordx4 %4, %6 offset:3072\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(a), "s"(b), "s"(la), "s"(lb)
      : "memory");
}

// The same for one tile: four vector memory operations.
__device__ __forceinline__ void dma_tile(const void* ga, const uint32_t* off, uint32_t lds_a) {
  const uint64_t a = uniform_u64(ga);
  const uint32_t la = uniform_u32(lds_a);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %6\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %5\n\t"
      "global_load_lds_dwordx4 %2, %5 offset:1024\n\t"
      "global_load_lds_dwordx4 %3, %5 offset:2048\n\t"
      "global_load_lds_dwordx4 %4, %5 offset:3072\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(a), "s"(la)
      : "memory");
}

// Two consecutive 1-KiB DMAs of contiguous bytes: lane l copies g + voff (+1024) to LDS
// lds + 16 * l (+1024); voff is normally 16 * lane. Two vector memory operations, non-temporal
// (for data read exactly once).
__device__ __forceinline__ void dma_lin2_nt(const void* g, uint32_t voff, uint32_t lds) {
  const uint64_t a = uniform_u64(g);
  const uint32_t la = uniform_u32(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2 nt\n\t"
      "global_load_lds_dwordx4 %1, %2 offset:1024 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(a), "s"(la)
      : "memory");
}

// 128 bytes of a small record: lanes 0..7 copy rec + roff to LDS lds_r + 16 * lane, with EXEC
// narrowed to them inside the asm block. One vector memory operation.
__device__ __forceinline__ void dma_rec128(const void* rec, uint32_t roff, uint32_t lds_r) {
  const uint64_t r = uniform_u64(rec);
  const uint32_t lr = uniform_u32(lds_r);
  uint32_t saved;
  uint64_t exec_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b64 %1, exec\n\t"
      "s_mov_b64 exec, 0xff\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b64 exec, %1\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved), "=&s"(exec_saved)
      : "v"(roff), "s"(r), "s"(lr)
      : "memory");
}

// dma_tile_pair plus 128 bytes of a small record: lanes 0..7 copy rec + roff (per-lane byte
// offsets) to LDS lds_r + 16 * lane. EXEC is narrowed to those lanes inside the asm block and
// restored, so the caller needs no divergent branch. Nine vector memory operations per wave.
__device__ __forceinline__ void dma_tile_pair_rec(const void* ga, const void* gb, const void* rec,
                                                  const uint32_t* off, uint32_t roff,
                                                  uint32_t lds_a, uint32_t lds_b,
                                                  uint32_t lds_r) {
  const uint64_t a = uniform_u64(ga), b = uniform_u64(gb), r = uniform_u64(rec);
  const uint32_t la = uniform_u32(lds_a), lb = uniform_u32(lds_b), lr = uniform_u32(lds_r);
  uint32_t saved;
  uint64_t exec_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %10\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %7\n\t"
      "global_load_lds_dwordx4 %3, %7 offset:1024\n\t"
      "global_load_lds_dwordx4 %4, %7 offset:2048\n\t"
      "global_load_lds_dwordx4 %5, %7 offset:3072\n\t"
      "s_mov_b32 m0, %11\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %8\n\t"
      "global_load_lds_dwordx4 %3, %8 offset:1024\n\t"
      "global_load_lds_dwordx4 %4, %8 offset:2048\n\t"
      "global_load_lds_dwordx4 %5, %8 offset:3072\n\t"
      "s_mov_b64 %1, exec\n\t"
      "s_mov_b64 exec, 0xff\n\t"
      "s_mov_b32 m0, %12\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %6, %9\n\t"
      "s_mov_b64 exec, %1\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved), "=&s"(exec_saved)
      : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "v"(roff), "s"(a), "s"(b), "s"(r),
        "s"(la), "s"(lb), "s"(lr)
      : "memory");
}

// Per-lane byte offsets inside a [64][128] 16-bit tile for the slices part, part + NPARTS, ... that
// tile_load_async<NPARTS> would issue (the same for every tile).
template <int NPARTS>
__device__ __forceinline__ void tile_offsets(uint32_t* off, int lane, int part) {
#pragma unroll
  for (int i = 0; i < 16 / NPARTS; ++i) {
    const int slot = (part + i * NPARTS) * 64 + lane;
    const int r = slot >> 4;
    const int cc = (slot & 15) ^ swz128(r);
    off[i] = (uint32_t)((r * HEAD_DIM + cc * 8) * 2);
  }
}

// Copy one tile with precomputed offsets: slice part + i*NPARTS goes to LDS lds + (part+i*NPARTS) KiB.
template <int NPARTS>
__device__ __forceinline__ void tile_load_async_off(const bf16* g, VSA_LDS char* lds,
                                                    const uint32_t* off, int part) {
#pragma unroll
  for (int i = 0; i < 16 / NPARTS; ++i)
    dma16_sb(g, off[i], (uint32_t)(uintptr_t)(lds + (part + i * NPARTS) * 1024));
}

__device__ __forceinline__ uint32_t lds_addr(const VSA_LDS void* p) {
  return (uint32_t)(uintptr_t)p;
}

// Copy one [64][128] 16-bit tile (row stride 128 elements) from global memory into the swizzled LDS
// format. A wave moves 64 lanes x 16 bytes per DMA; NPARTS waves share the tile, wave `part`
// issuing slices part, part + NPARTS, ... of the tile's 16 one-KiB slices.
template <int NPARTS>
__device__ __forceinline__ void tile_load_async(const bf16* __restrict__ g, VSA_LDS char* lds,
                                                int lane, int part) {
#pragma unroll
  for (int i = 0; i < 16 / NPARTS; ++i) {
    const int u = part + i * NPARTS;
    const int slot = u * 64 + lane;  // chunk slot this lane fills
    const int r = slot >> 4;
    const int cc = (slot & 15) ^ swz128(r);
    dma16(g + r * HEAD_DIM + cc * 8, lds_addr(lds + u * 1024));
  }
}

}  // namespace vsa
