// Device-side helpers shared by the HIP kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

#include "ma_internal.h"

namespace ma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Global position of local index t (segments are validated on the host).  The
// loops run over compile-time segment indices so that the descriptor stays in
// registers (a runtime index would copy it to scratch memory).
__device__ __forceinline__ int pos_at_dev(const KPos& p, int t) {
  int r = p.gb[0] + (t - p.lb[0]) * p.st[0];
#pragma unroll
  for (int s = 1; s < MA_MAX_SEGMENTS; ++s)
    if (s < p.nseg && t >= p.lb[s]) r = p.gb[s] + (t - p.lb[s]) * p.st[s];
  return r;
}

// Min and max global position over local indices [u0, u1) of a partition of length len.
__device__ __forceinline__ void pos_minmax_dev(const KPos& p, int len, int u0, int u1, int& mn, int& mx) {
  int lo = INT32_MAX, hi = INT32_MIN;
#pragma unroll
  for (int s = 0; s < MA_MAX_SEGMENTS; ++s) {
    if (s >= p.nseg) break;
    const int b = p.lb[s];
    const int e = (s + 1 < p.nseg) ? p.lb[s + 1 < MA_MAX_SEGMENTS ? s + 1 : s] : len;
    const int a0 = max(b, u0), a1 = min(e, u1);
    if (a0 < a1) {
      lo = min(lo, p.gb[s] + (a0 - b) * p.st[s]);
      hi = max(hi, p.gb[s] + (a1 - 1 - b) * p.st[s]);
    }
  }
  mn = lo;
  mx = hi;
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ bf16x2 cvt2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_convertvector(v, bf16x2);
}
__device__ __forceinline__ bf16x8 pack_bf16x8(const float* x) {
  bf16x2 a = cvt2(x[0], x[1]), b = cvt2(x[2], x[3]), c = cvt2(x[4], x[5]), d = cvt2(x[6], x[7]);
  bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}
__device__ __forceinline__ bf16x4 pack_bf16x4(const float* x) {
  bf16x2 a = cvt2(x[0], x[1]), b = cvt2(x[2], x[3]);
  bf16x4 r = {a[0], a[1], b[0], b[1]};
  return r;
}
__device__ __forceinline__ bf16x8 concat_bf16x4(bf16x4 lo, bf16x4 hi) {
  bf16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return r;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// ---------------------------------------------------------------------------
// LDS tiles of 64 rows x D bf16 (K/V blocks in the forward and the dQ kernel,
// Q/dO blocks in the dK/dV kernel).  Rows are 2*D bytes with no padding so that
// global_load_lds can fill them; 16-byte chunks are XOR-swizzled by row.
// ---------------------------------------------------------------------------

// XOR mask applied to the 16-byte chunk index of LDS row `row` (period 16 rows).
// D=128 (one row = 64 banks): rows 0..15 map a chunk to 16 distinct chunks, and
// rows 4k..4k+3 to distinct 64-byte groups, so the b128 fragment reads (16 rows,
// one chunk) and the transposed b64 reads (4 rows x 64 bytes per half-wave) are
// conflict-free.  D=64 (two rows per bank line): the same over (row parity, chunk).
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Row order of the 32-row MFMA operand whose accumulator is reused as the next
// product's operand: swapping bits 2 and 3 of the row index turns the 32x32
// accumulator layout (rows 8(e/4) + 4(lane/32) + e%4) into the B/A operand layout
// (rows 8(lane/32) + e for e < 8, 16 + 8(lane/32) + e - 8 for e >= 8).
__device__ __forceinline__ int perm_key(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

__device__ __forceinline__ float xhalf_max(float x) {  // max(x[l], x[l ^ 32])
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {  // x[l] + x[l ^ 32]
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __attribute__((address_space(3))) char lds_char;

// Element `T` at byte offset `off` of the kernel-argument segment.  Kernels index
// their parameter block with runtime (uniform) indices through this, so that the
// block is read with scalar loads where it lives instead of being copied to
// scratch memory, which the compiler does when a by-value parameter's address
// escapes into lambdas.
template <class T>
__device__ __forceinline__ T kernarg_at(size_t off) {  // off: 4-byte aligned, sizeof(T) % 4 == 0
  static_assert(sizeof(T) % 4 == 0, "kernarg_at reads whole dwords");
  typedef const __attribute__((address_space(4))) uint32_t* wptr;
  const wptr src = (wptr)((const __attribute__((address_space(4))) char*)__builtin_amdgcn_kernarg_segment_ptr() + off);
  struct Words {
    uint32_t w[sizeof(T) / 4];
  } r;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) r.w[i] = src[i];
  return __builtin_bit_cast(T, r);
}
// One byte of the kernel-argument segment (byte arrays such as head maps).
__device__ __forceinline__ int kernarg_byte(size_t off) {
  const uint32_t w = kernarg_at<uint32_t>(off & ~(size_t)3);
  return (int)((w >> (8 * (off & 3))) & 0xffu);
}

// Byte address of an LDS location, made opaque to the optimiser so that later
// constant offsets (stage, slice) fold into the 16-bit immediate of the DS
// instruction instead of creating one address register per constant.
__device__ __forceinline__ uint32_t lds_lane_addr(const void* p) {
  uint32_t a = (uint32_t)(uintptr_t)(const lds_char*)p;
  asm volatile("" : "+v"(a));
  return a;
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_char*)p; }

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane i's bytes land at LDS byte address lds_dst + 16 i; the global address is
// gbase + voff_bytes.  gbase and lds_dst are wave-uniform (readfirstlane only
// states that, it is free when they already sit in scalar registers).  Written as
// inline asm so that the compiler does not add vmcnt(0) waits in front of every
// LDS read; the kernels order these loads themselves with s_waitcnt vmcnt and a
// barrier.  M0 carries the LDS address and is declared clobbered; M0 is a reserved
// register, which the compiler does not promise to preserve across inline asm, so
// the kernels rely on its keeping nothing of its own in M0.  A test compiles every
// kernel to assembly and checks that M0 appears only in this sequence
// (tests/test_m0_discipline.py).
__device__ __forceinline__ void lds_dma16(const void* gbase, uint32_t voff_bytes, uint32_t lds_dst) {
  const uint64_t g = (uint64_t)(uintptr_t)gbase;
  // readfirstlane returns int: go through uint32_t so the low word is not sign-extended
  const uint32_t glo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)g);
  const uint32_t ghi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(g >> 32));
  const uint64_t gu = ((uint64_t)ghi << 32) | (uint64_t)glo;
  const uint32_t lu = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_dst);
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff_bytes), "s"(gu), "s"(lu)
      : "memory", "m0");
}
__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t addr) {
  return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)addr;
}
__device__ __forceinline__ f32x4 lds_read_f32x4(uint32_t addr) {
  return *(const __attribute__((address_space(3))) f32x4*)(uintptr_t)addr;
}
// Transposed LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, lane i
// receives element j from the 8 bytes addressed by lane 4j + i/4, at position i%4.
__device__ __forceinline__ bf16x4 lds_read_tr16(uint32_t addr) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                        (__attribute__((address_space(3))) i16x4*)(uintptr_t)addr));
}

// s_waitcnt immediate that waits until at most n vector-memory operations of this
// wave are outstanding (vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left free)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Per-lane LDS byte addresses of the two fragment kinds read from a 64 x D tile
// at `tile` (stage 0):
//  * rows_b128[ks]: the 32-row operand (rows perm_key(lane%32), chunk 2ks + lane/32),
//    +32*D*2 bytes for rows 32..63;
//  * tr[c][h]: transposed b64 reads giving, per lane, 8 consecutive rows of column
//    c*32 + lane%32 (rows 8(lane/32) + 4h + 0..3 of each 16-row slice, +16*D*2
//    bytes per slice).
template <int D>
__device__ __forceinline__ void tile_lane_addrs(const __bf16* tile, int lane, uint32_t (&rows_b128)[D / 16],
                                                uint32_t (&tr)[D / 32][2]) {
  const int l32 = lane & 31, hl = lane >> 5;
  const int row = perm_key(l32);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) rows_b128[ks] = lds_lane_addr(&tile[row * D + (((2 * ks + hl) ^ swz<D>(row)) << 3)]);
  const int G = lane >> 4, lam = lane & 15;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = (G >> 1) * 8 + (lam >> 2) + h * 4;
      const int col = c * 32 + (G & 1) * 16 + (lam & 3) * 4;
      tr[c][h] = lds_lane_addr(&tile[r * D + (((col >> 3) ^ swz<D>(r)) << 3) + (col & 7)]);
    }
}

}  // namespace ma
