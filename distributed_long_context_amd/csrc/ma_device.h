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

// Global position of local index t (segments are validated on the host).
__device__ __forceinline__ int pos_at_dev(const KPos& p, int t) {
  int s = p.nseg - 1;
  while (s > 0 && p.lb[s] > t) --s;
  return p.gb[s] + (t - p.lb[s]) * p.st[s];
}

// Min and max global position over local indices [u0, u1) of a partition of length len.
__device__ __forceinline__ void pos_minmax_dev(const KPos& p, int len, int u0, int u1, int& mn, int& mx) {
  int lo = INT32_MAX, hi = INT32_MIN;
  for (int s = 0; s < p.nseg; ++s) {
    const int b = p.lb[s];
    const int e = (s + 1 < p.nseg) ? p.lb[s + 1] : len;
    const int a0 = max(b, u0), a1 = min(e, u1);
    if (a0 >= a1) continue;
    lo = min(lo, p.gb[s] + (a0 - b) * p.st[s]);
    hi = max(hi, p.gb[s] + (a1 - 1 - b) * p.st[s]);
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

// Transposed LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, lane i
// receives element j from the 8 bytes addressed by lane 4j + i/4, at position i%4.
__device__ __forceinline__ bf16x4 ds_read_tr16(const __bf16* lds_ptr) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) void*)lds_ptr));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

}  // namespace ma
