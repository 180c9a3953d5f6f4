// Add-reduce of fp32 partial gradients, HBM-bound.
//
// [Mesh] section 3.5 sums the per-pair partial dQ_i and dKV_j across GPUs with
// a reduce-scatter that adds; this kernel is the summation of k buffers that a
// GPU holds once the pieces have arrived: out = in_0 + in_1 + ... + in_{k-1}.
//
// A thread owns one 16-byte chunk (float4) of the output; the grid covers the
// buffer once.  Inputs are taken in groups of G (2, 4 or 8, the smallest that
// covers k up to 8): the loads of the next group are issued before the current
// one is added, and within a group all loads come before any add (indices past k
// repeat the last input, a valid address, and are not added), so nothing
// branches between the loads.  Every input is read once and the sum is not read
// again here, so loads and stores are nontemporal (streaming).  The adds run in
// input order, so the result does not depend on the launch shape.  Measured on
// MI355X with the 256 MB MALL flushed, against 8-input groups in a grid-stride
// loop with cached loads: 8 inputs of 64M floats 4.4 -> 6.2 TB/s, 2 inputs of
// 32M 3.7 -> 6.0 TB/s, 20 inputs of 8M 3.9 -> 5.6 TB/s.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <cstdint>

#include "ma_internal.h"

namespace ma {

namespace {

constexpr int kThreads = 256;
typedef float f4 __attribute__((ext_vector_type(4)));

template <int G>
__global__ void __launch_bounds__(kThreads) reduce_add_kernel(const ReduceParams p) {
  const int64_t n4 = p.n / 4;
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool ok = i < n4;
  auto load_group = [&](int r0, f4 (&x)[G]) {
#pragma unroll
    for (int u = 0; u < G; ++u)
      x[u] = ok ? __builtin_nontemporal_load((const f4*)p.in[min(r0 + u, p.k - 1)] + i) : f4{0.f, 0.f, 0.f, 0.f};
  };
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  f4 x[G];
  load_group(0, x);
  for (int r0 = 0; r0 < p.k; r0 += G) {
    f4 xn[G];
    const bool more = r0 + G < p.k;  // uniform
    if (more) load_group(r0 + G, xn);
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (r0 + u < p.k) acc += x[u];
    if (more) {
#pragma unroll
      for (int u = 0; u < G; ++u) x[u] = xn[u];
    }
  }
  if (ok) __builtin_nontemporal_store(acc, (f4*)p.out + i);
  // the last n % 4 elements, one thread each
  const int64_t t = n4 * 4 + threadIdx.x;
  if (blockIdx.x == 0 && t < p.n) {
    float a = 0.f;
    for (int r = 0; r < p.k; ++r) a += p.in[r][t];
    p.out[t] = a;
  }
}

}  // namespace

int launch_reduce_add(const ReduceParams& p, void* stream) {
  if (p.n <= 0) return 0;
  const int64_t blocks = std::max<int64_t>(1, (p.n / 4 + kThreads - 1) / kThreads);
  if (blocks > INT32_MAX) return (int)hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  hipStream_t s = (hipStream_t)stream;
  if (p.k <= 2) hipLaunchKernelGGL(reduce_add_kernel<2>, grid, dim3(kThreads), 0, s, p);
  else if (p.k <= 4) hipLaunchKernelGGL(reduce_add_kernel<4>, grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL(reduce_add_kernel<8>, grid, dim3(kThreads), 0, s, p);
  return (int)hipGetLastError();
}

}  // namespace ma
