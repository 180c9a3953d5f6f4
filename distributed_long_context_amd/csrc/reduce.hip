// Add-reduce of fp32 partial gradients, HBM-bound.
//
// [Mesh] section 3.5 sums the per-pair partial dQ_i and dKV_j across GPUs with
// a reduce-scatter that adds; this kernel is the summation of k buffers that a
// GPU holds once the pieces have arrived: out = in_0 + in_1 + ... + in_{k-1}.
//
// A thread owns 16 bytes (one float4) per grid-stride step.  Inputs are taken
// in groups of 8 whose loads are all issued before the adds; indices past k
// repeat the last input (a valid address) and are not added, so nothing
// branches between the loads.  The adds run in input order, so the result does
// not depend on the launch shape.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <cstdint>

#include "ma_internal.h"

namespace ma {

namespace {

constexpr int kThreads = 256;
constexpr int kGroup = 8;

__global__ void __launch_bounds__(kThreads) reduce_add_kernel(const ReduceParams p) {
  const int64_t n4 = p.n / 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int r0 = 0; r0 < p.k; r0 += kGroup) {
      float4 x[kGroup];
#pragma unroll
      for (int u = 0; u < kGroup; ++u) x[u] = ((const float4*)p.in[min(r0 + u, p.k - 1)])[i];
#pragma unroll
      for (int u = 0; u < kGroup; ++u) {
        if (r0 + u < p.k) {
          acc.x += x[u].x;
          acc.y += x[u].y;
          acc.z += x[u].z;
          acc.w += x[u].w;
        }
      }
    }
    ((float4*)p.out)[i] = acc;
  }
  // the last n % 4 elements, one thread each
  const int64_t t = n4 * 4 + (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (blockIdx.x == 0 && t < p.n) {
    float acc = 0.f;
    for (int r = 0; r < p.k; ++r) acc += p.in[r][t];
    p.out[t] = acc;
  }
}

}  // namespace

int launch_reduce_add(const ReduceParams& p, void* stream) {
  if (p.n <= 0) return 0;
  // enough workgroups to fill the 256 CUs several times over, each thread a few float4 steps
  const int64_t n4 = (p.n + 3) / 4;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(256 * 16, (n4 + kThreads - 1) / kThreads));
  hipLaunchKernelGGL(reduce_add_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

}  // namespace ma
