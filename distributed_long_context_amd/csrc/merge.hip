// LSE merge of k partial (O, LSE) pairs, HBM-bound.
//
// [Mesh] section 2.2: partial outputs over different KV partitions are combined
// exactly by rescaling each with its log-sum-exp; section 3.3 uses this online
// softmax as the reducer of the output reduce-scatter.  [CHARM+] appendix A,
// Algorithm 2 (CommAndUpdate) folds a received output into the local one the
// same way.  Closed form per (b, h, t):
//   L* = max_r lse_r;  lse = L* + ln sum_r exp(lse_r - L*);  O = sum_r exp(lse_r - lse) O_r
// with all lse_r = -inf giving (0, -inf).
//
// Each thread owns 8 consecutive elements (16 bytes of bf16) of one output
// row; the D/8 threads of a row sit in one wave, so they read every partial's
// LSE before the row's first thread writes the merged one (this makes the
// in-place form lse_out == lse_in[0] safe).  The partial loop is unrolled by 8
// with all loads issued before the FMAs so that enough bytes are in flight.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "ma_internal.h"
#include "ma_device.h"

namespace ma {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

template <int D, bool BF16>
__global__ void __launch_bounds__(kThreads) merge_kernel(const MergeParams p) {
  constexpr int TPR = D / 8;  // threads per row
  const int64_t rows = (int64_t)p.batch * p.seqlen * p.heads;
  const int64_t r = (int64_t)blockIdx.x * (kThreads / TPR) + threadIdx.x / TPR;
  if (r >= rows) return;
  const int cpart = (threadIdx.x % TPR) * 8;
  const int h = (int)(r % p.heads);
  const int64_t t = (r / p.heads) % p.seqlen;
  const int64_t b = r / ((int64_t)p.heads * p.seqlen);
  const int64_t loff = b * p.l_sb + h * p.l_sh + t;
  const int64_t ooff = b * p.o_sb + t * p.o_ss + h * p.o_sh + cpart;

  // pass 1: max and log-sum-exp of the partial LSEs
  float Lmax = -INFINITY;
  for (int i = 0; i < p.k; ++i) Lmax = fmaxf(Lmax, p.lse_in[i][loff]);
  float lse = -INFINITY;
  if (Lmax != -INFINITY) {
    float sum = 0.f;
    for (int i = 0; i < p.k; ++i) sum += __expf(p.lse_in[i][loff] - Lmax);
    lse = Lmax + __logf(sum);
  }
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;
  if (lse != -INFINITY) {
    for (int i0 = 0; i0 < p.k; i0 += kUnroll) {
      float w[kUnroll];
      float x[kUnroll][8];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int i = i0 + u;
        if (i < p.k) {
          w[u] = __expf(p.lse_in[i][loff] - lse);
          if (BF16) {
            const uint4 v = *(const uint4*)((const __bf16*)p.o_in[i] + ooff);
            const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              x[u][2 * c] = __uint_as_float(wd[c] << 16);
              x[u][2 * c + 1] = __uint_as_float(wd[c] & 0xffff0000u);
            }
          } else {
            const float4 v0 = *(const float4*)((const float*)p.o_in[i] + ooff);
            const float4 v1 = *(const float4*)((const float*)p.o_in[i] + ooff + 4);
            x[u][0] = v0.x; x[u][1] = v0.y; x[u][2] = v0.z; x[u][3] = v0.w;
            x[u][4] = v1.x; x[u][5] = v1.y; x[u][6] = v1.z; x[u][7] = v1.w;
          }
        } else {
          w[u] = 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) x[u][c] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = __builtin_fmaf(w[u], x[u][c], acc[c]);
    }
  }
  if (BF16) {
    *(bf16x8*)((__bf16*)p.o_out + ooff) = pack_bf16x8(acc);
  } else {
    *(float4*)((float*)p.o_out + ooff) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *(float4*)((float*)p.o_out + ooff + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  if (cpart == 0) p.lse_out[loff] = lse;
}

}  // namespace

int launch_merge(const MergeParams& p, int dtype, int head_dim, void* stream) {
  const int64_t rows = (int64_t)p.batch * p.seqlen * p.heads;
  const int rpb = kThreads / (head_dim / 8);
  const int64_t blocks = (rows + rpb - 1) / rpb;
  if (blocks <= 0) return 0;
  dim3 grid((unsigned)blocks), block(kThreads);
  hipStream_t s = (hipStream_t)stream;
  if (head_dim == 128) {
    if (dtype == MA_BF16) hipLaunchKernelGGL((merge_kernel<128, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((merge_kernel<128, false>), grid, block, 0, s, p);
  } else {
    if (dtype == MA_BF16) hipLaunchKernelGGL((merge_kernel<64, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((merge_kernel<64, false>), grid, block, 0, s, p);
  }
  return (int)hipGetLastError();
}

}  // namespace ma
