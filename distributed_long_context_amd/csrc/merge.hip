// LSE merge of k partial (O, LSE) pairs, HBM-bound.
//
// [Mesh] section 2.2: partial outputs over different KV partitions are combined
// exactly by rescaling each with its log-sum-exp; section 3.3 uses this online
// softmax as the reducer of the output reduce-scatter.  [CHARM+] appendix A,
// Algorithm 2 (CommAndUpdate) folds a received output into the local one the
// same way.  Closed form per (b, h, t):
//   L* = max_r lse_r;  lse = L* + ln sum_r exp(lse_r - L*);  O = sum_r exp(lse_r - lse) O_r
// with all lse_r = -inf giving (0, -inf).  The kernel folds the partials in
// groups with the running-max recurrence of [Ring] "Ring Attention: Pass KV
// Blocks Around the Ring" (m, s, acc rescaled when m grows), which is the same
// value in exact arithmetic; only the rounding order differs.
//
// Layout on the chip (this file's own design): a workgroup owns 64 consecutive
// rows t of one (b, h), so a wave's LSE reads of one partial fall in one cache
// line; a thread owns one 16-byte column chunk of 64/RPP rows.  Partials are
// taken in groups of G (2, 4 or 8, the smallest that covers k up to 8) whose
// loads are all issued before any use: indices past k repeat the last partial
// (a valid address) and get weight 0, so there are no branches between the
// loads.  The partial outputs are read once and the merged output is not read
// again by this kernel, so loads and stores are marked nontemporal (streaming):
// with the MALL flushed before each merge that took the 2-way merge of 8192
// rows x 32 heads from 3.1 to 5.4 TB/s and the 27-way merge of 4096 x 32 from
// 3.8 to 4.7 TB/s on MI355X (the 8-way merges of 16384 x 32 stay near 5.0).
#include <hip/hip_runtime.h>
#include <cstdint>

#include "ma_internal.h"
#include "ma_device.h"

namespace ma {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 64;  // rows t per workgroup
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int D, bool BF16, int G>
__global__ void __launch_bounds__(kThreads) merge_kernel(const MergeParams p) {
  constexpr int ES = BF16 ? 2 : 4;            // element size
  constexpr int CPR = D * ES / 16;            // 16-byte chunks per row
  constexpr int RPP = kThreads / CPR;         // rows per pass
  constexpr int PASSES = kRows / RPP;
  constexpr int NE = BF16 ? 8 : 4;            // elements per chunk
  const int nblk = (p.seqlen + kRows - 1) / kRows;
  const int blk = blockIdx.x % nblk;
  const int bh = blockIdx.x / nblk;
  const int h = bh % p.heads, b = bh / p.heads;
  const int c = threadIdx.x % CPR, rs = threadIdx.x / CPR;
  const int64_t lbase = (int64_t)b * p.l_sb + (int64_t)h * p.l_sh;
  const int64_t obase = (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + c * (16 / ES);
#pragma unroll
  for (int j = 0; j < PASSES; ++j) {
    const int t = blk * kRows + rs + j * RPP;
    if (t >= p.seqlen) break;
    const int64_t off = obase + (int64_t)t * p.o_ss;  // elements
    float acc[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = 0.f;
    float m = -INFINITY, s = 0.f;  // running max and rescaled denominator
    for (int i0 = 0; i0 < p.k; i0 += G) {
      float l[G];
      uint4 raw[G];
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int i = min(i0 + u, p.k - 1);
        l[u] = p.lse_in[i][lbase + t];
        const u32x4 r = __builtin_nontemporal_load((const u32x4*)((const char*)p.o_in[i] + off * ES));
        raw[u] = make_uint4(r.x, r.y, r.z, r.w);
      }
#pragma unroll
      for (int u = 0; u < G; ++u)
        if (i0 + u >= p.k) l[u] = -INFINITY;  // repeated partial: weight 0
      float gm = l[0];
#pragma unroll
      for (int u = 1; u < G; ++u) gm = fmaxf(gm, l[u]);
      const float mn = fmaxf(m, gm);
      const float mref = (mn == -INFINITY) ? 0.f : mn;  // everything -inf so far: all weights 0
      const float so = __expf(m - mref);                 // m = -inf gives 0
      s *= so;
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[e] *= so;
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const float wu = __expf(l[u] - mref);
        s += wu;
        const uint32_t wd[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
        if (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] = __builtin_fmaf(wu, __uint_as_float(wd[q] << 16), acc[2 * q]);
            acc[2 * q + 1] = __builtin_fmaf(wu, __uint_as_float(wd[q] & 0xffff0000u), acc[2 * q + 1]);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(wu, __uint_as_float(wd[q]), acc[q]);
        }
      }
      m = mn;
    }
    const bool has = m != -INFINITY;
    const float inv = has ? 1.0f / s : 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] *= inv;
    // every lane of this row has read all partials (same wave) before the row's
    // first lane writes, so o_out == o_in[0] and lse_out == lse_in[0] are safe
    if (BF16) {
      const bf16x8 pk = pack_bf16x8(acc);
      __builtin_nontemporal_store(__builtin_bit_cast(u32x4, pk), (u32x4*)((__bf16*)p.o_out + off));
    } else {
      const u32x4 v = {__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]), __float_as_uint(acc[3])};
      __builtin_nontemporal_store(v, (u32x4*)((float*)p.o_out + off));
    }
    if (c == 0) p.lse_out[lbase + t] = has ? m + __logf(s) : -INFINITY;
  }
}

template <int D, bool BF16>
void launch_g(const MergeParams& p, dim3 grid, hipStream_t s) {
  if (p.k <= 2) hipLaunchKernelGGL((merge_kernel<D, BF16, 2>), grid, dim3(kThreads), 0, s, p);
  else if (p.k <= 4) hipLaunchKernelGGL((merge_kernel<D, BF16, 4>), grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL((merge_kernel<D, BF16, 8>), grid, dim3(kThreads), 0, s, p);
}

}  // namespace

int launch_merge(const MergeParams& p, int dtype, int head_dim, void* stream) {
  const int64_t blocks = (int64_t)p.batch * p.heads * ((p.seqlen + kRows - 1) / kRows);
  if (blocks <= 0) return 0;
  if (blocks > INT32_MAX) return (int)hipErrorInvalidValue;
  dim3 grid((unsigned)blocks);
  hipStream_t s = (hipStream_t)stream;
  if (head_dim == 128) {
    if (dtype == MA_BF16) launch_g<128, true>(p, grid, s);
    else launch_g<128, false>(p, grid, s);
  } else {
    if (dtype == MA_BF16) launch_g<64, true>(p, grid, s);
    else launch_g<64, false>(p, grid, s);
  }
  return (int)hipGetLastError();
}

}  // namespace ma
