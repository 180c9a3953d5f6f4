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
// Layout on the chip (this file's own design): a workgroup of 256 threads owns a
// small tile of rows, TH = 2 adjacent heads x 8 consecutive positions t (16 rows
// at d = 128 in bf16; the tile grows to one full pass of the workgroup for
// smaller rows), and a thread one 16-byte column chunk of a row.  Consecutive
// workgroups take consecutive head pairs at the same positions, so the
// workgroups in flight stream adjacent memory of every partial.  Partials are
// taken in groups of G (2, 4 or 8, the smallest that covers k up to 8); the loads
// of the next group are issued before the current one is folded, and within a
// group all loads come before any use: indices past k repeat the last partial (a
// valid address) with weight 0, so nothing branches between the loads.  The
// partial outputs are read once and the merged output is not read again here, so
// loads and stores are nontemporal (streaming).  Measured on MI355X with the
// 256 MB MALL flushed before each merge, against 64-row workgroups of one head:
// 2-way merge of 8192 x 32 heads 5.35 -> 5.7 TB/s, 27-way of 4096 x 32
// 4.7 -> 5.3 TB/s, 8-way of 16384 x 32 4.9 -> 6.45 TB/s; small workgroups also
// leave no half-empty last round of workgroups.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "ma_internal.h"
#include "ma_device.h"

namespace ma {

namespace {

constexpr int kThreads = 256;

// rows of one workgroup: at least one full pass of the 256 threads, and 16
template <int D, bool BF16>
struct MergeTile {
  static constexpr int ES = BF16 ? 2 : 4;      // element size
  static constexpr int CPR = D * ES / 16;      // 16-byte chunks per row
  static constexpr int RPP = kThreads / CPR;   // rows per pass
  static constexpr int ROWS = RPP > 16 ? RPP : 16;
  static constexpr int PASSES = ROWS / RPP;
};

template <int D, bool BF16, int G, int TH>
__global__ void __launch_bounds__(kThreads) merge_kernel(const MergeParams p) {
  using T = MergeTile<D, BF16>;
  constexpr int ES = T::ES, CPR = T::CPR, RPP = T::RPP;
  constexpr int TT = T::ROWS / TH;             // positions per workgroup
  constexpr int NE = BF16 ? 8 : 4;             // elements per chunk
  const int nth = p.heads / TH;
  const int ntb = (p.seqlen + TT - 1) / TT;
  const int hg = blockIdx.x % nth;
  const int tb = (blockIdx.x / nth) % ntb;
  const int b = blockIdx.x / (nth * ntb);
  const int c = threadIdx.x % CPR, rs = threadIdx.x / CPR;
#pragma unroll
  for (int j = 0; j < T::PASSES; ++j) {
    const int r = rs + j * RPP;  // row of the tile: head r % TH, position r / TH
    const int t = tb * TT + r / TH, h = hg * TH + r % TH;
    if (t >= p.seqlen) break;    // t grows with j
    const int64_t lbase = (int64_t)b * p.l_sb + (int64_t)h * p.l_sh;
    const int64_t off = (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)t * p.o_ss + c * (16 / ES);  // elements
    float acc[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = 0.f;
    float m = -INFINITY, s = 0.f;  // running max and rescaled denominator
    auto load_group = [&](int i0, float (&l)[G], u32x4 (&raw)[G]) {
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int i = min(i0 + u, p.k - 1);
        l[u] = p.lse_in[i][lbase + t];
        raw[u] = __builtin_nontemporal_load((const u32x4*)((const char*)p.o_in[i] + off * ES));
      }
    };
    float l[G];
    u32x4 raw[G];
    load_group(0, l, raw);
    for (int i0 = 0; i0 < p.k; i0 += G) {
      float ln[G];
      u32x4 rn[G];
      const bool more = i0 + G < p.k;  // uniform
      if (more) load_group(i0 + G, ln, rn);
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
      if (more) {
#pragma unroll
        for (int u = 0; u < G; ++u) {
          l[u] = ln[u];
          raw[u] = rn[u];
        }
      }
    }
    const bool has = m != -INFINITY;
    const float inv = has ? 1.0f / s : 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] *= inv;
    // the CPR lanes of this row are in one wave and have read all partials before
    // any of them writes, so o_out == o_in[0] and lse_out == lse_in[0] are safe
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

template <int D, bool BF16, int TH>
int launch_th(const MergeParams& p, hipStream_t s) {
  constexpr int TT = MergeTile<D, BF16>::ROWS / TH;
  const int64_t blocks = (int64_t)p.batch * (p.heads / TH) * ((p.seqlen + TT - 1) / TT);
  if (blocks <= 0) return 0;
  if (blocks > INT32_MAX) return (int)hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  if (p.k <= 2) hipLaunchKernelGGL((merge_kernel<D, BF16, 2, TH>), grid, dim3(kThreads), 0, s, p);
  else if (p.k <= 4) hipLaunchKernelGGL((merge_kernel<D, BF16, 4, TH>), grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL((merge_kernel<D, BF16, 8, TH>), grid, dim3(kThreads), 0, s, p);
  return (int)hipGetLastError();
}

// head pairs when the head count is even, single heads otherwise
template <int D, bool BF16>
int launch_d(const MergeParams& p, hipStream_t s) {
  return p.heads % 2 == 0 ? launch_th<D, BF16, 2>(p, s) : launch_th<D, BF16, 1>(p, s);
}

}  // namespace

int launch_merge(const MergeParams& p, int dtype, int head_dim, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (head_dim == 128) return dtype == MA_BF16 ? launch_d<128, true>(p, s) : launch_d<128, false>(p, s);
  return dtype == MA_BF16 ? launch_d<64, true>(p, s) : launch_d<64, false>(p, s);
}

}  // namespace ma
