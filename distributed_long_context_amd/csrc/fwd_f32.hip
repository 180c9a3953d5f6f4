// Tile forward for fp32 inputs (fp32 throughout), plus the fill used for EMPTY tiles.
//
// Same contract as the bf16 kernel ([Mesh] section 2.2 partial attention with
// LSE; [Ring] "Ring Attention: Pass KV Blocks Around the Ring" running max,
// denominator and output), on the vector ALUs: one lane owns one query row of
// one head, 32-key blocks of K and V are staged in LDS and shared by the 64
// rows of the wave.  This path serves fp32 partitions (small correctness
// shapes); the bf16 MFMA kernel is the throughput path.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "ma_internal.h"
#include "ma_device.h"

namespace ma {

namespace {

constexpr int kRows = 64;  // query rows per workgroup (one wave)
constexpr int kKB = 32;    // keys per LDS block

template <int D>
__global__ void __launch_bounds__(kRows) fwd_f32_kernel(const FwdParams p) {
  __shared__ __attribute__((aligned(16))) float Ksm[kKB * D];
  __shared__ __attribute__((aligned(16))) float Vsm[kKB * D];
  __shared__ int kpos_s[kKB];

  const int lane = threadIdx.x;
  const int w = blockIdx.x;
  int ti = 0;  // the count of later tiles that start at or before this workgroup
#pragma unroll
  for (int j = 1; j < kFwdTilesPerLaunch; ++j) ti += (j < p.ntiles && w >= p.tiles[j].wg_begin) ? 1 : 0;
  const FwdTile& T = p.tiles[ti];
  // workgroup -> (batch, query head, row block); T.chunks = row blocks
  int local = w - T.wg_begin;
  const int qb = local % T.chunks;
  local /= T.chunks;
  const int head = local % p.hq;
  const int b = local / p.hq;
  if (b >= p.batch) return;
  // KV head of this query head: find the run of heads_of that holds it
  int kv = 0;
  for (int x = 0; x < p.hkv; ++x)
    for (int y = p.kv_first[x]; y < p.kv_first[x + 1]; ++y)
      if (p.heads_of[y] == head) kv = x;

  const int row = qb * kRows + lane;
  const bool ok = row < T.sq;
  const int r0 = qb * kRows, r1 = min(T.sq, r0 + kRows);
  int pmin = 0, pmax = 0;
  if (p.mask) pos_minmax_dev(T.qp, T.sq, r0, r1, pmin, pmax);
  const int qpos = (p.mask && ok) ? pos_at_dev(T.qp, row) : 0;

  float q[D];
  const float* Qg = (const float*)T.q + (int64_t)b * p.q_sb + (int64_t)head * p.q_sh + (int64_t)row * p.q_ss;
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    float4 v = ok ? *(const float4*)(Qg + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    q[c] = v.x; q[c + 1] = v.y; q[c + 2] = v.z; q[c + 3] = v.w;
  }
  float o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) o[c] = 0.f;
  float m2 = -INFINITY, l = 0.f;
  const float c2 = p.scale_log2;

  const float* Kg = (const float*)T.k + (int64_t)b * p.k_sb + (int64_t)kv * p.k_sh;
  const float* Vg = (const float*)T.v + (int64_t)b * p.v_sb + (int64_t)kv * p.v_sh;
  for (int kb = 0; kb < T.sk; kb += kKB) {
    if (p.mask) {
      const int kmin = T.kgb + kb * T.kst;  // key positions grow with the index (one segment)
      if (kmin > pmax) continue;  // no allowed pair in this block (uniform)
    }
    __syncthreads();
    for (int i = lane; i < kKB * D / 4; i += kRows) {
      const int r = (i * 4) / D, c = (i * 4) % D;
      float4 kv4 = make_float4(0.f, 0.f, 0.f, 0.f), vv4 = kv4;
      if (kb + r < T.sk) {
        kv4 = *(const float4*)(Kg + (int64_t)(kb + r) * p.k_ss + c);
        vv4 = *(const float4*)(Vg + (int64_t)(kb + r) * p.v_ss + c);
      }
      *(float4*)(&Ksm[r * D + c]) = kv4;
      *(float4*)(&Vsm[r * D + c]) = vv4;
    }
    if (lane < kKB) {
      const int key = kb + lane;
      kpos_s[lane] = key >= T.sk ? INT32_MAX : (p.mask ? T.kgb + key * T.kst : INT32_MIN);
    }
    __syncthreads();
    float s[kKB];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKB; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) acc = __builtin_fmaf(q[c], Ksm[j * D + c], acc);
      s[j] = (kpos_s[j] <= qpos) ? acc : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float mb2 = mx * c2;
    if (mb2 > m2) {
      const float alpha = __builtin_amdgcn_exp2f(m2 - mb2);  // m2 = -inf gives 0
      l *= alpha;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] *= alpha;
      m2 = mb2;
    }
    const float mref = (m2 == -INFINITY) ? 0.f : m2;
#pragma unroll
    for (int j = 0; j < kKB; ++j) {
      const float pj = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], c2, -mref));
      l += pj;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = __builtin_fmaf(pj, Vsm[j * D + c], o[c]);
    }
  }
  if (!ok) return;
  const bool has = l > 0.f;
  float lse = has ? (m2 + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
  float wn = has ? 1.0f / l : 0.f;  // weight of this tile's unnormalised sums
  float wo = 0.f;                   // weight of the output already held (accumulate)
  float* Og = (float*)T.o + (int64_t)b * p.o_sb + (int64_t)head * p.o_sh + (int64_t)row * p.o_ss;
  float* Lp = T.lse + (int64_t)b * p.l_sb + (int64_t)head * p.l_sh + row;
  if (T.accumulate) {
    // fold into (O_old, lse_old): L = ln(e^lse_old + e^lse), O = e^(lse_old-L) O_old + e^(lse-L) O
    const float lo = *Lp;
    const float mx = fmaxf(lo, lse);
    if (mx == -INFINITY) {
      wn = 0.f;
    } else {
      const float eo = __expf(lo - mx), en = __expf(lse - mx);
      const float sum = eo + en;
      wo = eo / sum;
      wn *= en / sum;
      lse = mx + __logf(sum);
    }
  }
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    float4 r = make_float4(o[c] * wn, o[c + 1] * wn, o[c + 2] * wn, o[c + 3] * wn);
    if (T.accumulate) {
      const float4 old = *(const float4*)(Og + c);
      r.x = __builtin_fmaf(wo, old.x, r.x);
      r.y = __builtin_fmaf(wo, old.y, r.y);
      r.z = __builtin_fmaf(wo, old.z, r.z);
      r.w = __builtin_fmaf(wo, old.w, r.w);
    }
    *(float4*)(Og + c) = r;
  }
  *Lp = lse;
}

// O = 0 and LSE = -inf for a whole tile (the result of a tile with no allowed pair).
__global__ void fill_empty_kernel(void* o, float* lse, int dtype, int batch, int sq, int hq, int d,
                                  int64_t o_sb, int64_t o_ss, int64_t o_sh, int64_t l_sb, int64_t l_sh) {
  const int64_t rows = (int64_t)batch * sq * hq;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t r = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; r < rows; r += stride) {
    const int h = (int)(r % hq);
    const int64_t t = (r / hq) % sq;
    const int64_t b = r / ((int64_t)hq * sq);
    const int64_t off = b * o_sb + t * o_ss + h * o_sh;
    if (dtype == MA_F32) {
      float* op = (float*)o + off;
      for (int c = 0; c < d; c += 4) *(float4*)(op + c) = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      __bf16* op = (__bf16*)o + off;
      for (int c = 0; c < d; c += 8) *(uint4*)(op + c) = make_uint4(0, 0, 0, 0);
    }
    lse[b * l_sb + h * l_sh + t] = -INFINITY;
  }
}

}  // namespace

int launch_fwd_f32(const FwdParams& p, int head_dim, int total_wgs, void* stream) {
  if (total_wgs <= 0) return 0;
  dim3 grid(total_wgs), block(kRows);
  if (head_dim == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

int launch_fill_empty(void* o, float* lse, int dtype, int batch, int sq, int hq, int head_dim, int64_t o_sb,
                      int64_t o_ss, int64_t o_sh, int64_t l_sb, int64_t l_sh, void* stream) {
  const int64_t rows = (int64_t)batch * sq * hq;
  const int blocks = (int)std::min<int64_t>(4096, (rows + 255) / 256);
  hipLaunchKernelGGL(fill_empty_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, o, lse, dtype, batch, sq, hq,
                     head_dim, o_sb, o_ss, o_sh, l_sb, l_sh);
  return (int)hipGetLastError();
}

}  // namespace ma
