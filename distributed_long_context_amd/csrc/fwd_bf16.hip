// Tile forward, bf16 inputs, fp32 accumulation, for CDNA4 (gfx950).
//
// What one tile computes is the partial attention of [Mesh] section 2.2
// ((O_ij, lse_ij) = Attention(Q_i, K_j, V_j)) with the blockwise online softmax
// of [Ring] "Ring Attention: Pass KV Blocks Around the Ring" (running max,
// running denominator, unnormalised output).  The layout on the chip is this
// file's own design:
//
//  * A workgroup is 4 waves; each wave owns 64 query rows of one query head
//    (two 32-row MFMA sub-blocks) and all waves of a workgroup read the same KV
//    head, so one LDS copy of a 64-key K/V block serves 256 query rows.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    the accumulator puts one query per lane (16 of its keys; the other 16 in
//    lane l^32), so the row max needs one cross-lane exchange and the row sum
//    none until the end.  K rows are fed to the MFMA in a permuted order (bits
//    2 and 3 of the row index swapped) so that each lane's 16 accumulator
//    values are, unchanged, the B operand (P^T) of the P.V MFMA.
//  * O is accumulated transposed too (O^T = V^T P^T), so every lane again holds
//    only its own query's outputs and rescaling is lane-local.  V stays
//    row-major in LDS and is read transposed with ds_read_b64_tr_b16.
//  * Softmax runs in base 2 with scale*log2(e) folded into one FMA; the running
//    max is only raised when a row's block max exceeds it by more than 8
//    (factor 256), which keeps the result exact while skipping most rescales.
//  * Masks are resolved per 64-key block: blocks with no allowed pair are not
//    loaded, blocks with every pair allowed run unmasked, the rest compare
//    global positions element by element ([Mesh] section 3.7 pair classes).
#include <hip/hip_runtime.h>
#include <cstdint>

#include "ma_internal.h"
#include "ma_device.h"

namespace ma {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 64;  // query rows per wave
constexpr int kBN = 64;  // keys per block

template <int D>
struct FwdCfg {
  static constexpr int KROW = D + 8;                    // K row pitch in LDS (elements)
  static constexpr int VROW = D == 128 ? D + 32 : D + 32;  // V row pitch: 320 B (D=128), 192 B (D=64)
  static constexpr int KS = D / 16;                     // MFMA k-steps over d
  static constexpr int NC = D / 32;                     // 32-row chunks of O^T
  static constexpr int CH = D / 8;                      // 16-byte chunks per row
  static constexpr int LOADS = kBN * CH / kThreads;     // 16-byte loads per thread per tensor
  static constexpr int K_ELEMS = kBN * KROW;
  static constexpr int V_ELEMS = kBN * VROW;
};

__device__ __forceinline__ int perm_key(int m) {  // swap bits 2 and 3
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <int D>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(1, 1)))
fwd_bf16_kernel(const FwdParams p) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][C::K_ELEMS];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[2][C::V_ELEMS];
  __shared__ int kpos_s[2][kBN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // ---- which tile / batch / KV head / query block ----
  const int w = blockIdx.x;
  int ti = 0;
  while (ti + 1 < p.ntiles && w >= p.tiles[ti + 1].wg_begin) ++ti;
  const FwdTile& T = p.tiles[ti];
  const int local = w - T.wg_begin;
  const int kvh = local % p.hkv;
  const int rest = local / p.hkv;
  const int chunk = rest % T.chunks;
  const int b = rest / T.chunks;
  if (b >= p.batch) return;  // padding workgroup (uniform)
  const int g0 = p.kv_first[kvh];
  const int gsz = p.kv_first[kvh + 1] - g0;
  const int nqb = (T.sq + kQW - 1) / kQW;

  // units of this workgroup: (query block, head) pairs, query-block major
  int wg_qlo = INT32_MAX, wg_qhi = INT32_MIN;  // row range of the workgroup (for block skipping)
  bool any_valid = false;
  int my_qb = -1, my_head = 0;
  for (int wv = 0; wv < kWaves; ++wv) {
    const int u = chunk * kWaves + wv;
    if (gsz <= 0) break;
    const int qb = u / gsz;
    if (qb >= nqb) continue;
    any_valid = true;
    const int r0 = qb * kQW, r1 = min(T.sq, r0 + kQW);
    wg_qlo = min(wg_qlo, r0);
    wg_qhi = max(wg_qhi, r1);
    if (wv == wave) {
      my_qb = qb;
      my_head = p.heads_of[g0 + (u % gsz)];
    }
  }
  if (!any_valid) return;  // uniform across the workgroup
  const bool active = my_qb >= 0;
  const int q0 = active ? my_qb * kQW : 0;

  // position ranges for block classification
  int wg_pmin = 0, wg_pmax = 0;
  if (p.mask) pos_minmax_dev(T.qp, T.sq, wg_qlo, wg_qhi, wg_pmin, wg_pmax);
  int w_pmin = 0, w_pmax = 0;
  if (p.mask && active) pos_minmax_dev(T.qp, T.sq, q0, min(T.sq, q0 + kQW), w_pmin, w_pmax);

  const __bf16* __restrict__ Kg = (const __bf16*)T.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
  const __bf16* __restrict__ Vg = (const __bf16*)T.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh;

  // ---- query fragments (B operand of S^T = K Q^T) and query positions ----
  bf16x8 qf[2][C::KS];
  int qpos[2];
  {
    const __bf16* Qg = (const __bf16*)T.q + (int64_t)b * p.q_sb + (int64_t)my_head * p.q_sh;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const int row = q0 + qs * 32 + l32;
      const bool ok = active && row < T.sq;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        bf16x8 z = {};
        qf[qs][ks] = ok ? *(const bf16x8*)(Qg + (int64_t)row * p.q_ss + ks * 16 + hl * 8) : z;
      }
      qpos[qs] = (p.mask && ok) ? pos_at_dev(T.qp, row) : 0;
    }
  }

  // ---- KV block iteration over blocks that are not EMPTY for the workgroup ----
  const int nkb = (T.sk + kBN - 1) / kBN;
  auto block_class = [&](int kb, int pmin, int pmax) -> int {  // 0 empty, 1 partial, 2 full
    const int u0 = kb * kBN, u1 = min(T.sk, u0 + kBN);
    const bool tail = (u1 - u0) < kBN;
    if (!p.mask) return tail ? 1 : 2;
    int kmin, kmax;
    pos_minmax_dev(T.kp, T.sk, u0, u1, kmin, kmax);
    if (kmin > pmax) return 0;
    if (kmax <= pmin && !tail) return 2;
    return 1;
  };
  auto next_block = [&](int from) -> int {
    for (int kb = from; kb < nkb; ++kb)
      if (block_class(kb, wg_pmin, wg_pmax) != 0) return kb;
    return nkb;
  };

  uint4 kreg[C::LOADS], vreg[C::LOADS];
  auto gload = [&](int kb) {
#pragma unroll
    for (int it = 0; it < C::LOADS; ++it) {
      const int c = tid + it * kThreads;
      const int row = c / C::CH, col = (c % C::CH) * 8;
      const int key = kb * kBN + row;
      if (key < T.sk) {
        kreg[it] = *(const uint4*)(Kg + (int64_t)key * p.k_ss + col);
        vreg[it] = *(const uint4*)(Vg + (int64_t)key * p.v_ss + col);
      } else {
        kreg[it] = make_uint4(0, 0, 0, 0);
        vreg[it] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto swrite = [&](int buf, int kb) {
#pragma unroll
    for (int it = 0; it < C::LOADS; ++it) {
      const int c = tid + it * kThreads;
      const int row = c / C::CH, col = (c % C::CH) * 8;
      *(uint4*)(&Ks[buf][row * C::KROW + col]) = kreg[it];
      *(uint4*)(&Vs[buf][row * C::VROW + col]) = vreg[it];
    }
    if (tid < kBN) {
      const int key = kb * kBN + tid;
      int kp;
      if (key >= T.sk) kp = INT32_MAX;
      else kp = p.mask ? pos_at_dev(T.kp, key) : INT32_MIN;
      kpos_s[buf][tid] = kp;
    }
  };

  // ---- accumulators ----
  f32x16 oacc[2][C::NC];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
#pragma unroll
    for (int c = 0; c < C::NC; ++c) oacc[qs][c] = f32x16{};
  float m2[2] = {-INFINITY, -INFINITY};  // running max in log2 units (reference for exp2)
  float lsum[2] = {0.f, 0.f};            // this lane's share of the row sum
  const float c2 = p.scale_log2;

  int kb = next_block(0);
  int buf = 0;
  if (kb < nkb) {
    gload(kb);
    swrite(0, kb);
  }
  __syncthreads();
  int kb_next = (kb < nkb) ? next_block(kb + 1) : nkb;
  if (kb_next < nkb) gload(kb_next);

  while (kb < nkb) {
    const int cls = active ? block_class(kb, w_pmin, w_pmax) : 0;
    if (cls != 0) {
      const __bf16* Kl = Ks[buf];
      const __bf16* Vl = Vs[buf];
      // S^T = K Q^T for two 32-key sub-blocks and two 32-query sub-blocks
      f32x16 s[2][2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        s[0][kb2] = f32x16{};
        s[1][kb2] = f32x16{};
        const int krow = kb2 * 32 + perm_key(l32);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const bf16x8 kf = *(const bf16x8*)(Kl + krow * C::KROW + ks * 16 + hl * 8);
          s[0][kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[0][ks], s[0][kb2], 0, 0, 0);
          s[1][kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[1][ks], s[1][kb2], 0, 0, 0);
        }
      }
      // element masking on partial blocks
      if (cls == 1) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kb2 * 32 + (e >> 3) * 16 + hl * 8 + (e & 7);
            const int kp = kpos_s[buf][key];
#pragma unroll
            for (int qs = 0; qs < 2; ++qs)
              if (!(kp <= qpos[qs])) s[qs][kb2][e] = -INFINITY;
          }
      }
      // online softmax per query sub-block; P^T packed to bf16 as the B operand
      bf16x8 pf[2][4];
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[qs][kb2][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mb2 = mx * c2;
        if (__any(mb2 > m2[qs] + 8.0f)) {
          const float mn = fmaxf(m2[qs], mb2);
          const float alpha = (mn == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m2[qs] - mn);
          lsum[qs] *= alpha;
#pragma unroll
          for (int c = 0; c < C::NC; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[qs][c][i] *= alpha;
          m2[qs] = mn;
        }
        const float mref = (m2[qs] == -INFINITY) ? 0.0f : m2[qs];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            float pv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qs][kb2][half * 8 + i], c2, -mref));
              lsum[qs] += pv[i];
            }
            pf[qs][kb2 * 2 + half] = pack_bf16x8(pv);
          }
        }
      }
      // O^T += V^T P^T : V^T fragments read transposed from row-major LDS
      const int G = lane >> 4, lam = lane & 15;
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = j * 16 + (G >> 1) * 8 + (lam >> 2);
          const int col = c * 32 + (G & 1) * 16 + (lam & 3) * 4;
          const bf16x4 lo = ds_read_tr16(Vl + row * C::VROW + col);
          const bf16x4 hi = ds_read_tr16(Vl + (row + 4) * C::VROW + col);
          const bf16x8 vf = concat_bf16x4(lo, hi);
          oacc[0][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[0][j], oacc[0][c], 0, 0, 0);
          oacc[1][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[1][j], oacc[1][c], 0, 0, 0);
        }
      }
    }
    // stage the next block, then the one after it
    const int kb_after = (kb_next < nkb) ? next_block(kb_next + 1) : nkb;
    if (kb_next < nkb) swrite(buf ^ 1, kb_next);
    __syncthreads();
    if (kb_after < nkb) gload(kb_after);
    kb = kb_next;
    kb_next = kb_after;
    buf ^= 1;
  }

  if (!active) return;
  // ---- epilogue: normalise, store O (bf16) and LSE (fp32, natural log) ----
  __bf16* Og = (__bf16*)T.o + (int64_t)b * p.o_sb + (int64_t)my_head * p.o_sh;
  float* Lg = T.lse + (int64_t)b * p.l_sb + (int64_t)my_head * p.l_sh;
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const float ltot = lsum[qs] + __shfl_xor(lsum[qs], 32);
    const int row = q0 + qs * 32 + l32;
    const bool has = ltot > 0.0f;
    const float inv = has ? 1.0f / ltot : 0.0f;
    if (row < T.sq) {
#pragma unroll
      for (int c = 0; c < C::NC; ++c)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v4[i] = oacc[qs][c][g * 4 + i] * inv;
          *(bf16x4*)(Og + (int64_t)row * p.o_ss + c * 32 + g * 8 + hl * 4) = pack_bf16x4(v4);
        }
      if (hl == 0) Lg[row] = has ? (m2[qs] + __builtin_amdgcn_logf(ltot)) * 0.69314718055994531f : -INFINITY;
    }
  }
}

}  // namespace

int launch_fwd_bf16(const FwdParams& p, int head_dim, int total_wgs, void* stream) {
  if (total_wgs <= 0) return 0;
  dim3 grid(total_wgs), block(kThreads);
  if (head_dim == 128)
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, grid, block, 0, (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, grid, block, 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

}  // namespace ma
