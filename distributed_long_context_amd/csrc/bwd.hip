// Tile backward (dQ, dK, dV), bf16 inputs, fp32 accumulation, for CDNA4 (gfx950).
//
// [Mesh] section 3.5: the backward kernel runs per (Q_i, KV_j) pair with
// (Q_i, KV_j, O_i, dO_i) and the partial dQ_i and dKV_j are accumulated
// locally, addition being the reducer.  The pages print no formula; the kernels
// evaluate the derivative of the forward definition with P = exp(s - LSE):
//   D[t] = dO[t].O[t];  dP = dO V^T;  dS = P (dP - D);
//   dV = P^T dO;  dK = scale dS^T Q;  dQ = scale dS K.
//
// Layout on the chip (this file's own design): three kernels, no atomics.
//  * bwd_pre: per Q partition, LSE*log2(e) (+inf on rows without an allowed key,
//    so that P = 0 there) and D, written per 64-row block as 512 contiguous bytes.
//  * bwd_dq (Q-stationary, the forward's structure): 8 waves x 32 query rows,
//    two waves per SIMD, Q and dO fragments in registers; the 64-key K/V blocks
//    of every KV partition of the Q group stream through a 4-stage LDS ring
//    (direct-to-LDS loads, XOR-swizzled rows).  Per 32-key step: S^T = K Q^T and
//    dP^T = V dO^T with one query per lane, P and dS on the VALU, then
//    dQ^T += K^T dS^T with K^T read transposed (ds_read_b64_tr_b16); the next
//    step's S^T and dP^T MFMAs are issued under this step's exponentials.
//  * bwd_dkv (KV-stationary): 4 waves x 32 keys, one wave per SIMD, K and V
//    fragments and the dK, dV accumulators in registers for the whole walk over
//    every Q partition of the KV group, every query head reading the KV head and
//    every 64-row query block (Q, dO and the LSE/D block staged in LDS the same
//    way).  Per 32-query step: S = Q K^T and dP = dO V^T with one key per lane
//    and the query rows fed in permuted order, so that P and dS are directly the
//    A operands of dV += P^T dO and dK += dS^T Q (dO^T, Q^T read transposed).
//  * Blocks with no allowed pair are skipped, blocks with every pair allowed run
//    unmasked ([Mesh] section 3.7 pair classes), the rest mask element-wise.
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>
#include <type_traits>

#include "ma_internal.h"
#include "ma_device.h"

namespace ma {

namespace {

constexpr int kBN = 64;  // rows of one LDS tile: keys in bwd_dq, queries in bwd_dkv
constexpr int kStages = 4;

template <int D>
struct Cfg {
  static constexpr int CH = D / 8;      // 16-byte chunks per row
  static constexpr int KS = D / 16;     // MFMA k-steps over d
  static constexpr int NC = D / 32;     // 32-wide d chunks
  static constexpr int BLK = kBN * D;   // elements of one tile
  static constexpr uint32_t STAGE_BYTES = BLK * 2;
};

// Parameter-block access by uniform index (see kernarg_at).
__device__ __forceinline__ BwdEntry entry_at(int i) {
  return kernarg_at<BwdEntry>(offsetof(BwdParams, entries) + (size_t)i * sizeof(BwdEntry));
}
__device__ __forceinline__ BwdQPart qpart_at(int i) {
  return kernarg_at<BwdQPart>(offsetof(BwdParams, qparts) + (size_t)i * sizeof(BwdQPart));
}
__device__ __forceinline__ BwdKVPart kvpart_at(int i) {
  return kernarg_at<BwdKVPart>(offsetof(BwdParams, kvparts) + (size_t)i * sizeof(BwdKVPart));
}
// partner pi of entry ei (read in place: a dynamically indexed copy of the entry
// would be moved to per-thread memory)
__device__ __forceinline__ int partner_at(int ei, int pi) {
  return kernarg_at<int32_t>(offsetof(BwdParams, entries) + (size_t)ei * sizeof(BwdEntry) + offsetof(BwdEntry, partner) +
                             (size_t)pi * 4);
}
__device__ __forceinline__ int head_of(int i) { return kernarg_byte(offsetof(BwdParams, heads_of) + i); }
__device__ __forceinline__ int kv_first_at(int i) { return kernarg_byte(offsetof(BwdParams, kv_first) + i); }

// ---------------------------------------------------------------- preprocess --
// One thread per 8 elements of a row; rows are (b, 64-row block, t%64, h) so that
// a block of threads reads contiguous O/dO bytes.  Stored per row: -LSE/scale and
// -D.  With them a score accumulator that starts at -LSE/scale ends at
// S - LSE/scale, so P = exp2(scale*log2(e) * acc), and a dP accumulator that
// starts at -D ends at dP - D, the factor of dS.  Rows without an allowed key and
// rows past sq in the last block get -inf (P = 0) and 0.
template <int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(const BwdPreParams p) {
  constexpr int TPR = D / 8;
  const int nqb = (p.sq + kBN - 1) / kBN;
  const int64_t rows = (int64_t)p.batch * nqb * kBN * p.hq;
  const int64_t r = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  if (r >= rows) return;  // whole rows leave together (TPR divides the wave)
  const int c = (threadIdx.x % TPR) * 8;
  const int h = (int)(r % p.hq);
  const int64_t tt = (r / p.hq) % ((int64_t)nqb * kBN);
  const int64_t b = r / ((int64_t)p.hq * nqb * kBN);
  const int t = (int)tt;
  float acc = 0.f;
  const bool ok = t < p.sq;
  if (ok) {
    const int64_t off = b * p.q_sb + (int64_t)t * p.q_ss + (int64_t)h * p.q_sh + c;
    const uint4 o = *(const uint4*)((const __bf16*)p.o + off);
    const uint4 g = *(const uint4*)((const __bf16*)p.dout + off);
    const uint32_t ow[4] = {o.x, o.y, o.z, o.w}, gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += bf16_to_f32((uint16_t)(ow[i] & 0xffffu)) * bf16_to_f32((uint16_t)(gw[i] & 0xffffu));
      acc += bf16_to_f32((uint16_t)(ow[i] >> 16)) * bf16_to_f32((uint16_t)(gw[i] >> 16));
    }
  }
#pragma unroll
  for (int s = TPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s);
  if ((threadIdx.x % TPR) == 0) {
    float nl = -INFINITY;
    if (ok) {
      const float L = p.lse[b * p.l_sb + (int64_t)h * p.l_sh + t];
      nl = (L == -INFINITY) ? -INFINITY : -L / p.scale;
    }
    float* blk = p.lsed + ((b * p.hq + h) * nqb + t / kBN) * (2 * kBN);
    blk[t % kBN] = nl;
    blk[kBN + t % kBN] = ok ? -acc : 0.f;
  }
}

// mask of a block on an in-order walk: whole (uniform), else the lane's last
// allowed row or key index relative to the block start
struct BlkMask {
  int whole;
  int lim;
};

// ---------------------------------------------------------------- dQ kernel --
// MASKED: causal on positions; the key positions of every KV partition are one
// segment (they grow with the key index), so a lane's mask is the index of its
// last allowed key and the blocks with any allowed pair for the workgroup are a
// prefix of each partition.  Without it only keys past a partition's end are masked.
template <int D, bool MASKED>
__global__ void __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dq_kernel(const BwdParams p) {
  using C = Cfg<D>;
  constexpr int kWaves = 8, kQW = 32;
  constexpr int LPW = kBN * C::CH / 64 / kWaves;  // direct-to-LDS loads per wave per tensor
  // K stages, then V stages
  __shared__ __attribute__((aligned(1024))) __bf16 kv_s[2][kStages][C::BLK];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // ---- entry (Q group) / batch / KV head / unit ----
  const int w = blockIdx.x;
  int ei = 0;
  while (ei + 1 < p.nentries && w >= entry_at(ei + 1).wg_begin) ++ei;
  ei = __builtin_amdgcn_readfirstlane(ei);
  const BwdEntry E = entry_at(ei);
  const BwdQPart QP = qpart_at(E.self);
  const int local = w - E.wg_begin;
  const int kvh = local % p.hkv;
  const int rest = local / p.hkv;
  // causal tiles: later query rows see more keys, so the heaviest chunks go first
  const int chunk = MASKED ? E.chunks - 1 - rest % E.chunks : rest % E.chunks;
  const int b = rest / E.chunks;
  if (b >= p.batch) return;
  const int g0 = kv_first_at(kvh);
  const int gsz = kv_first_at(kvh + 1) - g0;
  if (gsz <= 0) return;
  const int nqb = (QP.sq + kQW - 1) / kQW;
  int wg_qlo = INT32_MAX, wg_qhi = INT32_MIN;
  int my_qb = -1, my_head = 0;
  for (int wv = 0; wv < kWaves; ++wv) {
    const int u = chunk * kWaves + wv;
    const int qb = u / gsz;
    if (qb >= nqb) continue;
    wg_qlo = min(wg_qlo, qb * kQW);
    wg_qhi = max(wg_qhi, min(QP.sq, qb * kQW + kQW));
    if (wv == wave) {
      my_qb = qb;
      my_head = head_of(g0 + (u % gsz));
    }
  }
  if (wg_qlo == INT32_MAX) return;
  const bool active = my_qb >= 0;
  const int q0 = active ? my_qb * kQW : wg_qlo;
  int wg_pmin = 0, wg_pmax = 0, w_pmin = 0, w_pmax = 0;
  if constexpr (MASKED) {
    pos_minmax_dev(QP.qp, QP.sq, wg_qlo, wg_qhi, wg_pmin, wg_pmax);
    pos_minmax_dev(QP.qp, QP.sq, q0, min(QP.sq, q0 + kQW), w_pmin, w_pmax);
  }

  // ---- Q and dO fragments (B operands), LSE2 and D of this lane's query ----
  bf16x8 qf[C::KS], gf[C::KS];
  float nl2 = -INFINITY, nd = 0.f;  // -LSE*log2(e) and -D of this lane's query
  int qpos = INT32_MIN;
  const int row = q0 + l32;
  const bool row_ok = active && row < QP.sq;
  {
    const int64_t off = (int64_t)b * p.q_sb + (int64_t)my_head * p.q_sh + (int64_t)row * p.q_ss;
    const __bf16* Qg = (const __bf16*)QP.q + off;
    const __bf16* Gg = (const __bf16*)QP.dout + off;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      bf16x8 z = {};
      qf[ks] = row_ok ? *(const bf16x8*)(Qg + ks * 16 + hl * 8) : z;
      gf[ks] = row_ok ? *(const bf16x8*)(Gg + ks * 16 + hl * 8) : z;
    }
    if (row_ok) {
      const int nqb64 = (QP.sq + kBN - 1) / kBN;
      const float* blk = QP.lsed + (((int64_t)b * p.hq + my_head) * nqb64 + row / kBN) * (2 * kBN);
      nl2 = blk[row % kBN] * p.scale_log2;
      nd = blk[kBN + row % kBN];
      if constexpr (MASKED) qpos = pos_at_dev(QP.qp, row);
    }
  }

  // ---- key blocks of every KV partition of the group ----
  // one key segment: the last key index allowed at query position pq (-1: none)
  auto last_key = [&](const BwdKVPart& KV, int pq) {
    const int gb = KV.kp.gb[0], st = KV.kp.st[0];
    return pq < gb ? -1 : min(KV.sk - 1, (pq - gb) / st);
  };
  auto part_blocks = [&](const BwdKVPart& KV) {
    if constexpr (MASKED) return (last_key(KV, wg_pmax) + kBN) / kBN;
    else return (KV.sk + kBN - 1) / kBN;
  };
  int total = 0;  // blocks of the walk
#pragma unroll
  for (int i = 0; i < kBwdPerLaunch; ++i) total += i < E.n ? part_blocks(kvpart_at(partner_at(ei, i))) : 0;
  auto next_block = [&](int from) -> int { return from < total ? from : total; };

  // ---- direct-to-LDS loads of one K block and one V block ----
  auto load_row = [&](int i) { return ((wave * LPW + i) * 64 + lane) / C::CH; };
  auto load_col = [&](int i) { return ((((wave * LPW + i) * 64 + lane) % C::CH) ^ swz<D>(load_row(i))) * 8; };
  const int k_ss = (int)p.k_ss;  // below 2^24 (checked by the caller)
  uint32_t go[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) go[i] = (uint32_t)(load_row(i) * k_ss + load_col(i)) * 2u;
  // The blocks are visited in order: a cursor (partner, block) and the current
  // partner's bases and mask data, refreshed only when the partner changes, stand
  // in for a per-block decode (a kernel-argument load in the loop would also make
  // the wave wait for all of its LDS reads); issue_at returns the mask of the
  // block it loads.
  int c_pi = 0, c_kb = 0, c_nkb = 0, c_sk = 0, c_kfull = 0, c_klast = 0;
  const __bf16* c_k = nullptr;
  const __bf16* c_v = nullptr;
  auto cur_load = [&]() {
    for (;;) {
      const BwdKVPart KV = kvpart_at(partner_at(ei, c_pi));
      c_sk = KV.sk;
      c_nkb = part_blocks(KV);
      const int64_t off = (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
      c_k = (const __bf16*)KV.k + off;
      c_v = (const __bf16*)KV.v + off;
      if constexpr (MASKED) {
        c_klast = last_key(KV, qpos);
        c_kfull = active ? (last_key(KV, w_pmin) + 1) / kBN : 0;
      }
      if (c_nkb > 0 || c_pi + 1 >= E.n) break;
      ++c_pi;  // no allowed pair with this partition
    }
  };
  auto issue_next = [&](int st) -> BlkMask {
    const int64_t roff = (int64_t)c_kb * kBN * p.k_ss;
    const __bf16* kbase = c_k + roff;
    const __bf16* vbase = c_v + roff;
    const int valid = c_sk - c_kb * kBN;
    if (valid >= kBN) {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        lds_dma16(kbase, go[i], lds_addr(&kv_s[0][st][(wave * LPW + i) * 512]));
        lds_dma16(vbase, go[i], lds_addr(&kv_s[1][st][(wave * LPW + i) * 512]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const uint32_t o2 = (uint32_t)(min(load_row(i), valid - 1) * k_ss + load_col(i)) * 2u;
        lds_dma16(kbase, o2, lds_addr(&kv_s[0][st][(wave * LPW + i) * 512]));
        lds_dma16(vbase, o2, lds_addr(&kv_s[1][st][(wave * LPW + i) * 512]));
      }
    }
    BlkMask bm;
    if constexpr (MASKED) {
      bm.whole = c_kb < c_kfull;
      bm.lim = c_klast - c_kb * kBN;
    } else {
      bm.whole = valid >= kBN;
      bm.lim = valid - 1;
    }
    if (++c_kb == c_nkb) {
      c_kb = 0;
      ++c_pi;
      if (c_pi < E.n) cur_load();
    }
    return bm;
  };
  auto issue_at = [&](int st, int /*position*/) -> BlkMask { return issue_next(st); };
  cur_load();
  auto wait_positions = [&](int n) {  // at most n later positions in flight
    if (n >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * LPW));
    else if (n == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPW));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  };

  uint32_t kaddr[C::KS], ktr[C::NC][2], vaddr[C::KS], vtr_unused[C::NC][2];
  tile_lane_addrs<D>(kv_s[0][0], lane, kaddr, ktr);
  tile_lane_addrs<D>(kv_s[1][0], lane, vaddr, vtr_unused);

  f32x16 acc[C::NC];  // dQ^T: lane's query, d = 32c + 8(e/4) + 4hl + e%4
#pragma unroll
  for (int c = 0; c < C::NC; ++c) acc[c] = f32x16{};
  const float c2 = p.scale_log2;

  // S^T and dP^T of one 32-key half (kb2) of the block in stage st
  auto sdp_half = [&](int st, int kb2, f32x16& s, f32x16& dp) {
    const uint32_t off = st * C::STAGE_BYTES + kb2 * 32 * D * 2;
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 kf = lds_read_b128(kaddr[ks] + off);
      const bf16x8 vf = lds_read_b128(vaddr[ks] + off);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, gf[ks], dp, 0, 0, 0);
    }
  };
  // mask of a 32-key half: key kb*64 + kb2*32 + 16*(e/8) + 8*hl + e%8.  On the
  // walk the block carries its mask: whole (no key masked), or the lane's last
  // allowed key index within the block (keys past a partition's end included;
  // -1 past the end of the walk: every key masked).
  auto mask_half = [&](int /*position*/, const BlkMask& bm, int kb2, f32x16& s) {
    if (__builtin_expect(bm.whole, 1)) return;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kk = kb2 * 32 + (e >> 3) * 16 + hl * 8 + (e & 7);
      s[e] = kk <= bm.lim ? s[e] : -INFINITY;
    }
  };
  // one 32-key step: P, dS of the current half; S^T, dP^T of the next half under
  // the exponentials; dQ^T += K^T dS^T; mask of the next half
  auto half_step = [&](int st, int kb2, f32x16& sc, f32x16& dc, int ng, const BlkMask& nv, int nst, int nkb2,
                       f32x16& sn, f32x16& dn) {
    // ask the scheduler to interleave the LDS reads with the MFMAs (measured: the dQ
    // kernel 1.46 -> 1.42 ms at the 8k tile)
    __builtin_amdgcn_iglp_opt(0);
    bf16x8 dsf[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[j * 8 + i], c2, nl2));
        v[i] = pe * (dc[j * 8 + i] + nd);
      }
      dsf[j] = pack_bf16x8(v);
    }
    sdp_half(nst, nkb2, sn, dn);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t off = st * C::STAGE_BYTES + (kb2 * 2 + j) * 16 * D * 2;
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        const bf16x8 kt = concat_bf16x4(lds_read_tr16(ktr[c][0] + off), lds_read_tr16(ktr[c][1] + off));
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, dsf[j], acc[c], 0, 0, 0);
      }
    }
    mask_half(ng, nv, nkb2, sn);
  };

  // ---- pipeline (the forward's): position j in stage j % 4, loaded 2 ahead ----
  int bj0 = next_block(0);
  int bj1 = bj0 < total ? next_block(bj0 + 1) : total;
  int bj2 = bj1 < total ? next_block(bj1 + 1) : total;
  // nv0..nv2: masks of positions bj0..bj2 (every key masked when past the end)
  BlkMask nv0{0, -1}, nv1{0, -1}, nv2{0, -1};
  if (bj0 < total) nv0 = issue_at(0, bj0);
  if (bj1 < total) nv1 = issue_at(1, bj1);
  if (bj2 < total) nv2 = issue_at(2, bj2);
  f32x16 sA, dA, sB, dB;
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // also retires the fragment loads
  if (bj0 < total) {
    __syncthreads();
    sdp_half(0, 0, sA, dA);
    mask_half(bj0, nv0, 0, sA);
  }
#define MA_DQ_BLOCK(ST)                                                  \
  {                                                                      \
    half_step((ST), 0, sA, dA, bj0, nv0, (ST), 1, sB, dB);               \
    const int bj3 = bj2 < total ? next_block(bj2 + 1) : total;           \
    wait_positions(bj2 < total ? 1 : 0);                                 \
    __syncthreads();                                                     \
    const BlkMask nv3 = bj3 < total ? issue_at(((ST) + 3) & 3, bj3) : BlkMask{0, -1}; \
    half_step((ST), 1, sB, dB, bj1, nv1, ((ST) + 1) & 3, 0, sA, dA);     \
    bj0 = bj1;                                                           \
    bj1 = bj2;                                                           \
    bj2 = bj3;                                                           \
    nv0 = nv1;                                                           \
    nv1 = nv2;                                                           \
    nv2 = nv3;                                                           \
    if (bj0 >= total) break;                                             \
  }
  while (bj0 < total) {
    MA_DQ_BLOCK(0)
    MA_DQ_BLOCK(1)
    MA_DQ_BLOCK(2)
    MA_DQ_BLOCK(3)
  }
#undef MA_DQ_BLOCK

  if (!row_ok) return;
  float* dQg = QP.dq + (int64_t)b * p.dq_sb + (int64_t)my_head * p.dq_sh + (int64_t)row * p.dq_ss;
#pragma unroll
  for (int c = 0; c < C::NC; ++c)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float4 v = make_float4(acc[c][4 * g] * p.scale, acc[c][4 * g + 1] * p.scale, acc[c][4 * g + 2] * p.scale,
                             acc[c][4 * g + 3] * p.scale);
      float4* dst = (float4*)(dQg + c * 32 + 8 * g + 4 * hl);
      if (E.accumulate) {
        const float4 o = *dst;
        v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
      }
      *dst = v;
    }
}

// --------------------------------------------------------------- dK/dV kernel --
// MASKED: causal on positions; the query positions of every Q partition are one
// segment (they grow with the row index), so a lane's mask is the index of the
// first row allowed to see its key and the blocks with any allowed pair for the
// workgroup are a suffix of each (partition, head).
template <int D, bool MASKED>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_dkv_kernel(const BwdParams p) {
  using C = Cfg<D>;
  constexpr int kWaves = 4, kKW = 32;
  constexpr int LPW = kBN * C::CH / 64 / kWaves;
  // Q stages, then dO stages; LSE2/D blocks
  __shared__ __attribute__((aligned(1024))) __bf16 qd_s[2][kStages][C::BLK];
  __shared__ __attribute__((aligned(1024))) float ld_s[kStages][2 * kBN];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // ---- entry (KV group) / batch / KV head / key block ----
  const int w = blockIdx.x;
  int ei = 0;
  while (ei + 1 < p.nentries && w >= entry_at(ei + 1).wg_begin) ++ei;
  ei = __builtin_amdgcn_readfirstlane(ei);
  const BwdEntry E = entry_at(ei);
  const BwdKVPart KV = kvpart_at(E.self);
  const int local = w - E.wg_begin;
  const int kvh = local % p.hkv;
  const int rest = local / p.hkv;
  const int kblk = rest % E.chunks;
  const int b = rest / E.chunks;
  if (b >= p.batch) return;
  const int g0 = kv_first_at(kvh);
  const int gsz = kv_first_at(kvh + 1) - g0;
  const int key0 = kblk * (kWaves * kKW);
  const int wg_keys = min(kWaves * kKW, KV.sk - key0);
  // a KV head that no query head reads (an explicit head map may leave one) still gets its
  // dK and dV written: its walk has no blocks, so the epilogue stores zeros (or adds nothing)
  if (wg_keys <= 0) return;
  const int my_key = key0 + wave * kKW + l32;
  const bool key_ok = my_key < KV.sk;
  int wg_kmin = 0, wg_kmax = 0, w_kmin = 0, w_kmax = 0, my_kpos = INT32_MAX;
  if constexpr (MASKED) {
    pos_minmax_dev(KV.kp, KV.sk, key0, key0 + wg_keys, wg_kmin, wg_kmax);
    const int wk0 = min(KV.sk - 1, key0 + wave * kKW);
    pos_minmax_dev(KV.kp, KV.sk, wk0, min(KV.sk, key0 + wave * kKW + kKW), w_kmin, w_kmax);
    if (key_ok) my_kpos = pos_at_dev(KV.kp, my_key);
  }

  // ---- K^T and V^T fragments of this lane's key (B operands) ----
  bf16x8 kf[C::KS], vf[C::KS];
  {
    const int64_t off = (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh + (int64_t)my_key * p.k_ss;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      bf16x8 z = {};
      kf[ks] = key_ok ? *(const bf16x8*)((const __bf16*)KV.k + off + ks * 16 + hl * 8) : z;
      vf[ks] = key_ok ? *(const bf16x8*)((const __bf16*)KV.v + off + ks * 16 + hl * 8) : z;
    }
  }

  // ---- query blocks: (Q partition, head of the group, 64-row block), flattened ----
  // one query segment: the first row index whose position is at or after key
  // position kp (sq: none)
  auto first_row = [&](const BwdQPart& QP, int kp) {
    const int gb = QP.qp.gb[0], st = QP.qp.st[0];
    return kp <= gb ? 0 : (int)min((int64_t)QP.sq, ((int64_t)kp - gb + st - 1) / st);
  };
  // The walk visits, per (Q partition, head of the group), the 64-row blocks from the first one
  // with any allowed pair for the workgroup.  Masked, it runs in two phases: first the blocks in
  // which some key of the workgroup needs the element mask (two or three: the workgroup's 128 keys
  // span 128 query positions of a one-segment map), with the masked body; then the blocks that
  // every key of the workgroup sees whole, with the unmasked body, so that the mask's VALU work
  // is spent on the diagonal blocks only.  [qbeg, qend): the blocks of partition QP in this phase.
  int phase = MASKED ? 0 : 1;
  auto seg_range = [&](const BwdQPart& QP, int& qbeg, int& qend) {
    const int nqb = (QP.sq + kBN - 1) / kBN;
    if constexpr (MASKED) {
      const int qb0 = first_row(QP, wg_kmin) / kBN;
      const int qwhole = max(qb0, min(nqb, (first_row(QP, wg_kmax) + kBN - 1) / kBN));
      qbeg = phase == 0 ? qb0 : qwhole;
      qend = phase == 0 ? qwhole : nqb;
    } else {
      qbeg = 0;
      qend = nqb;
    }
  };
  int total = 0;  // blocks of the walk in this phase
  auto count_blocks = [&]() {
    total = 0;
#pragma unroll
    for (int i = 0; i < kBwdPerLaunch; ++i) {
      if (i < E.n) {
        int qbeg, qend;
        seg_range(qpart_at(partner_at(ei, i)), qbeg, qend);
        total += gsz * (qend - qbeg);
      }
    }
  };
  auto next_block = [&](int from) -> int { return from < total ? from : total; };

  // ---- direct-to-LDS loads of one Q block, one dO block and the LSE2/D block ----
  auto load_row = [&](int i) { return ((wave * LPW + i) * 64 + lane) / C::CH; };
  auto load_col = [&](int i) { return ((((wave * LPW + i) * 64 + lane) % C::CH) ^ swz<D>(load_row(i))) * 8; };
  const int q_ss = (int)p.q_ss;  // below 2^24 (checked by the caller)
  uint32_t go[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) go[i] = (uint32_t)(load_row(i) * q_ss + load_col(i)) * 2u;
  // The blocks are visited in order, so a cursor (partner, head, 64-row block)
  // and the bases and mask data of the current (partner, head), refreshed only
  // when those change, stand in for a per-block decode: no division or parameter
  // load per block (a scalar load would also make the wave wait for all of its
  // LDS reads).
  int c_pi = 0, c_hi = 0, c_qb = 0, c_qb0 = 0, c_qend = 0, c_nqb = 0, c_sq = 0, c_qfull = 0, c_tfirst = 0;
  const __bf16* c_q = nullptr;
  const __bf16* c_g = nullptr;
  const float* c_l = nullptr;
  auto cur_load = [&]() {  // bases of (c_pi, c_hi); the cursor starts at the first block with work
    for (;;) {
      const BwdQPart QP = qpart_at(partner_at(ei, c_pi));
      c_sq = QP.sq;
      c_nqb = (QP.sq + kBN - 1) / kBN;
      seg_range(QP, c_qb0, c_qend);
      if constexpr (MASKED) {
        c_tfirst = key_ok ? first_row(QP, my_kpos) : 0;
        c_qfull = (first_row(QP, w_kmax) + kBN - 1) / kBN;
      }
      if (c_qb0 < c_qend || c_pi + 1 >= E.n) break;
      ++c_pi;  // no block of this partition in this phase
    }
    c_qb = c_qb0;
    const int h = head_of(g0 + c_hi);
    const BwdQPart QP = qpart_at(partner_at(ei, c_pi));
    const int64_t off = (int64_t)b * p.q_sb + (int64_t)h * p.q_sh;
    c_q = (const __bf16*)QP.q + off;
    c_g = (const __bf16*)QP.dout + off;
    c_l = QP.lsed + ((int64_t)b * p.hq + h) * c_nqb * (2 * kBN);
  };
  auto issue_next = [&](int st) -> BlkMask {
    const int64_t roff = (int64_t)c_qb * kBN * p.q_ss;
    const __bf16* qbase = c_q + roff;
    const __bf16* gbase = c_g + roff;
    const int valid = c_sq - c_qb * kBN;
    if (valid >= kBN) {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        lds_dma16(qbase, go[i], lds_addr(&qd_s[0][st][(wave * LPW + i) * 512]));
        lds_dma16(gbase, go[i], lds_addr(&qd_s[1][st][(wave * LPW + i) * 512]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const uint32_t o2 = (uint32_t)(min(load_row(i), valid - 1) * q_ss + load_col(i)) * 2u;
        lds_dma16(qbase, o2, lds_addr(&qd_s[0][st][(wave * LPW + i) * 512]));
        lds_dma16(gbase, o2, lds_addr(&qd_s[1][st][(wave * LPW + i) * 512]));
      }
    }
    if (lane < 8) lds_dma16(c_l + c_qb * (2 * kBN), (uint32_t)(wave * 128 + lane * 16), lds_addr(&ld_s[st][wave * 32]));
    BlkMask bm{1, 0};
    if constexpr (MASKED) {  // every row of a whole block passes (-2^30)
      bm.whole = c_qb >= c_qfull;
      bm.lim = bm.whole ? -(1 << 30) : c_tfirst - c_qb * kBN;
    }
    if (++c_qb == c_qend) {
      if (++c_hi == gsz) {
        c_hi = 0;
        ++c_pi;
      }
      if (c_pi < E.n) cur_load();
    }
    return bm;
  };
  auto issue_at = [&](int st, int /*position*/) -> BlkMask { return issue_next(st); };
  auto wait_positions = [&](int n) {  // at most n later positions in flight
    if (n >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * (2 * LPW + 1)));
    else if (n == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPW + 1));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  };

  uint32_t qaddr[C::KS], qtr[C::NC][2], gaddr[C::KS], gtr[C::NC][2];
  tile_lane_addrs<D>(qd_s[0][0], lane, qaddr, qtr);
  tile_lane_addrs<D>(qd_s[1][0], lane, gaddr, gtr);
  const uint32_t laddr = lds_lane_addr(&ld_s[0][8 * hl]);  // + 32u (+16) floats; D at +64 floats
  constexpr uint32_t kLdStage = 2 * kBN * 4;

  f32x16 dk_acc[C::NC], dv_acc[C::NC];  // rows = keys 8(e/4) + 4hl + e%4 of the wave, column d = 32c + l32
#pragma unroll
  for (int c = 0; c < C::NC; ++c) {
    dk_acc[c] = f32x16{};
    dv_acc[c] = f32x16{};
  }
  const float c2 = p.scale_log2;

  // S - LSE/scale and dP - D of one 32-query half (u) of the block in stage st:
  // the accumulators start at the row values of the LSE2/D block
  auto sdp_half = [&](int st, int u, f32x16& s, f32x16& dp) {
    const uint32_t off = st * C::STAGE_BYTES + u * 32 * D * 2;
    const uint32_t lo = laddr + st * kLdStage + u * 32 * 4;
    const f32x4 l0 = lds_read_f32x4(lo), l1 = lds_read_f32x4(lo + 16);
    const f32x4 l2 = lds_read_f32x4(lo + 64), l3 = lds_read_f32x4(lo + 80);
    const f32x4 d0 = lds_read_f32x4(lo + 256), d1 = lds_read_f32x4(lo + 272);
    const f32x4 d2 = lds_read_f32x4(lo + 320), d3 = lds_read_f32x4(lo + 336);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = l0[i]; s[4 + i] = l1[i]; s[8 + i] = l2[i]; s[12 + i] = l3[i];
      dp[i] = d0[i]; dp[4 + i] = d1[i]; dp[8 + i] = d2[i]; dp[12 + i] = d3[i];
    }
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 qa = lds_read_b128(qaddr[ks] + off);
      const bf16x8 ga = lds_read_b128(gaddr[ks] + off);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vf[ks], dp, 0, 0, 0);
    }
  };
  // one 32-query step: element e of the lane is query 32u + 16(e/8) + 8hl + e%8.
  // Keys past the end of the partition need no mask: their dK/dV rows are never
  // stored and do not feed any other key's rows.  With position masks, the first
  // phase's blocks (not fully allowed for the workgroup) take a second copy of the
  // body that zeroes P where the key comes after the query; both copies are
  // straight-line code, so the VALU work interleaves with the MFMAs.
  auto half_body = [&](auto masked, int /*position*/, const BlkMask& bm, int st, int u, f32x16& sc, f32x16& dc, int nst, int nu,
                       f32x16& sn, f32x16& dn) {
    // one wave per SIMD: ask the scheduler to interleave the LDS reads with the
    // MFMAs (measured: 14% faster than the default schedule for this kernel)
    __builtin_amdgcn_iglp_opt(0);
    float pe[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) pe[e] = __builtin_amdgcn_exp2f(sc[e] * c2);
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {  // row of the block at or after this key's first allowed row
        const int rr = 32 * u + 16 * (e >> 3) + 8 * hl + (e & 7);
        pe[e] = rr >= bm.lim ? pe[e] : 0.f;
      }
    }
    bf16x8 pf[2], dsf[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float ds[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ds[i] = pe[j * 8 + i] * dc[j * 8 + i];
      pf[j] = pack_bf16x8(&pe[j * 8]);
      dsf[j] = pack_bf16x8(ds);
    }
    sdp_half(nst, nu, sn, dn);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t off = st * C::STAGE_BYTES + (u * 2 + j) * 16 * D * 2;
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        const bf16x8 gt = concat_bf16x4(lds_read_tr16(gtr[c][0] + off), lds_read_tr16(gtr[c][1] + off));
        const bf16x8 qt = concat_bf16x4(lds_read_tr16(qtr[c][0] + off), lds_read_tr16(qtr[c][1] + off));
        dv_acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[j], gt, dv_acc[c], 0, 0, 0);
        dk_acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsf[j], qt, dk_acc[c], 0, 0, 0);
      }
    }
  };
  // One phase of the walk: the ring of 4 stages, 3 blocks ahead, over the phase's blocks; the body
  // of every block is the masked or the unmasked one, straight-line code either way.
  auto run_phase = [&](auto masked) {
  auto half_step = [&](int g, const BlkMask& bm, int st, int u, f32x16& sc, f32x16& dc, int nst, int nu, f32x16& sn,
                       f32x16& dn) { half_body(masked, g, bm, st, u, sc, dc, nst, nu, sn, dn); };
  c_pi = 0;
  c_hi = 0;
  count_blocks();
  cur_load();
  int bj0 = next_block(0);
  int bj1 = bj0 < total ? next_block(bj0 + 1) : total;
  int bj2 = bj1 < total ? next_block(bj1 + 1) : total;
  BlkMask m0{1, 0}, m1{1, 0}, m2{1, 0};  // masks of positions bj0..bj2
  if (bj0 < total) m0 = issue_at(0, bj0);
  if (bj1 < total) m1 = issue_at(1, bj1);
  if (bj2 < total) m2 = issue_at(2, bj2);
  f32x16 sA, dA, sB, dB;
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // also retires the fragment loads
  if (bj0 < total) {
    __syncthreads();
    sdp_half(0, 0, sA, dA);
  }
#define MA_DKV_BLOCK(ST)                                                 \
  {                                                                      \
    half_step(bj0, m0, (ST), 0, sA, dA, (ST), 1, sB, dB);                \
    const int bj3 = bj2 < total ? next_block(bj2 + 1) : total;           \
    wait_positions(bj2 < total ? 1 : 0);                                 \
    __syncthreads();                                                     \
    const BlkMask m3 = bj3 < total ? issue_at(((ST) + 3) & 3, bj3) : BlkMask{1, 0}; \
    half_step(bj0, m0, (ST), 1, sB, dB, ((ST) + 1) & 3, 0, sA, dA);      \
    bj0 = bj1;                                                           \
    bj1 = bj2;                                                           \
    bj2 = bj3;                                                           \
    m0 = m1;                                                             \
    m1 = m2;                                                             \
    m2 = m3;                                                             \
    if (bj0 >= total) break;                                             \
  }
  while (bj0 < total) {
    MA_DKV_BLOCK(0)
    MA_DKV_BLOCK(1)
    MA_DKV_BLOCK(2)
    MA_DKV_BLOCK(3)
  }
#undef MA_DKV_BLOCK
  };
  if constexpr (MASKED) {
    run_phase(std::true_type{});
    __syncthreads();  // every wave is done with the stages before the second phase refills them
    phase = 1;
    run_phase(std::false_type{});
  } else {
    run_phase(std::false_type{});
  }

  // ---- dK (scaled) and dV of the wave's 32 keys ----
  float* dKg = KV.dk + (int64_t)b * p.dk_sb + (int64_t)kvh * p.dk_sh;
  float* dVg = KV.dv + (int64_t)b * p.dk_sb + (int64_t)kvh * p.dk_sh;
#pragma unroll
  for (int c = 0; c < C::NC; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = key0 + wave * kKW + (e >> 2) * 8 + hl * 4 + (e & 3);
      if (key < KV.sk) {
        const int64_t off = (int64_t)key * p.dk_ss + c * 32 + l32;
        float kv = dk_acc[c][e] * p.scale, vv = dv_acc[c][e];
        if (E.accumulate) {
          kv += dKg[off];
          vv += dVg[off];
        }
        dKg[off] = kv;
        dVg[off] = vv;
      }
    }
}

}  // namespace

int launch_bwd_preprocess(const BwdPreParams& p, int head_dim, void* stream) {
  const int64_t nqb = (p.sq + kBN - 1) / kBN;
  const int64_t rows = (int64_t)p.batch * nqb * kBN * p.hq;
  const int rpb = 256 / (head_dim / 8);
  const int64_t blocks = (rows + rpb - 1) / rpb;
  if (blocks <= 0) return 0;
  if (head_dim == 128)
    hipLaunchKernelGGL(bwd_pre_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

int launch_bwd_dq(const BwdParams& p, int head_dim, int total_wgs, void* stream) {
  if (total_wgs <= 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  dim3 g(total_wgs), blk(512);
  if (head_dim == 128) {
    if (p.mask) hipLaunchKernelGGL((bwd_dq_kernel<128, true>), g, blk, 0, s, p);
    else hipLaunchKernelGGL((bwd_dq_kernel<128, false>), g, blk, 0, s, p);
  } else {
    if (p.mask) hipLaunchKernelGGL((bwd_dq_kernel<64, true>), g, blk, 0, s, p);
    else hipLaunchKernelGGL((bwd_dq_kernel<64, false>), g, blk, 0, s, p);
  }
  return (int)hipGetLastError();
}

int launch_bwd_dkv(const BwdParams& p, int head_dim, int total_wgs, void* stream) {
  if (total_wgs <= 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  dim3 g(total_wgs), blk(256);
  if (head_dim == 128) {
    if (p.mask) hipLaunchKernelGGL((bwd_dkv_kernel<128, true>), g, blk, 0, s, p);
    else hipLaunchKernelGGL((bwd_dkv_kernel<128, false>), g, blk, 0, s, p);
  } else {
    if (p.mask) hipLaunchKernelGGL((bwd_dkv_kernel<64, true>), g, blk, 0, s, p);
    else hipLaunchKernelGGL((bwd_dkv_kernel<64, false>), g, blk, 0, s, p);
  }
  return (int)hipGetLastError();
}

}  // namespace ma
