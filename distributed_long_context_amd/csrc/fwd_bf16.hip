// Tile forward, bf16 inputs, fp32 accumulation, for CDNA4 (gfx950).
//
// What one tile computes is the partial attention of [Mesh] section 2.2
// ((O_ij, lse_ij) = Attention(Q_i, K_j, V_j)) with the blockwise online softmax
// of [Ring] "Ring Attention: Pass KV Blocks Around the Ring" (running max,
// running denominator, unnormalised output).  The layout on the chip is this
// file's own design:
//
//  * A workgroup is 8 waves, two per SIMD; each wave owns 32 query rows of one
//    query head and all waves read the same KV head, so one LDS copy of a
//    64-key K/V block serves 256 query rows.  A wave's state (O^T, its Q
//    fragments, two score tiles) fits in the 256 architectural VGPRs, and the
//    two waves of a SIMD overlap one's softmax with the other's MFMAs.
//    Workgroup index modulo the KV head count picks the KV head, so with 8 KV
//    heads each XCD's L2 serves one.
//  * K and V blocks go from global memory straight into LDS
//    (global_load_lds_dwordx4, no register staging) through a ring of five
//    stages (all 160 KB of LDS at d = 128); two blocks are issued together every
//    other block, three and four blocks ahead, so one workgroup barrier covers
//    two blocks (measured 1% faster than four stages with a barrier per block).
//    16-byte chunks of each row are XOR-swizzled by row so that both the b128
//    reads of K and the transposed b64 reads of V are free of bank conflicts on
//    the 64-bank LDS.  K stages and V stages sit in two separate regions and the
//    loop is unrolled over ten blocks, so every fragment read is a lane offset
//    plus an immediate.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    each lane owns one query (16 of the keys of a 32-key tile, the other 16 in
//    lane l^32), so the row max needs one permlane32 swap.  K rows enter the
//    MFMA in a permuted order (bits 2 and 3 of the row index swapped) so that
//    each lane's 16 accumulator values are, unchanged, the B operand (P^T) of
//    O^T = V^T P^T; V^T fragments come from ds_read_b64_tr_b16.
//  * Software pipeline over 32-key steps: while the exponentials of step h run
//    on the VALU, the MFMAs of the scores of step h+1 are in flight; then
//    O^T += V_h^T P_h^T runs while step h+1 is masked and its row max taken.
//  * Softmax runs in base 2 with scale*log2(e) folded into one FMA; the running
//    max is only raised when a row's block max exceeds it by more than 8
//    (factor 256), which keeps the result exact while skipping most rescales.
//  * Masks are resolved per 64-key block ([Mesh] section 3.7 pair classes):
//    blocks with no allowed pair for the workgroup are never loaded, blocks with
//    every pair allowed run unmasked, the rest (and a ragged last block) are
//    masked element by element.  Tiles that are FULL as a whole run the kernel
//    without masks; the masked kernel takes key positions of one segment
//    (contiguous or striped; a tile of several key segments is cut by the host into
//    one piece per segment, chained in the tile table, and a workgroup runs the
//    pieces in turn with its softmax state in registers), which grow with the key
//    index, so a lane keeps only the
//    index of its last allowed key, a wave the count of leading blocks it sees
//    whole and the workgroup the count of blocks with any allowed pair; no
//    position data stays live in the loop.
//  * Three instances: the ring kernel above with 8 waves (long tiles) or 4 waves
//    and a two-stage ring (tiles of at most 16 key blocks, two workgroups per CU),
//    and a resident-KV kernel for unmasked tiles of a few hundred keys, whose
//    workgroup holds the tile's whole K and V in LDS and runs up to 32 units of
//    32 query rows against it, or from a tile table up to 128 units of the tiles
//    that share that K and V (see its own comment below).
#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>

#include "ma_internal.h"
#include "ma_device.h"

namespace ma {

namespace {

constexpr int kQW = 32;  // query rows per wave
constexpr int kBN = 64;  // keys per block

// WAVES = 8: one workgroup per CU, a five-stage ring (160 KB at d = 128).
// WAVES = 4: two workgroups per CU, a two-stage ring (64 KB), for tiles of few key
// blocks, where one workgroup's start-up (its first loads) then overlaps the other's
// loop (small tiles 15-20% faster; long tiles 6% slower than with eight waves).
template <int D, int WAVES>
struct FwdCfg {
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int KS = D / 16;                  // MFMA k-steps over d
  static constexpr int NC = D / 32;                  // 32-row chunks of O^T
  static constexpr int BLK = kBN * D;                // elements of one K or V block
  static constexpr int LPW = kBN * CH / 64 / WAVES;  // direct-to-LDS loads per wave per tensor
  static constexpr int STAGES = WAVES == 8 ? 5 : 2;
};

// The same address as a global-memory pointer: loads and stores through it are global, not flat,
// instructions (a flat access also counts against the LDS wait counter), also where the compiler
// cannot tell the address space itself, as for pointers read from a tile table.
template <class X>
__device__ __forceinline__ __attribute__((address_space(1))) X* gmem(X* ptr) {
  return (__attribute__((address_space(1))) X*)ptr;
}

// ---- pieces of a 32-key step shared by the ring and resident-KV kernels ----
// A wave owns 32 query rows (one per lane pair l, l^32); a 32-key half of a K/V block is one
// 32 x 32 score tile S^T = K Q^T whose lane holds its query's 16 keys 16*(e/8) + 8*hl + e%8.

// S^T of the half at LDS byte offset off (fragment addresses kaddr, query fragments qf)
template <int KS>
__device__ __forceinline__ void fwd_scores(const uint32_t (&kaddr)[KS], uint32_t off, const bf16x8 (&qf)[KS],
                                           f32x16& s) {
  s = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 kf = lds_read_b128(kaddr[ks] + off);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s, 0, 0, 0);
  }
}

// keys after klast set to -inf (key0: the key index of the half's first element); branch-free
__device__ __forceinline__ void fwd_mask_keys(f32x16& s, int key0, int hl, int klast) {
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int key = key0 + (e >> 3) * 16 + hl * 8 + (e & 7);
    s[e] = key <= klast ? s[e] : -INFINITY;
  }
}

// the row's max over the half, in log2 units (c2 = scale * log2(e))
__device__ __forceinline__ float fwd_row_max(const f32x16& s, float c2) {
  // a tree of three-input maxima (v_max3_f32): 8 instructions, 3 deep
  const float a = fmaxf(fmaxf(s[0], s[1]), s[2]), b = fmaxf(fmaxf(s[3], s[4]), s[5]);
  const float c = fmaxf(fmaxf(s[6], s[7]), s[8]), d = fmaxf(fmaxf(s[9], s[10]), s[11]);
  const float e = fmaxf(fmaxf(s[12], s[13]), s[14]);
  const float mx = fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), s[15]));
  return xhalf_max(mx) * c2;
}

// Lazy rescale: the running max m2 is raised only when some row's new max mb2 exceeds it by more
// than 8 (factor 256), which keeps the result exact while skipping most rescales.
template <int NC>
__device__ __forceinline__ void fwd_maybe_rescale(f32x16 (&oacc)[NC], float& m2, float& lsum, float mb2) {
  if (__any(mb2 > m2 + 8.0f)) {
    const float mn = fmaxf(m2, mb2);
    const float alpha = (mn == -INFINITY || m2 == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m2 - mn);
    lsum *= alpha;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[c][i] *= alpha;
    m2 = mn;
  }
}

// P = exp2(S c2 - m2) of the half, added to the lane's row sum and packed to bf16 (the B
// operand of O^T += V^T P^T)
__device__ __forceinline__ void fwd_probs(const f32x16& sc, float c2, float m2, float& lsum, bf16x8 (&pf)[2]) {
  const float mref = (m2 == -INFINITY) ? 0.0f : m2;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[half * 8 + i], c2, -mref));
      lsum += pv[i];
    }
    pf[half] = pack_bf16x8(pv);
  }
}

// O^T += V^T P^T over the half whose first 16-key slice starts at LDS byte offset off (V^T
// fragments read transposed; a slice is 16 rows of 2*D bytes)
template <int D, int NC>
__device__ __forceinline__ void fwd_pv(const uint32_t (&vaddr)[NC][2], uint32_t off, const bf16x8 (&pf)[2],
                                       f32x16 (&oacc)[NC]) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bf16x4 lo = lds_read_tr16(vaddr[c][0] + off + half * 16 * D * 2);
      const bf16x4 hi = lds_read_tr16(vaddr[c][1] + off + half * 16 * D * 2);
      oacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(concat_bf16x4(lo, hi), pf[half], oacc[c], 0, 0, 0);
    }
  }
}

// Epilogue of one wave's 32 query rows: normalise O^T by the row sum and store O (bf16) and
// LSE (fp32, natural log), or fold them into the (O, LSE) the buffers hold (accumulate):
// L = ln(e^lse_old + e^lse), O = e^(lse_old - L) O_old + e^(lse - L) O.  orow and lrow address
// the lane's row; m2 is the running max in log2 units, ltot the row sum (both halves of the wave).
template <int NC>
__device__ __forceinline__ void fwd_store_rows(const f32x16 (&oacc)[NC], float m2, float ltot, bool accumulate,
                                               __bf16* orow, float* lrow, int hl) {
  const bool has = ltot > 0.0f;
  float lse = has ? (m2 + __builtin_amdgcn_logf(ltot)) * 0.69314718055994531f : -INFINITY;
  float wn = has ? 1.0f / ltot : 0.0f;  // weight of this tile's unnormalised sums
  float wo = 0.0f;                      // weight of the output already held (accumulate)
  bf16x4 old[NC][4];                    // the output already held, all loads issued before any use
  if (accumulate) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int g = 0; g < 4; ++g) old[c][g] = *gmem((const bf16x4*)(orow + c * 32 + g * 8 + hl * 4));
    const float lo = *gmem(lrow);
    const float mx = fmaxf(lo, lse);
    if (mx == -INFINITY) {
      wn = 0.0f;
    } else {
      const float eo = __expf(lo - mx), en = __expf(lse - mx);
      const float sum = eo + en;
      wo = eo / sum;
      wn *= en / sum;
      lse = mx + __logf(sum);
    }
  }
  // Lane l holds columns c*32 + g*8 + {0..3} of its row and lane l^32 the next four, for g = 0..3.
  // One swap across the halves per packed dword gives lane l columns c*32 + 16*gp + {0..7} and
  // lane l^32 the eight after them, so each lane stores 16 contiguous bytes: half the store
  // instructions, each writing 32 contiguous bytes per row (measured 5% faster on 210-token tiles).
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    u32x2 w[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float v4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v4[i] = oacc[c][g * 4 + i] * wn;
      if (accumulate) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = __builtin_fmaf(wo, (float)old[c][g][i], v4[i]);
      }
      w[g] = __builtin_bit_cast(u32x2, pack_bf16x4(v4));
    }
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      u32x4 o4;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        // lanes 32-63 of the first operand trade places with lanes 0-31 of the second
        const auto r = __builtin_amdgcn_permlane32_swap(w[2 * gp][k], w[2 * gp + 1][k], false, false);
        o4[k] = r[0];
        o4[2 + k] = r[1];
      }
      *gmem((u32x4*)(orow + c * 32 + gp * 16 + hl * 8)) = o4;
    }
  }
  *gmem(lrow) = lse;  // lanes l and l^32 hold the same row and value: one store, no branch
}

// MASKED: causal on positions, the key positions one segment (global = kgb +
// t * kst, growing with t), so every mask decision reduces to the last allowed
// key index of a query position.  Without it only a ragged last block is masked.
template <int D, bool MASKED, int WAVES>
__global__ void __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_kernel(const FwdParams p) {
  using C = FwdCfg<D, WAVES>;
  constexpr int kWaves = WAVES;
  // K stages in the first half, V stages in the second: kv_s[0][st] is K, kv_s[1][st] is V
  __shared__ __attribute__((aligned(1024))) __bf16 kv_s[2][C::STAGES][C::BLK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // ---- which tile / batch / KV head / query block ----
  const int w = blockIdx.x;
  // tile of this workgroup: the count of later tiles that start at or before it
  // (independent scalar loads instead of a chain of dependent ones)
  int ti = 0;
#pragma unroll
  for (int j = 1; j < kFwdTilesPerLaunch; ++j) ti += (j < p.ntiles && w >= p.tiles[j].wg_begin) ? 1 : 0;
  // by value, with a provably uniform index: the parameter block stays in the
  // kernel-argument segment (scalar loads) instead of being copied to scratch
  const FwdTile T = p.tiles[__builtin_amdgcn_readfirstlane(ti)];
  const int local = w - T.wg_begin;
  const int kvh = local % p.hkv;
  const int rest = local / p.hkv;
  // causal tiles: later query rows see more keys, so the heaviest chunks go first
  const int chunk = MASKED ? T.chunks - 1 - rest % T.chunks : rest % T.chunks;
  const int b = rest / T.chunks;
  if (b >= p.batch) return;  // padding workgroup (uniform)
  const int g0 = p.kv_first[kvh];
  const int gsz = p.kv_first[kvh + 1] - g0;
  if (gsz <= 0) return;
  const int nqb = (T.sq + kQW - 1) / kQW;

  // units of this workgroup: (query block, head) pairs, query-block major
  int wg_qlo = INT32_MAX, wg_qhi = INT32_MIN;
  int my_qb = -1, my_head = 0;
  for (int wv = 0; wv < kWaves; ++wv) {
    const int u = chunk * kWaves + wv;
    const int qb = u / gsz;
    if (qb >= nqb) continue;
    wg_qlo = min(wg_qlo, qb * kQW);
    wg_qhi = max(wg_qhi, min(T.sq, qb * kQW + kQW));
    if (wv == wave) {
      my_qb = qb;
      my_head = p.heads_of[g0 + (u % gsz)];
    }
  }
  if (wg_qlo == INT32_MAX) return;  // no unit in this workgroup (uniform)
  const bool active = my_qb >= 0;
  const int q0 = active ? my_qb * kQW : wg_qlo;

  int wg_pmin = 0, wg_pmax = 0, w_pmin = 0, w_pmax = 0;
  if constexpr (MASKED) {
    pos_minmax_dev(T.qp, T.sq, wg_qlo, wg_qhi, wg_pmin, wg_pmax);
    pos_minmax_dev(T.qp, T.sq, q0, min(T.sq, q0 + kQW), w_pmin, w_pmax);
  }

  // key side of the current tile; a chain of tiles (one per key segment of a partition, the
  // masked instance only) changes it between pipelines while the softmax state carries over
  const __bf16* Kg = nullptr;
  const __bf16* Vg = nullptr;
  int sk = 0;
  const int k_ss = (int)p.k_ss, v_ss = (int)p.v_ss;  // below 2^24 (checked by the caller)

  // ---- query fragments (B operand of S^T = K Q^T) and query position ----
  bf16x8 qf[C::KS];
  int qpos = 0;
  {
    const __bf16* Qg = (const __bf16*)T.q + (int64_t)b * p.q_sb + (int64_t)my_head * p.q_sh;
    const int row = q0 + l32;
    const bool ok = active && row < T.sq;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      bf16x8 z = {};
      qf[ks] = ok ? *(const bf16x8*)(Qg + (int64_t)row * p.q_ss + ks * 16 + hl * 8) : z;
    }
    if constexpr (MASKED) qpos = ok ? pos_at_dev(T.qp, row) : INT32_MIN;
  }

  // ---- which blocks, and which keys of a block, a lane may see ----
  // klast: this lane's last allowed key (-1: none); kfull_w: the leading blocks
  // every row of the wave sees whole; nkb: the blocks with any allowed pair for
  // the workgroup (the blocks after them have none).  Without a mask every key
  // of the partition is allowed and only a ragged last block is partial.
  int klast = 0, kfull_w = 0, nkb = 0;
  auto set_keys = [&](const FwdTile& X) {
    Kg = (const __bf16*)X.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
    Vg = (const __bf16*)X.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh;
    sk = X.sk;
    klast = sk - 1;
    kfull_w = sk / kBN;
    nkb = (sk + kBN - 1) / kBN;
    if constexpr (MASKED) {
      const int kgb = X.kgb, kst = X.kst;
      auto last_key = [&](int pq) { return pq < kgb ? -1 : min(sk - 1, (pq - kgb) / kst); };
      klast = last_key(qpos);
      kfull_w = active ? (last_key(w_pmin) + 1) / kBN : 0;
      nkb = (last_key(wg_pmax) + kBN) / kBN;
    }
  };
  set_keys(T);

  // ---- direct-to-LDS loads: wave instruction i fills LDS chunks [(wave*LPW+i)*64, +64) ----
  auto load_row = [&](int i) { return ((wave * C::LPW + i) * 64 + lane) / C::CH; };
  auto load_col = [&](int i) { return ((((wave * C::LPW + i) * 64 + lane) % C::CH) ^ swz<D>(load_row(i))) * 8; };
  uint32_t kgo[C::LPW], vgo[C::LPW];  // byte offsets of this lane's chunks inside a full block
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    kgo[i] = (uint32_t)(load_row(i) * k_ss + load_col(i)) * 2u;
    vgo[i] = (uint32_t)(load_row(i) * v_ss + load_col(i)) * 2u;
  }
  auto issue = [&](int st, int kb) {
    const __bf16* kbase = Kg + (int64_t)kb * kBN * p.k_ss;
    const __bf16* vbase = Vg + (int64_t)kb * kBN * p.v_ss;
    const int valid = sk - kb * kBN;  // rows of this block inside the partition
    if (valid >= kBN) {
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) {
        lds_dma16(kbase, kgo[i], lds_addr(&kv_s[0][st][(wave * C::LPW + i) * 512]));
        lds_dma16(vbase, vgo[i], lds_addr(&kv_s[1][st][(wave * C::LPW + i) * 512]));
      }
    } else {  // ragged last block: rows past the end repeat the last row (finite; masked later)
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) {
        const int r = min(load_row(i), valid - 1);
        lds_dma16(kbase, (uint32_t)(r * k_ss + load_col(i)) * 2u, lds_addr(&kv_s[0][st][(wave * C::LPW + i) * 512]));
        lds_dma16(vbase, (uint32_t)(r * v_ss + load_col(i)) * 2u, lds_addr(&kv_s[1][st][(wave * C::LPW + i) * 512]));
      }
    }
  };

  // ---- per-lane LDS byte addresses of the K and V^T fragments (stage 0, first slice) ----
  uint32_t kaddr[C::KS], kaddr_tr_unused[C::NC][2], vaddr_b128_unused[C::KS], vaddr[C::NC][2];
  tile_lane_addrs<D>(kv_s[0][0], lane, kaddr, kaddr_tr_unused);
  tile_lane_addrs<D>(kv_s[1][0], lane, vaddr_b128_unused, vaddr);
  constexpr uint32_t kStageBytes = C::BLK * 2;

  // ---- accumulators ----
  f32x16 oacc[C::NC];
#pragma unroll
  for (int c = 0; c < C::NC; ++c) oacc[c] = f32x16{};
  float m2 = -INFINITY;  // running max in log2 units
  float lsum = 0.f;      // this lane's share of the row sum
  const float c2 = p.scale_log2;

  // S^T of one 32-key half (kb2) of the block in stage st
  auto s_half = [&](int st, int kb2, f32x16& s) { fwd_scores(kaddr, st * kStageBytes + kb2 * 32 * D * 2, qf, s); };
  // mask (when the block is not whole for this wave) and row max of a half
  float mb2 = -INFINITY;
  auto half_max = [&](int kb, int kb2, f32x16& s) {
    if (kb >= kfull_w) fwd_mask_keys(s, kb * kBN + kb2 * 32, hl, klast);
    mb2 = fwd_row_max(s, c2);
  };
  auto maybe_rescale = [&]() { fwd_maybe_rescale(oacc, m2, lsum, mb2); };

  // One pipeline step over a 32-key half (stage st, half kb2) whose scores are
  // in sc and whose max is already folded into m2: the exponentials while the
  // MFMAs of the next half's scores (block nkb_, stage nst, half nkb2) run, then
  // the half's PV MFMAs while the next half is masked and its row max taken.
  // A half past the last block reads a stale stage; half_max masks it to -inf
  // (no key of a block index >= nkb is allowed), so it never changes the state.
  // Without element masks (no position mask, key count a multiple of 64) the row
  // max of the next half needs no branch, so the whole step is one straight-line
  // region the scheduler can interleave; a half past the last block then only
  // has its max forced to -inf.
  auto half_max_plain = [&](bool valid, f32x16& s) {
    const float m = fwd_row_max(s, c2);
    mb2 = valid ? m : -INFINITY;
  };

  auto half_step = [&](auto may_mask, int st, int kb2, f32x16& sc, int nkb_, int nst, int nkb2, f32x16& sn) {
    // With position masks or four waves, the wave raises its priority for the exponentials and
    // MFMAs and drops it for the mask and max that follow, so the two waves of a SIMD alternate
    // more strictly (measured: the causal 8k diagonal tile 2% and 840-token tiles 2.5% faster;
    // the eight-wave instance without masks 1.4% slower, so not there).
    constexpr bool kPrio = MASKED || WAVES == 4;
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
    // scheduler hint: LDS reads interleaved with the MFMAs (measured 0.5-1% faster at the 8k tile)
    __builtin_amdgcn_iglp_opt(0);
    bf16x8 pf[2];
    fwd_probs(sc, c2, m2, lsum, pf);
    s_half(nst, nkb2, sn);
    fwd_pv<D>(vaddr, st * kStageBytes + kb2 * 32 * D * 2, pf, oacc);
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
    if constexpr (decltype(may_mask)::value) half_max(nkb_, nkb2, sn);
    else half_max_plain(nkb_ < nkb, sn);
  };

  // ---- pipeline over the blocks with any allowed pair for the workgroup ----
  // Block j lives in stage j % 5.  Blocks go in pairs (j even): after the first
  // step of block j every wave waits for its loads of blocks j+1 and j+2 and the
  // barrier publishes them (block j+2's keys are first read by the last step of
  // the pair); blocks j+3 and j+4 are then issued into the stages of blocks j-2
  // and j-1, which every wave has finished reading.
  auto pipeline = [&](auto may_mask) {
    if constexpr (C::STAGES == 2) {
      // Block j lives in stage j & 1.  Block j+1 is published (wait and barrier) after
      // the first half of block j, whose second half computes its first scores; block
      // j+2 is issued into stage j & 1 once every wave has finished block j.
      if (0 < nkb) issue(0, 0);
      if (1 < nkb) issue(1, 1);
      f32x16 sA, sB;
      if (1 < nkb) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * C::LPW));  // block 0 and the query fragments
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      if (nkb <= 0) return;
      __syncthreads();
      s_half(0, 0, sA);
      if constexpr (decltype(may_mask)::value) half_max(0, 0, sA);
      else half_max_plain(true, sA);
      maybe_rescale();
      // one block in stage ST (a compile-time stage, so every LDS offset is an immediate);
      // false once the last block is done
      auto block = [&](auto stage, int j) -> bool {
        constexpr int st = decltype(stage)::value;
        half_step(may_mask, st, 0, sA, j, st, 1, sB);
        maybe_rescale();
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        half_step(may_mask, st, 1, sB, j + 1, st ^ 1, 0, sA);
        maybe_rescale();
        if (j + 1 >= nkb) return false;
        __syncthreads();
        if (j + 2 < nkb) issue(st, j + 2);
        return true;
      };
      for (int j = 0;; j += 2) {
        if (!block(std::integral_constant<int, 0>{}, j)) break;
        if (!block(std::integral_constant<int, 1>{}, j + 1)) break;
      }
    } else {
    if (0 < nkb) issue(0, 0);
    if (1 < nkb) issue(1, 1);
    if (2 < nkb) issue(2, 2);
    f32x16 sA, sB;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    if (nkb <= 0) return;
    __syncthreads();
    s_half(0, 0, sA);
    if constexpr (decltype(may_mask)::value) half_max(0, 0, sA);
    else half_max_plain(true, sA);
    maybe_rescale();
    int j = 0;
#define MA_FWD_PAIR(ST)                                                                   \
  {                                                                                       \
    half_step(may_mask, (ST), 0, sA, j, (ST), 1, sB);                                     \
    maybe_rescale();                                                                      \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));                                             \
    __syncthreads();                                                                      \
    if (j + 3 < nkb) issue(((ST) + 3) % 5, j + 3);                                        \
    if (j + 4 < nkb) issue(((ST) + 4) % 5, j + 4);                                        \
    half_step(may_mask, (ST), 1, sB, j + 1, ((ST) + 1) % 5, 0, sA);                       \
    maybe_rescale();                                                                      \
    if (j + 1 >= nkb) break;                                                              \
    half_step(may_mask, ((ST) + 1) % 5, 0, sA, j + 1, ((ST) + 1) % 5, 1, sB);             \
    maybe_rescale();                                                                      \
    half_step(may_mask, ((ST) + 1) % 5, 1, sB, j + 2, ((ST) + 2) % 5, 0, sA);             \
    maybe_rescale();                                                                      \
    j += 2;                                                                               \
    if (j >= nkb) break;                                                                  \
  }
    while (true) {
      MA_FWD_PAIR(0)
      MA_FWD_PAIR(2)
      MA_FWD_PAIR(4)
      MA_FWD_PAIR(1)
      MA_FWD_PAIR(3)
    }
#undef MA_FWD_PAIR
    }
  };
  if constexpr (MASKED) {
    // the tile and the key segments chained to it: the entries after the tile flagged as
    // continuations (same query rows and output, one key segment each) run in turn
    int tj = __builtin_amdgcn_readfirstlane(ti);
    for (;;) {
      pipeline(std::true_type{});
      if (tj + 1 >= p.ntiles) break;
      const FwdTile N = p.tiles[__builtin_amdgcn_readfirstlane(tj + 1)];
      if (!(N.accumulate & kFwdChained)) break;
      ++tj;
      __syncthreads();  // every wave is done with the ring before it is refilled
      set_keys(N);
    }
  } else {
    if (sk % kBN != 0) pipeline(std::true_type{});  // ragged last block needs the key mask
    else pipeline(std::false_type{});
  }

  if (!active) return;
  // ---- epilogue ----
  const float ltot = xhalf_sum(lsum);
  const int row = q0 + l32;
  if (row >= T.sq) return;
  __bf16* orow = (__bf16*)T.o + (int64_t)b * p.o_sb + (int64_t)my_head * p.o_sh + (int64_t)row * p.o_ss;
  float* lrow = T.lse + (int64_t)b * p.l_sb + (int64_t)my_head * p.l_sh + row;
  fwd_store_rows(oacc, m2, ltot, T.accumulate & 1, orow, lrow, hl);
}

// Through the scalar cache: the tile table is written before the launch and never during it.
template <class X>
__device__ __forceinline__ X table_load(const X* ptr) {
  static_assert(sizeof(X) % 4 == 0, "whole dwords");
  typedef const __attribute__((address_space(4))) uint32_t* cptr;
  const cptr src = (cptr)(const __attribute__((address_space(4))) char*)(const char*)ptr;
  uint32_t w[sizeof(X) / 4];
#pragma unroll
  for (size_t i = 0; i < sizeof(X) / 4; ++i) w[i] = src[i];
  X x;
  __builtin_memcpy(&x, w, sizeof(X));
  return x;
}

// Resident-KV instance, for unmasked tiles of few keys (kFwdResMinKeys < sk <= kFwdResKeys<D>):
// one workgroup of 8 waves (two per SIMD) per (tile, batch, KV head, chunk of up to
// kFwdResUnits units) loads the whole K and V of its KV head into LDS once, then every wave runs
// its units (32 query rows of one query head; unit u of the chunk goes to wave u % 8) in turn
// against the resident blocks, with no barrier after the loads and the next unit's query
// fragments loaded under the current unit's blocks.  The ring kernel instead gives each
// workgroup only 4 or 8 units and re-streams K/V for every workgroup, so at a few hundred keys
// its start-up dominates.  A unit's online softmax is the ring kernel's, step for step (the
// results are the same bit for bit), over the 32-key halves that hold a key of the tile: a half
// wholly past the last key, and the scores after the last half, are not computed.
//
// TABLE: the tiles come from a table in device memory, for calls of many more tiles than the
// kernel-argument table holds.  Tiles with the same K and V form a group, and a workgroup runs a
// range of units of one group (p.res_wgs[p.wg_base + blockIdx.x]), whatever tiles they belong to,
// against one LDS copy of K/V: with many tiles sharing a KV partition a workgroup amortises its
// loads over up to kFwdResUnitsMax units, split evenly over its waves.  Before anything else every
// workgroup checks the table's header against what the host planned for these arguments (tile,
// entry and workgroup counts, hash); on a mismatch (a table packed for other arguments, or changed
// since) it returns at once, so the launch writes nothing rather than reading stale pointers.
template <int D, bool TABLE>
__global__ void __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_resident_kernel(const FwdParams p) {
  using C = FwdCfg<D, 8>;
  constexpr int kWaves = 8;
  constexpr int RB = kFwdResKeys<D> / kBN;  // resident blocks
  __shared__ __attribute__((aligned(1024))) __bf16 kv_s[2][RB][C::BLK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // ---- the workgroup's batch, KV head, K/V tile and range of units ----
  FwdTile T;  // the tile (TABLE: the group's first tile, whose K/V every tile of the group has)
  int b, kvh, u_begin, u_end, ent = 0;
  if constexpr (TABLE) {
    const FwdTableHeader hd = table_load(p.table_header);
    if (hd.magic != kFwdTableMagic || hd.ntiles != p.table_ntiles || hd.nents != p.table_nents ||
        hd.nwgs != p.table_nwgs || hd.hash != p.table_hash)
      return;  // uniform: not the table these arguments were packed into
    const FwdResWg R = table_load(p.res_wgs + p.wg_base + blockIdx.x);
    ent = R.ent;
    T = table_load(p.table + table_load(&p.res_ents[ent].tile));
    b = R.bk / p.hkv;
    kvh = R.bk % p.hkv;
    u_begin = R.u_begin;
    u_end = R.u_end;
  } else {
    const int w = blockIdx.x;
    int ti = 0;
#pragma unroll
    for (int j = 1; j < kFwdTilesPerLaunch; ++j) ti += (j < p.ntiles && w >= p.tiles[j].wg_begin) ? 1 : 0;
    T = p.tiles[__builtin_amdgcn_readfirstlane(ti)];
    const int local = w - T.wg_begin;
    kvh = local % p.hkv;
    const int rest = local / p.hkv;
    b = rest / T.chunks;
    u_begin = rest % T.chunks * kFwdResUnits;
    u_end = u_begin + kFwdResUnits;  // clipped to the tile's units below
    if (b >= p.batch) return;        // padding workgroup (uniform)
  }
  // byte arrays of the parameter block through scalar loads (a vector byte load would make the wave
  // wait for every vector memory operation in flight, the previous unit's stores included)
  const int g0 = kernarg_byte(offsetof(FwdParams, kv_first) + kvh);
  const int gsz = kernarg_byte(offsetof(FwdParams, kv_first) + kvh + 1) - g0;
  if (gsz <= 0) return;
  if constexpr (!TABLE) u_end = min(u_end, (T.sq + kQW - 1) / kQW * gsz);  // units (32-row block, head)
  if (u_begin >= u_end) return;  // uniform

  const __bf16* Kg = (const __bf16*)T.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
  const __bf16* Vg = (const __bf16*)T.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh;
  const int sk = T.sk;
  const int nkb = (sk + kBN - 1) / kBN;  // at most RB: the host routes longer tiles elsewhere
  const int klast = sk - 1;
  const int kfull = sk / kBN;  // blocks with every key inside the tile
  const int k_ss = (int)p.k_ss, v_ss = (int)p.v_ss;  // below 2^24 (checked by the caller)

  // ---- every K and V block into LDS (block kb in slot kb; rows past the end repeat the last) ----
  auto load_row = [&](int i) { return ((wave * C::LPW + i) * 64 + lane) / C::CH; };
  auto load_col = [&](int i) { return ((((wave * C::LPW + i) * 64 + lane) % C::CH) ^ swz<D>(load_row(i))) * 8; };
#pragma unroll
  for (int kb = 0; kb < RB; ++kb) {
    if (kb < nkb) {
      const __bf16* kbase = Kg + (int64_t)kb * kBN * p.k_ss;
      const __bf16* vbase = Vg + (int64_t)kb * kBN * p.v_ss;
      const int valid = sk - kb * kBN;
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) {
        const int r = min(load_row(i), valid - 1);
        lds_dma16(kbase, (uint32_t)(r * k_ss + load_col(i)) * 2u, lds_addr(&kv_s[0][kb][(wave * C::LPW + i) * 512]));
        lds_dma16(vbase, (uint32_t)(r * v_ss + load_col(i)) * 2u, lds_addr(&kv_s[1][kb][(wave * C::LPW + i) * 512]));
      }
    }
  }

  // ---- units: which rows of which tile, and their query fragments ----
  struct Unit {
    const __bf16* q;
    __bf16* o;
    float* lse;
    int sq, row0, head, acc;
  };
  // unit u of the workgroup's range; false for an empty head slot (a KV head with fewer than
  // gmax query heads).  TABLE: ent only moves forward (a wave's units grow), and the entries'
  // first units grow, so the entry holding u is the last one that starts at or before it.
  auto decode = [&](int u, Unit& x) -> bool {
    if constexpr (TABLE) {
      while (ent + 1 < p.table_nents && table_load(&p.res_ents[ent + 1].unit0) <= u) ++ent;
      const FwdResEnt en = table_load(p.res_ents + ent);
      const int lu = u - en.unit0;
      const int hs = lu % p.gmax;
      if (hs >= gsz) return false;
      const FwdTile* X = p.table + en.tile;
      x.q = (const __bf16*)table_load(&X->q);
      x.o = (__bf16*)table_load(&X->o);
      x.lse = table_load(&X->lse);
      x.sq = table_load(&X->sq);
      x.acc = table_load(&X->accumulate) & 1;
      x.row0 = lu / p.gmax * kQW;
      x.head = kernarg_byte(offsetof(FwdParams, heads_of) + g0 + hs);
    } else {
      x.q = (const __bf16*)T.q;
      x.o = (__bf16*)T.o;
      x.lse = T.lse;
      x.sq = T.sq;
      x.acc = T.accumulate & 1;
      x.row0 = u / gsz * kQW;
      x.head = kernarg_byte(offsetof(FwdParams, heads_of) + g0 + u % gsz);
    }
    return true;
  };
  // the first unit at or after u, in steps of kWaves, that has rows (u_end: none)
  auto seek = [&](int u, Unit& x) {
    while (u < u_end && !decode(u, x)) u += kWaves;
    return u;
  };
  // A lane whose row is past the tile's end takes the last row: it computes that row's result
  // bit for bit (its scores, max and sums are the same, and the wave's rescale decisions, taken
  // over all lanes, do not change) and stores the same values to the same place.  So no load or
  // store of a unit sits under a branch: a branch would make the wait for the next unit's query
  // fragments also wait for this unit's stores (the wait counter is merged over both paths).
  auto unit_row = [&](const Unit& x) { return min(x.row0 + l32, x.sq - 1); };
  auto load_q = [&](const Unit& x, bf16x8 (&f)[C::KS]) {
    const __bf16* Qg = x.q + (int64_t)b * p.q_sb + (int64_t)x.head * p.q_sh + (int64_t)unit_row(x) * p.q_ss;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) f[ks] = *gmem((const bf16x8*)(Qg + ks * 16 + hl * 8));
  };
  Unit cur;
  int u = seek(u_begin + wave, cur);
  bf16x8 qf[C::KS];
  if (u < u_end) load_q(cur, qf);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the blocks and the first fragments
  __syncthreads();
  if (u >= u_end) return;  // no unit for this wave

  uint32_t kaddr[C::KS], kaddr_tr_unused[C::NC][2], vaddr_b128_unused[C::KS], vaddr[C::NC][2];
  tile_lane_addrs<D>(kv_s[0][0], lane, kaddr, kaddr_tr_unused);
  tile_lane_addrs<D>(kv_s[1][0], lane, vaddr_b128_unused, vaddr);
  constexpr uint32_t kBlockBytes = C::BLK * 2;
  const float c2 = p.scale_log2;

  f32x16 oacc[C::NC];
  float m2, lsum, mb2;  // running max (log2 units), the lane's share of the row sum, a half's max
  // S^T of 32-key half kb2 of block kb
  auto s_half = [&](int kb, int kb2, f32x16& s) { fwd_scores(kaddr, kb * kBlockBytes + kb2 * 32 * D * 2, qf, s); };
  // mask (keys past the last one) and row max of a half
  auto half_max = [&](int kb, int kb2, f32x16& s, auto may_mask) {
    if constexpr (decltype(may_mask)::value) {
      if (kb >= kfull) fwd_mask_keys(s, kb * kBN + kb2 * 32, hl, klast);
    }
    mb2 = fwd_row_max(s, c2);
  };
  auto maybe_rescale = [&]() { fwd_maybe_rescale(oacc, m2, lsum, mb2); };
  auto has_keys = [&](int kb, int kb2) { return kb * kBN + kb2 * 32 < sk; };
  // One step over half kb2 of block kb, whose scores are in sc and whose max is already folded
  // into m2: the exponentials while the score MFMAs of the next half (block nkb_, half nkb2) run,
  // then the half's PV MFMAs and the next half's mask and max.  A half with no key of the tile is
  // only ever the last one (its step does nothing, and no scores follow it).
  auto half_step = [&](auto may_mask, int kb, int kb2, f32x16& sc, int nkb_, int nkb2, f32x16& sn) {
    const bool nxt = has_keys(nkb_, nkb2);
    if (!has_keys(kb, kb2)) {
      mb2 = -INFINITY;
      return;
    }
    // as in the ring kernel's step, with many units per workgroup (the table instance: measured
    // 1.3% faster; with the few units of a kernel-argument workgroup 5% slower, so not there)
    if constexpr (TABLE) __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_iglp_opt(0);
    bf16x8 pf[2];
    fwd_probs(sc, c2, m2, lsum, pf);
    if (nxt) s_half(nkb_, nkb2, sn);
    fwd_pv<D>(vaddr, kb * kBlockBytes + kb2 * 32 * D * 2, pf, oacc);
    if constexpr (TABLE) __builtin_amdgcn_s_setprio(0);
    if (nxt) half_max(nkb_, nkb2, sn, may_mask);
    else mb2 = -INFINITY;
  };
  // The first half's max becomes the running max directly: with no sums yet there is nothing to
  // rescale, and the lazy rescale from -inf would set the same value.
  auto run_unit = [&](auto may_mask) {
#pragma unroll
    for (int c = 0; c < C::NC; ++c) oacc[c] = f32x16{};
    lsum = 0.f;
    f32x16 sA, sB;
    s_half(0, 0, sA);
    half_max(0, 0, sA, may_mask);
    m2 = mb2;
    for (int j = 0; j < nkb; ++j) {
      half_step(may_mask, j, 0, sA, j, 1, sB);
      maybe_rescale();
      half_step(may_mask, j, 1, sB, j + 1, 0, sA);
      maybe_rescale();
    }
  };

  // ---- the wave's units: u_begin + wave + 8 i ----
  for (;;) {
    Unit nxt;
    const int un = seek(u + kWaves, nxt);
    bf16x8 qn[C::KS];
    if (un < u_end) load_q(nxt, qn);  // in flight under this unit's blocks
    if (sk % kBN != 0) run_unit(std::true_type{});  // the last block is ragged
    else run_unit(std::false_type{});
    const float ltot = xhalf_sum(lsum);
    const int row = unit_row(cur);
    __bf16* orow = cur.o + (int64_t)b * p.o_sb + (int64_t)cur.head * p.o_sh + (int64_t)row * p.o_ss;
    float* lrow = cur.lse + (int64_t)b * p.l_sb + (int64_t)cur.head * p.l_sh + row;
    fwd_store_rows(oacc, m2, ltot, cur.acc, orow, lrow, hl);
    u = un;
    if (u >= u_end) break;
    cur = nxt;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = qn[ks];
  }
}

template <int WAVES>
void launch_waves(const FwdParams& p, int head_dim, dim3 grid, hipStream_t s) {
  const dim3 block(WAVES * 64);
  if (head_dim == 128) {
    if (p.mask) hipLaunchKernelGGL((fwd_bf16_kernel<128, true, WAVES>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fwd_bf16_kernel<128, false, WAVES>), grid, block, 0, s, p);
  } else {
    if (p.mask) hipLaunchKernelGGL((fwd_bf16_kernel<64, true, WAVES>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fwd_bf16_kernel<64, false, WAVES>), grid, block, 0, s, p);
  }
}

}  // namespace

int launch_fwd_bf16_resident(const FwdParams& p, int head_dim, int total_wgs, void* stream) {
  if (total_wgs <= 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid(total_wgs), block(512);
  if (p.table) {
    if (head_dim == 128) hipLaunchKernelGGL((fwd_bf16_resident_kernel<128, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fwd_bf16_resident_kernel<64, true>), grid, block, 0, s, p);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((fwd_bf16_resident_kernel<128, false>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fwd_bf16_resident_kernel<64, false>), grid, block, 0, s, p);
  }
  return (int)hipGetLastError();
}

int launch_fwd_bf16(const FwdParams& p, int head_dim, int waves, int total_wgs, void* stream) {
  if (total_wgs <= 0) return 0;
  if (waves != 4 && waves != 8) return (int)hipErrorInvalidValue;
  const dim3 grid(total_wgs);
  hipStream_t s = (hipStream_t)stream;
  if (waves == 8) launch_waves<8>(p, head_dim, grid, s);
  else launch_waves<4>(p, head_dim, grid, s);
  return (int)hipGetLastError();
}

}  // namespace ma
