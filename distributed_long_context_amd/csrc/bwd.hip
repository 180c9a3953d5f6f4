// Tile backward (dQ, dK, dV), bf16 inputs, fp32 accumulation, for CDNA4 (gfx950).
//
// [Mesh] section 3.5: the backward kernel is called per (Q_i, KV_j) pair with
// (Q_i, KV_j, O_i, dO_i) and the partial dQ_i and dKV_j are accumulated
// locally, addition being the reducer.  The pages print no formula; the kernel
// evaluates the derivative of the forward definition with P = exp(s - LSE):
//   D[t] = dO[t].O[t];  dP = dO V^T;  dS = P (dP - D);
//   dV = P^T dO;  dK = scale dS^T Q;  dQ = scale dS K.
//
// Layout on the chip (this file's own design):
//  * Preprocessing: one pass over O and dO writes D per row to the workspace
//    and clears dQ when the call overwrites.
//  * Main kernel, KV-stationary: a workgroup owns 128 keys of one KV head
//    (32 per wave) and loops over every tile that reads this KV partition, every
//    query head of the group and every 64-row query block.  K and V fragments
//    and the dK, dV accumulators stay in registers for the whole loop, so dK/dV
//    are written once, without atomics.
//  * S = Q K^T and dP = dO V^T run on v_mfma_f32_32x32x16_bf16 with one key per
//    lane; query rows are fed in a permuted order (bits 2 and 3 of the row index
//    swapped) so that each lane's accumulator values are, unchanged, the A
//    operand (P^T, dS^T) of the dV and dK products.  dO and Q reach those
//    products through transposed LDS reads (ds_read_b64_tr_b16).
//  * dS is written to LDS as [key][query] and read back transposed as the A
//    operand of dQ = dS K; each wave covers one 32-column slice of d for the
//    whole workgroup's 128 keys and adds it to dQ with fp32 atomics.
//  * Query blocks with no allowed pair against the workgroup's keys are skipped;
//    fully allowed blocks run unmasked ([Mesh] section 3.7 pair classes).
#include <hip/hip_runtime.h>
#include <cstdint>

#include "ma_internal.h"
#include "ma_device.h"

namespace ma {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = 64;    // query rows per item
constexpr int kBN = 128;   // keys per workgroup (32 per wave)

template <int D>
struct BwdCfg {
  static constexpr int QROW = D + 8;           // Q / dO row pitch in LDS (elements)
  static constexpr int SROW = kBM + 8;         // dS^T row pitch (keys x queries)
  static constexpr int KROW = D + 8;           // K / V staging pitch
  static constexpr int KS = D / 16;            // k-steps over d
  static constexpr int NC = D / 32;            // 32-wide d chunks
  static constexpr int CH = D / 8;             // 16-byte chunks per row
  static constexpr int QLOADS = kBM * CH / kThreads;  // per tensor per thread
  static constexpr int Q_ELEMS = kBM * QROW;
  static constexpr int S_ELEMS = kBN * SROW;
  static constexpr int KV_ELEMS = kBN * KROW;
  // dQ work per wave: (query sub-block, d chunk) units
  static constexpr int DQ_UNITS = 2 * NC / kWaves;  // 2 (D=128) or 1 (D=64)
};

__device__ __forceinline__ int perm_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// ---------------------------------------------------------------- preprocess --
// D[b,h,t] = sum_c dO*O for every row of every tile; clear dQ when overwriting.
template <int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(const BwdParams p, int tile, int zero_dq) {
  constexpr int TPR = D / 8;  // threads per row
  const BwdTile& T = p.tiles[tile];
  const int64_t rows = (int64_t)p.batch * T.sq * p.hq;
  const int64_t r = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int c = (threadIdx.x % TPR) * 8;
  float acc = 0.f;
  int h = 0;
  int64_t t = 0, b = 0;
  if (r < rows) {
    h = (int)(r % p.hq);
    t = (r / p.hq) % T.sq;
    b = r / ((int64_t)p.hq * T.sq);
    const int64_t off = b * p.q_sb + t * p.q_ss + h * p.q_sh + c;
    const uint4 o = *(const uint4*)((const __bf16*)T.o + off);
    const uint4 g = *(const uint4*)((const __bf16*)T.dout + off);
    const uint32_t ow[4] = {o.x, o.y, o.z, o.w}, gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += __uint_as_float(ow[i] << 16) * __uint_as_float(gw[i] << 16);
      acc += __uint_as_float(ow[i] & 0xffff0000u) * __uint_as_float(gw[i] & 0xffff0000u);
    }
    if (zero_dq) {
      float* dq = T.dq + b * p.dq_sb + t * p.dq_ss + h * p.dq_sh + c;
      *(float4*)dq = make_float4(0.f, 0.f, 0.f, 0.f);
      *(float4*)(dq + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int s = TPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s);
  if (r < rows && (threadIdx.x % TPR) == 0) T.dscratch[(b * p.hq + h) * (int64_t)T.sq + t] = acc;
}

// ---------------------------------------------------------------- main kernel --
template <int D>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_main_kernel(const BwdParams p) {
  using C = BwdCfg<D>;
  // Q/dO double buffers; the first part doubles as K/V staging at start-up.
  constexpr int QDO_BYTES = 4 * C::Q_ELEMS * 2;
  constexpr int KV_BYTES = 2 * C::KV_ELEMS * 2;
  constexpr int RAW = QDO_BYTES > KV_BYTES ? QDO_BYTES : KV_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char raw[RAW];
  __shared__ __attribute__((aligned(16))) __bf16 dS_s[2][C::S_ELEMS];
  __shared__ __attribute__((aligned(16))) float lse2_s[2][kBM];
  __shared__ __attribute__((aligned(16))) float dd_s[2][kBM];
  __shared__ __attribute__((aligned(16))) int qpos_s[2][kBM];
  __bf16* const qdo = (__bf16*)raw;  // Q buffers at [0, 2*Q_ELEMS), dO buffers after them

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int G = lane >> 4, lam = lane & 15;

  // ---- workgroup -> (KV group, batch, KV head, key block) ----
  const int w = blockIdx.x;
  int gi = 0;
  while (gi + 1 < p.nkv && w >= p.kvs[gi + 1].wg_begin) ++gi;
  const BwdKV& KV = p.kvs[gi];
  const int nkb = (KV.sk + kBN - 1) / kBN;
  const int local = w - KV.wg_begin;
  const int kvh = local % p.hkv;
  const int rest = local / p.hkv;
  const int kblk = rest % nkb;
  const int b = rest / nkb;
  if (b >= p.batch) return;  // padding workgroup (uniform)
  const int g0 = p.kv_first[kvh];
  const int gsz = p.kv_first[kvh + 1] - g0;

  const int key0 = kblk * kBN;
  const int keys_here = min(kBN, KV.sk - key0);
  int kmin = 0, kmax = 0;
  if (p.mask) pos_minmax_dev(KV.kp, KV.sk, key0, key0 + keys_here, kmin, kmax);
  const int my_key = key0 + wave * 32 + l32;
  const int my_kpos = my_key >= KV.sk ? INT32_MAX : (p.mask ? pos_at_dev(KV.kp, my_key) : INT32_MIN);

  // ---- stage K and V of the 128 keys, load the stationary fragments ----
  {
    __bf16* Kst = (__bf16*)raw;
    __bf16* Vst = (__bf16*)raw + C::KV_ELEMS;
    const __bf16* Kg = (const __bf16*)KV.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
    const __bf16* Vg = (const __bf16*)KV.v + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
    for (int c = tid; c < kBN * C::CH; c += kThreads) {
      const int row = c / C::CH, col = (c % C::CH) * 8;
      const int key = key0 + row;
      uint4 kx = make_uint4(0, 0, 0, 0), vx = kx;
      if (key < KV.sk) {
        kx = *(const uint4*)(Kg + (int64_t)key * p.k_ss + col);
        vx = *(const uint4*)(Vg + (int64_t)key * p.k_ss + col);
      }
      *(uint4*)(Kst + row * C::KROW + col) = kx;
      *(uint4*)(Vst + row * C::KROW + col) = vx;
    }
  }
  __syncthreads();
  bf16x8 kf[C::KS], vf[C::KS];  // B operands of S = Q K^T and dP = dO V^T (this wave's 32 keys)
  bf16x8 ktf[8];                // B operands of dQ = dS K (all 128 keys, this wave's d chunk)
  // dQ work of this wave: d chunk dq_c for query sub-blocks dq_qs0 + u*(waves/NC)
  const int dq_c = wave % C::NC;
  const int dq_qs0 = wave / C::NC;
  {
    const __bf16* Kst = (const __bf16*)raw;
    const __bf16* Vst = (const __bf16*)raw + C::KV_ELEMS;
    const int krow = wave * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      kf[ks] = *(const bf16x8*)(Kst + krow * C::KROW + ks * 16 + hl * 8);
      vf[ks] = *(const bf16x8*)(Vst + krow * C::KROW + ks * 16 + hl * 8);
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int row = kk * 16 + (G >> 1) * 8 + (lam >> 2);
      const int col = dq_c * 32 + (G & 1) * 16 + (lam & 3) * 4;
      ktf[kk] = concat_bf16x4(ds_read_tr16(Kst + row * C::KROW + col), ds_read_tr16(Kst + (row + 4) * C::KROW + col));
    }
  }
  __syncthreads();  // staging area becomes the Q/dO buffers

  // ---- work items: (tile in this KV group, query head of the group, query block) ----
  // flat item index: ti-major, then head, then query block
  auto decode = [&](int it, int& ti, int& hi, int& qb) {
    ti = 0;
    int base = 0;
    for (;;) {
      const BwdTile& T = p.tiles[KV.tile_idx[ti]];
      const int nqb = (T.sq + kBM - 1) / kBM;
      const int n = nqb * gsz;
      if (it < base + n || ti + 1 == KV.ntiles) {
        const int r = it - base;
        hi = r / nqb;
        qb = r % nqb;
        return;
      }
      base += n;
      ++ti;
    }
  };
  int nitems = 0;
  for (int i = 0; i < KV.ntiles; ++i) nitems += ((p.tiles[KV.tile_idx[i]].sq + kBM - 1) / kBM) * gsz;
  auto cls_of = [&](int it) -> int {
    int ti, hi, qb;
    decode(it, ti, hi, qb);
    const BwdTile& T = p.tiles[KV.tile_idx[ti]];
    const int r0 = qb * kBM, r1 = min(T.sq, r0 + kBM);
    const bool tail = keys_here < kBN || (r1 - r0) < kBM;
    if (!p.mask) return tail ? 1 : 2;
    int qmin, qmax;
    pos_minmax_dev(T.qp, T.sq, r0, r1, qmin, qmax);
    if (kmin > qmax) return 0;
    if (kmax <= qmin && !tail) return 2;
    return 1;
  };
  auto next_item = [&](int from) -> int {
    for (int it = from; it < nitems; ++it)
      if (cls_of(it) != 0) return it;
    return nitems;
  };

  uint4 qreg[C::QLOADS], goreg[C::QLOADS];
  float lse_r = 0.f, dd_r = 0.f;
  int qp_r = 0;
  auto gload = [&](int it) {
    int ti, hi, qb;
    decode(it, ti, hi, qb);
    const BwdTile& T = p.tiles[KV.tile_idx[ti]];
    const int h = p.heads_of[g0 + hi];
    const int r0 = qb * kBM;
    const __bf16* Qg = (const __bf16*)T.q + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh;
    const __bf16* Gg = (const __bf16*)T.dout + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh;
#pragma unroll
    for (int i = 0; i < C::QLOADS; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / C::CH, col = (c % C::CH) * 8;
      const int t = r0 + row;
      if (t < T.sq) {
        qreg[i] = *(const uint4*)(Qg + (int64_t)t * p.q_ss + col);
        goreg[i] = *(const uint4*)(Gg + (int64_t)t * p.q_ss + col);
      } else {
        qreg[i] = make_uint4(0, 0, 0, 0);
        goreg[i] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < kBM) {
      const int t = r0 + tid;
      if (t < T.sq) {
        const float L = T.lse[(int64_t)b * p.l_sb + (int64_t)h * p.l_sh + t];
        lse_r = (L == -INFINITY) ? INFINITY : L * 1.4426950408889634f;  // +inf makes P = 0 on empty rows
        dd_r = T.dscratch[((int64_t)b * p.hq + h) * T.sq + t];
        qp_r = p.mask ? pos_at_dev(T.qp, t) : 0;
      } else {
        lse_r = INFINITY;
        dd_r = 0.f;
        qp_r = INT32_MIN;
      }
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::QLOADS; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / C::CH, col = (c % C::CH) * 8;
      *(uint4*)(qdo + buf * C::Q_ELEMS + row * C::QROW + col) = qreg[i];
      *(uint4*)(qdo + (2 + buf) * C::Q_ELEMS + row * C::QROW + col) = goreg[i];
    }
    if (tid < kBM) {
      lse2_s[buf][tid] = lse_r;
      dd_s[buf][tid] = dd_r;
      qpos_s[buf][tid] = qp_r;
    }
  };

  f32x16 dk_acc[C::NC], dv_acc[C::NC];
#pragma unroll
  for (int c = 0; c < C::NC; ++c) {
    dk_acc[c] = f32x16{};
    dv_acc[c] = f32x16{};
  }
  const float c2 = p.scale_log2;

  int it = next_item(0);
  int buf = 0;
  if (it < nitems) {
    gload(it);
    swrite(0);
  }
  __syncthreads();
  int it_next = (it < nitems) ? next_item(it + 1) : nitems;
  if (it_next < nitems) gload(it_next);

  while (it < nitems) {
    const int cls = cls_of(it);
    const __bf16* Ql = qdo + buf * C::Q_ELEMS;
    const __bf16* Gl = qdo + (2 + buf) * C::Q_ELEMS;
    // S = Q K^T and dP = dO V^T for two 32-row query sub-blocks (one key per lane)
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      s[qs] = f32x16{};
      dp[qs] = f32x16{};
      const int qrow = qs * 32 + perm_row(l32);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 qa = *(const bf16x8*)(Ql + qrow * C::QROW + ks * 16 + hl * 8);
        const bf16x8 ga = *(const bf16x8*)(Gl + qrow * C::QROW + ks * 16 + hl * 8);
        s[qs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], s[qs], 0, 0, 0);
        dp[qs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vf[ks], dp[qs], 0, 0, 0);
      }
    }
    // P and dS; element e of lane half hl is query qs*32 + 16*(e/8) + 8*hl + e%8
    bf16x8 pf[4], dsf[4];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int q0 = qs * 32 + half * 16 + hl * 8;
        const f32x4 l0 = *(const f32x4*)(&lse2_s[buf][q0]);
        const f32x4 l1 = *(const f32x4*)(&lse2_s[buf][q0 + 4]);
        const f32x4 d0 = *(const f32x4*)(&dd_s[buf][q0]);
        const f32x4 d1 = *(const f32x4*)(&dd_s[buf][q0 + 4]);
        const float lv[8] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
        const float dv8[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
        float pv[8], sv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int e = half * 8 + i;
          float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qs][e], c2, -lv[i]));
          if (cls == 1) {
            if (!(my_kpos <= qpos_s[buf][q0 + i])) pe = 0.f;
          }
          pv[i] = pe;
          sv[i] = pe * (dp[qs][e] - dv8[i]);
        }
        pf[qs * 2 + half] = pack_bf16x8(pv);
        dsf[qs * 2 + half] = pack_bf16x8(sv);
      }
    }
    // dV += P^T dO and dK += dS^T Q (B operands read transposed from LDS)
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = j * 16 + (G >> 1) * 8 + (lam >> 2);
        const int col = c * 32 + (G & 1) * 16 + (lam & 3) * 4;
        const bf16x8 gt = concat_bf16x4(ds_read_tr16(Gl + row * C::QROW + col), ds_read_tr16(Gl + (row + 4) * C::QROW + col));
        const bf16x8 qt = concat_bf16x4(ds_read_tr16(Ql + row * C::QROW + col), ds_read_tr16(Ql + (row + 4) * C::QROW + col));
        dv_acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[j], gt, dv_acc[c], 0, 0, 0);
        dk_acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsf[j], qt, dk_acc[c], 0, 0, 0);
      }
    }
    // dS^T to LDS: this lane's key row, 8 consecutive queries per store
    {
      __bf16* Sl = dS_s[buf] + (wave * 32 + l32) * C::SROW;
#pragma unroll
      for (int j = 0; j < 4; ++j) *(bf16x8*)(Sl + j * 16 + hl * 8) = dsf[j];
    }
    // stage the next item, then fetch the one after it
    int ti_cur, hi_cur, qb_cur;
    decode(it, ti_cur, hi_cur, qb_cur);
    const int it_after = (it_next < nitems) ? next_item(it_next + 1) : nitems;
    if (it_next < nitems) swrite(buf ^ 1);
    __syncthreads();
    if (it_after < nitems) gload(it_after);
    // dQ (this wave's units) = dS K over all 128 keys, added to global dQ
    {
      const BwdTile& T = p.tiles[KV.tile_idx[ti_cur]];
      const int h = p.heads_of[g0 + hi_cur];
      float* dQg = T.dq + (int64_t)b * p.dq_sb + (int64_t)h * p.dq_sh;
      const __bf16* Sl = dS_s[buf];
#pragma unroll
      for (int u = 0; u < C::DQ_UNITS; ++u) {
        const int qs = dq_qs0 + u * (kWaves / C::NC);
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const int row = kk * 16 + (G >> 1) * 8 + (lam >> 2);        // key
          const int col = qs * 32 + (G & 1) * 16 + (lam & 3) * 4;      // query
          const bf16x8 sa = concat_bf16x4(ds_read_tr16(Sl + row * C::SROW + col), ds_read_tr16(Sl + (row + 4) * C::SROW + col));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa, ktf[kk], acc, 0, 0, 0);
        }
        // lane holds d = 32*c + l32 for query rows (i/4)*8 + hl*4 + i%4 of the sub-block
        const int d = dq_c * 32 + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = qb_cur * kBM + qs * 32 + (i >> 2) * 8 + hl * 4 + (i & 3);
          if (t < T.sq) unsafeAtomicAdd(dQg + (int64_t)t * p.dq_ss + d, acc[i] * p.scale);
        }
      }
    }
    it = it_next;
    it_next = it_after;
    buf ^= 1;
  }

  // ---- dK (scaled) and dV: this wave's 32 keys; lane holds d = 32c + l32 ----
  float* dKg = KV.dk + (int64_t)b * p.dk_sb + (int64_t)kvh * p.dk_sh;
  float* dVg = KV.dv + (int64_t)b * p.dk_sb + (int64_t)kvh * p.dk_sh;
#pragma unroll
  for (int c = 0; c < C::NC; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + wave * 32 + (i >> 2) * 8 + hl * 4 + (i & 3);
      if (key < KV.sk) {
        const int64_t off = (int64_t)key * p.dk_ss + c * 32 + l32;
        float kv = dk_acc[c][i] * p.scale, vv = dv_acc[c][i];
        if (KV.accumulate) {
          kv += dKg[off];
          vv += dVg[off];
        }
        dKg[off] = kv;
        dVg[off] = vv;
      }
    }
}

}  // namespace

int launch_bwd_preprocess(const BwdParams& p, int head_dim, void* stream) {
  for (int t = 0; t < p.ntiles; ++t) {
    if (p.tiles[t].sq <= 0) continue;
    const int64_t rows = (int64_t)p.batch * p.tiles[t].sq * p.hq;
    const int rpb = 256 / (head_dim / 8);
    const int64_t blocks = (rows + rpb - 1) / rpb;
    const int zero = p.tiles[t].zero_dq;
    if (head_dim == 128)
      hipLaunchKernelGGL(bwd_pre_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, p, t, zero);
    else
      hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, p, t, zero);
    const int e = (int)hipGetLastError();
    if (e) return e;
  }
  return 0;
}

int launch_bwd_main(const BwdParams& p, int head_dim, int total_wgs, void* stream) {
  if (total_wgs <= 0) return 0;
  if (head_dim == 128)
    hipLaunchKernelGGL(bwd_main_kernel<128>, dim3(total_wgs), dim3(kThreads), 0, (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL(bwd_main_kernel<64>, dim3(total_wgs), dim3(kThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

}  // namespace ma
