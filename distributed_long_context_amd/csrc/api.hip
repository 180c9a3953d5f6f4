// C ABI of the tile library: argument validation, kernel-parameter packing and
// launches on the caller's stream.  No device allocation, no synchronisation,
// no state kept between calls (the error message is thread-local).
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>
#include <algorithm>

#include "mesh_attn.h"
#include "ma_internal.h"

namespace ma {

static thread_local std::string g_last_error;

int set_error(int code, const char* msg) {
  g_last_error = msg ? msg : "";
  return code;
}

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_hip(int e, const char* what) {
  if (e != 0) {
    std::string m = std::string(what) + ": " + hipGetErrorString((hipError_t)e);
    return set_error(MA_ERR_LAUNCH, m.c_str());
  }
  return MA_OK;
}

// Query heads grouped by KV head: heads_of lists query heads ordered by their KV
// head; kv_first[x] .. kv_first[x+1] is KV head x's run.  Returns the largest group.
int build_head_groups(int hq, int hkv, const int32_t* head_map, uint8_t* heads_of, uint8_t* kv_first,
                      const char** why) {
  std::vector<int> kv(hq);
  for (int h = 0; h < hq; ++h) {
    kv[h] = head_map ? head_map[h] : h / (hq / hkv);
    if (kv[h] < 0 || kv[h] >= hkv) {
      *why = "head_map entry out of range";
      return -1;
    }
  }
  int n = 0, gmax = 0;
  for (int x = 0; x < hkv; ++x) {
    kv_first[x] = (uint8_t)n;
    int g = 0;
    for (int h = 0; h < hq; ++h)
      if (kv[h] == x) {
        heads_of[n++] = (uint8_t)h;
        ++g;
      }
    gmax = std::max(gmax, g);
  }
  kv_first[hkv] = (uint8_t)n;
  return gmax;
}

bool to_kpos(const ma_pos& in, KPos& out) {
  std::memset(&out, 0, sizeof(out));
  out.nseg = in.nseg;
  for (int s = 0; s < in.nseg; ++s) {
    out.lb[s] = (int32_t)in.seg[s].local_begin;
    out.gb[s] = (int32_t)in.seg[s].global_begin;
    out.st[s] = (int32_t)in.seg[s].stride;
  }
  return true;
}

int check_positions(int mask_mode, const ma_pos& qp, int64_t sq, const ma_pos& kp, int64_t sk) {
  if (mask_mode == MA_MASK_NONE) return MA_OK;
  const char* why = nullptr;
  if (!pos_valid(&qp, sq, &why) || !pos_valid(&kp, sk, &why)) return set_error(MA_ERR_INVALID, why);
  if (mask_mode == MA_MASK_CAUSAL &&
      (qp.nseg != 1 || kp.nseg != 1 || qp.seg[0].stride != 1 || kp.seg[0].stride != 1))
    return set_error(MA_ERR_INVALID, "MA_MASK_CAUSAL takes one stride-1 segment per partition; "
                                     "use MA_MASK_STRIPED_ZIGZAG for zigzag or striped layouts");
  return MA_OK;
}

int check_common(int dtype, int batch, int hq, int hkv, int head_dim, int mask_mode, float scale) {
  if (dtype != MA_F32 && dtype != MA_BF16) return set_error(MA_ERR_INVALID, "dtype must be MA_F32 or MA_BF16");
  if (head_dim != 64 && head_dim != 128) return set_error(MA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (batch < 1 || hq < 1 || hq > MA_MAX_HEADS || hkv < 1 || hkv > hq)
    return set_error(MA_ERR_INVALID, "need batch >= 1, 1 <= hkv <= hq <= MA_MAX_HEADS");
  if (mask_mode != MA_MASK_NONE && mask_mode != MA_MASK_CAUSAL && mask_mode != MA_MASK_STRIPED_ZIGZAG)
    return set_error(MA_ERR_INVALID, "unknown mask mode");
  if (!std::isfinite(scale) || scale <= 0.f) return set_error(MA_ERR_INVALID, "scale must be finite and > 0");
  return MA_OK;
}

bool strides_ok(const int64_t* s, int n, int dtype) {
  const int64_t q = dtype == MA_BF16 ? 8 : 4;
  for (int i = 0; i < n; ++i)
    if (s[i] < 0 || s[i] % q) return false;
  return true;
}

}  // namespace
}  // namespace ma

using namespace ma;

extern "C" {

const char* mesh_attn_last_error(void) { return g_last_error.c_str(); }
int mesh_attn_version(void) { return MA_VERSION; }

int mesh_attn_tile_fwd(const ma_tile_fwd_args* a, void* stream) {
  if (!a) return set_error(MA_ERR_INVALID, "null args");
  int rc = check_common(a->dtype, a->batch, a->hq, a->hkv, a->head_dim, a->mask_mode, a->scale);
  if (rc) return rc;
  if (!a->head_map && a->hq % a->hkv) return set_error(MA_ERR_INVALID, "hq must be a multiple of hkv when head_map is NULL");
  if (a->ntiles < 0 || a->ntiles > MA_MAX_TILES) return set_error(MA_ERR_INVALID, "ntiles out of range");
  if (a->ntiles == 0) return MA_OK;
  if (!a->tiles) return set_error(MA_ERR_INVALID, "null tile list");
  if (!strides_ok(a->q_stride, 3, a->dtype) || !strides_ok(a->k_stride, 3, a->dtype) ||
      !strides_ok(a->v_stride, 3, a->dtype) || !strides_ok(a->o_stride, 3, a->dtype) || a->lse_stride[0] < 0 ||
      a->lse_stride[1] < 0)
    return set_error(MA_ERR_INVALID, "strides must be >= 0 and multiples of 16 bytes");

  FwdParams p;
  std::memset(&p, 0, sizeof(p));
  const char* why = nullptr;
  p.gmax = build_head_groups(a->hq, a->hkv, a->head_map, p.heads_of, p.kv_first, &why);
  if (p.gmax < 0) return set_error(MA_ERR_INVALID, why);
  p.batch = a->batch;
  p.hq = a->hq;
  p.hkv = a->hkv;
  p.mask = a->mask_mode != MA_MASK_NONE;
  p.scale = a->scale;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  p.q_sb = a->q_stride[0]; p.q_ss = a->q_stride[1]; p.q_sh = a->q_stride[2];
  p.k_sb = a->k_stride[0]; p.k_ss = a->k_stride[1]; p.k_sh = a->k_stride[2];
  p.v_sb = a->v_stride[0]; p.v_ss = a->v_stride[1]; p.v_sh = a->v_stride[2];
  p.o_sb = a->o_stride[0]; p.o_ss = a->o_stride[1]; p.o_sh = a->o_stride[2];
  p.l_sb = a->lse_stride[0]; p.l_sh = a->lse_stride[1];

  // validate every tile before enqueueing anything
  for (int i = 0; i < a->ntiles; ++i) {
    const ma_tile& t = a->tiles[i];
    if (!t.q || !t.k || !t.v || !t.o || !t.lse) return set_error(MA_ERR_INVALID, "null tensor pointer in a tile");
    if (!aligned16(t.q) || !aligned16(t.k) || !aligned16(t.v) || !aligned16(t.o) || ((uintptr_t)t.lse & 3u))
      return set_error(MA_ERR_INVALID, "tensor pointers must be 16-byte aligned (lse 4-byte)");
    if (t.sq < 1 || t.sk < 1 || t.sq >= INT32_MAX || t.sk >= INT32_MAX)
      return set_error(MA_ERR_INVALID, "tile sizes must be in [1, 2^31-1)");
    rc = check_positions(a->mask_mode, t.q_pos, t.sq, t.k_pos, t.sk);
    if (rc) return rc;
  }

  const bool bf16 = a->dtype == MA_BF16;
  int n = 0, wg = 0;
  auto flush = [&]() -> int {
    if (n == 0) return MA_OK;
    p.ntiles = n;
    int e = bf16 ? launch_fwd_bf16(p, a->head_dim, wg, stream) : launch_fwd_f32(p, a->head_dim, wg, stream);
    n = 0;
    wg = 0;
    return check_hip(e, "tile_fwd launch");
  };
  for (int i = 0; i < a->ntiles; ++i) {
    const ma_tile& t = a->tiles[i];
    if (a->mask_mode != MA_MASK_NONE &&
        mesh_attn_classify(&t.q_pos, t.sq, &t.k_pos, t.sk, a->mask_mode) == MA_TILE_EMPTY) {
      int e = launch_fill_empty(t.o, t.lse, a->dtype, a->batch, (int)t.sq, a->hq, a->head_dim, p.o_sb, p.o_ss,
                                p.o_sh, p.l_sb, p.l_sh, stream);
      rc = check_hip(e, "fill launch");
      if (rc) return rc;
      continue;
    }
    FwdTile& ft = p.tiles[n];
    ft.q = t.q; ft.k = t.k; ft.v = t.v; ft.o = t.o; ft.lse = t.lse;
    ft.sq = (int32_t)t.sq;
    ft.sk = (int32_t)t.sk;
    if (a->mask_mode != MA_MASK_NONE) {
      to_kpos(t.q_pos, ft.qp);
      to_kpos(t.k_pos, ft.kp);
    } else {
      ft.qp.nseg = ft.kp.nseg = 1;
    }
    int64_t wgs;
    if (bf16) {
      const int64_t nqb = (t.sq + 63) / 64;
      ft.chunks = (int32_t)((nqb * p.gmax + 3) / 4);
      wgs = (int64_t)a->batch * a->hkv * ft.chunks;
      wgs = (wgs + 7) / 8 * 8;  // keep each tile's first workgroup on XCD 0
    } else {
      ft.chunks = (int32_t)((t.sq + 63) / 64);
      wgs = (int64_t)a->batch * a->hq * ft.chunks;
    }
    if (wgs + wg >= INT32_MAX) return set_error(MA_ERR_INVALID, "tile too large for one launch");
    ft.wg_begin = wg;
    wg += (int)wgs;
    ++n;
    if (n == kFwdTilesPerLaunch) {
      rc = flush();
      if (rc) return rc;
    }
  }
  return flush();
}

int mesh_attn_merge(const ma_merge_args* a, void* stream) {
  if (!a) return set_error(MA_ERR_INVALID, "null args");
  if (a->dtype != MA_F32 && a->dtype != MA_BF16) return set_error(MA_ERR_INVALID, "dtype must be MA_F32 or MA_BF16");
  if (a->head_dim != 64 && a->head_dim != 128) return set_error(MA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (a->k < 1 || a->k > MA_MAX_MERGE) return set_error(MA_ERR_INVALID, "k must be in 1..MA_MAX_MERGE");
  if (a->batch < 1 || a->seqlen < 1 || a->heads < 1) return set_error(MA_ERR_INVALID, "batch, seqlen, heads must be >= 1");
  if (!a->o_in || !a->lse_in || !a->o_out || !a->lse_out) return set_error(MA_ERR_INVALID, "null pointer");
  if (!strides_ok(a->o_stride, 3, a->dtype) || a->lse_stride[0] < 0 || a->lse_stride[1] < 0)
    return set_error(MA_ERR_INVALID, "strides must be >= 0 and multiples of 16 bytes");
  if (!aligned16(a->o_out) || ((uintptr_t)a->lse_out & 3u)) return set_error(MA_ERR_INVALID, "misaligned output");
  MergeParams p;
  std::memset(&p, 0, sizeof(p));
  for (int i = 0; i < a->k; ++i) {
    if (!a->o_in[i] || !a->lse_in[i]) return set_error(MA_ERR_INVALID, "null partial pointer");
    if (!aligned16(a->o_in[i]) || ((uintptr_t)a->lse_in[i] & 3u)) return set_error(MA_ERR_INVALID, "misaligned partial");
    p.o_in[i] = a->o_in[i];
    p.lse_in[i] = a->lse_in[i];
  }
  p.k = a->k;
  p.batch = a->batch;
  p.seqlen = a->seqlen;
  p.heads = a->heads;
  p.o_sb = a->o_stride[0]; p.o_ss = a->o_stride[1]; p.o_sh = a->o_stride[2];
  p.l_sb = a->lse_stride[0]; p.l_sh = a->lse_stride[1];
  p.o_out = a->o_out;
  p.lse_out = a->lse_out;
  return check_hip(launch_merge(p, a->dtype, a->head_dim, stream), "merge launch");
}

size_t mesh_attn_tile_bwd_workspace_size(const ma_tile_bwd_args* a) {
  if (!a || a->ntiles < 0 || (a->ntiles > 0 && !a->tiles) || a->batch < 1 || a->hq < 1) return 0;
  size_t bytes = 0;
  for (int i = 0; i < a->ntiles; ++i) {
    const int64_t sq = a->tiles[i].sq < 0 ? 0 : a->tiles[i].sq;
    bytes += ((size_t)a->batch * a->hq * sq * sizeof(float) + 255) / 256 * 256;
  }
  return bytes;
}

int mesh_attn_tile_bwd(const ma_tile_bwd_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace; (void)workspace_bytes; (void)stream;
  if (!a) return set_error(MA_ERR_INVALID, "null args");
  return set_error(MA_ERR_UNSUPPORTED, "tile_bwd: not built yet");
}

}  // extern "C"
