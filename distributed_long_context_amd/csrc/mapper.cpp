// Host-only partition and position mapper of the C ABI.
//
// Closed-form counterpart of the assignment-matrix model in [Mesh] sections
// 3.1-3.3 (basic 2-D tiling, KV partition rotation, Q and KV groups), the
// zigzag and striped token layouts of [Ring] "Causal masks and load balancing"
// and [Mesh] section 3.7, and the tile classes of [Mesh] section 3.7.  No
// device work, no allocation.
//
// [Mesh] = "Mesh-Attention: A New Communication-Efficient Distributed Attention
//           with Improved Data Locality"
// [Ring] = "Ring Attention and Context Parallelism: How Long-Context LLMs Are
//           Trained Across GPUs"
#include <cstdint>
#include <cstring>
#include <algorithm>

#include "mesh_attn.h"
#include "ma_internal.h"

namespace ma {

bool pos_valid(const ma_pos* p, int64_t len, const char** why) {
  if (!p) { *why = "null position descriptor"; return false; }
  if (p->nseg < 1 || p->nseg > MA_MAX_SEGMENTS) { *why = "nseg must be in 1..4"; return false; }
  if (p->seg[0].local_begin != 0) { *why = "first segment must start at local index 0"; return false; }
  for (int s = 0; s < p->nseg; ++s) {
    const ma_segment& g = p->seg[s];
    int64_t end = (s + 1 < p->nseg) ? p->seg[s + 1].local_begin : len;
    if (g.stride < 1) { *why = "segment stride must be >= 1"; return false; }
    if (g.global_begin < 0) { *why = "global positions must be >= 0"; return false; }
    if (end <= g.local_begin && s + 1 < p->nseg) { *why = "segment local_begin must increase"; return false; }
    if (g.local_begin >= len) {
      *why = "segment starts beyond the partition length";
      return false;
    }
    // last position of this segment must fit in int32 (kernels use 32-bit positions)
    int64_t n = end - g.local_begin;
    if (n > 0) {
      if (g.stride > (INT32_MAX - 1) / std::max<int64_t>(1, n)) { *why = "positions exceed 2^31-1"; return false; }
      int64_t last = g.global_begin + (n - 1) * g.stride;
      if (last >= (int64_t)INT32_MAX) { *why = "positions exceed 2^31-1"; return false; }
    }
  }
  return true;
}

int64_t pos_at(const ma_pos* p, int64_t t) {
  int s = p->nseg - 1;
  while (s > 0 && p->seg[s].local_begin > t) --s;
  return p->seg[s].global_begin + (t - p->seg[s].local_begin) * p->seg[s].stride;
}

// min and max global position over local indices [u0, u1) (non-empty range)
void pos_minmax(const ma_pos* p, int64_t len, int64_t u0, int64_t u1, int64_t* mn, int64_t* mx) {
  int64_t lo = INT64_MAX, hi = INT64_MIN;
  for (int s = 0; s < p->nseg; ++s) {
    int64_t b = p->seg[s].local_begin;
    int64_t e = (s + 1 < p->nseg) ? p->seg[s + 1].local_begin : len;
    int64_t a0 = std::max(b, u0), a1 = std::min(e, u1);
    if (a0 >= a1) continue;
    int64_t first = p->seg[s].global_begin + (a0 - b) * p->seg[s].stride;
    int64_t last = p->seg[s].global_begin + (a1 - 1 - b) * p->seg[s].stride;
    lo = std::min(lo, first);
    hi = std::max(hi, last);
  }
  *mn = lo;
  *mx = hi;
}

// number of keys of a partition whose position is <= p (segments are increasing runs)
static int64_t keys_at_or_before(const ma_pos* k, int64_t sk, int64_t p) {
  int64_t cnt = 0;
  for (int s = 0; s < k->nseg; ++s) {
    int64_t b = k->seg[s].local_begin;
    int64_t e = (s + 1 < k->nseg) ? k->seg[s + 1].local_begin : sk;
    int64_t n = e - b;
    if (n <= 0) continue;
    int64_t g = k->seg[s].global_begin, st = k->seg[s].stride;
    if (p < g) continue;
    int64_t m = (p - g) / st + 1;  // positions g, g+st, ... <= p
    cnt += std::min(m, n);
  }
  return cnt;
}

}  // namespace ma

using namespace ma;

extern "C" {

int mesh_attn_map_mesh_tile(int32_t n, int32_t a, int32_t b, int32_t g, int32_t kvr,
                            int32_t* q_parts, int32_t* kv_parts) {
  if (n < 1 || a < 1 || b < 1 || (int64_t)a * b != n || g < 0 || g >= n || !q_parts || !kv_parts)
    return set_error(MA_ERR_INVALID, "map_mesh_tile: need n = a*b, 0 <= g < n, non-null outputs");
  const int32_t r = g / a, c = g % a;
  for (int32_t x = 0; x < a; ++x) q_parts[x] = r * a + x;
  for (int32_t t = 0; t < b; ++t) kv_parts[t] = kvr ? c + t * a : c * b + t;
  return MA_OK;
}

int mesh_attn_map_groups(int32_t n, int32_t a, int32_t b, int32_t g, int32_t* q_group, int32_t* kv_group) {
  if (n < 1 || a < 1 || b < 1 || (int64_t)a * b != n || g < 0 || g >= n || !q_group || !kv_group)
    return set_error(MA_ERR_INVALID, "map_groups: need n = a*b, 0 <= g < n, non-null outputs");
  const int32_t r = g / a, c = g % a;
  for (int32_t x = 0; x < a; ++x) q_group[x] = r * a + x;
  for (int32_t x = 0; x < b; ++x) kv_group[x] = c + a * x;
  return MA_OK;
}

int mesh_attn_map_zigzag(int32_t N, int32_t r, int32_t chunks[2]) {
  if (N < 1 || r < 0 || r >= N || !chunks) return set_error(MA_ERR_INVALID, "map_zigzag: need 0 <= r < N");
  chunks[0] = r;
  chunks[1] = 2 * N - 1 - r;
  return MA_OK;
}

int mesh_attn_pos_contiguous(int64_t global_begin, ma_pos* out) {
  if (!out || global_begin < 0) return set_error(MA_ERR_INVALID, "pos_contiguous: bad argument");
  std::memset(out, 0, sizeof(*out));
  out->nseg = 1;
  out->seg[0] = {0, global_begin, 1};
  return MA_OK;
}

int mesh_attn_pos_zigzag(int32_t N, int32_t r, int64_t chunk_len, ma_pos* out) {
  if (!out || N < 1 || r < 0 || r >= N || chunk_len < 1) return set_error(MA_ERR_INVALID, "pos_zigzag: bad argument");
  std::memset(out, 0, sizeof(*out));
  out->nseg = 2;
  out->seg[0] = {0, (int64_t)r * chunk_len, 1};
  out->seg[1] = {chunk_len, (int64_t)(2 * N - 1 - r) * chunk_len, 1};
  return MA_OK;
}

int mesh_attn_pos_striped(int32_t N, int32_t r, ma_pos* out) {
  if (!out || N < 1 || r < 0 || r >= N) return set_error(MA_ERR_INVALID, "pos_striped: need 0 <= r < N");
  std::memset(out, 0, sizeof(*out));
  out->nseg = 1;
  out->seg[0] = {0, r, N};
  return MA_OK;
}

int64_t mesh_attn_pos_at(const ma_pos* pos, int64_t t) {
  if (!pos || pos->nseg < 1 || pos->nseg > MA_MAX_SEGMENTS || t < 0 || pos->seg[0].local_begin != 0) return -1;
  return pos_at(pos, t);
}

int mesh_attn_classify(const ma_pos* q_pos, int64_t sq, const ma_pos* k_pos, int64_t sk, int32_t mask_mode) {
  if (sq < 1 || sk < 1) return -set_error(MA_ERR_INVALID, "classify: sizes must be >= 1");
  if (mask_mode == MA_MASK_NONE) return MA_TILE_FULL;
  if (mask_mode != MA_MASK_CAUSAL && mask_mode != MA_MASK_STRIPED_ZIGZAG)
    return -set_error(MA_ERR_INVALID, "classify: unknown mask mode");
  const char* why = nullptr;
  if (!pos_valid(q_pos, sq, &why) || !pos_valid(k_pos, sk, &why)) return -set_error(MA_ERR_INVALID, why);
  int64_t qmin, qmax, kmin, kmax;
  pos_minmax(q_pos, sq, 0, sq, &qmin, &qmax);
  pos_minmax(k_pos, sk, 0, sk, &kmin, &kmax);
  if (kmin > qmax) return MA_TILE_EMPTY;
  if (kmax <= qmin) return MA_TILE_FULL;
  // Ranges overlap; with several segments some pair may still be allowed or not:
  // decide exactly by counting allowed pairs.
  int64_t cnt = mesh_attn_count_allowed(q_pos, sq, k_pos, sk, mask_mode);
  if (cnt == 0) return MA_TILE_EMPTY;
  if (cnt == sq * sk) return MA_TILE_FULL;
  return MA_TILE_PARTIAL;
}

int64_t mesh_attn_count_allowed(const ma_pos* q_pos, int64_t sq, const ma_pos* k_pos, int64_t sk, int32_t mask_mode) {
  if (sq < 1 || sk < 1) return -1;
  if (mask_mode == MA_MASK_NONE) return sq * sk;
  if (mask_mode != MA_MASK_CAUSAL && mask_mode != MA_MASK_STRIPED_ZIGZAG) return -1;
  const char* why = nullptr;
  if (!pos_valid(q_pos, sq, &why) || !pos_valid(k_pos, sk, &why)) return -1;
  int64_t total = 0;
  for (int s = 0; s < q_pos->nseg; ++s) {
    int64_t b = q_pos->seg[s].local_begin;
    int64_t e = (s + 1 < q_pos->nseg) ? q_pos->seg[s + 1].local_begin : sq;
    for (int64_t t = b; t < e; ++t)
      total += keys_at_or_before(k_pos, sk, q_pos->seg[s].global_begin + (t - b) * q_pos->seg[s].stride);
  }
  return total;
}

int32_t mesh_attn_build_worklist(int32_t nq, const ma_pos* q_pos, const int64_t* sq, int32_t nk,
                                 const ma_pos* k_pos, const int64_t* sk, int32_t mask_mode, int32_t max_out,
                                 int32_t* out_q, int32_t* out_k, int32_t* out_class) {
  if (nq < 0 || nk < 0 || max_out < 0 || (nq && (!q_pos || !sq)) || (nk && (!k_pos || !sk)) ||
      (max_out > 0 && (!out_q || !out_k || !out_class))) {
    set_error(MA_ERR_INVALID, "build_worklist: bad argument");
    return -1;
  }
  int32_t cnt = 0;
  for (int32_t i = 0; i < nq; ++i)
    for (int32_t j = 0; j < nk; ++j) {
      int c = mesh_attn_classify(&q_pos[i], sq[i], &k_pos[j], sk[j], mask_mode);
      if (c < 0) return -1;
      if (c == MA_TILE_EMPTY) continue;
      if (cnt < max_out) { out_q[cnt] = i; out_k[cnt] = j; out_class[cnt] = c; }
      ++cnt;
    }
  return cnt;
}

}  // extern "C"
