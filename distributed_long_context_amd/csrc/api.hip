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
#include <mutex>
#include <tuple>
#include <unordered_map>
#include <unordered_set>
#include <utility>

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

// p advanced by `bytes`, as address arithmetic (well defined for any pointer value, so the
// workspace query can expand the segments of tiles whose pointers are not set)
template <class T>
T* byte_offset(T* p, int64_t bytes) {
  return (T*)((uintptr_t)p + (uintptr_t)bytes);
}

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


// Outputs of two tiles that are the same buffer shifted along the sequence axis: the
// base pointers differ by a non-zero whole number of rows (row_bytes apart) that is
// smaller than the rows of the earlier view, so some rows are written by both tiles
// in one launch.  Such a call is rejected; identical outputs are allowed (the tiles
// are then applied in list order).  Other partial overlaps of output buffers are
// undefined.
template <class PtrOf, class RowsOf>
int check_shifted_outputs(int n, PtrOf ptr_of, RowsOf rows_of, int64_t row_bytes, const char* what) {
  if (row_bytes <= 0 || n < 2) return MA_OK;
  std::vector<std::pair<uintptr_t, int64_t>> v;  // (address, rows), sorted by address
  v.reserve(n);
  for (int i = 0; i < n; ++i) v.emplace_back((uintptr_t)ptr_of(i), rows_of(i));
  std::sort(v.begin(), v.end());
  // each view is compared with the one before it and with the earlier view reaching furthest
  size_t far = 0;
  auto shifted = [&](size_t j, size_t i) {
    const uintptr_t d = v[i].first - v[j].first;
    return d != 0 && d % (uintptr_t)row_bytes == 0 && (int64_t)(d / (uintptr_t)row_bytes) < v[j].second;
  };
  auto end_of = [&](size_t j) { return v[j].first + (uintptr_t)(v[j].second * row_bytes); };
  for (size_t i = 1; i < v.size(); ++i) {
    if (shifted(i - 1, i) || shifted(far, i)) {
      std::string m = std::string(what) + " buffers of two tiles overlap (the same buffer shifted by fewer rows than "
                                          "it holds); give each tile its own rows or the same buffer";
      return set_error(MA_ERR_INVALID, m.c_str());
    }
    if (end_of(i) > end_of(far)) far = i;
  }
  return MA_OK;
}

// One forward call, planned before anything is enqueued: its launches in order (a launch class
// with its kernel parameters, or the (0, -inf) fill of an EMPTY tile) and, when the resident-KV
// tiles go through a tile table in device memory, that table (tiles, group entries, workgroup
// records).
constexpr int kClasses = 5, kResident = 4;
struct FwdPlan {
  struct Launch {
    int m;    // launch class; -1: fill an EMPTY tile's output with (0, -inf)
    int wgs;  // workgroups of the launch
    int idx;  // class launches: index into batches; fills: the tile's index
  };
  FwdParams p;
  std::vector<Launch> launches;
  std::vector<FwdParams> batches;
  std::vector<FwdTile> table;
  std::vector<FwdResEnt> ents;
  std::vector<FwdResWg> wgs;
  int64_t units = 0;  // units numbered so far in the table
};

// FNV-1a (64-bit) over the table's tiles, entries and workgroup records, taken as 64-bit words
uint64_t table_hash(const FwdPlan& plan) {
  uint64_t h = 1469598103934665603ull;
  auto mix = [&](const void* data, size_t n) {
    const unsigned char* b = (const unsigned char*)data;
    for (size_t i = 0; i + 8 <= n; i += 8) {
      uint64_t w;
      std::memcpy(&w, b + i, 8);
      h = (h ^ w) * 1099511628211ull;
    }
  };
  mix(plan.table.data(), plan.table.size() * sizeof(FwdTile));
  mix(plan.ents.data(), plan.ents.size() * sizeof(FwdResEnt));
  mix(plan.wgs.data(), plan.wgs.size() * sizeof(FwdResWg));
  return h;
}

size_t table_bytes(const FwdPlan& plan) {
  return sizeof(FwdTableHeader) + plan.table.size() * sizeof(FwdTile) + plan.ents.size() * sizeof(FwdResEnt) +
         plan.wgs.size() * sizeof(FwdResWg);
}

int plan_fwd(const ma_tile_fwd_args* a, bool use_table, FwdPlan& plan) {
  if (!a) return set_error(MA_ERR_INVALID, "null args");
  int rc = check_common(a->dtype, a->batch, a->hq, a->hkv, a->head_dim, a->mask_mode, a->scale);
  if (rc) return rc;
  if (!a->head_map && a->hq % a->hkv) return set_error(MA_ERR_INVALID, "hq must be a multiple of hkv when head_map is NULL");
  if (a->ntiles < 0 || a->ntiles > MA_MAX_TILES) return set_error(MA_ERR_INVALID, "ntiles out of range");
  if (a->accumulate != 0 && a->accumulate != 1) return set_error(MA_ERR_INVALID, "accumulate must be 0 or 1");
  if (a->ntiles == 0) return MA_OK;
  if (!a->tiles) return set_error(MA_ERR_INVALID, "null tile list");
  if (!strides_ok(a->q_stride, 3, a->dtype) || !strides_ok(a->k_stride, 3, a->dtype) ||
      !strides_ok(a->v_stride, 3, a->dtype) || !strides_ok(a->o_stride, 3, a->dtype) || a->lse_stride[0] < 0 ||
      a->lse_stride[1] < 0)
    return set_error(MA_ERR_INVALID, "strides must be >= 0 and multiples of 16 bytes");
  if (a->dtype == MA_BF16 && (a->k_stride[1] >= (1 << 24) || a->v_stride[1] >= (1 << 24)))
    return set_error(MA_ERR_UNSUPPORTED, "K/V sequence strides must be below 2^24 elements");

  FwdParams& p = plan.p;
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
  const int64_t esize = bf16 ? 2 : 4;
  rc = check_shifted_outputs(a->ntiles, [&](int i) { return a->tiles[i].o; },
                             [&](int i) { return a->tiles[i].sq; }, a->o_stride[1] * esize, "o");
  if (rc) return rc;
  rc = check_shifted_outputs(a->ntiles, [&](int i) { return (const void*)a->tiles[i].lse; },
                             [&](int i) { return a->tiles[i].sq; }, 4, "lse");
  if (rc) return rc;
  // Tiles go to one of five launch classes: by how much masking they need (bit 0) and, in
  // bf16, by length (bit 1), or the resident-KV kernel (kResident), which takes the unmasked
  // bf16 tiles of kFwdResMinKeys < sk <= kFwdResKeys keys.  FULL tiles (and every tile
  // without a mask) run the unmasked kernel, PARTIAL ones the masked kernel, whose key
  // positions must be one segment: a tile whose key positions have several segments is cut into one piece
  // per segment (the keys of a segment are contiguous rows) and its pieces with any
  // allowed pair go to the masked kernel as a chain of consecutive entries, which one
  // workgroup runs in turn with the softmax state in registers, so the output is
  // written (and rounded) once.  Tiles of at most kFwdSmallBlocks key blocks run the
  // four-wave kernel.  A tile naming the output of one already queued waits for it.
  // The whole call is planned first and launched afterwards, so an argument error
  // found on any tile leaves nothing enqueued.
  // With a table (use_table), the resident-KV tiles go to plan.table instead: no limit of tiles
  // per launch; a launch is a span of the table, cut where a tile names an output already
  // queued.  The span's tiles with the same K and V form groups, and a workgroup runs a range of
  // one group's units (group_span below).
  std::vector<FwdPlan::Launch>& launches = plan.launches;
  std::vector<FwdParams>& batches = plan.batches;
  FwdParams bp[kClasses];
  int bn[kClasses] = {}, bwg[kClasses] = {};
  for (int m = 0; m < kClasses; ++m) {
    bp[m] = p;
    bp[m].mask = m != kResident && (m & 1);
  }
  size_t tab_first = 0;  // first table tile of the resident span being filled
  int64_t tab_units = 0;  // units of the table's tiles so far
  // outputs (O and LSE addresses) of the resident span being filled: a set, so that a call of
  // thousands of tiles checks each new tile in constant time
  std::unordered_set<uintptr_t> tab_o, tab_lse;
  // Groups the span's tiles by K/V (pointers and length: one LDS copy serves them all) and writes
  // each group's entries (its tiles, units numbered on from plan.units) and workgroup records:
  // per chunk of `cap` consecutive units of the group, one workgroup per (batch, KV head), the KV
  // head fastest (so the XCD of a workgroup follows its KV head).  cap grows from kFwdResUnits to
  // kFwdResUnitsMax while the span still gives about 2048 workgroups (8 per CU): more units per
  // workgroup spread its K/V loads over more work and split evenly over the 8 waves.  Returns the
  // span's workgroup count.
  auto group_span = [&](size_t first, size_t last) -> int64_t {
    std::vector<size_t> idx;
    for (size_t j = first; j < last; ++j) idx.push_back(j);
    auto key = [&](size_t j) {
      return std::make_tuple((uintptr_t)plan.table[j].k, (uintptr_t)plan.table[j].v, plan.table[j].sk);
    };
    std::stable_sort(idx.begin(), idx.end(), [&](size_t x, size_t y) { return key(x) < key(y); });
    auto units_of = [&](size_t j) { return (int64_t)(plan.table[j].sq + 31) / 32 * p.gmax; };
    int64_t total = 0;
    for (size_t j : idx) total += units_of(j);
    const int64_t per_wg = (int64_t)a->batch * a->hkv * total / 2048 / 8 * 8;
    const int64_t cap = std::min<int64_t>(kFwdResUnitsMax, std::max<int64_t>(kFwdResUnits, per_wg));
    const size_t wg0 = plan.wgs.size();
    for (size_t g = 0; g < idx.size();) {
      size_t g_end = g + 1;
      while (g_end < idx.size() && key(idx[g_end]) == key(idx[g])) ++g_end;
      const size_t e0 = plan.ents.size();
      const int64_t u0 = plan.units;
      for (size_t i = g; i < g_end; ++i) {
        plan.ents.push_back(FwdResEnt{(int32_t)idx[i], (int32_t)plan.units});
        plan.units += units_of(idx[i]);
      }
      size_t e = e0;
      for (int64_t c = u0; c < plan.units; c += cap) {
        while (e + 1 < plan.ents.size() && plan.ents[e + 1].unit0 <= c) ++e;
        for (int b = 0; b < a->batch; ++b)
          for (int h = 0; h < a->hkv; ++h)
            plan.wgs.push_back(FwdResWg{(int32_t)e, (int32_t)c, (int32_t)std::min(plan.units, c + cap),
                                        (int32_t)(b * a->hkv + h)});
      }
      g = g_end;
    }
    return (int64_t)(plan.wgs.size() - wg0);
  };
  auto flush = [&](int m) {
    if (bn[m] == 0) return;
    bp[m].ntiles = bn[m];
    if (use_table && m == kResident) {
      bp[m].wg_base = (int32_t)plan.wgs.size();
      bwg[m] = (int)group_span(tab_first, plan.table.size());
      tab_first = plan.table.size();
      tab_o.clear();
      tab_lse.clear();
    }
    launches.push_back(FwdPlan::Launch{m, bwg[m], (int)batches.size()});
    batches.push_back(bp[m]);
    bn[m] = 0;
    bwg[m] = 0;
  };
  auto flush_all = [&]() {
    for (int m = 0; m < kClasses; ++m) flush(m);
  };
  // queue one tile (or the pieces of one, as a chain): cls is the class of the tile (any
  // chain runs masked), acc its accumulate flag, pieces the key segments after the first
  auto enqueue_chain = [&](const ma_tile* pcs, int npcs, int cls, int acc) -> int {
    bool dup = false;
    for (int k = 0; k < kClasses; ++k)
      for (int j = 0; j < bn[k] && !(use_table && k == kResident); ++j)
        dup = dup || bp[k].tiles[j].o == pcs[0].o || bp[k].tiles[j].lse == pcs[0].lse;
    dup = dup || tab_o.count((uintptr_t)pcs[0].o) || tab_lse.count((uintptr_t)pcs[0].lse);
    if (dup) flush_all();
    int64_t blocks = 0;
    for (int i = 0; i < npcs; ++i) blocks += (pcs[i].sk + 63) / 64;
    const bool small = bf16 && blocks <= kFwdSmallBlocks;
    const bool whole = cls == MA_TILE_FULL && npcs == 1;
    const int64_t res_lo = a->head_dim == 128 ? kFwdResMinKeys<128> : kFwdResMinKeys<64>;
    const int64_t res_hi = a->head_dim == 128 ? kFwdResKeys<128> : kFwdResKeys<64>;
    const bool resident = bf16 && whole && pcs[0].sk > res_lo && pcs[0].sk <= res_hi;
    const int m = resident ? kResident : (whole ? 0 : 1) | (small ? 2 : 0);
    const ma_tile& t = pcs[0];
    int64_t wgs, chunks;
    if (bf16) {
      // units are (32-row block, head of the group): 8 (or 4) per workgroup of the ring
      // kernel, one per wave; up to kFwdResUnits per workgroup of the resident kernel
      const int waves = small ? 4 : 8;
      const int64_t nqb = (t.sq + 31) / 32;
      const int units = resident ? kFwdResUnits : waves;
      chunks = (nqb * p.gmax + units - 1) / units;
      wgs = (int64_t)a->batch * a->hkv * chunks;
      wgs = (wgs + 7) / 8 * 8;  // keep each tile's first workgroup on XCD 0
    } else {
      chunks = (t.sq + 63) / 64;
      wgs = (int64_t)a->batch * a->hq * chunks;
    }
    if (wgs >= INT32_MAX) return set_error(MA_ERR_INVALID, "tile too large for one launch");
    // a chain stays in one launch, and a launch's workgroup count stays below 2^31
    const bool tabled = use_table && m == kResident;
    // the table's workgroups (at most the tiles' own counts: grouping only merges chunks) and
    // units stay below 2^31
    if (tabled && ((int64_t)plan.wgs.size() + bwg[m] + wgs >= INT32_MAX ||
                   tab_units + (t.sq + 31) / 32 * p.gmax >= INT32_MAX))
      return set_error(MA_ERR_INVALID, "the tile table's workgroups and units must stay below 2^31");
    if ((!tabled && bn[m] + npcs > kFwdTilesPerLaunch) || bwg[m] + wgs >= INT32_MAX) flush(m);
    FwdTile scratch_tile;
    FwdTile& ft = tabled ? scratch_tile : bp[m].tiles[bn[m]];
    std::memset(&ft, 0, sizeof(ft));
    ft.q = t.q; ft.k = t.k; ft.v = t.v; ft.o = t.o; ft.lse = t.lse;
    ft.sq = (int32_t)t.sq;
    ft.sk = (int32_t)t.sk;
    ft.accumulate = acc;
    ft.chunks = (int32_t)chunks;
    if (m & 1) {  // key positions are one segment here (split below)
      to_kpos(t.q_pos, ft.qp);
      ft.kgb = (int32_t)t.k_pos.seg[0].global_begin;
      ft.kst = (int32_t)t.k_pos.seg[0].stride;
    } else {
      ft.qp.nseg = 1;
    }
    if (tabled) {  // one tile entry in the table; its workgroups come when the span is flushed
      ft.wg_begin = 0;
      ft.chunks = 0;
      plan.table.push_back(ft);
      tab_o.insert((uintptr_t)t.o);
      tab_lse.insert((uintptr_t)t.lse);
      tab_units += (t.sq + 31) / 32 * p.gmax;
      bwg[m] += (int)wgs;
      ++bn[m];
      return MA_OK;  // resident tiles have no chained pieces
    }
    ft.wg_begin = bwg[m];
    bwg[m] += (int)wgs;
    ++bn[m];
    // the chained key segments: no workgroups of their own (their first workgroup is where
    // the next tile's begin, so the kernel's tile lookup skips them)
    for (int i = 1; i < npcs; ++i) {
      FwdTile& ct = bp[m].tiles[bn[m]];
      ct = ft;
      ct.k = pcs[i].k;
      ct.v = pcs[i].v;
      ct.sk = (int32_t)pcs[i].sk;
      ct.kgb = (int32_t)pcs[i].k_pos.seg[0].global_begin;
      ct.kst = (int32_t)pcs[i].k_pos.seg[0].stride;
      ct.accumulate = kFwdChained;
      ct.wg_begin = bwg[m];
      ++bn[m];
    }
    if (bn[m] == kFwdTilesPerLaunch) flush(m);
    return MA_OK;
  };
  for (int i = 0; i < a->ntiles; ++i) {
    const ma_tile& t = a->tiles[i];
    const int nseg = a->mask_mode == MA_MASK_NONE ? 1 : t.k_pos.nseg;
    ma_tile pcs[MA_MAX_SEGMENTS];
    int pcls[MA_MAX_SEGMENTS];
    int npcs = 0, cls_all = MA_TILE_FULL;
    for (int sgi = 0; sgi < nseg; ++sgi) {
      ma_tile u = t;
      if (nseg > 1) {
        const int64_t lb = t.k_pos.seg[sgi].local_begin;
        const int64_t le = sgi + 1 < nseg ? t.k_pos.seg[sgi + 1].local_begin : t.sk;
        u.k = byte_offset(t.k, lb * a->k_stride[1] * esize);
        u.v = byte_offset(t.v, lb * a->v_stride[1] * esize);
        u.sk = le - lb;
        std::memset(&u.k_pos, 0, sizeof(u.k_pos));
        u.k_pos.nseg = 1;
        u.k_pos.seg[0].local_begin = 0;
        u.k_pos.seg[0].global_begin = t.k_pos.seg[sgi].global_begin;
        u.k_pos.seg[0].stride = t.k_pos.seg[sgi].stride;
      }
      const int cls = a->mask_mode == MA_MASK_NONE ? MA_TILE_FULL
                                                   : mesh_attn_classify(&u.q_pos, u.sq, &u.k_pos, u.sk, a->mask_mode);
      if (cls == MA_TILE_EMPTY) continue;
      if (cls != MA_TILE_FULL) cls_all = cls;
      pcls[npcs] = cls;
      pcs[npcs++] = u;
    }
    if (npcs > 0 && bf16) {
      rc = enqueue_chain(pcs, npcs, cls_all, a->accumulate);
      if (rc) return rc;
    } else if (npcs > 0) {
      // fp32: one tile per piece, the later pieces folding into the first (fp32 outputs
      // lose nothing by being stored between pieces)
      for (int i = 0; i < npcs; ++i) {
        rc = enqueue_chain(&pcs[i], 1, pcls[i], i == 0 ? a->accumulate : 1);
        if (rc) return rc;
      }
    } else if (a->accumulate == 0) {  // no piece had an allowed pair: the tile's result is (0, -inf)
      flush_all();  // a queued tile may name the same output
      launches.push_back(FwdPlan::Launch{-1, 0, i});
    }
  }
  flush_all();
  return MA_OK;
}

// Enqueues a planned forward; dev_table: the device copy of the plan's tile table (with one).
int launch_fwd_plan(const ma_tile_fwd_args* a, FwdPlan& plan, const void* dev_table, void* stream) {
  const FwdParams& p = plan.p;
  const bool bf16 = a->dtype == MA_BF16;
  const uint64_t hash = dev_table ? table_hash(plan) : 0;
  for (const FwdPlan::Launch& pl : plan.launches) {
    int e;
    if (pl.m < 0) {
      const ma_tile& t = a->tiles[pl.idx];
      e = launch_fill_empty(t.o, t.lse, a->dtype, a->batch, (int)t.sq, a->hq, a->head_dim, p.o_sb, p.o_ss, p.o_sh,
                            p.l_sb, p.l_sh, stream);
    } else if (pl.m == kResident) {
      FwdParams& rp = plan.batches[pl.idx];
      if (dev_table) {
        rp.table_header = (const FwdTableHeader*)dev_table;
        rp.table = (const FwdTile*)byte_offset(dev_table, sizeof(FwdTableHeader));
        const size_t ents_off = sizeof(FwdTableHeader) + plan.table.size() * sizeof(FwdTile);
        rp.res_ents = (const FwdResEnt*)byte_offset(dev_table, ents_off);
        rp.res_wgs = (const FwdResWg*)byte_offset(dev_table, ents_off + plan.ents.size() * sizeof(FwdResEnt));
        rp.table_ntiles = (int32_t)plan.table.size();
        rp.table_nents = (int32_t)plan.ents.size();
        rp.table_nwgs = (int32_t)plan.wgs.size();
        rp.table_hash = hash;
      }
      e = launch_fwd_bf16_resident(rp, a->head_dim, pl.wgs, stream);
    } else if (bf16) {
      e = launch_fwd_bf16(plan.batches[pl.idx], a->head_dim, pl.m & 2 ? 4 : 8, pl.wgs, stream);
    } else {
      e = launch_fwd_f32(plan.batches[pl.idx], a->head_dim, pl.wgs, stream);
    }
    const int rc = check_hip(e, pl.m < 0 ? "fill launch" : "tile_fwd launch");
    if (rc) return rc;
  }
  return MA_OK;
}

}  // namespace
}  // namespace ma

using namespace ma;

extern "C" {

const char* mesh_attn_last_error(void) { return g_last_error.c_str(); }
int mesh_attn_version(void) { return MA_VERSION; }

int mesh_attn_tile_fwd(const ma_tile_fwd_args* a, void* stream) {
  FwdPlan plan;
  const int rc = plan_fwd(a, false, plan);
  if (rc || !a->ntiles) return rc;
  return launch_fwd_plan(a, plan, nullptr, stream);
}

size_t mesh_attn_tile_fwd_table_bytes(const ma_tile_fwd_args* a) {
  FwdPlan plan;
  if (plan_fwd(a, true, plan)) return 0;
  return table_bytes(plan);
}

int mesh_attn_tile_fwd_pack(const ma_tile_fwd_args* a, void* table, size_t bytes) {
  FwdPlan plan;
  const int rc = plan_fwd(a, true, plan);
  if (rc) return rc;
  const size_t need = table_bytes(plan);
  if (!table || bytes < need) return set_error(MA_ERR_INVALID, "table missing or smaller than mesh_attn_tile_fwd_table_bytes");
  FwdTableHeader h;
  std::memset(&h, 0, sizeof(h));
  h.magic = kFwdTableMagic;
  h.ntiles = (int32_t)plan.table.size();
  h.nwgs = (int32_t)plan.wgs.size();
  h.nents = (int32_t)plan.ents.size();
  h.hash = table_hash(plan);
  unsigned char* out = (unsigned char*)table;
  std::memcpy(out, &h, sizeof(h));
  out += sizeof(h);
  if (!plan.table.empty()) std::memcpy(out, plan.table.data(), plan.table.size() * sizeof(FwdTile));
  out += plan.table.size() * sizeof(FwdTile);
  if (!plan.ents.empty()) std::memcpy(out, plan.ents.data(), plan.ents.size() * sizeof(FwdResEnt));
  out += plan.ents.size() * sizeof(FwdResEnt);
  if (!plan.wgs.empty()) std::memcpy(out, plan.wgs.data(), plan.wgs.size() * sizeof(FwdResWg));
  return MA_OK;
}

int mesh_attn_tile_fwd_tabled(const ma_tile_fwd_args* a, const void* table, size_t bytes, void* stream) {
  FwdPlan plan;
  const int rc = plan_fwd(a, true, plan);
  if (rc || !a->ntiles) return rc;
  if (!table || !aligned16(table) || bytes < table_bytes(plan))
    return set_error(MA_ERR_INVALID, "device table missing, not 16-byte aligned or smaller than mesh_attn_tile_fwd_table_bytes");
  return launch_fwd_plan(a, plan, table, stream);
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

int mesh_attn_reduce_add(const ma_reduce_args* a, void* stream) {
  if (!a) return set_error(MA_ERR_INVALID, "null args");
  if (a->k < 1 || a->k > MA_MAX_MERGE) return set_error(MA_ERR_INVALID, "k must be in 1..MA_MAX_MERGE");
  if (a->n < 0) return set_error(MA_ERR_INVALID, "n must be >= 0");
  if (a->n == 0) return MA_OK;
  if (!a->in || !a->out) return set_error(MA_ERR_INVALID, "null pointer");
  if (!aligned16(a->out)) return set_error(MA_ERR_INVALID, "out must be 16-byte aligned");
  ReduceParams p;
  std::memset(&p, 0, sizeof(p));
  for (int r = 0; r < a->k; ++r) {
    if (!a->in[r]) return set_error(MA_ERR_INVALID, "null input pointer");
    if (!aligned16(a->in[r])) return set_error(MA_ERR_INVALID, "inputs must be 16-byte aligned");
    p.in[r] = a->in[r];
  }
  p.k = a->k;
  p.n = a->n;
  p.out = a->out;
  return check_hip(launch_reduce_add(p, stream), "reduce_add launch");
}

}  // extern "C"

namespace ma {
namespace {

// Q groups (tiles sharing a dq buffer) and KV groups (tiles sharing a dk buffer)
// of a backward call, with the tiles of each group in call order.
struct BwdGroups {
  std::vector<int> q_of, kv_of;                 // group of each tile
  std::vector<std::vector<int>> qg, kvg;        // tiles of each group
};

// Under a mask, a tile whose Q or K positions have several segments runs as one
// piece per (Q segment, K segment): the rows of a segment are contiguous, so a
// piece is the same buffers at a row offset with a one-segment position map.  The
// pieces of a tile's Q segment share its dq rows (summed like any Q group) and
// those of a K segment its dk/dv rows.  Returns a or the expanded copy in e.
const ma_tile_bwd_args* expand_bwd_segments(const ma_tile_bwd_args* a, std::vector<ma_bwd_tile>& ex,
                                            ma_tile_bwd_args& e) {
  if (a->mask_mode == MA_MASK_NONE) return a;
  bool any = false;
  for (int i = 0; i < a->ntiles; ++i) any = any || a->tiles[i].q_pos.nseg > 1 || a->tiles[i].k_pos.nseg > 1;
  if (!any) return a;
  auto seg_end = [](const ma_pos& ps, int s, int64_t len) {
    return s + 1 < ps.nseg ? ps.seg[s + 1].local_begin : len;
  };
  auto one_seg = [](const ma_pos& ps, int s) {
    ma_pos o;
    std::memset(&o, 0, sizeof(o));
    o.nseg = 1;
    o.seg[0].global_begin = ps.seg[s].global_begin;
    o.seg[0].stride = ps.seg[s].stride;
    return o;
  };
  for (int i = 0; i < a->ntiles; ++i) {
    const ma_bwd_tile& t = a->tiles[i];
    for (int qs = 0; qs < t.q_pos.nseg; ++qs)
      for (int ks = 0; ks < t.k_pos.nseg; ++ks) {
        ma_bwd_tile u = t;
        const int64_t qb = t.q_pos.seg[qs].local_begin, kb = t.k_pos.seg[ks].local_begin;
        if (t.q_pos.nseg > 1) {
          u.q = byte_offset(t.q, qb * a->q_stride[1] * 2);
          u.o = byte_offset(t.o, qb * a->q_stride[1] * 2);
          u.dout = byte_offset(t.dout, qb * a->q_stride[1] * 2);
          u.lse = byte_offset(t.lse, qb * 4);
          u.dq = byte_offset(t.dq, qb * a->dq_stride[1] * 4);
          u.sq = seg_end(t.q_pos, qs, t.sq) - qb;
          u.q_pos = one_seg(t.q_pos, qs);
        }
        if (t.k_pos.nseg > 1) {
          u.k = byte_offset(t.k, kb * a->k_stride[1] * 2);
          u.v = byte_offset(t.v, kb * a->k_stride[1] * 2);
          u.dk = byte_offset(t.dk, kb * a->dk_stride[1] * 4);
          u.dv = byte_offset(t.dv, kb * a->dk_stride[1] * 4);
          u.sk = seg_end(t.k_pos, ks, t.sk) - kb;
          u.k_pos = one_seg(t.k_pos, ks);
        }
        ex.push_back(u);
      }
  }
  e = *a;
  e.tiles = ex.data();
  e.ntiles = (int32_t)ex.size();
  return &e;
}

BwdGroups bwd_groups(const ma_tile_bwd_args* a) {
  BwdGroups g;
  g.q_of.assign(a->ntiles, -1);
  g.kv_of.assign(a->ntiles, -1);
  std::unordered_map<uintptr_t, int> q_group, kv_group;  // dq / dk address -> group
  for (int i = 0; i < a->ntiles; ++i) {
    const auto q = q_group.emplace((uintptr_t)a->tiles[i].dq, (int)g.qg.size());
    if (q.second) g.qg.emplace_back();
    g.q_of[i] = q.first->second;
    g.qg[g.q_of[i]].push_back(i);
    const auto kv = kv_group.emplace((uintptr_t)a->tiles[i].dk, (int)g.kvg.size());
    if (kv.second) g.kvg.emplace_back();
    g.kv_of[i] = kv.first->second;
    g.kvg[g.kv_of[i]].push_back(i);
  }
  return g;
}

// bytes of the blocked LSE2/D arrays of one Q partition
size_t lsed_bytes(int batch, int hq, int64_t sq) {
  const int64_t nqb = (sq + 63) / 64;
  return ((size_t)batch * hq * nqb * 128 * sizeof(float) + 255) / 256 * 256;
}

}  // namespace
}  // namespace ma

extern "C" {

size_t mesh_attn_tile_bwd_workspace_size(const ma_tile_bwd_args* a0) {
  if (!a0 || a0->ntiles <= 0 || a0->ntiles > MA_MAX_TILES || !a0->tiles || a0->batch < 1 || a0->hq < 1 ||
      a0->hq > MA_MAX_HEADS)
    return 0;
  for (int i = 0; i < a0->ntiles; ++i) {
    const ma_bwd_tile& t = a0->tiles[i];
    if (t.sq < 1 || t.sk < 1 || t.sq >= INT32_MAX || t.sk >= INT32_MAX) return 0;
    // the segments are expanded below: they must be valid first
    if (a0->mask_mode != MA_MASK_NONE && check_positions(a0->mask_mode, t.q_pos, t.sq, t.k_pos, t.sk) != MA_OK)
      return 0;
  }
  std::vector<ma_bwd_tile> ex;
  ma_tile_bwd_args e;
  const ma_tile_bwd_args* a = expand_bwd_segments(a0, ex, e);
  const BwdGroups g = bwd_groups(a);
  size_t bytes = 0;
  for (const auto& grp : g.qg) bytes += lsed_bytes(a->batch, a->hq, a->tiles[grp[0]].sq);
  return bytes;
}

}  // extern "C"

namespace ma {
namespace {

// Every argument check of the backward (nothing is enqueued before they all pass).
int validate_bwd(const ma_tile_bwd_args* a) {
  if (!a) return set_error(MA_ERR_INVALID, "null args");
  if (a->dtype != MA_BF16) return set_error(a->dtype == MA_F32 ? MA_ERR_UNSUPPORTED : MA_ERR_INVALID,
                                            "tile_bwd supports bf16 inputs only");
  int rc = check_common(a->dtype, a->batch, a->hq, a->hkv, a->head_dim, a->mask_mode, a->scale);
  if (rc) return rc;
  if (!a->head_map && a->hq % a->hkv) return set_error(MA_ERR_INVALID, "hq must be a multiple of hkv when head_map is NULL");
  if (a->ntiles < 0 || a->ntiles > MA_MAX_TILES) return set_error(MA_ERR_INVALID, "ntiles out of range");
  if (a->ntiles == 0) return MA_OK;
  if (!a->tiles) return set_error(MA_ERR_INVALID, "null tile list");
  if (!strides_ok(a->q_stride, 3, MA_BF16) || !strides_ok(a->k_stride, 3, MA_BF16) ||
      !strides_ok(a->dq_stride, 3, MA_F32) || !strides_ok(a->dk_stride, 3, MA_F32) || a->lse_stride[0] < 0 ||
      a->lse_stride[1] < 0)
    return set_error(MA_ERR_INVALID, "strides must be >= 0 and multiples of 16 bytes");
  if (a->q_stride[1] >= (1 << 24) || a->k_stride[1] >= (1 << 24))
    return set_error(MA_ERR_UNSUPPORTED, "Q/K/V sequence strides must be below 2^24 elements");
  std::unordered_map<uintptr_t, int> kv_first, q_first;  // output address -> first tile naming it
  for (int i = 0; i < a->ntiles; ++i) {
    const ma_bwd_tile& t = a->tiles[i];
    if (!t.q || !t.k || !t.v || !t.o || !t.dout || !t.lse || !t.dq || !t.dk || !t.dv)
      return set_error(MA_ERR_INVALID, "null tensor pointer in a tile");
    if (!aligned16(t.q) || !aligned16(t.k) || !aligned16(t.v) || !aligned16(t.o) || !aligned16(t.dout) ||
        !aligned16(t.dq) || !aligned16(t.dk) || !aligned16(t.dv) || ((uintptr_t)t.lse & 3u))
      return set_error(MA_ERR_INVALID, "tensor pointers must be 16-byte aligned (lse 4-byte)");
    if (t.sq < 1 || t.sk < 1 || t.sq >= INT32_MAX || t.sk >= INT32_MAX)
      return set_error(MA_ERR_INVALID, "tile sizes must be in [1, 2^31-1)");
    rc = check_positions(a->mask_mode, t.q_pos, t.sq, t.k_pos, t.sk);
    if (rc) return rc;
    // Tiles sharing dk or dv must share the whole KV description, and tiles sharing dq the whole
    // Q description.  Each tile is compared with the first tile that named the same address (the
    // tiles before it that named it were all found equal to that one), found through hash maps so
    // that a call of thousands of tiles is checked in linear time.
    const auto kv_same_as = [&](const ma_bwd_tile& u) {
      return u.dk == t.dk && u.dv == t.dv && u.k == t.k && u.v == t.v && u.sk == t.sk &&
             (a->mask_mode == MA_MASK_NONE || std::memcmp(&u.k_pos, &t.k_pos, sizeof(ma_pos)) == 0);
    };
    for (const void* addr : {(const void*)t.dk, (const void*)t.dv}) {
      const auto it = kv_first.find((uintptr_t)addr);
      if (it != kv_first.end() && !kv_same_as(a->tiles[it->second]))
        return set_error(MA_ERR_INVALID, "tiles naming the same dk/dv must name the same k, v, sk and k_pos");
    }
    kv_first.emplace((uintptr_t)t.dk, i);
    kv_first.emplace((uintptr_t)t.dv, i);
    const auto qit = q_first.find((uintptr_t)t.dq);
    if (qit != q_first.end()) {
      const ma_bwd_tile& u = a->tiles[qit->second];
      if (u.q != t.q || u.o != t.o || u.dout != t.dout || u.lse != t.lse || u.sq != t.sq ||
          (a->mask_mode != MA_MASK_NONE && std::memcmp(&u.q_pos, &t.q_pos, sizeof(ma_pos)) != 0))
        return set_error(MA_ERR_INVALID, "tiles naming the same dq must name the same q, o, dout, lse, sq and q_pos");
    } else {
      q_first.emplace((uintptr_t)t.dq, i);
    }
  }
  rc = check_shifted_outputs(a->ntiles, [&](int i) { return (const void*)a->tiles[i].dq; },
                             [&](int i) { return a->tiles[i].sq; }, a->dq_stride[1] * 4, "dq");
  if (rc) return rc;
  rc = check_shifted_outputs(a->ntiles, [&](int i) { return (const void*)a->tiles[i].dk; },
                             [&](int i) { return a->tiles[i].sk; }, a->dk_stride[1] * 4, "dk");
  if (rc) return rc;
  rc = check_shifted_outputs(a->ntiles, [&](int i) { return (const void*)a->tiles[i].dv; },
                             [&](int i) { return a->tiles[i].sk; }, a->dk_stride[1] * 4, "dv");
  if (rc) return rc;
  return MA_OK;
}

// The backward of validated arguments with a workspace of at least the required size.
int run_bwd(const ma_tile_bwd_args* a, void* workspace, void* stream) {
  int rc;
  // from here on the tiles are single-segment pieces
  std::vector<ma_bwd_tile> ex;
  ma_tile_bwd_args e;
  a = expand_bwd_segments(a, ex, e);
  const BwdGroups grp = bwd_groups(a);
  BwdParams base;
  std::memset(&base, 0, sizeof(base));
  const char* why = nullptr;
  base.gmax = build_head_groups(a->hq, a->hkv, a->head_map, base.heads_of, base.kv_first, &why);
  if (base.gmax < 0) return set_error(MA_ERR_INVALID, why);
  base.batch = a->batch;
  base.hq = a->hq;
  base.hkv = a->hkv;
  base.mask = a->mask_mode != MA_MASK_NONE;
  base.scale = a->scale;
  base.scale_log2 = a->scale * 1.4426950408889634f;
  base.q_sb = a->q_stride[0]; base.q_ss = a->q_stride[1]; base.q_sh = a->q_stride[2];
  base.k_sb = a->k_stride[0]; base.k_ss = a->k_stride[1]; base.k_sh = a->k_stride[2];
  base.dq_sb = a->dq_stride[0]; base.dq_ss = a->dq_stride[1]; base.dq_sh = a->dq_stride[2];
  base.dk_sb = a->dk_stride[0]; base.dk_ss = a->dk_stride[1]; base.dk_sh = a->dk_stride[2];

  // 1) per Q group: blocked LSE2 / D in its workspace slice
  std::vector<BwdQPart> qparts(grp.qg.size());
  size_t off = 0;
  for (size_t gi = 0; gi < grp.qg.size(); ++gi) {
    const ma_bwd_tile& t = a->tiles[grp.qg[gi][0]];
    BwdQPart& q = qparts[gi];
    std::memset(&q, 0, sizeof(q));
    q.q = t.q; q.dout = t.dout; q.dq = t.dq;
    q.lsed = (const float*)((char*)workspace + off);
    q.sq = (int32_t)t.sq;
    if (a->mask_mode != MA_MASK_NONE) to_kpos(t.q_pos, q.qp);
    else q.qp.nseg = 1;
    BwdPreParams pp;
    pp.batch = a->batch; pp.hq = a->hq; pp.sq = (int32_t)t.sq; pp.scale = a->scale;
    pp.o = t.o; pp.dout = t.dout; pp.lse = t.lse; pp.lsed = (float*)((char*)workspace + off);
    pp.q_sb = a->q_stride[0]; pp.q_ss = a->q_stride[1]; pp.q_sh = a->q_stride[2];
    pp.l_sb = a->lse_stride[0]; pp.l_sh = a->lse_stride[1];
    off += lsed_bytes(a->batch, a->hq, t.sq);
    rc = check_hip(launch_bwd_preprocess(pp, a->head_dim, stream), "tile_bwd preprocess launch");
    if (rc) return rc;
  }
  std::vector<BwdKVPart> kvparts(grp.kvg.size());
  for (size_t gi = 0; gi < grp.kvg.size(); ++gi) {
    const ma_bwd_tile& t = a->tiles[grp.kvg[gi][0]];
    BwdKVPart& k = kvparts[gi];
    std::memset(&k, 0, sizeof(k));
    k.k = t.k; k.v = t.v; k.dk = t.dk; k.dv = t.dv;
    k.sk = (int32_t)t.sk;
    if (a->mask_mode != MA_MASK_NONE) to_kpos(t.k_pos, k.kp);
    else k.kp.nseg = 1;
  }

  // 2) dQ launches (entries = Q groups with their KV partitions), then dK/dV launches
  //    (entries = KV groups with their Q partitions).  A group's partners are split
  //    by pair class: FULL pairs run in unmasked launches, PARTIAL (and EMPTY) pairs
  //    in masked ones, FULL first.  A group with more than 8 partners of one kind is
  //    split further; every piece after a group's first adds to the earlier ones and
  //    runs in a later launch.  Each launch holds at most 8 entries, 8 partitions of
  //    either side, and one piece per group, all of one mask kind.
  std::vector<int> tile_cls(a->ntiles, MA_TILE_FULL);
  if (a->mask_mode != MA_MASK_NONE)
    for (int i = 0; i < a->ntiles; ++i)
      tile_cls[i] = mesh_attn_classify(&a->tiles[i].q_pos, a->tiles[i].sq, &a->tiles[i].k_pos, a->tiles[i].sk,
                                       a->mask_mode);
  for (int side = 0; side < 2; ++side) {
    const bool dq_side = side == 0;
    const auto& own = dq_side ? grp.qg : grp.kvg;
    // kind 0: unmasked; 1: masked
    struct Piece { int group; std::vector<int> partners; int accumulate; int kind; };
    std::vector<Piece> pieces;
    // (partner group, kind) -> the last own group that listed it: partners listed once, in the
    // order the group's tiles name them, in time linear in the tile count
    std::vector<int> listed(2 * (dq_side ? grp.kvg.size() : grp.qg.size()), -1);
    for (int gi = 0; gi < (int)own.size(); ++gi) {
      std::vector<int> full, other;  // partner groups of FULL pairs; of PARTIAL or EMPTY pairs
      for (int ti : own[gi]) {
        const int pg = dq_side ? grp.kv_of[ti] : grp.q_of[ti];
        const int kind = tile_cls[ti] == MA_TILE_FULL ? 0 : 1;
        if (listed[2 * pg + kind] == gi) continue;
        listed[2 * pg + kind] = gi;
        (kind == 0 ? full : other).push_back(pg);
      }
      bool first = true;
      for (int kind = 0; kind < 2; ++kind) {
        const auto& lst = kind == 0 ? full : other;
        for (size_t s0 = 0; s0 < lst.size(); s0 += kBwdPerLaunch) {
          Piece pc;
          pc.group = gi;
          pc.partners.assign(lst.begin() + s0, lst.begin() + std::min(lst.size(), s0 + kBwdPerLaunch));
          pc.accumulate = first ? (a->accumulate ? 1 : 0) : 1;
          pc.kind = kind;  // pieces have one-segment positions (expand_bwd_segments)
          first = false;
          pieces.push_back(pc);
        }
      }
    }
    // A group's pieces are consecutive in `pieces`; next_of[g] is the first of group g's pieces
    // that has not run (none: pieces.size()), the only one of them that may join a launch.
    std::vector<bool> done(pieces.size(), false);
    std::vector<size_t> next_of(own.size(), pieces.size());
    for (size_t pi = pieces.size(); pi-- > 0;) next_of[pieces[pi].group] = pi;
    size_t remaining = pieces.size(), first_open = 0;  // pieces before first_open have all run
    while (remaining > 0) {
      BwdParams p = base;
      std::vector<int> own_tab, part_tab, groups_in;
      int ne = 0, wg = 0, kind = -1;  // kind: mask kind of this launch, set by its first piece
      while (done[first_open]) ++first_open;
      for (size_t pi = first_open; pi < pieces.size() && ne < kBwdPerLaunch; ++pi) {
        if (done[pi]) continue;
        const Piece& pc = pieces[pi];
        if (std::find(groups_in.begin(), groups_in.end(), pc.group) != groups_in.end()) continue;
        // earlier pieces of this group must have run in an earlier launch
        if (next_of[pc.group] != pi) continue;
        if (kind >= 0 && kind != pc.kind) continue;
        std::vector<int> new_part = part_tab;
        for (int x : pc.partners)
          if (std::find(new_part.begin(), new_part.end(), x) == new_part.end()) new_part.push_back(x);
        const bool own_new = std::find(own_tab.begin(), own_tab.end(), pc.group) == own_tab.end();
        if ((int)new_part.size() > kBwdPerLaunch || (int)own_tab.size() + (own_new ? 1 : 0) > kBwdPerLaunch) continue;
        part_tab = new_part;
        if (own_new) own_tab.push_back(pc.group);
        groups_in.push_back(pc.group);
        kind = pc.kind;
        BwdEntry& en = p.entries[ne];
        en.self = (int32_t)(std::find(own_tab.begin(), own_tab.end(), pc.group) - own_tab.begin());
        en.n = (int32_t)pc.partners.size();
        for (int j = 0; j < en.n; ++j)
          en.partner[j] = (int32_t)(std::find(part_tab.begin(), part_tab.end(), pc.partners[j]) - part_tab.begin());
        en.accumulate = pc.accumulate;
        int64_t wgs;
        if (dq_side) {
          const int64_t nqb = (qparts[pc.group].sq + 31) / 32;
          en.chunks = (int32_t)((nqb * base.gmax + 7) / 8);
        } else {
          en.chunks = (int32_t)((kvparts[pc.group].sk + 127) / 128);
        }
        wgs = (int64_t)a->batch * a->hkv * en.chunks;
        wgs = (wgs + 7) / 8 * 8;  // keep each entry's first workgroup on XCD 0
        if (wg + wgs >= INT32_MAX) return set_error(MA_ERR_INVALID, "backward too large for one launch");
        en.wg_begin = wg;
        wg += (int)wgs;
        ++ne;
        done[pi] = true;
        next_of[pc.group] = pi + 1 < pieces.size() && pieces[pi + 1].group == pc.group ? pi + 1 : pieces.size();
        --remaining;
      }
      p.nentries = ne;
      p.mask = kind;
      for (size_t i = 0; i < own_tab.size(); ++i) {
        if (dq_side) p.qparts[i] = qparts[own_tab[i]];
        else p.kvparts[i] = kvparts[own_tab[i]];
      }
      for (size_t i = 0; i < part_tab.size(); ++i) {
        if (dq_side) p.kvparts[i] = kvparts[part_tab[i]];
        else p.qparts[i] = qparts[part_tab[i]];
      }
      rc = check_hip(dq_side ? launch_bwd_dq(p, a->head_dim, wg, stream) : launch_bwd_dkv(p, a->head_dim, wg, stream),
                     "tile_bwd launch");
      if (rc) return rc;
    }
  }
  return MA_OK;
}

}  // namespace
}  // namespace ma

extern "C" {

int mesh_attn_tile_bwd(const ma_tile_bwd_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_bwd(a);
  if (rc) return rc;
  if (a->ntiles == 0) return MA_OK;
  const size_t need = mesh_attn_tile_bwd_workspace_size(a);
  if (workspace_bytes < need || (need > 0 && !workspace) || ((uintptr_t)workspace & 255u))
    return set_error(MA_ERR_INVALID, "workspace missing, too small or not 256-byte aligned");
  return run_bwd(a, workspace, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The backward without any allocation.  Its only scratch buffer, the blocked LSE/D
// workspace, lives in this device array (one copy per GPU, held until the process
// ends).  In host code the name `scratch` is a host-side stand-in, never a device
// address: its device address is looked up once per device with
// hipGetSymbolAddress and only that pointer is handed to the kernels.
static __device__ __align__(256) unsigned char scratch[MA_BWD_NOALLOC_MAX_WORKSPACE];

namespace ma {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (the current device, which must be the
// stream's); looked up on the first call on each device.
int scratch_for_device(void* stream, void** out) {
  int dev = -1;
  int rc = check_hip((int)hipGetDevice(&dev), "hipGetDevice");
  if (rc) return rc;
  if (stream) {
    int sdev = -1;
    rc = check_hip((int)hipStreamGetDevice((hipStream_t)stream, &sdev), "hipStreamGetDevice");
    if (rc) return rc;
    if (sdev != dev) return set_error(MA_ERR_INVALID, "the stream belongs to another device than the current one");
  }
  if (dev < 0 || dev >= kMaxDevices) return set_error(MA_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    rc = check_hip((int)hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (rc) return rc;
    if (!ptr || ((uintptr_t)ptr & 255u)) return set_error(MA_ERR_LAUNCH, "scratch array has no usable device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MA_OK;
}

}  // namespace
}  // namespace ma

extern "C" {

int mesh_attn_tile_bwd_noalloc(const ma_tile_bwd_args* a, void* stream) {
  int rc = validate_bwd(a);
  if (rc) return rc;
  if (a->ntiles == 0) return MA_OK;
  const size_t need = mesh_attn_tile_bwd_workspace_size(a);
  if (need > (size_t)MA_BWD_NOALLOC_MAX_WORKSPACE) {
    std::string m = "this backward needs " + std::to_string(need) + " bytes of workspace; the built-in scratch holds " +
                    std::to_string((size_t)MA_BWD_NOALLOC_MAX_WORKSPACE) + " (use mesh_attn_tile_bwd with a workspace)";
    return set_error(MA_ERR_INVALID, m.c_str());
  }
  void* ws = nullptr;
  rc = scratch_for_device(stream, &ws);
  if (rc) return rc;
  return run_bwd(a, ws, stream);
}

}  // extern "C"
