// Internal declarations shared by the ABI layer and the kernels (not installed).
#pragma once
#include <cstdint>
#include <cstddef>

#include "mesh_attn.h"

namespace ma {

// ---- error reporting (thread-local message, see mesh_attn_last_error) ----
int set_error(int code, const char* msg);

// ---- position helpers (host) ----
bool pos_valid(const ma_pos* p, int64_t len, const char** why);
int64_t pos_at(const ma_pos* p, int64_t t);
void pos_minmax(const ma_pos* p, int64_t len, int64_t u0, int64_t u1, int64_t* mn, int64_t* mx);

// ---- compact positions as the kernels see them (validated to fit in int32) ----
struct KPos {
  int32_t nseg;
  int32_t lb[MA_MAX_SEGMENTS];  // local_begin
  int32_t gb[MA_MAX_SEGMENTS];  // global_begin
  int32_t st[MA_MAX_SEGMENTS];  // stride
};

// ---- tile forward ----
constexpr int kFwdTilesPerLaunch = 30;
constexpr int32_t kFwdChained = 2;  // FwdTile::accumulate flag of a chained key segment

struct FwdTile {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int32_t sq, sk;
  int32_t wg_begin;    // first workgroup of this tile in the launch
  int32_t chunks;      // workgroup chunks per (batch, kv head)
  int32_t accumulate;  // bit 0: fold into the (O, LSE) held by the output buffers; kFwdChained:
                       // continues the previous entry (same rows and output, next key segment)
  int32_t kgb, kst;    // key positions, one segment: global = kgb + kst * t (the host chains the others)
  KPos qp;
};

struct FwdParams {
  int32_t ntiles;
  int32_t batch, hq, hkv;
  int32_t mask;           // 0 none; 1 causal, one key segment per tile
  int32_t gmax;           // largest number of query heads sharing one KV head
  float scale;            // softmax scale
  float scale_log2;       // scale * log2(e)
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t l_sb, l_sh;
  uint8_t heads_of[MA_MAX_HEADS];      // query heads ordered by KV head
  uint8_t kv_first[MA_MAX_HEADS + 1];  // start of each KV head's run in heads_of
  FwdTile tiles[kFwdTilesPerLaunch];
  // A resident-KV launch from a tile table in device memory (table != nullptr; tiles[] unused):
  // the table's tiles, group entries and workgroup records, the launch's first workgroup record,
  // and what the table's header must hold for the launch to run (the kernel checks it before
  // anything else).
  const struct FwdTableHeader* table_header;
  const FwdTile* table;
  const struct FwdResEnt* res_ents;
  const struct FwdResWg* res_wgs;
  int32_t wg_base;
  int32_t table_ntiles;
  int32_t table_nents;
  int32_t table_nwgs;
  uint64_t table_hash;
};

// Tile table in device memory (mesh_attn_tile_fwd_pack / mesh_attn_tile_fwd_tabled): this
// header, then the resident-KV tiles (FwdTile, in call order), then the group entries
// (FwdResEnt), then one record per workgroup (FwdResWg).  Tiles with the same K and V (pointers
// and length) form a group, whose workgroups share one LDS copy of K/V per (batch, KV head).
// A tile's units are (32-row block, head slot of the KV head's group of gmax slots), numbered
// block-major; units are numbered across the whole table, group after group, so each entry's
// unit0 is larger than the one before.  hash is FNV-1a (64-bit) taken over the tiles, entries
// and records as 64-bit words.
constexpr uint32_t kFwdTableMagic = 0x5441424du;  // "MBAT"
struct FwdTableHeader {
  uint32_t magic;
  int32_t ntiles;
  int32_t nwgs;
  int32_t nents;
  uint64_t hash;
  uint64_t reserved;
};
struct FwdResEnt {
  int32_t tile;   // index into the table's tiles
  int32_t unit0;  // the tile's first unit
};
struct FwdResWg {
  int32_t ent;      // the entry holding unit u_begin (the group's K/V are its tile's)
  int32_t u_begin;  // units [u_begin, u_end) of the group, unit u to wave u % 8
  int32_t u_end;
  int32_t bk;       // batch * hkv + KV head
};
static_assert(sizeof(FwdTableHeader) == 32 && sizeof(FwdTile) % 8 == 0 && sizeof(FwdResEnt) == 8 &&
                  sizeof(FwdResWg) == 16,
              "table layout");

// launchers (return hipError_t as int)
static_assert(sizeof(FwdParams) <= 4096, "forward parameters exceed the kernel-argument limit");
// bf16 forward: waves = 8 (five-stage ring, one workgroup per CU) or 4 (two-stage ring,
// two workgroups per CU; for tiles of at most kFwdSmallBlocks key blocks)
constexpr int kFwdSmallBlocks = 16;
int launch_fwd_bf16(const FwdParams& p, int head_dim, int waves, int total_wgs, void* stream);
// bf16 forward with the whole K and V of a tile resident in LDS, for unmasked tiles of
// kFwdResMinKeys<D> < sk <= kFwdResKeys<D> keys; a workgroup of 8 waves runs up to kFwdResUnits
// units of (32 query rows, query head) of one (tile, batch, KV head), or from a tile table
// kFwdResUnits to kFwdResUnitsMax units of a group of tiles sharing K/V
template <int D>
constexpr int kFwdResKeys = D == 128 ? 256 : 512;
template <int D>
constexpr int kFwdResMinKeys = D == 128 ? 128 : 0;
constexpr int kFwdResUnits = 32;
constexpr int kFwdResUnitsMax = 128;
int launch_fwd_bf16_resident(const FwdParams& p, int head_dim, int total_wgs, void* stream);
int launch_fwd_f32(const FwdParams& p, int head_dim, int total_wgs, void* stream);
int launch_fill_empty(void* o, float* lse, int dtype, int batch, int sq, int hq, int head_dim,
                      int64_t o_sb, int64_t o_ss, int64_t o_sh, int64_t l_sb, int64_t l_sh, void* stream);

// ---- merge ----
struct MergeParams {
  int32_t k;
  int32_t batch, seqlen, heads;
  int64_t o_sb, o_ss, o_sh;
  int64_t l_sb, l_sh;
  void* o_out;
  float* lse_out;
  const void* o_in[MA_MAX_MERGE];
  const float* lse_in[MA_MAX_MERGE];
};
int launch_merge(const MergeParams& p, int dtype, int head_dim, void* stream);

// ---- add-reduce ----
struct ReduceParams {
  int32_t k;
  int64_t n;
  float* out;
  const float* in[MA_MAX_MERGE];
};
int launch_reduce_add(const ReduceParams& p, void* stream);

// ---- backward ----
// The backward runs per (Q partition, KV partition) pair ([Mesh] section 3.5).
// Tiles sharing a dq buffer form a Q group (same Q partition), tiles sharing a
// dk/dv buffer form a KV group.  The dQ kernel takes one Q group per work entry
// and walks all its KV partitions; the dK/dV kernel takes one KV group per
// entry and walks all its Q partitions; neither needs atomics.
constexpr int kBwdPerLaunch = 8;

struct BwdQPart {        // a Q partition and its dq buffer
  const void* q;
  const void* dout;
  const float* lsed;     // workspace: per (b, h, 64-row block) [LSE*log2(e) x 64, D x 64] fp32
  float* dq;
  int32_t sq;
  KPos qp;
};

struct BwdKVPart {       // a KV partition and its dk, dv buffers
  const void* k;
  const void* v;
  float* dk;
  float* dv;
  int32_t sk;
  KPos kp;
};

struct BwdEntry {        // one group: its own partition and the partner partitions it meets
  int32_t self;          // index into qparts (dQ launch) or kvparts (dK/dV launch)
  int32_t n;             // number of partners
  int32_t partner[kBwdPerLaunch];
  int32_t wg_begin;      // first workgroup of this entry in the launch
  int32_t chunks;        // workgroups per (batch, KV head)
  int32_t accumulate;    // add to the output buffers instead of overwriting
};

struct BwdParams {
  int32_t nentries;
  int32_t batch, hq, hkv, gmax;
  int32_t mask;  // 0 none; 1 causal, positions of one segment on both sides
  float scale, scale_log2;
  int64_t q_sb, q_ss, q_sh;    // q, o, dout
  int64_t k_sb, k_ss, k_sh;    // k, v
  int64_t dq_sb, dq_ss, dq_sh;
  int64_t dk_sb, dk_ss, dk_sh;
  uint8_t heads_of[MA_MAX_HEADS];
  uint8_t kv_first[MA_MAX_HEADS + 1];
  BwdQPart qparts[kBwdPerLaunch];
  BwdKVPart kvparts[kBwdPerLaunch];
  BwdEntry entries[kBwdPerLaunch];
};
static_assert(sizeof(BwdParams) <= 4096, "backward parameters exceed the kernel-argument limit");

// LSE*log2(e) (+inf for rows without an allowed key) and D = rowsum(dO*O) of a Q
// partition, in the blocked layout the main kernels stage into LDS.
struct BwdPreParams {
  int32_t batch, hq, sq;
  float scale;
  const void* o;
  const void* dout;
  const float* lse;
  float* lsed;
  int64_t q_sb, q_ss, q_sh;
  int64_t l_sb, l_sh;
};
int launch_bwd_preprocess(const BwdPreParams& p, int head_dim, void* stream);
int launch_bwd_dq(const BwdParams& p, int head_dim, int total_wgs, void* stream);
int launch_bwd_dkv(const BwdParams& p, int head_dim, int total_wgs, void* stream);

}  // namespace ma
