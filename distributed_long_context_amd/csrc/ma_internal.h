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
constexpr int kFwdTilesPerLaunch = 8;

struct FwdTile {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int32_t sq, sk;
  int32_t wg_begin;  // first workgroup of this tile in the launch
  int32_t chunks;    // workgroup chunks per (batch, kv head)
  KPos qp, kp;
};

struct FwdParams {
  int32_t ntiles;
  int32_t batch, hq, hkv;
  int32_t mask;           // 0 none, 1 causal on positions
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
};

// launchers (return hipError_t as int)
int launch_fwd_bf16(const FwdParams& p, int head_dim, int total_wgs, void* stream);
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

// ---- backward ----
constexpr int kBwdTilesPerLaunch = 8;

struct BwdTile {
  const void* q;
  const void* o;
  const void* dout;
  const float* lse;
  float* dq;
  float* dscratch;  // D = rowsum(dO*O), [B, Hq, sq] float32 in the workspace
  int32_t sq;
  int32_t zero_dq;  // clear dq in the preprocessing pass (overwrite mode)
  KPos qp;
};

struct BwdKV {  // one KV partition with the tiles that read it
  const void* k;
  const void* v;
  float* dk;
  float* dv;
  int32_t sk;
  int32_t ntiles;
  int32_t wg_begin;    // first workgroup of this KV partition in the launch
  int32_t accumulate;  // add dK/dV to the buffers instead of overwriting
  int32_t tile_idx[kBwdTilesPerLaunch];
  KPos kp;
};

struct BwdParams {
  int32_t nkv, ntiles;
  int32_t batch, hq, hkv, gmax;
  int32_t mask;
  int32_t accumulate;
  float scale, scale_log2;
  int64_t q_sb, q_ss, q_sh;    // q, o, dout
  int64_t k_sb, k_ss, k_sh;    // k, v
  int64_t dq_sb, dq_ss, dq_sh;
  int64_t dk_sb, dk_ss, dk_sh;
  int64_t l_sb, l_sh;
  uint8_t heads_of[MA_MAX_HEADS];
  uint8_t kv_first[MA_MAX_HEADS + 1];
  BwdTile tiles[kBwdTilesPerLaunch];
  BwdKV kvs[kBwdTilesPerLaunch];
};
int launch_bwd_preprocess(const BwdParams& p, int head_dim, void* stream);
int launch_bwd_main(const BwdParams& p, int head_dim, int total_wgs, void* stream);

}  // namespace ma
