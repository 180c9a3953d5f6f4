/*
 * mesh_attn.h - C ABI of the MI355X (gfx950) attention-tile library.
 *
 * One GPU's share of the Q-KV assignment matrix of distributed attention:
 *   - mesh_attn_tile_fwd : exact attention of (Q partition, KV partition) tiles,
 *                          each emitting a partial output O and a per-row LSE
 *                          (mesh_attn_tile_fwd_tabled: the same with the tile
 *                          table in device memory, for thousands of small tiles);
 *   - mesh_attn_merge    : the LSE-based merge that folds k partial (O, LSE)
 *                          pairs of one Q partition into its output;
 *   - mesh_attn_tile_bwd : the matching backward (dQ, dK, dV from O, LSE, dO);
 *   - host-only mapper   : Mesh tiles with KV partition rotation, Q/KV groups,
 *                          zigzag and striped token positions, tile classes.
 *
 * Sources, cited by title and section:
 *   [Mesh]   "Mesh-Attention: A New Communication-Efficient Distributed Attention
 *             with Improved Data Locality" (arXiv 2512.20968)
 *   [CHARM+] "CHARM+: Cross-Hardware Attention with Re-Merge Multistream
 *             Mechanism" (arXiv 2611.05906v1)
 *   [Ring]   "Ring Attention and Context Parallelism: How Long-Context LLMs Are
 *             Trained Across GPUs"
 *
 * Conventions for every call:
 *   - Return value: MA_OK (0) or an MA_ERR_* code; no call aborts or throws.
 *     mesh_attn_last_error() returns a message for the calling thread's last error.
 *   - Device pointers are borrowed for the work enqueued on `stream` (a
 *     hipStream_t passed as void*, NULL = the default stream); the caller keeps
 *     them alive until the stream reaches that point.  Calls are asynchronous
 *     and never synchronise the device.  Host arrays (tile lists, head maps,
 *     pointer lists) are read before the call returns.
 *   - The library allocates no device memory and keeps no state between calls,
 *     except for mesh_attn_tile_bwd_noalloc's scratch array (a static device
 *     array, one per GPU) and the table of its device addresses.
 *   - Every argument is checked before anything is enqueued, so a call that
 *     returns MA_ERR_INVALID or MA_ERR_UNSUPPORTED has enqueued nothing.  A call
 *     that returns MA_ERR_LAUNCH (the runtime refused a launch) may have
 *     enqueued the launches before it.
 *   - Layouts: Q, O, dO are [B, S, Hq, d]; K, V are [B, S, Hkv, d]; LSE is
 *     [B, Hq, S] float32 (natural log).  Strides are in ELEMENTS; the d axis
 *     (and the S axis of LSE) must have stride 1.  bf16 tensors need 16-byte
 *     aligned base pointers and strides that are multiples of 8 elements;
 *     fp32 tensors 16-byte aligned bases and strides multiple of 4.
 *   - Head map: query head h reads KV head head_map[h] (host array of Hq
 *     entries).  NULL means groups of Hq/Hkv consecutive query heads share one
 *     KV head, kv(h) = h / (Hq/Hkv) ([Mesh] section 4.8, GQA).
 *   - Masks act on GLOBAL token positions ([Ring], "Gotchas": masks must use
 *     global positions): key u is allowed for query t iff pos_k(u) <= pos_q(t)
 *     ([Mesh] section 3.7; [Ring] "Causal masks and load balancing").  A query
 *     row with no allowed key gets O = 0 and LSE = -inf, never NaN.
 */
#ifndef MESH_ATTN_H
#define MESH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MA_VERSION 1

/* status codes */
#define MA_OK 0
#define MA_ERR_INVALID 1      /* bad argument: null pointer, size <= 0, out-of-range map, ... */
#define MA_ERR_UNSUPPORTED 2  /* valid but not implemented: head_dim not 64/128, fp32 backward, ... */
#define MA_ERR_LAUNCH 3       /* the HIP runtime reported an error while enqueueing */

/* element types */
#define MA_F32 0
#define MA_BF16 1

/* mask modes */
#define MA_MASK_NONE 0            /* every key allowed; positions ignored */
#define MA_MASK_CAUSAL 1          /* causal; q_pos and k_pos must each be ONE segment of stride 1 */
#define MA_MASK_STRIPED_ZIGZAG 2  /* causal; up to MA_MAX_SEGMENTS segments of any stride >= 1
                                     (zigzag shares = 2 contiguous segments, [Ring] "Causal masks
                                     and load balancing"; striped = stride N, [Mesh] section 3.7) */

/* tile classes ([Mesh] section 3.7: masked, triangular, dense pairs) */
#define MA_TILE_EMPTY 0    /* no (query, key) pair allowed */
#define MA_TILE_PARTIAL 1  /* some allowed */
#define MA_TILE_FULL 2     /* all allowed */

#define MA_MAX_SEGMENTS 4
#define MA_MAX_MERGE 64
#define MA_MAX_HEADS 128
#define MA_MAX_TILES 4096

/*
 * Token positions of a partition.  Segment s covers local indices
 * [local_begin_s, local_begin_{s+1}) (the last runs to the partition end); local
 * index t in it has global position global_begin_s + (t - local_begin_s)*stride_s.
 * Segments are given in increasing local_begin order, the first at 0; strides
 * are >= 1; every position must lie in [0, 2^31 - 1).  Contiguous partition =
 * one segment of stride 1; zigzag share = two segments; striped rank r of N =
 * one segment {0, r, N}.
 */
typedef struct {
  int64_t local_begin;
  int64_t global_begin;
  int64_t stride;
} ma_segment;

typedef struct {
  int32_t nseg; /* 1..MA_MAX_SEGMENTS; ignored under MA_MASK_NONE */
  int32_t reserved;
  ma_segment seg[MA_MAX_SEGMENTS];
} ma_pos;

/* ---------------------------------------------------------------------------
 * Tile forward.  [Mesh] section 2.2: one (Q_i, KV_j) pair yields
 * (O_ij, lse_ij) = Attention(Q_i, K_j, V_j); [Mesh] section 2.1 softmax
 * attention; [CHARM+] appendix A, Algorithm 2 (CompAttention).
 *
 * For each tile, batch b and query head h, query row t:
 *   s[t,u] = scale * q[t] . k[u]   over keys u of KV head head_map[h]
 *   LSE[t] = ln sum_{u allowed} exp(s[t,u])
 *   O[t]   = sum_{u allowed} exp(s[t,u] - LSE[t]) v[u]
 * Accumulation is fp32; bf16 O is rounded to nearest even at the store.
 * accumulate = 0: every tile writes its own (O, LSE) over its whole [sq] range.
 * A tile that is EMPTY under the mask is not computed: its O is filled with 0
 * and its LSE with -inf (callers normally leave EMPTY tiles out; see
 * mesh_attn_classify).
 * accumulate = 1: the tile's result is folded into the (O, LSE) pair already
 * held by its o and lse buffers, the running update of [Mesh] section 2.2 and
 * of [CHARM+] appendix A, Algorithm 2 (CompAttention updates out in place):
 *   L = ln(exp(lse_old) + exp(lse_tile));
 *   O = exp(lse_old - L) O_old + exp(lse_tile - L) O_tile;
 * with (0, -inf) when both are -inf.  The buffers must hold a valid pair (for
 * example the first tile's output, or O = 0 and LSE = -inf); EMPTY tiles leave
 * them unchanged.  The arithmetic is fp32 and O is rounded once, at the store;
 * this holds too for a tile whose key positions have several segments (in bf16
 * its segments are computed in turn by one workgroup, the softmax state carried
 * in fp32 between them).
 * In either mode, tiles of one call that name the same o are applied in list
 * order (each waits for the one before), so a ring of KV partitions can be
 * handed over as one call.  Outputs of different tiles that are one buffer
 * shifted along the sequence axis by fewer rows than the earlier view holds are
 * rejected (MA_ERR_INVALID); other partial overlaps between different outputs,
 * and outputs that alias inputs, are undefined.
 * --------------------------------------------------------------------------- */
typedef struct {
  const void* q;  /* device, [B, sq, Hq, d], dtype */
  const void* k;  /* device, [B, sk, Hkv, d], dtype */
  const void* v;  /* device, [B, sk, Hkv, d], dtype */
  void* o;        /* device, [B, sq, Hq, d], dtype (written) */
  float* lse;     /* device, [B, Hq, sq] float32 (written) */
  int64_t sq;     /* >= 1 */
  int64_t sk;     /* >= 1 */
  ma_pos q_pos;
  ma_pos k_pos;
} ma_tile;

typedef struct {
  int32_t dtype;      /* MA_BF16 or MA_F32 (inputs and O) */
  int32_t batch;      /* B >= 1 */
  int32_t hq;         /* 1..MA_MAX_HEADS */
  int32_t hkv;        /* 1..hq */
  int32_t head_dim;   /* 64 or 128 */
  int32_t mask_mode;  /* MA_MASK_* */
  float scale;        /* softmax scale, e.g. 1/sqrt(d) ([Mesh] section 2.1) */
  int32_t ntiles;     /* 0..MA_MAX_TILES (0 is a no-op) */
  int32_t accumulate; /* 0: write (O, LSE); 1: fold into the (O, LSE) held by the buffers */
  int32_t reserved;   /* 0 */
  const int32_t* head_map;  /* host, hq entries in [0, hkv), or NULL */
  const ma_tile* tiles;     /* host array of ntiles */
  int64_t q_stride[3];      /* b, s, h (elements) - shared by all tiles */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  int64_t lse_stride[2];    /* b, h */
} ma_tile_fwd_args;

int mesh_attn_tile_fwd(const ma_tile_fwd_args* args, void* stream);

/* ---------------------------------------------------------------------------
 * Tile forward with a tile table in device memory, for calls of many small
 * tiles: at [CHARM+]'s smallest partition sizes (its scaling table, 13440
 * tokens over 64 partitions: tiles of 210 tokens) one GPU's share is thousands
 * of tiles.  mesh_attn_tile_fwd hands tiles to the kernels in kernel arguments,
 * a few dozen per launch; here the tiles of its resident-KV class (unmasked bf16
 * tiles of 129-256 keys at d = 128, of at most 512 keys at d = 64) run from a
 * table in device memory, all in one launch (one more wherever a tile names the
 * output of a tile before it), and every other tile as in mesh_attn_tile_fwd.
 * Tiles with the same K and V (pointers and length), such as the tiles of one
 * KV partition in a Mesh share ([Mesh] section 3.1), share one copy of K/V per
 * workgroup.  Results, accumulate mode, output ordering and argument checks are
 * those of mesh_attn_tile_fwd on the same arguments, bit for bit.
 *
 * mesh_attn_tile_fwd_table_bytes: the table's size for these arguments (at
 *   least 32 bytes; 0 when the arguments are invalid, see mesh_attn_last_error).
 * mesh_attn_tile_fwd_pack: checks the arguments as mesh_attn_tile_fwd does and
 *   writes the table into host memory `table` of `bytes` >= that size (host
 *   only; nothing is enqueued).  The caller copies it to device memory, for
 *   example through pinned memory on the stream of the launch.
 * mesh_attn_tile_fwd_tabled: the forward, with `table` (device, 16-byte
 *   aligned, `bytes` >= the size above) holding what mesh_attn_tile_fwd_pack
 *   wrote for the same arguments by the time the stream reaches the call, and
 *   unchanged until the launch has run.  The table holds the tiles' device
 *   pointers, so the library checks it in the kernel: its header must carry the
 *   tile, group-entry and workgroup counts and the 64-bit hash planned for these
 *   arguments, or
 *   the resident-KV launch returns without reading the tiles or writing any
 *   output (a table packed for other arguments is not run).  Ownership and
 *   errors as in mesh_attn_tile_fwd; the table is the caller's memory.
 * --------------------------------------------------------------------------- */
size_t mesh_attn_tile_fwd_table_bytes(const ma_tile_fwd_args* args);
int mesh_attn_tile_fwd_pack(const ma_tile_fwd_args* args, void* table, size_t bytes);
int mesh_attn_tile_fwd_tabled(const ma_tile_fwd_args* args, const void* table, size_t bytes, void* stream);

/* ---------------------------------------------------------------------------
 * LSE merge.  [Mesh] section 2.2 (online softmax rescales partial outputs by
 * their LSE), section 3.3 (online softmax as the reduce-scatter reducer);
 * [CHARM+] appendix A, Algorithm 2 (CommAndUpdate); [Ring] "Ring Attention:
 * Pass KV Blocks Around the Ring".  For each (b, h, t):
 *   L* = max_r lse_r;  lse = L* + ln sum_r exp(lse_r - L*);
 *   O  = sum_r exp(lse_r - lse) * O_r;   all lse_r = -inf -> (0, -inf).
 * Math in fp32; bf16 O rounded to nearest even.  o_out may equal o_in[0] and
 * lse_out may equal lse_in[0] (in place); other overlaps are undefined.
 * --------------------------------------------------------------------------- */
typedef struct {
  int32_t dtype;      /* MA_BF16 or MA_F32 (all O tensors) */
  int32_t batch;      /* >= 1 */
  int32_t seqlen;     /* S >= 1 */
  int32_t heads;      /* H >= 1 */
  int32_t head_dim;   /* 64 or 128 */
  int32_t k;          /* 1..MA_MAX_MERGE partials */
  const void* const* o_in;     /* host array of k device pointers, [B, S, H, d] */
  const float* const* lse_in;  /* host array of k device pointers, [B, H, S] */
  void* o_out;                 /* device, [B, S, H, d] */
  float* lse_out;              /* device, [B, H, S] */
  int64_t o_stride[3];         /* b, s, h - shared by inputs and output */
  int64_t lse_stride[2];       /* b, h */
} ma_merge_args;

int mesh_attn_merge(const ma_merge_args* args, void* stream);

/* ---------------------------------------------------------------------------
 * Add-reduce of partial gradients.  [Mesh] section 3.5: the partial dQ_i and
 * dKV_j of the per-pair backward calls are summed across the GPUs that hold
 * them (a reduce-scatter with addition); this is the per-GPU summation step
 * of that reduce: out[e] = sum_r in_r[e] for e < n, in fp32, added in the
 * order r = 0, 1, ..., k-1 (the same bits on every call).  Every pointer is
 * 16-byte aligned; out may equal in[0] (in place), other overlaps are
 * undefined.  n = 0 is a no-op.
 * --------------------------------------------------------------------------- */
typedef struct {
  int32_t k;               /* 1..MA_MAX_MERGE inputs */
  int32_t reserved;        /* 0 */
  int64_t n;               /* float32 elements per input, >= 0 */
  const float* const* in;  /* host array of k device pointers */
  float* out;              /* device, n floats */
} ma_reduce_args;

int mesh_attn_reduce_add(const ma_reduce_args* args, void* stream);

/* ---------------------------------------------------------------------------
 * Tile backward.  [Mesh] section 3.5: the backward kernel runs per pair with
 * (Q_i, KV_j, O_i, dO_i) and its partial dQ_i, dKV_j are accumulated locally
 * with addition.  The pages print no formula; this is the derivative of the
 * forward with P = exp(s - LSE) on allowed entries:
 *   D[t] = dO[t].O[t];  dS = P (dO[t].v[u] - D[t]);
 *   dQ[t] = scale sum_u dS k[u];  dK[u] = scale sum dS q[t];  dV[u] = sum P dO[t],
 * dK/dV summed over the query heads that read the KV head and over every tile
 * in the call that names the same dk/dv buffers.  O and LSE may be the row's
 * FINAL values over a larger KV set (the distributed case); then the outputs
 * are this KV partition's share.
 *
 * accumulate = 0: dq, dk, dv are overwritten; = 1: the results are added to
 * what the buffers hold.  All tiles naming the same dk (or dv) buffer must name
 * the same k and v buffers and sk.  dq (dk, dv) buffers of different tiles
 * must not overlap unless they are identical (then contributions add): one
 * buffer shifted along the sequence axis by fewer rows than the earlier view
 * holds is rejected (MA_ERR_INVALID), other partial overlaps are undefined.
 * bf16 only.  The workspace (device, >= mesh_attn_tile_bwd_workspace_size
 * bytes, 256-byte aligned) holds D and per-call scratch; its contents on entry
 * do not matter.  mesh_attn_tile_bwd_workspace_size returns 0 for arguments it
 * cannot size (no tiles, sizes out of range, invalid positions under a mask).
 * --------------------------------------------------------------------------- */
typedef struct {
  const void* q;     /* device bf16 [B, sq, Hq, d] */
  const void* k;     /* device bf16 [B, sk, Hkv, d] */
  const void* v;     /* device bf16 [B, sk, Hkv, d] */
  const void* o;     /* device bf16 [B, sq, Hq, d] */
  const void* dout;  /* device bf16 [B, sq, Hq, d] */
  const float* lse;  /* device float32 [B, Hq, sq] */
  float* dq;         /* device float32 [B, sq, Hq, d] */
  float* dk;         /* device float32 [B, sk, Hkv, d] */
  float* dv;         /* device float32 [B, sk, Hkv, d] */
  int64_t sq;
  int64_t sk;
  ma_pos q_pos;
  ma_pos k_pos;
} ma_bwd_tile;

typedef struct {
  int32_t dtype;      /* MA_BF16 */
  int32_t batch;
  int32_t hq;
  int32_t hkv;
  int32_t head_dim;   /* 64 or 128 */
  int32_t mask_mode;
  float scale;
  int32_t ntiles;
  int32_t accumulate;
  int32_t reserved;
  const int32_t* head_map;     /* host or NULL */
  const ma_bwd_tile* tiles;    /* host array */
  int64_t q_stride[3];         /* q, o, dout share these (b, s, h) */
  int64_t k_stride[3];         /* k and v share these */
  int64_t dq_stride[3];        /* float32 dq */
  int64_t dk_stride[3];        /* float32 dk and dv share these */
  int64_t lse_stride[2];       /* b, h */
} ma_tile_bwd_args;

size_t mesh_attn_tile_bwd_workspace_size(const ma_tile_bwd_args* args);
int mesh_attn_tile_bwd(const ma_tile_bwd_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Tile backward that allocates nothing, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, validation and results as
 * mesh_attn_tile_bwd, but the workspace is a scratch array built into the
 * library: MA_BWD_NOALLOC_MAX_WORKSPACE bytes on each GPU the library runs on,
 * held until the process ends.  A call whose mesh_attn_tile_bwd_workspace_size
 * exceeds that size returns MA_ERR_INVALID without enqueueing anything.  The
 * stream must belong to the current device.  No hipMalloc/hipFree or allocating
 * library call is made; the first call on a device looks up the array's device
 * address.  All calls on one GPU share its array (nothing in it needs clearing:
 * each call writes every byte it reads), so calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race.
 * --------------------------------------------------------------------------- */
#define MA_BWD_NOALLOC_MAX_WORKSPACE (32u << 20) /* bytes: 8 Q partitions of 16384 rows x 32 heads */
int mesh_attn_tile_bwd_noalloc(const ma_tile_bwd_args* args, void* stream);

/* ---------------------------------------------------------------------------
 * Host-only mapper.  Pure functions: no device work, no allocation; output
 * arrays are caller-sized.  Return MA_OK or MA_ERR_INVALID.
 * --------------------------------------------------------------------------- */

/* [Mesh] sections 3.2-3.3: GPU g of n = a*b computes Q partitions
 * r*a .. r*a+a-1 (r = g / a) against KV partitions c*b .. c*b+b-1 (basic, kvr=0)
 * or {c + t*a : 0 <= t < b} (KV partition rotation, kvr=1), c = g mod a.
 * q_parts gets a entries, kv_parts b entries (tile order). */
int mesh_attn_map_mesh_tile(int32_t n, int32_t a, int32_t b, int32_t g, int32_t kvr,
                            int32_t* q_parts, int32_t* kv_parts);

/* [Mesh] section 3.3: Q group {r*a + x : x < a} and KV group {c + a*x : x < b} of GPU g. */
int mesh_attn_map_groups(int32_t n, int32_t a, int32_t b, int32_t g,
                         int32_t* q_group, int32_t* kv_group);

/* [Ring] "Causal masks and load balancing": with 2N chunks, rank r holds chunks r and 2N-1-r. */
int mesh_attn_map_zigzag(int32_t N, int32_t r, int32_t chunks[2]);

/* Position descriptors: contiguous partition starting at global_begin; zigzag share
 * of rank r (two chunks of chunk_len tokens); striped rank r of N (positions r + N*t). */
int mesh_attn_pos_contiguous(int64_t global_begin, ma_pos* out);
int mesh_attn_pos_zigzag(int32_t N, int32_t r, int64_t chunk_len, ma_pos* out);
int mesh_attn_pos_striped(int32_t N, int32_t r, ma_pos* out);

/* Global position of local index t (t in [0, length)); -1 on invalid input. */
int64_t mesh_attn_pos_at(const ma_pos* pos, int64_t t);

/* Class of a (Q partition, KV partition) pair under mask_mode: MA_TILE_EMPTY,
 * MA_TILE_PARTIAL or MA_TILE_FULL (MA_MASK_NONE always FULL); negative
 * (-MA_ERR_INVALID) on invalid input. */
int mesh_attn_classify(const ma_pos* q_pos, int64_t sq, const ma_pos* k_pos, int64_t sk, int32_t mask_mode);

/* Exact number of allowed (query, key) pairs of the pair (per head); -1 on invalid input. */
int64_t mesh_attn_count_allowed(const ma_pos* q_pos, int64_t sq, const ma_pos* k_pos, int64_t sk,
                                int32_t mask_mode);

/* Non-EMPTY pairs among nq Q partitions x nk KV partitions (row-major scan).
 * Writes up to max_out entries of (q index, kv index, class) into out_q, out_k,
 * out_class and returns the number of non-EMPTY pairs (may exceed max_out),
 * or -1 on invalid input. */
int32_t mesh_attn_build_worklist(int32_t nq, const ma_pos* q_pos, const int64_t* sq,
                                 int32_t nk, const ma_pos* k_pos, const int64_t* sk,
                                 int32_t mask_mode, int32_t max_out,
                                 int32_t* out_q, int32_t* out_k, int32_t* out_class);

/* ---------------------------------------------------------------------------
 * GOO step planner (host only).  [Mesh] section 3.4 (2-D Greedy Overlapping
 * Optimization): the Q partitions of a GPU's tile are cut into k_q chunks and
 * the KV partitions into k_kv chunks, giving communication tasks AG-Q-i, RS-Q-i
 * (i < k_q), AG-KV-j (j < k_kv) and compute tasks C-i-j.  C-i-j is ready when
 * AG-Q-i and AG-KV-j are done, RS-Q-i when every C-i-j is done.  Each step runs
 * one communication task with compute tasks that were ready when it began, and
 * finishes before the next.  The communication task is the candidate with the
 * largest profit = (compute time it makes ready) / (its own time); candidates
 * are the lowest-index unscheduled chunk of each type (RS-Q once ready), ties
 * go to AG-KV, then AG-Q, then RS-Q.  Ready compute tasks join in (i, j) order
 * while their summed time is below gamma * (the step's communication time).
 * With no communication task possible and computation ready, a compute-only step
 * runs one ready task.  Deterministic: every GPU given the same costs gets the
 * same schedule, as the section requires.
 *
 * Returns the number of steps written (at most 2 k_q + k_kv + k_q k_kv), or
 * -MA_ERR_INVALID (k_q, k_kv < 1 or k_q k_kv > MA_GOO_MAX_COMPUTE, a
 * communication time <= 0, a compute time or gamma < 0 or not finite, null
 * pointers, max_steps too small).  No allocation; t_c and steps are host arrays.
 * --------------------------------------------------------------------------- */
#define MA_GOO_MAX_COMPUTE 16
#define MA_GOO_NONE 0   /* compute-only step */
#define MA_GOO_AG_Q 1
#define MA_GOO_AG_KV 2
#define MA_GOO_RS_Q 3

typedef struct {
  int32_t comm_type;   /* MA_GOO_* */
  int32_t comm_index;  /* chunk index of the communication task (0 in a compute-only step) */
  int32_t ncompute;    /* compute tasks in the step */
  int32_t compute[MA_GOO_MAX_COMPUTE];  /* C-i-j written as i * k_kv + j, in the order taken */
} ma_goo_step;

int32_t mesh_attn_goo_plan(int32_t k_q, int32_t k_kv, double t_ag_q, double t_ag_kv, double t_rs_q,
                           const double* t_c, double gamma, int32_t max_steps, ma_goo_step* steps);

/* diagnostics */
const char* mesh_attn_last_error(void);
int mesh_attn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MESH_ATTN_H */
