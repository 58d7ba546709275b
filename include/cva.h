/*
 * cva.h -- C ABI of libcva: one context-parallel rank's share of packed
 * variable-length (THD) attention with online softmax, for AMD MI355X (gfx950).
 *
 * The operation (MindSpeed RFC "EOD-aware load balancing for KVAllGather CP
 * with THD", gitcode Ascend/MindSpeed issue 232):
 *   - every EOD sub-sequence of a packed batch is cut into 2*cp_size equal
 *     chunks and rank r holds chunks r and 2*cp_size-r-1 (section 2);
 *   - K/V of all ranks are all-gathered in rank order ("rank-major"), and each
 *     local Q chunk attends to its causal K/V prefix, selected from the
 *     rank-major K/V by a direct index; both local chunks of every
 *     sub-sequence run in one fused attention call (section 3.1, 3.3);
 *   - the backward adds dK/dV into a rank-major gradient buffer through the
 *     same index (section 3.1).
 * The attention itself is masked softmax attention evaluated block-wise with
 * the online-softmax trick (DCP paper, background section and its block-wise
 * listing); besides causal/EOD-reset it supports the DCP paper's lambda mask
 * (attention sink + sliding window) and shared-question mask (sparse-mask
 * section, Fig. 6(b) and 6(d)).
 *
 * Conventions shared by every call:
 *   - Every call returns a cva_status.  On any error nothing has been
 *     enqueued on the GPU, and cva_last_error() returns a message for the
 *     calling thread.
 *   - Tensors are caller-owned, contiguous, row-major, in device memory:
 *       q     [T_loc, Hq,  Dqk]   local queries (this rank's two chunks of
 *                                 every sub-sequence, local order)
 *       k_rm  [T,     Hkv, Dqk]   rank-major gathered keys
 *       v_rm  [T,     Hkv, Dv ]   rank-major gathered values
 *       o     [T_loc, Hq,  Dv ]   output, same dtype as q
 *       lse   [Hq, T_loc] float   natural-log sum-exp of the scaled logits
 *     with T = cu_seqlens[n], T_loc = T / cp_size.  Query head h uses K/V head
 *     h / (Hq/Hkv) (grouped-query attention, contiguous groups).
 *   - A stream argument is a hipStream_t passed as void* (NULL: the null
 *     stream).  Kernel calls are asynchronous on it.
 *   - Plans are built on the host from (cu_seqlens, cp_size, rank, mask,
 *     head shape, dtype), are immutable afterwards except for binding their
 *     device copy with cva_plan_upload, and can be reused for every layer that
 *     sees the same batch (the RFC caches the same metadata, section 3.3).
 */
#ifndef CVA_H
#define CVA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CVA_OK = 0,
  CVA_E_ARG = 1,          /* null pointer, negative count, bad size argument    */
  CVA_E_CU_SEQLENS = 2,   /* empty, not starting at 0, or not strictly increasing */
  CVA_E_ALIGN = 3,        /* a sub-sequence length not divisible by 2*cp_size    */
  CVA_E_RANK = 4,         /* cp_size < 1 or rank outside [0, cp_size)            */
  CVA_E_HEADS = 5,        /* Hq or Hkv < 1, or Hq not a multiple of Hkv          */
  CVA_E_HEADDIM = 6,      /* head dims not supported (Dqk < Dv, or no kernel)    */
  CVA_E_DTYPE = 7,        /* unknown dtype                                        */
  CVA_E_MASK = 8,         /* bad mask descriptor                                  */
  CVA_E_UNSUPPORTED = 9,  /* valid request that the library does not implement     */
  CVA_E_WORKLOAD = 10,    /* per-rank sum(q_len*kv_len) not equal (never for valid input) */
  CVA_E_HIP = 11,         /* a HIP runtime call failed                            */
  CVA_E_SCALE = 12,       /* softmax_scale not finite or not > 0                  */
  CVA_E_WORKSPACE = 13,   /* workspace missing or too small                       */
  CVA_E_NOT_UPLOADED = 14 /* the plan has no device copy yet (cva_plan_upload)    */
} cva_status;

typedef enum { CVA_BF16 = 0, CVA_FP16 = 1, CVA_FP32 = 2 } cva_dtype;

typedef enum {
  CVA_MASK_CAUSAL = 0,        /* key k visible to query q iff k <= q (positions within the sub-sequence) */
  CVA_MASK_LAMBDA = 1,        /* causal and (k < sink or q - k < window)                                 */
  CVA_MASK_SHARED_PREFIX = 2, /* prefix rows causal; an answer row sees the prefix and itself causally   */
  CVA_MASK_BLOCKWISE = 3      /* causal blockwise: blocks of `block` tokens; a query of block b sees keys
                                 k <= q in the first `sink` blocks or in blocks b-window+1 .. b; a query
                                 of the sub-sequence's last block (the test sample) sees every k <= q  */
} cva_mask_type;

/* Mask descriptor, copied into the plan by cva_plan_create.
 *   type          cva_mask_type
 *   sink, window  lambda mask: tokens, sink >= 0, window >= 1 (window counts the diagonal);
 *                 blockwise mask: blocks, sink >= 0, window >= 1 (window counts the own block)
 *   block         blockwise mask only: tokens per block, >= 1 (DCP paper, evaluation: 256,
 *                 window 2 blocks, one sink block, one test block)
 *   n_branches    shared-prefix only: answers per sequence, >= 1
 *   branch_bounds shared-prefix only: int32 [n_seqs][n_branches + 1], per sequence
 *                 {prefix_end, end_of_answer_0, ..., end_of_answer_{n_branches-1}}
 *                 as in-sequence positions, non-decreasing, last == sequence length.
 *                 Caller-owned, read only during cva_plan_create.
 * A NULL descriptor means causal. */
typedef struct {
  int32_t type;
  int32_t sink;
  int32_t window;
  int32_t n_branches;
  const int32_t* branch_bounds;
  int32_t block;
} cva_mask_desc;

typedef struct cva_plan cva_plan;

/* Metadata of one rank (RFC interface get_thd_load_balanced_cp_metadata,
 * section 3.5.2.1).  All arrays are owned by the plan and live as long as it.
 *   local_cu          [n_seqs+1]      cu_seqlens / cp_size: local offsets of the sub-sequences
 *   actual_seq_qlen   [n_segments+1]  cumulative query lengths, leading 0; segment 2i is
 *                                     chunk r of sub-sequence i, segment 2i+1 chunk 2R-1-r
 *   actual_seq_kvlen  [n_segments+1]  cumulative K/V prefix lengths, leading 0
 *   kv_index          [kv_index_len]  rank-major row of every prefix position, segment by
 *                                     segment, positions 0..kv_len-1 in order
 *   seg_q_pos0        [n_segments]    in-sequence position of each segment's first query
 *   workload_per_rank [cp_size]       sum(q_len * kv_len) of every rank (all equal)
 *   visible_pairs     unmasked (query, key) pairs of this rank, per query head
 *   visible_pairs_per_rank [cp_size] the same count for every rank: equal under the causal
 *                     mask, unequal under the sparse masks (the zig-zag split balances
 *                     sum(q_len*kv_len), not the visible pairs; DCP paper, sparse masks)
 *   fwd_tiles         non-empty (Q tile, K/V tile) pairs the forward schedule visits, per item head group */
typedef struct {
  int64_t local_tokens;
  int64_t global_tokens;
  int32_t n_seqs;
  int32_t n_segments;
  int32_t cp_size;
  int32_t rank;
  const int32_t* local_cu;
  const int32_t* actual_seq_qlen;
  const int32_t* actual_seq_kvlen;
  const int32_t* kv_index;
  const int32_t* seg_q_pos0;
  int64_t kv_index_len;
  const int64_t* workload_per_rank;
  int64_t visible_pairs;
  int64_t fwd_tiles;
  const int64_t* visible_pairs_per_rank;
} cva_metadata;

/* Message for the last failed call on this thread ("" if none). */
const char* cva_last_error(void);

/* Build a plan on the host: validate (RFC section 2 usage limits and section
 * 3.4 reliability: sequence, rank, head and head-dim checks before any device
 * work), build the metadata and the tile schedules.  dtype is a cva_dtype.
 * Supported head dims: (Dqk, Dv) in {(64,64), (128,128), (192,128)}; fp32 is a
 * forward-only correctness path (VALU kernel), bf16/fp16 run on MFMA.
 * For 32768 or more local rows the row and block passes run on up to 8 host
 * threads (joined before the call returns; the plan does not depend on them;
 * the environment variable CVA_PLAN_THREADS lowers the cap, 1 = no threads).
 * On success *out owns a new plan (release with cva_plan_destroy). */
cva_status cva_plan_create(const int32_t* cu_seqlens, int32_t n_seqs, int32_t cp_size,
                           int32_t rank, const cva_mask_desc* mask, int32_t hq, int32_t hkv,
                           int32_t d_qk, int32_t d_v, int32_t dtype, cva_plan** out);

void cva_plan_destroy(cva_plan* plan);

/* Fill *out with views of the plan's host metadata. */
cva_status cva_plan_get_metadata(const cva_plan* plan, cva_metadata* out);

/* Bytes of device memory the plan's tables need (4-byte aligned blob). */
size_t cva_plan_device_bytes(const cva_plan* plan);

/* Copy the plan's tables to caller-owned device memory dev_buf (at least
 * cva_plan_device_bytes bytes, 256-byte aligned) on `stream`, and bind the plan
 * to that buffer for later cva_fwd / cva_bwd calls.  The copy is asynchronous:
 * the call returns once it is enqueued (the plan keeps its host tables alive
 * until the copy has completed; cva_plan_destroy waits for it).  Calls that use
 * the plan on `stream` are ordered after the copy; on another stream the caller
 * orders them (e.g. with an event recorded on `stream`).  The buffer must stay
 * alive and untouched while those calls may run. */
cva_status cva_plan_upload(cva_plan* plan, void* dev_buf, size_t bytes, void* stream);

/* Forward (RFC interface AttnFuncWithCPAndKVAllGatherForTHDLoadBalanced,
 * section 3.5.2.2, forward half; k/v arrive already gathered rank-major):
 * o = softmax(scale * q k^T masked) v for this rank's rows, plus lse.
 * softmax_scale must be finite and > 0 (the binding maps None to 1/sqrt(Dqk)). */
cva_status cva_fwd(const cva_plan* plan, const void* q, const void* k_rm, const void* v_rm,
                   void* o, float* lse, float softmax_scale, void* stream);

/* Forward with split K/V ranges (DCP paper, background: block-wise attention
 * with online softmax; a query block's K/V range is cut into pieces whose
 * partial outputs are merged through their log-sum-exp).  With A the average
 * work per compute unit in 64-key K/V tiles (at least 8), the plan cuts every
 * forward Q tile whose K/V walk is longer than 4/3 A (longer than 8 when A is
 * 8) into up to 8 pieces of at most A tiles; when the environment variable
 * CVA_FWD_SPLIT_CAP holds an integer c >= 1 at cva_plan_create, every tile
 * longer than c is cut into pieces of at most c.  Each piece writes an fp32
 * partial output and LSE
 * to the workspace and a second kernel merges them into o and lse.  Same
 * arguments and results as cva_fwd, plus a caller-owned device workspace of at
 * least cva_fwd_workspace_bytes bytes (256-byte aligned) that must not be used
 * by another call while this one may run.  When the plan cuts nothing (the
 * workspace size is 0) or dtype is fp32, this is exactly cva_fwd and workspace
 * may be NULL.  Errors: CVA_E_WORKSPACE if the workspace is missing or too
 * small, otherwise as cva_fwd. */
size_t cva_fwd_workspace_bytes(const cva_plan* plan);
cva_status cva_fwd_split(const cva_plan* plan, const void* q, const void* k_rm, const void* v_rm,
                         void* o, float* lse, float softmax_scale, void* workspace,
                         size_t ws_bytes, void* stream);

/* Forward with attention dropout (RFC interface section 3.5.2.2: the
 * attention_dropout argument, a probability p in [0, 1)).  Every softmax
 * probability P[q,k] is kept or set to zero before it multiplies V; kept ones
 * are scaled by 256 / (256 - t); lse is that of the undropped softmax.  The
 * keep decision of a (sequence, query head, query, key) is a pure function of
 * the seed and the in-sequence positions, so it does not depend on the CP
 * split or the tiling: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011) with
 * key = seed (low word first) and counter (k / 4, q / 4, query head, sequence
 * index) gives one 128-bit output per 4 x 4 block; the pair's byte is byte
 * k % 4 of word q % 4, and the pair is kept iff that byte >= t, where
 * t = round(256 p) clamped to 255 (so the realised drop probability is t/256;
 * t = 0 drops nothing).  workspace NULL: one launch per item as cva_fwd;
 * otherwise as cva_fwd_split with that workspace.  The backward must be called
 * through cva_bwd_dropout with the same p and seed.  bf16, fp16 and fp32.
 * Errors: CVA_E_ARG if p is outside [0, 1), otherwise as cva_fwd /
 * cva_fwd_split. */
cva_status cva_fwd_dropout(const cva_plan* plan, const void* q, const void* k_rm, const void* v_rm,
                           void* o, float* lse, float softmax_scale, float dropout_p, uint64_t seed,
                           void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes cva_bwd needs (fp32 row statistics: Delta and LSE*log2(e),
 * 2 * T_loc * Hq floats). */
size_t cva_bwd_workspace_bytes(const cva_plan* plan);

/* Backward (same interface, backward half): given dout [T_loc, Hq, Dv] and the
 * forward's o and lse, write dq [T_loc, Hq, Dqk] and the rank-major
 * dk_rm [T, Hkv, Dqk], dv_rm [T, Hkv, Dv].  dk_rm/dv_rm are fully written:
 * rows no local query attends to are zero, so the result equals index_add_ of
 * the per-segment gradients into a zeroed buffer (RFC section 3.1).
 * Deterministic: no atomics, fixed summation order.  bf16/fp16 only. */
cva_status cva_bwd(const cva_plan* plan, const void* q, const void* k_rm, const void* v_rm,
                    const void* o, const float* lse, const void* dout, void* dq, void* dk_rm,
                    void* dv_rm, void* workspace, size_t ws_bytes, float softmax_scale,
                    void* stream);

/* Backward of cva_fwd_dropout (same p and seed; o and lse from that forward):
 * the same keep mask zeroes the dropped pairs' share of dV and of dP, and kept
 * pairs are scaled by 256 / (256 - t) in both; Delta = rowsum(dO * O) with the
 * dropped forward's O.  Arguments, workspace and results otherwise as cva_bwd.
 * Errors: CVA_E_ARG if p is outside [0, 1), otherwise as cva_bwd. */
cva_status cva_bwd_dropout(const cva_plan* plan, const void* q, const void* k_rm, const void* v_rm,
                           const void* o, const float* lse, const void* dout, void* dq, void* dk_rm,
                           void* dv_rm, void* workspace, size_t ws_bytes, float softmax_scale,
                           float dropout_p, uint64_t seed, void* stream);

/* Allocation-free backward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels and results as cva_bwd without the
 * workspace: the row statistics (Delta and LSE*log2(e), cva_bwd_workspace_bytes
 * bytes) go to a device array the library holds on every GPU it runs on until
 * the process ends, of cva_bwd_noalloc_max_bytes() bytes (16 MiB: Hq * T_loc up
 * to 2^21, e.g. 32 heads x 65536 local rows).  The call allocates nothing (no
 * hipMalloc/hipFree); its first call on a GPU looks up that GPU's copy of the
 * array.  Every call on one GPU shares the array, whose contents are left from
 * the last call (everything it reads is written earlier in the same call):
 * calls that may run at the same time on one GPU (unordered streams) race and
 * must not be made.  Errors: CVA_E_WORKSPACE if the plan needs more than the
 * array holds, CVA_E_HIP if the array cannot be looked up, otherwise as
 * cva_bwd. */
size_t cva_bwd_noalloc_max_bytes(void);
cva_status cva_bwd_noalloc(const cva_plan* plan, const void* q, const void* k_rm, const void* v_rm,
                           const void* o, const float* lse, const void* dout, void* dq,
                           void* dk_rm, void* dv_rm, float softmax_scale, void* stream);

/* Schedule introspection for tests and tools.  which: 0 forward, 1 backward dQ,
 * 2 backward dK/dV, 3 forward with split K/V ranges (the items of
 * cva_fwd_split, same record layout as 0; pieces of one Q tile share its
 * segment and first query).  Returns the tile sizes and a host view of the schedule:
 *   forward / dQ:  q tiles {segment, first local query of the tile (segment-relative),
 *                  rows in tile, span_begin, span_count}; spans {first K/V tile,
 *                  end K/V tile, partial flag} in units of tile_kv keys.
 *   dK/dV:         kv tiles {sequence, first key position, keys in tile, span_begin,
 *                  span_count}; spans {segment, first q tile, end q tile, partial flag}
 *                  with q tiles of tile_q rows counted from the segment start.
 * Arrays are owned by the plan. */
typedef struct {
  int32_t tile_q;
  int32_t tile_kv;
  int32_t n_tiles;
  int32_t n_spans;
  const int32_t* tiles; /* [n_tiles][5] */
  const int32_t* spans; /* [n_spans][4] */
} cva_schedule;

cva_status cva_plan_get_schedule(const cva_plan* plan, int32_t which, cva_schedule* out);

/* The plan's remaining device tables, as cva_plan_upload copies them (host
 * views owned by the plan), for tests and tools that check every index a
 * kernel dereferences (MindSpeed RFC section 3.4: reliability).
 *   segs          [n_segs][8] {sequence, chunk (placement share: Q block), queries,
 *                 K/V prefix length, first local row, offset in kv_index, in-sequence
 *                 position of the first query, sequence length}
 *   kv_index      [kv_index_len] rank-major row of every prefix position
 *   row_iv        [n_rows][4] visible keys of every local row, [a0, a1) u [b0, b1),
 *                 in positions of its segment's prefix
 *   zero_rows     [n_zero_ranges][2] rank-major row ranges the backward zero-fills
 *   split_slot    [n_split_items] partial slot of every item of schedule 3, or -1
 *   split_combine [n_combine][5] {segment, first query, rows, first slot, pieces}
 *   n_split_slots partial slots of schedule 3
 *   fwd_deal_*    the streamed forward's deal of schedule 0's items (the
 *                 environment variable CVA_FWD_STREAM_WGS, an integer >= 1 at
 *                 cva_plan_create, caps wgs): wgs
 *                 work-groups per head group (0: one work-group per item), work-group
 *                 w takes items fwd_deal_items[fwd_deal_start[w] ..
 *                 fwd_deal_start[w+1]) (start has wgs+1 entries)
 *   split_deal_*  the same for schedule 3 */
typedef struct {
  int32_t n_segs;
  const int32_t* segs;
  int64_t kv_index_len;
  const int32_t* kv_index;
  int64_t n_rows;
  const int32_t* row_iv;
  int32_t n_zero_ranges;
  const int32_t* zero_rows;
  int32_t n_split_items;
  const int32_t* split_slot;
  int32_t n_combine;
  const int32_t* split_combine;
  int32_t n_split_slots;
  int32_t fwd_deal_wgs;
  const int32_t* fwd_deal_start;
  const int32_t* fwd_deal_items;
  int32_t n_fwd_deal_items;
  int32_t split_deal_wgs;
  const int32_t* split_deal_start;
  const int32_t* split_deal_items;
  int32_t n_split_deal_items;
} cva_plan_tables;

cva_status cva_plan_get_tables(const cva_plan* plan, cva_plan_tables* out);

/* Block placement over n_devices (DCP paper, section 4.1 and its placement
 * model): data blocks are the Q, K/V and O rows (all heads) of `block`
 * consecutive tokens of one sequence, kept on one device; computation blocks
 * are (Q block, K/V block) pairs of one sequence whose mask is not all zero.
 * A greedy planner stands in for the page's hypergraph partitioner: data
 * blocks balanced in tokens, computation blocks balanced in visible pairs
 * within (1 + epsilon) of the mean where possible, and the connectivity
 * volume (each remote input block fetched once per computing device, each
 * partial output block returned once per computing device) kept low.  Host
 * only; the kernels of this library run one rank's share of the RFC's zig-zag
 * split, whose per-rank pairs and K/V all-gather volume are reported beside it.
 *   data_blocks    [n_data_blocks][4]  {sequence, first token, tokens, device}
 *   comp_blocks    [n_comp_blocks][4]  {sequence, q block, k/v block, device}
 *   comp_pairs     [n_comp_blocks]     visible (query, key) pairs per head
 *   device_tokens / device_pairs / device_send_bytes / device_recv_bytes
 *                  [n_devices], under the connectivity volume
 *   total_comm_bytes  connectivity volume: sum over data blocks of size times
 *                  (devices spanned - 1)
 *   block_comm_bytes  the page's per-computation-block volume: sizes of the
 *                  remote inputs and outputs of every computation block
 *   zigzag_valid   1 when every sequence length divides by 2*n_devices
 *   zigzag_pairs   [n_devices] visible pairs per rank under the zig-zag split
 *   zigzag_comm_bytes  K/V bytes all ranks receive in the zig-zag all-gather
 * Sizes come from hq, hkv, d_qk, d_v and dtype (a cva_dtype).  Sequences need
 * not be aligned.  n_devices in [1, 64], block >= 1, epsilon >= 0.  Errors as
 * cva_plan_create; the object owns every array until cva_placement_destroy. */
typedef struct cva_placement cva_placement;
typedef struct {
  int32_t n_devices;
  int32_t block;
  int32_t n_data_blocks;
  int32_t n_comp_blocks;
  const int32_t* data_blocks;
  const int32_t* comp_blocks;
  const int64_t* comp_pairs;
  const int64_t* device_tokens;
  const int64_t* device_pairs;
  const int64_t* device_send_bytes;
  const int64_t* device_recv_bytes;
  int64_t total_comm_bytes;
  int64_t block_comm_bytes;
  int32_t zigzag_valid;
  const int64_t* zigzag_pairs;
  int64_t zigzag_comm_bytes;
} cva_placement_info;

cva_status cva_placement_create(const int32_t* cu_seqlens, int32_t n_seqs, const cva_mask_desc* mask,
                                int32_t n_devices, int32_t block, int32_t hq, int32_t hkv,
                                int32_t d_qk, int32_t d_v, int32_t dtype, double epsilon,
                                cva_placement** out);
cva_status cva_placement_get(const cva_placement* placement, cva_placement_info* out);

/* One device's share of a placement as a plan (DCP paper, section 4.1: every
 * computation block pairs a Q block with a K/V block; Fig. 9(b): when several
 * computation blocks feed one output block their partial results are reduced).
 * The plan computes every computation block the placement gives `device`: the
 * block's query rows against its K/V block's keys under the placement's mask,
 * one fp32 partial output and LSE per block (per 64..256-row query tile), and
 * merges the partials of blocks that feed the same O block by log-sum-exp.  Run
 * it with cva_fwd_split (cva_fwd, cva_bwd and cva_plan_get_metadata return
 * CVA_E_UNSUPPORTED) on the packed, unsplit tensors, every block in place:
 * q [T, Hq, Dqk], k_rm [T, Hkv, Dqk], v_rm [T, Hkv, Dv], o [T, Hq, Dv],
 * lse [Hq, T] with T = cu_seqlens[n].  It writes the rows of the O blocks the
 * device contributes to -- the device's partial result over its own
 * computation blocks, normalised, with its LSE (what it would send to the O
 * block's owner; the owner merges the devices' results the same way) -- and
 * leaves every other row untouched.  Needs bf16/fp16, a supported head shape
 * and a block size that is a multiple of 64.  The plan is independent of the
 * placement object afterwards (release with cva_plan_destroy).  Errors:
 * CVA_E_RANK (device out of range), CVA_E_UNSUPPORTED, CVA_E_HEADS,
 * CVA_E_HEADDIM. */
cva_status cva_placement_plan_create(const cva_placement* placement, int32_t device,
                                     cva_plan** out);
void cva_placement_destroy(cva_placement* placement);

/* Per-kernel timing, for benchmarks.  While enabled, cva_fwd and cva_bwd
 * record a hipEvent before and after every kernel they launch, on the stream
 * the kernel is launched on.  cva_timing_read waits for the recorded events,
 * folds their elapsed times into per-kernel totals and returns the totals
 * since the last cva_timing_enable(1) (which resets them).  Kernel ids:
 *   0 forward, 3 backward dK/dV, 4 backward dQ (which also forms Delta and
 *   zero-fills the uncovered dK/dV rows), 5 forward merge of split pieces;
 *   ids 1 and 2 are reserved (no kernel of their own any more).
 * Process-wide state, safe to use from several host threads (a mutex guards it;
 * launches are timed while they are being enqueued, one at a time). */
#define CVA_N_KERNELS 6
typedef struct {
  int64_t launches[CVA_N_KERNELS];
  double total_ms[CVA_N_KERNELS];
} cva_kernel_times;

cva_status cva_timing_enable(int32_t on);
cva_status cva_timing_read(cva_kernel_times* out);
/* Restrict timing to the kernels whose id bit is set in kernel_mask (bit k =
 * kernel id k; all kernels by default), so that a timed loop can carry events
 * around one kernel only.  Takes effect for launches after the call. */
cva_status cva_timing_select(uint32_t kernel_mask);

#ifdef __cplusplus
}
#endif

#endif /* CVA_H */
