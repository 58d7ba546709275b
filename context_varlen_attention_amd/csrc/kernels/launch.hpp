// Kernel parameter blocks and launchers shared by the C ABI and the HIP kernels.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace cva {

// Device tables of a plan (int32, see plan.hpp for the record layouts).
struct PlanTables {
  const int32_t* segs;
  const int32_t* kv_index;
  const int32_t* row_iv;
  const int32_t* fwd_tiles;
  const int32_t* fwd_spans;
  const int32_t* dq_tiles;
  const int32_t* dq_spans;
  const int32_t* kv_tiles;
  const int32_t* kv_spans;
  const int32_t* zero_rows;
  const int32_t* fwds_slot;     // split forward: partial slot per item (-1: direct)
  const int32_t* fwds_combine;  // split forward: merge records
  const int32_t* deal_start;    // streamed forward: [wgs + 1] of the schedule launched
  const int32_t* deal_items;    // streamed forward: items per work-group
};

// Attention dropout of a launch (random bytes: Philox4x32-10 per 4 x 4 block
// of (query, key) positions, see the kernels' common helpers).
struct DropParams {
  uint32_t t;               // byte threshold round(256 p); 0 = no dropout
  uint32_t seed_lo, seed_hi;
  float scale;              // 256 / (256 - t): applied to kept probabilities
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  PlanTables t;
  int32_t n_tiles;         // forward Q tiles
  int32_t n_head_groups;   // hq / heads_per_tile
  int32_t heads_per_tile;
  int32_t hq, hkv, group;  // group = hq / hkv
  int32_t t_loc;
  int32_t tile_q;
  int32_t tile_kv;
  float scale_log2;        // softmax_scale * log2(e)
  // split forward (slot == nullptr: every item writes o/lse directly)
  const int32_t* slot;     // [n_tiles] partial slot of each item, or -1
  float* ws_o;             // [slots * hq * tile_q][Dv] fp32 partial outputs
  float* ws_lse;           // [slots * hq * tile_q] partial LSE (natural log)
  const int32_t* combine;  // [n_combine][5] merge records
  int32_t n_combine;
  // streamed forward: work-groups per head group, each walking its items
  // (t.deal_start / t.deal_items) as one stream of K/V tiles (0: one
  // work-group per item)
  int32_t stream_wgs;
  DropParams drop;         // drop.t == 0: no dropout (the streamed form has none)
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;            // [hq, t_loc] workspace: Delta = rowsum(dO * O)
  float* lse2;             // [hq, t_loc] workspace: LSE * log2(e)
  PlanTables t;
  int32_t n_dq_tiles, n_kv_tiles, n_zero_ranges;
  int32_t dq_heads_per_tile, dq_head_groups;
  int32_t hq, hkv, group;
  int32_t t_loc;
  int64_t t_total;
  float scale;             // softmax_scale
  float scale_log2;        // softmax_scale * log2(e)
  DropParams drop;         // drop.t == 0: no dropout
};

// Optional hook around every kernel launch (timing); ids as in cva.h.
// (ids 1 and 2, the former Delta and zero-fill launches, are reserved: that
// work runs inside the dQ kernel)
enum KernelId { K_FWD = 0, K_BWD_DKDV = 3, K_BWD_DQ = 4, K_FWD_MERGE = 5 };
struct LaunchHook {
  virtual void before(int kernel, hipStream_t s) = 0;
  virtual void after(int kernel, hipStream_t s) = 0;
  virtual ~LaunchHook() = default;
};

// dtype: 0 bf16, 1 fp16, 2 fp32.  Return hipSuccess or the launch error.
hipError_t launch_fwd(int dtype, int d_qk, int d_v, const FwdParams& p, hipStream_t stream,
                      LaunchHook* hook);
hipError_t launch_bwd(int dtype, int d_qk, int d_v, const BwdParams& p, hipStream_t stream,
                      LaunchHook* hook);

// Allocation-free backward: bytes of the library-held device array that takes
// the place of the caller's workspace, and its address on the device of
// `stream` (looked up once per device; no allocation).
constexpr size_t kBwdNoAllocScratchBytes = size_t(16) << 20;
hipError_t bwd_noalloc_scratch(hipStream_t stream, float** ptr);

}  // namespace cva
