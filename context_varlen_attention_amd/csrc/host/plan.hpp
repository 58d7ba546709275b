// Host-side plan: validation, metadata and tile schedules for one CP rank.
// Pure C++17; no HIP calls, so it builds and runs on a machine without a GPU.
#pragma once

#include <cstdint>
#include <string>
#include <utility>
#include <vector>

#include "cva.h"

namespace cva {

// Per-segment record as laid out in the device blob (8 int32 each).
// A segment is one (sub-sequence, chunk) pair of this rank, in local order.
enum SegField {
  SEG_SEQ = 0,     // sub-sequence index
  SEG_CHUNK = 1,   // chunk id j (r or 2R-1-r)
  SEG_QLEN = 2,    // queries in the segment (= chunk length c)
  SEG_KVLEN = 3,   // causal K/V prefix length (j+1)*c
  SEG_QROW0 = 4,   // local row of the first query
  SEG_KVOFF = 5,   // offset of the segment's prefix in kv_index
  SEG_QPOS0 = 6,   // in-sequence position of the first query (j*c)
  SEG_SEQLEN = 7,  // length of the sub-sequence
  SEG_INTS = 8
};

// Q-stationary tile record (forward and backward dQ), 5 int32.
enum QTileField { QT_SEG = 0, QT_Q0 = 1, QT_ROWS = 2, QT_SPAN0 = 3, QT_NSPAN = 4, QT_INTS = 5 };
// K/V-stationary tile record (backward dK/dV), 5 int32.
enum KvTileField { KT_SEQ = 0, KT_K0 = 1, KT_KEYS = 2, KT_SPAN0 = 3, KT_NSPAN = 4, KT_INTS = 5 };
// Span record, 4 int32.  Q-stationary: {kv tile begin, kv tile end, partial, 0}.
// K/V-stationary: {segment, q tile begin, q tile end, partial}.
enum { SPAN_INTS = 4 };

struct Schedule {
  int32_t tile_q = 0;   // query positions per Q tile
  int32_t tile_kv = 0;  // keys per K/V tile
  std::vector<int32_t> tiles;  // [n][5], launch order (most work first)
  std::vector<int32_t> spans;  // [m][4]
  int64_t tile_pairs = 0;      // non-empty (Q tile, K/V tile) pairs
  int32_t n_tiles() const { return (int32_t)(tiles.size() / 5); }
  int32_t n_spans() const { return (int32_t)(spans.size() / SPAN_INTS); }
};

// Offsets (in int32 elements) of the tables inside the device blob.
struct BlobLayout {
  int64_t segs = 0, kv_index = 0, row_iv = 0;
  int64_t fwd_tiles = 0, fwd_spans = 0;
  int64_t dq_tiles = 0, dq_spans = 0;
  int64_t kv_tiles = 0, kv_spans = 0;
  int64_t zero_rows = 0;
  int64_t fwds_tiles = 0, fwds_spans = 0, fwds_slot = 0, fwds_combine = 0;
  int64_t fwd_deal_start = 0, fwd_deal_items = 0, fwds_deal_start = 0, fwds_deal_items = 0;
  int64_t total = 0;
};

// Streamed forward (one work-group per CU walking a list of work items as one
// stream of K/V tiles): the items of a forward schedule dealt to `wgs`
// work-groups per head group (every head group gets the same deal), each
// work-group's items in work-group order.  wgs == 0: one work-group per item.
constexpr int32_t kFwdStreamMaxItems = 48;  // items one work-group holds in LDS
constexpr int32_t kStreamItemSteps = 1;     // an item boundary's cost, in K/V tile steps
struct StreamDeal {
  int32_t wgs = 0;
  std::vector<int32_t> start;  // [wgs + 1] into items
  std::vector<int32_t> items;  // schedule item indices
};

// Combine record of a Q tile whose K/V range was split over several forward
// work items: {segment, first query, rows, first partial slot, pieces}.
enum CombineField { CB_SEG = 0, CB_Q0 = 1, CB_ROWS = 2, CB_SLOT0 = 3, CB_NPIECE = 4, CB_INTS = 5 };

struct Plan {
  // request
  int32_t n_seqs = 0, cp_size = 1, rank = 0;
  int32_t hq = 0, hkv = 0, d_qk = 0, d_v = 0, dtype = 0;
  int32_t mask_type = CVA_MASK_CAUSAL, sink = 0, window = 0, n_branches = 0, block = 0;
  std::vector<int32_t> cu;             // [n+1]
  std::vector<int32_t> branch_bounds;  // [n][n_branches+1] (shared prefix)

  // metadata
  int64_t T = 0, T_loc = 0;
  std::vector<int32_t> local_cu, aq, akv, kv_index, seg_q_pos0;
  std::vector<int64_t> workload;
  int64_t visible_pairs = 0;
  std::vector<int64_t> visible_pairs_per_rank;  // [cp_size]
  std::vector<int32_t> segs;    // [2n][8]
  std::vector<int32_t> row_iv;  // [T_loc][4]: visible keys = [a0,a1) u [b0,b1)

  // kernel configuration + schedules
  int32_t fwd_heads_per_tile = 1;  // query heads of one K/V group sharing a forward work-group
  Schedule fwd, dq, dkdv;
  // Forward with split K/V ranges: the forward schedule with every Q tile that
  // walks more than fwd_split_cap K/V tiles cut into pieces, each writing an
  // fp32 partial result to a slot of the forward workspace, merged by LSE.
  Schedule fwds;
  std::vector<int32_t> fwds_slot;     // [n items]: partial slot, or -1 (writes o/lse directly)
  std::vector<int32_t> fwds_combine;  // [m][CB_INTS]
  int32_t n_split_slots = 0;
  int32_t fwd_split_cap = 0;
  StreamDeal fwd_deal, fwds_deal;  // streamed forward deals of fwd and fwds
  std::vector<int32_t> zero_rows;  // [m][2] rank-major row ranges no local query sees (<= 8 rows each)

  // one device's share of a block placement (build_placed_plan): segments are
  // the Q blocks the device computes on, the only schedule is fwds (one item per
  // computation block and Q tile, each with its own partial slot)
  bool placed = false;
  int32_t placed_device = -1;

  // device copy
  std::vector<int32_t> blob;
  BlobLayout layout;
  void* dev = nullptr;
  size_t dev_bytes = 0;
  void* upload_done = nullptr;  // hipEvent_t recorded after the last upload's copy (C ABI layer)
};

// The visible keys of a row, [iv0, iv1) u [iv2, iv3), as at most two disjoint,
// sorted intervals (overlapping or touching intervals merged).
struct KeySet {
  int n = 0;
  std::pair<int32_t, int32_t> v[2];
};
inline KeySet key_set(const int32_t* iv) {
  KeySet r;
  std::pair<int32_t, int32_t> a{iv[0], iv[1]}, b{iv[2], iv[3]};
  if (a.second <= a.first) std::swap(a, b);
  if (a.second <= a.first) return r;  // both empty
  if (b.second <= b.first) {
    r.n = 1;
    r.v[0] = a;
    return r;
  }
  if (b.first < a.first) std::swap(a, b);
  if (b.first <= a.second) {
    r.n = 1;
    r.v[0] = {a.first, a.second > b.second ? a.second : b.second};
  } else {
    r.n = 2;
    r.v[0] = a;
    r.v[1] = b;
  }
  return r;
}

// Placement of data and computation blocks over devices (placement.cpp).
struct Placement {
  Plan mask;  // the request's sequences and mask (cu, n_seqs, mask fields)
  int32_t n_devices = 1, block = 1;
  int32_t hq = 1, hkv = 1, d_qk = 0, d_v = 0, dtype = 0;
  double epsilon = 0.1;             // computation imbalance tolerance
  std::vector<int32_t> data;        // [n][4] {sequence, first token, tokens, device}
  std::vector<int32_t> comp;        // [m][4] {sequence, q block, k/v block, device}
  std::vector<int64_t> comp_pairs;  // [m] visible pairs per head
  std::vector<int64_t> device_tokens, device_pairs, device_send_bytes, device_recv_bytes;  // [n_devices]
  int64_t total_comm_bytes = 0;     // connectivity: each remote block moved once per device
  int64_t block_comm_bytes = 0;     // per computation block: every remote use counted
  bool zigzag_ok = false;
  std::vector<int64_t> zigzag_pairs;  // [n_devices]
  int64_t zigzag_comm_bytes = 0;      // K/V all-gather of the zig-zag split
};
cva_status build_placement(Placement& pl);

// A computation block of a placed plan: Q block segment `seg` against the keys
// [k0, k1) of its sequence (in-sequence positions).
struct PlacedBlock {
  int32_t seg, k0, k1;
};
// Device `device`'s computation blocks of a placement as a plan (placement.cpp).
cva_status build_placed_plan(const Placement& pl, int32_t device, Plan& p);
// Its forward items, partial slots and merge records (schedule.cpp).
cva_status build_placed_schedule(Plan& p, const std::vector<PlacedBlock>& blocks);

// Thread-local error message used by the C ABI.
void set_error(const std::string& msg);
const char* last_error();

// validate.cpp
cva_status validate_request(const int32_t* cu_seqlens, int32_t n_seqs, int32_t cp_size,
                            int32_t rank, const cva_mask_desc* mask, int32_t hq, int32_t hkv,
                            int32_t d_qk, int32_t d_v, int32_t dtype);

// Mask descriptor checks (also used by the block placement); cu is validated.
cva_status validate_mask(const cva_mask_desc* mask, const int32_t* cu, int32_t n_seqs);

// Supported kernel head shapes (validate.cpp).
bool head_dims_supported(int32_t dtype, int32_t d_qk, int32_t d_v);

// metadata.cpp
cva_status build_metadata(Plan& p);

// schedule.cpp
void row_intervals(const Plan& p, int seg, int32_t a, int32_t iv[4]);
// Visible keys of query position q of sub-sequence seq: [iv0, iv1) u [iv2, iv3).
void position_intervals(const Plan& p, int32_t seq, int32_t q, int32_t iv[4]);
cva_status build_schedules(Plan& p);
void build_blob(Plan& p);
void build_fwd_split(Plan& p);
// Deal of schedule s's items to the streamed forward's work-groups
// (kSplitCUs / head groups of them, at most one per item), round by round:
// every work-group takes one item per round, the round's items (longest first)
// going to the least loaded work-groups (load: K/V tile steps +
// kStreamItemSteps per item); no deal (wgs = 0) for fp32 or when a work-group
// would get more than kFwdStreamMaxItems items.
void build_stream_deal(const Plan& p, const Schedule& s, StreamDeal& d);

// Tile shape of the forward kernel for a plan's head shape.
struct FwdShape {
  int32_t heads_per_tile;  // query heads per work-group (share one K/V head)
  int32_t tile_q;          // query positions per work-group
  int32_t tile_kv;
};
FwdShape forward_shape(const Plan& p);
// Query positions per dQ work-group (4 waves of 32 rows, heads_per_tile heads).
int32_t dq_tile_q(const Plan& p);

constexpr int32_t kWavesPerFwdTile = 8;  // forward: two groups of 4 waves (ping-pong)
constexpr int32_t kWavesPerDqTile = 4;
constexpr int32_t kFwdMaxSpans = 8;   // forward kernel keeps a work item's spans in LDS
constexpr int32_t kDkvMaxSpans = 16;  // dK/dV kernel keeps a work item's spans in LDS
constexpr int32_t kDqMaxSpans = 8;    // dQ kernel keeps a work item's spans in LDS
constexpr int32_t kRowsPerWave = 32;
constexpr int32_t kFwdTileKv = 64;
constexpr int32_t kDqTileKv = 64;     // dQ kernel: keys per K/V tile (query tile as forward)
constexpr int32_t kDkvTileQ = 64;     // dK/dV kernel: queries per Q tile
constexpr int32_t kDkvTileKv = 128;   // dK/dV kernel: keys per work-group (4 wave pairs x 32)
constexpr int32_t kZeroRowsPerBlock = 8;  // rank-major rows per zero-fill work-group
constexpr int32_t kSplitCUs = 256;        // compute units the split balances over (MI355X)
constexpr int32_t kSplitMinSteps = 8;     // never cut a piece shorter than this many K/V tiles
constexpr int32_t kSplitMaxPieces = 8;    // pieces the split forward cuts a Q tile into, at most

}  // namespace cva
